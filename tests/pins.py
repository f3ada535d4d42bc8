"""Independent pins for the fp64 oracle.

Each pin checks an implementation against something other than itself: a
brute-force evaluation of the definition with pure-Python loops, closed forms
derived by hand (stored under tests/golden/ with their derivation), and
invariants that hold for softmax attention whatever the inputs.  The pins take
the functions under test as arguments so the same checks can be run on the
oracle (they must pass) and on copies of it with a planted mistake (some pin
must fail).  They raise AssertionError on failure.
"""
from __future__ import annotations

import json
import math
import os
from typing import Callable

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    err = np.where(same_inf, 0.0, np.abs(a - b))
    assert not np.isnan(err).any(), f"{what}: NaN"
    m = float(err.max()) if err.size else 0.0
    assert m <= tol, f"{what}: max abs error {m:.3e} > {tol:.1e}"


def brute_force_row(q_row, keys, vals, scale):
    """softmax(q.K^T*scale) V for one query row, straight from the definition,
    with pure-Python loops and no max shift (inputs here are small)."""
    scores = [scale * math.fsum(qd * kd for qd, kd in zip(q_row, k)) for k in keys]
    e = [math.exp(s) for s in scores]
    z = math.fsum(e)
    D = len(vals[0])
    o = [math.fsum(e[j] * vals[j][d] for j in range(len(keys))) / z for d in range(D)]
    return o, math.log(z)


def _rand(rng, *shape, s=1.0):
    return rng.standard_normal(shape) * s


# ---------------------------------------------------------------- attention

def pin_brute_force(attn: Callable):
    rng = np.random.default_rng(1234)
    for (B, Sq, Skv, H, D) in [(1, 1, 1, 1, 1), (2, 2, 3, 2, 4), (1, 3, 2, 3, 8),
                               (2, 10, 10, 2, 4), (1, 5, 7, 1, 3)]:
        q, k, v = (_rand(rng, B, S, H, D) for S in (Sq, Skv, Skv))
        o, lse = attn(q, k, v)
        for b in range(B):
            for h in range(H):
                keys = k[b, :, h, :].tolist()
                vals = v[b, :, h, :].tolist()
                for i in range(Sq):
                    ob, lb = brute_force_row(q[b, i, h, :].tolist(), keys, vals,
                                             1.0 / math.sqrt(D))
                    _close(o[b, i, h, :], ob, 1e-12, "brute force O")
                    _close(lse[b, h, i], lb, 1e-12, "brute force LSE")
    # a few rows of the tiny fp32 workload's shape: S = 256, D = 64, H = 2
    q, k, v = (_rand(rng, 1, 256, 2, 64) for _ in range(3))
    o, lse = attn(q, k, v)
    for h in range(2):
        keys = k[0, :, h, :].tolist()
        vals = v[0, :, h, :].tolist()
        for i in (0, 97, 255):
            ob, lb = brute_force_row(q[0, i, h, :].tolist(), keys, vals, 1.0 / 8.0)
            _close(o[0, i, h, :], ob, 1e-12, "brute force O (S=256)")
            _close(lse[0, h, i], lb, 1e-12, "brute force LSE (S=256)")


def pin_golden(attn: Callable):
    g = _golden("two_keys_ln3.json")
    q = np.array(g["q"]).reshape(1, 1, 1, 4)
    k = np.array(g["k"]).reshape(1, 2, 1, 4)
    v = np.array(g["v"]).reshape(1, 2, 1, 4)
    o, lse = attn(q, k, v, scale=g["scale"])
    _close(o[0, 0, 0], g["o"], 1e-14, "two_keys_ln3 O")
    _close(lse[0, 0, 0], g["lse"], 1e-14, "two_keys_ln3 LSE")
    g = _golden("three_keys_d1.json")
    q = np.array(g["q"]).reshape(1, 1, 1, 1)
    k = np.array(g["k"]).reshape(1, 3, 1, 1)
    v = np.array(g["v"]).reshape(1, 3, 1, 1)
    o, lse = attn(q, k, v, scale=g["scale"])
    _close(o[0, 0, 0, 0], g["o"], 1e-13, "three_keys_d1 O")
    _close(lse[0, 0, 0], g["lse"], 1e-14, "three_keys_d1 LSE")


def pin_single_key(attn: Callable):
    """One key: its weight is 1, O = v_0 and LSE = its score."""
    rng = np.random.default_rng(7)
    q, k, v = _rand(rng, 2, 5, 3, 16), _rand(rng, 2, 1, 3, 16), _rand(rng, 2, 1, 3, 16)
    o, lse = attn(q, k, v)
    _close(o, np.broadcast_to(v, o.shape), 1e-14, "single key O")
    s = np.einsum("bihd,bjhd->bhi", q, k) / 4.0
    _close(lse, s, 1e-13, "single key LSE")


def pin_zero_keys(attn: Callable):
    """K = 0: every score is 0, O = mean of V rows, LSE = ln Skv."""
    rng = np.random.default_rng(8)
    Skv = 37
    q, v = _rand(rng, 1, 6, 2, 8), _rand(rng, 1, Skv, 2, 8)
    k = np.zeros((1, Skv, 2, 8))
    o, lse = attn(q, k, v)
    _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), 1e-14, "K=0 O")
    _close(lse, np.full(lse.shape, math.log(Skv)), 1e-14, "K=0 LSE")


def pin_constant_v(attn: Callable):
    """All V rows equal c: the weights sum to 1, so O = c."""
    rng = np.random.default_rng(9)
    q, k = _rand(rng, 1, 20, 2, 16, s=3.0), _rand(rng, 1, 33, 2, 16, s=3.0)
    c = _rand(rng, 1, 1, 2, 16)
    v = np.broadcast_to(c, (1, 33, 2, 16)).copy()
    o, _ = attn(q, k, v)
    _close(o, np.broadcast_to(c, o.shape), 1e-13, "constant V")


def pin_two_keys(attn: Callable):
    """Two keys: O = sigma(s1 - s2) v1 + sigma(s2 - s1) v2."""
    rng = np.random.default_rng(10)
    q, k, v = _rand(rng, 1, 9, 2, 8), _rand(rng, 1, 2, 2, 8), _rand(rng, 1, 2, 2, 8)
    o, lse = attn(q, k, v)
    for h in range(2):
        for i in range(9):
            s1 = float(q[0, i, h] @ k[0, 0, h]) / math.sqrt(8)
            s2 = float(q[0, i, h] @ k[0, 1, h]) / math.sqrt(8)
            w1 = 1.0 / (1.0 + math.exp(s2 - s1))
            w2 = 1.0 / (1.0 + math.exp(s1 - s2))
            _close(o[0, i, h], w1 * v[0, 0, h] + w2 * v[0, 1, h], 1e-13, "two keys O")
            _close(lse[0, h, i], max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2))),
                   1e-13, "two keys LSE")


def pin_linearity(attn: Callable):
    """O is affine in V: O(a V + 1 b^T) = a O(V) + b (weights sum to 1)."""
    rng = np.random.default_rng(11)
    q, k, v = (_rand(rng, 2, 17, 3, 8) for _ in range(3))
    bvec = _rand(rng, 1, 1, 3, 8)
    o1, l1 = attn(q, k, v)
    o2, l2 = attn(q, k, -2.5 * v + bvec)
    _close(o2, -2.5 * o1 + bvec, 1e-12, "linearity O")
    _close(l2, l1, 0.0, "linearity LSE")


def pin_permutation(attn: Callable):
    """Permuting K and V rows together changes nothing; permuting Q rows
    permutes the output rows."""
    rng = np.random.default_rng(12)
    q, k, v = _rand(rng, 1, 13, 2, 8), _rand(rng, 1, 29, 2, 8), _rand(rng, 1, 29, 2, 8)
    o, lse = attn(q, k, v)
    pk = rng.permutation(29)
    o2, l2 = attn(q, k[:, pk], v[:, pk])
    _close(o2, o, 1e-13, "K/V permutation O")
    _close(l2, lse, 1e-13, "K/V permutation LSE")
    pq = rng.permutation(13)
    o3, l3 = attn(q[:, pq], k, v)
    _close(o3, o[:, pq], 1e-14, "Q permutation O")
    _close(l3, lse[:, :, pq], 1e-14, "Q permutation LSE")


def pin_key_shift(attn: Callable):
    """Adding the same vector u to every key adds q.u*scale to each of row i's
    scores: O is unchanged and LSE moves by exactly that amount."""
    rng = np.random.default_rng(13)
    q, k, v = _rand(rng, 1, 11, 2, 16), _rand(rng, 1, 19, 2, 16), _rand(rng, 1, 19, 2, 16)
    u = _rand(rng, 1, 1, 2, 16, s=4.0)
    o1, l1 = attn(q, k, v)
    o2, l2 = attn(q, k + u, v)
    shift = np.einsum("bihd,bjhd->bhi", q, u) / 4.0
    _close(o2, o1, 1e-12, "key shift O")
    _close(l2, l1 + shift, 1e-12, "key shift LSE")


def pin_scale(attn: Callable):
    """The scale argument multiplies the scores; 1/sqrt(D) is the default."""
    rng = np.random.default_rng(14)
    q, k, v = _rand(rng, 1, 7, 1, 16), _rand(rng, 1, 9, 1, 16), _rand(rng, 1, 9, 1, 16)
    o1, l1 = attn(q, k, v)
    o2, l2 = attn(q, k, v, scale=0.25)
    _close(o2, o1, 0.0, "default scale O")
    _close(l2, l1, 0.0, "default scale LSE")
    o3, l3 = attn(2.0 * q, k, v, scale=0.125)
    _close(o3, o1, 1e-14, "scale argument O")
    _close(l3, l1, 1e-14, "scale argument LSE")


def pin_empty(attn: Callable):
    """No keys: O = 0, LSE = -inf; no query rows: empty outputs."""
    rng = np.random.default_rng(15)
    q = _rand(rng, 1, 4, 2, 8)
    o, lse = attn(q, np.zeros((1, 0, 2, 8)), np.zeros((1, 0, 2, 8)))
    assert o.shape == (1, 4, 2, 8) and lse.shape == (1, 2, 4)
    assert (o == 0).all() and np.isneginf(lse).all(), "empty K/V"
    o, lse = attn(np.zeros((1, 0, 2, 8)), _rand(rng, 1, 5, 2, 8), _rand(rng, 1, 5, 2, 8))
    assert o.shape == (1, 0, 2, 8) and lse.shape == (1, 2, 0)


ATTENTION_PINS = (pin_brute_force, pin_golden, pin_single_key, pin_zero_keys,
                  pin_constant_v, pin_two_keys, pin_linearity, pin_permutation,
                  pin_key_shift, pin_scale, pin_empty)


# -------------------------------------------------------------------- merge

def pin_merge_golden(merge: Callable):
    g = _golden("merge_two_parts.json")
    os_, ls = [], []
    for p in g["parts"]:
        os_.append(np.array(p["o"]).reshape(1, 1, 1, 2))
        ls.append(np.array(float(p["lse"])).reshape(1, 1, 1))
    o, lse = merge(os_[:2], ls[:2])
    _close(o[0, 0, 0], g["o"], 1e-15, "merge golden O")
    _close(lse[0, 0, 0], g["lse"], 1e-15, "merge golden LSE")
    for order in ([0, 1, 2], [2, 0, 1], [0, 2, 1]):
        o, lse = merge([os_[i] for i in order], [ls[i] for i in order])
        _close(o[0, 0, 0], g["o"], 1e-15, f"merge golden O with empty part {order}")
        _close(lse[0, 0, 0], g["lse"], 1e-15, f"merge golden LSE with empty part {order}")


def pin_merge_identities(merge: Callable):
    rng = np.random.default_rng(16)
    o = _rand(rng, 2, 5, 3, 4)
    L = _rand(rng, 2, 3, 5, s=3.0)
    o1, l1 = merge([o], [L])
    _close(o1, o, 0.0, "merge of one part O")
    _close(l1, L, 0.0, "merge of one part LSE")
    o2, l2 = merge([o, o], [L, L])
    _close(o2, o, 1e-14, "merge of a duplicate O")
    _close(l2, L + math.log(2.0), 1e-14, "merge of a duplicate LSE")
    empty_o = np.zeros_like(o)
    empty_l = np.full_like(L, -np.inf)
    o3, l3 = merge([empty_o, empty_o], [empty_l, empty_l])
    assert (o3 == 0).all() and np.isneginf(l3).all(), "merge of empty parts"
    # unequal masses: part weights must be e^{L_c - L}
    L2 = L - 2.0
    oo = _rand(rng, 2, 5, 3, 4)
    o4, l4 = merge([o, oo], [L, L2])
    w1 = 1.0 / (1.0 + math.exp(-2.0))
    _close(o4, w1 * o + (1 - w1) * oo, 1e-14, "merge weights O")
    _close(l4, L + math.log1p(math.exp(-2.0)), 1e-14, "merge weights LSE")


def pin_chunked_equals_full(attn: Callable, merge: Callable, bounds: Callable):
    """Cutting K/V into chunks and merging the partials gives the unchunked
    result, for any cut: size-1 chunks, empty chunks, uneven chunks."""
    rng = np.random.default_rng(17)
    q, k, v = (_rand(rng, 2, S, 3, 8, s=2.0) for S in (11, 23, 23))
    o_ref, l_ref = attn(q, k, v)
    cuts = [[23], [1] * 23, [0, 23], [5, 0, 18], [7, 7, 7, 2], [22, 1],
            [0, 0, 23, 0], None]
    for sizes in cuts:
        n = len(sizes) if sizes is not None else 8
        parts_o, parts_l = [], []
        for (a, b) in bounds(23, n, sizes):
            oc, lc = attn(q, k[:, a:b], v[:, a:b])
            parts_o.append(oc)
            parts_l.append(lc)
        o, lse = merge(parts_o, parts_l)
        _close(o, o_ref, 1e-13, f"chunked {sizes} O")
        _close(lse, l_ref, 1e-13, f"chunked {sizes} LSE")


MERGE_PINS = (pin_merge_golden, pin_merge_identities)


# ------------------------------------------------------------------- chunks

def pin_chunk_bounds(bounds: Callable):
    assert bounds(4645, 8) == [(0, 581), (581, 1162), (1162, 1743), (1743, 2324),
                               (2324, 2905), (2905, 3485), (3485, 4065),
                               (4065, 4645)], "ring-anything split of 4645 into 8"
    assert bounds(4608, 8) == [(576 * c, 576 * (c + 1)) for c in range(8)]
    assert bounds(256, 4) == [(0, 64), (64, 128), (128, 192), (192, 256)]
    assert bounds(3, 5) == [(0, 1), (1, 2), (2, 3), (3, 3), (3, 3)]
    for S in range(0, 40):
        for n in range(1, 10):
            b = bounds(S, n)
            sizes = [y - x for x, y in b]
            assert len(b) == n and b[0][0] == 0 and b[-1][1] == S
            assert all(b[i][1] == b[i + 1][0] for i in range(n - 1))
            assert max(sizes) - min(sizes) <= 1
            assert sizes == sorted(sizes, reverse=True)


# ------------------------------------------------------------------ layouts

def pin_layout(s2h: Callable, h2s: Callable):
    g = _golden("ulysses_index_map.json")
    x = np.array(g["x"])
    y = s2h(x, g["P"])
    assert y.shape == np.array(g["y"]).shape and (y == np.array(g["y"])).all(), \
        "seq2head golden map"
    assert (h2s(y, g["P"]) == x).all(), "head2seq golden map"
    rng = np.random.default_rng(18)
    for (B, S, H, D, P) in [(2, 3, 6, 2, 3), (1, 5, 4, 3, 2), (2, 2, 8, 1, 8), (1, 4, 5, 2, 1)]:
        x = rng.standard_normal((B, S, H, D))
        y = s2h(x, P)
        Hp = H // P
        assert y.shape == (P, B, S, Hp, D)
        for p in range(P):
            for b in range(B):
                for s in range(S):
                    for j in range(Hp):
                        for d in range(D):
                            assert y[p, b, s, j, d] == x[b, s, p * Hp + j, d], \
                                "seq2head index map"
        back = h2s(y, P)
        assert back.shape == x.shape and (back.view(np.uint64) == x.view(np.uint64)).all(), \
            "round trip not bit-exact"


def pin_ulysses_share(attn: Callable, s2h: Callable):
    """Attention per head is independent of the other heads, so group p's share
    is heads [p*H/P, (p+1)*H/P) of the full result."""
    rng = np.random.default_rng(19)
    q, k, v = (_rand(rng, 2, 14, 6, 8) for _ in range(3))
    o, lse = attn(q, k, v)
    for P in (1, 2, 3, 6):
        Hp = 6 // P
        for p in range(P):
            qs, ks, vs = (s2h(a, P)[p] for a in (q, k, v))
            os_, ls = attn(qs, ks, vs)
            _close(os_, o[:, :, p * Hp:(p + 1) * Hp], 1e-14, f"ulysses share O P={P}")
            _close(ls, lse[:, p * Hp:(p + 1) * Hp], 1e-14, f"ulysses share LSE P={P}")


def pin_head_groups(groups: Callable, to_seq: Callable, s2h: Callable):
    """Near-equal head groups: sizes worked out by hand, every index checked
    by a loop, a bit-exact round trip, and the seq2head groups when P | H."""
    rng = np.random.default_rng(21)
    # 30 heads over 4 groups: 30 = 4*7 + 2, so the first two groups hold 8;
    # 3 heads over 5 groups: one head each for three, two empty groups
    for (H, P, sizes) in [(30, 4, [8, 8, 7, 7]), (3, 5, [1, 1, 1, 0, 0]), (7, 3, [3, 2, 2]),
                          (6, 3, [2, 2, 2]), (5, 1, [5])]:
        B, S, D = 2, 3, 2
        x = rng.standard_normal((B, S, H, D))
        gs = groups(x, P)
        assert [g.shape[2] for g in gs] == sizes, f"group sizes H={H} P={P}"
        h0 = 0
        for g in gs:
            assert g.shape[:2] == (B, S) and g.shape[3] == D
            for b in range(B):
                for s in range(S):
                    for j in range(g.shape[2]):
                        for d in range(D):
                            assert g[b, s, j, d] == x[b, s, h0 + j, d], "head group index map"
            h0 += g.shape[2]
        back = to_seq(gs)
        assert back.shape == x.shape and (back.view(np.uint64) == x.view(np.uint64)).all(), \
            "group round trip not bit-exact"
        if H % P == 0:
            y = s2h(x, P)
            for p in range(P):
                assert (y[p] == gs[p]).all(), "groups differ from seq2head for P | H"


def pin_ulysses_anything_share(attn: Callable, groups: Callable):
    """Attention per head does not depend on the other heads, so group p's
    share is its heads of the full result, whatever the group sizes."""
    rng = np.random.default_rng(22)
    q, k, v = (_rand(rng, 2, 11, 7, 8) for _ in range(3))
    o, lse = attn(q, k, v)
    for P in (2, 3, 4, 5):
        h0 = 0
        for p in range(P):
            qs, ks, vs = (groups(a, P)[p] for a in (q, k, v))
            hp = qs.shape[2]
            os_, ls = attn(qs, ks, vs)
            _close(os_, o[:, :, h0:h0 + hp], 1e-14, f"ulysses anything share O P={P}")
            _close(ls, lse[:, h0:h0 + hp], 1e-14, f"ulysses anything share LSE P={P}")
            h0 += hp
        assert h0 == 7


def pin_usp(attn: Callable, usp_attention: Callable, usp_share: Callable):
    """Unified attention reaches the plain result: the full composition
    equals attention to fp64 rounding, and device (u, r)'s share is rows of
    chunk r and heads of group u of it."""
    rng = np.random.default_rng(23)
    B, S, H, D = 2, 24, 6, 8
    q, k, v = (_rand(rng, B, S, H, D, s=1.5) for _ in range(3))
    o, lse = attn(q, k, v)
    for (Pu, Pr) in [(1, 1), (2, 2), (3, 2), (2, 4), (6, 4), (1, 3)]:
        ou, lu = usp_attention(q, k, v, Pu, Pr)
        _close(ou, o, 1e-12, f"usp O {Pu}x{Pr}")
        _close(lu, lse, 1e-12, f"usp LSE {Pu}x{Pr}")
    Pu, Pr = 3, 4
    Hp, n = H // Pu, S // Pr
    for u in range(Pu):
        for r in range(Pr):
            os_, ls = usp_share(q, k, v, Pu, Pr, u, r)
            _close(os_, o[:, r * n:(r + 1) * n, u * Hp:(u + 1) * Hp], 1e-12, "usp share O")
            _close(ls, lse[:, u * Hp:(u + 1) * Hp, r * n:(r + 1) * n], 1e-12, "usp share LSE")
    try:
        usp_share(q, k, v, 2, 5, 0, 0)          # 24 rows do not shard over 10 devices
    except ValueError:
        pass
    else:
        raise AssertionError("usp share accepted S not divisible by the mesh")
