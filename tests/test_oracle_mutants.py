"""Plant a mistake in a copy of the oracle and check that some pin catches it.

Each mutant is one textual change to oracle/attention.py (a dropped term, a
wrong sign, axis, index or operand); the changed source is executed into a
fresh namespace, the real oracle is untouched.  The test passes only when at
least one pin fails on the mutant, which shows the pins constrain that line.
"""
import importlib
import types

import numpy as np
import pytest

import pins

# the package re-exports the function ``attention``, so fetch the module itself
_MOD = importlib.import_module("oracle.attention")
with open(_MOD.__file__) as _f:
    SRC = _f.read()

MUTANTS = [
    # attention
    ("attn: scale dropped", "@ kt) * scale", "@ kt)"),
    ("attn: scale inverted", "scale = 1.0 / math.sqrt(D)", "scale = math.sqrt(D)"),
    ("attn: max over the wrong axis", "m = s.max(axis=1, keepdims=True)",
     "m = s.max(axis=0, keepdims=True)"),
    ("attn: LSE without the max", "lse[b, h, i0:i1] = m[:, 0] + np.log(l[:, 0])",
     "lse[b, h, i0:i1] = np.log(l[:, 0])"),
    ("attn: LSE in base 2", "m[:, 0] + np.log(l[:, 0])", "m[:, 0] + np.log2(l[:, 0])"),
    ("attn: no normalisation", "(p @ vh) / l", "(p @ vh)"),
    ("attn: sign of the shift", "p = np.exp(s - m)", "p = np.exp(m - s)"),
    ("attn: V used as K", "kt = k[b, :, h, :].T", "kt = v[b, :, h, :].T"),
    ("attn: wrong head of V", "vh = v[b, :, h, :]", "vh = v[b, :, 0, :]"),
    ("attn: empty LSE not -inf", "lse = np.full((B, H, Sq), NEG_INF",
     "lse = np.full((B, H, Sq), 0.0"),
    ("attn: row block skips a row", "for i0 in range(0, Sq, row_block):\n                i1 = min(Sq, i0 + row_block)",
     "for i0 in range(0, Sq, row_block):\n                i1 = min(Sq - 1, i0 + row_block) if Sq > 1 else Sq"),
    # in-order fold
    ("fold: sign of the first weight", "ea = np.where(a_fin, np.exp(np.where(a_fin, L, 0.0) - m), 0.0)",
     "ea = np.where(a_fin, np.exp(m - np.where(a_fin, L, 0.0)), 0.0)"),
    ("fold: dropped new part", "o = wa * o + wc * oc", "o = wa * o"),
    ("fold: LSE without the max", "Lnew = np.where(any_fin, m + np.log(",
     "Lnew = np.where(any_fin, np.log("),
    ("fold: unnormalised weights", "wc = np.where(any_fin, ec / np.where(any_fin, tot, 1.0), 0.0)",
     "wc = np.where(any_fin, ec, 0.0)"),
    # closed-form merge
    ("closed: sign of the weights", "np.exp(L - np.where(finite, lse, 0.0)[None])",
     "np.exp(np.where(finite, lse, 0.0)[None] - L)"),
    ("closed: LSE without the max", "lse = np.where(finite, Ms + np.log(",
     "lse = np.where(finite, np.log("),
    ("closed: weights on the wrong axes", "w = np.transpose(w, (0, 1, 3, 2))[..., None]",
     "w = w[..., None]"),
    # chunking
    ("bounds: extra rows to the last chunks", "(1 if c < extra else 0)",
     "(1 if c >= n - extra else 0)"),
    ("bounds: overlapping chunks", "bounds.append((start, start + x))",
     "bounds.append((max(0, start - 1), start + x))"),
    # layouts
    ("seq2head: heads split the wrong way", "x.reshape(B, S, P, H // P, D).transpose(2, 0, 1, 3, 4)",
     "x.reshape(B, S, H // P, P, D).transpose(3, 0, 1, 2, 4)"),
    ("head2seq: wrong inverse", "y.transpose(1, 2, 0, 3, 4)", "y.transpose(1, 2, 3, 0, 4)"),
    ("groups: one head too many", "x[:, :, a:b]) for a, b in chunk_bounds(x.shape[2], P)]",
     "x[:, :, a:b + 1]) for a, b in chunk_bounds(x.shape[2], P)]"),
    ("groups: inverse reverses the order", "np.concatenate(list(groups), axis=2)",
     "np.concatenate(list(groups)[::-1], axis=2)"),
    ("anything share: wrong group", "(head_groups(a, P)[p] for a in (q, k, v))",
     "(head_groups(a, P)[0] for a in (q, k, v))"),
    ("usp: wrong ring chunk", "return ring_share(qs, ks, vs, ring_degree, ring_rank, scale=scale, merge=merge)",
     "return ring_share(qs, ks, vs, ring_degree, 0, scale=scale, merge=merge)"),
    ("usp: output into the wrong group", "o_groups[u, :, a:b] = o", "o_groups[0, :, a:b] = o"),
    ("usp: LSE heads not offset", "lse[:, u * Hp:(u + 1) * Hp, a:b] = l", "lse[:, 0:Hp, a:b] = l"),
]


def _mutant_module(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _all_pins(m):
    checks = [lambda p=p: p(m.attention) for p in pins.ATTENTION_PINS]
    for merge in (m.merge_fold, m.merge_closed_form):
        checks += [lambda p=p, mg=merge: p(mg) for p in pins.MERGE_PINS]
        checks.append(lambda mg=merge: pins.pin_chunked_equals_full(m.attention, mg, m.chunk_bounds))
    checks.append(lambda: pins.pin_chunk_bounds(m.chunk_bounds))
    checks.append(lambda: pins.pin_layout(m.seq2head, m.head2seq))
    checks.append(lambda: pins.pin_ulysses_share(m.attention, m.seq2head))
    checks.append(lambda: pins.pin_head_groups(m.head_groups, m.groups_to_seq, m.seq2head))
    checks.append(lambda: pins.pin_ulysses_anything_share(m.attention, m.head_groups))
    checks.append(lambda: pins.pin_usp(m.attention, m.usp_attention, m.usp_share))
    checks.append(lambda: _anything_share_check(m))
    return checks


def _anything_share_check(m):
    # the named share function against the groups' own attention
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 9, 5, 4)) for _ in range(3))
    o, l = m.ulysses_anything_share(q, k, v, 2, 1)
    o_ref, l_ref = m.attention(q[:, :, 3:], k[:, :, 3:], v[:, :, 3:])
    assert np.abs(o - o_ref).max() == 0 and np.abs(l - l_ref).max() == 0


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    m = _mutant_module(old, new)
    caught = []
    for check in _all_pins(m):
        try:
            check()
        except Exception as e:          # a failed pin or a crash both count
            caught.append(type(e).__name__)
            break
    assert caught, f"no pin caught the mutant: {name}"


def test_unmutated_copy_passes_every_pin():
    m = _mutant_module("NEG_INF = -np.inf", "NEG_INF = -np.inf")
    for check in _all_pins(m):
        check()
