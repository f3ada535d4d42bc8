"""fp64 CPU oracle for context-parallel attention (test infrastructure).

This file is test infrastructure.  Only the tests, the smoke entry point and
the CPU-baseline leg of the benchmark may import or run it; the product path
(the HIP library and its Python binding) never touches it and shares no code
with it.

Every function is the plain definition of what the path computes, written
with numpy float64 arrays.  Tensors are [B, S, H, D]; the per-row log-sum-exp
(LSE) is [B, H, S].  Sources (the pages this follows):

* diffusers "Attention backends" page, "Available backends" table: the
  default ``native`` backend is PyTorch's scaled_dot_product_attention, i.e.
  O = softmax(Q K^T / sqrt(D)) V per (batch, head), non-causal, no mask.
* diffusers "Parallelism" API page, ContextParallelConfig, ``convert_to_fp32``:
  ring attention carries an output *and* its LSE per step.
* diffusers "Context parallelism" guide, "Ring Attention" section: each
  device attends its Q to one K/V block after another until it has seen all
  of them; "Ring Anything Attention" section: blocks of unequal length.
* same guide, "Ulysses Attention" section: an all-to-all regroups the data so
  a device holds every token of a subset of heads, and a second one regroups
  the results by token; "Ulysses Anything Attention" section: the head count
  and sequence length need not divide by the degree.
* same guide, "Unified Attention" section: on a 2-D mesh of ulysses_degree x
  ring_degree devices, the Ulysses all-to-all regroups heads and tokens, ring
  attention runs on the result, and the reverse all-to-all restores the
  layout.

Readings where the pages are silent (each is also listed in the design
notes): the softmax scale is 1/sqrt(D); LSE is the natural log; uneven
chunks give the first S mod N chunks one extra row; partial results are
folded in ascending chunk order; an empty chunk contributes O = 0 and
LSE = -inf and is skipped by the merge.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = ["attention", "chunk_bounds", "merge_closed_form", "merge_fold",
           "chunked_attention", "ring_share", "seq2head", "head2seq",
           "ulysses_share", "head_groups", "groups_to_seq", "ulysses_anything_share",
           "usp_share", "usp_attention"]

NEG_INF = -np.inf


def _check4(name: str, a: np.ndarray) -> None:
    if a.ndim != 4:
        raise ValueError(f"{name} must be [B, S, H, D], got shape {a.shape}")


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              scale: Optional[float] = None,
              row_block: int = 512) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention with its per-row LSE, in float64.

    For every batch b, head h and query row i:
        s_ij = scale * <q_i, k_j>           (scale defaults to 1/sqrt(D))
        LSE_i = log sum_j exp(s_ij)
        O_i = sum_j exp(s_ij - LSE_i) v_j
    evaluated stably as m = max_j s_ij, p_ij = exp(s_ij - m),
    l = sum_j p_ij, O_i = (p v)_i / l, LSE_i = m + log l.
    With no keys, O_i = 0 and LSE_i = -inf.

    Query rows are independent, so they are evaluated ``row_block`` at a
    time only to bound memory.  Returns (O [B,Sq,H,D], LSE [B,H,Sq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    for name, a in (("q", q), ("k", k), ("v", v)):
        _check4(name, a)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != (B, Skv, H, D) or v.shape != (B, Skv, H, D):
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = np.zeros((B, Sq, H, D), dtype=np.float64)
    lse = np.full((B, H, Sq), NEG_INF, dtype=np.float64)
    if Skv == 0 or Sq == 0:
        return o, lse
    for b in range(B):
        for h in range(H):
            kt = k[b, :, h, :].T            # [D, Skv]
            vh = v[b, :, h, :]              # [Skv, D]
            for i0 in range(0, Sq, row_block):
                i1 = min(Sq, i0 + row_block)
                s = (q[b, i0:i1, h, :] @ kt) * scale       # [rows, Skv]
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                o[b, i0:i1, h, :] = (p @ vh) / l
                lse[b, h, i0:i1] = m[:, 0] + np.log(l[:, 0])
    return o, lse


def chunk_bounds(S: int, n: int,
                 sizes: Optional[Sequence[int]] = None) -> List[Tuple[int, int]]:
    """Split rows [0, S) into n consecutive chunks.

    With ``sizes`` given they are used as they are (they must sum to S);
    otherwise the split is near-equal: chunk c has S // n rows plus one more
    when c < S mod n, so sizes differ by at most one and a divisible S gives
    equal chunks (the "Ring Anything" reading).
    """
    if n < 1:
        raise ValueError("n must be >= 1")
    if sizes is None:
        base, extra = divmod(S, n)
        sizes = [base + (1 if c < extra else 0) for c in range(n)]
    sizes = [int(x) for x in sizes]
    if len(sizes) != n or any(x < 0 for x in sizes) or sum(sizes) != S:
        raise ValueError(f"bad chunk sizes {sizes} for S={S}, n={n}")
    bounds, start = [], 0
    for x in sizes:
        bounds.append((start, start + x))
        start += x
    return bounds


def merge_closed_form(o_parts: Sequence[np.ndarray],
                      lse_parts: Sequence[np.ndarray]
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """Combine partial results over disjoint key sets in one step.

    With M = max_c LSE_c:  LSE = M + log sum_c exp(LSE_c - M),
                           O   = sum_c exp(LSE_c - LSE) O_c.
    This is exact: exp(LSE_c - LSE) * exp(s_j - LSE_c) = exp(s_j - LSE), so
    the weight each key gets is its weight in the unchunked softmax.
    Rows where every LSE_c is -inf (no keys at all) give O = 0, LSE = -inf.
    o_parts: [B,S,H,D] each; lse_parts: [B,H,S] each.
    """
    if len(o_parts) == 0 or len(o_parts) != len(lse_parts):
        raise ValueError("need one LSE per partial output, at least one")
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lse_parts])  # [N,B,H,S]
    O = np.stack([np.asarray(x, dtype=np.float64) for x in o_parts])    # [N,B,S,H,D]
    M = L.max(axis=0)                                                   # [B,H,S]
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    with np.errstate(invalid="ignore"):
        total = np.exp(L - Ms[None]).sum(axis=0)
    lse = np.where(finite, Ms + np.log(np.where(finite, total, 1.0)), NEG_INF)
    w = np.where(finite[None], np.exp(L - np.where(finite, lse, 0.0)[None]), 0.0)
    # w is [N,B,H,S]; move it to O's [N,B,S,H] row order
    w = np.transpose(w, (0, 1, 3, 2))[..., None]
    o = (w * O).sum(axis=0)
    return o, lse


def merge_fold(o_parts: Sequence[np.ndarray],
               lse_parts: Sequence[np.ndarray]
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Fold partial results one at a time, in ascending order, as a ring does.

    Start from (O_0, L_0); for each next (O_c, L_c):
        L' = log(exp(L) + exp(L_c))   (computed as m + log(e^(L-m) + e^(L_c-m)),
                                       m = max(L, L_c))
        O  <- exp(L - L') O + exp(L_c - L') O_c,  L <- L'.
    A part with L_c = -inf is skipped; while L = -inf the next part is taken
    as it is.
    """
    if len(o_parts) == 0 or len(o_parts) != len(lse_parts):
        raise ValueError("need one LSE per partial output, at least one")
    o = np.array(o_parts[0], dtype=np.float64, copy=True)
    L = np.array(lse_parts[0], dtype=np.float64, copy=True)
    for oc, Lc in zip(o_parts[1:], lse_parts[1:]):
        oc = np.asarray(oc, dtype=np.float64)
        Lc = np.asarray(Lc, dtype=np.float64)
        a_fin = np.isfinite(L)
        c_fin = np.isfinite(Lc)
        m = np.where(a_fin, np.maximum(L, np.where(c_fin, Lc, L)), Lc)
        m = np.where(np.isfinite(m), m, 0.0)
        ea = np.where(a_fin, np.exp(np.where(a_fin, L, 0.0) - m), 0.0)
        ec = np.where(c_fin, np.exp(np.where(c_fin, Lc, 0.0) - m), 0.0)
        tot = ea + ec
        any_fin = a_fin | c_fin
        Lnew = np.where(any_fin, m + np.log(np.where(any_fin, tot, 1.0)), NEG_INF)
        wa = np.where(any_fin, ea / np.where(any_fin, tot, 1.0), 0.0)
        wc = np.where(any_fin, ec / np.where(any_fin, tot, 1.0), 0.0)
        wa = np.transpose(wa, (0, 2, 1))[..., None]   # [B,H,S] -> [B,S,H,1]
        wc = np.transpose(wc, (0, 2, 1))[..., None]
        o = wa * o + wc * oc
        L = Lnew
    return o, L


def chunked_attention(q, k, v, n_chunks: int,
                      sizes: Optional[Sequence[int]] = None,
                      scale: Optional[float] = None, merge: str = "fold"
                      ) -> Tuple[np.ndarray, np.ndarray]:
    """All query rows against K/V cut into chunks, partials merged.

    Each chunk's partial is ``attention`` restricted to that chunk's key rows;
    the partials are combined by ``merge_fold`` (ascending order) or
    ``merge_closed_form``.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    parts_o, parts_l = [], []
    for (a, b) in chunk_bounds(k.shape[1], n_chunks, sizes):
        oc, lc = attention(q, k[:, a:b], v[:, a:b], scale=scale)
        parts_o.append(oc)
        parts_l.append(lc)
    fn = merge_fold if merge == "fold" else merge_closed_form
    return fn(parts_o, parts_l)


def ring_share(q, k, v, n_chunks: int, rank: int,
               sizes: Optional[Sequence[int]] = None,
               scale: Optional[float] = None, merge: str = "fold"
               ) -> Tuple[np.ndarray, np.ndarray]:
    """One ring rank's share: its own Q rows against every K/V chunk.

    The rank's Q rows are chunk ``rank`` of the same split that cuts K/V
    (each device holds one slice of the sequence); its result must equal those
    rows of the full attention.
    """
    q = np.asarray(q, dtype=np.float64)
    a, b = chunk_bounds(q.shape[1], n_chunks, sizes)[rank]
    return chunked_attention(q[:, a:b], k, v, n_chunks, sizes, scale, merge)


def seq2head(x: np.ndarray, P: int) -> np.ndarray:
    """The net effect of Ulysses' first all-to-all, on one device.

    [B, S, H, D] -> [P, B, S, H/P, D] with y[p, b, s, j, d] = x[b, s, p*H/P + j, d]:
    group p holds every token of heads [p*H/P, (p+1)*H/P).
    """
    x = np.asarray(x)
    B, S, H, D = x.shape
    if H % P:
        raise ValueError(f"H={H} not divisible by P={P}")
    return np.ascontiguousarray(
        x.reshape(B, S, P, H // P, D).transpose(2, 0, 1, 3, 4))


def head2seq(y: np.ndarray, P: int) -> np.ndarray:
    """The inverse of ``seq2head``: [P, B, S, H/P, D] -> [B, S, H, D]."""
    y = np.asarray(y)
    Pn, B, S, Hp, D = y.shape
    if Pn != P:
        raise ValueError(f"leading dim {Pn} != P={P}")
    return np.ascontiguousarray(y.transpose(1, 2, 0, 3, 4).reshape(B, S, P * Hp, D))


def ulysses_share(q, k, v, P: int, p: int, scale: Optional[float] = None
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """One Ulysses rank's share: attention over heads group p at full length."""
    qs, ks, vs = (seq2head(a, P)[p] for a in (q, k, v))
    return attention(qs, ks, vs, scale=scale)


def head_groups(x: np.ndarray, P: int) -> List[np.ndarray]:
    """Ulysses Anything's first all-to-all, on one device: the heads cut into
    P consecutive groups by the near-equal rule of ``chunk_bounds`` (the first
    H mod P groups hold one head more; groups may be empty when P > H); group
    p is [B, S, Hp_p, D] with every token.  For H divisible by P the groups
    are those of ``seq2head``."""
    x = np.asarray(x)
    _check4("x", x)
    return [np.ascontiguousarray(x[:, :, a:b]) for a, b in chunk_bounds(x.shape[2], P)]


def groups_to_seq(groups: Sequence[np.ndarray]) -> np.ndarray:
    """The inverse of ``head_groups``: the groups' heads back in order."""
    return np.ascontiguousarray(np.concatenate(list(groups), axis=2))


def ulysses_anything_share(q, k, v, P: int, p: int, scale: Optional[float] = None
                           ) -> Tuple[np.ndarray, np.ndarray]:
    """One Ulysses Anything rank's share: attention over head group p."""
    qs, ks, vs = (head_groups(a, P)[p] for a in (q, k, v))
    return attention(qs, ks, vs, scale=scale)


def usp_share(q, k, v, ulysses_degree: int, ring_degree: int, ulysses_rank: int,
              ring_rank: int, scale: Optional[float] = None, merge: str = "fold"
              ) -> Tuple[np.ndarray, np.ndarray]:
    """The share of device (u, r) of Unified attention on a ulysses_degree x
    ring_degree mesh: after the Ulysses regrouping it holds head group u of
    every token, and the ring over ring_degree sequence chunks gives it the
    query rows of chunk r.  The sequence is sharded over the whole mesh, so
    S must divide by ulysses_degree * ring_degree."""
    q = np.asarray(q, dtype=np.float64)
    S = q.shape[1]
    if S % (ulysses_degree * ring_degree):
        raise ValueError(f"S={S} not divisible by {ulysses_degree} x {ring_degree}")
    qs, ks, vs = (seq2head(a, ulysses_degree)[ulysses_rank] for a in (q, k, v))
    return ring_share(qs, ks, vs, ring_degree, ring_rank, scale=scale, merge=merge)


def usp_attention(q, k, v, ulysses_degree: int, ring_degree: int,
                  scale: Optional[float] = None, merge: str = "fold"
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Every device's Unified-attention share, put back in place by the
    reverse all-to-all: the [B, S, H, D] output and the [B, H, S] LSE."""
    q = np.asarray(q, dtype=np.float64)
    B, S, H, D = q.shape
    Hp = H // ulysses_degree
    o_groups = np.zeros((ulysses_degree, B, S, Hp, D))
    lse = np.full((B, H, S), NEG_INF)
    for u in range(ulysses_degree):
        for r, (a, b) in enumerate(chunk_bounds(S, ring_degree)):
            o, l = usp_share(q, k, v, ulysses_degree, ring_degree, u, r, scale, merge)
            o_groups[u, :, a:b] = o
            lse[:, u * Hp:(u + 1) * Hp, a:b] = l
    return head2seq(o_groups, ulysses_degree), lse
