"""cru_ring_emulate_noalloc (partials in the library's static scratch array)
against cru_ring_emulate with a caller workspace, through the C ABI."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import context_ring_ulysses_amd as cru
import oracle
from workloads import random_qkv, to_f64

pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 2e-2, 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def noalloc(qs, k, v, n, *, anything=0, fused=0, fp32=1, out_dtype=None):
    """One call of the C entry point; outputs allocated here, before the call."""
    o = torch.empty(qs.shape, dtype=out_dtype or qs.dtype, device=qs.device)
    lse = torch.empty(qs.shape[0], qs.shape[2], qs.shape[1], dtype=torch.float32,
                      device=qs.device)
    L = cru.lib()
    st = L.cru_ring_emulate_noalloc(
        cru._desc(qs, "q_share"), cru._desc(k, "k"), cru._desc(v, "v"), n, anything, None,
        fused, fp32, cru._desc(o, "out"), cru._ref(cru._lse_desc(lse, "lse")),
        ctypes.c_float(0.0), cru._stream(qs))
    cru._check(st)
    return o, lse


@pytest.mark.parametrize("fused", [0, 1])
def test_noalloc_matches_workspace_entry_point_twice(fused):
    # first call: FLUX-1024's ring rank-3 share shape at reduced heads
    # (576 rows x 8 chunks of 576, 6 heads); second call a smaller, ragged
    # one (uneven chunks, Ring Anything), so the scratch holds the first
    # call's partials when the second starts
    cases = [
        dict(seed=70, B=1, S=4608, H=6, D=128, N=8, rank=3, anything=0, fp32=1),
        dict(seed=71, B=2, S=1001, H=3, D=64, N=5, rank=4, anything=1, fp32=0),
    ]
    for c in cases:
        q, k, v = random_qkv(c["seed"], c["B"], c["S"], c["S"], c["H"], c["D"], gain=1.7)
        qd, kd, vd = (t.cuda() for t in (q, k, v))
        a, b = cru.ring_chunk_bounds(c["S"], c["N"], anything=bool(c["anything"]))[c["rank"]]
        say(f"noalloc fused={fused}: {c}")
        o_ref, l_ref = cru.ring_emulate(qd[:, a:b], kd, vd, c["N"], anything=bool(c["anything"]),
                                        fused=bool(fused), convert_to_fp32=bool(c["fp32"]))
        o_na, l_na = noalloc(qd[:, a:b], kd, vd, c["N"], anything=c["anything"], fused=fused,
                             fp32=c["fp32"])
        torch.cuda.synchronize()
        # the same kernels on the same partials: bit-identical
        assert torch.equal(o_na, o_ref) and torch.equal(l_na, l_ref)
        # and within the bars of the oracle's ring share
        o64, l64 = oracle.ring_share(to_f64(q), to_f64(k), to_f64(v), c["N"], c["rank"])
        tol_o = TOL_O if c["fp32"] else TOL_O + 2.0 ** -8 * float(v.float().abs().max())
        eo = float(np.abs(to_f64(o_na) - o64).max())
        el = float(np.abs(to_f64(l_na) - l64).max())
        say(f"  max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}")
        assert eo <= tol_o and el <= TOL_LSE


def test_noalloc_refuses_shares_beyond_the_scratch():
    # 8 chunks of fp32 partials for 1024 rows x 24 heads x 128 dims need
    # 8 * 12.6 MB: over the 64 MiB array, refused before anything runs
    q = torch.empty(1, 1024, 24, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(1, 8192, 24, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cru.CruWorkspaceError, match="static scratch"):
        noalloc(q, k, k, 8)
