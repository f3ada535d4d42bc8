"""The C-ABI library loads, exports what include/cru.h declares, and rejects bad
arguments on the host (no GPU needed: every check runs before any HIP call,
and the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import context_ring_ulysses_amd as cru
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cru.h")

OK, EINVAL, ENOTDIV, EUNSUPPORTED, EDEVICE, EWORKSPACE, EHIP = range(7)
FAKE = 1 << 20           # 16-byte aligned, never dereferenced


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cru_[a-z0-9_]+)\s*\(", text)))


def T(B=1, S=16, H=2, D=64, dtype=cru.BF16, data=FAKE, strides=None):
    if strides is None:
        strides = (S * H * D, H * D, D)
    return cru.CruTensor(data, dtype, 0, B, S, H, D, *strides)


def L(B=1, H=2, S=16, data=FAKE):
    return cru.CruLse(data, B, H, S, H * S, S)


def last_error():
    return cru.lib().cru_last_error().decode()


def test_exports_every_declared_symbol():
    syms = declared_symbols()
    assert "cru_attn_fwd_lse" in syms and len(syms) >= 10
    L_ = cru.lib()
    for s in syms:
        assert hasattr(L_, s), f"{s} declared in cru.h but not exported"


def test_abi_version_and_status_strings():
    L_ = cru.lib()
    assert L_.cru_abi_version() == 2
    names = [L_.cru_status_str(i).decode() for i in range(7)]
    assert names == ["CRU_OK", "CRU_EINVAL", "CRU_ENOTDIV", "CRU_EUNSUPPORTED",
                     "CRU_EDEVICE", "CRU_EWORKSPACE", "CRU_EHIP"]
    assert L_.cru_status_str(99).decode() == "CRU_UNKNOWN"


def fwd(q, k, v, o, lse=None, scale=0.0):
    return cru.lib().cru_attn_fwd_lse(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                      ctypes.byref(o), None if lse is None else ctypes.byref(lse),
                                      ctypes.c_float(scale), None)


@pytest.mark.parametrize("case,expect", [
    ("k head dim differs", EINVAL),
    ("v length differs from k", EINVAL),
    ("o shape differs", EINVAL),
    ("head dim 96", EUNSUPPORTED),
    ("mixed dtypes", EUNSUPPORTED),
    ("fp32 in, bf16 out", EUNSUPPORTED),
    ("unknown dtype", EUNSUPPORTED),
    ("misaligned data", EINVAL),
    ("stride not a vector multiple", EINVAL),
    ("negative size", EINVAL),
    ("null data", EINVAL),
    ("negative scale", EINVAL),
    ("nan scale", EINVAL),
    ("lse shape", EINVAL),
    ("reserved field", EINVAL),
])
def test_attn_fwd_validation(case, expect):
    q, k, v, o = T(), T(S=24), T(S=24), T()
    lse, scale = None, 0.0
    if case == "k head dim differs":
        k = T(S=24, D=128)
    elif case == "v length differs from k":
        v = T(S=23)
    elif case == "o shape differs":
        o = T(S=17)
    elif case == "head dim 96":
        q, k, v, o = T(D=96), T(S=24, D=96), T(S=24, D=96), T(D=96)
    elif case == "mixed dtypes":
        k = T(S=24, dtype=cru.F32)
    elif case == "fp32 in, bf16 out":
        q, k, v = T(dtype=cru.F32), T(S=24, dtype=cru.F32), T(S=24, dtype=cru.F32)
    elif case == "unknown dtype":
        q = T(dtype=7)
    elif case == "misaligned data":
        q = T(data=FAKE + 2)
    elif case == "stride not a vector multiple":
        q = T(strides=(16 * 2 * 64, 2 * 64 + 4, 64))
    elif case == "negative size":
        q = T(S=-1)
    elif case == "null data":
        q = T(data=0)
    elif case == "negative scale":
        scale = -1.0
    elif case == "nan scale":
        scale = float("nan")
    elif case == "lse shape":
        lse = L(S=15)
    elif case == "reserved field":
        q = T()
        q.reserved = 1
    st = fwd(q, k, v, o, lse, scale)
    assert st == expect, (case, st, last_error())
    assert last_error() != ""


def test_sizes_whose_product_overflows_are_rejected():
    # every size is within 2^30, but their product is far above any tensor
    # (and above 2^63): refused before any product of sizes is formed
    huge = dict(B=1 << 30, S=1 << 30, H=1 << 10, D=64, strides=(8, 8, 8))
    q = T(**huge)
    assert fwd(q, T(S=24), T(S=24), T()) == EINVAL
    assert "2^48" in last_error()
    assert merge([T(dtype=cru.F32, **huge)], [L()], T()) == EINVAL
    need = ctypes.c_size_t(0)
    assert cru.lib().cru_ring_workspace_bytes(ctypes.byref(q), 4, ctypes.byref(need)) == EINVAL
    assert s2h([q], 2) == EINVAL
    assert h2s([q], 2) == EINVAL
    # just under the cap is accepted by the size check (these fail later, on
    # the fake pointer or the per-call index range)
    ok = T(B=1 << 18, S=1 << 12, H=1 << 12, D=64, strides=(8, 8, 8))
    assert fwd(ok, T(S=24), T(S=24), T()) == EINVAL
    assert "2^48" not in last_error()


def test_views_reaching_past_2_60_elements_are_refused():
    # the sizes are small but a stride is huge: the largest offset the view
    # reaches would leave no headroom in the kernels' 64-bit offsets
    far = T(B=2, strides=(1 << 61, 2 * 64, 64))
    assert fwd(far, T(S=24), T(S=24), T()) == EINVAL
    assert "2^60" in last_error()
    assert fwd(T(B=2), T(B=2, S=24), T(B=2, S=24), far) == EINVAL
    assert "2^60" in last_error()
    assert h2s([far], 2) == EINVAL
    assert "2^60" in last_error()
    # strides whose sum of offsets would pass 2^63 (no wrap-around: refused)
    wrap = T(B=4, S=2, H=2, strides=((1 << 62) + 64, 1 << 61, 64))
    assert fwd(T(B=4, S=2), T(B=4, S=24), T(B=4, S=24), wrap) == EINVAL
    assert "2^60" in last_error()
    lse = cru.CruLse(FAKE, 2, 2, 16, 1 << 61, 16)
    assert fwd(T(B=2), T(B=2, S=24), T(B=2, S=24), T(B=2), lse) == EINVAL
    assert "2^60" in last_error()
    # just under the limit passes the host checks (stops at the fake pointer)
    near = T(B=2, strides=((1 << 59), 2 * 64, 64))
    assert fwd(near, T(B=2, S=24), T(B=2, S=24), T(B=2)) == EDEVICE, last_error()


def test_valid_call_reaches_device_check_without_gpu():
    # well-formed arguments pass every host check; the fake pointer is then
    # rejected as not being device memory (or there is no device here)
    st = fwd(T(), T(S=24), T(S=24), T(), L())
    assert st == EDEVICE, last_error()


def test_broadcast_and_overlapping_inputs_pass_host_checks():
    # inputs may repeat elements: k and v broadcast along the sequence
    # (stride 0, what torch's expand() gives) or rows that overlap (stride
    # below D); such calls pass every host check and stop at the fake pointer
    q = T()
    kb = T(S=24, strides=(0, 0, 64))
    assert fwd(q, kb, kb, T(), L()) == EDEVICE, last_error()
    kover = T(S=24, strides=(24 * 8 + 64 * 2, 8, 64))
    assert fwd(q, kover, kover, T(), L()) == EDEVICE, last_error()
    qb = T(strides=(0, 0, 0))
    assert fwd(qb, T(S=24), T(S=24), T(), L()) == EDEVICE, last_error()


@pytest.mark.parametrize("strides", [(16 * 2 * 64, 0, 64), (16 * 2 * 64, 64, 64),
                                     (16 * 2 * 64, 2 * 64, 32), (16 * 2 * 64, 2 * 64, 0)])
def test_overlapping_outputs_are_refused(strides):
    # an output whose elements share addresses would have threads race on
    # them: refused with CRU_EINVAL before anything is enqueued
    o = T(strides=strides)
    assert fwd(T(), T(S=24), T(S=24), o) == EINVAL
    assert "overlap" in last_error()
    assert merge([T(dtype=cru.F32)], [L()], o) == EINVAL
    assert h2s([T(S=16, H=2, strides=strides)], 2) == EINVAL


def test_overlapping_lse_is_refused():
    lse = cru.CruLse(FAKE, 1, 2, 16, 2 * 16, 8)       # heads 8 apart, rows of 16
    assert fwd(T(), T(S=24), T(S=24), T(), lse) == EINVAL
    assert "overlap" in last_error()
    lse = cru.CruLse(FAKE, 2, 2, 16, 16, 16)          # batch 1 lands on head 1
    assert fwd(T(B=2), T(B=2, S=24), T(B=2, S=24), T(B=2), lse) == EINVAL
    # head-major or padded layouts are fine
    lse = cru.CruLse(FAKE, 2, 2, 16, 16, 32)          # [H, B, S] storage
    assert fwd(T(B=2), T(B=2, S=24), T(B=2, S=24), T(B=2), lse) == EDEVICE, last_error()


def test_empty_query_is_a_no_op():
    st = fwd(T(S=0, data=0), T(S=24), T(S=24), T(S=0, data=0), L(S=0, data=0))
    assert st == OK, last_error()


def merge(parts, lparts, o, lse=None, n=None):
    n = len(parts) if n is None else n
    P = (cru.CruTensor * max(1, len(parts)))(*parts)
    Lp = (cru.CruLse * max(1, len(lparts)))(*lparts)
    return cru.lib().cru_attn_merge_lse(n, P, Lp, ctypes.byref(o),
                                        None if lse is None else ctypes.byref(lse), None)


def test_merge_validation():
    part = T(dtype=cru.F32)
    assert merge([part], [L()], T(), n=0) == EINVAL
    assert merge([part], [L()], T(), n=cru.MAX_PARTS + 1) == EINVAL
    assert merge([T()], [L()], T()) == EDEVICE                         # bf16 partials pass
    assert merge([part, T()], [L(), L()], T()) == EUNSUPPORTED         # mixed part dtypes
    assert merge([part, T(S=17, dtype=cru.F32)], [L(), L()], T()) == EINVAL
    odd = T(dtype=cru.F32, strides=(16 * 2 * 64 * 2, 2 * 64, 64))
    assert merge([part, odd], [L(), L()], T()) == EINVAL               # strides differ
    assert merge([part], [L(S=3)], T()) == EINVAL
    assert merge([part], [L()], T(S=3)) == EINVAL
    assert merge([T(D=32, dtype=cru.F32)], [L()], T(D=32)) == EUNSUPPORTED
    assert merge([part, part], [L(), L()], T(), L()) == EDEVICE, last_error()


def bounds(S, n, anything):
    starts = (ctypes.c_int64 * (n + 1))()
    st = cru.lib().cru_ring_chunk_bounds(S, n, anything, starts)
    return st, [(starts[c], starts[c + 1]) for c in range(n)]


def test_chunk_bounds_match_the_oracle_split():
    for S in (0, 1, 7, 64, 256, 4608, 4645):
        for n in (1, 2, 3, 4, 8, 13):
            st, b = bounds(S, n, 1)
            assert st == OK
            assert b == oracle.chunk_bounds(S, n)
    assert cru.ring_chunk_bounds(4645, 8, anything=True)[0] == (0, 581)


def test_chunk_bounds_divisibility():
    assert bounds(4645, 8, 0)[0] == ENOTDIV          # plain ring needs S % N == 0
    assert "not divisible" in last_error()
    assert bounds(4608, 8, 0)[0] == OK
    assert bounds(10, 0, 1)[0] == EINVAL
    assert bounds(10, cru.MAX_PARTS + 1, 1)[0] == EINVAL
    with pytest.raises(cru.CruNotDivisible):
        cru.ring_chunk_bounds(4481, 4)               # FLUX 1008x1008 on 4 devices


def ring(q, k, v, n, anything=0, sizes=None, fused=0, o=None, ws=FAKE * 4, ws_bytes=1 << 40,
         fp32=1):
    o = o or T(S=q.S, D=q.D, dtype=q.dtype)
    arr = None if sizes is None else (ctypes.c_int64 * len(sizes))(*sizes)
    return cru.lib().cru_ring_emulate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), n,
                                      anything, arr, fused, fp32, ctypes.byref(o), None,
                                      ctypes.c_float(0.0), ws, ws_bytes, None)


def test_ring_validation():
    q, k, v = T(S=10), T(S=37), T(S=37)
    assert ring(q, k, v, 8) == ENOTDIV                       # 37 % 8
    assert ring(q, k, v, 8, anything=1) == EDEVICE           # Ring Anything passes host checks
    assert ring(q, k, v, 2, sizes=[20, 17]) == ENOTDIV       # unequal needs anything
    assert ring(q, k, v, 2, anything=1, sizes=[20, 17]) == EDEVICE
    assert ring(q, k, v, 2, anything=1, sizes=[20, 16]) == EINVAL   # sum != Skv
    assert ring(q, k, v, 2, anything=1, sizes=[38, -1]) == EINVAL
    # sizes whose int64 sum wraps around to Skv are refused chunk by chunk
    big = (1 << 63) - 1
    assert ring(q, k, v, 3, anything=1, sizes=[big, big, 39]) == EINVAL
    assert "pass the 37 K/V rows" in last_error()
    assert ring(q, k, v, 3, anything=1, sizes=[10, 30, -3]) == EINVAL
    assert ring(q, k, v, 0) == EINVAL
    assert ring(q, k, v, 1, anything=2) == EINVAL
    assert ring(q, k, v, 1, fused=3) == EINVAL
    assert ring(q, k, v, 1, ws=0) == EWORKSPACE
    assert ring(q, k, v, 1, ws=FAKE + 16) == EWORKSPACE      # not 256-byte aligned
    need = ctypes.c_size_t(0)
    assert cru.lib().cru_ring_workspace_bytes(ctypes.byref(q), 4, ctypes.byref(need)) == OK
    rows = 1 * 10 * 2
    a256 = lambda x: (x + 255) // 256 * 256
    assert need.value == 4 * (a256(rows * 64 * 4) + a256(rows * 4))
    assert ring(q, k, v, 4, anything=1, ws_bytes=need.value - 1) == EWORKSPACE
    assert ring(q, k, v, 4, anything=1, ws_bytes=need.value) == EDEVICE
    # fp32 inputs take the fp32 path; bf16 output for them is refused
    qf, kf, vf = T(S=10, dtype=cru.F32), T(S=36, dtype=cru.F32), T(S=36, dtype=cru.F32)
    assert ring(qf, kf, vf, 4, o=T(S=10)) == EUNSUPPORTED
    # bf16 partials (convert_to_fp32 off): bf16 inputs only
    assert ring(q, k, v, 4, anything=1, fp32=0) == EDEVICE
    assert ring(qf, kf, vf, 4, fp32=0, o=T(S=10, dtype=cru.F32)) == EUNSUPPORTED
    assert ring(q, k, v, 4, anything=1, fp32=2) == EINVAL


def ring_na(q, k, v, n, anything=0, fused=0, fp32=1):
    o = T(S=q.S, H=q.H, D=q.D, dtype=q.dtype)
    return cru.lib().cru_ring_emulate_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                              n, anything, None, fused, fp32, ctypes.byref(o),
                                              None, ctypes.c_float(0.0), None)


def test_ring_noalloc_validation():
    # the same host checks as cru_ring_emulate, then the scratch size limit,
    # all before any device call (the fake pointers stop it at the device check)
    q, k, v = T(S=10), T(S=37), T(S=37)
    assert ring_na(q, k, v, 8) == ENOTDIV
    assert ring_na(q, k, v, 8, anything=1) == EDEVICE, last_error()
    # 8 fp32 partials of 1024 x 24 x 128 need 8 * 12.6 MB > 64 MiB
    big_q = T(S=1024, H=24, D=128)
    big_kv = T(S=8192, H=24, D=128)
    assert ring_na(big_q, big_kv, big_kv, 8) == EWORKSPACE
    assert "static scratch" in last_error()
    # FLUX-1024's ring share (576 rows x 24 heads, 8 chunks) fits
    share = T(S=576, H=24, D=128)
    kv = T(S=4608, H=24, D=128)
    assert ring_na(share, kv, kv, 8) == EDEVICE, last_error()


def s2h(xs, P, ys=None, anything=0):
    n = len(xs)
    X = (cru.CruTensor * n)(*xs)
    Y = (ctypes.c_void_p * n)(*(ys or [FAKE * 8] * n))
    return cru.lib().cru_ulysses_seq2head(n, X, Y, P, anything, None)


def h2s(xs, P, ys=None, anything=0):
    n = len(xs)
    X = (cru.CruTensor * n)(*xs)
    Y = (ctypes.c_void_p * n)(*(ys or [FAKE * 8] * n))
    return cru.lib().cru_ulysses_head2seq(n, Y, X, P, anything, None)


def test_ulysses_validation():
    x = T(S=16, H=6)
    assert s2h([x], 4) == ENOTDIV                 # 6 heads over 4 devices
    assert "head count" in last_error()
    assert s2h([T(S=15, H=6)], 2) == ENOTDIV      # 15 tokens over 2 devices
    assert "sequence length" in last_error()
    assert s2h([x], 0) == EINVAL
    assert s2h([x] * 9, 2) == EINVAL
    assert s2h([x, T(S=16, H=6, dtype=cru.F32)], 2) == EINVAL
    assert s2h([x], 2, ys=[FAKE + 8]) == EINVAL   # misaligned output
    assert s2h([x], 2) == EDEVICE                 # passes host checks
    assert h2s([x], 4) == ENOTDIV
    assert h2s([x], 2) == EDEVICE
    # Ulysses Anything: uneven heads and tokens pass the host checks
    assert s2h([x], 4, anything=1) == EDEVICE
    assert s2h([T(S=15, H=6)], 2, anything=1) == EDEVICE
    assert h2s([T(S=15, H=7)], 3, anything=1) == EDEVICE
    assert s2h([x], 7, anything=1) == EDEVICE     # more groups than heads: some are empty
    assert s2h([x], 2, anything=2) == EINVAL


def head_bounds(H, P, anything):
    starts = (ctypes.c_int64 * (P + 1))()
    st = cru.lib().cru_ulysses_head_bounds(H, P, anything, starts)
    return st, [(starts[p], starts[p + 1]) for p in range(P)]


def test_head_bounds():
    assert head_bounds(24, 2, 0) == (OK, [(0, 12), (12, 24)])
    assert head_bounds(30, 4, 0)[0] == ENOTDIV
    assert head_bounds(30, 4, 1) == (OK, [(0, 8), (8, 16), (16, 23), (23, 30)])
    assert head_bounds(3, 5, 1) == (OK, [(0, 1), (1, 2), (2, 3), (3, 3), (3, 3)])
    assert head_bounds(8, 0, 1)[0] == EINVAL
    for H in range(0, 40):
        for P in range(1, 9):
            st, b = head_bounds(H, P, 1)
            assert st == OK and b == oracle.chunk_bounds(H, P)   # the same near-equal rule
    assert cru.ulysses_head_bounds(30, 4, anything=True)[2] == (16, 23)


def usp(q, k, v, Pu, Pr, fused=0, o=None, ws=FAKE * 4, ws_bytes=1 << 40, fp32=1):
    o = o or T(S=q.S, H=q.H, D=q.D, dtype=q.dtype)
    return cru.lib().cru_usp_emulate(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), Pu, Pr,
                                     fused, fp32, ctypes.byref(o), None, ctypes.c_float(0.0), ws,
                                     ws_bytes, None)


def test_usp_validation():
    q = T(S=16, H=4)
    assert usp(q, q, q, 2, 2) == EDEVICE                     # passes host checks
    assert usp(T(S=16, H=6), T(S=16, H=6), T(S=16, H=6), 4, 2) == ENOTDIV   # H % Pu
    assert usp(T(S=12, H=4), T(S=12, H=4), T(S=12, H=4), 2, 4) == ENOTDIV   # S % (Pu Pr)
    assert "ulysses_degree * ring_degree" in last_error()
    assert usp(q, T(S=8, H=4), T(S=8, H=4), 2, 2) == EINVAL  # one sequence: Skv == Sq
    assert usp(q, q, q, 0, 2) == EINVAL
    assert usp(q, q, q, 2, 0) == EINVAL
    assert usp(q, q, q, 2, 2, fused=2) == EINVAL
    assert usp(q, q, q, 2, 2, fp32=0) == EDEVICE
    assert usp(q, q, q, 2, 2, fp32=5) == EINVAL
    assert usp(q, q, q, 2, 2, ws=0) == EWORKSPACE
    need = ctypes.c_size_t(0)
    assert cru.lib().cru_usp_workspace_bytes(ctypes.byref(q), 2, 2, ctypes.byref(need)) == OK
    a256 = lambda x: (x + 255) // 256 * 256
    elems = 1 * 16 * 4 * 64
    rows_g = 1 * 16 * 2
    # the three regrouped inputs and one ring workspace of fp32 partials (the
    # groups' results are stored straight into o)
    assert need.value == 3 * a256(elems * 2) + 2 * (a256(rows_g * 64 * 4) + a256(rows_g * 4))
    assert usp(q, q, q, 2, 2, ws_bytes=need.value - 1) == EWORKSPACE
    assert usp(q, q, q, 2, 2, ws_bytes=need.value) == EDEVICE


def test_config_rules():
    C = cru.ContextParallelConfig
    C(ring_degree=8)
    C(ulysses_degree=2)
    C(ring_degree=2, ulysses_degree=2)
    C(ring_degree=8, ring_anything=True)
    with pytest.raises(ValueError):
        C(ring_degree=0)
    with pytest.raises(ValueError):
        C(ring_degree=2, ulysses_degree=2, ring_anything=True)
    with pytest.raises(ValueError):
        C(ring_degree=1, ring_anything=True)
    with pytest.raises(ValueError):
        C(ulysses_degree=2, ring_degree=2, ulysses_anything=True)
    C(ulysses_degree=4, ulysses_anything=True)
    C(ring_degree=2, convert_to_fp32=False)


def test_binding_rejects_bad_tensors_before_the_library():
    import torch
    with pytest.raises(cru.CruInvalid):
        cru.attn_fwd_lse(torch.zeros(2, 3, 4), torch.zeros(2, 3, 4), torch.zeros(2, 3, 4))
    with pytest.raises(cru.CruUnsupported):
        z = torch.zeros(1, 4, 2, 64, dtype=torch.float16)
        cru.attn_fwd_lse(z, z, z)
    with pytest.raises(cru.CruInvalid):
        z = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16)[..., ::2]
        cru.attn_fwd_lse(z, z, z)
