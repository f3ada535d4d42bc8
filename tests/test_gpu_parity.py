"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Tolerances: fp32 inputs 1e-5 (max abs, O and LSE); bf16 inputs 2e-2 on O and
1e-3 on LSE against the oracle; layout shuffles bit-exact.  Where several
results are correct (a chunked sum rounds differently from an unchunked
one), two GPU results are compared with twice those bounds: each is within
the bound of the exact result, so they are within twice it of each other
(at |O| >= 4 one bf16 step is 2^-5, more than the single bound).  Where the
arithmetic is identical by construction (a head's attention does not depend
on which other heads share the launch, the step-wise and fused ring
schedules run the same per-chunk code) they are compared bit for bit.
"""
import functools
import math
import sys

import numpy as np
import pytest
import torch

import context_ring_ulysses_amd as cru
import oracle
from workloads import make_inputs, random_qkv, to_f64, workload

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_O = 2e-2
TOL_LSE = 1e-3
TOL_PAIR_O = 2 * TOL_O        # two GPU results, each within TOL_O of the oracle
TOL_PAIR_LSE = 2 * TOL_LSE


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    cru.lib()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both_ninf = np.isneginf(a) & np.isneginf(b)
    with np.errstate(invalid="ignore"):          # -inf - -inf, masked just below
        e = np.where(both_ninf, 0.0, np.abs(a - b))
    assert not np.isnan(e).any(), "NaN in comparison"
    return float(e.max()) if e.size else 0.0


def cuda(*ts):
    return [t.cuda() for t in ts]


@functools.lru_cache(maxsize=2)
def inputs(idx):
    q, k, v = make_inputs(idx)
    return (q, k, v), tuple(cuda(q, k, v))


@functools.lru_cache(maxsize=4)
def oracle_full(idx):
    """The oracle's attention over every row of a workload (fp64)."""
    (q, k, v), _ = inputs(idx)
    return oracle.attention(to_f64(q), to_f64(k), to_f64(v))


def check_all(o_gpu, l_gpu, o_ref, l_ref, tol_o, tol_l, what):
    """Every element of O and LSE against the oracle."""
    eo = err(to_f64(o_gpu), o_ref)
    el = err(to_f64(l_gpu), l_ref)
    say(f"  {what}: max|dO| = {eo:.3e}, max|dLSE| = {el:.3e} over all {o_ref.shape[1]} rows")
    assert eo <= tol_o, f"{what}: O error {eo}"
    assert el <= tol_l, f"{what}: LSE error {el}"


# ------------------------------------------------------------ fp32 (workload 1)

def test_fp32_tiny_full():
    (q, k, v), (qd, kd, vd) = inputs(1)
    say("tiny fp32 full forward", tuple(q.shape))
    o, l = cru.attn_fwd_lse(qd, kd, vd)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    assert err(to_f64(o), o_ref) <= TOL_F32
    assert err(to_f64(l), l_ref) <= TOL_F32


@pytest.mark.parametrize("D", [64, 128])
def test_fp32_several_tiles_ragged(D):
    # exact fp32 path past one tile both ways: 257 query rows (3 row tiles of
    # 128, the last with one row), 300 keys (10 key tiles of 32, the last
    # with 12), two batches, k given as a strided view
    q, k, v = random_qkv(17 + D, 2, 257, 300, 3, D, dtype="f32")
    kd = torch.empty(2, 300, 5, D).cuda()[:, :, 1:4]
    kd.copy_(k.cuda())
    assert not kd.is_contiguous()
    o, l = cru.attn_fwd_lse(q.cuda(), kd, v.cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    assert err(to_f64(o), o_ref) <= TOL_F32
    assert err(to_f64(l), l_ref) <= TOL_F32


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_fp32_tiny_ring_share(rank, fused):
    (q, k, v), (qd, kd, vd) = inputs(1)
    N = workload(1).ring_degree
    a, b = cru.ring_chunk_bounds(q.shape[1], N)[rank]
    say(f"tiny fp32 ring share rank {rank} of {N}, fused={fused}")
    o, l = cru.ring_emulate(qd[:, a:b], kd, vd, N, fused=fused)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.ring_share(to_f64(q), to_f64(k), to_f64(v), N, rank)
    assert err(to_f64(o), o_ref) <= TOL_F32
    assert err(to_f64(l), l_ref) <= TOL_F32


# --------------------------------------------- bf16, small sizes, every element

@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_ragged_full(D, out_dtype):
    # several query tiles and key tiles, with ragged tails on both
    q, k, v = random_qkv(100 + D, B=2, Sq=300, Skv=517, H=3, D=D, gain=math.sqrt(3.0))
    say(f"bf16 ragged D={D} out={out_dtype}")
    o, l = cru.attn_fwd_lse(*cuda(q, k, v), out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    eo, el = err(to_f64(o), o_ref), err(to_f64(l), l_ref)
    say(f"  max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}")
    assert eo <= TOL_O and el <= TOL_LSE


# The launch picks 8-, 4- or 2-wave workgroups (256, 128 or 64 query rows)
# by how many tiles the call has; on a 256-CU MI355X these head counts give
# each of the three shapes at Sq=300 (test_attn_shape.py checks the choice).
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("H,waves", [(128, 8), (150, 4), (8, 2)])
def test_bf16_workgroup_shapes(H, waves, D, out_dtype):
    q, k, v = random_qkv(300 + H + D, B=1, Sq=300, Skv=203, H=H, D=D, gain=math.sqrt(3.0))
    say(f"bf16 H={H} (expect {waves}-wave workgroups) D={D} out={out_dtype}")
    o, l = cru.attn_fwd_lse(*cuda(q, k, v), out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    check_all(o, l, o_ref, l_ref, TOL_O, TOL_LSE, f"H={H}, every head")


@pytest.mark.parametrize("shape", [(1, 10, 10, 8, 64), (1, 1, 1, 1, 128), (3, 1, 700, 2, 64),
                                   (1, 129, 65, 5, 128), (2, 257, 129, 1, 64)])
def test_bf16_odd_shapes(shape):
    B, Sq, Skv, H, D = shape
    q, k, v = random_qkv(7, B, Sq, Skv, H, D)
    say("bf16 shape", shape)
    o, l = cru.attn_fwd_lse(*cuda(q, k, v))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    assert err(to_f64(o), o_ref) <= TOL_O
    assert err(to_f64(l), l_ref) <= TOL_LSE


def test_strided_views_and_scale():
    # q, k, v as non-contiguous views ([B, H, S, D] storage) and an explicit scale
    q, k, v = random_qkv(8, 2, 150, 190, 4, 128)
    qd, kd, vd = (t.cuda().permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3) for t in (q, k, v))
    assert qd.stride(1) == 128 and not qd.is_contiguous()
    o, l = cru.attn_fwd_lse(qd, kd, vd, scale=0.05)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v), scale=0.05)
    assert err(to_f64(o), o_ref) <= TOL_O
    assert err(to_f64(l), l_ref) <= TOL_LSE


def _views(base, shape, strides, dev):
    """The same strided view of one buffer on the device and on the host."""
    return (torch.as_strided(base.to(dev), shape, strides),
            torch.as_strided(base, shape, strides))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_broadcast_and_overlapping_input_views(D, dtype):
    # Inputs whose elements repeat: K and V expand()-ed along the sequence
    # (stride 0: one key row seen Skv times), Q expanded likewise, and rows
    # that overlap (sequence stride 8 elements < D).  Every element against
    # the oracle on the same values made contiguous.
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    tol_o, tol_l = (TOL_O, TOL_LSE) if dtype == "bf16" else (TOL_F32, TOL_F32)
    g = torch.Generator().manual_seed(60 + D)
    B, Sq, Skv, H = 2, 200, 300, 3
    q, k, v = random_qkv(61 + D, B, Sq, Skv, H, D, gain=math.sqrt(3.0), dtype=dtype)
    cases = {}
    # k, v: one row per (b, h), broadcast over all 300 keys.  Every key then
    # gets the same weight and O = v exactly; in fp32 the kernel sums 300
    # equal terms for the numerator and for the denominator, each within
    # (Skv - 1) * 2^-24 relative, so O is within twice that of v (the bound
    # the constant-V test derives), above 1e-5 once |v| passes about 0.6
    k1 = k[:, :1].expand(B, Skv, H, D)
    v1 = v[:, :1].expand(B, Skv, H, D)
    assert k1.stride(1) == 0
    tol_rep = max(tol_o, 2 * (Skv - 1) * 2.0 ** -24 * float(v1.float().abs().max()))
    cases["k, v expand()-ed along S"] = (q.cuda(), k1.cuda(), v1.cuda(), q, k1, v1, tol_rep)
    # q broadcast as well (all query rows equal)
    q1 = q[:, :1].expand(B, Sq, H, D)
    cases["q, k, v expand()-ed along S"] = (q1.cuda(), k1.cuda(), v1.cuda(), q1, k1, v1,
                                            tol_rep)
    # overlapping rows: row s starts 8 elements after row s-1
    n = (Skv - 1) * 8 + D
    shape, strides = (B, Skv, H, D), (H * n, 8, n, 1)
    kb = torch.randn(B * H * n, generator=g).to(tdt)
    vb = torch.randn(B * H * n, generator=g).to(tdt)
    kd, kh = _views(kb, shape, strides, "cuda")
    vd, vh = _views(vb, shape, strides, "cuda")
    cases["k, v rows overlapping (stride 8)"] = (q.cuda(), kd, vd, q, kh, vh, tol_o)
    for what, (qd, kd, vd, qh, kh, vh, tol) in cases.items():
        say(f"{what}: D={D} {dtype}")
        o, l = cru.attn_fwd_lse(qd, kd, vd, out_dtype=torch.float32)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(to_f64(qh.contiguous()), to_f64(kh.contiguous()),
                                        to_f64(vh.contiguous()))
        check_all(o, l, o_ref, l_ref, tol, tol_l, what)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_degenerate_cases(dtype):
    q, k, v = random_qkv(9, 1, 70, 1, 2, 64, dtype=dtype)
    qd, kd, vd = cuda(q, k, v)
    say("degenerate cases", dtype)
    # one key: its weight is 1, so O = v_0 (up to the rounding of 1/l) and
    # LSE = its score
    o, l = cru.attn_fwd_lse(qd, kd, vd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    v0 = to_f64(v.float().expand(1, 70, 2, 64))
    assert err(to_f64(o), v0) <= 1e-6 * max(1.0, float(np.abs(v0).max()))
    s = np.einsum("bihd,bjhd->bhi", to_f64(q), to_f64(k)) / 8.0
    assert err(to_f64(l), s) <= (TOL_F32 if dtype == "f32" else TOL_LSE)
    # no keys: O = 0, LSE = -inf
    o, l = cru.attn_fwd_lse(qd, kd[:, :0], vd[:, :0], out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o.cpu() == 0).all() and torch.isneginf(l.cpu()).all()
    # no queries: nothing to do
    o, l = cru.attn_fwd_lse(qd[:, :0], kd, vd)
    torch.cuda.synchronize()
    assert o.shape == (1, 0, 2, 64) and l.shape == (1, 2, 0)


def test_constant_v_and_zero_k():
    q, k, v = random_qkv(10, 1, 200, 300, 2, 128, gain=math.sqrt(3.0))
    c = torch.randn(1, 1, 2, 128, generator=torch.Generator().manual_seed(0)).to(torch.bfloat16)
    vc = c.expand(1, 300, 2, 128).contiguous()
    o, _ = cru.attn_fwd_lse(*cuda(q, k, vc), out_dtype=torch.float32)
    ob, _ = cru.attn_fwd_lse(*cuda(q, k, vc))
    torch.cuda.synchronize()
    # O is normalised by the sum of the same bf16 P the P V product uses, so
    # the weights sum to one up to fp32 rounding of two 300-term sums of
    # positive values (each within 299 * 2^-24 relative): O = c to 4e-5 |c|,
    # and exactly c once rounded to bf16 (half a bf16 step is 2^-9 relative)
    assert err(to_f64(o), np.broadcast_to(to_f64(c), o.shape)) <= 4e-5 * float(c.abs().max())
    assert torch.equal(ob.cpu(), c.expand(1, 200, 2, 128))
    o, l = cru.attn_fwd_lse(*cuda(q, torch.zeros_like(k), v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert err(to_f64(o), np.broadcast_to(to_f64(v).mean(1, keepdims=True), o.shape)) <= 1e-5
    assert err(to_f64(l), np.full(l.shape, math.log(300))) <= 1e-5


@pytest.mark.parametrize("D", [64, 128])
def test_identity_v_gives_probabilities(D):
    # V = identity: O[i, j] is exactly the weight key j gets in row i, so any
    # pairing of a score with the wrong value row shows up column by column
    # (the LSE alone cannot see it: it does not depend on the key order)
    q, k, _ = random_qkv(15, 1, 160, D, 2, D, gain=2.0)
    v = torch.zeros(1, D, 2, D, dtype=torch.bfloat16)
    for j in range(D):
        v[0, j, :, j] = 1.0
    o, _ = cru.attn_fwd_lse(*cuda(q, k, v), out_dtype=torch.float32)
    torch.cuda.synchronize()
    s = np.einsum("bihd,bjhd->bhij", to_f64(q), to_f64(k)) / math.sqrt(D)
    p = np.exp(s - s.max(-1, keepdims=True))
    p /= p.sum(-1, keepdims=True)
    got = np.transpose(to_f64(o), (0, 2, 1, 3))          # [b, h, i, j]
    assert err(got, p) <= 4e-3                           # bf16 rounding of P


# --------------------------------------------------------------------- merge

@pytest.mark.parametrize("n", [1, 2, 5, 8, 13, 17, 40])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("part_dtype", [torch.float32, torch.bfloat16])
def test_merge_kernel(part_dtype, out_dtype, n):
    g = torch.Generator().manual_seed(11 + n)
    shape = (2, 333, 3, 128) if n <= 8 else (1, 77, 2, 64)
    # the oracle merges exactly the values the GPU reads (bf16 parts upcast)
    parts = [torch.randn(shape, generator=g).to(part_dtype) for _ in range(n)]
    B, S, H, _ = shape
    lses = [torch.randn(B, H, S, generator=g) * 4 for _ in range(n)]
    lses[n // 2][:, :, :50] = -float("inf")     # one part empty for some rows
    parts[n // 2][:, :50] = float("nan")        # ... whose O must then be ignored
    for c in range(n):
        lses[c][B - 1, H - 1, 7] = -float("inf")   # a row with no keys at all
        parts[c][B - 1, 7, H - 1] = 0.0
    o, l = cru.attn_merge_lse([p.cuda() for p in parts], [x.cuda() for x in lses],
                              out_dtype=out_dtype)
    torch.cuda.synchronize()
    ref_parts = [p.double().numpy() for p in parts]
    assert parts[0].dtype == part_dtype
    ref_parts[n // 2] = np.nan_to_num(ref_parts[n // 2])   # the oracle weights them by 0
    o_ref, l_ref = oracle.merge_closed_form(ref_parts, [x.double().numpy() for x in lses])
    tol = TOL_F32 if out_dtype == torch.float32 else TOL_O
    assert err(to_f64(o), o_ref) <= tol
    assert err(to_f64(l), l_ref) <= TOL_F32
    assert torch.isneginf(l[B - 1, H - 1, 7]).item() and (o[B - 1, 7, H - 1] == 0).all().item()


# ------------------------------------------- adversarial softmax and long rows

def _ramp_inputs(seed, S, D, slope, B=1, H=2):
    """Keys along one direction with growing weight, so every query's logits
    climb along the keys and the running max moves at every tile."""
    g = torch.Generator().manual_seed(seed)
    u = torch.randn(D, generator=g)
    u = u / u.norm()
    q = (u * math.sqrt(D)).expand(B, S, H, D).clone() + 0.05 * torch.randn(B, S, H, D, generator=g)
    ramp = torch.linspace(0.0, slope, S).view(1, S, 1, 1)
    k = ramp * u.view(1, 1, 1, D) + 0.05 * torch.randn(B, S, H, D, generator=g)
    v = torch.randn(B, S, H, D, generator=g)
    return tuple(t.to(torch.bfloat16) for t in (q, k, v))


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("slope", [20.0, 200.0])
def test_running_max_moves_every_tile(D, slope):
    # logits rise by up to slope*sqrt(D)/sqrt(D) = slope over the keys, and
    # the last tile's keys dominate.  The kernel moves its running max only
    # when a half-row's sum of a tile's P passes 2^32: at slope 200 (about 36
    # log2 units per 64-key tile) every tile takes that path, at slope 20 a
    # few do and the rest run far above the first tile's max
    q, k, v = _ramp_inputs(7, 517, D, slope)
    o, l = cru.attn_fwd_lse(*cuda(q, k, v))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    eo, el = err(to_f64(o), o_ref), err(to_f64(l), l_ref)
    say(f"ramp D={D} slope={slope}: max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}, LSE range "
        f"[{l_ref.min():.1f}, {l_ref.max():.1f}]")
    assert eo <= TOL_O and el <= TOL_LSE


@pytest.mark.parametrize("scale_to", [300.0, -300.0, 1e-4])
def test_extreme_logit_ranges(scale_to):
    # all logits near +-300 (exp of the raw value would overflow fp32) or
    # nearly zero (uniform weights); the max shift must keep P in range
    g = torch.Generator().manual_seed(13)
    B, S, H, D = 1, 200, 2, 128
    q = torch.randn(B, S, H, D, generator=g)
    k = torch.randn(B, S, H, D, generator=g)
    v = torch.randn(B, S, H, D, generator=g)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    # s = scale * q.k with |q| = 1, |k| = |scale_to| / scale, k along +-q for half the keys
    k[:, ::2] = q[:, ::2].sign() * q[:, ::2].abs()
    k = k * (abs(scale_to) * math.sqrt(D))
    if scale_to < 0:
        k = -k
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, l = cru.attn_fwd_lse(*cuda(q, k, v))
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(l).all().item()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    assert err(to_f64(o), o_ref) <= TOL_O
    # |s| reaches 300 here: the fp32 sum of D products in the MFMA rounds by
    # at most D * 2^-24 * max|s|, which the LSE inherits
    assert err(to_f64(l), l_ref) <= TOL_LSE + D * 2.0 ** -24 * 300.0


@pytest.mark.parametrize("vscale_log2", [80, 90])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_large_v_near_the_sum_cap(vscale_log2, out_dtype):
    # The running max moves only when a half-row's running sum of P would
    # pass 2^32, so O's accumulator can reach about 2^33 * max|V|.  Here the
    # first key tile has logits near 0 and every later key about 17.5: tiles
    # 1 and 2 add about 2^30.9 each to a half-row's sum without a move (the
    # logits fix that sum: 32 keys of 2^(17.5 log2 e - m) each), tile 3
    # forces one.  With V scaled
    # by 2^90 (exact in bf16, max|V| about 2^92) the accumulator reaches
    # about 2^125, below the fp32 limit; O / 2^s must match the oracle.
    g = torch.Generator().manual_seed(15)
    B, Sq, Skv, H, D = 1, 40, 640, 2, 128
    q1 = torch.randn(B, 1, H, D, generator=g)
    q1 = q1 / q1.norm(dim=-1, keepdim=True)
    q = q1.expand(B, Sq, H, D).contiguous() + 0.01 * torch.randn(B, Sq, H, D, generator=g)
    k = torch.randn(B, Skv, H, D, generator=g) * 0.01
    k[:, 64:] += q1 * (17.5 * math.sqrt(D))
    v = torch.randn(B, Skv, H, D, generator=g) * 2.0 ** vscale_log2
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, l = cru.attn_fwd_lse(*cuda(q, k, v), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(l).all().item()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v) / 2.0 ** vscale_log2)
    assert err(to_f64(o) / 2.0 ** vscale_log2, o_ref) <= TOL_O
    # logits reach about 17.5 (plus a bf16 rounding of q and k): the fp32
    # score sum rounds by at most D * 2^-24 * 18, which the LSE inherits
    assert err(to_f64(l), l_ref) <= TOL_LSE


def test_dominant_last_key_in_ragged_tile():
    # one key, the last of a ragged final tile, outweighs all others by e^40
    g = torch.Generator().manual_seed(14)
    B, S, H, D = 1, 131, 3, 64
    q = torch.randn(B, 70, H, D, generator=g)
    k = torch.randn(B, S, H, D, generator=g) * 0.1
    v = torch.randn(B, S, H, D, generator=g)
    k[:, S - 1] = q[:, 0] / q[:, 0].norm(dim=-1, keepdim=True) * 40.0 * math.sqrt(D) / \
        q[:, 0].norm(dim=-1, keepdim=True)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o, l = cru.attn_fwd_lse(*cuda(q, k, v))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    assert err(to_f64(o), o_ref) <= TOL_O and err(to_f64(l), l_ref) <= TOL_LSE


@pytest.mark.parametrize("D", [64, 128])
def test_long_sequence_all_rows(D):
    # 40000 keys: index arithmetic well past 2^16 rows, 625 key tiles; every
    # row against the oracle, which runs 2500 query rows at a time
    B, S, H = 1, 40000, 2
    q, k, v = random_qkv(500 + D, B=B, Sq=S, Skv=S, H=H, D=D, gain=math.sqrt(3.0))
    say(f"long sequence S={S} D={D}")
    o, l = cru.attn_fwd_lse(*cuda(q, k, v))
    torch.cuda.synchronize()
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o64, l64 = to_f64(o), to_f64(l)
    eo = el = 0.0
    for a in range(0, S, 2500):
        o_ref, l_ref = oracle.attention(q64[:, a:a + 2500], k64, v64)
        eo = max(eo, err(o64[:, a:a + 2500], o_ref))
        el = max(el, err(l64[:, :, a:a + 2500], l_ref))
    say(f"  S={S} D={D}: max|dO| = {eo:.3e}, max|dLSE| = {el:.3e} over all {S} rows")
    assert eo <= TOL_O and el <= TOL_LSE


# Batch strides past 2^31 elements: every batch offset needs 64-bit address
# arithmetic in the kernels.  The views sit in 4-9 GB device buffers of which
# only the used rows are written or read.
BIG_SB = (1 << 31) + 12288


def _big_view(x, dtype, sb=BIG_SB):
    """A [B, S, H, D] device view of x (CPU) whose batch stride is sb elements."""
    B, S, H, D = x.shape
    buf = torch.empty((B - 1) * sb + S * H * D, dtype=dtype, device="cuda")
    for b in range(B):
        buf[b * sb: b * sb + S * H * D].copy_(x[b].reshape(-1).to(dtype))
    return torch.as_strided(buf, (B, S, H, D), (sb, H * D, D, 1))


def _big_empty(shape, dtype, sb=BIG_SB):
    B, S, H, D = shape
    buf = torch.empty((B - 1) * sb + S * H * D, dtype=dtype, device="cuda")
    return torch.as_strided(buf, shape, (sb, H * D, D, 1))


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_attention_batch_stride_past_2_31(dtype):
    B, S, H, D = 2, 200, 2, 128
    q, k, v = random_qkv(41, B=B, Sq=S, Skv=S, H=H, D=D, gain=math.sqrt(3.0),
                         dtype="bf16" if dtype == torch.bfloat16 else "f32")
    say(f"attention ({dtype}) with batch strides of {BIG_SB} elements")
    qd, kd, vd = (_big_view(t, dtype) for t in (q, k, v))
    o = _big_empty((B, S, H, D), dtype)
    lbuf = torch.empty((B - 1) * BIG_SB + H * S, dtype=torch.float32, device="cuda")
    l = torch.as_strided(lbuf, (B, H, S), (BIG_SB, S, 1))
    cru.attn_fwd_lse(qd, kd, vd, out=o, lse=l)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    o_h = torch.stack([o[b].cpu() for b in range(B)])
    l_h = torch.stack([l[b].cpu() for b in range(B)])
    del qd, kd, vd, o, l, lbuf
    _free()
    bf16 = dtype == torch.bfloat16
    assert err(to_f64(o_h), o_ref) <= (TOL_O if bf16 else TOL_F32)
    assert err(to_f64(l_h), l_ref) <= (TOL_LSE if bf16 else TOL_F32)


def test_merge_batch_stride_past_2_31():
    B, S, H, D, n = 2, 150, 3, 128, 3
    g = torch.Generator().manual_seed(42)
    parts = [torch.randn(B, S, H, D, generator=g) for _ in range(n)]
    lses = [torch.randn(B, H, S, generator=g) * 4 for _ in range(n)]
    say(f"merge of {n} fp32 parts with batch strides of {BIG_SB} elements")
    pd = [_big_view(x, torch.float32) for x in parts]
    o = _big_empty((B, S, H, D), torch.bfloat16)
    cru.attn_merge_lse(pd, [x.cuda() for x in lses], out=o)
    torch.cuda.synchronize()
    o_h = torch.stack([o[b].cpu() for b in range(B)])
    del pd, o
    _free()
    o_ref, _ = oracle.merge_closed_form([x.double().numpy() for x in parts],
                                        [x.double().numpy() for x in lses])
    assert err(to_f64(o_h), o_ref) <= TOL_O


def test_layouts_batch_stride_past_2_31():
    B, S, H, D, P = 2, 96, 6, 64, 3
    x = torch.randn(B, S, H, D, generator=torch.Generator().manual_seed(43)).to(torch.bfloat16)
    say(f"seq2head/head2seq with batch strides of {BIG_SB} elements")
    xd = _big_view(x, torch.bfloat16)
    y = cru.ulysses_seq2head(xd, P)
    back = _big_empty((B, S, H, D), torch.bfloat16)
    cru.ulysses_head2seq(y, P, out=back)
    torch.cuda.synchronize()
    y_h = y.cpu()
    back_h = torch.stack([back[b].cpu() for b in range(B)])
    del xd, y, back
    _free()
    assert np.array_equal(y_h.view(torch.int16).numpy(), oracle.seq2head(x.view(torch.int16).numpy(), P))
    assert torch.equal(back_h.view(torch.int16), x.view(torch.int16))


# -------------------------------------------------------- layouts, bit-exact

@pytest.mark.parametrize("idx", [2, 5])
def test_ulysses_layouts_bit_exact(idx):
    w = workload(idx)
    (q, k, v), (qd, kd, vd) = inputs(idx)
    P = w.ulysses_degree
    say(f"seq2head/head2seq {w.name} P={P}")
    ys = cru.ulysses_seq2head([qd, kd, vd], P)
    torch.cuda.synchronize()
    for y, x in zip(ys, (q, k, v)):
        ref = oracle.seq2head(x.view(torch.int16).numpy(), P)
        assert np.array_equal(y.cpu().view(torch.int16).numpy(), ref)
    back = cru.ulysses_head2seq(ys, P)
    torch.cuda.synchronize()
    for b_, x in zip(back, (q, k, v)):
        assert torch.equal(b_.cpu().view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_layout_strided_and_other_degrees(dtype):
    g = torch.Generator().manual_seed(12)
    big = torch.randn(2, 40, 12, 64, generator=g).to(dtype).cuda()
    x = big[:, :, 4:, :]                       # [2, 40, 8, 64], strided over heads
    for P in (1, 2, 4, 8):
        y = cru.ulysses_seq2head(x, P)
        torch.cuda.synchronize()
        ref = oracle.seq2head(x.cpu().float().numpy(), P)
        assert np.array_equal(y.cpu().float().numpy(), ref)
        out = torch.zeros_like(big)
        cru.ulysses_head2seq(y, P, out=out[:, :, 4:, :])
        torch.cuda.synchronize()
        assert torch.equal(out[:, :, 4:, :].cpu(), x.cpu())
        assert (out[:, :, :4, :] == 0).all().item()   # nothing written outside the view


# ----------------------------------------- Ulysses Anything: uneven head groups

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 37, 7, 64, 3), (1, 16, 3, 128, 5), (2, 21, 30, 64, 4),
                                   (1, 9, 6, 64, 4), (1, 12, 8, 128, 2)])
def test_ulysses_anything_layouts_bit_exact(shape, dtype):
    B, S, H, D, P = shape
    say(f"ulysses anything layout B={B} S={S} H={H} D={D} P={P} {dtype}")
    g = torch.Generator().manual_seed(B * 1000 + S + H + P)
    big = torch.randn(B, S, H + 2, D, generator=g).to(dtype).cuda()
    x = big[:, :, 1:H + 1, :]                 # strided over heads
    y = cru.ulysses_seq2head(x, P, anything=True)
    torch.cuda.synchronize()
    ref = oracle.head_groups(x.cpu().float().numpy(), P)
    views = cru.ulysses_groups(y, B, S, H, D, P)
    assert [t.shape[2] for t in views] == [r.shape[2] for r in ref]
    for t, r in zip(views, ref):
        assert np.array_equal(t.cpu().float().numpy(), r)
    out = torch.zeros_like(big)
    cru.ulysses_head2seq(y, P, anything=True, out=out[:, :, 1:H + 1, :])
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 1:H + 1, :].cpu(), x.cpu())
    assert (out[:, :, 0, :] == 0).all().item() and (out[:, :, H + 1, :] == 0).all().item()
    if H % P == 0:                            # the even layout is the same bytes
        assert torch.equal(y.view(P, B, S, H // P, D), cru.ulysses_seq2head(x, P))


@pytest.mark.parametrize("P", [4, 7])
def test_ulysses_anything_share_bitwise(P):
    w = workload(5)                           # 30 heads: groups of 8,8,7,7 (P=4), 5,5,4,4,4,4,4 (P=7)
    (q, k, v), (qd, kd, vd) = inputs(5)
    B, S, H, D = qd.shape
    o_full, l_full = cru.attn_fwd_lse(qd, kd, vd)
    packed = cru.ulysses_seq2head([qd, kd, vd], P, anything=True)
    groups = [cru.ulysses_groups(t, B, S, H, D, P) for t in packed]
    o_packed = torch.empty_like(packed[0])
    o_views = cru.ulysses_groups(o_packed, B, S, H, D, P)
    for p, (h0, h1) in enumerate(cru.ulysses_head_bounds(H, P, anything=True)):
        say(f"ulysses anything share {w.name} P={P} group {p}: heads [{h0}, {h1})")
        o_p, l_p = cru.attn_fwd_lse(groups[0][p], groups[1][p], groups[2][p], out=o_views[p])
        torch.cuda.synchronize()
        # per-head arithmetic is the same whatever the launch's head count
        assert torch.equal(o_p, o_full[:, :, h0:h1]) and torch.equal(l_p, l_full[:, h0:h1])
    back = cru.ulysses_head2seq(o_packed, P, anything=True, shape=(B, S, H, D))
    torch.cuda.synchronize()
    assert torch.equal(back, o_full)
    q2, k2, v2 = (oracle.head_groups(to_f64(t), P)[1] for t in (q, k, v))
    h0, h1 = cru.ulysses_head_bounds(H, P, anything=True)[1]
    o_ref, l_ref = oracle.attention(q2, k2, v2)
    check_all(o_full[:, :, h0:h1], l_full[:, h0:h1], o_ref, l_ref, TOL_O, TOL_LSE,
              f"{w.name} anything group 1")


# ------------------------------------------------ Unified (USP) attention

@pytest.mark.parametrize("fused", [False, True])
def test_usp_tiny_fp32_matches_oracle(fused):
    (q, k, v), (qd, kd, vd) = inputs(1)
    for (Pu, Pr) in [(2, 4), (2, 2), (1, 4), (2, 1)]:
        say(f"usp tiny fp32 {Pu} x {Pr} fused={fused}")
        o, l = cru.usp_emulate(qd, kd, vd, Pu, Pr, fused=fused)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.usp_attention(to_f64(q), to_f64(k), to_f64(v), Pu, Pr)
        assert err(to_f64(o), o_ref) <= TOL_F32
        assert err(to_f64(l), l_ref) <= TOL_F32


@pytest.mark.parametrize("idx,Pu,Pr", [(2, 2, 2), (2, 4, 3), (2, 24, 1), (5, 2, 2), (3, 2, 4)])
def test_usp_bf16_workloads(idx, Pu, Pr):
    w = workload(idx)
    (q, k, v), (qd, kd, vd) = inputs(idx)
    say(f"usp {w.name} {Pu} x {Pr}")
    o_s, l_s = cru.usp_emulate(qd, kd, vd, Pu, Pr, fused=False)
    o_f, l_f = cru.usp_emulate(qd, kd, vd, Pu, Pr, fused=True)
    o_full, l_full = cru.attn_fwd_lse(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_f) and torch.equal(l_s, l_f)   # same per-chunk code
    # against the unchunked GPU forward: same result up to the fold's rounding
    assert err(to_f64(o_s), to_f64(o_full)) <= TOL_PAIR_O
    assert err(to_f64(l_s), to_f64(l_full)) <= TOL_PAIR_LSE
    o_ref, l_ref = oracle_full(idx)
    check_all(o_s, l_s, o_ref, l_ref, TOL_O, TOL_LSE, f"usp {w.name}")


# --------------------------------- partials in the model dtype (bf16)

def tol_bf16_partials(v):
    """Partial outputs rounded to bf16 (unit roundoff 2^-8) add at most
    2^-8 * max|O_c| <= 2^-8 * max|V| to the final error: the merge's weights
    sum to one, and every partial output is a convex combination of V rows."""
    return TOL_O + 2.0 ** -8 * float(v.abs().max())


@pytest.mark.parametrize("fused", [False, True])
def test_ring_bf16_partials(fused):
    w = workload(3)
    (q, k, v), (qd, kd, vd) = inputs(3)
    N = w.ring_degree
    a, b = cru.ring_chunk_bounds(w.S, N)[0]
    say(f"flux-1024 ring share, bf16 partials, fused={fused}")
    o16, l16 = cru.ring_emulate(qd[:, a:b], kd, vd, N, fused=fused, convert_to_fp32=False)
    o32, l32 = cru.ring_emulate(qd[:, a:b], kd, vd, N, fused=fused)
    torch.cuda.synchronize()
    tol = tol_bf16_partials(vd)
    # the LSE does not depend on the partials' dtype
    assert torch.equal(l16, l32)
    assert err(to_f64(o16), to_f64(o32)) <= tol + TOL_O
    o_ref, l_ref = oracle_full(3)
    check_all(o16, l16, o_ref[:, a:b], l_ref[:, :, a:b], tol, TOL_LSE,
              f"bf16 partials (O bound {tol:.3e})")


def test_ring_bf16_partials_fused_equals_stepwise_and_anything():
    (q, k, v), (qd, kd, vd) = inputs(4)
    w = workload(4)
    o_s, l_s = cru.ring_emulate(qd, kd, vd, w.ring_degree, anything=True, convert_to_fp32=False)
    o_f, l_f = cru.ring_emulate(qd, kd, vd, w.ring_degree, anything=True, fused=True,
                                convert_to_fp32=False)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_f) and torch.equal(l_s, l_f)
    o_ref, l_ref = oracle_full(4)
    check_all(o_s, l_s, o_ref, l_ref, tol_bf16_partials(vd), TOL_LSE,
              "ring anything, bf16 partials")


def test_usp_bf16_partials():
    w = workload(2)
    (q, k, v), (qd, kd, vd) = inputs(2)
    o, l = cru.usp_emulate(qd, kd, vd, 2, 3, fused=True, convert_to_fp32=False)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(2)
    check_all(o, l, o_ref, l_ref, tol_bf16_partials(vd), TOL_LSE, "usp 2 x 3, bf16 partials")


# ------------------------------------------------- the five workloads, full size

@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_workload_full_forward(idx):
    w = workload(idx)
    (q, k, v), (qd, kd, vd) = inputs(idx)
    say(f"full forward {w.name} B={w.B} S={w.S} H={w.H} D={w.D}")
    o, l = cru.attn_fwd_lse(qd, kd, vd)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(l).all().item()
    o_ref, l_ref = oracle_full(idx)
    check_all(o, l, o_ref, l_ref, TOL_O, TOL_LSE, w.name)


def test_degree_sweep_same_seed():
    # one fixed-seed input (FLUX-512: S and H divide by 1, 2, 4 and 8) under
    # every degree.  Ulysses: the regrouped shares, put back together, are
    # bit-identical to the full forward at every degree.  Ring: every rank's
    # share assembled agrees with degree 1 within twice the bar (both are
    # within it of the exact result) and with the oracle on every row.
    w = workload(2)
    (q, k, v), (qd, kd, vd) = inputs(2)
    S, H = w.S, w.H
    o1, l1 = cru.attn_fwd_lse(qd, kd, vd)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_full(2)
    for P in (1, 2, 4, 8):
        say(f"degree sweep: Ulysses P={P}")
        ys = cru.ulysses_seq2head([qd, kd, vd], P)
        og = torch.empty_like(ys[0])
        for p in range(P):
            cru.attn_fwd_lse(ys[0][p], ys[1][p], ys[2][p], out=og[p])
        back = cru.ulysses_head2seq(og, P)
        torch.cuda.synchronize()
        assert torch.equal(back, o1), P
    for N in (1, 2, 4, 8):
        say(f"degree sweep: ring N={N}")
        o_n = torch.empty_like(o1)
        l_n = torch.empty_like(l1)
        for r, (a, b) in enumerate(cru.ring_chunk_bounds(S, N)):
            o_r, l_r = cru.ring_emulate(qd[:, a:b], kd, vd, N, fused=True)
            o_n[:, a:b] = o_r
            l_n[:, :, a:b] = l_r
        torch.cuda.synchronize()
        assert err(to_f64(o_n), to_f64(o1)) <= TOL_PAIR_O, N
        assert err(to_f64(l_n), to_f64(l1)) <= TOL_PAIR_LSE, N
        check_all(o_n, l_n, o_ref, l_ref, TOL_O, TOL_LSE, f"ring degree {N}, all ranks")


@pytest.mark.parametrize("idx", [2, 5])
def test_ulysses_share_matches_full_forward_bitwise(idx):
    w = workload(idx)
    (q, k, v), (qd, kd, vd) = inputs(idx)
    P = w.ulysses_degree
    Hp = w.H // P
    o_full, l_full = cru.attn_fwd_lse(qd, kd, vd)
    qs, ks, vs = cru.ulysses_seq2head([qd, kd, vd], P)
    o_groups = []
    for p in range(P):
        say(f"ulysses share {w.name} group {p} of {P}")
        o_p, l_p = cru.attn_fwd_lse(qs[p], ks[p], vs[p])
        torch.cuda.synchronize()
        # a head's arithmetic does not depend on its neighbours: bit-identical
        assert torch.equal(o_p, o_full[:, :, p * Hp:(p + 1) * Hp])
        assert torch.equal(l_p, l_full[:, p * Hp:(p + 1) * Hp])
        o_groups.append(o_p)
    o_back = cru.ulysses_head2seq(torch.stack(o_groups), P)
    torch.cuda.synchronize()
    assert torch.equal(o_back, o_full)
    # and the share itself against the oracle's attention on the regrouped
    # heads (group 0, every row)
    q0, k0, v0 = (oracle.seq2head(to_f64(t), P)[0] for t in (q, k, v))
    o_ref, l_ref = oracle.attention(q0, k0, v0)
    check_all(o_groups[0], l_full[:, :Hp], o_ref, l_ref, TOL_O, TOL_LSE,
              f"{w.name} ulysses group 0")


@pytest.mark.parametrize("rank", [0, 5, 7])
def test_flux1024_ring_share(rank):
    w = workload(3)
    (q, k, v), (qd, kd, vd) = inputs(3)
    N = w.ring_degree
    a, b = cru.ring_chunk_bounds(w.S, N)[rank]
    say(f"flux-1024 ring share rank {rank}: rows [{a}, {b}) x {N} chunks")
    o_s, l_s = cru.ring_emulate(qd[:, a:b], kd, vd, N, fused=False)
    o_f, l_f = cru.ring_emulate(qd[:, a:b], kd, vd, N, fused=True)
    torch.cuda.synchronize()
    assert torch.equal(o_s, o_f) and torch.equal(l_s, l_f)   # same per-chunk code
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    # every row of the share: the unchunked definition ...
    o_ref, l_ref = oracle_full(3)
    check_all(o_s, l_s, o_ref[:, a:b], l_ref[:, :, a:b], TOL_O, TOL_LSE, f"rank {rank} share")
    # ... and the oracle's own ring share, folded chunk by chunk
    o_ring, l_ring = oracle.ring_share(q64, k64, v64, N, rank)
    check_all(o_s, l_s, o_ring, l_ring, TOL_O, TOL_LSE, f"rank {rank} share (oracle ring fold)")


def test_flux1024_all_rows_chunked_merge():
    """All 4608 query rows against 8 chunks, merged (the merge at full size)."""
    w = workload(3)
    (q, k, v), (qd, kd, vd) = inputs(3)
    o_full, l_full = cru.attn_fwd_lse(qd, kd, vd)
    o_c, l_c = cru.ring_emulate(qd, kd, vd, w.ring_degree, fused=True)
    torch.cuda.synchronize()
    eo = err(to_f64(o_c), to_f64(o_full))
    el = err(to_f64(l_c), to_f64(l_full))
    say(f"  chunked+merged vs unchunked (GPU): max|dO| = {eo:.3e}, max|dLSE| = {el:.3e}")
    assert eo <= TOL_PAIR_O and el <= TOL_PAIR_LSE
    o_ref, l_ref = oracle_full(3)
    check_all(o_c, l_c, o_ref, l_ref, TOL_O, TOL_LSE, "flux-1024 chunked+merged")


@pytest.mark.parametrize("fused", [False, True])
def test_ring_anything_uneven_chunks(fused):
    w = workload(4)
    (q, k, v), (qd, kd, vd) = inputs(4)
    N = w.ring_degree
    with pytest.raises(cru.CruNotDivisible):
        cru.ring_emulate(qd, kd, vd, N)                 # plain ring refuses S % N != 0
    say(f"ring anything S={w.S} N={N} fused={fused}")
    o_c, l_c = cru.ring_emulate(qd, kd, vd, N, anything=True, fused=fused)
    o_full, l_full = cru.attn_fwd_lse(qd, kd, vd)
    torch.cuda.synchronize()
    assert err(to_f64(o_c), to_f64(o_full)) <= TOL_PAIR_O
    assert err(to_f64(l_c), to_f64(l_full)) <= TOL_PAIR_LSE
    o_ref, l_ref = oracle_full(4)
    check_all(o_c, l_c, o_ref, l_ref, TOL_O, TOL_LSE, "ring anything chunked+merged")
    # rank 0's share: its 581 rows
    a, b = cru.ring_chunk_bounds(w.S, N, anything=True)[0]
    assert (a, b) == (0, 581)
    o_r, l_r = cru.ring_emulate(qd[:, a:b], kd, vd, N, anything=True, fused=fused)
    torch.cuda.synchronize()
    assert err(to_f64(o_r), to_f64(o_c)[:, a:b]) <= TOL_PAIR_O
    check_all(o_r, l_r, o_ref[:, a:b], l_ref[:, :, a:b], TOL_O, TOL_LSE, "ring anything rank 0")


@pytest.mark.parametrize("fused", [False, True])
def test_ring_empty_and_explicit_chunks(fused):
    q, k, v = random_qkv(13, 1, 100, 90, 2, 128)
    qd, kd, vd = cuda(q, k, v)
    sizes = [0, 40, 0, 1, 49, 0]
    o, l = cru.ring_emulate(qd, kd, vd, len(sizes), anything=True, chunk_sizes=sizes, fused=fused)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.chunked_attention(to_f64(q), to_f64(k), to_f64(v), len(sizes), sizes)
    assert err(to_f64(o), o_ref) <= TOL_O and err(to_f64(l), l_ref) <= TOL_LSE


@pytest.mark.parametrize("fused", [False, True])
def test_ring_degenerate_degrees(fused):
    # a ring of one chunk is plain attention; a ring whose chunks are all
    # empty has no keys at all (O = 0, LSE = -inf)
    q, k, v = random_qkv(16, 2, 75, 75, 3, 64)
    qd, kd, vd = cuda(q, k, v)
    o, l = cru.ring_emulate(qd, kd, vd, 1, fused=fused)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
    assert err(to_f64(o), o_ref) <= TOL_O and err(to_f64(l), l_ref) <= TOL_LSE
    o, l = cru.ring_emulate(qd, kd[:, :0], vd[:, :0], 4, anything=True, fused=fused,
                            out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o.cpu() == 0).all() and torch.isneginf(l.cpu()).all()


def test_random_shape_sweep():
    # seeded random shapes, each checked against the oracle: attention (bf16,
    # both head dims, any row and key counts including 1 and ragged tails),
    # the layouts (bit-exact, even and uneven head groups, both dtypes) and
    # the merge (random part counts)
    rng = np.random.default_rng(2024)
    for case in range(12):
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 6))
        D = int(rng.choice([64, 128]))
        Sq = int(rng.integers(1, 400))
        Skv = int(rng.integers(1, 400))
        say(f"sweep {case}: attention B={B} Sq={Sq} Skv={Skv} H={H} D={D}")
        q, k, v = random_qkv(100 + case, B, Sq, Skv, H, D, gain=float(rng.uniform(0.5, 2.0)))
        o, l = cru.attn_fwd_lse(*cuda(q, k, v))
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.attention(to_f64(q), to_f64(k), to_f64(v))
        assert err(to_f64(o), o_ref) <= TOL_O, case
        assert err(to_f64(l), l_ref) <= TOL_LSE, case

        P = int(rng.integers(1, 6))
        anything = H % P != 0 or Skv % P != 0 or bool(rng.integers(0, 2))
        dtype = torch.bfloat16 if rng.integers(0, 2) else torch.float32
        say(f"sweep {case}: layouts B={B} S={Skv} H={H} D={D} P={P} anything={anything} {dtype}")
        x = torch.randn(B, Skv, H, D, generator=torch.Generator().manual_seed(case)).to(dtype)
        y = cru.ulysses_seq2head(x.cuda(), P, anything=anything)
        back = cru.ulysses_head2seq(y, P, anything=anything, shape=x.shape)
        torch.cuda.synchronize()
        ints = torch.int16 if dtype == torch.bfloat16 else torch.int32
        groups = cru.ulysses_groups(y, B, Skv, H, D, P)
        ref = oracle.head_groups(x.view(ints).numpy(), P)
        assert all(np.array_equal(gr.cpu().view(ints).numpy(), r) for gr, r in zip(groups, ref)), case
        assert torch.equal(back.cpu().view(ints), x.view(ints)), case

        n = int(rng.integers(1, 20))
        say(f"sweep {case}: merge of {n} parts")
        parts = [torch.randn(B, Sq, H, D, generator=torch.Generator().manual_seed(1000 * case + c))
                 for c in range(n)]
        lses = [torch.randn(B, H, Sq, generator=torch.Generator().manual_seed(2000 * case + c)) * 3
                for c in range(n)]
        om, lm = cru.attn_merge_lse([t.cuda() for t in parts], [t.cuda() for t in lses],
                                    out_dtype=torch.float32)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.merge_closed_form([t.double().numpy() for t in parts],
                                                [t.double().numpy() for t in lses])
        assert err(to_f64(om), o_ref) <= TOL_F32 and err(to_f64(lm), l_ref) <= TOL_F32, case


def test_graph_capture_replays_match_eager():
    # every entry point only enqueues kernels (no allocation, memset or
    # synchronisation), so a sequence of calls can be captured in a graph.
    # Each replay, with eager work in between, must equal the eager result
    # bit for bit.
    q, k, v = (t.cuda() for t in random_qkv(18, 1, 600, 600, 4, 128, gain=1.7))
    a, b = cru.ring_chunk_bounds(600, 4)[1]
    qs = q[:, a:b]
    ws = torch.empty(cru.ring_workspace_bytes(qs, 4), dtype=torch.uint8, device="cuda")
    uws = torch.empty(cru.usp_workspace_bytes(q, 2, 3), dtype=torch.uint8, device="cuda")
    outs = {
        "o": torch.empty_like(q), "l": torch.empty(1, 4, 600, device="cuda"),
        "or": torch.empty_like(qs), "lr": torch.empty(1, 4, b - a, device="cuda"),
        "om": torch.empty_like(q), "lm": torch.empty(1, 4, 600, device="cuda"),
        "y": torch.empty(2, 1, 600, 2, 128, dtype=q.dtype, device="cuda"),
        "x": torch.empty_like(q),
        "ou": torch.empty_like(q), "lu": torch.empty(1, 4, 600, device="cuda"),
    }
    parts_o = [torch.randn(1, 600, 4, 128, device="cuda") for _ in range(3)]
    parts_l = [torch.randn(1, 4, 600, device="cuda") for _ in range(3)]

    def run():
        cru.attn_fwd_lse(q, k, v, out=outs["o"], lse=outs["l"])
        cru.ring_emulate(qs, k, v, 4, fused=True, out=outs["or"], lse=outs["lr"], workspace=ws)
        cru.attn_merge_lse(parts_o, parts_l, out=outs["om"], lse=outs["lm"])
        cru.ulysses_seq2head(q, 2, out=outs["y"])
        cru.ulysses_head2seq(outs["y"], 2, out=outs["x"])
        cru.usp_emulate(q, k, v, 2, 3, fused=True, out=outs["ou"], lse=outs["lu"], workspace=uws)

    run()
    torch.cuda.synchronize()
    ref = {n: t.clone() for n, t in outs.items()}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs.values():
            t.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, t in outs.items():
            assert torch.equal(t, ref[n]), (rep, n)
    assert torch.equal(ref["x"], q)


def test_calls_on_two_streams_match_one_stream():
    # the library keeps no state between calls (outside the no-allocation
    # entry point's scratch), so independent calls on two streams at the
    # default priority, running at the same time, give the results the same
    # calls give one after another, bit for bit
    q, k, v = (t.cuda() for t in random_qkv(21, 1, 1200, 1200, 6, 128, gain=1.7))
    qs = q[:, :300]
    ws = torch.empty(cru.ring_workspace_bytes(qs, 4), dtype=torch.uint8, device="cuda")
    parts_o = [torch.randn(1, 1200, 6, 128, device="cuda") for _ in range(5)]
    parts_l = [torch.randn(1, 6, 1200, device="cuda") for _ in range(5)]
    outs = [torch.empty_like(q), torch.empty(1, 6, 1200, device="cuda"),
            torch.empty_like(qs), torch.empty(1, 6, 300, device="cuda"),
            torch.empty(1, 1200, 6, 128, dtype=torch.bfloat16, device="cuda"),
            torch.empty(1, 6, 1200, device="cuda")]

    def first():
        cru.attn_fwd_lse(q, k, v, out=outs[0], lse=outs[1])

    def second():
        cru.ring_emulate(qs, k, v, 4, fused=True, out=outs[2], lse=outs[3], workspace=ws)
        cru.attn_merge_lse(parts_o, parts_l, out=outs[4], lse=outs[5])

    first()
    second()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    for rep in range(3):
        for t in outs:
            t.fill_(5.0)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            second()
        first()
        main.wait_stream(side)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), (rep, i)


def test_device_errors():
    q, k, v = random_qkv(14, 1, 16, 16, 2, 64)
    with pytest.raises(cru.CruDeviceError):
        cru.attn_fwd_lse(q.cuda(), k, v.cuda())          # k left in host memory
