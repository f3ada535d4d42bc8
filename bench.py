"""Benchmark of the context-parallel attention hot path on one MI355X.

One step is one pass of the whole path over the FLUX.1-dev 1024x1024 joint
attention shape (B=1, H=24, S=4096+512=4608, D=128, bf16, synthetic inputs):

  1. the full forward: attention with per-row LSE over all 4608 rows;
  2. ring rank 0's share at ring degree 8: its 576 query rows against the
     8 K/V chunks (all resident, as after the ring's all-gather), the 8
     per-chunk partials from one split-KV launch, then the in-order fold
     (bitwise the same result as one launch per chunk);
  3. the 8-way LSE merge over all 4608 rows (8 fp32 partials -> bf16 O);
  4. Ulysses rank 0's share at degree 2: seq2head of Q, K, V, then attention
     over its 12 heads at full length whose epilogue stores straight into
     those heads of the [B, S, H, D] output (the regrouping by token fused
     into the store; the standalone head2seq kernel is timed cold below).

The parts are independent; the timed step runs parts 2 and 3 on a second
stream (default priority) beside 4's seq2head, 1 and 4's attention on the
first, so the memory-bound merge and the short ring launches fill CUs the
full forward leaves idle.  A second pass with the parts one after another
gives the per-part breakdown.

Inputs (and the merge's partials) are resident in HBM before timing starts.
``value`` is the attention work of a step (4*B*H*Sq*Skv*D summed over parts
1, 2 and 4) divided by the step time.  The JSON line also carries each
part's own time, the attention kernel's roofline (achieved TFLOP/s from HIP
events on its stream, 100 timed launches of the full forward on their own,
vs the bf16 dense peak), cold-cache bandwidth of the merge and layout
kernels, and the fp64 oracle timed on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --copy-calibration   # plain copy of known size, for counters
    python bench.py --attn-only N        # N FLUX-1024 forwards only, for counters
    python bench.py --attn-only N --heads H   # the same shape with H heads
    python bench.py --load-sweep         # FLUX-1024-shaped forward at 1..48 heads
    python bench.py --ceilings           # library GEMM, copy and read rates, for context
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak
METRIC = "attention TFLOP/s and % bf16 MFMA peak at FLUX-1024 shape; merge GB/s"
ATTN_SOURCE = os.path.join(ROOT, "context_ring_ulysses_amd", "csrc", "attn_fwd_bf16.hip")
COUNTERS = os.path.join(ROOT, "profiles", "attn_fwd_bf16_flux1024_counters.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flops(B, H, Sq, Skv, D):
    return 4.0 * B * H * Sq * Skv * D


def merge_bytes(n, B, S, H, D, out_bytes=2, part_bytes=4):
    """Algorithmic bytes of an n-way merge: every part's O and LSE read once,
    O and LSE written once."""
    rows = B * S * H
    return n * (rows * D * part_bytes + rows * 4) + rows * D * out_bytes + rows * 4


def source_sha256(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def counters_traffic():
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on a different kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    kv = {}
    for line in open(COUNTERS):
        if ":" in line:
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_sha256(ATTN_SOURCE):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(budget_s=10.0, max_forwards=480):
    """The fp64 oracle's full forward on FLUX-1024, one head at a time (heads
    cycled) until about ``budget_s`` of host time is spent; TFLOP/s with the
    same flop count as the GPU."""
    import oracle
    from workloads import make_inputs, to_f64, workload
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        cores = max([d.get("num_threads", 1) for d in pools] or [1])
        if pools:
            blas = ", ".join(f"{d.get('internal_api', '?')} {d.get('version', '')}".strip()
                             for d in pools)
    except Exception:
        cores = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    w = workload(3)
    q, k, v = make_inputs(3)
    done, spent = 0, 0.0
    while done < max_forwards and spent < budget_s:
        h = done % w.H
        qh, kh, vh = (to_f64(t[:, :, h:h + 1]) for t in (q, k, v))
        t0 = time.perf_counter()
        oracle.attention(qh, kh, vh)
        spent += time.perf_counter() - t0
        done += 1
    flops = attn_flops(1, done, w.S, w.S, w.D)
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "cpu_model": cpu_model, "blas": blas,
            "host_cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"fp64 oracle full forward of FLUX-1024 (S=4608, D=128, all rows), "
                      f"{done} single-head forwards (heads cycled), {spent:.1f} s",
            "per_config": cpu_per_config()}


def cpu_per_config(budget_s=2.5):
    """The oracle on the other bf16 workloads and on FLUX-1024's ring share
    (its 576 rows against the 8 chunks, folded in order), one (batch, head)
    at a time until about ``budget_s`` each; TFLOP/s with the GPU's flop
    count.  Reported beside the headline baseline, not a target."""
    import oracle
    from workloads import make_inputs, to_f64, workload
    out = {}

    def run(name, idx, fn, flops_per_call):
        w = workload(idx)
        q, k, v = make_inputs(idx)
        done, spent = 0, 0.0
        while spent < budget_s:
            b, h = (done // w.H) % w.B, done % w.H
            qh, kh, vh = (to_f64(t[b:b + 1, :, h:h + 1]) for t in (q, k, v))
            t0 = time.perf_counter()
            fn(qh, kh, vh, w)
            spent += time.perf_counter() - t0
            done += 1
        out[name] = {"TFLOP/s": done * flops_per_call(w) / spent / 1e12,
                     "sample": f"{done} single-head calls, {spent:.1f} s"}

    full = lambda qh, kh, vh, w: oracle.attention(qh, kh, vh)
    run("flux-512 full forward", 2, full, lambda w: attn_flops(1, 1, w.S, w.S, w.D))
    run("ring-anything-4645 full forward", 4, full, lambda w: attn_flops(1, 1, w.S, w.S, w.D))
    run("video-dit-4276 full forward", 5, full, lambda w: attn_flops(1, 1, w.S, w.S, w.D))
    run("flux-1024 ring rank-0 share (8 chunks, fold)", 3,
        lambda qh, kh, vh, w: oracle.ring_share(qh, kh, vh, w.ring_degree, 0),
        lambda w: attn_flops(1, 1, oracle.chunk_bounds(w.S, w.ring_degree)[0][1], w.S, w.D))
    return out


def copy_calibration():
    import torch
    n = 1 << 30
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))


def attn_only(n, heads=0):
    """n full forwards at FLUX-1024 and nothing else, for counter collection.
    heads > 0: the same shape (S=4608, D=128) with that many heads instead,
    to see how the counters change with the number of busy CUs (18
    workgroups of 256 query rows per head)."""
    import torch
    import context_ring_ulysses_amd as cru
    from workloads import make_inputs, random_qkv, workload
    w = workload(3)
    if heads > 0:
        q, k, v = (t.cuda() for t in random_qkv(11, 1, w.S, w.S, heads, w.D, gain=3 ** 0.5))
    else:
        q, k, v = (t.cuda() for t in make_inputs(3))
    o = torch.empty_like(q)
    l = torch.empty(q.shape[0], q.shape[2], q.shape[1], dtype=torch.float32, device=q.device)
    for _ in range(n):
        cru.attn_fwd_lse(q, k, v, out=o, lse=l)
    torch.cuda.synchronize()
    log(f"[bench] {n} forwards done, {q.shape[2]} heads")


def ceilings():
    """What this GPU reaches on plain library work, beside the published
    peaks the bars use: a dense bf16 GEMM through torch (hipBLASLt), a 1 GiB
    device copy (read + write) and a 1 GiB read (a sum), each back to back
    after a settling half second; the median of 20."""
    import torch
    dev = torch.device("cuda:0")

    def timed(fn, reps=20):
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.5:
            fn()
            torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        evs[0].record()
        for i in range(reps):
            fn()
            evs[i + 1].record()
        torch.cuda.synchronize()
        return statistics.median(evs[i].elapsed_time(evs[i + 1]) for i in range(reps))

    out = {}
    n = 8192
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev, generator=g).to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device=dev)
    t = timed(lambda: torch.mm(a, b, out=c))
    out["bf16_gemm_8192"] = {"ms_median": t, "TFLOP/s": 2.0 * n ** 3 / (t * 1e-3) / 1e12,
                             "frac_of_2500": 2.0 * n ** 3 / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    del a, b, c
    nb = 1 << 30
    x = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    t = timed(lambda: y.copy_(x))
    out["copy_1GiB"] = {"ms_median": t, "GB/s": 2 * nb / (t * 1e-3) / 1e9,
                        "frac_of_8000": 2 * nb / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}
    sink = torch.empty((), dtype=torch.float32, device=dev)
    t = timed(lambda: torch.sum(x, dim=0, out=sink))
    out["read_1GiB"] = {"ms_median": t, "GB/s": nb / (t * 1e-3) / 1e9,
                        "frac_of_8000": nb / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}
    # cold plain copies of several sizes, timed like the merge and layout
    # legs (a 1 GiB read between reps evicts L2 and the MALL): a straight
    # line through them splits each copy's time into a fixed cost and a
    # steady rate, which bounds what a memory-bound launch of a given size
    # can reach
    stream = torch.cuda.current_stream()
    sweep = []
    for mib in (8, 16, 32, 64, 128, 256, 512):
        n_el = mib * (1 << 20) // 2
        src = torch.empty(n_el, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        ts = []
        for _ in range(25):
            torch.sum(x, dim=0, out=sink)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        t = statistics.median(ts)
        sweep.append({"bytes_rw": 4 * n_el, "ms_median": t, "GB/s": 4 * n_el / (t * 1e-3) / 1e9})
        del src, dst
    # least-squares line t = t0 + bytes / rate over the sizes that bracket
    # the layout and merge launches (64 to 537 MB moved)
    pts = [(s_["bytes_rw"], s_["ms_median"]) for s_ in sweep[2:6]]
    mx = statistics.mean(p[0] for p in pts)
    my = statistics.mean(p[1] for p in pts)
    slope = sum((p[0] - mx) * (p[1] - my) for p in pts) / sum((p[0] - mx) ** 2 for p in pts)
    out["cold_copy_sweep"] = {"points": sweep,
                              "fixed_us": (my - slope * mx) * 1e3,
                              "steady_GB/s": 1.0 / (slope * 1e-3) / 1e9}
    del x, y
    for k, v in out.items():
        log(f"[bench] ceiling {k}: {v}")
    print(json.dumps({"ceilings": out}))


def load_sweep():
    """The S=4608, D=128 forward at several head counts: throughput as the
    number of busy CUs grows (4608 rows make 18 tiles of 256 rows per head;
    the launch picks its own workgroup shape, 8 waves from 14 heads up)."""
    import torch
    import context_ring_ulysses_amd as cru
    S, D = 4608, 128
    g = torch.Generator(device="cuda").manual_seed(0)
    rows = []
    for H in (1, 2, 4, 7, 10, 14, 24, 48):
        q = (torch.randn(1, S, H, D, device="cuda", generator=g) * 3 ** 0.5).to(torch.bfloat16)
        k = (torch.randn(1, S, H, D, device="cuda", generator=g) * 3 ** 0.5).to(torch.bfloat16)
        v = torch.randn(1, S, H, D, device="cuda", generator=g).to(torch.bfloat16)
        o = torch.empty_like(q)
        l = torch.empty(1, H, S, device="cuda")
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.5:
            for _ in range(10):
                cru.attn_fwd_lse(q, k, v, out=o, lse=l)
            torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(51)]
        evs[0].record()
        for i in range(50):
            cru.attn_fwd_lse(q, k, v, out=o, lse=l)
            evs[i + 1].record()
        torch.cuda.synchronize()
        t = statistics.median(evs[i].elapsed_time(evs[i + 1]) for i in range(50))
        tiles = 18 * H
        rows.append({"heads": H, "row_tiles_of_256": tiles, "ms_median": t,
                     "TFLOP/s": attn_flops(1, H, S, S, D) / (t * 1e-3) / 1e12})
        log(f"[bench] load sweep H={H}: {rows[-1]}")
    print(json.dumps({"load_sweep": rows}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cold-reps", type=int, default=50)
    ap.add_argument("--attn-reps", type=int, default=100,
                    help="timed launches of the full forward for the roofline leg")
    ap.add_argument("--load-sweep", action="store_true")
    ap.add_argument("--ceilings", action="store_true",
                    help="library GEMM, copy and read rates on this GPU, for context")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--attn-only", type=int, default=0, metavar="N",
                    help="run N FLUX-1024 full forwards and exit (for counter passes)")
    ap.add_argument("--heads", type=int, default=0,
                    help="with --attn-only: this many heads instead of 24")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the work on one GPU and has no "
              "multi-GPU mode (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import context_ring_ulysses_amd as cru
    from workloads import make_inputs, workload

    if args.copy_calibration:
        copy_calibration()
        return
    if args.attn_only:
        attn_only(args.attn_only, args.heads)
        return
    if args.load_sweep:
        load_sweep()
        return
    if args.ceilings:
        ceilings()
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workload(3)
    B, S, H, D = w.B, w.S, w.H, w.D
    N = w.ring_degree
    P = 2
    Hp = H // P
    log(f"[bench] workload {w.name}: B={B} S={S} H={H} D={D} ring={N} ulysses={P}")
    q, k, v = (t.to(dev) for t in make_inputs(3))

    # outputs and the merge's partials, all resident before timing
    o_full = torch.empty_like(q)
    l_full = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    a0, b0 = cru.ring_chunk_bounds(S, N)[0]
    q_share = q[:, a0:b0]
    o_ring = torch.empty_like(q_share)
    l_ring = torch.empty(B, H, b0 - a0, dtype=torch.float32, device=dev)
    ws = torch.empty(cru.ring_workspace_bytes(q_share, N), dtype=torch.uint8, device=dev)
    parts_o, parts_l = [], []
    for (a, b) in cru.ring_chunk_bounds(S, N):
        o_c, l_c = cru.attn_fwd_lse(q, k[:, a:b], v[:, a:b], out_dtype=torch.float32)
        parts_o.append(o_c)
        parts_l.append(l_c)
    o_merge = torch.empty_like(q)
    l_merge = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    ys = [torch.empty(P, B, S, Hp, D, dtype=q.dtype, device=dev) for _ in range(3)]
    l_u = torch.empty(B, Hp, S, dtype=torch.float32, device=dev)
    o_u = torch.empty_like(q)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # a second stream at the default priority for the step's memory-bound
    # and short parts
    side = torch.cuda.Stream()

    def step_parts(marks):
        """One step with the parts one after another on one stream, an event
        between parts: the per-part breakdown."""
        m = marks
        m[0].record(stream)
        cru.attn_fwd_lse(q, k, v, out=o_full, lse=l_full)
        m[1].record(stream)
        cru.ring_emulate(q_share, k, v, N, fused=True, out=o_ring, lse=l_ring, workspace=ws)
        m[2].record(stream)
        cru.attn_merge_lse(parts_o, parts_l, out=o_merge, lse=l_merge)
        m[3].record(stream)
        cru.ulysses_seq2head([q, k, v], P, out=ys)
        # group 0's heads of the [B, S, H, D] output: a strided view the
        # epilogue stores into directly (head2seq of this group, fused)
        cru.attn_fwd_lse(ys[0][0], ys[1][0], ys[2][0], out=o_u[:, :, :Hp], lse=l_u)
        m[4].record(stream)

    def step():
        """One step as timed: the ring share and the merge on the second
        stream, beside the Ulysses share's seq2head, the full forward and
        the Ulysses share's attention on the first; the step ends when both
        are done.  The parts are independent, so the memory-bound merge and
        the short ring launches fill the CUs the full forward leaves idle in
        its partial last round of workgroups.  Same results, bit for bit, as
        the parts one after another."""
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            cru.ring_emulate(q_share, k, v, N, fused=True, out=o_ring, lse=l_ring, workspace=ws)
            cru.attn_merge_lse(parts_o, parts_l, out=o_merge, lse=l_merge)
        cru.ulysses_seq2head([q, k, v], P, out=ys)
        cru.attn_fwd_lse(q, k, v, out=o_full, lse=l_full)
        cru.attn_fwd_lse(ys[0][0], ys[1][0], ys[2][0], out=o_u[:, :, :Hp], lse=l_u)
        stream.wait_stream(side)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # the same step with its parts one after another on one stream, for the
    # breakdown (and the step time without the overlap)
    marks = [[ev() for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step_parts(marks[i])
    torch.cuda.synchronize()
    part_ms = {name: statistics.mean(m[j].elapsed_time(m[j + 1]) for m in marks)
               for j, name in enumerate(["attn_full", "ring_share", "merge_all_rows", "ulysses_share"])}
    ms_per_step_seq = statistics.mean(m[0].elapsed_time(m[4]) for m in marks)

    f_full = attn_flops(B, H, S, S, D)
    f_ring = attn_flops(B, H, b0 - a0, S, D)
    f_uly = attn_flops(B, Hp, S, S, D)
    step_flops = f_full + f_ring + f_uly
    value = step_flops / (ms_per_step * 1e-3) / 1e12
    attn_tflops = f_full / (part_ms["attn_full"] * 1e-3) / 1e12
    mbytes = merge_bytes(N, B, S, H, D)
    merge_gbs = mbytes / (part_ms["merge_all_rows"] * 1e-3) / 1e9
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step (parts one after another: "
        f"{ms_per_step_seq:.3f} ms); attn {part_ms['attn_full']:.3f} ms "
        f"= {attn_tflops:.1f} TFLOP/s; merge {merge_gbs:.0f} GB/s")

    # cold-cache bandwidth: reading 1 GiB between reps evicts L2 and the MALL
    # (a read leaves clean lines, so no write-back lands in the timed kernel)
    scrub = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)

    def cold(fn, reps):
        ts = []
        for _ in range(reps):
            torch.sum(scrub, dim=0, out=sink)
            e0, e1 = ev(), ev()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts), min(ts)

    med, mn = cold(lambda: cru.attn_merge_lse(parts_o, parts_l, out=o_merge, lse=l_merge),
                   args.cold_reps)
    # the roofline leg: the full forward on its own, each launch timed by the
    # events around it on the library's stream (torch's current stream),
    # after about a second of back-to-back forwards, so the clocks have
    # settled where a running job holds them
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 1.0:
        for _ in range(20):
            cru.attn_fwd_lse(q, k, v, out=o_full, lse=l_full)
        torch.cuda.synchronize()
    # back to back: an event after every launch, so consecutive events
    # bracket exactly one forward and no host sync sits between launches
    evs = [ev() for _ in range(args.attn_reps + 1)]
    evs[0].record(stream)
    for i in range(args.attn_reps):
        cru.attn_fwd_lse(q, k, v, out=o_full, lse=l_full)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    attn_ts = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.attn_reps)]
    attn_mean = statistics.mean(attn_ts)
    log(f"[bench] full forward alone: {args.attn_reps} launches, mean {attn_mean * 1e3:.1f} us, "
        f"median {statistics.median(attn_ts) * 1e3:.1f} us, min {min(attn_ts) * 1e3:.1f} us")

    cold_merge = {"workload": "flux-1024, 8 fp32 partials over all 4608 rows -> bf16 O + LSE",
                  "bytes": mbytes, "ms_median": med, "ms_min": mn,
                  "GB/s": mbytes / (med * 1e-3) / 1e9,
                  "frac_hbm_peak": mbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS}
    # the same merge with partials kept in bf16 (convert_to_fp32 off)
    parts_b = [p_.to(torch.bfloat16) for p_ in parts_o]
    del parts_o
    mbytes_b = merge_bytes(N, B, S, H, D, part_bytes=2)
    medb, mnb = cold(lambda: cru.attn_merge_lse(parts_b, parts_l, out=o_merge, lse=l_merge),
                     args.cold_reps)
    cold_merge_bf16 = {"workload": "flux-1024, 8 bf16 partials over all 4608 rows -> bf16 O + LSE",
                       "bytes": mbytes_b, "ms_median": medb, "ms_min": mnb,
                       "GB/s": mbytes_b / (medb * 1e-3) / 1e9,
                       "frac_hbm_peak": mbytes_b / (medb * 1e-3) / 1e9 / PEAK_HBM_GBS}
    del parts_b, parts_l

    wv = workload(5)
    qv, kv_, vv = (t.to(dev) for t in make_inputs(5))
    Pv = wv.ulysses_degree
    ysv = [torch.empty(Pv, wv.B, wv.S, wv.H // Pv, wv.D, dtype=qv.dtype, device=dev)
           for _ in range(3)]
    ov = torch.empty_like(qv)
    tbytes = qv.numel() * qv.element_size()
    med1, mn1 = cold(lambda: cru.ulysses_seq2head([qv, kv_, vv], Pv, out=ysv), args.cold_reps)
    med2, mn2 = cold(lambda: cru.ulysses_head2seq(ysv[0], Pv, out=ov), args.cold_reps)
    # reference: torch's plain contiguous device copy of the same byte counts
    # (what a copy of this size reaches on this GPU, launch and ramp included)
    src3 = torch.empty(3 * qv.numel(), dtype=qv.dtype, device=dev)
    dst3 = torch.empty_like(src3)
    medc1, _ = cold(lambda: dst3.copy_(src3), args.cold_reps)
    medc2, _ = cold(lambda: ov.copy_(qv), args.cold_reps)
    del src3, dst3
    cold_layout = {
        "workload": "video-dit-4276 (B=2, S=4276, H=30, D=64, bf16), P=2",
        "seq2head_qkv": {"bytes": 6 * tbytes, "ms_median": med1, "ms_min": mn1,
                         "GB/s": 6 * tbytes / (med1 * 1e-3) / 1e9,
                         "frac_hbm_peak": 6 * tbytes / (med1 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "plain_copy_same_bytes_GB/s": 6 * tbytes / (medc1 * 1e-3) / 1e9},
        "head2seq_o": {"bytes": 2 * tbytes, "ms_median": med2, "ms_min": mn2,
                       "GB/s": 2 * tbytes / (med2 * 1e-3) / 1e9,
                       "frac_hbm_peak": 2 * tbytes / (med2 * 1e-3) / 1e9 / PEAK_HBM_GBS,
                       "plain_copy_same_bytes_GB/s": 2 * tbytes / (medc2 * 1e-3) / 1e9},
        # both all-to-alls' layouts of a Ulysses step: their bytes over their
        # summed cold times
        "seq2head_plus_head2seq": {"bytes": 8 * tbytes, "ms": med1 + med2,
                                   "GB/s": 8 * tbytes / ((med1 + med2) * 1e-3) / 1e9,
                                   "frac_hbm_peak": 8 * tbytes / ((med1 + med2) * 1e-3) / 1e9
                                   / PEAK_HBM_GBS}}
    # Ulysses Anything: the video shape at degree 4 (30 heads -> groups of 8, 8, 7, 7)
    Pa = 4
    ysa = [torch.empty(qv.numel(), dtype=qv.dtype, device=dev) for _ in range(3)]
    meda1, _ = cold(lambda: cru.ulysses_seq2head([qv, kv_, vv], Pa, anything=True, out=ysa),
                    args.cold_reps)
    meda2, _ = cold(lambda: cru.ulysses_head2seq(ysa[0], Pa, anything=True, out=ov),
                    args.cold_reps)
    anything_layout = {
        "workload": "video-dit-4276 (B=2, S=4276, H=30, D=64, bf16), P=4: head groups 8,8,7,7",
        "seq2head_qkv": {"bytes": 6 * tbytes, "ms_median": meda1,
                         "GB/s": 6 * tbytes / (meda1 * 1e-3) / 1e9,
                         "frac_hbm_peak": 6 * tbytes / (meda1 * 1e-3) / 1e9 / PEAK_HBM_GBS},
        "head2seq_o": {"bytes": 2 * tbytes, "ms_median": meda2,
                       "GB/s": 2 * tbytes / (meda2 * 1e-3) / 1e9,
                       "frac_hbm_peak": 2 * tbytes / (meda2 * 1e-3) / 1e9 / PEAK_HBM_GBS}}

    def warm(fn, reps=10, batch=10):
        # back to back, as a running job issues them: after a settling
        # quarter second, `reps` batches of `batch` launches between two
        # events; the median batch over batch size.  (Timing one launch at a
        # time with a host sync in between charges each short launch the
        # GPU's idle gap and clock ramp: FLUX-512's 49 us forward reads
        # about 70 us that way.)
        t_w = time.perf_counter()
        while time.perf_counter() - t_w < 0.25:
            for _ in range(batch):
                fn()
            torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(batch):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) / batch)
        return statistics.median(ts)

    # the other bf16 workloads' attention, timed warm like the step (parity
    # workloads: reported, not targets)
    lv = torch.empty(wv.B, wv.H, wv.S, dtype=torch.float32, device=dev)
    fv = attn_flops(wv.B, wv.H, wv.S, wv.S, wv.D)
    tv_full = warm(lambda: cru.attn_fwd_lse(qv, kv_, vv, out=ov, lse=lv))
    ov_u = torch.empty_like(ysv[0][0])
    lv_u = torch.empty(wv.B, wv.H // Pv, wv.S, dtype=torch.float32, device=dev)
    tv_u = warm(lambda: cru.attn_fwd_lse(ysv[0][0], ysv[1][0], ysv[2][0], out=ov_u, lse=lv_u))
    w2 = workload(2)
    q2, k2, v2 = (t.to(dev) for t in make_inputs(2))
    P2 = w2.ulysses_degree
    o2 = torch.empty_like(q2)
    l2 = torch.empty(w2.B, w2.H, w2.S, dtype=torch.float32, device=dev)
    f2 = attn_flops(w2.B, w2.H, w2.S, w2.S, w2.D)
    t2_full = warm(lambda: cru.attn_fwd_lse(q2, k2, v2, out=o2, lse=l2))
    ys2 = [torch.empty(P2, w2.B, w2.S, w2.H // P2, w2.D, dtype=q2.dtype, device=dev)
           for _ in range(3)]
    og2 = torch.zeros(P2, w2.B, w2.S, w2.H // P2, w2.D, dtype=q2.dtype, device=dev)
    lu2 = torch.empty(w2.B, w2.H // P2, w2.S, dtype=torch.float32, device=dev)
    Hp2 = w2.H // P2

    def uly2():
        # as in the step: the share's attention stores straight into its
        # heads of the [B, S, H, D] output (head2seq fused into the store)
        cru.ulysses_seq2head([q2, k2, v2], P2, out=ys2)
        cru.attn_fwd_lse(ys2[0][0], ys2[1][0], ys2[2][0], out=o2[:, :, :Hp2], lse=lu2)

    t2_u = warm(uly2)
    t2b = q2.numel() * q2.element_size()
    m2s, _ = cold(lambda: cru.ulysses_seq2head([q2, k2, v2], P2, out=ys2), args.cold_reps)
    m2h, _ = cold(lambda: cru.ulysses_head2seq(og2, P2, out=o2), args.cold_reps)
    other = {
        "flux-512": {
            "workload": "flux-512 (B=1, S=1536, H=24, D=128, bf16)",
            "full_forward": {"ms_median": t2_full, "TFLOP/s": f2 / (t2_full * 1e-3) / 1e12},
            "ulysses_share_incl_seq2head": {"P": P2, "ms_median": t2_u,
                                            "TFLOP/s": f2 / P2 / (t2_u * 1e-3) / 1e12},
            "cold_layouts": {"note": "9.4 MB per tensor: launch-bound, and cache-resident "
                                     "in a real step",
                             "seq2head_qkv_GB/s": 6 * t2b / (m2s * 1e-3) / 1e9,
                             "head2seq_o_GB/s": 2 * t2b / (m2h * 1e-3) / 1e9}},
        "video-dit-4276": {
            "workload": "video-dit-4276 (B=2, S=4276, H=30, D=64, bf16)",
            "full_forward": {"ms_median": tv_full, "TFLOP/s": fv / (tv_full * 1e-3) / 1e12},
            "ulysses_share_attention": {"P": Pv, "ms_median": tv_u,
                                        "TFLOP/s": fv / Pv / (tv_u * 1e-3) / 1e12}}}
    log(f"[bench] flux-512 full {other['flux-512']['full_forward']['TFLOP/s']:.0f} TFLOP/s; "
        f"video full {other['video-dit-4276']['full_forward']['TFLOP/s']:.0f} TFLOP/s")
    del q2, k2, v2, o2, ys2, og2, lu2, l2, lv, ov_u, lv_u
    del qv, kv_, vv, ysv, ov, ysa, scrub, sink
    torch.cuda.synchronize()

    # Unified attention: FLUX-1024 on a 2 (Ulysses) x 4 (ring) mesh, every
    # device's share on this GPU (seq2head, a fused ring share per head group,
    # head2seq), timed back to back like the other legs
    Pu, Pr = 2, 4
    usp_ws = torch.empty(cru.usp_workspace_bytes(q, Pu, Pr), dtype=torch.uint8, device=dev)
    o_usp = torch.empty_like(q)
    l_usp = torch.empty(B, H, S, dtype=torch.float32, device=dev)
    run_usp = lambda: cru.usp_emulate(q, k, v, Pu, Pr, fused=True, out=o_usp, lse=l_usp,
                                      workspace=usp_ws)
    usp_ms = warm(run_usp)
    usp = {"workload": f"flux-1024, ulysses {Pu} x ring {Pr}, all devices' shares, fused ring",
           "ms_median": usp_ms, "TFLOP/s": f_full / (usp_ms * 1e-3) / 1e12}

    # the step's ring share with partials kept in bf16 (convert_to_fp32 off)
    run_rb = lambda: cru.ring_emulate(q_share, k, v, N, fused=True, convert_to_fp32=False,
                                      out=o_ring, lse=l_ring, workspace=ws)
    rb_ms = warm(run_rb)
    ring_bf16 = {"workload": "flux-1024 ring rank-0 share (576 rows x 8 chunks), bf16 partials",
                 "ms_median": rb_ms, "TFLOP/s": f_ring / (rb_ms * 1e-3) / 1e12,
                 "fp32_partials_ms_in_step": part_ms["ring_share"]}
    del usp_ws, o_usp, l_usp
    torch.cuda.synchronize()

    traffic = counters_traffic()
    achieved = f_full / (attn_mean * 1e-3) / 1e12
    roofline = {"kernel": "attn_fwd_bf16 (full forward, FLUX-1024)", "bound": "mfma",
                "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "algorithmic_flops_per_launch": f_full,
                "avg_launch_ms": attn_mean,
                "launches_timed": args.attn_reps,
                "median_launch_ms": statistics.median(attn_ts),
                "min_launch_ms": min(attn_ts),
                "frac_at_min": f_full / (min(attn_ts) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "in_step_avg_launch_ms": part_ms["attn_full"]}

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host cores")
        cpu = cpu_baseline()
        log(f"[bench] oracle: {cpu['value'] * 1e3:.2f} GFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "flux-1024", "B": B, "H": H, "S": S, "D": D,
                   "ring_degree": N, "ulysses_degree": P,
                   "step": "full forward + ring rank-0 share (8 chunks, one split-KV launch) + "
                           "8-way merge over all rows + Ulysses rank-0 share (P=2, output "
                           "stored straight into its heads of [B, S, H, D]); the ring share "
                           "and the merge on a second stream beside the rest",
                   "step_attention_flops": step_flops},
        "ms_per_step_parts_in_sequence": ms_per_step_seq,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "usp": usp,
        "ring_share_bf16_partials": ring_bf16,
        "cold_merge_bf16_partials": cold_merge_bf16,
        "other_workloads": other,
        "ulysses_anything_cold_layout": anything_layout,
        "parts_ms": part_ms,   # from the steps with the parts in sequence
        "attn_full_tflops": attn_tflops,
        "attn_full_frac_bf16_peak": attn_tflops / PEAK_BF16_TFLOPS,
        "ring_share_tflops": f_ring / (part_ms["ring_share"] * 1e-3) / 1e12,
        "ulysses_share_tflops_incl_layouts": f_uly / (part_ms["ulysses_share"] * 1e-3) / 1e12,
        "merge_all_rows_GB/s_in_step": merge_gbs,
        "cold_merge": cold_merge,
        "cold_layout": cold_layout,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
