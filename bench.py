"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one call of the C-ABI ``attn_fwd`` over the whole workload (one
kernel launch: tile schedule, Q/K/V staging, QK^T, mask, online softmax, PV,
epilogue).

``--workload hbm_causal_n256_d128`` / ``hbm_noncausal_n512_d128`` measure the
short, bandwidth-bound shapes instead: the line then reports achieved GB/s
(algorithmic bytes: Q, K, V read once, O and LSE written once) against the
8 TB/s HBM peak, and successive launches rotate over three copies of the
inputs at different addresses so that no launch finds its inputs in cache. Inputs are synthetic seeded bf16 tensors already resident in HBM
when the timed region starts. Warm-up: at least W untimed steps and, whatever
W is, at least WARMUP_MIN_S seconds of back-to-back launches, because the
GPU's clock needs that long to settle under this load (the first ~10 launches
run at a high clock, the next ~100 dip, then it holds); the JSON records how
many warm-up launches ran. Then exactly K timed steps launched back to back,
bracketed by a device synchronisation on both sides; the timed region is
measured with two HIP events recorded on the stream the kernel is launched
on, and the average launch duration is that time / K. A second pass of K
launches outside the timed region, with an event after each, gives the
per-launch median, min and max (events between launches add ~2.5 % to each,
which is why they stay out of the timed region).

Prints ONE JSON line on stdout. ``value`` is TFLOP/s with the counted flops
4*B*H*N_q*N_k*d (halved when causal). ``roofline`` prices the kernel against
the MI355X dense bf16 MFMA peak; ``cpu_baseline`` times the fp64 CPU oracle on
a bounded sample of the same workload (test infrastructure, never the product
path).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from workloads import HBM_PROBES, HEADLINE, REFERENCE, WORKLOADS, make_inputs  # noqa: E402

ALL_WORKLOADS = {**WORKLOADS, **HBM_PROBES, **REFERENCE}

MFMA_BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
WARMUP_MIN_S = 0.5                # minimum warm-up time, whatever --warmup says
HBM_PEAK_GBS = 8000.0             # MI355X HBM3E, published
METRIC = "attention fwd TFLOP/s (bf16, causal, N=4096, d=128) + % of MFMA bf16 peak"
HBM_METRIC = "attention fwd achieved HBM GB/s (bf16, short sequences) + % of HBM peak"
FP8_METRIC = "attention fwd TFLOP/s (FP8 E4M3 operands, causal, N=4096, d=128) + % of MFMA fp8 peak"


def fp8_metric_of(w) -> str:
    """The metric string of an FP8 forward line (the headline shape's is FP8_METRIC)."""
    if w.name == HEADLINE:
        return FP8_METRIC
    mask = "causal" if w.causal else "non-causal"
    return f"attention fwd TFLOP/s (FP8 E4M3 operands, {mask}, B={w.B}, H={w.H}, N={w.N_q}, d={w.d}) + % of MFMA fp8 peak"
MFMA_FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, published
BWD_METRIC = "attention bwd TFLOP/s (bf16, dQ dK dV, counted 10*B*H*N_q*N_k*d, halved when causal) + % of MFMA bf16 peak"


def bwd_metric_of(w) -> str:
    """The metric string of a backward line (the headline shape's is BWD_METRIC)."""
    if w.name == HEADLINE:
        return BWD_METRIC
    mask = "causal" if w.causal else ("varlen" if w.seqlens_range is not None else "non-causal")
    return (f"attention bwd TFLOP/s (bf16, dQ dK dV, {mask}, B={w.B}, H={w.H}, N={w.N_q}, d={w.d}, "
            f"counted 10*B*H*N_q*N_k*d, halved when causal) + % of MFMA bf16 peak")
KERNEL_SRC = os.path.join(ROOT, "tiled_attention_16_amd", "csrc", "attn_fwd.hip")
BWD_SRC = os.path.join(ROOT, "tiled_attention_16_amd", "csrc", "attn_bwd.hip")
FP8_SRC = os.path.join(ROOT, "tiled_attention_16_amd", "csrc", "attn_fwd_fp8.hip")
PROFILES = os.path.join(ROOT, "profiles")


def metric_of(w) -> str:
    """The metric string of a forward workload (the headline's is METRIC)."""
    if w.name == HEADLINE:
        return METRIC
    mask = "causal" if w.causal else ("varlen" if w.seqlens_range is not None else "non-causal")
    return f"attention fwd TFLOP/s (bf16, {mask}, B={w.B}, H={w.H}, N={w.N_q}, d={w.d}) + % of MFMA bf16 peak"


def effective_flops(w, inp) -> float:
    """4*d flops per (query, key) pair that a mask allows, summed exactly over
    every (batch, head): keys below seqlens_k[b], rows at or after q_start[b],
    and j <= i under a causal mask. For square causal shapes this is the
    counted N*(N+1)/2 pairs rather than the metric's N*N/2."""
    total = 0
    for b in range(w.B):
        kv = w.N_k if inp.seqlens_k is None else min(max(int(inp.seqlens_k[b]), 0), w.N_k)
        qs = 0 if inp.q_start is None else min(max(int(inp.q_start[b]), 0), w.N_q)
        i = np.arange(qs, w.N_q, dtype=np.int64)
        keys = np.minimum(kv, i + 1) if w.causal else np.full(i.shape, kv, dtype=np.int64)
        total += int(keys.sum())
    return 4.0 * w.d * w.H * total


def warm_up(step, torch, dev, n_min: int, min_s: float = WARMUP_MIN_S):
    """At least n_min launches and at least min_s seconds of them; returns (launches, seconds)."""
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(max(1, min(50, n_min - n)) if n < n_min else 50):
            step()
            n += 1
        torch.cuda.synchronize(dev)
        dt = time.perf_counter() - t0
        if n >= n_min and dt >= min_s:
            return n, dt


def timed(step, torch, stream, dev, steps: int):
    """The timed region: exactly `steps` launches back to back on `stream`
    between two events, synchronised on both sides. Then, outside it, the same
    number of launches with an event after each, for the per-launch median,
    min and max (an event between launches lengthens them by ~2.5 %, so those
    events stay out of the timed region). Returns (bracket ms, per-launch ms
    array, wall s of the timed region)."""
    torch.cuda.synchronize(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize(dev)
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    return e0.elapsed_time(e1), per, wall


def launch_stats(total_ms: float, per, steps: int) -> dict:
    """mean: the timed region / K; median, min, max: per-launch durations from
    the second pass (one event after each launch, outside the timed region)."""
    return {"mean": round(total_ms / steps, 5), "median": round(float(np.median(per)), 5),
            "min": round(float(per.min()), 5), "max": round(float(per.max()), 5),
            "per_launch_pass": f"{steps} more launches, an event after each"}


def kernel_source_hash(path: str = KERNEL_SRC) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_bwd_traffic(workload: str):
    """HBM bytes per attn_bwd call (its three kernels) from the committed counter
    summary, or None when it is missing or covers an older kernel source."""
    path = os.path.join(PROFILES, f"attn_bwd_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not src or src.group(1) != kernel_source_hash(BWD_SRC):
        return None
    m = re.search(rf"traffic_bytes_per_call\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def measured_fp8_traffic(workload: str):
    """HBM bytes per attn_fwd_fp8 launch from the committed counter summary, or
    None when it is missing or covers an older kernel source."""
    path = os.path.join(PROFILES, f"attn_fwd_fp8_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not src or src.group(1) != kernel_source_hash(FP8_SRC):
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when the summary is missing, covers another workload or an older kernel."""
    path = os.path.join(PROFILES, f"attn_fwd_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path, encoding="utf-8").read()
    src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    if not src or src.group(1) != kernel_source_hash():
        return None
    m = re.search(rf"traffic_bytes_per_launch\[{re.escape(workload)}\]:\s*([0-9.eE+]+)", text)
    return float(m.group(1)) if m else None


def cpu_baseline(w, inp, budget_s: float = 12.0):
    """Time the fp64 oracle on whole heads of the workload until the budget is spent."""
    import threadpoolctl

    from oracle import attention, bf16_bits_to_f64

    heads_done = 0
    t0 = time.perf_counter()
    b = 0
    for h in range(w.H):
        sl = None if inp.seqlens_k is None else inp.seqlens_k[b:b + 1]
        qs = None if inp.q_start is None else inp.q_start[b:b + 1]
        attention(bf16_bits_to_f64(inp.q[b:b + 1, h:h + 1]), bf16_bits_to_f64(inp.k[b:b + 1, h:h + 1]),
                  bf16_bits_to_f64(inp.v[b:b + 1, h:h + 1]), float(inp.scale), w.causal, seqlens_k=sl, q_start=qs)
        heads_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.flops() / (w.B * w.H) * heads_done
    blas = [d.get("num_threads", 1) for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle on {heads_done} of {w.B * w.H} (batch, head) pairs of {w.name}, all "
                      f"{w.N_q} rows each, {dt:.1f} s wall; {len(os.sched_getaffinity(0))} host cores visible",
            "seconds": dt}


def copy_calibration(torch, mib: int):
    """Plain device-to-device copies of a known size: each launch reads and writes
    exactly ``mib`` MiB, so the counters it reads calibrate the attention kernel's."""
    n = mib << 20
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)


def run_probes(torch):
    """Instruction-rate microbenchmarks (``libattn_probe.so``): the MFMA-only
    rate and clock, VALU work hidden under MFMAs, v_exp_f32 against v_fma_f32,
    and LDS read rates. Each probe kernel records per-workgroup shader-clock
    cycles (s_memtime) and the 100 MHz real-time counter (s_memrealtime)."""
    import ctypes

    lib = ctypes.CDLL(os.path.join(ROOT, "tiled_attention_16_amd", "libattn_probe.so"))
    lib.attn_probe.restype = ctypes.c_int
    lib.attn_probe.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    stream = torch.cuda.current_stream(dev)
    sink = torch.zeros(512, dtype=torch.float32, device=dev)

    def one(kind, op, nv, threads, iters, blocks=None):
        blocks = blocks or n_cu
        t = torch.zeros(4 * blocks, dtype=torch.int64, device=dev)
        for _ in range(2):   # the first launch warms the clock and loads the code
            rc = lib.attn_probe(kind, op, nv, blocks, threads, iters, t.data_ptr(), sink.data_ptr(),
                                ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"attn_probe({kind}, {op}, {nv}) failed: {rc}")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        lib.attn_probe(kind, op, nv, blocks, threads, iters, t.data_ptr(), sink.data_ptr(),
                       ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1)
        a = t.cpu().numpy().astype(np.float64).reshape(blocks, 4)
        cyc = np.median(a[:, 2] - a[:, 0])
        rt = np.median(a[:, 3] - a[:, 1])
        return ms, cyc, cyc / rt * 100e6   # ms, cycles per workgroup, clock in Hz

    out = {"probe": "gfx950 instruction rates", "compute_units": n_cu,
           "note": "cycles are shader-clock cycles (s_memtime); per SIMD means summed over the waves of a SIMD"}
    iters = 40000
    valu = ((0, "v_fma_f32"), (1, "v_exp_f32"), (2, "v_cvt_pk_bf16_f32"), (3, "v_add_f32"))
    for waves in (1, 2):
        ms, cyc, clk = one(0, 0, 0, 256 * waves, iters)
        flops = n_cu * 4 * waves * iters * 4 * 32768.0
        out[f"mfma_only_{waves}wave_per_simd"] = {
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "clock_ghz": round(clk / 1e9, 3),
            "cycles_per_mfma_per_simd": round(cyc / (iters * 4 * waves), 2)}
        for op, name in valu:
            row = {}
            for nv in (2, 4, 6, 8):
                ms, cyc, clk = one(0, op, nv, 256 * waves, iters // 2)
                row[str(nv)] = round(cyc / (iters // 2 * 4 * waves), 2)
            out[f"cycles_per_mfma_per_simd_with_n_{name}_after_each_{waves}wave_per_simd"] = row
    for chains in (1, 2):
        for waves in (1, 2):
            ms, cyc, clk = one(4, chains, 0, 256 * waves, iters)
            out[f"mfma_{chains}_dependent_chain_{waves}wave_per_simd"] = {
                "cycles_per_mfma_per_simd": round(cyc / (iters * 4 * waves), 2), "clock_ghz": round(clk / 1e9, 3)}
    for waves in (1, 2):
        ms, cyc, clk = one(3, 0, 0, 256 * waves, iters)
        flops = n_cu * 4 * waves * iters * 4 * 16384.0
        out[f"mfma16x16x32_only_{waves}wave_per_simd"] = {
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "clock_ghz": round(clk / 1e9, 3),
            "cycles_per_mfma_per_simd": round(cyc / (iters * 4 * waves), 2)}
    for op, name in valu:
        ms, cyc, clk = one(1, op, 32, 256, iters // 4)
        c1 = cyc / (iters // 4 * 32)
        ms, cyc, clk = one(1, op, 32, 512, iters // 4)
        out[f"{name}_cycles_per_instruction"] = {"1wave_per_simd": round(c1, 2),
                                                 "2waves_per_simd_per_simd": round(cyc / (iters // 4 * 32 * 2), 2)}
    for op, name, nbytes in ((0, "ds_read_b128", 1024), (1, "ds_read_b64_tr_b16", 512)):
        ms, cyc, clk = one(2, op, 0, 512, iters // 8)
        out[f"{name}_bytes_per_clock_per_cu_8waves"] = round(8 * (iters // 8) * 8 * nbytes / cyc, 1)
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-min-s", type=float, default=WARMUP_MIN_S, metavar="S",
                    help="minimum warm-up time in seconds, whatever --warmup is (default %(default)s: the clock "
                         "settles under this load after ~0.05 s); 0 for counter runs under a profiler")
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(ALL_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window", type=int, default=0, metavar="W",
                    help="forward with a dense boolean mask (attn_fwd_masked): key j visible to row i iff "
                         "i - W < j <= i, one mask shared by all heads, packed once before the timed region")
    ap.add_argument("--block-density", type=float, default=0.0, metavar="P",
                    help="block-sparse forward (attn_fwd_block_sparse): each (256-row, 128-key) block "
                         "kept with probability P (seeded, shared by all heads); value counts the kept blocks' work")
    ap.add_argument("--backward", action="store_true",
                    help="time attn_bwd (dQ, dK, dV; its three launches) instead of the forward; O and LSE come "
                         "from one attn_fwd call before the timed region")
    ap.add_argument("--fp8", action="store_true",
                    help="time attn_fwd_fp8 on E4M3 inputs of the workload's shape (per-tensor scales, V "
                         "transposed) instead of the bf16 forward")
    ap.add_argument("--probe", action="store_true",
                    help="instead of the benchmark, run the instruction-rate microbenchmarks (MFMA-only rate and "
                         "clock, VALU work hidden under MFMAs, v_exp_f32 cost, LDS read rates) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device copies of MIB MiB each (the reference "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the attention forward of this library runs on a single "
              "MI355X; multi-GPU runs are not supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        copy_calibration(torch, args.copy_calibration)
        return
    if args.probe:
        run_probes(torch)
        return

    import tiled_attention_16_amd as ta

    ta.load_library()
    w = ALL_WORKLOADS[args.workload]
    hbm_probe = w.name in HBM_PROBES
    inp = make_inputs(w)
    dev = torch.device("cuda:0")

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    q, k, v = to_dev(inp.q), to_dev(inp.k), to_dev(inp.v)
    sl = torch.from_numpy(inp.seqlens_k).to(dev) if inp.seqlens_k is not None else None
    qs = torch.from_numpy(inp.q_start).to(dev) if inp.q_start is not None else None
    sets = [(q, k, v, torch.empty_like(q), torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev))]
    if hbm_probe:   # two more input/output sets at other addresses, launched in turn
        for _ in range(2):
            sets.append(tuple(t.clone() for t in sets[0][:3]) + (torch.empty_like(q), torch.empty_like(sets[0][4])))
    stream = torch.cuda.current_stream(dev)
    n_step = [0]
    packed = None
    bmask = None
    if args.block_density:
        nqb, nkb = -(-w.N_q // 256), -(-w.N_k // 128)
        keep = np.random.default_rng(w.seed + 700).random((1, 1, nqb, nkb)) < args.block_density
        bmask = torch.from_numpy(keep).to(dev)
        # counted flops of the kept blocks: allowed (row, key) pairs inside kept blocks
        i = np.arange(w.N_q)[:, None]
        j = np.arange(w.N_k)[None, :]
        allowed = (j <= i) if w.causal else np.ones((w.N_q, w.N_k), bool)
        kept = keep[0, 0][np.arange(w.N_q) // 256][:, np.arange(w.N_k) // 128]
        sparse_frac = float((allowed & kept).sum()) / float(allowed.sum())
    if args.fp8:
        return bench_fp8(args, torch, ta, w, dev)
    if args.backward:
        return bench_backward(args, torch, ta, w, inp, sets[0], sl, qs, stream, dev, bmask,
                              sparse_frac if args.block_density else 1.0)

    if args.window:
        i = torch.arange(w.N_q, device=dev)[:, None]
        j = torch.arange(w.N_k, device=dev)[None, :]
        packed = ta.pack_mask(((j > i - args.window) & (j <= i))[None, None], stream=stream)

    def step():
        sq, sk, sv, so, slse = sets[n_step[0] % len(sets)]
        n_step[0] += 1
        ta.attn_fwd(sq, sk, sv, causal=w.causal, scale=float(inp.scale), seqlens_k=sl, q_start=qs, out=so,
                    lse=slse, stream=stream, packed_mask=packed, block_mask=bmask)

    n_warm, warm_s = warm_up(step, torch, dev, args.warmup, args.warmup_min_s)
    # The timed region: exactly `steps` launches back to back on one stream,
    # bracketed by events (and a synchronisation on both sides). The average
    # launch duration used for the roofline is the bracket / K.
    total_ms, per, wall = timed(step, torch, stream, dev, args.steps)
    ms_per_step = total_ms / args.steps
    flops = w.flops() * (sparse_frac if args.block_density else 1.0)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    varlen = inp.seqlens_k is not None or inp.q_start is not None
    eff = effective_flops(w, inp) if varlen and not (args.window or args.block_density) else None
    # the roofline prices the work the kernel has to do: for a varlen
    # workload that is the allowed pairs, not the nominal square
    achieved = eff / (ms_per_step * 1e-3) / 1e12 if eff is not None else tflops
    traffic = measured_traffic(w.name) if not (args.window or args.block_density) else None
    if hbm_probe:
        gbs = w.algorithmic_bytes() / (ms_per_step * 1e-3) / 1e9
        result = {
            "metric": HBM_METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.N_q, "N_k": w.N_k, "d": w.d,
                       "causal": w.causal, "varlen": False, "input_sets": len(sets)},
            "tflops": round(tflops, 2),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
            "launch_ms": launch_stats(total_ms, per, args.steps),
            "warmup_run": {"launches": n_warm, "seconds": round(warm_s, 3), "min_seconds": args.warmup_min_s},
            "wall_s_timed": round(wall, 4),
        }
        print(json.dumps(result), flush=True)
        return
    result = {
        "metric": metric_of(w),
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.N_q, "N_k": w.N_k, "d": w.d,
                   "causal": w.causal, "varlen": inp.seqlens_k is not None,
                   **({"dense_mask": f"sliding window {args.window}"} if args.window else {}),
                   **({"block_sparse": f"density {args.block_density}, kept fraction of the counted work "
                                       f"{sparse_frac:.3f}"} if args.block_density else {})},
        "pct_of_mfma_bf16_peak": round(100.0 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        **({"effective": {"flops": eff, "tflops": round(achieved, 2),
                          "fraction_of_nominal": round(eff / w.flops(), 4),
                          "note": "4*d flops per allowed (query, key) pair: keys below seqlens_k[b], "
                                  "rows at or after q_start[b]"}} if eff is not None else {}),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic},
        "launch_ms": launch_stats(total_ms, per, args.steps),
        "warmup_run": {"launches": n_warm, "seconds": round(warm_s, 3), "min_seconds": args.warmup_min_s},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(result), flush=True)


def bench_fp8(args, torch, ta, w, dev):
    """One step = one attn_fwd_fp8 launch over the workload's shape."""
    from workloads import make_fp8

    if w.seqlens_range is not None or w.q_start_batches:
        raise SystemExit("--fp8 takes a workload without variable lengths")
    x = make_fp8(w.B, w.H, w.N_q, w.N_k, w.d, seed=w.seed)
    S = ta.fp8_vt_stride(w.N_k)
    vt = np.zeros((w.B, w.H, w.d, S), dtype=np.uint8)
    vt[..., :w.N_k] = x.vt8
    q, k, vtd = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (x.q8, x.k8, vt))
    o = torch.empty((w.B, w.H, w.N_q, w.d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.H, w.N_q), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    scale = float(w.scale)

    def step():
        ta.attn_fwd_fp8(q, k, vtd, q_descale=x.q_descale, k_descale=x.k_descale, v_descale=x.v_descale,
                        causal=w.causal, scale=scale, out=o, lse=lse, stream=stream)

    n_warm, warm_s = warm_up(step, torch, dev, args.warmup, args.warmup_min_s)
    total_ms, per, wall = timed(step, torch, stream, dev, args.steps)
    ms_per_step = total_ms / args.steps
    tflops = w.flops() / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": fp8_metric_of(w), "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": w.name + "_fp8", "B": w.B, "H": w.H, "N_q": w.N_q, "N_k": w.N_k, "d": w.d,
                   "causal": w.causal, "inputs": "E4M3 codes, one descale per tensor, V transposed"},
        "pct_of_mfma_fp8_peak": round(100.0 * tflops / MFMA_FP8_PEAK_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_FP8_PEAK_TFLOPS, 4), "traffic": measured_fp8_traffic(w.name)},
        "launch_ms": launch_stats(total_ms, per, args.steps),
        "warmup_run": {"launches": n_warm, "seconds": round(warm_s, 3), "min_seconds": args.warmup_min_s},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_fp8(w, x)
    print(json.dumps(result), flush=True)


def cpu_baseline_fp8(w, x, budget_s: float = 12.0):
    """Time the fp64 FP8 oracle on whole heads of the workload until the budget is spent."""
    import threadpoolctl

    from oracle import attention_fp8

    heads_done = 0
    t0 = time.perf_counter()
    for h in range(w.H):
        attention_fp8(x.q8[:1, h:h + 1], x.k8[:1, h:h + 1], x.vt8[:1, h:h + 1], float(w.scale), x.q_descale,
                      x.k_descale, x.v_descale, w.causal)
        heads_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = w.flops() / (w.B * w.H) * heads_done
    blas = [d.get("num_threads", 1) for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(max(blas) if blas else 1), "kind": "oracle",
            "sample": f"fp64 FP8 oracle (decode, then attention) on {heads_done} of {w.B * w.H} (batch, head) "
                      f"pairs of {w.name}, all {w.N_q} rows each, {dt:.1f} s wall", "seconds": dt}


def bench_backward(args, torch, ta, w, inp, tensors, sl, qs, stream, dev, bmask=None, kept=1.0):
    """Time the backward pass: a step is one attn_bwd call (Delta, dQ, dK/dV kernels)."""
    from workloads import make_dout

    q, k, v, o, lse = tensors
    g = torch.from_numpy(make_dout((w.B, w.H, w.N_q, w.d), seed=w.seed + 500).view(np.int16)).to(dev).view(
        torch.bfloat16)
    ta.attn_fwd(q, k, v, causal=w.causal, scale=float(inp.scale), seqlens_k=sl, q_start=qs, out=o, lse=lse,
                stream=stream, block_mask=bmask)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((w.B, w.H, w.N_q, 2), dtype=torch.float32, device=dev)

    def step():
        ta.attn_bwd(q, k, v, o, lse, g, causal=w.causal, scale=float(inp.scale), seqlens_k=sl, q_start=qs, dq=dq,
                    dk=dk, dv=dv, delta=delta, stream=stream, block_mask=bmask)

    n_warm, warm_s = warm_up(step, torch, dev, args.warmup, args.warmup_min_s)
    total_ms, per, wall = timed(step, torch, stream, dev, args.steps)
    ms = total_ms / args.steps
    flops = 2.5 * w.flops() * kept   # five N_q x N_k x d products (S, dP, dV, dK, dQ) against the forward's two
    tflops = flops / (ms * 1e-3) / 1e12
    varlen = inp.seqlens_k is not None or inp.q_start is not None
    eff = 2.5 * effective_flops(w, inp) if varlen and bmask is None else None
    achieved = eff / (ms * 1e-3) / 1e12 if eff is not None else tflops
    result = {
        "metric": bwd_metric_of(w), "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N_q": w.N_q, "N_k": w.N_k, "d": w.d, "causal": w.causal,
                   "varlen": inp.seqlens_k is not None, "pass": "backward",
                   **({"block_sparse": f"density {args.block_density}, kept fraction {kept:.3f}"}
                      if bmask is not None else {})},
        **({"effective": {"flops": eff, "tflops": round(achieved, 2), "fraction_of_nominal": round(eff / (2.5 * w.flops()), 4),
                          "note": "10*d flops per allowed (query, key) pair"}} if eff is not None else {}),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": measured_bwd_traffic(w.name) if bmask is None else None},
        "launch_ms": launch_stats(total_ms, per, args.steps),
        "warmup_run": {"launches": n_warm, "seconds": round(warm_s, 3), "min_seconds": args.warmup_min_s},
        "wall_s_timed": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_backward(w, inp)
    print(json.dumps(result), flush=True)


def cpu_baseline_backward(w, inp, budget_s: float = 12.0):
    """Time the fp64 backward oracle on whole heads of the workload until the budget is spent."""
    import threadpoolctl

    from oracle import attention_bwd, bf16_bits_to_f64
    from workloads import make_dout

    g = make_dout((w.B, w.H, w.N_q, w.d), seed=w.seed + 500)
    heads_done = 0
    t0 = time.perf_counter()
    b = 0
    for h in range(w.H):
        sl = None if inp.seqlens_k is None else inp.seqlens_k[b:b + 1]
        qs = None if inp.q_start is None else inp.q_start[b:b + 1]
        attention_bwd(bf16_bits_to_f64(inp.q[b:b + 1, h:h + 1]), bf16_bits_to_f64(inp.k[b:b + 1, h:h + 1]),
                      bf16_bits_to_f64(inp.v[b:b + 1, h:h + 1]), bf16_bits_to_f64(g[b:b + 1, h:h + 1]),
                      float(inp.scale), w.causal, seqlens_k=sl, q_start=qs)
        heads_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 2.5 * w.flops() / (w.B * w.H) * heads_done
    blas = [d.get("num_threads", 1) for d in threadpoolctl.threadpool_info() if d.get("user_api") == "blas"]
    cores = max(blas) if blas else 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 backward oracle on {heads_done} of {w.B * w.H} (batch, head) pairs of {w.name}, "
                      f"{dt:.1f} s wall; {len(os.sched_getaffinity(0))} host cores visible",
            "seconds": dt}


if __name__ == "__main__":
    main()
