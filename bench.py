"""Bench: batch-invariant bf16 GEMM throughput on one MI355X.

Headline (``value``): TFLOP/s of Y[4096,4096] = X[4096,4096] . W[4096,4096]
(bf16 in, fp32 accumulate, fp32 out; X ~ N(0,1), W ~ N(0,0.02), the
projection workload at K = N = 4096), one step = one GEMM call through the C
ABI with inputs resident in HBM. Also reported:

* ``m_sweep``: TFLOP/s and % of the bf16 MFMA peak for M = 1 ... 4096 at
  K = N = 4096 (small M rotates among buffer sets larger than the 256 MB
  last-level cache, so W is read from HBM; ``us_graph`` is the same rotating
  calls replayed from a captured HIP graph, without the host dispatch of each
  Python call; ``us_warm_llc`` is the same call on one buffer set), with
  achieved algorithmic HBM GB/s and % of the roofline
  bound max(flops / MFMA peak, algorithmic bytes / HBM peak);
* ``other_types_k4096_n4096``: the MXFP8 kernel (E4M3, K-varying E8M0 scales),
  fp16 inputs, bf16 output and int8 inputs at M = 1024 and 4096, each against
  its dense MFMA peak (context, not the metric); MXFP8 and int8 also at M = 1
  and 64 with a cold last-level cache (W rotating over copies, as in
  ``m_sweep``), with algorithmic HBM GB/s (and ``us_graph``, as in the
  sweep); for bf16, MXFP8 and int8 also
  W given as [N, K] rows (MXFP8 scales [N, K/32]), timed in blocks of
  back-to-back launches alternating with blocks of the [K, N] call (median
  over four rounds); ``w_transposed_byte_diffs`` compares the [N, K]-row bf16
  call at M = 4096 with the headline output bit for bit (must be 0);
* ``split_k_context``: the opt-in pinned-chunk split-K handle at small M (cold
  LLC) and on the long-K workload, against the unsplit kernel (context);
* ``rmsnorm_bf16_context``: the batch-invariant RMSNorm (bf16, D = 4096) against
  the HBM peak (context), by events around back-to-back Python calls and, as
  ``us_graph``, around replays of the same calls captured in a HIP graph (the
  kernels without the host dispatch of each call);
* ``paged_attention_decode_context``: the batch-invariant paged attention
  (fixed 256-position KV splits, bf16 cache in blocks of 32, one query token
  per sequence at its last position, fp32 output) for several batch / context
  / head shapes, with algorithmic HBM GB/s against the HBM peak (context);
* ``invariance_byte_diffs``: every row of every sweep result compared with the
  same row of the M = 4096 result (must be 0);
* ``roofline``: the kernel's algorithmic flops per launch over its average
  launch time (HIP events on the launch stream) against the datasheet peak;
* ``cpu_baseline``: the CPU oracle timed on the same workload (rank 0, one
  GPU only), and ``cpu_oracle_m_sweep`` at M = 1, 64, 1024, 4096.

Timing method (``timing`` in the line), the same for every GPU figure: each
point is first warmed for a fixed time (launches back to back for at least
WARM_S seconds, whatever --warmup says, so that the engine clock has settled
at its sustained, power-limited value), then timed as back-to-back blocks of
launches, each block between two HIP events recorded on the launch stream with
no host synchronisation between blocks; a point's time per call is the median
over its blocks. The headline times exactly --steps launches that way (one
bracketed region, split into blocks), and ``value`` is computed from the whole
region (total time / steps); the median block is reported beside it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 / MXFP8 MFMA
PEAK_I8_TOPS = 5033.2       # MI355X dense int8 MFMA (TOP/s)
M_SWEEP = [1, 16, 64, 128, 256, 512, 1024, 2048, 4096]
K = N = 4096


WARM_S = 0.3          # seconds of back-to-back launches before any point is timed
BLOCKS = 5            # timed blocks per point (median taken)


def _warm(torch, fn, seconds=None):
    """Launch fn back to back for at least `seconds` (default WARM_S; synchronising every 20 launches)."""
    seconds = WARM_S if seconds is None else min(seconds, WARM_S)
    if seconds <= 0:
        return
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(20):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def _blocks(torch, stream, fn, reps, blocks=BLOCKS):
    """`blocks` back-to-back blocks of `reps` launches, each between two events on the launch
    stream (no host synchronisation between blocks). Returns (median ms per call over the
    blocks, total ms of the whole region, number of launches)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    ev[0].record(stream)
    i = 0
    for b in range(blocks):
        for _ in range(reps):
            fn(i)
            i += 1
        ev[b + 1].record(stream)
    ev[-1].synchronize()
    per = sorted(ev[b].elapsed_time(ev[b + 1]) / reps for b in range(blocks))
    return per[blocks // 2], ev[0].elapsed_time(ev[-1]), blocks * reps


def _time_point(torch, stream, fn, reps, warm_s=None):
    """One figure of the bench: warm for warm_s seconds, then the median of BLOCKS blocks."""
    _warm(torch, fn, warm_s)
    return _blocks(torch, stream, fn, reps)[0]


def _small_m_entry(kind, m, N, K, t, byts, peak, tg=None):
    """A small-M point of the other types (t in ms per call; byts the algorithmic bytes; tg the
    same calls replayed from a HIP graph, ms per call)."""
    f = 2.0 * m * N * K
    e = {"kind": kind, "M": m, "us": round(t * 1e3, 2), "tflops": round(f / (t * 1e-3) / 1e12, 1),
         "pct_peak": round(100 * f / (t * 1e-3) / 1e12 / peak, 2),
         "hbm_gbs_algorithmic": round(byts / (t * 1e-3) / 1e9, 0), "cold_llc": True}
    if tg is not None:
        e["us_graph"] = round(tg * 1e3, 2)
    return e


def _time_ab(torch, stream, fa, fb, reps=10, rounds=BLOCKS):
    """fa and fb in alternating blocks (same clock and thermal state for both), after warming
    both; returns the median ms per call of each."""
    _warm(torch, lambda i: (fa(i), fb(i)))
    ta, tb = [], []
    for _ in range(rounds):
        ta.append(_blocks(torch, stream, fa, reps, 1)[0])
        tb.append(_blocks(torch, stream, fb, reps, 1)[0])
    return sorted(ta)[rounds // 2], sorted(tb)[rounds // 2]


def _time_graph(torch, stream, fn, reps, replays=BLOCKS):
    """fn called `reps` times inside one captured HIP graph (torch.cuda.CUDAGraph), so the host
    dispatch of each call is out of the timed region; returns the median ms per call over
    `replays` timed replays (after one untimed replay)."""
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(replays):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        g.replay()
        e.record(stream)
        e.synchronize()
        ts.append(s.elapsed_time(e) / reps)
    del g
    return sorted(ts)[replays // 2]


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "bigemm_bf16_kernel_m4096_k4096_n4096_traffic.md")
KERNEL_SOURCE = os.path.join(ROOT, "invariant_gemm_deterministic_amd", "csrc", "bigemm_kernels.hip")


def measured_traffic():
    """HBM-side bytes per launch at M=K=N=4096 from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when the kernel source changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_SUMMARY).read()
        digest = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    vals = dict(ln.split("=", 1) for ln in text.splitlines() if "=" in ln and not ln.startswith(("#", "`", "|")))
    if vals.get("kernel_source_sha256", "").strip() != digest:
        return None
    return int(float(vals["traffic_bytes_per_launch"]))


def _cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_oracle_sweep(X, W, ms=(1, 64, 1024, 4096)):
    """The oracle (fp64 accumulate, OpenMP over rows, as built) on the first M rows of the
    workload at each M: median of three runs below M = 4096, one run at M = 4096."""
    import oracle
    threads = oracle.set_threads(0)
    out = []
    for m in ms:
        ts = []
        for _ in range(1 if m >= 4096 else 3):
            t0 = time.perf_counter()
            oracle.gemm_bf16(X[:m], W, want_s=False)
            ts.append(time.perf_counter() - t0)
        dt = sorted(ts)[len(ts) // 2]
        f = 2.0 * m * W.shape[0] * W.shape[1]
        out.append({"M": m, "s": round(dt, 4), "gflops": round(f / dt / 1e9, 2)})
    return out, threads


def cpu_baseline(sweep, threads, N, K):
    """The headline workload (M = 4096) on the oracle, from the sweep's last point."""
    last = sweep[-1]
    f = 2.0 * last["M"] * N * K
    return {"value": round(f / last["s"] / 1e12, 5), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole M=4096 K=N=4096 bf16 workload, all rows ({f / 1e9:.1f} GFLOP of fp64 "
                      f"accumulation in {last['s']:.1f} s on {threads} threads of {_cpu_model()})"}


def cpu_baseline_one_thread(X, W, rows: int = 16):
    """The same oracle on one thread, on a few rows (context beside the all-cores figure)."""
    import oracle
    threads = oracle.set_threads(0)
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.gemm_bf16(X[:rows], W, want_s=False)
        dt = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    flops = 2.0 * rows * W.shape[0] * W.shape[1]
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows} of {X.shape[0]} rows of the M=4096 K=N=4096 bf16 workload "
                      f"({flops / 1e9:.1f} GFLOP in {dt:.1f} s, fp64 accumulate)"}


def main():
    global WARM_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--m", type=int, default=4096, help="rows of the timed headline call (profiling other M)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="one 256 MiB device copy kernel before the GEMMs (scale reference for byte counters)")
    ap.add_argument("--kind", choices=("bf16", "mxfp8", "i8"), default="bf16",
                    help="input family of the headline call (profiling the MXFP8 or int8 kernel; the bench line is bf16)")
    ap.add_argument("--warm-s", type=float, default=WARM_S,
                    help="seconds of launches before each timed point (profiling runs under counters use 0)")
    args = ap.parse_args()
    WARM_S = args.warm_s
    if args.kind != "bf16" and not args.no_sweep:
        ap.error("--kind mxfp8 / i8 profiles that kernel alone: use it with --no-sweep")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the GEMM would shard by rows "
              f"or columns with no exchange, and no multi-GPU launch is implemented.", file=sys.stderr)
        sys.exit(2)

    import torch
    import invariant_gemm_deterministic_amd as bg
    from bigemm_inputs import SEED_W, SEED_X, normal_bf16

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    Xh = normal_bf16(SEED_X, (4096, K))
    Wh = normal_bf16(SEED_W, (K, N), 0.02)
    X = torch.from_numpy(Xh.view(np.int16)).to(dev)
    W = torch.from_numpy(Wh.view(np.int16)).to(dev)
    Y = torch.empty((4096, N), dtype=torch.float32, device=dev)

    if args.calib_copy:
        # 256 MiB read and 256 MiB written by one elementwise kernel (b = a * 1), so that it shows
        # under the counters as a dispatch (a plain copy_ may run on a DMA engine instead)
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        del a, b

    # ---------------------------------------------------------------- headline
    M = args.m
    assert 1 <= M <= 4096
    Xm, Ym = X[:M], Y[:M]
    head = lambda i: bg.mm(Xm, W, out=Ym)
    head_peak = PEAK_BF16_TFLOPS
    if args.kind == "mxfp8":   # E4M3 with K-varying E8M0 scales on both sides, as in other_types
        from bigemm_inputs import SCALE_SEED_OFFSET, e8m0_scales, normal_e4m3
        Xq = torch.from_numpy(normal_e4m3(SEED_X, (M, K))).to(dev)
        Wq = torch.from_numpy(normal_e4m3(SEED_W, (K, N))).to(dev)
        XSq = torch.from_numpy(e8m0_scales(SEED_X + SCALE_SEED_OFFSET, (M, K // 32), "var")).to(dev)
        WSq = torch.from_numpy(e8m0_scales(SEED_W + SCALE_SEED_OFFSET, (K // 32, N), "var")).to(dev)
        head = lambda i: bg.mm(Xq, Wq, XSq, WSq, out=Ym)
        head_peak = PEAK_FP8_TFLOPS
    elif args.kind == "i8":    # uniform int8 values, as in other_types
        from bigemm_inputs import int_i8
        Xq = torch.from_numpy(int_i8(SEED_X, (M, K))).to(dev)
        Wq = torch.from_numpy(int_i8(SEED_W, (K, N))).to(dev)
        Yq = torch.empty((M, N), dtype=torch.int32, device=dev)
        head = lambda i: bg.mm(Xq, Wq, out=Yq)
        head_peak = PEAK_I8_TOPS
    for i in range(args.warmup):
        head(i)
    if WARM_S > 0:
        _warm(torch, head)                 # the sustained clock, whatever --warmup is
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    nblk = BLOCKS if args.steps % BLOCKS == 0 and args.steps >= BLOCKS else 1
    med_ms, total_ms, n = _blocks(torch, stream, head, args.steps // nblk, nblk)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert n == args.steps
    ms = total_ms / args.steps
    flops = 2.0 * M * N * K
    tflops = flops / (ms * 1e-3) / 1e12
    Yfull = Y.clone()

    # ------------------------------------------------------------------ sweep
    sweep = []
    diffs = 0
    if not args.no_sweep:
        for m in M_SWEEP:
            # enough buffer sets to exceed the 256 MB last-level cache for small M
            set_bytes = 2 * m * K + 2 * K * N + 4 * m * N
            nsets = 1 if m >= 1024 else max(2, int(np.ceil(600e6 / set_bytes)))
            Ws = [W] + [W.clone() for _ in range(nsets - 1)]
            Xs = [X[:m]] + [X[:m].clone() for _ in range(nsets - 1)]
            Ys = [torch.empty((m, N), dtype=torch.float32, device=dev) for _ in range(nsets)]
            reps = max(20, 2 * nsets)
            t = _time_point(torch, stream, lambda i: bg.mm(Xs[i % nsets], Ws[i % nsets], out=Ys[i % nsets]), reps)
            torch.cuda.synchronize()
            if M == 4096:
                for y in Ys:
                    diffs += int((y.view(torch.int32) != Yfull[:m].view(torch.int32)).sum().item())
            f = 2.0 * m * N * K
            byts = 2 * m * K + 2 * K * N + 4 * m * N
            # roofline time: the larger of the MFMA time and the HBM time of the algorithmic bytes
            t_roof = max(f / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
            entry = {"M": m, "us": round(t * 1e3, 2), "tflops": round(f / (t * 1e-3) / 1e12, 1),
                     "pct_peak": round(100 * f / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1),
                     "pct_roofline": round(100 * t_roof / (t * 1e-3), 1),
                     "hbm_gbs_algorithmic": round(byts / (t * 1e-3) / 1e9, 0),
                     "cold_llc": nsets > 1}
            if nsets > 1:
                # the same rotating calls replayed from a HIP graph (no host dispatch per call: where
                # one Python call takes longer to dispatch than the kernel runs, the events above time
                # the host), and the call with one buffer set, W warm in the last-level cache
                tg = _time_graph(torch, stream, lambda i: bg.mm(Xs[i % nsets], Ws[i % nsets], out=Ys[i % nsets]),
                                 reps)
                entry["us_graph"] = round(tg * 1e3, 2)
                tw = _time_point(torch, stream, lambda i: bg.mm(Xs[0], Ws[0], out=Ys[0]), 20, 0.1)
                entry["us_warm_llc"] = round(tw * 1e3, 2)
            sweep.append(entry)
            del Ws, Xs, Ys
            torch.cuda.empty_cache()

    # ------------------------------------------------ opt-in split-K (context)
    # The pinned-chunk split-K handle (not the measured kernel: it sums K in
    # chunks of 512 then adds the chunk sums, so its bytes differ from the
    # unsplit ones; still batch-invariant). Small M with cold-LLC rotation as
    # in the sweep, and the long-K workload [1024,16384] . [16384,1024].
    split = []
    if not args.no_sweep:
        kc = 512
        for m in (1, 16, 64, 128, 256):
            set_bytes = 2 * m * K + 2 * K * N + 4 * m * N
            nsets = max(2, int(np.ceil(600e6 / set_bytes)))
            Ws = [W] + [W.clone() for _ in range(nsets - 1)]
            Ys = [torch.empty((m, N), dtype=torch.float32, device=dev) for _ in range(nsets)]
            ws = torch.empty(bg.bigemm_workspace_size(bg._handle("bf16", 0, bg.BIGEMM_F32, kc), m, N, K),
                             dtype=torch.uint8, device=dev)
            xm = X[:m]
            t = _time_point(torch, stream, lambda i: bg.mm(xm, Ws[i % nsets], out=Ys[i % nsets], k_chunk=kc,
                                                           workspace=ws), max(20, 2 * nsets), 0.1)
            f = 2.0 * m * N * K
            byts = 2 * m * K + 2 * K * N + 4 * m * N
            t_roof = max(f / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
            split.append({"M": m, "K": K, "N": N, "k_chunk": kc, "us": round(t * 1e3, 2),
                          "tflops": round(f / (t * 1e-3) / 1e12, 1),
                          "hbm_gbs_algorithmic": round(byts / (t * 1e-3) / 1e9, 0),
                          "pct_roofline": round(100 * t_roof / (t * 1e-3), 1), "cold_llc": True})
            del Ws, Ys, ws
        XL = torch.from_numpy(normal_bf16(SEED_X, (1024, 16384)).view(np.int16)).to(dev)
        WL = torch.from_numpy(normal_bf16(SEED_W, (16384, 1024)).view(np.int16)).to(dev)
        YL = torch.empty((1024, 1024), dtype=torch.float32, device=dev)
        wsl = torch.empty(bg.bigemm_workspace_size(bg._handle("bf16", 0, bg.BIGEMM_F32, 2048), 1024, 1024, 16384),
                          dtype=torch.uint8, device=dev)
        for kcl in (None, 2048):
            t = _time_point(torch, stream, lambda i: bg.mm(XL, WL, out=YL, k_chunk=kcl, workspace=wsl if kcl else None),
                            20, 0.1)
            f = 2.0 * 1024 * 16384 * 1024
            byts = 2 * 1024 * 16384 * 2 + 4 * 1024 * 1024
            t_roof = max(f / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9))
            split.append({"M": 1024, "K": 16384, "N": 1024, "k_chunk": kcl, "us": round(t * 1e3, 2),
                          "tflops": round(f / (t * 1e-3) / 1e12, 1),
                          "pct_roofline": round(100 * t_roof / (t * 1e-3), 1)})
        del XL, WL, YL, wsl
        torch.cuda.empty_cache()

    # ------------------------------------------------ RMSNorm (context)
    # The batch-invariant RMSNorm (one workgroup per row), bf16, D = 4096;
    # algorithmic bytes 2*M*D read + 2*M*D written + 2*D, against 8 TB/s HBM.
    norm = []
    if not args.no_sweep:
        D = 4096
        G = torch.from_numpy(normal_bf16(SEED_W, (D,)).view(np.int16)).to(dev)
        for m in (1, 128, 4096, 16384):
            XN = torch.from_numpy(normal_bf16(SEED_X + 1, (m, D)).view(np.int16)).to(dev)
            YN = torch.empty_like(XN)
            t = _time_point(torch, stream, lambda i: bg.rmsnorm(XN, G, 1e-6, out=YN), 50, 0.1)
            # the same 50 calls replayed from a captured graph: the kernel without the Python dispatch
            tg = _time_graph(torch, stream, lambda i: bg.rmsnorm(XN, G, 1e-6, out=YN), 50)
            byts = 4 * m * D + 2 * D
            norm.append({"M": m, "D": D, "us": round(t * 1e3, 2), "gbs_algorithmic": round(byts / (t * 1e-3) / 1e9, 0),
                         "pct_hbm_peak": round(100 * byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                         "us_graph": round(tg * 1e3, 2),
                         "pct_hbm_peak_graph": round(100 * byts / (tg * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)})
            del XN, YN

    # ----------------------------------------- paged attention, decode (context)
    # Algorithmic bytes per call: the K and V rows of every context position read
    # once (B*L*Hkv*D*2 bytes each), Q read, O written (fp32), and the split
    # partials (B*H*splits*(D+2)*4 bytes) written once and read once. Inputs are
    # N(0,1) bf16 from torch's seeded generator on the device (the timing does
    # not depend on the values); blocks are assigned by a seeded permutation.
    attn = []
    if not args.no_sweep:
        gen = torch.Generator(device=dev)
        for (B, L, Hq, Hkv, D) in ((64, 4096, 32, 8, 128), (64, 4096, 64, 8, 128), (64, 4096, 8, 8, 128),
                                   (64, 4096, 28, 4, 128), (8, 32768, 32, 8, 128), (1, 131072, 32, 8, 128),
                                   (64, 4096, 32, 8, 64)):
            gen.manual_seed(B * 7 + L)
            bs = 32
            nbps = L // bs
            kc = torch.randn((B * nbps, Hkv, bs, D), device=dev, generator=gen).to(torch.bfloat16)
            vc = torch.randn((B * nbps, Hkv, bs, D), device=dev, generator=gen).to(torch.bfloat16)
            bt = torch.randperm(B * nbps, device=dev, generator=gen).to(torch.int32).reshape(B, nbps)
            q = torch.randn((B, Hq, D), device=dev, generator=gen).to(torch.bfloat16)
            seqs = torch.arange(B, device=dev, dtype=torch.int32)
            poss = torch.full((B,), L - 1, device=dev, dtype=torch.int32)
            o = torch.empty((B, Hq, D), device=dev, dtype=torch.float32)
            need = bg.bigemm_attn_workspace_size(bg._kv_layout(kc, bt), B, Hq, L)
            wsa = torch.empty(need, dtype=torch.uint8, device=dev)

            def call(i):
                bg.paged_attention(q, kc, vc, bt, seqs, poss, max_context=L, out=o, workspace=wsa)

            t = _time_point(torch, stream, call, 20, 0.1)
            byts = 4 * B * L * Hkv * D + 2 * B * Hq * D + 4 * B * Hq * D + 2 * need
            attn.append({"B": B, "context": L, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "us": round(t * 1e3, 2),
                         "gbs_algorithmic": round(byts / (t * 1e-3) / 1e9, 0),
                         "pct_hbm_peak": round(100 * byts / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)})
            del kc, vc, bt, q, o, wsa
        torch.cuda.empty_cache()

    # ------------------------------------------------------- MXFP8 (context)
    mx = []
    wt_byte_diffs = None
    if not args.no_sweep:
        from bigemm_inputs import SCALE_SEED_OFFSET, e8m0_scales, normal_e4m3
        Xm = torch.from_numpy(normal_e4m3(SEED_X, (4096, K))).to(dev)
        Wm = torch.from_numpy(normal_e4m3(SEED_W, (K, N))).to(dev)
        XS = torch.from_numpy(e8m0_scales(SEED_X + SCALE_SEED_OFFSET, (4096, K // 32), "var")).to(dev)
        WS = torch.from_numpy(e8m0_scales(SEED_W + SCALE_SEED_OFFSET, (K // 32, N), "var")).to(dev)
        WmT, WST = Wm.t().contiguous(), WS.t().contiguous()   # W and its scales as [N, K] and [N, K/32] rows
        # The two W layouts in alternating launches, so that both see the same thermal state of the chip.
        wmt, wst = WmT.t(), WST.t()
        for m in (1024, 4096):
            xm, xs, ym = Xm[:m], XS[:m], Y[:m]   # views made once: the timed calls do no slicing on the host
            fa = lambda i: bg.mm(xm, Wm, xs, WS, out=ym)
            fb = lambda i: bg.mm(xm, wmt, xs, wst, out=ym)
            ta, tb = _time_ab(torch, stream, fa, fb)
            f = 2.0 * m * N * K
            for kind, t in (("mxfp8", ta), ("mxfp8_w_transposed", tb)):
                mx.append({"kind": kind, "M": m, "us": round(t * 1e3, 2), "tflops": round(f / (t * 1e-3) / 1e12, 1),
                           "pct_peak": round(100 * f / (t * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 1)})
        # small M with a cold last-level cache (W and its scales rotate over copies, as in the sweep)
        for m in (1, 64):
            byts = m * K + K * N + (m * K + K * N) // 32 + 4 * m * N
            nsets = max(2, int(np.ceil(600e6 / byts)))
            Wc = [Wm] + [Wm.clone() for _ in range(nsets - 1)]
            WSc = [WS] + [WS.clone() for _ in range(nsets - 1)]
            xm, xs, ym = Xm[:m], XS[:m], Y[:m]
            fn = lambda i: bg.mm(xm, Wc[i % nsets], xs, WSc[i % nsets], out=ym)
            t = _time_point(torch, stream, fn, max(20, 2 * nsets))
            tg = _time_graph(torch, stream, fn, max(20, 2 * nsets))
            mx.append(_small_m_entry("mxfp8", m, N, K, t, byts, PEAK_FP8_TFLOPS, tg))
            del Wc, WSc
        del Xm, Wm, XS, WS, WmT, WST
        # fp16 inputs and int8 inputs on the same tile skeleton, and bf16 output (context)
        from bigemm_inputs import int_i8, normal_f16
        X16 = torch.from_numpy(normal_f16(SEED_X, (4096, K))).view(torch.float16).to(dev)
        W16 = torch.from_numpy(normal_f16(SEED_W, (K, N), 0.02)).view(torch.float16).to(dev)
        Xi = torch.from_numpy(int_i8(SEED_X, (4096, K))).to(dev)
        Wi = torch.from_numpy(int_i8(SEED_W, (K, N))).to(dev)
        Yi = torch.empty((4096, N), dtype=torch.int32, device=dev)
        Yb = torch.empty((4096, N), dtype=torch.bfloat16, device=dev)
        # W given as [N, K] rows (a linear layer's weight layout): same bytes as the [K, N] call
        WT = W.t().contiguous()
        for _ in range(2):
            bg.mm(X, WT.t(), out=Y)
        torch.cuda.synchronize()
        wt_byte_diffs = int((Y.view(torch.int32) != Yfull.view(torch.int32)).sum().item()) if M == 4096 else None
        WiT = Wi.t().contiguous()
        wt, wit = WT.t(), WiT.t()
        for m in (1024, 4096):
            x16, xb, xi, ym, yb, yi = X16[:m], X[:m], Xi[:m], Y[:m], Yb[:m], Yi[:m]
            for name, fn, peak in (("f16", lambda i: bg.mm(x16, W16, out=ym), PEAK_BF16_TFLOPS),
                                   ("bf16_out", lambda i: bg.mm(xb, W, out=yb), PEAK_BF16_TFLOPS)):
                t = _time_point(torch, stream, fn, 20)
                f = 2.0 * m * N * K
                mx.append({"kind": name, "M": m, "us": round(t * 1e3, 2), "tflops": round(f / (t * 1e-3) / 1e12, 1),
                           "pct_peak": round(100 * f / (t * 1e-3) / 1e12 / peak, 1)})
            # each W layout against the other in alternating launches (bf16, int8)
            for names, fa, fb, peak in ((("bf16", "bf16_w_transposed"), lambda i: bg.mm(xb, W, out=ym),
                                         lambda i: bg.mm(xb, wt, out=ym), PEAK_BF16_TFLOPS),
                                        (("i8", "i8_w_transposed"), lambda i: bg.mm(xi, Wi, out=yi),
                                         lambda i: bg.mm(xi, wit, out=yi), PEAK_I8_TOPS)):
                ta, tb = _time_ab(torch, stream, fa, fb)
                f = 2.0 * m * N * K
                for name, t in zip(names, (ta, tb)):
                    mx.append({"kind": name, "M": m, "us": round(t * 1e3, 2),
                               "tflops": round(f / (t * 1e-3) / 1e12, 1),
                               "pct_peak": round(100 * f / (t * 1e-3) / 1e12 / peak, 1)})
        for m in (1, 64):   # int8 at small M, cold last-level cache
            byts = m * K + K * N + 4 * m * N
            nsets = max(2, int(np.ceil(600e6 / byts)))
            Wc = [Wi] + [Wi.clone() for _ in range(nsets - 1)]
            xi, yi = Xi[:m], Yi[:m]
            fn = lambda i: bg.mm(xi, Wc[i % nsets], out=yi)
            t = _time_point(torch, stream, fn, max(20, 2 * nsets))
            tg = _time_graph(torch, stream, fn, max(20, 2 * nsets))
            mx.append(_small_m_entry("i8", m, N, K, t, byts, PEAK_I8_TOPS, tg))
            del Wc
        del X16, W16, Xi, Wi, WiT, Yi, Yb, WT

    line = {
        "metric": "TFLOP/s vs M (1-4096) at K=N=4096, % MFMA peak; invariance byte-diffs=0",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "ms_per_step_median_block": round(med_ms, 5),
        "timing": f"{WARM_S:g} s of back-to-back launches, then the timed launches in back-to-back blocks "
                  f"between HIP events on the launch stream; headline: {args.steps} launches in {nblk} "
                  f"block(s), value = total / steps; every other point: median of {BLOCKS} blocks",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "mxfp8": "e4m3", "i8": "int8"}[args.kind],
        "data": "synthetic",
        "config": {"workload": (f"bf16 projection GEMM Y[{M},4096] = X[{M},4096] . W[4096,4096], "
                                "X~N(0,1), W~N(0,0.02), fp32 accumulate and output, batch-invariant fixed tile")
                   if args.kind == "bf16" else
                   (f"MXFP8 GEMM Y[{M},4096] = X[{M},4096] . W[4096,4096], E4M3 from N(0,1) with K-varying "
                    "E8M0 scales in [-4,4] on both sides, fp32 accumulate and output (profiling run)")
                   if args.kind == "mxfp8" else
                   (f"int8 GEMM Y[{M},4096] = X[{M},4096] . W[4096,4096], uniform int8, int32 accumulate and "
                    "output (profiling run)"),
                   "M": M, "N": N, "K": K,
                   "tile": list(bg.bigemm_get_config(
                       bg._handle("i8", 0, bg.BIGEMM_I32) if args.kind == "i8"
                       else bg._handle("bf16" if args.kind == "bf16" else "mx", 0)))},
        "pct_mfma_peak": round(100 * tflops / head_peak, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": head_peak,
                     "unit": "TFLOP/s", "frac": round(tflops / head_peak, 4),
                     "traffic": measured_traffic() if M == 4096 and args.kind == "bf16" else None},
        "m_sweep": sweep,
        "other_types_k4096_n4096": mx,
        "w_transposed_byte_diffs": wt_byte_diffs if mx else None,
        "split_k_context": split,
        "rmsnorm_bf16_context": norm,
        "paged_attention_decode_context": attn,
        "invariance_byte_diffs": diffs if sweep else None,
        "timed_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        sweep_cpu, threads = cpu_oracle_sweep(Xh, Wh)
        line["cpu_baseline"] = cpu_baseline(sweep_cpu, threads, N, K)
        line["cpu_oracle_m_sweep"] = {"cores": threads, "cpu": _cpu_model(), "k": K, "n": N, "points": sweep_cpu}
        line["cpu_baseline_one_thread"] = cpu_baseline_one_thread(Xh, Wh)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
