"""Benchmark of the XPress Jacobi refinement step on one MI355X.

A step is one xpress_jacobi_step over the synthetic 32-block, full-vocabulary workload (N=32
blocks of B=16 slots, r=256, H=4096, M=512, V=151936): hidden cache, starting block from the base
argmax, then K=15 Jacobi passes (latent + readout GEMM + fused add/argmax), inputs resident in HBM.
The step is recorded once as a HIP graph (xpress_jacobi_step_graph) and replayed, one launch per
step; the eager (kernel-by-kernel) rate is reported beside it, and both must give the same draft.

Prints one JSON line. `value` is Jacobi passes per second of whole steps (per-step setup
included). Also reported:
  * `roofline`: the readout kernel (the dominant kernel: the full-vocabulary MFMA readout, or the
    top-C readout when the workload has C > 0, reading w2[cand] through the ids as the step does),
    algorithmic bytes per launch (w2 + base + lat, or the candidates' w2 rows + base_c + cand +
    lat) over its average duration measured with HIP events on
    the launch stream, against the 8 TB/s HBM peak; its rate against the 2.5 PFLOP/s bf16 MFMA
    peak is in `extra`;
  * `extra.measured_peaks`: achievable yardsticks timed on the same GPU with library kernels
    (a 1 GiB device-to-device copy and a 2 GiB reduction for HBM, an 8192^3 bf16 torch.matmul
    for the matrix cores), and the readout's fractions of them;
  * `cpu_baseline`: the CPU oracle timed on this host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "Jacobi passes/s at N=32,B=16,V=151936; HBM TB/s & MFMA % of peak"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3,
                    help="synthetic workload id (1..5; the tiny workload 1 runs K = B passes)")
    ap.add_argument("--kernel-reps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured streaming-read and bf16-GEMM reference peaks")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="OpenMP threads of the oracle baseline (0: all the host's)")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="also run a plain device-to-device copy of this many MiB three times "
                         "(reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


def traffic_record(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were taken on the
    current kernel source (else None)."""
    f = ROOT / "profiles" / "traffic.json"
    if not f.exists():
        return None
    import hashlib

    rec = json.loads(f.read_text()).get(f"{kernel}@{workload}")
    if not rec:
        return None
    src = ROOT / "jacobi_block_refiner_amd" / "csrc" / rec["source"]
    digest = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    if digest != rec.get("source_sha256_16"):
        return None
    return rec["hbm_bytes_per_launch"]


def main() -> int:
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the pass library has no multi-GPU path here "
              "(blocks shard with zero communication; see the design notes).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from jacobi_block_refiner_amd import synth, upload, xpress

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    wl = synth.WORKLOADS[args.workload]
    # the tiny workload runs to the fixed point in its parity tests; timed here as B passes
    K = wl.K if wl.K > 0 else wl.B
    log(f"workload {wl.name}: drawing inputs")
    inp = synth.make_inputs(wl)
    log("uploading")
    w = upload.weights(inp, dev)
    h = upload.bf16_tensor(inp.h, dev)
    base = upload.base_logits(inp.base, dev)
    anchor = upload.tokens(inp.anchor, dev)
    am1 = upload.tokens(inp.am1, dev)
    blk = torch.zeros(wl.N, wl.B, dtype=torch.int64, device=dev)
    ws = xpress.alloc_workspace(wl.N, wl.B, wl.r, wl.V, wl.C, K, dev)
    torch.cuda.synchronize()

    def step():
        xpress.jacobi_step(w, h, base, anchor, am1, blk, K=K, C=wl.C,
                           flags=xpress.INIT_FROM_BASE, ws=ws)

    def time_steps(fn, label):
        log(f"{label}: warmup {args.warmup} steps")
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        log(f"{label}: timing {args.steps} steps of {K} passes")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return max(e0.elapsed_time(e1), wall * 1e3) / args.steps

    eager_ms = time_steps(step, "eager")
    draft_eager = blk.cpu().numpy()
    # The same step recorded once as a HIP graph and replayed (one launch per step).
    graph = xpress.StepGraph(w, h, base, anchor, am1, blk, K=K, C=wl.C,
                             flags=xpress.INIT_FROM_BASE, ws=ws)
    graph_ms = time_steps(graph.launch, "graph")
    draft = blk.cpu().numpy()
    graph.close()
    if not np.array_equal(draft, draft_eager):
        raise SystemExit("graph replay and eager step disagree")
    ms_per_step = graph_ms
    passes_per_s = K / (ms_per_step / 1e3)

    # Per-kernel timing with HIP events on the launch stream (the current torch stream), same
    # inputs and launch configuration as inside the step.
    rows = wl.rows
    xh = torch.empty(wl.N, wl.B, wl.r, dtype=torch.float32, device=dev)
    xpress.hidden_cache(w, h, xh, ws)
    # the latent layout the step keeps: fragment order for the full-vocabulary readout,
    # row-major for the top-C readout
    lay = xpress.LAT_ROWS if wl.C > 0 else xpress.LAT_FRAGMENTS
    lat = xpress.lat_buffer(wl.N, wl.B, wl.r, lay, dev)
    blk2 = blk.clone()
    xpress.latent_pass(w, blk2, am1, xh, lat, ws, layout=lay)
    ntiles = xpress.readout_tiles(wl.V, rows)
    part = torch.empty(ntiles, rows, 2, dtype=torch.int32, device=dev)

    def timed(fn, reps):
        """Average time per launch of `reps` back-to-back launches between two HIP events on the
        launch stream (torch's current stream, which the binding passes to the library). A spin
        kernel first lets the host queue every launch before the GPU reaches them, so the
        interval holds the kernels and the dispatch gaps between them, not host latency."""
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(10_000_000)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps  # us

    reps = args.kernel_reps
    if wl.C > 0:
        cand = torch.empty(rows, wl.C, dtype=torch.int64, device=dev)
        base_c = torch.empty(rows, wl.C, dtype=torch.bfloat16, device=dev)
        xpress.topc_prepare(w, base, wl.N, wl.C, cand, base_c)  # no gathered copy: the step's form
        fn_readout = lambda: xpress.readout_argmax_topc_ids(w, lat, base_c, cand, blk2)
        fn_reduce = None
        readout_pass = fn_readout
    else:
        fn_readout = lambda: xpress.readout_partials(w, lat, base, part, layout=lay)
        fn_reduce = lambda: xpress.argmax_reduce(part, blk2)
        readout_pass = lambda: xpress.readout_argmax(w, lat, base, blk2, ws, layout=lay)
    fn_latent = lambda: xpress.latent_pass(w, blk2, am1, xh, lat, ws, layout=lay)
    for f in (fn_readout, fn_reduce, fn_latent):
        if f is not None:
            f()
    torch.cuda.synchronize()
    readout_us = timed(fn_readout, reps)
    reduce_us = timed(fn_reduce, reps) if fn_reduce is not None else 0.0
    latent_us = timed(fn_latent, reps)

    # The K-pass loop alone (per-step setup excluded), through the per-pass entry points.
    xpress.initial_block(base, anchor, blk2)

    def loop():
        for _ in range(K):
            xpress.latent_pass(w, blk2, am1, xh, lat, ws, layout=lay)
            readout_pass()

    loop()
    torch.cuda.synchronize()
    loop_us = timed(loop, max(3, args.steps // 2))

    if args.copy_ref_mib > 0:
        src = torch.ones(args.copy_ref_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if wl.C > 0:
        # the candidates' w2 rows (one per row and candidate) + base_c + cand (int64) + lat
        alg_bytes = rows * wl.C * (wl.r * 2 + 2 + 8) + rows * wl.r * 2
        kname = "topc_readout_kernel"
        kdesc = "topc_readout_kernel (GEMV over w2[cand] + base_c add + argmax into blk)"
    else:
        alg_bytes = wl.V * wl.r * 2 + rows * wl.V * 2 + rows * wl.r * 2
        kname = "readout_partial_kernel"
        kdesc = "readout_partial_kernel (bf16 MFMA readout + base add + running argmax)"
    flops = 2.0 * rows * (wl.C if wl.C > 0 else wl.V) * wl.r
    achieved_gbs = alg_bytes / (readout_us * 1e-6) / 1e9
    mfma_tflops = flops / (readout_us * 1e-6) / 1e12
    # The readout's arithmetic intensity caps its MFMA fraction at the HBM peak: a kernel that
    # streamed its bytes at 8 TB/s would reach (flops / bytes) * 8 TB/s of bf16 MFMA work.
    mfma_cap = flops / alg_bytes * HBM_PEAK_GBS * 1e9 / (MFMA_BF16_PEAK_TFLOPS * 1e12)
    # Latent bytes per pass, each operand once: gate, up and down weights, the folded mixer, xh,
    # the 16 gathered rows per block (projected fp32 table rows on the two-launch path, bf16 w1
    # rows plus in_proj's embedding block on the three-launch one) and lat written.
    table_path = wl.N * (wl.M // 64) <= 256
    latent_bytes = (3 * wl.M * wl.r * 2 + wl.B * wl.B * wl.r * 2 + wl.N * wl.B * wl.r * 4
                    + (wl.N * wl.B * wl.r * 4 if table_path else wl.N * wl.B * wl.r * 2 + wl.r * wl.r * 2)
                    + rows * wl.r * 2)
    traffic = traffic_record(kname, wl.name)

    out = {
        "metric": METRIC,
        "value": round(passes_per_s, 2),
        "unit": "passes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded NumPy PCG64 draws; random-init head weights)",
        "config": {"workload": wl.name, "N": wl.N, "B": wl.B, "r": wl.r, "H": wl.H, "M": wl.M,
                   "V": wl.V, "topc": wl.C, "passes_per_step": K},
        "roofline": {
            "kernel": kdesc,
            "bound": "hbm",
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
            "avg_launch_us": round(readout_us, 2),
        },
        "extra": {
            "rows_x_scored_ids_per_s": round(rows * (wl.C if wl.C > 0 else wl.V) * passes_per_s, 1),
            "eager_ms_per_step": round(eager_ms, 4),
            "eager_passes_per_s": round(K / (eager_ms / 1e3), 2),
            "loop_only_passes_per_s": round(K / (loop_us * 1e-6), 1),
            "readout_tflops": round(mfma_tflops, 1),
            "readout_frac_of_bf16_mfma_peak": round(mfma_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "readout_mfma_frac_cap_at_hbm_peak": round(mfma_cap, 4),
            "argmax_reduce_us": round(reduce_us, 2),
            "latent_us": round(latent_us, 2),
            "latent_path": "table (2 launches)" if table_path else "projection (3 launches)",
            "latent_algorithmic_bytes": latent_bytes,
            "latent_frac_of_hbm_peak": round(latent_bytes / (latent_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "latent_share_of_pass": round(latent_us / (loop_us / K), 4),
            "pass_loop_us_per_pass": round(loop_us / K, 2),
            "draft_checksum": int(np.sum(draft * (np.arange(draft.size).reshape(draft.shape) + 1)) % (1 << 61)),
        },
    }

    if not args.no_peaks:
        pk = measured_peaks(dev)
        out["extra"]["measured_peaks"] = pk
        out["extra"]["readout_frac_of_measured_hbm"] = round(achieved_gbs / pk["hbm_GBps"], 4)
        out["extra"]["readout_frac_of_measured_bf16_gemm"] = round(mfma_tflops / pk["bf16_gemm_TFLOPs"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, K, args.cpu_seconds, args.cpu_threads)
    print(json.dumps(out), flush=True)
    return 0


def measured_peaks(dev):
    """Achievable references on this GPU, beside the published peaks: the HBM rate of a reduction
    over 2 GiB and of a 1 GiB device-to-device copy (torch's own kernels; the larger is the
    reference) and the throughput of a large bf16 GEMM (torch.matmul, i.e. hipBLASLt). Library
    kernels, timed here only as yardsticks."""
    import torch

    log("measured peaks: streaming read and bf16 GEMM references")
    x = torch.empty(1 << 29, dtype=torch.float32, device=dev).fill_(1.0)  # 2 GiB
    a = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
    x.sum()
    torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        x.sum()
    e1.record()
    torch.cuda.synchronize()
    read_gbs = 10 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    y = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB copied from half of x
    y.copy_(x[: 1 << 28])
    e0.record()
    for _ in range(10):
        y.copy_(x[: 1 << 28])
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * y.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del y
    e0.record()
    for _ in range(10):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 10 * 2.0 * 8192 ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, a, b
    torch.cuda.empty_cache()
    return {"hbm_GBps": round(max(read_gbs, copy_gbs), 1),
            "sum_read_GBps": round(read_gbs, 1), "sum_kernel": "torch sum over 2 GiB fp32",
            "copy_GBps": round(copy_gbs, 1), "copy": "1 GiB device-to-device copy, read + write bytes",
            "bf16_gemm_TFLOPs": round(gemm_tflops, 1),
            "bf16_gemm": "torch.matmul 8192 x 8192 x 8192 bf16"}


def cpu_baseline(inp, K, budget_s, threads=0):
    """The oracle (plain C, double, OpenMP over rows/blocks) on this host: hidden cache, starting
    block, then whole passes over all rows until about budget_s seconds have been spent (at least
    one pass). threads > 0 limits the OpenMP threads."""
    import numpy as np

    from jacobi_block_refiner_amd import synth
    from oracle import oracle as O

    wl = inp.wl
    if threads > 0:
        O.set_threads(threads)
    log(f"cpu baseline: oracle on {O.max_threads()} threads, budget {budget_s:.0f} s")
    t0 = time.perf_counter()
    L = synth.bf16_round(O.fold_mixer(inp.raw_L).astype(np.float32))
    xh = O.hidden_cache(inp.h, inp.down_h, inp.down_g, inp.in_proj)
    blk = O.initial_block(inp.base, inp.anchor, wl.N, wl.B)
    cand = O.topc_select(inp.base, wl.C) if wl.C > 0 else None
    passes = 0
    while passes < K:
        blk, _, _, _ = O.jacobi(inp, L, xh, blk, K=1, stop_at_fixed_point=False, cand=cand)
        passes += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(passes / dt, 4), "unit": "passes/s", "cores": O.max_threads(),
            "kind": "oracle",
            "sample": f"{wl.name}: hidden cache + starting block{' + top-C select' if wl.C else ''}"
                      f" + {passes} of {K} passes over all {wl.rows} rows ({dt:.1f} s)"}


if __name__ == "__main__":
    sys.exit(main())
