#!/usr/bin/env python3
"""Throughput of strict selected-token logprob + entropy on one MI355X.

Headline workload: the logits path on Qwen3-vocabulary data -- T = 1024 rows of
V = 151936 fp32 logits ~ N(0, 3^2) with 1% of rows spiked (+25 at one column), targets
drawn from softmax(X); one step = one rlk_logprob_from_logits call (logprob + entropy,
vocab split 1).  Inputs are resident in HBM before timing starts.

Also reported on the same JSON line:
  roofline      HBM roofline of the row-reduce kernel: algorithmic bytes per launch
                (1024 x 607760 B: every logit once, the target id, two fp32 outputs)
                over its mean launch time (HIP events on the launch stream), vs 8 TB/s;
  cpu_baseline  the float64 CPU oracle on the same rows, on a thread pool over every usable
                host core (at most 16), with the host's CPU model and BLAS recorded;
  fused         the fused linear-logp path on the Qwen3-8B shape (T = 2048, d = 4096,
                V = 151936 bf16) as tokens/s and fraction of the 2.5 PFLOP/s bf16
                MFMA peak (2 T V d flops per call); fused.configs adds the Qwen3-Next
                shape (T = 1024, d = 2048) and the large ragged batch (T = 16384,
                d = 4096, temperature 0.7, its own H and W, and targets drawn from the
                oracle's tempered softmax as stored with the parity goldens), each with its
                fraction next to the 50% target; fused.logprob_only times the same call
                without the entropy output; fused.cpu_baseline times the oracle on every
                row of the T = 1024, d = 2048 shape; fused.configs[*].vendor_gemm times
                the same 2 T V d flops as one plain torch.mm H W^T (hipBLASLt) with bf16
                and with fp32 logits out, for context (no softmax epilogue, logits written);
  splits        ms per call of the logits path at vocab splits 2, 4, 8;
  bf16_logits   the same rows rounded to bf16 through rlk_logprob_from_logits_bf16
                (1024 x 303888 B per call) as GB/s against 8 TB/s;
  backward      rlk_logprob_backward_from_logits on the same rows (gradient of
                g_lp * logprob + g_ent * entropy): ms per call and GB/s over its
                algorithmic bytes (one read of the logits, one write of the gradient);
  fused_backward  rlk_linear_logprob_backward on the Qwen3-8B shape: ms per call and
                TFLOP/s over 3 x 2 T V d flops (logits, dH, dW) vs the bf16 peak.
  ceilings      what the chip sustains outside the logprob kernels (include/rlk_probes.h):
                a streaming read of the same 622 MB of logits (GB/s) and a register-only
                bf16 MFMA loop on random operands (TFLOP/s); roofline.frac_of_probe and
                fused.roofline.frac_of_probe state the kernels' rates against them.

The MFMA-bound calls (fused, fused.configs, fused_backward) are timed after about 0.13 s of
back-to-back warmup calls: after an idle gap the chip's clock takes ~30 ms of MFMA load to
settle (at T = 2048 the first five calls run at ~40% of peak, from the fifteenth on ~49.5%),
and a training loop runs at the settled clock.

    python bench.py [--gpus 1] [--steps 100] [--warmup 20] [--no-fused]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s selected-logprob+entropy at V=151936; % HBM BW / % MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# Targets: the logits path at >= 70% of the HBM peak, the fused path at >= 50% of the bf16
# MFMA peak (reported next to each fused shape's fraction).
HBM_TARGET_FRAC = 0.70
FUSED_TARGET_FRAC = 0.50
BYTES_PER_TOKEN_LOGITS = 151936 * 4 + 8 + 8
BYTES_PER_TOKEN_BF16 = 151936 * 2 + 8 + 8
BYTES_PER_TOKEN_BACKWARD = 151936 * 4 * 2 + 8 + 4 + 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "row_reduce_T1024_V151936_traffic.json")
TRAFFIC_FILE_BF16 = os.path.join(ROOT, "profiles", "row_reduce_bf16_T1024_V151936_traffic.json")
# Warmup calls of the fused path at T = 2048 (~0.13 s; see the module docstring).
FUSED_WARMUP_CALLS = 60
# MFMA probe: one workgroup per CU, ~5 ms per launch (20 warmup launches, 5 timed).
MFMA_PROBE_BLOCKS = 256
MFMA_PROBE_ITERS = 32768
TRAFFIC_SOURCES = ["entropy_rlk_logprob_amd/csrc/rlk_logits.hip",
                   "entropy_rlk_logprob_amd/csrc/rlk_state.hpp",
                   "entropy_rlk_logprob_amd/csrc/rlk_launch.hpp"]


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sources_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path: str = TRAFFIC_FILE):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    there is none or the kernel source changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != sources_hash(TRAFFIC_SOURCES):
        return None
    return t.get("bytes_per_launch")


def time_calls(fn, steps: int, warmup: int):
    """Mean ms per call over `steps` back-to-back calls, from one pair of HIP events
    recorded on the current stream (the stream the library launches on) around all of them;
    also the wall-clock ms per call over the same region (host launch cost included)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end) / steps, wall_ms / steps


def fused_config_rate(lib, h, w, t, tau, steps, warmup):
    """ms per rlk_linear_logprob call and fraction of the bf16 MFMA peak on one shape."""
    import torch
    from entropy_rlk_logprob_amd import binding
    T, d = h.shape
    V = w.shape[0]
    lp = torch.empty(T, dtype=torch.float32, device="cuda")
    ent = torch.empty(T, dtype=torch.float32, device="cuda")
    ws = torch.empty(lib.workspace_bytes(binding.OP_LINEAR, T, V, d, 1), dtype=torch.uint8,
                     device="cuda")
    log(f"timing fused path T={T} d={d}: steps {steps}")
    ms, _ = time_calls(lambda: lib.linear_logprob(h, w, t, tau, 1, out=(lp, ent), workspace=ws),
                       steps, warmup)
    tf = 2.0 * T * V * d / (ms / 1e3) / 1e12
    del ws
    log(f"timing torch.mm (hipBLASLt) T={T} d={d}")
    return {"n_tokens": T, "hidden": d, "temperature": tau, "ms_per_call": round(ms, 4),
            "tokens_per_s": round(T / (ms / 1e3), 1), "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "vendor_gemm": vendor_gemm_rate(h, w, min(steps, 5), 3)}


def vendor_gemm_rate(h, w, steps, warmup):
    """The same 2 T V d flops as one plain GEMM H W^T through torch.mm (hipBLASLt), with the
    logits written out in bf16 and in fp32: context for the fused path's fraction of peak (the
    library GEMM has no softmax epilogue, but it writes T x V logits).  h, w: bf16 bits."""
    import torch
    hb, wb = h.view(torch.bfloat16), w.view(torch.bfloat16)
    T, d = hb.shape
    V = wb.shape[0]
    out = {}
    for name, dt in (("bf16_out", torch.bfloat16), ("fp32_out", torch.float32)):
        ms, _ = time_calls(lambda dt=dt: torch.mm(hb, wb.t(), out_dtype=dt), steps, warmup)
        tf = 2.0 * T * V * d / (ms / 1e3) / 1e12
        out[name] = {"ms_per_call": round(ms, 4), "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
    torch.cuda.empty_cache()
    return out


def host_description() -> dict:
    """The host the CPU baseline runs on: usable cores, CPU model, BLAS library."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [d for d in threadpool_info() if d.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
    except Exception:
        pass
    return {"os_cpu_count": os.cpu_count(), "usable_cores": len(os.sched_getaffinity(0)),
            "cpu_model": model, "blas": blas}


def cpu_workers() -> int:
    """Threads for the CPU baseline: every core this process may use, at most 16 (one GPU's
    share of a shared host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool_map(fn, blocks, workers):
    """Run fn over row blocks on `workers` threads, each with a one-thread BLAS (so that the
    pool, not BLAS, spreads the work and the cores are not oversubscribed); NumPy releases
    the GIL inside its array operations."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(max_workers=workers) as ex:
            return list(ex.map(fn, blocks))


def cpu_baseline(case):
    """The float64 oracle as it stands on the logits workload: all rows, in row blocks on a
    thread pool, repeated until at least 10 s have passed."""
    import oracle
    n = case.x.shape[0]
    workers = cpu_workers()
    blocks = [(r, min(n, r + 16)) for r in range(0, n, 16)]

    def run(b):
        return oracle.logprob_entropy(case.x[b[0]:b[1]], case.targets[b[0]:b[1]],
                                      case.temperature)

    passes = 0
    t0 = time.perf_counter()
    while True:
        _pool_map(run, blocks, workers)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or passes >= 50:
            break
    return {"value": round(passes * n / dt, 1), "unit": "tokens/s", "cores": workers,
            "kind": "oracle", "host": host_description(),
            "sample": f"all {n} rows of the logits workload, {passes} passes ({dt:.1f} s); "
                      f"oracle.logprob_entropy (NumPy float64) on 16-row blocks over a pool "
                      f"of {workers} threads"}


def cpu_baseline_fused(fc, tau):
    """The float64 oracle as it stands on the fused T=1024, d=2048 workload: every row, the
    weight widened to float64 once (timed), then row blocks on a thread pool, each block one
    float64 matrix product against the whole weight and the row definition."""
    import numpy as np

    import oracle
    from entropy_rlk_logprob_amd import synthetic as S
    n = fc.h_bits.shape[0]
    workers = cpu_workers()
    h = S.bf16_bits_to_f32(fc.h_bits)
    w = S.bf16_bits_to_f32(fc.w_bits)
    rows = max(1, n // workers)
    blocks = [(r, min(n, r + rows)) for r in range(0, n, rows)]
    t0 = time.perf_counter()
    w64 = np.asarray(w, dtype=np.float64)

    def run(b):
        return oracle.linear_logprob_entropy(h[b[0]:b[1]], w64, fc.targets[b[0]:b[1]], tau,
                                             block=b[1] - b[0])

    _pool_map(run, blocks, workers)
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 1), "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "host": host_description(),
            "sample": f"all {n} rows of {S.WORKLOADS[3].name}, once ({dt:.1f} s); "
                      f"oracle.linear_logprob_entropy (NumPy float64, one-thread BLAS per "
                      f"worker) on {len(blocks)} row blocks over a pool of {workers} threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-fused", action="store_true")
    ap.add_argument("--no-fused-configs", action="store_true",
                    help="skip the T=1024 d=2048 and T=16384 d=4096 fused shapes")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run 5 device-to-device copies of the logits tensor (a plain copy of "
                         "known size, used to calibrate the FETCH_SIZE/WRITE_SIZE counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(vocab splits are emulated on one GPU); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from entropy_rlk_logprob_amd import binding
    from entropy_rlk_logprob_amd import synthetic as S

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    lib = binding.load()
    log("generating logits workload T=1024 V=151936")
    case = S.logits_workload(2)
    T, V = case.x.shape
    x = torch.from_numpy(case.x).cuda()
    t = torch.from_numpy(case.targets).cuda()
    # The bf16 rows are made here, not just before their line: a 311 MB allocation there left
    # the device idle for about 20 ms, and the calls after an idle spell run through a power
    # transient (56 -> 72 -> 62 us per call over the first hundred bf16 calls, against 55-56 us
    # under continuous load).
    xh = x.to(torch.bfloat16)
    lp = torch.empty(T, dtype=torch.float32, device="cuda")
    ent = torch.empty(T, dtype=torch.float32, device="cuda")

    def step():
        lib.logprob_from_logits(x, t, 1.0, 1, out=(lp, ent))

    log(f"timing logits path: warmup {args.warmup}, steps {args.steps}")
    k_ms, wall_ms = time_calls(step, args.steps, args.warmup)
    tokens_per_s = T / (wall_ms / 1e3)
    alg_bytes = T * BYTES_PER_TOKEN_LOGITS
    achieved = alg_bytes / (k_ms / 1e3) / 1e9
    traffic = measured_traffic()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": "row_reduce_kernel<float,8,true>",
                "kernel_ms": round(k_ms, 5), "algorithmic_bytes": alg_bytes,
                "target_frac": HBM_TARGET_FRAC}

    probes = binding.load_probes()
    sink = torch.empty(probes.READ_BLOCKS * probes.THREADS, dtype=torch.float32, device="cuda")
    log("timing the streaming-read probe")
    r_ms, _ = time_calls(lambda: probes.stream_read(x, sink), 20, 5)
    read_gbs = x.numel() * 4 / (r_ms / 1e3) / 1e9
    ceilings = {"hbm_stream_read": {
        "achieved": round(read_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(read_gbs / HBM_PEAK_GBS, 4),
        "probe": "rlk_probe_stream_read: the 622 MB logits read once, 2048 x 256 threads, "
                 "16-byte non-temporal loads"}}
    roofline["frac_of_probe"] = round(achieved / read_gbs, 4)

    if args.copy_probe:
        dst = torch.empty_like(x)
        for _ in range(5):
            dst.copy_(x)
        torch.cuda.synchronize()
        del dst

    splits = {}
    for sp in (2, 4, 8):
        wsb = lib.workspace_bytes(binding.OP_FROM_LOGITS, T, V, 0, sp)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        fn = (lambda sp=sp, ws=ws: lib.logprob_from_logits(x, t, 1.0, sp, out=(lp, ent),
                                                           workspace=ws))
        ms, _ = time_calls(fn, max(5, args.steps // 5), 10)
        splits[str(sp)] = round(ms, 5)

    log("timing backward of the logits path")
    gl = torch.randn(T, generator=torch.Generator().manual_seed(7)).cuda()
    ge = torch.randn(T, generator=torch.Generator().manual_seed(8)).cuda()
    gout = torch.empty_like(x)
    bw_ws = torch.empty(max(1, lib.workspace_bytes(binding.OP_BACKWARD_FROM_LOGITS, T, V, 0, 1)),
                        dtype=torch.uint8, device="cuda")
    states = lib.row_states_buffer(T)
    lib.logprob_from_logits(x, t, 1.0, 1, out=(lp, ent), row_states=states)
    g_ms, g_wall = time_calls(lambda: lib.logprob_backward_from_logits(
        x, t, 1.0, 1, gl, ge, out=gout, workspace=bw_ws, row_states=states),
        max(5, args.steps // 2), 5)
    g_ms_re, _ = time_calls(lambda: lib.logprob_backward_from_logits(
        x, t, 1.0, 1, gl, ge, out=gout, workspace=bw_ws), max(5, args.steps // 4), 3)
    g_gbs = T * BYTES_PER_TOKEN_BACKWARD / (g_ms / 1e3) / 1e9
    backward = {"ms_per_call": round(g_ms, 5), "tokens_per_s": round(T / (g_wall / 1e3), 1),
                "row_states": "saved by the forward call",
                "ms_per_call_recomputing_row_states": round(g_ms_re, 5),
                "kernels": "logits_grad_kernel (+ row_reduce_kernel when recomputing)",
                "roofline": {"bound": "hbm", "achieved": round(g_gbs, 1), "peak": HBM_PEAK_GBS,
                             "unit": "GB/s", "frac": round(g_gbs / HBM_PEAK_GBS, 4),
                             "algorithmic_bytes": T * BYTES_PER_TOKEN_BACKWARD}}
    del gout, bw_ws

    log("timing bf16-logits path")
    bsteps = max(5, args.steps)
    b_ms, b_wall = time_calls(lambda: lib.logprob_from_logits(xh, t, 1.0, 1, out=(lp, ent)),
                                 bsteps, 10)
    b_gbs = T * BYTES_PER_TOKEN_BF16 / (b_ms / 1e3) / 1e9
    bf16 = {"ms_per_call": round(b_ms, 5), "tokens_per_s": round(T / (b_wall / 1e3), 1),
            "roofline": {"bound": "hbm", "achieved": round(b_gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(b_gbs / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic(TRAFFIC_FILE_BF16),
                         "kernel": "row_reduce_kernel<unsigned short,8,true>",
                         "algorithmic_bytes": T * BYTES_PER_TOKEN_BF16}}
    del xh, x

    fused = None
    fused_backward = None
    if not args.no_fused:
        log("generating fused workload T=2048 d=4096 V=151936 (bf16)")
        fc = S.fused_workload(4)
        h = torch.from_numpy(fc.h_bits.view(np.int16)).cuda()
        w = torch.from_numpy(fc.w_bits.view(np.int16)).cuda()
        tt = torch.from_numpy(fc.targets).cuda()
        Tf, d = fc.h_bits.shape
        flp = torch.empty(Tf, dtype=torch.float32, device="cuda")
        fent = torch.empty(Tf, dtype=torch.float32, device="cuda")
        fws = torch.empty(lib.workspace_bytes(binding.OP_LINEAR, Tf, V, d, 1),
                          dtype=torch.uint8, device="cuda")

        def fstep():
            lib.linear_logprob(h, w, tt, 1.0, 1, out=(flp, fent), workspace=fws)

        fsteps = max(5, min(args.steps, 20))
        log(f"timing fused path: steps {fsteps}")
        f_ms, f_wall = time_calls(fstep, fsteps, FUSED_WARMUP_CALLS)
        log("timing fused path, logprob only")
        flo_ms, _ = time_calls(
            lambda: lib.linear_logprob(h, w, tt, 1.0, 1, with_entropy=False, out=(flp, None),
                                       workspace=fws), fsteps, 5)
        log("timing fused backward")
        fgl = torch.randn(Tf, generator=torch.Generator().manual_seed(9)).cuda()
        fge = torch.randn(Tf, generator=torch.Generator().manual_seed(10)).cuda()
        fdh = torch.empty((Tf, d), dtype=torch.float32, device="cuda")
        fdw = torch.empty((V, d), dtype=torch.float32, device="cuda")
        fbws = torch.empty(lib.workspace_bytes(binding.OP_LINEAR_BACKWARD, Tf, V, d, 1),
                           dtype=torch.uint8, device="cuda")

        fstates = lib.row_states_buffer(Tf)
        lib.linear_logprob(h, w, tt, 1.0, 1, out=(flp, fent), workspace=fws, row_states=fstates)

        def bstep(states=fstates):
            lib.linear_logprob_backward(h, w, tt, 1.0, 1, fgl, fge, out=(fdh, fdw),
                                        workspace=fbws, row_states=states)

        b_ms_f, b_wall_f = time_calls(bstep, max(3, min(args.steps, 10)), 20)
        b_ms_re, _ = time_calls(lambda: bstep(None), 3, 1)
        bflops = 3 * 2.0 * Tf * V * d
        btf = bflops / (b_ms_f / 1e3) / 1e12
        fused_backward = {"ms_per_call": round(b_ms_f, 4),
                          "tokens_per_s": round(Tf / (b_wall_f / 1e3), 1),
                          "row_states": "saved by the forward call",
                          "ms_per_call_recomputing_row_states": round(b_ms_re, 4),
                          "roofline": {"bound": "mfma", "achieved": round(btf, 1),
                                       "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                       "frac": round(btf / BF16_PEAK_TFLOPS, 4),
                                       "flops_per_call": bflops}}
        del fdh, fdw, fbws
        flops = 2.0 * Tf * V * d
        tflops = flops / (f_ms / 1e3) / 1e12
        fused = {"workload": S.WORKLOADS[4].name, "n_tokens": Tf, "hidden": d, "vocab": V,
                 "ms_per_call": round(f_ms, 4), "tokens_per_s": round(Tf / (f_wall / 1e3), 1),
                 "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                              "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(tflops / BF16_PEAK_TFLOPS, 4),
                              "flops_per_call": flops},
                 "logprob_only": {"ms_per_call": round(flo_ms, 4),
                                  "frac": round(flops / (flo_ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS,
                                                4)}}
        log("timing the MFMA probe")
        msink = torch.empty(MFMA_PROBE_BLOCKS * probes.THREADS, dtype=torch.float32,
                            device="cuda")
        mflops = probes.mfma(MFMA_PROBE_BLOCKS, MFMA_PROBE_ITERS, msink)
        m_ms, _ = time_calls(lambda: probes.mfma(MFMA_PROBE_BLOCKS, MFMA_PROBE_ITERS, msink),
                             5, 20)
        mtf = mflops / (m_ms / 1e3) / 1e12
        ceilings["mfma_bf16"] = {
            "achieved": round(mtf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(mtf / BF16_PEAK_TFLOPS, 4),
            "probe": "rlk_probe_mfma: register-only v_mfma_f32_32x32x16_bf16, 8 accumulators "
                     "per wave, random bf16 operands rotated every step, one workgroup of 4 "
                     "waves per CU"}
        fused["roofline"]["frac_of_probe"] = round(tflops / mtf, 4)
        fused_backward["roofline"]["frac_of_probe"] = round(btf / mtf, 4)
        log("timing torch.mm (hipBLASLt) T=2048 d=4096")
        fused_configs = {S.WORKLOADS[4].name: {"ms_per_call": fused["ms_per_call"],
                                               "frac": fused["roofline"]["frac"],
                                               "vendor_gemm": vendor_gemm_rate(h, w, 5, 3)}}
        if not args.no_fused_configs:
            del w
            # The large ragged batch with its own inputs: H and W from its seed, and the
            # targets of every row drawn from the oracle's tempered softmax, as stored by
            # tests/golden/make_fused_goldens.py (the same targets the parity tests use).
            w5 = S.WORKLOADS[5]
            log(f"generating fused workload {w5.name}")
            fc5 = S.fused_workload(5)
            with np.load(os.path.join(ROOT, "tests", "golden", f"fused_{w5.name}.npz"),
                         allow_pickle=False) as z:
                t5 = torch.from_numpy(z["targets"]).cuda()
            h5 = torch.from_numpy(fc5.h_bits.view(np.int16)).cuda()
            w5d = torch.from_numpy(fc5.w_bits.view(np.int16)).cuda()
            del fc5
            fused_configs[w5.name] = fused_config_rate(lib, h5, w5d, t5, w5.temperature, 3, 8)
            del h5, w5d, t5
            log("generating fused workload T=1024 d=2048 V=151936 (bf16)")
            fc3 = S.fused_workload(3)
            h3 = torch.from_numpy(fc3.h_bits.view(np.int16)).cuda()
            w3 = torch.from_numpy(fc3.w_bits.view(np.int16)).cuda()
            t3 = torch.from_numpy(fc3.targets).cuda()
            fused_configs[S.WORKLOADS[3].name] = fused_config_rate(lib, h3, w3, t3, 1.0, 20, 200)
            del h3, w3, t3
            if not args.no_cpu:
                log("CPU baseline of the fused path (oracle, T=1024 d=2048)")
                fused["cpu_baseline"] = cpu_baseline_fused(fc3, 1.0)
            del fc3
        for c in fused_configs.values():
            c["target_frac"] = FUSED_TARGET_FRAC
            c["meets_target"] = c["frac"] >= FUSED_TARGET_FRAC
        fused["configs"] = fused_configs
        del h

    cpu = None if args.no_cpu else cpu_baseline(case)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": S.WORKLOADS[2].name, "n_tokens": T, "vocab": V,
                   "vocab_splits": 1, "temperature": 1.0, "logits_dtype": "f32",
                   "parallelism": "single-gpu"},
        "backend": lib.backend_id(),
        "roofline": roofline, "cpu_baseline": cpu, "fused": fused,
        "fused_backward": fused_backward, "splits_ms": splits,
        "bf16_logits": bf16, "backward": backward, "ceilings": ceilings,
        "device": dict(name=torch.cuda.get_device_name(0), **probes.device_info()),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
