"""Benchmark of the diagonal-SSM layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one full forward of the layer by the convolution view (kernel
generation, kernel spectrum, FFT convolution with the D skip) on the
long-sequence workload B=4, H=128, N=64, L=16384 (log_re scaled by 0.1),
seeded synthetic inputs already resident in device memory.  Several
input/output sets (over 512 MB in all) are rotated so that the 256 MB
Infinity Cache does not hold a step's inputs from an earlier step.

Prints ONE JSON line:
* value: elements (B*H*L) per second over the K timed steps, plain library
  calls between two device synchronisations (no events inside);
* step_ms_distribution: median / p10 / p90 of the per-step GPU time over at
  least 100 further steps, each bracketed by an event pair on the launch
  stream;
* roofline: the dominant kernel (the convolution) on its algorithmic bytes
  (u read + y written, 8 bytes per element) against the 8 TB/s HBM peak, its
  average duration from GPU-stamped events around it over K more steps on the
  launch stream, with the vector-ALU co-limit beside it;
* extra.configs: every workload on both paths (the DLR workloads by the FFT
  and the recurrence views, the S5 workload by the scan and FFT methods),
  plus the continuous-time S5, the gradients, the recurrence view's sequence
  split on few long rows, streaming prefill and a device copy;
* cpu_baseline: the float64 oracle on the host's cores (a process pool over
  channels), with the single-core figure, taken before the GPU is touched.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# Seconds of untimed calls before each side workload's timed region (its clocks at
# steady state; the headline takes an exact count of warm-up steps instead).
WARM_S = 0.1

HBM_PEAK_GBS = 8000.0
# FP32 vector rate without packed FP32 (the library is compiled without it):
# 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz.  The published
# 157.3 TFLOP/s counts packed FMAs (two per lane per clock).
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
FP32_PUBLISHED_TFLOPS = 157.3
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense
METRIC = "SSM layer fwd elements/s (B·H·L) and achieved HBM GB/s vs peak, L=16384"
WORKLOAD = "long_sequence"
COMPUTE_NOTE = ("float32 I/O and FFT convolution (float32 vector ALU); the kernel generator "
                "and the chunked recurrence view run their contractions on fp16 matrix cores "
                "with split operands (fp16 hi + lo, 3 products, float32 accumulation: ~22 "
                "significant bits per operand)")

# Counter record of the convolution kernel (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# calibrated on a device copy of known size), valid only for the kernel
# sources it was taken on.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "conv_kernel_long_sequence_counters.md")
KERNEL_SOURCES = ["long_convolution_sequence_amd/csrc/fft.hip",
                  "long_convolution_sequence_amd/csrc/dssm_internal.h",
                  "long_convolution_sequence_amd/csrc/gen_twiddles.py",
                  "long_convolution_sequence_amd/build.py"]


def kernel_sources_digest():
    import hashlib

    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_record(name):
    """The committed counter record `name` of the convolution (a JSON line in
    the counters profile), or None when there is none or the kernel sources
    changed since it was taken."""
    tag = name + "-record: "
    try:
        with open(TRAFFIC_RECORD) as f:
            for ln in f:
                if ln.startswith(tag):
                    rec = json.loads(ln[len(tag):])
                    if rec.get("sources_sha256") == kernel_sources_digest():
                        return rec
    except (OSError, ValueError):
        pass
    return None


def measured_traffic():
    """HBM bytes per launch of the convolution (FETCH_SIZE + WRITE_SIZE,
    calibrated), from the counter record."""
    rec = counter_record("traffic")
    return rec["fetch_bytes"] + rec["write_bytes"] if rec else None


def measured_valu():
    """The convolution's vector-ALU issue against its measured busy cycles
    (SQ_INSTS_VALU, SQ_WAVES, SQ_BUSY_CU_CYCLES from the counter record): the
    clock the CUs sustained during the launch, the share of their cycles the
    vector ALU issues (a wave64 instruction holds its SIMD 4 cycles, and a
    CU's waves spread over 4 SIMDs), and the launch time the VALU
    instructions alone need at that clock."""
    rec = counter_record("valu")
    if not rec:
        return None
    issue = rec["valu_instr_per_wave"] * 4 * rec["waves_per_cu"] / 4  # cycles per SIMD
    clock = rec["busy_cycles_per_cu"] / (rec["launch_us"] * 1e-6)
    return {"sustained_clock_ghz": clock / 1e9,
            "valu_issue_frac": issue / rec["busy_cycles_per_cu"],
            "valu_floor_ms_at_sustained_clock": issue / clock * 1e3,
            "source": "counter record (SQ_INSTS_VALU, SQ_WAVES, SQ_BUSY_CU_CYCLES)"}


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on the host, in a pool of fresh worker
# processes, run before the GPU is used
# ---------------------------------------------------------------------------
def _oracle_rows(job):
    """One pool job: the oracle form `kind` on a slice of channels of the
    workload (u [B, h, L] and the parameters of those channels)."""
    import oracle

    kind, u, log_re, log_im, W, D, bi = job
    f = oracle.dlr_recurrence if kind == "rec" else oracle.dlr_direct
    return f(u, log_re, log_im, W, D, bi)


def _one_blas_thread():
    """Pool initialiser: one BLAS thread per worker process (the pool is the
    parallelism; several workers' spinning BLAS threads oversubscribe the
    cores and can stall the pool)."""
    import numpy  # noqa: F401  (loads the BLAS library the limit applies to)
    from threadpoolctl import threadpool_limits

    threadpool_limits(1)


def _jobs(kind, x, bi, hs_groups):
    return [(kind, x["u"][:, hs], x["log_re"][:, hs], x["log_im"][:, hs], x["W"][:, hs],
             x["D"][:, hs], bi) for hs in hs_groups]


def _groups(n, parts):
    step = max(1, -(-n // parts))
    return [list(range(h, min(n, h + step))) for h in range(0, n, step)]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(x, bi, direct_channels):
    """The float64 oracle as it stands, timed on the host:
    * the sequential recurrence (dlr_recurrence) over the whole workload, in a
      process pool (one worker per usable core, at most 16, one BLAS thread
      each) whose workers take groups of channels, and on one core;
    * the direct O(L^2) sum (dlr_direct) on `direct_channels` channels, pooled
      and on one core (a quarter of them).
    Returns the report and the pooled recurrence output (the reference the GPU
    outputs are then compared with)."""
    import multiprocessing as mp

    import numpy as np

    B, H, L = x["u"].shape
    # the host's usable cores, at most the 16 of a one-GPU machine's share
    cores = max(1, min(len(os.sched_getaffinity(0)), 16))
    # fresh worker processes (spawn), one BLAS thread each
    ctx = mp.get_context("spawn")
    saved = {k: os.environ.get(k) for k in ("OPENBLAS_NUM_THREADS", "OMP_NUM_THREADS")}
    os.environ.update(OPENBLAS_NUM_THREADS="1", OMP_NUM_THREADS="1")  # inherited by the workers
    try:
        pool = ctx.Pool(cores, initializer=_one_blas_thread)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    with pool:
        pool.map(_oracle_rows, _jobs("rec", x, bi, [[0]] * cores))  # workers up and importing
        jobs = _jobs("rec", x, bi, _groups(H, cores))
        t = time.perf_counter()
        parts = pool.map(_oracle_rows, jobs)
        t_rec = time.perf_counter() - t
        ref = np.concatenate(parts, axis=1)
        jobs = _jobs("dir", x, bi, _groups(direct_channels, cores))
        t = time.perf_counter()
        pool.map(_oracle_rows, jobs)
        t_dir = time.perf_counter() - t
    from threadpoolctl import threadpool_limits

    d1 = max(1, direct_channels // 4)
    with threadpool_limits(1):  # one core
        t = time.perf_counter()
        _oracle_rows(_jobs("rec", x, bi, [list(range(H))])[0])
        t_rec1 = time.perf_counter() - t
        t = time.perf_counter()
        _oracle_rows(_jobs("dir", x, bi, [list(range(d1))])[0])
        t_dir1 = time.perf_counter() - t
    elems = B * H * L
    report = {
        "value": elems / t_rec,
        "unit": "elements/s",
        "cores": cores,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": ("oracle.dlr_recurrence (float64 sequential recurrence) over the whole "
                   "workload (%d elements) in a pool of %d processes over channel groups: "
                   "%.2f s; on one core %.2f s (%.3g elements/s).  oracle.dlr_direct (O(L^2) "
                   "sum) on %d of %d channels pooled: %.3g elements/s; on one core (%d "
                   "channels): %.3g elements/s"
                   % (elems, cores, t_rec, t_rec1, elems / t_rec1, direct_channels, H,
                      B * direct_channels * L / t_dir, d1, B * d1 * L / t_dir1)),
        "single_core_value": elems / t_rec1,
    }
    return report, ref


def errors_vs(y, ref):
    import numpy as np

    d = y.astype(np.float64) - ref
    return {"rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)),
            "max_over_rms": float(np.max(np.abs(d)) / np.sqrt(np.mean(ref ** 2)))}


# ---------------------------------------------------------------------------
# GPU timing helpers
# ---------------------------------------------------------------------------
def wall_ms(call, steps, warmup, min_warm_s=0.0):
    """Mean wall ms per call over `steps` plain calls (after `warmup` calls, and
    then more until `min_warm_s` seconds of them have run), between two device
    synchronisations.  The chip's clocks ramp up under sustained load over tens
    of milliseconds: the long-sequence step takes ~65 us over its first ~150
    calls and 58-60 us at steady state."""
    import torch

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    k = warmup
    while time.perf_counter() - t0 < min_warm_s:
        for _ in range(10):
            call(k)
            k += 1
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        call(k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def step_distribution(call, iters, hip):
    """Per-call GPU time of `iters` calls, each bracketed by a start/stop event
    pair recorded on the launch stream: median, p10, p90 (ms)."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream().cuda_stream
    evs = [hip.create(2) for _ in range(iters)]
    for k in range(iters):
        hip.record(evs[k][0], stream)
        call(k)
        hip.record(evs[k][1], stream)
    torch.cuda.synchronize()
    ms = np.array([hip.ms(e[0], e[1]) for e in evs])
    for e in evs:
        hip.destroy(e)
    return {"iters": iters, "median_ms": float(np.median(ms)),
            "p10_ms": float(np.percentile(ms, 10)), "p90_ms": float(np.percentile(ms, 90))}


def stage_times(call_timed, nstage, iters, hip, only=None):
    """Mean ms of each stage of a timing-variant call over `iters` calls (the
    GPU stamps each stage's start and end: hipExtLaunchKernel events).  With
    `only`, just that stage is stamped (one stamped launch per call)."""
    import torch

    evs = [hip.create(2 * nstage) for _ in range(iters)]
    for k in range(iters):
        e = list(evs[k])
        if only is not None:
            e = [h if i // 2 == only else None for i, h in enumerate(e)]
        call_timed(k, e)
    torch.cuda.synchronize()
    out = []
    for s in range(nstage):
        if only is not None and s != only:
            out.append(None)
            continue
        out.append(sum(hip.ms(e[2 * s], e[2 * s + 1]) for e in evs) / iters)
    for e in evs:
        hip.destroy(e)
    return out


def rotated(t, total_bytes_min=600 << 20):
    """Copies of tensor t (input sets) and as many outputs, enough that one
    round of inputs and outputs exceeds the 256 MB MALL twice over."""
    import torch

    per = 2 * t.numel() * t.element_size()
    r = max(2, -(-total_bytes_min // per)) if per >= (1 << 20) else 1
    us = [t] + [t.clone() for _ in range(r - 1)]
    ys = [torch.empty_like(t) for _ in range(r)]
    return us, ys


def hbm(elems, ms):
    gbs = 8.0 * elems / (ms * 1e-3) / 1e9
    return gbs, gbs / HBM_PEAK_GBS


def conv_alg_flop(B, H, L, ndir=1):
    """Algorithmic flops of the FFT convolution per launch: per (b, h) row two
    real FFTs of n = 2L points (2 n log2 n - 4 n each), the spectrum product on
    L + 1 bins (6 each) and the D skip (2 per element); the bidirectional
    kernel is folded into the one spectrum, so ndir does not double it."""
    import math

    n = 2 * L
    return B * H * (2 * (2 * n * math.log2(n) - 4 * n) + 6 * (L + 1) + 2 * L)


def chunk_mfma_flop(B, H, L, ndir):
    """fp16 matrix-core flops the chunked recurrence executes: per (direction,
    channel, batch row) and block of 64 chunks of 64 steps, 4 waves x (48 + 72)
    v_mfma_f32_16x16x32_f16 of 16384 flops (three products per split pair)."""
    nblk = -(-(-(-L // 64)) // 64)
    return ndir * H * B * nblk * 4 * (48 + 72) * 16384


def dlr_config(name, steps, hip):
    """Both paths of a DLR workload: plain-call wall ms per forward over rotated
    sets, the step distribution, the dominant kernel's stamped duration and the
    HBM fraction on algorithmic bytes; errors against the float64 recurrence
    on sampled channels."""
    import numpy as np
    import torch

    import oracle
    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config(name)
    B, H, N, L, bi = c["B"], c["H"], c["N"], c["L"], c["bidirectional"]
    x = inputs.inputs_for(c)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us, ys = rotated(dev["u"])
    R = len(us)
    elems = B * H * L
    hs = sorted(set([0, H // 2, H - 1]))  # oracle sample: 3 channels, every batch row
    ref = oracle.dlr_recurrence(x["u"][:, hs], x["log_re"][:, hs], x["log_im"][:, hs],
                                x["W"][:, hs], x["D"][:, hs], bi)
    out = {"workload": name, "B": B, "H": H, "N": N, "L": L, "bidirectional": bool(bi),
           "elements": elems, "rotated_sets": R}
    for path, fn, op in (("fft", bd.forward_fft, bd.OP_FFT), ("scan", bd.forward_scan, bd.OP_SCAN)):
        ws = torch.empty(max(256, bd.workspace_size(op, B, H, N, L, bi)), dtype=torch.uint8,
                         device="cuda")

        def call(k, fn=fn, ws=ws):
            fn(us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"], bidirectional=bi,
               y=ys[k % R], workspace=ws)

        def call_timed(k, evs, path=path, ws=ws):
            bd.forward_timed(path, us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                             evs, bidirectional=bi, y=ys[k % R], workspace=ws)

        ms = wall_ms(call, steps, 3, WARM_S)
        dist = step_distribution(call, max(100, steps), hip)
        # (the chunked form for N <= 64 is one kernel: its first stage has none)
        chunked = path == "scan" and N <= 64
        st = stage_times(call_timed, 2, max(20, steps // 2), hip, only=1 if chunked else None)
        gbs, frac = hbm(elems, ms)
        kgbs, kfrac = hbm(elems, st[1])
        call(0)
        torch.cuda.synchronize()
        y = ys[0].cpu().numpy()[:, hs]
        p = {"ms_per_forward": ms, "elements_per_s": elems / (ms * 1e-3),
             "layer_hbm_gbs": gbs, "layer_hbm_frac": frac, "step_distribution": dist,
             "stage_ms": ({"kernel_spectrum": st[0], "conv": st[1]} if path == "fft"
                          else {"scan": st[1]} if chunked else {"consts": st[0], "scan": st[1]}),
             "kernel_hbm_gbs": kgbs, "kernel_hbm_frac": kfrac,
             "vs_oracle_sampled_channels": errors_vs(y, ref)}
        if path == "fft":
            p["conv_alu_frac_nonpacked"] = conv_alg_flop(B, H, L) / (st[1] * 1e-3) / 1e12 / ALU_PEAK_TFLOPS
        elif N <= 64:
            tf = chunk_mfma_flop(B, H, L, 1 + bi) / (st[1] * 1e-3) / 1e12
            p["kernel"] = "chunk_kernel (chunked matrix-core form)"
            p["mfma_f16_tflops_executed"] = tf
            p["mfma_f16_frac_of_dense_peak"] = tf / FP16_MFMA_PEAK_TFLOPS
        out[path] = p
    return out


def scan_split(hip, reps=5):
    """The recurrence view when rows are few and the sequence long (B=1, H=4,
    N=64, L=2^20, one and two directions): the sequence cut into segments
    (a state-only pass, the join of the segments' states into the state each
    one enters, the output pass) against the walk of one workgroup per row it
    replaces.  That walk is bounded from below by kernel times of whole rows:
    one row of one block alone, and 512 rows (one workgroup each, two to a
    CU) of one and of two blocks, whose difference is the CU time of two
    blocks -- a block of a lone workgroup takes at least half of it."""
    import numpy as np
    import torch

    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    def kernel_ms(B, H, N, L, bi, seed):
        x = inputs.dlr_inputs(B, H, N, L, bidirectional=bi, seed=seed, re_scale=0.1)
        dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
        y = torch.empty_like(dev["u"])
        ws = torch.empty(max(256, bd.workspace_size(bd.OP_SCAN, B, H, N, L, bi)),
                         dtype=torch.uint8, device="cuda")

        def call_timed(k, evs):
            bd.forward_timed("scan", dev["u"], dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                             evs, bidirectional=bi, y=y, workspace=ws)

        call_timed(0, [None] * 4)
        return stage_times(call_timed, 2, reps, hip, only=1)[1]

    out = {}
    L = 1 << 20
    one_row = kernel_ms(1, 1, 64, 4096, False, 51)
    rows1 = kernel_ms(1, 512, 64, 4096, False, 52)
    rows2 = kernel_ms(1, 512, 64, 8192, False, 52)
    blk_lone_min = max(rows2 - rows1, 0.0) / 2
    for bi in (False, True):
        ms = kernel_ms(1, 4, 64, L, bi, 53)
        ndir = 2 if bi else 1
        walk = ndir * (one_row + (L // 4096 - 1) * blk_lone_min)
        out["bidirectional" if bi else "unidirectional"] = {
            "B": 1, "H": 4, "N": 64, "L": L, "kernels_ms": ms,
            "elements_per_s": 4 * L / (ms * 1e-3),
            "one_workgroup_per_row_walk_ms_lower_bound": walk,
            "speedup_over_walk_at_least": walk / ms,
        }
    out["walk_bound_from"] = {"one_row_one_block_ms": one_row,
                              "rows512_one_block_ms": rows1, "rows512_two_blocks_ms": rows2,
                              "lone_block_ms_at_least": blk_lone_min}
    return out


def stream_prefill(steps, hip):
    """Streaming prefill on the long-sequence workload: dssm_forward_scan_state
    from a random state (state read, outputs, last state written back)."""
    import numpy as np
    import torch

    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config("long_sequence")
    B, H, N, L = c["B"], c["H"], c["N"], c["L"]
    x = inputs.inputs_for(c)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us, ys = rotated(dev["u"])
    R = len(us)
    x0 = torch.from_numpy(inputs.dlr_state(B, H, N, seed=3)).cuda()
    ws = torch.empty(max(256, bd.workspace_size(bd.OP_SCAN, B, H, N, L)), dtype=torch.uint8,
                     device="cuda")

    def call(k):
        bd.forward_scan_state(us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"], x0,
                              y=ys[k % R], workspace=ws)

    ms = wall_ms(call, steps, 3, WARM_S)
    return {"workload": "long_sequence", "ms_per_prefill": ms,
            "elements_per_s": B * H * L / (ms * 1e-3), "path": "chunked form, state in and out"}


def _s5_fused_segments(B, H, P, L):
    """Segments per batch row of the fused S5 scan (0 where the fused form does
    not apply), as the library plans them: about 256 workgroups of whole
    64-step tiles.  Used only to attribute the flops of the report."""
    if not (P <= 128 and H <= 256 and H * L <= 1 << 29):
        return 0
    nt = -(-L // 64)
    want = max(1, -(-256 // B))
    seg_tiles = max(1, -(-nt // want))
    return -(-nt // seg_tiles)


def s5_config(steps, hip):
    """The S5 workload by both methods: plain-call wall ms over rotated sets and
    the four stages' stamped durations; errors against the float64 recurrence
    on one batch row."""
    import numpy as np
    import torch

    import oracle
    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config("s5_mimo")
    B, H, P, L = c["B"], c["H"], c["P"], c["L"]
    x = inputs.inputs_for(c)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us, ys = rotated(t["u"], 700 << 20)
    R = len(us)
    elems = B * H * L
    ref = oracle.s5_recurrence(x["u"][:1], x["lam"], x["Bbar"], x["C"], x["D"])
    gemm_flop = 2.0 * (2 * P) * H * L * B  # one projection, as float32 products
    out = {"workload": "s5_mimo", "B": B, "H": H, "P": P, "L": L, "elements": elems,
           "rotated_sets": R}
    for name, method in (("scan", bd.S5_SCAN), ("fft", bd.S5_FFT), ("fused", bd.S5_FUSED)):
        ws = torch.empty(bd.s5_workspace_size(B, H, P, L, method), dtype=torch.uint8,
                         device="cuda")

        def call(k, ws=ws, method=method):
            bd.s5_forward(us[k % R], t["lam"], t["Bbar"], t["C"], t["D"], y=ys[k % R],
                          workspace=ws, method=method)

        def call_timed(k, evs, ws=ws, method=method):
            bd.s5_forward(us[k % R], t["lam"], t["Bbar"], t["C"], t["D"], y=ys[k % R],
                          workspace=ws, method=method, events=evs)

        ms = wall_ms(call, steps, 2, WARM_S)
        st = stage_times(call_timed, 4, max(10, steps // 2), hip)
        call(0)
        torch.cuda.synchronize()
        y = ys[0].cpu().numpy()[:1]
        gbs, frac = hbm(elems, ms)
        out[name] = {
            "ms_per_forward": ms, "elements_per_s": elems / (ms * 1e-3),
            "layer_hbm_gbs": gbs, "layer_hbm_frac": frac,
            "mfma_f16_dense_peak_tflops": FP16_MFMA_PEAK_TFLOPS,
            "vs_oracle_batch_row_0": errors_vs(y, ref),
        }
        if name == "fused":
            # one kernel per pass: the state-only pass runs the input
            # projection and the recurrence on every segment but the last;
            # the output pass runs both projections and the recurrence (and
            # joins the segment states)
            f = 1.0 - 1.0 / _s5_fused_segments(B, H, P, L)
            out[name]["form"] = "v and x on chip"
            out[name]["stage_ms"] = {"pack": st[0], "state_only_pass": st[1],
                                     "lambda_powers": st[2], "output_pass": st[3]}
            # the projections run 3 fp16 products per float32 product
            out[name]["state_pass_mfma_f16_tflops_executed"] = (
                3 * gemm_flop * f / (st[1] * 1e-3) / 1e12)
            out[name]["output_pass_mfma_f16_tflops_executed"] = (
                2 * 3 * gemm_flop / (st[3] * 1e-3) / 1e12)
        else:
            out[name]["form"] = "v and x through HBM"
            out[name]["stage_ms"] = {"pack": st[0], "proj_in": st[1],
                                     ("scan" if name == "scan" else "spectrum+conv"): st[2],
                                     "proj_out": st[3]}
            out[name]["proj_in_mfma_f16_tflops_executed"] = 3 * gemm_flop / (st[1] * 1e-3) / 1e12
            out[name]["proj_out_mfma_f16_tflops_executed"] = 3 * gemm_flop / (st[3] * 1e-3) / 1e12
    return out


def time_s5_tv(steps):
    """Continuous-time S5 with irregular step sizes (uniform in [0.5, 1.5]) on
    the S5 workload shape: plain calls over rotated sets, wall clock."""
    import numpy as np
    import torch

    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config("s5_mimo")
    x = inputs.s5_tv_inputs(c["B"], c["H"], c["P"], c["L"], seed=c["seed"])
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us, ys = rotated(t["u"], 700 << 20)
    R = len(us)
    ws = torch.empty(bd.s5_tv_workspace_size(c["B"], c["H"], c["P"], c["L"]), dtype=torch.uint8,
                     device="cuda")

    def call(k):
        bd.s5_forward_tv(us[k % R], t["lam_c"], t["Bt"], t["C"], t["D"], t["delta"],
                         t["step"], y=ys[k % R], workspace=ws)

    ms = wall_ms(call, steps, 2, WARM_S)
    B, H, L = c["B"], c["H"], c["L"]
    return {"workload": "s5_mimo shape, continuous-time, steps ~ U(0.5, 1.5)",
            "ms_per_forward": ms, "elements_per_s": B * H * L / (ms * 1e-3), "rotated_sets": R}


def time_backward(dev, us, ys, bi, steps):
    """Gradient passes (dssm_backward) on the bench workload with a seeded
    output cotangent; wall clock between two synchronisations."""
    import torch

    from long_convolution_sequence_amd import binding as bd

    R = len(us)
    B, H, L = us[0].shape
    N = dev["log_re"].shape[-1]
    dy = torch.randn(B, H, L, generator=torch.Generator().manual_seed(7)).cuda()
    need = bd.workspace_size(bd.OP_BWD, B, H, N, L, bi)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")

    def call(k):
        bd.backward(us[k % R], dy, dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                    bidirectional=bi, du=ys[k % R], workspace=ws)

    ms = wall_ms(call, steps, 2, WARM_S)
    return {"ms_per_step": ms, "elements_per_s": B * H * L / (ms * 1e-3),
            "workspace_bytes": need,
            "note": "du and the four parameter gradients for f = sum(dy y); kernels: generator, "
                    "conjugate spectrum + convolution for du, batch-summed correlations of u and "
                    "dy (frequency domain), parameter reductions on float32 matrix cores"}


def time_copy(src, dst, reps, hip):
    """A plain device copy of `src` into `dst` (torch's copy kernel): the
    practically attainable HBM rate, and the calibration kernel of known size
    for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    dst.copy_(src)
    ev = hip.create(2)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    hip.record(ev[0], stream)
    for _ in range(reps):
        dst.copy_(src)
    hip.record(ev[1], stream)
    torch.cuda.synchronize()
    ms = hip.ms(ev[0], ev[1]) / reps
    hip.destroy(ev)
    nbytes = 2 * src.numel() * src.element_size()
    return {"bytes_per_copy": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # (steady state: 2000 warm-up steps are ~120 ms of the long-sequence step)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--side-steps", type=int, default=20,
                    help="plain calls per side measurement (other workloads and paths)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-side", action="store_true", help="headline only")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the layer's channels are independent, so a "
              "multi-GPU run is the same kernels on each GPU's share (no figure at several "
              "GPUs is produced here).", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    from long_convolution_sequence_amd import inputs

    cfg = inputs.config(WORKLOAD)
    B, H, N, L, bi = cfg["B"], cfg["H"], cfg["N"], cfg["L"], cfg["bidirectional"]
    x = inputs.inputs_for(cfg)
    cpu = ref = None
    if not a.no_cpu_baseline:  # before anything initialises the GPU
        cpu, ref = cpu_baseline(x, bi, direct_channels=H)

    import torch

    from long_convolution_sequence_amd import binding as bd

    torch.cuda.set_device(0)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us, ys = rotated(dev["u"])
    R = len(us)
    ws = torch.empty(bd.workspace_size(bd.OP_FFT, B, H, N, L, bi), dtype=torch.uint8,
                     device="cuda")
    hip = bd.HipEvents()

    def call(k):
        bd.forward_fft(us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                       bidirectional=bi, y=ys[k % R], workspace=ws)

    def call_timed(k, evs):
        bd.forward_timed("fft", us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                         evs, bidirectional=bi, y=ys[k % R], workspace=ws)

    # the timed region: K plain calls
    ms = wall_ms(call, a.steps, a.warmup)
    # after it: the per-step distribution, the convolution alone stamped over K
    # calls (its average launch duration), then every stage stamped
    dist = step_distribution(call, max(100, a.steps), hip)
    conv_ms = stage_times(call_timed, 2, a.steps, hip, only=1)[1]
    stages = stage_times(call_timed, 2, max(20, a.steps // 2), hip)
    call(0)
    torch.cuda.synchronize()
    y_fft = ys[0].cpu().numpy()

    elems = B * H * L
    alg_bytes = 8 * elems  # u read + y write, float32
    hbm_gbs = alg_bytes / (conv_ms * 1e-3) / 1e9
    alg_flop = conv_alg_flop(B, H, L)
    tflops = alg_flop / (conv_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC,
        "value": elems / (ms * 1e-3),
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "dtype_note": COMPUTE_NOTE,
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "H": H, "N": N, "L": L,
                   "bidirectional": bool(bi), "path": "fft", "parallelism": "none"},
        "step_ms_distribution": dist,
        # The metric's bound: HBM on the algorithmic 8 bytes per element.  The
        # convolution is in fact held by the vector ALU (non-packed FP32): its
        # VALU instructions alone take ~25 us of a launch, the bytes 8.4 us at
        # the HBM peak; that co-limit rides along (alu_*).
        "roofline": {
            "bound": "hbm",
            "kernel": "conv_kernel<14> (FFT convolution)",
            "achieved": hbm_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": hbm_gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_ms": conv_ms,
            "launches_timed": a.steps,
            "alu_achieved_tflops": tflops,
            "alu_alg_flop_per_launch": alg_flop,
            "alu_frac_nonpacked_fp32": tflops / ALU_PEAK_TFLOPS,
            "alu_frac_published_fp32": tflops / FP32_PUBLISHED_TFLOPS,
            # what actually holds it: vector-ALU issue at the clock the CUs
            # sustain under this load (below the 2.4 GHz peak)
            "valu_measured": measured_valu(),
        },
        "extra": {
            "stage_ms_breakdown": {"kernel_spectrum": stages[0], "conv": stages[1]},
            "layer_hbm_gbs": alg_bytes / (ms * 1e-3) / 1e9,
            "rotated_sets": R,
            "gpu_vs_oracle": errors_vs(y_fft, ref) if ref is not None else None,
        },
    }
    if not a.no_side:
        ex = line["extra"]
        ex["device_copy"] = time_copy(us[1 % R], ys[1 % R], 10, hip)
        ex["configs"] = {name: dlr_config(name, a.side_steps, hip)
                         for name in ("tiny", "image_length", "bidirectional", "long_sequence")}
        ex["configs"]["s5_mimo"] = s5_config(max(4, a.side_steps // 2), hip)
        ex["s5_tv_path"] = time_s5_tv(max(4, a.side_steps // 2))
        ex["scan_sequence_split"] = scan_split(hip)
        ex["streaming_prefill"] = stream_prefill(a.side_steps, hip)
        ex["backward"] = time_backward(dev, us, ys, bi, max(4, a.side_steps // 2))
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
