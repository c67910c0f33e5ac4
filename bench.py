"""Benchmark of the diagonal-SSM layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one full forward of the layer by the convolution view (kernel
generation, kernel spectrum, FFT convolution with the D skip)
on the long-sequence workload B=4, H=128, N=64, L=16384 (log_re scaled by
0.1), seeded synthetic inputs already resident in device memory.  Several
input/output sets (576 MiB in all) are rotated so that the 256 MB Infinity Cache
does not hold the step's inputs from an earlier step.

Prints ONE JSON line: value = elements (B*H*L) per second over the timed
steps (wall clock between two device synchronisations), the per-kernel
durations from the start/stop HIP events the GPU stamps around each kernel, the
roofline of the dominant kernel (the convolution: bound by the vector ALU,
on its algorithmic flops, with its HBM rate on algorithmic bytes, u read + y
write = 8 bytes per element, beside it), and the float64 oracle timed on the
host as the CPU baseline.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# FP32 vector peak without packed FP32 (the library is compiled without it): 256 CUs x 4
# SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz.  The published 157.3 TFLOP/s
# counts packed FMAs (two per lane per clock).
ALU_PEAK_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
METRIC = "SSM layer fwd elements/s (B·H·L) and achieved HBM GB/s vs peak, L=16384"
WORKLOAD = "long_sequence"


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


def measured_traffic():
    """HBM bytes per launch of the convolution from the committed counter
    record, or None when there is none or the kernel sources changed since."""
    try:
        with open(TRAFFIC_RECORD) as f:
            for ln in f:
                if ln.startswith("traffic-record: "):
                    rec = json.loads(ln[len("traffic-record: "):])
                    if rec.get("sources_sha256") == kernel_sources_digest():
                        return rec["fetch_bytes"] + rec["write_bytes"]
    except (OSError, ValueError, KeyError):
        pass
    return None


def time_path(path, dev, us, ys, ws, steps, warmup, bi, hip, breakdown_steps=20):
    """Run `warmup` untimed steps, then `steps` timed steps in which only the
    dominant kernel (the convolution, or the scan) is bracketed by the
    start/stop events the GPU stamps around it -- an event-stamped launch costs
    the host tens of microseconds, so stamping every kernel would starve the
    GPU -- then `breakdown_steps` more with every kernel stamped.

    Returns wall ms/step of the timed steps, the dominant kernel's mean ms in
    them, and the mean per-kernel ms of the breakdown steps."""
    import torch
    from long_convolution_sequence_amd import binding as bd

    nk = 2
    R = len(us)
    f = bd.forward_fft if path == "fft" else bd.forward_scan

    def call(k, evs=None):
        if evs is None:
            f(us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"], bidirectional=bi,
              y=ys[k % R], workspace=ws)
        else:
            bd.forward_timed(path, us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                             evs, bidirectional=bi, y=ys[k % R], workspace=ws)

    for k in range(warmup):
        call(k)
    main = [hip.create(2) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        call(k, [None] * (2 * nk - 2) + main[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom = sum(hip.ms(e[0], e[1]) for e in main) / steps
    for e in main:
        hip.destroy(e)
    full = [hip.create(2 * nk) for _ in range(breakdown_steps)]
    for k in range(breakdown_steps):
        call(k, full[k])
    torch.cuda.synchronize()
    stages = [sum(hip.ms(e[2 * i], e[2 * i + 1]) for e in full) / breakdown_steps
              for i in range(nk)]
    for e in full:
        hip.destroy(e)
    return (t1 - t0) * 1e3 / steps, dom, stages


def time_plain(dev, us, ys, ws, steps, bi):
    """Wall ms per layer forward (FFT view) by plain calls with no event stamps,
    for comparison with the timed region, whose convolution launch carries a
    GPU event pair on every step."""
    import torch
    from long_convolution_sequence_amd import binding as bd

    R = len(us)

    def call(k):
        bd.forward_fft(us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                       bidirectional=bi, y=ys[k % R], workspace=ws)

    for k in range(3):
        call(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        call(k)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def time_s5(steps, warmup, hip, rotate=5, breakdown_steps=10):
    """Timed S5 layer forwards on the S5 workload (B=4, H=256, P=128, L=16384):
    plain calls over `rotate` input/output sets (5 x 2 x 67 MB, beyond the
    256 MB MALL) for the wall clock, then `breakdown_steps` more with each of
    the four kernels stamped by GPU events for the per-kernel times."""
    import numpy as np
    import torch
    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config("s5_mimo")
    x = inputs.inputs_for(c)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us = [t["u"]] + [t["u"].clone() for _ in range(rotate - 1)]
    ys = [torch.empty_like(t["u"]) for _ in range(rotate)]
    ws = torch.empty(bd.s5_workspace_size(c["B"], c["H"], c["P"], c["L"]), dtype=torch.uint8,
                     device="cuda")

    def call(k, evs=None):
        bd.s5_forward(us[k % rotate], t["lam"], t["Bbar"], t["C"], t["D"], y=ys[k % rotate],
                      workspace=ws, events=evs)

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        call(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    evs = [hip.create(8) for _ in range(breakdown_steps)]
    for k in range(breakdown_steps):
        call(k, evs[k])
    torch.cuda.synchronize()
    st = [sum(hip.ms(e[2 * i], e[2 * i + 1]) for e in evs) / breakdown_steps for i in range(4)]
    for e in evs:
        hip.destroy(e)
    ms = (t1 - t0) * 1e3 / steps
    B, H, P, L = c["B"], c["H"], c["P"], c["L"]
    gemm_flop = 2.0 * (2 * P) * H * L * B  # one projection
    return {
        "workload": "s5_mimo", "B": B, "H": H, "P": P, "L": L,
        "ms_per_step": ms, "elements_per_s": B * H * L / (ms * 1e-3), "rotated_sets": rotate,
        "stage_ms": {"pack": st[0], "proj_in": st[1], "scan": st[2], "proj_out": st[3]},
        "proj_in_fp32_tflops": gemm_flop / (st[1] * 1e-3) / 1e12,
        "proj_out_fp32_tflops": gemm_flop / (st[3] * 1e-3) / 1e12,
        "mfma_fp32_peak_tflops": 157.3,
    }


def time_s5_tv(steps, warmup, rotate=5):
    """Timed forwards of the continuous-time S5 layer with irregular per-step
    step sizes (uniform in [0.5, 1.5]) on the S5 workload shape: plain calls
    over `rotate` input/output sets, wall clock."""
    import numpy as np
    import torch
    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config("s5_mimo")
    x = inputs.s5_tv_inputs(c["B"], c["H"], c["P"], c["L"], seed=c["seed"])
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us = [t["u"]] + [t["u"].clone() for _ in range(rotate - 1)]
    ys = [torch.empty_like(t["u"]) for _ in range(rotate)]
    ws = torch.empty(bd.s5_workspace_size(c["B"], c["H"], c["P"], c["L"]), dtype=torch.uint8,
                     device="cuda")

    def call(k):
        bd.s5_forward_tv(us[k % rotate], t["lam_c"], t["Bt"], t["C"], t["D"], t["delta"],
                         t["step"], y=ys[k % rotate], workspace=ws)

    for k in range(warmup):
        call(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        call(k)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    B, H, L = c["B"], c["H"], c["L"]
    return {"workload": "s5_mimo shape, continuous-time, steps ~ U(0.5, 1.5)",
            "ms_per_step": ms, "elements_per_s": B * H * L / (ms * 1e-3), "rotated_sets": rotate}


def time_backward(dev, us, ys, bi, steps, warmup):
    """Timed gradient passes (dssm_backward) of the layer on the bench workload,
    with a seeded output cotangent; wall clock between two synchronisations."""
    import torch
    from long_convolution_sequence_amd import binding as bd

    R = len(us)
    B, H, L = us[0].shape
    N = dev["log_re"].shape[-1]
    dy = torch.randn(B, H, L, generator=torch.Generator().manual_seed(7)).cuda()
    shape = bd.Shape(B, H, N, L, int(bool(bi)))
    need = ctypes_size(bd, bd.OP_BWD, shape)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for k in range(warmup):
        bd.backward(us[k % R], dy, dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                    bidirectional=bi, du=ys[k % R], workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        bd.backward(us[k % R], dy, dev["log_re"], dev["log_im"], dev["W"], dev["D"],
                    bidirectional=bi, du=ys[k % R], workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    elems = B * H * L
    return {"ms_per_step": ms, "elements_per_s": elems / (ms * 1e-3), "workspace_bytes": need,
            "note": "du and the four parameter gradients for f = sum(dy y); kernels: generator, "
                    "conjugate spectrum + convolution for du, batch-summed correlations of u and "
                    "dy (frequency domain), parameter reductions on float32 matrix cores"}


def ctypes_size(bd, op, shape):
    import ctypes
    out = ctypes.c_size_t(0)
    bd.check(bd.lib().dssm_workspace_size(op, ctypes.byref(shape), ctypes.byref(out)))
    return max(out.value, 256)


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


def cpu_baseline(x, bi, y_gpu):
    """The float64 oracle as it stands, single process, on the host: the
    sequential recurrence over the whole workload, plus the direct O(L^2) sum
    on a sample of rows.  Also reports each GPU path's error against it
    (y_gpu: path name -> output)."""
    import numpy as np

    import oracle

    B, H, L = x["u"].shape
    t = time.perf_counter()
    ref = oracle.dlr_recurrence(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], bi)
    t_rec = time.perf_counter() - t
    hs = min(H, 48)  # direct-sum sample: ~8 s of host work on the long-sequence workload
    t = time.perf_counter()
    refd = oracle.dlr_direct(x["u"][:, :hs], x["log_re"][:, :hs], x["log_im"][:, :hs],
                             x["W"][:, :hs], x["D"][:, :hs], bi)
    t_dir = time.perf_counter() - t
    rms = np.sqrt(np.mean(ref ** 2))
    errs = {}
    for name, y in y_gpu.items():
        d = y.astype(np.float64) - ref
        dd = y[:, :hs].astype(np.float64) - refd
        errs[name] = {"rel_l2": float(np.linalg.norm(d) / np.linalg.norm(ref)),
                      "max_over_rms": float(np.max(np.abs(d)) / rms),
                      "direct_sample_rel_l2": float(np.linalg.norm(dd) / np.linalg.norm(refd))}
    return {
        "value": B * H * L / t_rec,
        "unit": "elements/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "oracle.dlr_recurrence (float64 sequential recurrence) over the whole "
                  "workload (%d elements, %.1f s); oracle.dlr_direct (O(L^2) sum) on %d of %d "
                  "channels: %.3g elements/s" % (B * H * L, t_rec, hs, H, B * hs * L / t_dir),
        "gpu_vs_oracle": errs,
    }


def scan_path_summary(B, H, N, L, bi, ms, kernel_ms, stages):
    """The recurrence view's layer forward.  With N <= 64 modes it is one
    kernel, the chunked matrix-core form (chunks of T = 64 steps, blocks of 64
    chunks): per (direction, channel, batch row) and block, 4 waves x (48 + 72)
    v_mfma_f32_16x16x32_f16 of 16384 flops each (the split operands triple the
    contraction).  Otherwise the segmented scan (constants kernel + scan)."""
    elems = B * H * L
    ndir = 2 if bi else 1
    out = {"ms_per_step": ms, "elements_per_s": elems / (ms * 1e-3), "kernel_ms": kernel_ms}
    alg_bytes = 8 * elems
    out["hbm_gbs"] = alg_bytes / (kernel_ms * 1e-3) / 1e9
    out["hbm_frac"] = out["hbm_gbs"] / HBM_PEAK_GBS
    if N <= 64:
        nblk = -(-(-(-L // 64)) // 64)
        mfma_flop = ndir * H * B * nblk * 4 * (48 + 72) * 16384
        out["kernel"] = "chunk_kernel (chunked matrix-core form)"
        out["mfma_f16_tflops_executed"] = mfma_flop / (kernel_ms * 1e-3) / 1e12
        out["mfma_f16_frac"] = out["mfma_f16_tflops_executed"] / 2500.0
        out["alg_fp32_tflops"] = 12 * N * ndir * elems / (kernel_ms * 1e-3) / 1e12
    else:
        out["kernel"] = "scan_kernel (segmented scan)"
        out["stage_ms_breakdown"] = {"consts": stages[0], "scan": stages[1]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=9,
                    help="input/output sets rotated per step (9 x 64 MiB > the 256 MB MALL x 2)")
    ap.add_argument("--scan-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the layer's channels are independent, so a "
              "multi-GPU run is the same kernels on each GPU's share (no figure at several "
              "GPUs is produced here).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    cfg = inputs.config(WORKLOAD)
    B, H, N, L, bi = cfg["B"], cfg["H"], cfg["N"], cfg["L"], cfg["bidirectional"]
    x = inputs.inputs_for(cfg)
    torch.cuda.set_device(0)
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    us = [dev["u"]] + [dev["u"].clone() for _ in range(a.rotate - 1)]
    ys = [torch.empty_like(dev["u"]) for _ in range(a.rotate)]
    ws_fft = torch.empty(bd.workspace_size(bd.OP_FFT, B, H, N, L, bi), dtype=torch.uint8,
                         device="cuda")
    ws_scan = torch.empty(bd.workspace_size(bd.OP_SCAN, B, H, N, L, bi), dtype=torch.uint8,
                          device="cuda")
    hip = bd.HipEvents()

    copy = time_copy(us[1], ys[1], 10, hip)
    ms, conv_ms, stages = time_path("fft", dev, us, ys, ws_fft, a.steps, a.warmup, bi, hip)
    y_fft = ys[(a.steps - 1) % a.rotate].cpu().numpy()
    ms_scan, scan_ms, stages_scan = time_path("scan", dev, us, ys, ws_scan, a.scan_steps,
                                              min(a.warmup, 2), bi, hip, a.scan_steps)
    y_scan = ys[(a.scan_steps - 1) % a.rotate].cpu().numpy()

    elems = B * H * L
    alg_bytes = 8 * elems  # u read + y write, float32
    hbm_gbs = alg_bytes / (conv_ms * 1e-3) / 1e9
    # algorithmic flops of the convolution per (b, h) row: two real FFTs of
    # n = 2L points (2 n log2 n - 4 n each), the spectrum product on L + 1
    # bins (6 each) and the D skip (2 per element)
    n = 2 * L
    alg_flop = B * H * (2 * (2 * n * np.log2(n) - 4 * n) + 6 * (L + 1) + 2 * L)
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
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": B, "H": H, "N": N, "L": L,
                   "bidirectional": bool(bi), "path": "fft", "parallelism": "none"},
        # The convolution is bound by the vector ALU (non-packed FP32): its
        # VALU instructions alone take ~25 of its ~42 us, its algorithmic
        # bytes 8.4 us at the HBM peak.  The HBM figures of the metric ride
        # along (hbm_*).
        "roofline": {
            "bound": "alu",
            "kernel": "conv_kernel<14> (FFT convolution)",
            "achieved": tflops,
            "peak": ALU_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / ALU_PEAK_TFLOPS,
            "traffic": measured_traffic(),
            "alg_flop_per_launch": alg_flop,
            "frac_of_published_packed_fp32": tflops / 157.3,
            "hbm_achieved_gbs": hbm_gbs,
            "hbm_peak_gbs": HBM_PEAK_GBS,
            "hbm_frac": hbm_gbs / HBM_PEAK_GBS,
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_ms": conv_ms,
        },
        "extra": {
            "stage_ms_breakdown": {"kernel_spectrum": stages[0], "conv": stages[1]},
            "fft_plain_calls_ms_per_step": time_plain(dev, us, ys, ws_fft, a.steps, bi),
            "full_call_hbm_gbs": alg_bytes / (ms * 1e-3) / 1e9,
            "scan_path": scan_path_summary(B, H, N, L, bi, ms_scan, scan_ms, stages_scan),
            "rotated_sets": a.rotate,
            "device_copy": copy,
            "s5_path": time_s5(max(2, a.scan_steps), 2, hip),
            "s5_tv_path": time_s5_tv(max(2, a.scan_steps), 2),
            "backward": time_backward(dev, us, ys, bi, max(2, a.scan_steps), 2),
        },
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, bi, {"fft": y_fft, "scan": y_scan})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
