"""Benchmark of the diagonal-SSM layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one full forward of the layer by the convolution view (kernel
generation, kernel spectrum, FFT convolution with the D skip)
on the long-sequence workload B=4, H=128, N=64, L=16384 (log_re scaled by
0.1), seeded synthetic inputs already resident in device memory.  Several
input/output sets are rotated so that the 256 MB Infinity Cache does not hold
the step's inputs from the previous step.

Prints ONE JSON line: value = elements (B*H*L) per second over the timed
steps (wall clock between two device synchronisations), the per-kernel
durations from HIP events recorded by the library on the launch stream, the
roofline of the dominant kernel (the convolution) on algorithmic bytes
(u read + y write = 8 bytes per element), and the float64 oracle timed on
the host as the CPU baseline.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "SSM layer fwd elements/s (B·H·L) and achieved HBM GB/s vs peak, L=16384"
WORKLOAD = "long_sequence"


class HipEvents:
    """Raw hipEvent_t handles through libamdhip64 (timing plumbing only)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.h.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError("hipEventCreate failed: %d" % rc)
            out.append(e.value)
        return out

    def ms(self, a, b):
        t = ctypes.c_float()
        rc = self.h.hipEventElapsedTime(ctypes.byref(t), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed: %d" % rc)
        return t.value

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(ctypes.c_void_p(e))


def time_path(path, dev, us, ys, ws, steps, warmup, bi, hip):
    """Run `warmup` untimed and `steps` timed steps; return wall ms/step and
    mean per-stage ms from the library's events."""
    import torch
    from long_convolution_sequence_amd import binding as bd

    nev = 4 if path == "fft" else 3
    R = len(us)
    f = bd.forward_fft if path == "fft" else bd.forward_scan
    for k in range(warmup):
        f(us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"], bidirectional=bi,
          y=ys[k % R], workspace=ws)
    evs = [hip.create(nev) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        bd.forward_timed(path, us[k % R], dev["log_re"], dev["log_im"], dev["W"], dev["D"], evs[k],
                         bidirectional=bi, y=ys[k % R], workspace=ws)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = [sum(hip.ms(e[i], e[i + 1]) for e in evs) / steps for i in range(nev - 1)]
    gpu = sum(hip.ms(e[0], e[-1]) for e in evs) / steps
    for e in evs:
        hip.destroy(e)
    return (t1 - t0) * 1e3 / steps, stages, gpu


def time_s5(steps, warmup, hip):
    """Timed S5 layer forwards on the S5 workload (B=4, H=256, P=128, L=16384)."""
    import numpy as np
    import torch
    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    c = inputs.config("s5_mimo")
    x = inputs.inputs_for(c)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    y = torch.empty_like(t["u"])
    ws = torch.empty(bd.s5_workspace_size(c["B"], c["H"], c["P"], c["L"]), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        bd.s5_forward(t["u"], t["lam"], t["Bbar"], t["C"], t["D"], y=y, workspace=ws)
    evs = [hip.create(5) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        bd.s5_forward(t["u"], t["lam"], t["Bbar"], t["C"], t["D"], y=y, workspace=ws, events=evs[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    st = [sum(hip.ms(e[i], e[i + 1]) for e in evs) / steps for i in range(4)]
    for e in evs:
        hip.destroy(e)
    ms = (t1 - t0) * 1e3 / steps
    B, H, P, L = c["B"], c["H"], c["P"], c["L"]
    gemm_flop = 2.0 * (2 * P) * H * L * B  # one projection
    return {
        "workload": "s5_mimo", "B": B, "H": H, "P": P, "L": L,
        "ms_per_step": ms, "elements_per_s": B * H * L / (ms * 1e-3),
        "stage_ms": {"pack": st[0], "proj_in": st[1], "scan": st[2], "proj_out": st[3]},
        "proj_in_fp32_tflops": gemm_flop / (st[1] * 1e-3) / 1e12,
        "proj_out_fp32_tflops": gemm_flop / (st[3] * 1e-3) / 1e12,
        "mfma_fp32_peak_tflops": 157.3,
    }


def time_copy(src, dst, reps, hip):
    """A plain device copy of `src` into `dst` (torch's copy kernel): the
    practically attainable HBM rate, and the calibration kernel of known size
    for the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    dst.copy_(src)
    ev = hip.create(2)
    torch.cuda.synchronize()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hip.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.h.hipEventRecord(ctypes.c_void_p(ev[0]), stream)
    for _ in range(reps):
        dst.copy_(src)
    hip.h.hipEventRecord(ctypes.c_void_p(ev[1]), stream)
    torch.cuda.synchronize()
    ms = hip.ms(ev[0], ev[1]) / reps
    hip.destroy(ev)
    nbytes = 2 * src.numel() * src.element_size()
    return {"bytes_per_copy": nbytes, "ms": ms, "gbs": nbytes / (ms * 1e-3) / 1e9}


def cpu_baseline(x, bi, y_gpu):
    """The float64 oracle as it stands, single process, on the host: the
    sequential recurrence over the whole workload, plus the direct O(L^2) sum
    on a sample of rows.  Also reports the GPU output's error against it."""
    import numpy as np

    import oracle

    B, H, L = x["u"].shape
    t = time.perf_counter()
    ref = oracle.dlr_recurrence(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], bi)
    t_rec = time.perf_counter() - t
    hs = 4
    t = time.perf_counter()
    refd = oracle.dlr_direct(x["u"][:, :hs], x["log_re"][:, :hs], x["log_im"][:, :hs],
                             x["W"][:, :hs], x["D"][:, :hs], bi)
    t_dir = time.perf_counter() - t
    d = y_gpu.astype(np.float64) - ref
    rel = float(np.linalg.norm(d) / np.linalg.norm(ref))
    mx = float(np.max(np.abs(d)) / np.sqrt(np.mean(ref ** 2)))
    dd = y_gpu[:, :hs].astype(np.float64) - refd
    rel_d = float(np.linalg.norm(dd) / np.linalg.norm(refd))
    return {
        "value": B * H * L / t_rec,
        "unit": "elements/s",
        "cores": 1,
        "kind": "oracle",
        "sample": "oracle.dlr_recurrence (float64 sequential recurrence) over the whole "
                  "workload (%d elements, %.1f s); oracle.dlr_direct (O(L^2) sum) on %d of %d "
                  "channels: %.3g elements/s" % (B * H * L, t_rec, hs, H, B * hs * L / t_dir),
        "gpu_vs_oracle": {"rel_l2": rel, "max_over_rms": mx, "direct_sample_rel_l2": rel_d},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--rotate", type=int, default=6, help="input/output sets rotated per step")
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
    hip = HipEvents()

    copy = time_copy(us[1], ys[1], 10, hip)
    ms, stages, gpu_ms = time_path("fft", dev, us, ys, ws_fft, a.steps, a.warmup, bi, hip)
    y_fft = ys[(a.steps - 1) % a.rotate].cpu().numpy()
    ms_scan, stages_scan, gpu_scan = time_path("scan", dev, us, ys, ws_scan, a.scan_steps,
                                               min(a.warmup, 2), bi, hip)

    elems = B * H * L
    alg_bytes = 8 * elems  # u read + y write, float32
    conv_ms = stages[2]
    achieved = alg_bytes / (conv_ms * 1e-3) / 1e9
    # convolution flops on the 2M = 32768 circle: 4 complex transforms of
    # M = 16384 points per pair of rows, counted as 5 M log2 M each, plus the
    # spectrum product (6 flops per bin) and the odd-bin twiddles
    M = 1 << max(4, (L - 1).bit_length())
    pairs = H * ((B + 1) // 2)
    conv_flop = pairs * (4 * 5 * M * np.log2(M) + 2 * 6 * M + 4 * 6 * M)
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
        "roofline": {
            "bound": "hbm",
            "kernel": "conv_kernel<14> (FFT convolution)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": None,
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_ms": conv_ms,
        },
        "extra": {
            "gpu_ms_per_step_events": gpu_ms,
            "stage_ms": {"kernel_gen": stages[0], "spectrum": stages[1], "conv": stages[2]},
            "full_call_hbm_gbs": alg_bytes / (ms * 1e-3) / 1e9,
            "conv_fp32_tflops_est": conv_flop / (conv_ms * 1e-3) / 1e12,
            "scan_path": {"ms_per_step": ms_scan, "elements_per_s": elems / (ms_scan * 1e-3),
                          "stage_ms": {"consts": stages_scan[0], "scan": stages_scan[1]},
                          "gpu_ms_events": gpu_scan},
            "rotated_sets": a.rotate,
            "device_copy": copy,
            "s5_path": time_s5(max(2, a.scan_steps), 2, hip),
        },
    }
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, bi, y_fft)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
