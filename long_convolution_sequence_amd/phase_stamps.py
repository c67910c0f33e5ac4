"""Per-phase cycle counts of the kernel generator, the FFT convolution and the
chunked recurrence on the long-sequence workload (B=4 H=128 N=64 L=16384),
and of the S5 scan method's output projection and the fused S5 form's output
pass on the S5 workload (B=4 H=256 P=128 L=16384), from the instrumented
library libdssm_stamps.so:

    python -m long_convolution_sequence_amd.build --phase-stamps
    python -m long_convolution_sequence_amd.phase_stamps [--reps 5]

The instrumented kernels read the shader-clock counter at their phase
boundaries and add each phase's cycles to a register slot, written once at
the end of the kernel (so the stamps add no memory waits to the phases they
time).  Printed per kernel: the mean over workgroups and waves of each
phase's cycles, their sum, and for the convolution and the recurrence the
launch time (GPU-stamped events around the kernel) and the clock the two
imply (every wave of these launches is resident from the start of the launch
to its end; the generator shares its stamped stage with the spectrum).  The
same input set is used on every call, so it is partly served from the
caches: phases that wait on memory read shorter here than in bench.py, which
rotates input sets larger than the caches.
"""
import argparse
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_STAMPS = os.path.join(HERE, "libdssm_stamps.so")

SLOTS = 16
MAX_WAVES = 4096 * 16  # buffer rows: up to 4096 workgroups of up to 16 waves

CONV_PHASES = ["entry: twiddle table, input requested", "even half forward",
               "even half: spectrum read, product", "even half inverse", "odd half forward",
               "odd half: spectrum read, product", "odd half inverse",
               "combination, stores issued"]
GEN_PHASES = ["lambda and W (wave 0, float64), barrier", "tables (float64 chains), split",
              "largest anchor entry, barrier", "contraction (matrix cores)", "stores issued"]
CHUNK_PHASES = ["prologue: fragments, barrier", "block: barrier", "input staged, next requested",
                "barrier", "chunk states (matrix cores)", "barrier", "recurrence, first part",
                "barrier", "recurrence, second part", "barrier", "outputs (matrix cores)",
                "prologue: entry, loads issued", "prologue: lambda (float64), barrier",
                "prologue: powers, Q and KR tables, barrier", "prologue: taps, barrier",
                "prologue: power planes, barrier"]
S5_PIPE_PHASES = ["prologue: fragments, first tile loaded and staged", "next tile requested",
                  "product (matrix cores)", "outputs scaled (+ D u), stores issued",
                  "next tile received, split, staged (2 barriers)"]
S5_PHASES = ["prologue: parameters, entering state, first u tile requested",
             "u tile in LDS (first tile), barrier", "u scaled, split, staged; D u (2 barriers)",
             "input projection (matrix cores)", "recurrence on the tile",
             "x maximum (barrier), scaled, split, staged", "next u tile in LDS, barrier",
             "output projection (matrix cores), stores issued"]


def _phases(buf, nwg, waves, names):
    d = buf.cpu().numpy().reshape(-1, SLOTS)[: nwg * waves].astype(np.float64)
    tot = d[:, : len(names)].sum(axis=1)
    rows = [(nm, d[:, k].mean()) for k, nm in enumerate(names)]
    return rows, tot.mean()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=5)
    a = ap.parse_args()
    if not os.path.exists(LIB_STAMPS):
        raise SystemExit("%s is missing: python -m long_convolution_sequence_amd.build "
                         "--phase-stamps" % LIB_STAMPS)
    import torch

    from long_convolution_sequence_amd import binding as bd
    from long_convolution_sequence_amd import inputs

    bd.LIB_PATH = LIB_STAMPS
    lib = bd.lib()
    for fn in ("dssm_phase_stamps_fft", "dssm_phase_stamps_chunk", "dssm_phase_stamps_gen",
               "dssm_phase_stamps_s5"):
        getattr(lib, fn).argtypes = [ctypes.c_void_p]
        getattr(lib, fn).restype = ctypes.c_int

    c = inputs.config("long_sequence")
    B, H = c["B"], c["H"]
    x = inputs.inputs_for(c)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x.items()}
    args = (t["u"], t["log_re"], t["log_im"], t["W"], t["D"])
    hip = bd.HipEvents()
    # (grid of the kernel on this workload, waves per workgroup)
    L = c["L"]
    kinds = [(None, "dssm_phase_stamps_gen", "gen_kernel", (H * ((L + 4095) // 4096), 4),
              GEN_PHASES, bd.forward_fft),
             ("fft", "dssm_phase_stamps_fft", "conv_kernel<14>", (H * ((B + 1) // 2), 16),
              CONV_PHASES, bd.forward_fft),
             ("scan", "dssm_phase_stamps_chunk", "chunk_kernel", (H * B, 4), CHUNK_PHASES,
              bd.forward_scan)]
    # the streaming call (state in, end state out) from a random state
    x0 = torch.from_numpy(inputs.dlr_state(B, H, c["N"], seed=3)).cuda()
    kinds.append((None, "dssm_phase_stamps_chunk", "chunk_kernel, streaming", (H * B, 4),
                  CHUNK_PHASES, lambda *a_: bd.forward_scan_state(*a_, x0.clone())))
    for path, setter, kname, (nwg, waves), names, fn in kinds:
        assert nwg * waves <= MAX_WAVES
        buf = torch.zeros(MAX_WAVES * SLOTS, dtype=torch.int64, device="cuda")
        if getattr(lib, setter)(buf.data_ptr()) != 0:
            raise SystemExit("%s failed" % setter)
        for _ in range(a.reps):
            fn(*args)
        torch.cuda.synchronize()
        rows, total = _phases(buf, nwg, waves, names)
        if getattr(lib, setter)(None) != 0:
            raise SystemExit("%s failed" % setter)
        if path is None:
            print("%s (%d workgroups x %d waves): %.0f cycles per wave" % (kname, nwg, waves, total))
            for nm, v in rows:
                print("  %-42s %8.0f  %5.1f%%" % (nm, v, 100.0 * v / total))
            continue
        evs = [hip.create(4) for _ in range(a.reps + 5)]
        for e in evs:
            bd.forward_timed(path, *args, e)
        torch.cuda.synchronize()
        ms = sorted(hip.ms(e[2], e[3]) for e in evs[3:])
        launch_us = 1e3 * ms[len(ms) // 2]
        for e in evs:
            hip.destroy(e)
        print("%s (%d workgroups x %d waves): %.0f cycles per wave, launch %.1f us, "
              "%.2f GHz" % (kname, nwg, waves, total, launch_us, total / launch_us / 1e3))
        for nm, v in rows:
            print("  %-42s %8.0f  %5.1f%%" % (nm, v, 100.0 * v / total))

    # the S5 scan method: its output projection is the last launch to write the stamps
    c5 = inputs.config("s5_mimo")
    x5 = inputs.inputs_for(c5)
    t5 = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x5.items()}
    ws5 = torch.empty(bd.s5_workspace_size(c5["B"], c5["H"], c5["P"], c5["L"], bd.S5_SCAN),
                      dtype=torch.uint8, device="cuda")
    buf = torch.zeros(MAX_WAVES * SLOTS, dtype=torch.int64, device="cuda")
    if lib.dssm_phase_stamps_s5(buf.data_ptr()) != 0:
        raise SystemExit("dssm_phase_stamps_s5 failed")
    for _ in range(a.reps):
        bd.s5_forward(t5["u"], t5["lam"], t5["Bbar"], t5["C"], t5["D"], workspace=ws5,
                      method=bd.S5_SCAN)
    torch.cuda.synchronize()
    rows, total = _phases(buf, 256, 8, S5_PIPE_PHASES)
    dp = buf.cpu().numpy().reshape(-1, SLOTS)[8192: 8192 + 256 * 8].astype(np.float64)
    in_rows = [(nm, dp[:, k].mean()) for k, nm in enumerate(S5_PIPE_PHASES)]
    in_total = dp[:, : len(S5_PIPE_PHASES)].sum(axis=1).mean()
    if lib.dssm_phase_stamps_s5(None) != 0:
        raise SystemExit("dssm_phase_stamps_s5 failed")
    for kname, tot, rws in (("s5_gemm_pipe_kernel<false>, input projection", in_total, in_rows),
                            ("s5_gemm_pipe_kernel<true>, output projection", total, rows)):
        print("%s (256 workgroups x 8 waves): %.0f cycles per wave" % (kname, tot))
        for nm, v in rws:
            print("  %-42s %8.0f  %5.1f%%" % (nm, v, 100.0 * v / tot))

    # the fused S5 form: its output pass is the last launch to write the stamps
    c5 = inputs.config("s5_mimo")
    x5 = inputs.inputs_for(c5)
    t5 = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in x5.items()}
    ws = torch.empty(bd.s5_workspace_size(c5["B"], c5["H"], c5["P"], c5["L"], bd.S5_FUSED),
                     dtype=torch.uint8, device="cuda")

    def s5(evs=None):
        bd.s5_forward(t5["u"], t5["lam"], t5["Bbar"], t5["C"], t5["D"], workspace=ws,
                      method=bd.S5_FUSED, events=evs)

    buf = torch.zeros(MAX_WAVES * SLOTS, dtype=torch.int64, device="cuda")
    if lib.dssm_phase_stamps_s5(buf.data_ptr()) != 0:
        raise SystemExit("dssm_phase_stamps_s5 failed")
    for _ in range(a.reps):
        s5()
    torch.cuda.synchronize()
    nwg, waves = 256, 8  # the output pass's grid on this workload
    rows, total = _phases(buf, nwg, waves, S5_PHASES)
    # the state-only pass: its stamps from row 4096 on (its last segments'
    # workgroups return at once and leave none)
    d = buf.cpu().numpy().reshape(-1, SLOTS)[4096: 4096 + nwg * waves].astype(np.float64)
    d = d[d[:, : len(S5_PHASES)].sum(axis=1) > 0]
    st_rows = [(nm, d[:, k].mean()) for k, nm in enumerate(S5_PHASES)]
    st_total = d[:, : len(S5_PHASES)].sum(axis=1).mean()
    if lib.dssm_phase_stamps_s5(None) != 0:
        raise SystemExit("dssm_phase_stamps_s5 failed")
    evs = [hip.create(8) for _ in range(a.reps + 5)]
    for e in evs:
        s5(e)
    torch.cuda.synchronize()
    ms = sorted(hip.ms(e[6], e[7]) for e in evs[3:])  # stage 3: the output pass
    launch_us = 1e3 * ms[len(ms) // 2]
    for e in evs:
        hip.destroy(e)
    print("s5_fused_kernel, output pass (%d workgroups x %d waves): %.0f cycles per wave, "
          "launch %.1f us, %.2f GHz" % (nwg, waves, total, launch_us, total / launch_us / 1e3))
    for nm, v in rows:
        print("  %-42s %8.0f  %5.1f%%" % (nm, v, 100.0 * v / total))
    print("s5_fused_kernel, state-only pass (%d waves with stamps): %.0f cycles per wave"
          % (len(d), st_total))
    for nm, v in st_rows:
        print("  %-42s %8.0f  %5.1f%%" % (nm, v, 100.0 * v / st_total))


if __name__ == "__main__":
    main()
