"""Build libdssm.so in-tree for gfx950 with hipcc (no torch involved).

    python -m long_convolution_sequence_amd.build [--verbose] [--phase-stamps]

Steps: generate the twiddle table include, compile every csrc/*.hip to an
object (in parallel), link the shared library next to this file.  With
--phase-stamps the sources are compiled with DSSM_PHASE_STAMPS into a
separate libdssm_stamps.so (kernels that keep per-phase cycle counts; see
phase_stamps.py); libdssm.so is not touched.
"""
import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libdssm.so")
BUILD_STAMPS = os.path.join(HERE, "_build_stamps")
LIB_STAMPS = os.path.join(HERE, "libdssm_stamps.so")
SOURCES = ["api.hip", "chunk.hip", "eig_gen.hip", "fft.hip", "grad.hip", "scan.hip", "s5.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 instructions are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout or "") + (r.stderr or "")
    # the host pass does not know the device-only target feature: harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), "\n".join(lines)))
    return "\n".join(lines)


def build(verbose=False, resource_usage=False, phase_stamps=False):
    bdir, lib = (BUILD_STAMPS, LIB_STAMPS) if phase_stamps else (BUILD, LIB)
    os.makedirs(bdir, exist_ok=True)
    inc = os.path.join(CSRC, "twiddle_table.inc")
    subprocess.run([sys.executable, os.path.join(CSRC, "gen_twiddles.py"), inc], check=True)
    extra = ["-Rpass-analysis=kernel-resource-usage"] if resource_usage else []
    if phase_stamps:
        extra.append("-DDSSM_PHASE_STAMPS")

    def compile_one(src):
        obj = os.path.join(bdir, src.replace(".hip", ".o"))
        cmd = [HIPCC] + FLAGS + extra + ["-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        return obj, _run(cmd, verbose)

    with cf.ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    logs = [log for _, log in results if log.strip()]
    if logs and (verbose or resource_usage):
        print("\n".join(logs))
    objs = [o for o, _ in results]
    tmp = lib + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, lib)
    return lib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--resource-usage", action="store_true")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="build libdssm_stamps.so with per-phase cycle stamps")
    a = ap.parse_args()
    print(build(a.verbose, a.resource_usage, a.phase_stamps))


if __name__ == "__main__":
    main()
