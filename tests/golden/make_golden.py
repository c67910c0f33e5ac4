"""Write the golden fixtures of this folder.  Calls only ``oracle/`` (and the
seeded input generator); run from the repository root:

    python tests/golden/make_golden.py

shift_r3_n8.txt -- the Shift construction of "Simplifying and Understanding
State Space Models with Diagonal Linear RNNs", section 3.1 (a one-hot kernel at
r shifts the sequence by r), realised as a DLR with (log L)_re = 0,
(log L)_im = 2 pi n / N and w_n = exp(-2 pi i n r / N) / N (N = 8, r = 3,
D = 0.75), on an integer input of length 40.  Columns: k, u_k, y_k.

tiny_dlr.txt -- the tiny workload (B=1, H=4, N=16, L=256, seed 0) through
oracle.dlr_direct.  Columns: h, k, u, y.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from long_convolution_sequence_amd import inputs  # noqa: E402


def main():
    N, L, r = 8, 40, 3
    n = np.arange(N)
    re = np.zeros((1, 1, N))
    im = (2 * np.pi * n / N)[None, None, :]
    w = (np.exp(-2j * np.pi * n * r / N) / N)[None, None, :]
    u = np.random.default_rng(1).integers(-5, 6, size=(1, 1, L)).astype(np.float64)
    y = oracle.dlr_direct(u, re, im, w, np.array([[0.75]]))
    np.savetxt(os.path.join(HERE, "shift_r3_n8.txt"),
               np.stack([np.arange(L), u[0, 0], y[0, 0]], axis=1),
               fmt=["%d", "%.1f", "%.17g"],
               header="Shift pin (DLR page, section 3.1), N=8 r=3 D=0.75; written by make_golden.py from oracle.dlr_direct\nk u y")
    c = inputs.config("tiny")
    x = inputs.inputs_for(c)
    y = oracle.dlr_direct(x["u"], x["log_re"], x["log_im"], x["W"], x["D"], False)
    H, L = c["H"], c["L"]
    hh, kk = np.meshgrid(np.arange(H), np.arange(L), indexing="ij")
    np.savetxt(os.path.join(HERE, "tiny_dlr.txt"),
               np.stack([hh.ravel(), kk.ravel(), x["u"][0].ravel().astype(np.float64), y[0].ravel()], axis=1),
               fmt=["%d", "%d", "%.9g", "%.17g"],
               header="tiny workload (B=1 H=4 N=16 L=256 seed 0) through oracle.dlr_direct; written by make_golden.py\nh k u y")


if __name__ == "__main__":
    main()
