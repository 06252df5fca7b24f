"""Write tests/golden/integer_scan.txt by calling only the oracle.

The pages print no worked numeric example, so the only stored expected values
are exact-integer results of the oracle: decay 1 (A = 0), unit step (softplus
off), small integer u, B, C, D, and impulses placed at both sides of the chunk
boundaries t = kK - 1, kK, kK + 1 for K = 16.  Every intermediate value is an
integer below 2^24, so any correct float evaluation reproduces them exactly.
Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

OUT = os.path.join(HERE, "integer_scan.txt")


def inputs():
    batch, d_inner, N, L = 1, 2, 4, 50
    u = np.zeros((batch, d_inner, L))
    for k in (1, 2, 3):
        for t in (16 * k - 1, 16 * k, 16 * k + 1):
            u[0, 0, t] = (t % 5) - 2 or 1
            u[0, 1, t] = 2 - (t % 3)
    u[0, :, 0] = [3, -1]
    u[0, :, L - 1] = [-2, 2]
    t = np.arange(L)
    B = np.stack([(t * (n + 1)) % 5 - 2 for n in range(N)])[None].astype(np.float64)
    C = np.stack([(t + 2 * n) % 3 - 1 for n in range(N)])[None].astype(np.float64)
    D = np.array([2.0, -1.0])
    return u, np.ones_like(u), np.zeros((d_inner, N)), B, C, D


def main():
    u, dt, A, B, C, D = inputs()
    y, last = oracle.scan_fwd(u, dt, A, B, C, D, softplus=False)
    with open(OUT, "w") as f:
        f.write("# exact-integer scan written by tests/golden/make_golden.py (oracle only)\n")
        f.write("# inputs: see make_golden.inputs(); shape batch=1 d_inner=2 N=4 L=50\n")
        for d in range(2):
            f.write("y%d %s\n" % (d, " ".join("%d" % v for v in y[0, d])))
        for d in range(2):
            f.write("h%d %s\n" % (d, " ".join("%d" % v for v in last[0, d])))


if __name__ == "__main__":
    main()
