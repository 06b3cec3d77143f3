"""Writes the oracle's regression fixtures in this folder.

It calls only the CPU oracle (and the seeded input generator); nothing here
comes from the GPU library. Run from the repository root:
    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import ffn_inputs as fi  # noqa: E402
import oracle  # noqa: E402


def main():
    here = os.path.dirname(os.path.abspath(__file__))
    out = oracle.ffn(fi.make_config(0))
    np.savetxt(os.path.join(here, "tiny_silu_m1_out.txt"), out.reshape(-1), fmt="%.17g",
               header="oracle output of the tiny SwiGLU case (M=1, K=256, N=512, seed 20261202), "
                      "written by tests/golden/make_golden.py")


if __name__ == "__main__":
    main()
