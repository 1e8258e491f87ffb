"""Writes tests/golden/tiny_oracle_f64.txt from the CPU oracle only.

The pages print no Gated DeltaNet values, so this fixture is a regression
pin of the oracle itself on the tiny workload (1 sequence, T=128, one head,
d_k = d_v = 32, fp32 inputs, seed 0); its correctness rests on the pins in
tests/test_oracle.py.  Run from the repository root:
    python tests/golden/make_golden.py
"""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import gdn_inputs as gi  # noqa: E402
import oracle  # noqa: E402


def main():
    x = gi.tiny()
    out, fin, _ = oracle.forward_inputs(x, precision="f64")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle_f64.txt")
    fmt = lambda a: " ".join(f"{float(v):.17g}" for v in np.ravel(a))
    with open(path, "w") as f:
        f.write("# CPU oracle (fp64) on the tiny workload: T=128, H=1, d=32, seed 0.\n")
        f.write("# Written by tests/golden/make_golden.py; calls only oracle/.\n")
        f.write(f"out[::16,0,:4] = {fmt(out[::16, 0, :4])}\n")
        f.write(f"final[0,0,::8,::8] = {fmt(fin[0, 0, ::8, ::8])}\n")
        f.write(f"norm(out) = {fmt([np.linalg.norm(out)])}\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
