"""Writes the stored expected values under tests/golden/ from the oracle alone.

Run from the repository root:  python tests/golden/make_golden.py
It imports only oracle/ (and numpy); nothing here comes from the HIP path.
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import nf4  # noqa: E402


def main():
    q = nf4.codebook_f32()
    with open(os.path.join(HERE, "nf4_codebook_f32.txt"), "w") as f:
        f.write("# NF4 levels (code, float32 bit pattern, value); written by make_golden.py from oracle.nf4\n")
        for c, (bits, v) in enumerate(zip(q.view(np.uint32), q)):
            f.write(f"{c} {bits:08x} {float(v)!r}\n")


if __name__ == "__main__":
    main()
