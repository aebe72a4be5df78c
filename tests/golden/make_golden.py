"""Writes the stored expected values under tests/golden/ from the CPU oracle only.

    python tests/golden/make_golden.py

nf4_codebook.txt: the 16 float32 NF4 levels (index, hex, decimal) of the oracle's derivation
(QLoRA construction from standard-normal quantiles; the Unsloth pages name NF4 in the
v0.1.463-beta release article, "About the Unsloth Project", but print no values).

e2m1_codebook.txt: the 16 E2M1 values by code (1 sign, 2 exponent and 1 mantissa bits, largest
magnitude 6, as the NVFP4 update article's section "NVFP4: A Quantization Format for the Next
Generation of Hardware" gives them), from oracle/fp4.py.
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import fp4, nf4  # noqa: E402


def main():
    c = nf4.codebook()
    with open(os.path.join(HERE, "nf4_codebook.txt"), "w") as f:
        f.write("# NF4 levels, float32, written by tests/golden/make_golden.py from oracle/nf4.py\n")
        f.write("# index  hex  decimal\n")
        for i, v in enumerate(c):
            f.write(f"{i:2d} {float(v).hex()} {float(v):.9g}\n")
    with open(os.path.join(HERE, "e2m1_codebook.txt"), "w") as f:
        f.write("# E2M1 values by code (sign bit 3), written by tests/golden/make_golden.py from "
                "oracle/fp4.py\n")
        f.write("# code  hex  decimal\n")
        for i, v in enumerate(fp4.e2m1_codebook()):
            f.write(f"{i:2d} {float(v).hex()} {float(v):.9g}\n")


if __name__ == "__main__":
    main()
