"""Writes the frozen oracle tables under tests/golden/.  Calls only oracle/.

    python tests/golden/make_golden.py

nf4_codebook.txt: the 16 NF4 levels q and the 15 level midpoints m, as fp32 hex floats.
The pages print no codebook ("Can You Fine-Tune a 27B Model on a Laptop?", transcript
@2:19 only says the levels sit where normally distributed weights fall); the table is the
oracle's reading (normal quantiles, QLoRA's construction), frozen here so that any later
change to it shows up as a test failure.
"""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import nf4  # noqa: E402


def main():
    q = nf4.codebook()
    m = nf4.code_thresholds()
    with open(os.path.join(HERE, "nf4_codebook.txt"), "w") as f:
        f.write("# NF4 codebook (oracle reading: normal quantiles, P_MAX = %r)\n" % nf4.P_MAX)
        f.write("# kind index fp32-hex decimal\n")
        for i, v in enumerate(q):
            f.write(f"q {float(v).hex()} {i} {float(v):.9g}\n")
        for i, v in enumerate(m):
            f.write(f"m {float(v).hex()} {i} {float(v):.9g}\n")
    assert q.dtype == np.float32


if __name__ == "__main__":
    main()
