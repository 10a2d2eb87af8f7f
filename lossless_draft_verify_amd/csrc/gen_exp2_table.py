"""Writes exp2_table.inc: 2^(j/2048) for j = 0..2047 as C99 hex-float literals,
each the double nearest the exact value (computed with 60-digit decimal
arithmetic; float() of a decimal string rounds correctly).

    python lossless_draft_verify_amd/csrc/gen_exp2_table.py
"""
import os
from decimal import Decimal, getcontext

getcontext().prec = 60


def main():
    ln2 = Decimal(2).ln()
    vals = [float(str((ln2 * Decimal(j) / Decimal(2048)).exp())) for j in range(2048)]
    assert vals[0] == 1.0 and all(1.0 <= v < 2.0 for v in vals)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exp2_table.inc")
    with open(out, "w") as fh:
        fh.write("// 2^(j/2048), j = 0..2047, nearest doubles; written by gen_exp2_table.py\n")
        for i in range(0, 2048, 4):
            fh.write("    " + ", ".join(v.hex() for v in vals[i:i + 4]) + ",\n")
    print(out)


if __name__ == "__main__":
    main()
