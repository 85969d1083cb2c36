"""Writes the 2^(j/64) table of csrc/sd_exp.h (j = 0 .. 63), each value correctly rounded to fp64.

Run from the repository root: python query_adaptive_sparse_amd/gen_exp_table.py (prints the macro
body to paste into the header).
"""
from decimal import Decimal, getcontext


def table():
    getcontext().prec = 60
    ln2 = Decimal(2).ln()
    # float() of a decimal string rounds correctly to the nearest fp64 value
    return [float(str((ln2 * j / 64).exp())) for j in range(64)]


if __name__ == "__main__":
    t = table()
    for i in range(0, 64, 4):
        print("    " + ", ".join(v.hex() for v in t[i:i + 4]) + ", \\")
