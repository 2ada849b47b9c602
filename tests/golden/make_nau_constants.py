"""Writes nau_constants.txt from exact integer arithmetic (no oracle or kernel code).

Y_i = rint(2^(i/8) * 2^30), i = 0..8: the endpoints of the 8 chords of 2^v per
octave (the 8-segment first-order approximation of 2^v named on the FastMamba
review page, "What carries the argument").  rint is decided from
floor(2 * value) = floor((2^(i+248))^(1/8)), an exact integer 8th root.
LOG2E_Q30 = rint(log2(e) * 2^30) from 50-digit decimal arithmetic.
"""
import os
from decimal import Decimal, getcontext


def iroot(n, k):
    lo, hi = 0, 1 << (n.bit_length() // k + 2)
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if mid ** k <= n:
            lo = mid
        else:
            hi = mid - 1
    return lo


def main():
    lines = ["# name value  (see make_nau_constants.py for the derivation)"]
    for i in range(9):
        twice = iroot(2 ** (i + 248), 8)
        lines.append(f"Y{i} {twice // 2 + (twice & 1)}")
    getcontext().prec = 50
    log2e = Decimal(1) / Decimal(2).ln()
    lines.append(f"LOG2E_Q30 {int((log2e * 2 ** 30).to_integral_value())}")
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "nau_constants.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
