"""Writes the closed-form fixtures in this folder.

Calls nothing but the Python standard library: every value is a closed form of
the mathematics, not an output of any implementation.

* geometric_series.txt -- [RN-zh] "2) Retention 的循環表征", Eq. (6) with
  d_k = d_v = 1 and q = k = v = 1: S_n = gamma S_{n-1} + 1, o_n = S_n, so
  o_n = sum_{m=0..n} gamma^m = (1 - gamma^(n+1)) / (1 - gamma)  (n + 1 when
  gamma = 1).
* rotary_unit.txt -- [RN-zh] "Retention", Eq. (3)-(4) (xPos): the pair
  (1, 0) read as 1 + 0i multiplied by e^{i p theta_j}, theta_j =
  base^(-2j/d), becomes (cos p theta_j, sin p theta_j).
"""
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    with open(os.path.join(HERE, "geometric_series.txt"), "w") as f:
        f.write("# gamma n o_n   (closed form of Eq. (6) with unit q, k, v; see make_golden.py)\n")
        for gamma in (0.0, 0.5, 0.75, 0.96875, 1.0):
            for n in range(12):
                o = n + 1.0 if gamma == 1.0 else (1.0 - gamma ** (n + 1)) / (1.0 - gamma)
                f.write(f"{gamma!r} {n} {o!r}\n")
    with open(os.path.join(HERE, "rotary_unit.txt"), "w") as f:
        f.write("# base d j p cos(p*theta_j) sin(p*theta_j), theta_j = base^(-2j/d)\n")
        for base, d in ((10000.0, 4), (10000.0, 64), (500.0, 8)):
            for j in (0, 1, d // 2 - 1):
                for p in (0, 1, 2, 7, 100, 8191):
                    th = base ** (-2.0 * j / d)
                    f.write(f"{base!r} {d} {j} {p} {math.cos(p * th)!r} {math.sin(p * th)!r}\n")


if __name__ == "__main__":
    main()
