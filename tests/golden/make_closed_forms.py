"""Writes cnp_closed_forms.txt: exact values of the Cayley-Neumann block G and of
the exact Cayley transform C for small skew-symmetric Q, from closed forms.

Derivation (from the k = 3 form G = (I + Q)(I + Q + Q^2 + Q^3) of the POET
paper notes, "Reparameterized LLM Training via Orthogonal Equivalence
Transformation", 关键设计 2, and its expansion in the zhichai.net POET-X blog,
第四斧 item 2):

  2 x 2, Q = [[0, q], [-q, 0]]:  Q^2 = -q^2 I, so
      G = (1 - q^2) [[1 - q^2, 2q], [-2q, 1 - q^2]]
      C = [[1 - q^2, 2q], [-2q, 1 - q^2]] / (1 + q^2)
  3 x 3, Q = [[0, a, b], [-a, 0, c], [-b, -c, 0]], t = a^2 + b^2 + c^2:
      Q^3 = -t Q, so
      G = I + (2 - 2t) Q + (2 - t) Q^2
      C = I + 2 (Q + Q^2) / (1 + t)

Everything is exact rational arithmetic (fractions); no oracle code is used.
Run:  python tests/golden/make_closed_forms.py
"""

from fractions import Fraction as F
from pathlib import Path


def mat_mul(A, B):
    n, k, m = len(A), len(B), len(B[0])
    return [[sum(A[i][t] * B[t][j] for t in range(k)) for j in range(m)] for i in range(n)]


def two_by_two(q):
    s = 1 - q * q
    G = [[s * s, s * 2 * q], [-s * 2 * q, s * s]]
    C = [[s / (1 + q * q), 2 * q / (1 + q * q)], [-2 * q / (1 + q * q), s / (1 + q * q)]]
    return G, C


def three_by_three(a, b, c):
    Q = [[F(0), a, b], [-a, F(0), c], [-b, -c, F(0)]]
    Q2 = mat_mul(Q, Q)
    t = a * a + b * b + c * c
    I = [[F(int(i == j)) for j in range(3)] for i in range(3)]
    G = [[I[i][j] + (2 - 2 * t) * Q[i][j] + (2 - t) * Q2[i][j] for j in range(3)] for i in range(3)]
    C = [[I[i][j] + 2 * (Q[i][j] + Q2[i][j]) / (1 + t) for j in range(3)] for i in range(3)]
    return G, C


def fmt(M):
    return " ".join(f"{x.numerator}/{x.denominator}" for row in M for x in row)


def main():
    lines = [
        "# Closed-form CNP (k = 3) and exact Cayley blocks; see make_closed_forms.py for the derivation.",
        "# format: case <name> | q <packed upper triangle, row-major> | G <row-major> | C <row-major>",
    ]
    for q in (F(3, 10), F(-1, 7), F(1, 2)):
        G, C = two_by_two(q)
        lines.append(f"case 2x2 | q {q.numerator}/{q.denominator} | G {fmt(G)} | C {fmt(C)}")
    for a, b, c in ((F(1, 5), F(-3, 10), F(1, 10)), (F(1, 20), F(1, 40), F(-1, 8))):
        G, C = three_by_three(a, b, c)
        q = " ".join(f"{x.numerator}/{x.denominator}" for x in (a, b, c))
        lines.append(f"case 3x3 | q {q} | G {fmt(G)} | C {fmt(C)}")
    out = Path(__file__).with_name("cnp_closed_forms.txt")
    out.write_text("\n".join(lines) + "\n")
    print(f"wrote {out}")


if __name__ == "__main__":
    main()
