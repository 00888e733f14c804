"""Write the closed-form fixtures under tests/golden/ (exact integer math).

Fixtures:
* ``log_delannoy.json``: ln Del(N-1, M-1) for the workload shapes.  With a
  zero distance matrix (x and y the same constant sequence) every one of the
  Del(N-1, M-1) alignment paths costs 0, so Soft-DTW equals
  -gamma * ln Del(N-1, M-1): negative, as the README "SoftDTW-CUDA (PyTorch +
  Numba)" says Soft-DTW may be ("Notes").  Del(m, n) counts lattice paths
  with unit steps right, up and diagonal (Delannoy numbers).
* ``two_by_two.json``: a 2x2 worked case of the closed form
  sdtw = D00 + D11 - g ln(1 + e^{-D01/g} + e^{-D10/g}) with exact inputs.

Run: python tests/golden/make_golden.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))


def delannoy(m, n):
    row = [1] * (n + 1)
    for _ in range(1, m + 1):
        new = [1] * (n + 1)
        for j in range(1, n + 1):
            new[j] = new[j - 1] + row[j] + row[j - 1]
        row = new
    return row[n]


def main():
    shapes = [(16, 16), (100, 100), (256, 256), (512, 512), (1024, 1024),
              (2048, 2048), (4096, 4096), (4096, 1000), (16, 9), (1, 7)]
    out = {"source": "exact Delannoy numbers (integer recurrence), ln taken "
                     "by math.log on the integer",
           "values": [{"N": n, "M": m, "log_delannoy": math.log(delannoy(n - 1, m - 1))}
                      for n, m in shapes]}
    with open(os.path.join(HERE, "log_delannoy.json"), "w") as f:
        json.dump(out, f, indent=1)
    # 2x2 worked case: inputs are small dyadic numbers, exact in fp32/fp64.
    d = [[0.5, 1.25], [2.0, 0.75]]
    g = 0.5
    val = d[0][0] + d[1][1] - g * math.log(1 + math.exp(-d[0][1] / g) + math.exp(-d[1][0] / g))
    z = 1 + math.exp(-d[0][1] / g) + math.exp(-d[1][0] / g)
    E = [[1.0, math.exp(-d[0][1] / g) / z], [math.exp(-d[1][0] / g) / z, 1.0]]
    with open(os.path.join(HERE, "two_by_two.json"), "w") as f:
        json.dump({"source": "closed form of the 3 paths of a 2x2 grid",
                   "dist": d, "gamma": g, "value": val, "E": E}, f, indent=1)


if __name__ == "__main__":
    main()
