"""Write tests/golden/tiny_bruteforce.json from oracle/bruteforce.py only.

The LightTransfer pages print no worked example for the lazy ratio, so the
stored values come from the 50-digit brute force of the plain definitions on
a small fixed input (integers over 4, exact in every float format).  Run:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import bruteforce as bf  # noqa: E402

# B=1, Hq=2, Hkv=1, N=6, D=2; values are small integers / 4.
Q = [[[[1, 0], [0, 2], [-1, 1], [2, 2], [0, -1], [1, 3]],
      [[-2, 1], [1, 1], [0, 0], [3, -1], [1, 2], [-1, -1]]]]
K = [[[[4, 0], [0, 1], [1, -1], [-2, 1], [1, 1], [0, 3]]]]
V = [[[[1, 2], [3, -1], [0, 0], [-2, 4], [1, 1], [2, -3]]]]
Q = [[[[x / 4 for x in row] for row in h] for h in b] for b in Q]
K = [[[[x / 4 for x in row] for row in h] for h in b] for b in K]
V = [[[[x / 4 for x in row] for row in h] for h in b] for b in V]
S, R, W = 1, 2, 3


def main():
    res = bf.attention(Q, K, V, S=S, R=R, W=W)

    def s(x):
        if isinstance(x, list):
            return [s(y) for y in x]
        return str(x)

    out = {"source": "oracle/bruteforce.py, 50 significant digits",
           "S": S, "R": R, "W": W, "q": Q, "k": K, "v": V,
           "expected": {key: s(val) for key, val in res.items()}}
    with open(os.path.join(HERE, "tiny_bruteforce.json"), "w") as f:
        json.dump(out, f, indent=1)


if __name__ == "__main__":
    main()
