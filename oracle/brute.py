"""Pure-Python evaluation of the attention definition for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).

No NumPy: explicit loops over nested lists indexed [b][n][h][d], dot products
and sums with math.fsum (exactly rounded sums), math.exp and math.log.  It is
an independent route to the same definition as ``attention.py`` (see that
module for the citations) and exists to catch vectorisation mistakes there:
a transposed operand, a reduction over the wrong axis, a causal mask facing
the wrong way or a layout mix-up between [B][N][H][d] and [B][H][N][d].
"""

import math


def attention_brute(q, k, v, scale, causal):
    """q, k, v: nested lists [B][N][H][d] of floats.

    Returns (o, lse) as nested lists [B][N][H][d] and [B][H][N].
    """
    B = len(q)
    N = len(q[0])
    H = len(q[0][0])
    d = len(q[0][0][0])
    o = [[[[0.0] * d for _ in range(H)] for _ in range(N)] for _ in range(B)]
    lse = [[[0.0] * N for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(N):
                visible = [j for j in range(N) if (not causal) or j <= i]
                scores = [scale * math.fsum(q[b][i][h][c] * k[b][j][h][c] for c in range(d))
                          for j in visible]
                top = max(scores)
                weights = [math.exp(s - top) for s in scores]
                total = math.fsum(weights)
                for c in range(d):
                    o[b][i][h][c] = math.fsum(w * v[b][j][h][c]
                                              for w, j in zip(weights, visible)) / total
                lse[b][h][i] = top + math.log(total)
    return o, lse
