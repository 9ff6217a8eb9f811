"""Independent brute-force evaluation of attention for tiny inputs.

Written from the definition on the kbench page ("The three GPU kernels":
O = softmax(Q K^T / sqrt(d)) V) in 50-digit decimal arithmetic, and on
purpose shaped differently from the oracle: no max subtraction (decimal exp
cannot overflow here), the mask enters as a 0/1 factor on every key's weight,
and the output is assembled column by column as a ratio of two sums.
"""
from decimal import Decimal, localcontext


def brute_sdpa(Q, K, V, causal, scale=None):
    """Q, K, V: nested lists [S][d] of floats (one head).  Returns [S][d] Decimals."""
    with localcontext() as ctx:
        ctx.prec = 50
        S, d = len(Q), len(Q[0])
        sc = (Decimal(1) / Decimal(d).sqrt()) if scale is None else Decimal(scale)
        out = []
        for i in range(S):
            weights = []
            for j in range(S):
                visible = 0 if (causal and j > i) else 1
                logit = sc * sum(Decimal(float(Q[i][c])) * Decimal(float(K[j][c])) for c in range(d))
                weights.append(visible * logit.exp())
            total = sum(weights)
            row = []
            for c in range(d):
                num = sum(weights[j] * Decimal(float(V[j][c])) for j in range(S))
                row.append(num / total)
            out.append(row)
        return out
