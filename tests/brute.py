"""Brute-force reference loops for tiny inputs: plain Python floats, math.erf and
math.exp, no numpy arithmetic. Used only to pin the vectorised oracle."""
import math


def matmul(A, B):
    n, k = len(A), len(A[0])
    m = len(B[0])
    assert len(B) == k
    return [[sum(A[i][p] * B[p][j] for p in range(k)) for j in range(m)] for i in range(n)]


def gelu(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def mlp(X, A, B):
    U = matmul(X, A)
    Y = [[gelu(u) for u in row] for row in U]
    return matmul(Y, B)


def attention_head(q, k, v, causal):
    """q, k, v: lists of rows (s x d). Returns s x d."""
    s, d = len(q), len(q[0])
    out = []
    for t in range(s):
        last = t + 1 if causal else s
        sc = [sum(q[t][c] * k[u][c] for c in range(d)) / math.sqrt(d) for u in range(last)]
        m = max(sc)
        e = [math.exp(x - m) for x in sc]
        z = sum(e)
        out.append([sum(e[u] * v[u][c] for u in range(last)) / z for c in range(d)])
    return out


def layernorm(X, gamma, beta, eps):
    """Row by row: mean, biased variance, normalise, scale and shift."""
    out = []
    for row in X:
        n = len(row)
        mu = sum(row) / n
        var = sum((x - mu) * (x - mu) for x in row) / n
        inv = 1.0 / math.sqrt(var + eps)
        out.append([(x - mu) * inv * g + b for x, g, b in zip(row, gamma, beta)])
    return out
