"""Pure-Python scalar loops: an independent second reading of the shard's definitions.

Written element by element from the definitions (no numpy arithmetic), for tiny inputs only.  Used
to pin the oracle; never used as the reference for the GPU.
"""

import math


def tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def matmul_bias(A, W, b=None):
    A, W = tolist(A), tolist(W)
    b = tolist(b) if b is not None else None
    n, k, m = len(A), len(W), len(W[0])
    out = []
    for i in range(n):
        row = []
        for j in range(m):
            s = 0.0
            for t in range(k):
                s += A[i][t] * W[t][j]
            if b is not None:
                s += b[j]
            row.append(s)
        out.append(row)
    return out


def gelu(x):
    return 0.5 * x * (1.0 + math.erf(x / math.sqrt(2.0)))


def gelu_prime(x):
    return 0.5 * (1.0 + math.erf(x / math.sqrt(2.0))) + x * math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)


def attention(QKV, B, S, nh, d):
    """ctx[b*S+i][h*d+c], lse[b][h][i] from the interleaved columns h*3d + s*d + c."""
    QKV = tolist(QKV)
    ctx = [[0.0] * (nh * d) for _ in range(B * S)]
    lse = [[[0.0] * S for _ in range(nh)] for _ in range(B)]
    for b in range(B):
        for h in range(nh):
            for i in range(S):
                qi = QKV[b * S + i][h * 3 * d: h * 3 * d + d]
                scores = []
                for j in range(i + 1):
                    kj = QKV[b * S + j][h * 3 * d + d: h * 3 * d + 2 * d]
                    scores.append(sum(qi[c] * kj[c] for c in range(d)) / math.sqrt(d))
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = sum(w)
                for c in range(d):
                    acc = 0.0
                    for j in range(i + 1):
                        acc += w[j] * QKV[b * S + j][h * 3 * d + 2 * d + c]
                    ctx[b * S + i][h * d + c] = acc / z
                lse[b][h][i] = m + math.log(z)
    return ctx, lse


def mlp_forward(X, W1, b1, W2, b2):
    A1 = matmul_bias(X, W1, b1)
    Y = [[gelu(v) for v in row] for row in A1]
    Z = matmul_bias(Y, W2, b2)
    return A1, Y, Z


def mlp_backward(X, W1, W2, A1, Y, dZ):
    """dX, dW1, db1, dW2, db2 element by element."""
    X, W1, W2, A1, Y, dZ = map(tolist, (X, W1, W2, A1, Y, dZ))
    T, H, F = len(X), len(X[0]), len(W1[0])
    dA1 = [[sum(dZ[t][c] * W2[f][c] for c in range(H)) * gelu_prime(A1[t][f]) for f in range(F)]
           for t in range(T)]
    dW2 = [[sum(Y[t][f] * dZ[t][c] for t in range(T)) for c in range(H)] for f in range(F)]
    db2 = [sum(dZ[t][c] for t in range(T)) for c in range(H)]
    db1 = [sum(dA1[t][f] for t in range(T)) for f in range(F)]
    dW1 = [[sum(X[t][i] * dA1[t][f] for t in range(T)) for f in range(F)] for i in range(H)]
    dX = [[sum(dA1[t][f] * W1[i][f] for f in range(F)) for i in range(H)] for t in range(T)]
    return {"dX": dX, "dW1": dW1, "db1": db1, "dW2": dW2, "db2": db2}


def linear_backward(X, W, dY):
    X, W, dY = map(tolist, (X, W, dY))
    T, H, N = len(X), len(X[0]), len(W[0])
    dW = [[sum(X[t][i] * dY[t][j] for t in range(T)) for j in range(N)] for i in range(H)]
    db = [sum(dY[t][j] for t in range(T)) for j in range(N)]
    dX = [[sum(dY[t][j] * W[i][j] for j in range(N)) for i in range(H)] for t in range(T)]
    return {"dX": dX, "dW": dW, "db": db}


def layernorm(h, gamma, beta, eps):
    """y, mean, rstd of each row by scalar loops: two passes (mean, then the biased variance)."""
    h, gamma, beta = map(tolist, (h, gamma, beta))
    ys, means, rstds = [], [], []
    for row in h:
        n = len(row)
        m = 0.0
        for v in row:
            m += v
        m /= n
        var = 0.0
        for v in row:
            var += (v - m) * (v - m)
        var /= n
        r = 1.0 / math.sqrt(var + eps)
        ys.append([(row[j] - m) * r * gamma[j] + beta[j] for j in range(n)])
        means.append(m)
        rstds.append(r)
    return ys, means, rstds
