"""Brute-force versions of the path's steps in plain Python (tiny inputs only).

Written directly from the definitions, with Python floats and the math
module, independently of the C oracle: nested loops, a full sort for the
selection, a materialised softmax without max subtraction.
"""
import math


def gelu(x):
    return x * 0.5 * (1.0 + math.erf(x / math.sqrt(2.0)))


def scores(h, w1, b1, w2, b2, eps):
    out = []
    for row in h:
        d = len(row)
        r = 1.0 / math.sqrt(sum(x * x for x in row) / d + eps)
        s = 0.0
        for j, wj in enumerate(w1):
            a = r * sum(x * w for x, w in zip(row, wj)) + (b1[j] if b1 is not None else 0.0)
            s += w2[j] * gelu(a)
        out.append(s + b2)
    return out


def seq_norm(s, eps):
    rho = math.sqrt(sum(x * x for x in s) / len(s) + eps)
    return [x / rho for x in s]


def select(score, forced, k):
    n = len(score)
    prunable = [i for i in range(n) if not forced[i]]
    f = n - len(prunable)
    ranked = sorted(prunable, key=lambda i: (-score[i], i))
    kept = set(i for i in range(n) if forced[i]) | set(ranked[: k - f])
    return sorted(kept)


def attention(q, k, v, ks, gains, c, pos):
    """q[t][h][e], k/v[j][hk][e]; returns out[t][h][e]."""
    K = len(q)
    hq = len(q[0])
    hkv = len(k[0])
    D = len(q[0][0])
    G = hq // hkv
    out = []
    for t in range(K):
        lam = 1.0 + c * math.log((t + 1) / (pos[t] + 1))
        row = []
        for h in range(hq):
            hk = h // G
            w = []
            for j in range(t + 1):
                dot = sum(q[t][h][e] * k[j][hk][e] for e in range(D))
                w.append(math.exp(lam * (dot / math.sqrt(D) + gains[h] * ks[j])))
            den = sum(w)
            row.append([sum(w[j] * v[j][hk][e] for j in range(t + 1)) / den for e in range(D)])
        out.append(row)
    return out
