"""Small helpers for the oracle pins: bf16 inputs with chosen values, and a
pure-Python attention that materialises the whole score matrix (tiny sizes
only).  It is written independently of the C oracle: one dense L x L score
matrix, then the weights, then the products."""
import math

import numpy as np

from synthetic import bf16_bits_to_f32, f32_to_bf16_bits

SIGMOID, SOFTMAX, SOFTMAX1 = 0, 1, 2
BIAS_NONE, BIAS_LOG_SEQLEN, BIAS_LOG_PADLEN = 0, 1, 2


def bf16(x):
    """float array -> bf16 bits (uint16)."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def widen(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def random_inputs(rng, B, H, L, d, names=("q", "k", "v")):
    return [bf16(rng.standard_normal((B, H, L, d))) for _ in names]


def dense_python(qf, kf, vf, n, mask_b, bias, variant, scale):
    """One head.  qf, kf, vf: float lists/arrays [L][d].  Returns (o, weights)."""
    L = len(qf)
    d = len(qf[0])
    n = max(0, min(int(n), L))
    beta = 0.0
    if n > 0 and bias == BIAS_LOG_SEQLEN:
        beta = -math.log(n)
    elif n > 0 and bias == BIAS_LOG_PADLEN:
        beta = -math.log(L)
    S = [[None] * L for _ in range(L)]
    for r in range(L):
        for c in range(L):
            ok = r < n and c < n and (mask_b is None or mask_b[r][c] != 0)
            if ok:
                S[r][c] = scale * sum(float(qf[r][t]) * float(kf[c][t]) for t in range(d)) + beta
    W = [[0.0] * L for _ in range(L)]
    for r in range(L):
        row = [S[r][c] for c in range(L) if S[r][c] is not None]
        if r >= n or (not row and variant != SOFTMAX1):
            continue
        if variant == SIGMOID:
            for c in range(L):
                if S[r][c] is not None:
                    W[r][c] = 1.0 / (1.0 + math.exp(-S[r][c]))
        elif variant == SOFTMAX:
            total = sum(math.exp(x) for x in row)
            for c in range(L):
                if S[r][c] is not None:
                    W[r][c] = math.exp(S[r][c]) / total
        else:
            total = 1.0 + sum(math.exp(x) for x in row)
            for c in range(L):
                if S[r][c] is not None:
                    W[r][c] = math.exp(S[r][c]) / total
    O = [[sum(W[r][c] * float(vf[c][t]) for c in range(L)) for t in range(d)] for r in range(L)]
    return np.array(O), np.array(W)
