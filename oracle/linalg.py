"""fp64 matmul, SwiGLU, bf16 rounding and the parity error metric.

TEST INFRASTRUCTURE ONLY (see the package docstring).

GEMM. With x in bf16 and BFP-decoded weights (at most 8 significant bits each) every
product x_k * w_k is exact in fp64; the oracle sums them in fp64 (a BLAS matmul serves as
the summation step) and rounds once at the declared output precision. Rows of x share
one pass over the weights, as the pages' multi-user decode does ("Qwen3.8-27B ...",
section "What changed in this release (s27v6-20261024)": up to 32 rows fit one tile row
and every weight is read once per step).

SwiGLU. h = silu(g) * u with silu(g) = g / (1 + exp(-g)), in fp64.

Greedy pick. The token greedy decoding emits is the column of the largest LM-head logit
("Qwen3.6-35B-A3B ...", section "Fused decode kernels": greedy argmax over the tiled
logits, up to 16 rows). The pages say nothing of ties or NaN; the reading taken: the
first such column, NaN counting as larger than every number, -0 equal to +0.

Error metric. A GPU result y is compared per output element with
|y - y_oracle| / sum_k |x_k * w_k|, the normaliser computed here in fp64 from the same
operands; if the normaliser is 0 the values must be equal.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round fp64 values straight to bf16 (8 significant bits), ties to even.

    Returns the rounded values as fp64 (exactly bf16-representable). Rounding goes
    directly from fp64 (no fp32 detour, so no double rounding). With v = f * 2**e,
    f in [0.5, 1), the bf16 quantum is 2**(max(e, -125) - 8): 8 significant bits for
    normal results, a fixed 2**-133 step in the subnormal range. Results that round
    past the largest finite bf16 become inf.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    q = np.maximum(e, -125) - 8
    out = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    big = np.abs(out) >= 2.0 ** 128
    if np.any(big):
        out = np.where(big, np.copysign(np.inf, v), out)
    return out


def gemm(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y[m][n] = sum_k x[m][k] * w[n][k] in fp64 (x [M][K], w [N][K], both fp64 values)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return x @ w.T


def normaliser(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """sum_k |x[m][k] * w[n][k]| in fp64: the scale the parity tolerance is relative to."""
    return np.abs(np.asarray(x, np.float64)) @ np.abs(np.asarray(w, np.float64)).T


def silu(g: np.ndarray) -> np.ndarray:
    """g / (1 + exp(-g)) in fp64, written so that exp never overflows."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    pos = g >= 0
    out[pos] = g[pos] / (1.0 + np.exp(-g[pos]))
    eg = np.exp(g[~pos])
    out[~pos] = g[~pos] * eg / (1.0 + eg)
    return out


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """h = silu(g) * u (gate projection g, up projection u)."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def sigmoid(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def rel_err(y: np.ndarray, y_ref: np.ndarray, norm: np.ndarray) -> np.ndarray:
    """|y - y_ref| / norm elementwise; where norm == 0 the result is 0 if equal else inf."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    norm = np.asarray(norm, dtype=np.float64)
    d = np.abs(y - y_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(norm > 0, d / np.where(norm > 0, norm, 1.0), np.where(d == 0, 0.0, math.inf))
    return r


def greedy_pick(y: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per row of logits y [M][N]: (index, value) of the first column holding the row's
    maximum, NaN counting as larger than any number (so the first NaN wins) and -0 as equal
    to +0. A plain scan over the columns in order; returns int64 [M] and y's dtype [M]."""
    y = np.asarray(y)
    m, n = y.shape
    idx = np.zeros(m, dtype=np.int64)
    val = np.zeros(m, dtype=y.dtype)
    for i in range(m):
        best = 0
        for j in range(1, n):
            if math.isnan(y[i, best]):
                break
            v = y[i, j]
            if math.isnan(v) or v > y[i, best]:
                best = j
        idx[i] = best
        val[i] = y[i, best]
    return idx, val
