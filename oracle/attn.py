"""BFP8 KV cache and single-token decode attention, fp64 — TEST INFRASTRUCTURE ONLY.

(See the package docstring: only the tests, the smoke check and the bench's CPU leg use it.)

Sources:

* "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8 (GPTQ experts), single P150", table in
  "Precision as served" (the KV cache is stored in BFP8) and the serving-settings table,
  KV-precision row (BFP8 halves the cache, 20.0 -> 10.6 KiB per token; decode attention
  reads the whole cache every step, so the smaller cache makes it faster at long contexts).
* "Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", changes in s27-20261005, DFlash2 at 262K
  (the long-context cache keeps K in BFP8 and V in 4-bit BFP4 after a Hadamard rotation).

Readings (the pages name the cache format only):

* Every cached key and value vector (one token, one KV head, ``head_dim`` values) is
  encoded like a weight row: 16-value blocks along ``head_dim``, exactly ``bfp.encode``.
* Cache layout (ours): per KV head, tokens in order: ``exp[kv_heads][tokens][head_dim/16]``
  and ``code[kv_heads][tokens][head_dim]`` for K and for V.
* The rotated 4-bit V (the pages name only "4-bit after a Hadamard rotation"): each value
  vector v (head_dim a power of two) is replaced by H v / sqrt(head_dim), H the Sylvester
  Hadamard matrix (H_1 = [1], H_2n = [[H, H], [H, -H]]), computed in fp64 by the fast
  transform (stages h = 1, 2, 4, ...: x_j, x_j+h <- x_j + x_j+h, x_j - x_j+h within blocks of
  2h), times the fp64 constant 1/sqrt(head_dim), rounded to fp32, then encoded in BFP4. The
  transform is orthonormal and its own inverse, so attention over the decoded rotated values
  is rotated back by the same transform.
* Decode attention is the usual scaled dot-product attention of one query token over the
  first ``L`` cached tokens, with grouped query heads: query head h reads KV head
  h // (q_heads / kv_heads). Scores s_t = scale * q . k_t, probabilities p = softmax(s)
  over t < L, output sum_t p_t v_t; the keys and values are the decoded cache entries.
"""
from __future__ import annotations

import numpy as np

from .bfp import BFP4, BFP8, decode, encode

# 1 / sqrt(head_dim) as fp64 constants (written out: the transform must scale by exactly these)
INV_SQRT = {64: 0.125, 128: 0.08838834764831845, 256: 0.0625}


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """H x / sqrt(d) along the last axis (d = 64, 128 or 256), fp64, by the fast transform's
    stages in order (see the module notes)."""
    y = np.array(x, dtype=np.float64)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        y = y.reshape(*lead, d // (2 * h), 2, h)
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*lead, d)
        h *= 2
    return y * INV_SQRT[d]


def kv_encode_rotated(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The 4-bit V of the rotated cache: rows rotated (fp64), rounded to fp32, BFP4-encoded;
    cache layout as kv_encode."""
    r = hadamard_rotate(np.asarray(x, dtype=np.float32)).astype(np.float32)
    return kv_encode(r, BFP4)


def kv_encode(x: np.ndarray, fmt: int = BFP8) -> tuple[np.ndarray, np.ndarray]:
    """Encode cache rows. x: fp32 [tokens][kv_heads][head_dim]. Returns (exp, code) in the
    cache layout: exp uint8 [kv_heads][tokens][head_dim/16], code uint8 [kv_heads][tokens][...]."""
    x = np.asarray(x, dtype=np.float32)
    t, h, d = x.shape
    rows = np.ascontiguousarray(x.transpose(1, 0, 2)).reshape(h * t, d)
    exp, code = encode(rows, fmt)
    return exp.reshape(h, t, d // 16), code.reshape(h, t, -1)


def kv_decode(exp: np.ndarray, code: np.ndarray, fmt: int, head_dim: int) -> np.ndarray:
    """Decoded cache entries, fp64 [kv_heads][tokens][head_dim]."""
    h, t = exp.shape[0], exp.shape[1]
    rows = decode(exp.reshape(h * t, -1), code.reshape(h * t, -1), fmt, h * t, head_dim)
    return rows.reshape(h, t, head_dim)


def decode_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> tuple[np.ndarray, np.ndarray]:
    """One query token against L cached tokens, fp64.

    q: [q_heads][head_dim]; k, v: [kv_heads][L][head_dim] (decoded values). Returns
    (out [q_heads][head_dim], norm [q_heads][head_dim]) with norm = sum_t p_t |v_t|, the
    scale the parity tolerance of an output is relative to."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    hq, d = q.shape
    hkv, L, _ = k.shape
    group = hq // hkv
    out = np.zeros((hq, d))
    norm = np.zeros((hq, d))
    for h in range(hq):
        g = h // group
        s = scale * (k[g] @ q[h])            # [L]
        e = np.exp(s - s.max())
        p = e / e.sum()
        out[h] = p @ v[g]
        norm[h] = p @ np.abs(v[g])
    return out, norm
