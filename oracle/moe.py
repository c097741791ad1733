"""MoE layer with BFP4 experts: router, top-k, SwiGLU experts, shared expert, dispatch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The layer ("qwen3.6-a3b-blackhole" bundle page, introduction; "Qwen3.6-35B-A3B ...",
section "Precision as served"): 256 routed experts with top-8 routing plus one shared
expert; routed and shared experts in BFP4; the router in BF16. Decode runs device top-k
routing and batched expert streams ("Qwen3.6-35B-A3B ...", section "Fused decode
kernels"); prefill runs in 2,048-token chunks ("Qwen3.8-27B ...", section "What changed
in this release (s27v6-20261024)").

Readings taken where the pages are silent:

* Router logits l_e = sum_k x_k * Wr[e][k] (+ b_e when a per-expert bias is given), from
  exact bf16 x bf16 products summed in fp64.
* Selection: the top-k experts by (logit descending, expert index ascending), reported
  in that order. Where fp64 rounding could decide it (two logits that the selection compares
  closer than their error bound), the logits in question are recomputed exactly.
* Weights: p = softmax over all experts; r_j = p[e_j] / sum of p over the selected
  experts (softmax restricted to the top-k, renormalised).
* Shared-expert gate: g = sigmoid(x . g_s) with a bf16 vector g_s.
* Expert e: h = silu(x Wg_e^T) * (x Wu_e^T); o = h Wd_e^T.
* Output: y_t = sum_j r_tj * o_tj (slots in rank order) + g_t * shared(x_t).
* Decode keeps h unrounded; prefill rounds h to bf16 (ties to even) before the down
  projection, the point where a bf16 matrix-core path must round it.
* Dispatch for grouped execution: counts_e, offsets (exclusive prefix sum, E+1 entries)
  and the pair ids p = k*t + j sorted by (expert ascending, token ascending).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .bfp import decode, encode
from .linalg import bf16_round, bf16_to_f64, sigmoid, swiglu


def _exact_logits(x_row: np.ndarray, w_rows: np.ndarray, bias: np.ndarray | None) -> list:
    """Exact router logits as Fractions: every bf16 value is an integer multiple of 2**-133
    (the smallest bf16 subnormal), so x_k * w_k * 2**266 is an integer and the sum over k is
    exact in Python integers; a fp32 bias is added as the exact rational it is."""
    xi = [int(v) for v in np.ldexp(x_row, 133)]
    out = []
    for e, w in enumerate(w_rows):
        wi = [int(v) for v in np.ldexp(w, 133)]
        f = Fraction(sum(a * b for a, b in zip(xi, wi) if a and b), 2 ** 266)
        if bias is not None:
            f += Fraction(float(bias[e]))
        out.append(f)
    return out


def route(x_bits: np.ndarray, router_bits: np.ndarray, top_k: int = 8,
          bias: np.ndarray | None = None, sh_gate_bits: np.ndarray | None = None) -> dict:
    """Router + top-k + renormalised softmax weights + shared-expert gate (fp64).

    The logits are fp64 sums of exact bf16 products, so each is within
    d_e = 2 (n + 2) 2**-53 (sum_k |x_k w_k| + |b_e| + |l_e|) of its exact value (any
    summation order). Per token, the experts that could still reach the top-k are those whose
    upper end l_e + d_e is not below the k-th largest lower end; if any two of their intervals
    overlap, the order among them is not settled by the fp64 values, and their logits are
    recomputed exactly (``_exact_logits``) and replaced by the nearest doubles of the exact
    values before the selection and the weights. The selection itself is a plain sort by
    (logit descending, expert ascending).
    """
    x = bf16_to_f64(x_bits)
    wr = bf16_to_f64(router_bits)
    logits = x @ wr.T
    b64 = None
    if bias is not None:
        b64 = np.asarray(bias, dtype=np.float32).astype(np.float64)
        logits = logits + b64[None, :]
    m, n_exp = logits.shape
    n = x.shape[1]
    a = np.abs(x) @ np.abs(wr).T
    d = 2.0 * (n + 2) * 2.0 ** -53 * (a + np.abs(logits) + (np.abs(b64)[None, :] if b64 is not None else 0.0))
    exact = np.zeros(m, dtype=bool)
    for t in range(m):
        lo, hi = logits[t] - d[t], logits[t] + d[t]
        lk = np.sort(lo)[::-1][top_k - 1]              # k-th largest lower end
        cand = np.nonzero(hi >= lk)[0]
        lc, hc = lo[cand], hi[cand]
        overlap = (lc[:, None] <= hc[None, :]) & (lc[None, :] <= hc[:, None])
        np.fill_diagonal(overlap, False)
        if overlap.any():
            ex = _exact_logits(x[t], wr[cand], None if b64 is None else b64[cand])
            logits[t, cand] = [float(f) for f in ex]
            exact[t] = True
    ids = np.empty((m, top_k), np.int32)
    for t in range(m):
        order = sorted(range(n_exp), key=lambda e: (-logits[t, e], e))
        ids[t] = order[:top_k]
    lmax = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - lmax)
    p = p / p.sum(axis=1, keepdims=True)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    r = sel / sel.sum(axis=1, keepdims=True)
    out = {"ids": ids, "r": r, "logits": logits, "exact": exact}
    if sh_gate_bits is not None:
        out["g"] = sigmoid(x @ bf16_to_f64(sh_gate_bits))
    return out


def encode_layer(layer: dict) -> dict:
    """Encode every BFP4 matrix of a layer dict (fp32 weights) -> dict of (exp, code)."""
    fmt = layer["fmt"]
    q = {}
    for role in ("gate", "up", "down", "sh_gate", "sh_up", "sh_down"):
        q[role] = encode(layer[role], fmt)
    return q


class ExpertBank:
    """Decodes expert matrices from the stacked (exp, code) planes on demand."""

    def __init__(self, layer: dict, q: dict):
        self.fmt = layer["fmt"]
        self.hidden = layer["hidden"]
        self.inter = layer["inter"]
        self.q = q
        self._cache: dict = {}

    def _rows(self, role: str, r0: int, r1: int, k: int) -> np.ndarray:
        exp, code = self.q[role]
        cpr = code.shape[1]
        return decode(exp[r0:r1], code[r0:r1].reshape(-1, cpr), self.fmt, r1 - r0, k)

    def expert(self, e: int):
        """(Wg, Wu, Wd) decoded to fp64 for routed expert e, or the shared one for e < 0."""
        if e in self._cache:
            return self._cache[e]
        h, f = self.hidden, self.inter
        if e < 0:
            w = (self._rows("sh_gate", 0, f, h), self._rows("sh_up", 0, f, h),
                 self._rows("sh_down", 0, h, f))
        else:
            w = (self._rows("gate", e * f, (e + 1) * f, h), self._rows("up", e * f, (e + 1) * f, h),
                 self._rows("down", e * h, (e + 1) * h, f))
        self._cache[e] = w
        return w


def _moe(bank: ExpertBank, x_bits: np.ndarray, ids: np.ndarray, r: np.ndarray, g: np.ndarray,
         round_h: bool) -> tuple[np.ndarray, np.ndarray]:
    x = bf16_to_f64(x_bits)
    m, top_k = ids.shape
    hid = bank.hidden
    o = np.zeros((m, top_k, hid))
    onorm = np.zeros((m, top_k, hid))
    for e in np.unique(ids):
        wg, wu, wd = bank.expert(int(e))
        tok, slot = np.nonzero(ids == e)
        xe = x[tok]
        h = swiglu(xe @ wg.T, xe @ wu.T)
        if round_h:
            h = bf16_round(h)
        o[tok, slot] = h @ wd.T
        onorm[tok, slot] = np.abs(h) @ np.abs(wd).T
    wg, wu, wd = bank.expert(-1)
    hs = swiglu(x @ wg.T, x @ wu.T)
    if round_h:
        hs = bf16_round(hs)
    s = hs @ wd.T
    snorm = np.abs(hs) @ np.abs(wd).T
    y = np.zeros((m, hid))
    norm = np.zeros((m, hid))
    for j in range(top_k):
        y += r[:, j:j + 1] * o[:, j]
        norm += np.abs(r[:, j:j + 1]) * onorm[:, j]
    y += g[:, None] * s
    norm += np.abs(g)[:, None] * snorm
    return y, norm


def moe_decode(bank: ExpertBank, x_bits: np.ndarray, routing: dict) -> tuple[np.ndarray, np.ndarray]:
    """Decode MoE (h unrounded). Returns (y fp64 [M][hidden], normaliser [M][hidden])."""
    return _moe(bank, x_bits, routing["ids"], routing["r"], routing["g"], round_h=False)


def moe_prefill(bank: ExpertBank, x_bits: np.ndarray, routing: dict) -> tuple[np.ndarray, np.ndarray]:
    """Prefill MoE (h rounded to bf16 before the down projection)."""
    return _moe(bank, x_bits, routing["ids"], routing["r"], routing["g"], round_h=True)


def dispatch(ids: np.ndarray, n_experts: int) -> dict:
    """Counting-sort structure for expert-grouped execution.

    counts[e] = number of (token, slot) pairs routed to e; offsets[e] = sum of counts
    below e (E+1 entries); perm = pair ids p = top_k*t + j ordered by (expert, token).
    A token selects an expert at most once, so the order is unique.
    """
    ids = np.asarray(ids, dtype=np.int64)
    m, top_k = ids.shape
    counts = np.zeros(n_experts, np.int64)
    for e in ids.ravel():
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, np.int64)
    for e in range(n_experts):
        offsets[e + 1] = offsets[e] + counts[e]
    pairs = sorted(range(m * top_k), key=lambda p: (ids[p // top_k, p % top_k], p // top_k))
    return {"counts": counts.astype(np.int32), "offsets": offsets.astype(np.int32),
            "perm": np.asarray(pairs, dtype=np.int32)}
