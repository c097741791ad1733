"""GPU greedy pick over a skinny matmul's outputs (bfp_gemm_argmax) against bfp_gemm and the
oracle.

Bit for bit: the pick equals the first maximum of the fp32 outputs bfp_gemm writes for the
same call (same kernels, same sums), and the value equals that output (-0 reported as +0, a
NaN as the quiet NaN 0x7fc00000).
Against the oracle's fp64 outputs y (normaliser s = sum_k |x_k w_k|, parity tolerance
2e-3 s per output): the picked column must be a maximum within the tolerance,
y[idx] >= y[j] - 2e-3 (s[idx] + s[j]) for every column j checked, and equal to the oracle's
own pick where the oracle's top two are further apart than that; the value must be within
2e-3 s[idx] of y[idx].
"""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import oracle
import synth
from oracle import BFP4, BFP8
from gpu_util import dev_bf16, dev_f32, matrix_from_oracle, note

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _first_max(y32: np.ndarray):
    """Pick of the rule above over fp32 rows (numpy's argmax: first maximum, first NaN)."""
    idx = np.argmax(y32, axis=1)
    val = y32[np.arange(y32.shape[0]), idx] + np.float32(0.0)        # -0 -> +0
    val[np.isnan(val)] = np.uint32(0x7FC00000).view(np.float32)     # NaN -> the quiet NaN
    return idx, val


def _bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


def _check_vs_gemm(wm, xt, what):
    idx, val = bfq.bfp_gemm_argmax(wm, xt)
    y = bfq.bfp_gemm(wm, xt).cpu().numpy()
    ref_idx, ref_val = _first_max(y)
    got_idx, got_val = idx.cpu().numpy(), val.cpu().numpy()
    assert np.array_equal(got_idx, ref_idx), f"{what}: pick {got_idx} != first max of bfp_gemm {ref_idx}"
    assert np.array_equal(_bits(got_val), _bits(ref_val)), f"{what}: value {got_val} != {ref_val}"
    return got_idx, got_val, y


def _check_vs_oracle(got_idx, got_val, y_or, norm, cols=None, what=""):
    """y_or, norm: oracle outputs and normalisers [M][C] for columns `cols` (all if None)."""
    m = y_or.shape[0]
    cols = np.arange(y_or.shape[1]) if cols is None else np.asarray(cols)
    pos = {int(c): i for i, c in enumerate(cols)}
    o_idx, _ = oracle.greedy_pick(y_or)
    for i in range(m):
        p = pos[int(got_idx[i])]
        slack = TOL * (norm[i, p] + norm[i])
        assert np.all(y_or[i, p] >= y_or[i] - slack), f"{what} row {i}: column {got_idx[i]} is not a maximum"
        assert abs(float(got_val[i]) - y_or[i, p]) <= TOL * norm[i, p], f"{what} row {i}: value"
        # the oracle's pick is clear of every other column by more than both tolerances
        o = int(o_idx[i])
        others = np.delete(y_or[i] + TOL * norm[i], o)
        if others.size == 0 or y_or[i, o] - TOL * norm[i, o] > others.max():
            assert cols[o] == got_idx[i], f"{what} row {i}: clear maximum at {cols[o]}, got {got_idx[i]}"


def _case(fmt, n, k, m, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02 * rng.lognormal(0, 0.5, (n, 1))).astype(np.float32)
    exp, code = oracle.encode(w, fmt)
    wd = oracle.decode(exp, code, fmt, n, k)
    xb = synth.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    return matrix_from_oracle(fmt, exp, code, n, k), wd, oracle.bf16_to_f64(xb), dev_bf16(xb)


# (n, k): ragged N and K; K up to one step (one K slice on the matrix cores) and longer K
# (sliced on the matrix cores for these N)
@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k", [(1, 16), (37, 48), (777, 112), (1000, 2048), (3001, 1040), (9, 1024), (2500, 5120)])
@pytest.mark.parametrize("m", [1, 2, 5, 16, 32])
def test_argmax_small_shapes(fmt, n, k, m):
    note(f"argmax fmt={fmt} n={n} k={k} m={m}")
    wm, wd, x64, xt = _case(fmt, n, k, m, seed=3 * n + k + m + fmt)
    got_idx, got_val, _ = _check_vs_gemm(wm, xt, "small")
    _check_vs_oracle(got_idx, got_val, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), what="small")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("k", [128, 2048])
@pytest.mark.parametrize("m", [1, 3])
def test_argmax_ties_pick_first_column(fmt, k, m):
    """Equal largest outputs in one workgroup (columns 10, 11) and in others (500, 999): the
    first column wins."""
    note(f"argmax ties fmt={fmt} k={k} m={m}")
    n = 1000
    rng = np.random.default_rng(k + m)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    for r in (999, 500, 11, 10):
        w[r] = 0.05
    exp, code = oracle.encode(w, fmt)
    wd = oracle.decode(exp, code, fmt, n, k)
    xb = synth.bf16_bits(np.abs(rng.standard_normal((m, k))).astype(np.float32))
    x64 = oracle.bf16_to_f64(xb)
    wm = matrix_from_oracle(fmt, exp, code, n, k)
    got_idx, got_val, _ = _check_vs_gemm(wm, dev_bf16(xb), "ties")
    assert got_idx.tolist() == [10] * m
    o_idx, o_val = oracle.greedy_pick(oracle.gemm(x64, wd))
    assert o_idx.tolist() == [10] * m
    assert np.all(np.abs(got_val - o_val) <= TOL * oracle.normaliser(x64, wd)[:, 10])


@pytest.mark.parametrize("k", [112, 1040])
@pytest.mark.parametrize("m", [1, 4])
def test_argmax_nan_and_zero_rows(k, m):
    """A row of x holding a NaN makes every output of that row NaN: column 0 is picked, value
    NaN. A zero row gives all-zero outputs (some -0): column 0, value +0. Other rows are
    unaffected."""
    note(f"argmax nan/zero rows k={k} m={m}")
    n = 700
    wm, wd, x64, _ = _case(BFP8, n, k, m, seed=77 + m)
    xb = synth.bf16_bits(np.random.default_rng(m).standard_normal((m, k)).astype(np.float32))
    xb[0, 5] = 0x7FC0                       # bf16 quiet NaN
    if m > 1:
        xb[2] = 0
    got_idx, got_val, _ = _check_vs_gemm(wm, dev_bf16(xb), "nan")
    assert got_idx[0] == 0 and np.isnan(got_val[0])
    if m > 1:
        assert got_idx[2] == 0 and _bits(got_val[2]) == 0
        x64 = oracle.bf16_to_f64(xb)
        rest = [1, 3]
        y_or = oracle.gemm(x64[rest], wd)
        _check_vs_oracle(got_idx[rest], got_val[rest], y_or, oracle.normaliser(x64[rest], wd), what="nan rest")


def test_argmax_deterministic():
    note("argmax deterministic")
    wm, _, _, xt = _case(BFP4, 5000, 2048, 16, seed=5)
    a = [bfq.bfp_gemm_argmax(wm, xt) for _ in range(3)]
    for i, v in a[1:]:
        assert torch.equal(i, a[0][0]) and torch.equal(v.view(torch.int32), a[0][1].view(torch.int32))


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_argmax_batch_invariant_flag(fmt):
    """With BFP_GEMM_BATCH_INVARIANT the pick and value of row i are the same for every m,
    one-row calls included, and equal the first maximum of bfp_gemm's flagged outputs."""
    note(f"argmax batch-invariant fmt={fmt}")
    wm, wd, x64, xt = _case(fmt, 5000, 2048, 32, seed=40 + fmt)
    i32, v32 = (t.cpu().numpy() for t in bfq.bfp_gemm_argmax(wm, xt, batch_invariant=True))
    y = bfq.bfp_gemm(wm, xt, batch_invariant=True).cpu().numpy()
    ref_idx, ref_val = _first_max(y)
    assert np.array_equal(i32, ref_idx) and np.array_equal(_bits(v32), _bits(ref_val))
    for a, b in [(0, 1), (9, 10), (31, 32), (4, 20)]:
        i, v = (t.cpu().numpy() for t in bfq.bfp_gemm_argmax(wm, xt[a:b].contiguous(), batch_invariant=True))
        assert np.array_equal(i, i32[a:b]) and np.array_equal(_bits(v), _bits(v32[a:b])), f"rows {a}:{b}"
    _check_vs_oracle(i32, v32, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), what="invariant")


def _sampled(n, count, seed):
    return np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).integers(0, n, count)]))


@pytest.mark.parametrize("M", [1, 16])
def test_workload_lm_head_argmax(M):
    """LM head 2048 -> 151,936 BFP8 at its full size (one K slice on the matrix cores), the
    matrix encoded by the oracle (in chunks) and streamed by the GPU from those bytes: bit for
    bit against bfp_gemm's first maximum; against the oracle over every column of every row."""
    note(f"workload: LM head argmax M={M}")
    c = synth.proj_case(M, 0)
    w = c["wlm"]
    n, k = w.shape
    exp = np.empty((n, k // 16), np.uint8)
    code = np.empty((n, k), np.uint8)
    for r0 in range(0, n, 16384):
        r1 = min(n, r0 + 16384)
        exp[r0:r1], code[r0:r1] = oracle.encode(w[r0:r1], BFP8)
    wm = matrix_from_oracle(BFP8, exp, code, n, k)
    got_idx, got_val, _ = _check_vs_gemm(wm, dev_bf16(c["x"]), "lm head")
    x64 = oracle.bf16_to_f64(c["x"])
    y_or = np.empty((M, n))
    norm = np.empty((M, n))
    for r0 in range(0, n, 16384):
        r1 = min(n, r0 + 16384)
        wd = oracle.decode(exp[r0:r1], code[r0:r1], BFP8, r1 - r0, k)
        y_or[:, r0:r1] = oracle.gemm(x64, wd)
        norm[:, r0:r1] = oracle.normaliser(x64, wd)
    _check_vs_oracle(got_idx, got_val, y_or, norm, what="lm head (all columns)")
