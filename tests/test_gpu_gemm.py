"""GPU skinny BFP matmul (bfp_gemm) against the oracle.

Tolerance: every fp32 output within 2e-3 of sum_k |x_k w_k| (computed by the oracle in
fp64). bf16 outputs additionally get half a bf16 ulp of the exact value for their final
rounding. One-hot activations must match bit for bit (one exact product, no sums).
"""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import oracle
import synth
from oracle import BFP4, BFP8
from gpu_util import assert_within, dev_bf16, dev_f32, host_bits_bf16, matrix_from_oracle, note

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _case(fmt, n, k, m, seed, x_dtype="bf16"):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02 * rng.lognormal(0, 0.5, (n, 1))).astype(np.float32)
    exp, code = oracle.encode(w, fmt)
    wd = oracle.decode(exp, code, fmt, n, k)
    if x_dtype == "bf16":
        xb = synth.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
        x64 = oracle.bf16_to_f64(xb)
        xt = dev_bf16(xb)
    else:
        xf = rng.standard_normal((m, k)).astype(np.float32)
        x64 = xf.astype(np.float64)
        xt = dev_f32(xf)
    return matrix_from_oracle(fmt, exp, code, n, k), wd, x64, xt


def _bf16_values(bits):
    return synth.bf16_values(bits).astype(np.float64)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k", [(1, 16), (37, 48), (129, 1040), (300, 2064), (70, 512)])
@pytest.mark.parametrize("m", [1, 3, 8, 13, 32])
def test_gemm_small_shapes(fmt, n, k, m):
    note(f"gemm fmt={fmt} n={n} k={k} m={m}")
    wm, wd, x64, xt = _case(fmt, n, k, m, seed=n * 7 + k + m + fmt)
    y = bfq.bfp_gemm(wm, xt).cpu().numpy()
    assert_within(y, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="gemm")


# one activation row with K a multiple of 1024 runs the wave-per-row kernel: slices of 1..5
# steps (bf16 x) or 1..2 (fp32 x), one workgroup per compute unit, ragged row shares; K = 36864
# stages a 144 KB fp32 row (72 KB bf16) in LDS, near the 160 KB the kernel may take
@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k", [(1, 1024), (7, 2048), (300, 3072), (257, 4096), (2049, 5120), (96, 6144),
                                 (5000, 2048), (40, 17408), (64, 36864)])
@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_gemm_one_row_shapes(fmt, n, k, x_dtype):
    note(f"gemm m=1 fmt={fmt} n={n} k={k} x={x_dtype}")
    wm, wd, x64, xt = _case(fmt, n, k, 1, seed=n + k + fmt, x_dtype=x_dtype)
    y = bfq.bfp_gemm(wm, xt).cpu().numpy()
    assert_within(y, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="gemm m=1")
    yb = bfq.bfp_gemm(wm, xt, out_dtype=torch.bfloat16)
    ref = oracle.gemm(x64, wd)
    assert_within(_bf16_values(host_bits_bf16(yb)), ref, oracle.normaliser(x64, wd), TOL,
                  extra=2.0 ** -8 * np.abs(ref), what="gemm m=1 bf16 out")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k", [(5, 1024), (333, 5120), (1200, 3072)])
def test_gemm_one_row_swiglu(fmt, n, k):
    note(f"gemm m=1 swiglu fmt={fmt} n={n} k={k}")
    wg, gd, x64, xt = _case(fmt, n, k, 1, seed=n + 3 * k + fmt)
    rng = np.random.default_rng(n + 1)
    wu = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    eu, cu = oracle.encode(wu, fmt)
    ud = oracle.decode(eu, cu, fmt, n, k)
    h = bfq.bfp_gemm(wg, xt, w_up=matrix_from_oracle(fmt, eu, cu, n, k)).cpu().numpy()
    g, u = oracle.gemm(x64, gd), oracle.gemm(x64, ud)
    ref = oracle.swiglu(g, u)
    norm = 1.1 * oracle.normaliser(x64, gd) * np.abs(u) + np.abs(oracle.silu(g)) * oracle.normaliser(x64, ud)
    assert_within(h, ref, norm, TOL, extra=1e-6 * np.abs(ref), what="swiglu m=1")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_gemm_one_row_one_hot_bit_exact(fmt):
    """A one-hot row through the wave-per-row kernel: one exact product per output."""
    note(f"gemm m=1 one-hot fmt={fmt}")
    n, k = 777, 5120
    wm, wd, _, _ = _case(fmt, n, k, 1, seed=9 + fmt)
    for col, val in ((4099, -1.375), (0, 3.0e-3), (5119, 7.5)):
        xb = np.zeros((1, k), np.uint16)
        xb[0, col] = synth.bf16_bits(np.array([val], np.float32))[0]
        y = bfq.bfp_gemm(wm, dev_bf16(xb)).cpu().numpy()
        want = (oracle.bf16_to_f64(xb) @ wd.T).astype(np.float32)
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), f"column {col}"


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("m", [1, 5, 16])
def test_gemm_fp32_x_and_bf16_y(fmt, m):
    note(f"gemm fp32-x bf16-y fmt={fmt} m={m}")
    wm, wd, x64, xt = _case(fmt, 203, 3088, m, seed=m + 100 * fmt, x_dtype="f32")
    y = bfq.bfp_gemm(wm, xt, out_dtype=torch.bfloat16)
    yv = _bf16_values(host_bits_bf16(y))
    ref = oracle.gemm(x64, wd)
    assert_within(yv, ref, oracle.normaliser(x64, wd), TOL, extra=2.0 ** -8 * np.abs(ref), what="gemm bf16 out")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("m", [1, 4, 32])
def test_gemm_swiglu(fmt, m):
    note(f"gemm swiglu fmt={fmt} m={m}")
    n, k = 333, 2080
    wg, gd, x64, xt = _case(fmt, n, k, m, seed=m + 11 * fmt)
    rng = np.random.default_rng(m + 5)
    wu = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    eu, cu = oracle.encode(wu, fmt)
    ud = oracle.decode(eu, cu, fmt, n, k)
    um = matrix_from_oracle(fmt, eu, cu, n, k)
    h = bfq.bfp_gemm(wg, xt, w_up=um).cpu().numpy()
    g, u = oracle.gemm(x64, gd), oracle.gemm(x64, ud)
    ref = oracle.swiglu(g, u)
    # the tolerance carries through silu: |dh| <= |silu'(g)| |dg| |u| + |silu(g)| |du|
    ng, nu = oracle.normaliser(x64, gd), oracle.normaliser(x64, ud)
    norm = 1.1 * ng * np.abs(u) + np.abs(oracle.silu(g)) * nu   # |silu'| < 1.1 everywhere
    assert_within(h, ref, norm, TOL, extra=1e-6 * np.abs(ref), what="swiglu")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_gemm_one_hot_bit_exact(fmt):
    note(f"gemm one-hot fmt={fmt}")
    n, k = 200, 1056
    wm, wd, _, _ = _case(fmt, n, k, 1, seed=3 + fmt)
    xb = np.zeros((2, k), np.uint16)
    xb[0, 777] = synth.bf16_bits(np.array([-1.375], np.float32))[0]
    xb[1, 5] = synth.bf16_bits(np.array([3.0e-3], np.float32))[0]
    y = bfq.bfp_gemm(wm, dev_bf16(xb)).cpu().numpy()
    want = (oracle.bf16_to_f64(xb) @ wd.T).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))


def test_gemm_rows_are_independent_of_m():
    """Row i of an m-row call (2 <= m <= 32, the matrix-core kernel) does not depend on m or on
    the other rows: same reduction order for every m. A one-row call runs the vector kernel
    and agrees within the tolerance."""
    note("gemm batch invariance")
    wm, wd, x64, xt = _case(BFP4, 150, 4096, 8, seed=77)
    y8 = bfq.bfp_gemm(wm, xt).cpu().numpy()
    for i in range(0, 8, 2):
        y2 = bfq.bfp_gemm(wm, xt[i:i + 2].contiguous()).cpu().numpy()
        assert np.array_equal(y8[i:i + 2].view(np.uint32), y2.view(np.uint32))
    y1 = bfq.bfp_gemm(wm, xt[3:4].contiguous()).cpu().numpy()
    assert_within(y1, oracle.gemm(x64[3:4], wd), oracle.normaliser(x64[3:4], wd), TOL, what="gemm m=1")


@pytest.mark.parametrize("x_dtype", ["bf16", "f32"])
def test_gemm_rows_independent_of_m_long_k(x_dtype):
    """Same property on a long-K shape whose K is cut into slices, for m up to 32 (two row
    tiles) and for fp32 activations (hi + lo planes)."""
    note(f"gemm batch invariance long K {x_dtype}")
    wm, wd, x64, xt = _case(BFP4, 96, 17408, 32, seed=91, x_dtype=x_dtype)
    y32 = bfq.bfp_gemm(wm, xt).cpu().numpy()
    y7 = bfq.bfp_gemm(wm, xt[5:12].contiguous()).cpu().numpy()
    y2 = bfq.bfp_gemm(wm, xt[20:22].contiguous()).cpu().numpy()
    assert np.array_equal(y32[5:12].view(np.uint32), y7.view(np.uint32))
    assert np.array_equal(y32[20:22].view(np.uint32), y2.view(np.uint32))
    assert_within(y32, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="gemm long K")


def _sampled_rows_from_device(wm, idx):
    """The oracle's fp64 values of weight rows idx of a device BfpMatrix (read back, decoded)."""
    nb = wm.k // 16
    cpr = wm.code.numel() // wm.n
    e = wm.exp.view(wm.n, nb)[idx].cpu().numpy()
    c = wm.code.view(wm.n, cpr)[idx].cpu().numpy()
    return oracle.decode(e, c, wm.fmt, len(idx), wm.k)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("steps", [3, 9, 13])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("m", [8, 32])
def test_gemm_long_slices(fmt, steps, swiglu, m):
    """25,600 weight rows, so that K is cut into few, long slices: with 3 / 9 / 13 steps of K
    the slices hold 3 / 5 + 4 / 7 + 6 steps, around the lengths at which the matrix-core kernel
    switches between its steady loop (every load unconditional) and its guarded form, for one
    and two matrices and one and two row tiles. Weights quantized on the device (bit-exact with
    the oracle's encoding, tested elsewhere); 160 sampled output columns (the first and last
    rows of the matrix among them) against the oracle on the read-back blocks."""
    n = 25600
    sk = 128 if fmt == BFP8 else 256
    k = steps * sk
    note(f"gemm long slices fmt={fmt} k={k} swiglu={swiglu} m={m}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1000 * steps + 10 * fmt + m + int(swiglu))
    wm = bfq.bfp_quantize(fmt, torch.randn((n, k), generator=gen, device="cuda") * 0.02)
    um = bfq.bfp_quantize(fmt, torch.randn((n, k), generator=gen, device="cuda") * 0.02) if swiglu else None
    rng = np.random.default_rng(steps + m)
    xb = synth.bf16_bits(rng.standard_normal((m, k)).astype(np.float32))
    x64 = oracle.bf16_to_f64(xb)
    y = bfq.bfp_gemm(wm, dev_bf16(xb), w_up=um).cpu().numpy()
    idx = np.unique(np.concatenate([[0, 127, 128, n - 1], rng.choice(n, 156, replace=False)]))
    wd = _sampled_rows_from_device(wm, idx)
    if swiglu:
        ud = _sampled_rows_from_device(um, idx)
        g, u = oracle.gemm(x64, wd), oracle.gemm(x64, ud)
        ref = oracle.swiglu(g, u)
        norm = 1.1 * oracle.normaliser(x64, wd) * np.abs(u) + np.abs(oracle.silu(g)) * oracle.normaliser(x64, ud)
        assert_within(y[:, idx], ref, norm, TOL, extra=1e-6 * np.abs(ref), what="long slices swiglu")
    else:
        assert_within(y[:, idx], oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="long slices")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k,x_dtype,swiglu", [(300, 2064, "bf16", False), (96, 17408, "bf16", True),
                                                 (200, 1040, "f32", False), (5000, 2048, "bf16", False)])
def test_gemm_batch_invariant_flag(fmt, n, k, x_dtype, swiglu):
    """With BFP_GEMM_BATCH_INVARIANT, row i of an m-row call is the same bits for every m in
    1..32, the one-row call included (short and sliced K, SwiGLU, fp32 x, one and two row
    tiles), and within the tolerance of the oracle."""
    note(f"gemm batch-invariant flag fmt={fmt} n={n} k={k} x={x_dtype} swiglu={swiglu}")
    wm, wd, x64, xt = _case(fmt, n, k, 32, seed=n + k + fmt, x_dtype=x_dtype)
    um = ud = None
    if swiglu:
        wu = (np.random.default_rng(n).standard_normal((n, k)) * 0.02).astype(np.float32)
        eu, cu = oracle.encode(wu, fmt)
        ud = oracle.decode(eu, cu, fmt, n, k)
        um = matrix_from_oracle(fmt, eu, cu, n, k)
    y32 = bfq.bfp_gemm(wm, xt, w_up=um, batch_invariant=True).cpu().numpy()
    for a, b in [(0, 1), (7, 8), (31, 32), (3, 5), (10, 26), (16, 32), (0, 17)]:
        y = bfq.bfp_gemm(wm, xt[a:b].contiguous(), w_up=um, batch_invariant=True).cpu().numpy()
        assert np.array_equal(y.view(np.uint32), y32[a:b].view(np.uint32)), f"rows {a}:{b} differ from the 32-row call"
    if swiglu:
        g, u = oracle.gemm(x64, wd), oracle.gemm(x64, ud)
        ref = oracle.swiglu(g, u)
        norm = 1.1 * oracle.normaliser(x64, wd) * np.abs(u) + np.abs(oracle.silu(g)) * oracle.normaliser(x64, ud)
        assert_within(y32, ref, norm, TOL, extra=1e-6 * np.abs(ref), what="invariant swiglu")
    else:
        assert_within(y32, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="invariant gemm")


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("wscale,xscale", [(2.0 ** -128, 2.0 ** 60), (2.0 ** -124, 2.0 ** 50),
                                           (2.0 ** 121, 2.0 ** -100), (2.0 ** 125, 2.0 ** -110)])
@pytest.mark.parametrize("m", [1, 3])
def test_gemm_extreme_exponents(fmt, wscale, xscale, m):
    """Shared exponents far from 1 (fp32 subnormal weights, E < 8, E up to 254) mixed with
    all-zero blocks, on the vector kernel (m = 1) and the matrix cores (m = 3): the unpack and
    the block scale must stay exact over the whole exponent range (a BFP4 multiplier 2^(E-120)
    held as a float overflows for E >= 248). x is scaled so that the products stay normal fp32
    numbers."""
    note(f"gemm extreme exponents fmt={fmt} w={wscale:.3g} x={xscale:.3g} m={m}")
    n, k = 80, 1024
    rng = np.random.default_rng(17 + fmt)
    w = rng.standard_normal((n, k)) * wscale
    w[np.repeat(rng.random((n, k // 16)) < 0.25, 16, axis=1)] = 0.0
    w = w.astype(np.float32)
    exp, code = oracle.encode(w, fmt)
    wd = oracle.decode(exp, code, fmt, n, k)
    assert np.count_nonzero(wd) > n * k // 2
    if wscale > 2.0 ** 124:
        assert exp.max() >= 250
    xb = synth.bf16_bits((rng.standard_normal((m, k)) * xscale).astype(np.float32))
    x64 = oracle.bf16_to_f64(xb)
    y = bfq.bfp_gemm(matrix_from_oracle(fmt, exp, code, n, k), dev_bf16(xb)).cpu().numpy()
    assert_within(y, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="gemm extreme exponents")


def test_gemm_deterministic():
    note("gemm determinism")
    wm, wd, x64, xt = _case(BFP8, 999, 2048, 16, seed=5)
    a = bfq.bfp_gemm(wm, xt)
    b = bfq.bfp_gemm(wm, xt)
    assert torch.equal(a, b)


# ---- workload sizes ------------------------------------------------------------------------

def _sampled_rows(n, count, seed):
    return np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).integers(0, n, count)]))


def test_workload_single_bfp8_gemv():
    """2048 x 2048 BFP8, x 1 x 2048, all outputs."""
    note("workload: single BFP8 GEMV 2048x2048")
    c = synth.gemv_case(0)
    w = c["w"]
    m = bfq.bfp_quantize(BFP8, dev_f32(w))
    exp, code = oracle.encode(w, BFP8)
    wd = oracle.decode(exp, code, BFP8, *w.shape)
    x64 = oracle.bf16_to_f64(c["x"])
    y = bfq.bfp_gemm(m, dev_bf16(c["x"])).cpu().numpy()
    assert_within(y, oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL, what="gemv2048")


@pytest.fixture(scope="module")
def mlp_oracle():
    """The 27B-class MLP's weights encoded by the oracle, their exact decodes and magnitudes
    (fp64), and device copies of the oracle's bytes (the GPU streams exactly what the oracle
    decodes)."""
    note("building the dense MLP oracle (17408 x 5120 BFP4, three matrices)")
    c = synth.mlp_case(1, 0)
    out = {}
    for name, (n, k) in (("wg", (17408, 5120)), ("wu", (17408, 5120)), ("wd", (5120, 17408))):
        e, cc = oracle.encode(c[name], BFP4)
        wd = oracle.decode(e, cc, BFP4, n, k)
        out[name] = (matrix_from_oracle(BFP4, e, cc, n, k), wd, np.abs(wd))
    return out


@pytest.mark.parametrize("M", [1, 8, 16, 32])
def test_workload_dense_mlp(mlp_oracle, M):
    """27B-class BFP4 MLP, every output: gate/up 5120->17408 with SwiGLU (all 17,408 h per
    row), down 17408->5120 in bf16 (all 5,120 y per row) against the oracle's own chain
    x -> h -> y. The y tolerance runs through h: the down projection's own 2e-3 of
    sum_k |h_k Wd_k| plus the allowed h error carried through |Wd| (sum_k norm_h,k |Wd_k|),
    plus half a bf16 ulp for the output rounding."""
    note(f"workload: dense BFP4 MLP M={M}")
    (gm, gd, ga), (um, ud, ua), (dm, dd, da) = mlp_oracle["wg"], mlp_oracle["wu"], mlp_oracle["wd"]
    xb = synth.mlp_case(M, 0)["x"]
    x = dev_bf16(xb)
    h = bfq.bfp_gemm(gm, x, w_up=um)
    y = bfq.bfp_gemm(dm, h, out_dtype=torch.bfloat16)
    h_np = h.cpu().numpy()
    y_np = _bf16_values(host_bits_bf16(y))
    x64 = oracle.bf16_to_f64(xb)
    gg, uu = oracle.gemm(x64, gd), oracle.gemm(x64, ud)
    h_ref = oracle.swiglu(gg, uu)
    ax = np.abs(x64)
    norm_h = 1.1 * (ax @ ga.T) * np.abs(uu) + np.abs(oracle.silu(gg)) * (ax @ ua.T)
    assert_within(h_np, h_ref, norm_h, TOL, extra=1e-6 * np.abs(h_ref), what="mlp h (all 17408)")
    y_ref = oracle.gemm(h_ref, dd)
    norm_y = (np.abs(h_ref) + norm_h + 1e-6 * np.abs(h_ref)) @ da.T
    assert_within(y_np, y_ref, norm_y, TOL, extra=2.0 ** -8 * np.abs(y_ref), what="mlp y (all 5120)")


def _lm_chunks(w, fmt, rows=16384):
    """The LM head encoded by the oracle chunk by chunk (bounded host memory)."""
    for r0 in range(0, w.shape[0], rows):
        r1 = min(w.shape[0], r0 + rows)
        e, c = oracle.encode(w[r0:r1], fmt)
        yield r0, r1, e, c


@pytest.mark.parametrize("M", [1, 16])
def test_workload_bfp8_projections_and_lm_head(M):
    """Fused QKV 2048->5120, O 4096->2048 and the LM head 2048->151,936, every fp32 output
    against the oracle (the LM head's 151,936 rows encoded and decoded by the oracle in
    chunks; the GPU streams the oracle's bytes)."""
    note(f"workload: BFP8 projections + LM head M={M}")
    c = synth.proj_case(M, 0)
    x64 = oracle.bf16_to_f64(c["x"])
    xo64 = oracle.bf16_to_f64(c["xo"])
    for name, xx, x_bits in (("wqkv", x64, c["x"]), ("wo", xo64, c["xo"])):
        w = c[name]
        n, k = w.shape
        e, cc = oracle.encode(w, BFP8)
        wd = oracle.decode(e, cc, BFP8, n, k)
        y = bfq.bfp_gemm(matrix_from_oracle(BFP8, e, cc, n, k), dev_bf16(x_bits)).cpu().numpy()
        assert_within(y, oracle.gemm(xx, wd), oracle.normaliser(xx, wd), TOL, what=name)
    w = c["wlm"]
    n, k = w.shape
    exp = np.empty((n, k // 16), np.uint8)
    code = np.empty((n, k), np.uint8)
    for r0, r1, e, cc in _lm_chunks(w, BFP8):
        exp[r0:r1], code[r0:r1] = e, cc
    y = bfq.bfp_gemm(matrix_from_oracle(BFP8, exp, code, n, k), dev_bf16(c["x"])).cpu().numpy()
    worst = 0.0
    for r0 in range(0, n, 16384):
        r1 = min(n, r0 + 16384)
        wd = oracle.decode(exp[r0:r1], code[r0:r1], BFP8, r1 - r0, k)
        worst = max(worst, assert_within(y[:, r0:r1], oracle.gemm(x64, wd), oracle.normaliser(x64, wd), TOL,
                                         what=f"lm head rows {r0}:{r1}"))
    note(f"lm head M={M}: all {n} logits per row within tolerance (largest relative error {worst:.2e})")
