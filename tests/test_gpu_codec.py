"""GPU encode/decode are bit-exact against the oracle (codes, exponents, decoded values)."""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import oracle
import synth
from oracle import BFP4, BFP8
from gpu_util import dev_f32, host_bits_bf16, note, quantize_on_gpu

pytestmark = pytest.mark.gpu


def _edge_matrix(rng, n, k):
    """Random rows plus blocks that exercise ties, carries, zeros, signed zeros, subnormals."""
    w = (rng.standard_normal((n, k)) * np.exp2(rng.integers(-12, 4, (n, 1)))).astype(np.float32)
    blocks = w.reshape(n, k // 16, 16)
    nb = blocks.shape[1]
    for r in range(n):
        b = rng.integers(0, nb)
        kind = r % 7
        if kind == 0:
            blocks[r, b] = 0.0
        elif kind == 1:
            blocks[r, b] = -0.0
        elif kind == 2:   # subnormals only
            blocks[r, b] = rng.integers(0, 1 << 23, 16).astype(np.uint32).view(np.float32)
        elif kind == 3:   # exact grid ties
            blocks[r, b] = (rng.integers(0, 32, 16) / 2.0 * 2.0 ** -4).astype(np.float32)
            blocks[r, b, 0] = 1.0
        elif kind == 4:   # rounding carry at the top
            blocks[r, b] = np.float32(1.9999) * np.sign(rng.standard_normal(16)).astype(np.float32)
        elif kind == 5:   # huge and tiny mixed
            blocks[r, b] = (rng.standard_normal(16) * np.exp2(rng.integers(-140, 120, 16))).astype(np.float32)
        else:             # shared exponent 248..254 (|w| >= 2^121): a BFP4 block scale 2^(E-129)
            blocks[r, b] = (rng.uniform(-1.9, 1.9, 16) * np.exp2(rng.integers(121, 128))).astype(np.float32)
    return blocks.reshape(n, k)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k", [(1, 16), (7, 48), (33, 1040), (300, 2064)])
def test_quantize_bit_exact(fmt, n, k):
    note(f"quantize fmt={fmt} n={n} k={k}")
    rng = np.random.default_rng(n * 131 + k + fmt)
    w = _edge_matrix(rng, n, k)
    m = quantize_on_gpu(fmt, w)
    exp, code = oracle.encode(w, fmt)
    assert np.array_equal(m.exp.cpu().numpy(), exp.ravel())
    assert np.array_equal(m.code.cpu().numpy(), code.ravel())


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_quantize_row_stride(fmt):
    """Rows ldw = k + 20 values apart (a column slice of a wider matrix): the first k values
    of every row are encoded, the padding is never read into the result."""
    note(f"quantize row stride fmt={fmt}")
    rng = np.random.default_rng(40 + fmt)
    n, k = 37, 1040
    wide = _edge_matrix(rng, n, k + 32)[:, :k + 20]
    t = dev_f32(wide)[:, :k]
    assert t.stride(0) == k + 20
    m = bfq.bfp_quantize(fmt, t)
    exp, code = oracle.encode(np.ascontiguousarray(wide[:, :k]), fmt)
    assert np.array_equal(m.exp.cpu().numpy(), exp.ravel())
    assert np.array_equal(m.code.cpu().numpy(), code.ravel())


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
@pytest.mark.parametrize("n,k", [(5, 32), (257, 1024)])
def test_dequantize_bit_exact(fmt, n, k):
    note(f"dequantize fmt={fmt} n={n} k={k}")
    rng = np.random.default_rng(n + k + fmt)
    w = _edge_matrix(rng, n, k)
    m = quantize_on_gpu(fmt, w)
    want = oracle.decode(*oracle.encode(w, fmt), fmt, n, k)
    got32 = bfq.bfp_dequantize(m, torch.float32).cpu().numpy()
    assert np.array_equal(got32.view(np.uint32), want.astype(np.float32).view(np.uint32))
    got16 = host_bits_bf16(bfq.bfp_dequantize(m, torch.bfloat16))
    want16 = (want.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(got16.reshape(n, k), want16)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_reencode_of_decoded_is_identity(fmt):
    note(f"re-encode fmt={fmt}")
    rng = np.random.default_rng(17)
    w = _edge_matrix(rng, 64, 512)
    m = quantize_on_gpu(fmt, w)
    v = bfq.bfp_dequantize(m, torch.float32)
    m2 = bfq.bfp_quantize(fmt, v)
    assert torch.equal(m2.exp, m.exp) and torch.equal(m2.code, m.code)


def test_quantize_rejects_nonfinite():
    note("quantize non-finite")
    w = np.ones((4, 32), np.float32)
    w[2, 5] = np.inf
    with pytest.raises(bfq.BfpError) as e:
        quantize_on_gpu(BFP4, w)
    assert e.value.status == 4
    w[2, 5] = np.nan
    with pytest.raises(bfq.BfpError):
        quantize_on_gpu(BFP8, w)
    # the flag is cleared between calls
    w[2, 5] = 1.0
    quantize_on_gpu(BFP8, w)


@pytest.mark.parametrize("which", ["gemv2048", "mlp_gate", "lm_head_rows"])
def test_quantize_full_size_workloads(which):
    """Workload-size matrices: the GPU encodes all of it; every byte equals the oracle's (the
    LM head compared in row chunks)."""
    note(f"quantize full-size {which}")
    if which == "gemv2048":
        w, fmt = synth.gemv_case(0)["w"], BFP8
    elif which == "mlp_gate":
        w, fmt = synth.dense_weights(0, 2, "gate", 17408, 5120, 0.02, row_sigma=0.5), BFP4
    else:
        w, fmt = synth.dense_weights(0, 3, "lm", 151936, 2048, 0.02), BFP8
    n, k = w.shape
    m = quantize_on_gpu(fmt, w)
    ge = m.exp.view(n, -1).cpu().numpy()
    gc = m.code.view(n, -1).cpu().numpy()
    for r0 in range(0, n, 16384):
        r1 = min(n, r0 + 16384)
        exp, code = oracle.encode(w[r0:r1], fmt)
        assert np.array_equal(ge[r0:r1], exp) and np.array_equal(gc[r0:r1], code), f"rows {r0}:{r1}"
