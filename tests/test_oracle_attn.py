"""Pins for the oracle's KV-cache encoding and decode attention (CPU only)."""
import math
from fractions import Fraction

import numpy as np

import oracle
from oracle import BFP8


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_kv_encode_is_the_weight_encoding_per_row():
    # the cache layout is [kv_head][token][...]: row (h, t) is token t of head h
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 2, 32)).astype(np.float32)
    exp, code = oracle.kv_encode(x)
    assert exp.shape == (2, 5, 2) and code.shape == (2, 5, 32)
    for h in range(2):
        for t in range(5):
            e1, c1 = oracle.encode(x[t, h][None, :], BFP8)
            assert np.array_equal(exp[h, t], e1[0]) and np.array_equal(code[h, t], c1[0])
    back = oracle.kv_decode(exp, code, BFP8, 32)
    assert back.shape == (2, 5, 32)
    # decoded entries are within half a step of the inputs (steps are 2^(E-133) for BFP8)
    assert np.all(np.abs(back.transpose(1, 0, 2) - x) <= np.abs(x).max() * 2.0 ** -7)


def test_attention_one_token_returns_its_value():
    rng = np.random.default_rng(1)
    q, k, v = _rand(rng, 4, 16), _rand(rng, 2, 1, 16), _rand(rng, 2, 1, 16)
    out, norm = oracle.decode_attention(q, k, v, 0.25)
    assert np.array_equal(out, v[np.arange(4) // 2, 0])
    assert np.array_equal(norm, np.abs(v[np.arange(4) // 2, 0]))


def test_attention_equal_scores_average_the_values():
    rng = np.random.default_rng(2)
    k, v = _rand(rng, 1, 6, 8), _rand(rng, 1, 6, 8)
    out, _ = oracle.decode_attention(np.zeros((3, 8)), k, v, 1.0)
    assert np.allclose(out, v[0].mean(axis=0), rtol=0, atol=1e-15)


def test_attention_two_tokens_closed_form():
    # p_0 = 1 / (1 + e^(s1 - s0)) with s = scale q.k
    q = np.array([[1.0, 2.0]])
    k = np.array([[[0.5, 0.25], [-1.0, 0.5]]])
    v = np.array([[[3.0, -1.0], [1.0, 5.0]]])
    s0, s1 = 0.7 * (0.5 + 0.5), 0.7 * (-1.0 + 1.0)
    p0 = 1.0 / (1.0 + math.exp(s1 - s0))
    out, _ = oracle.decode_attention(q, k, v, 0.7)
    assert np.allclose(out[0], p0 * v[0, 0] + (1 - p0) * v[0, 1], rtol=1e-15, atol=0)


def test_attention_groups_queries_onto_kv_heads():
    # KV head g holds constant values g + 1: query head h must return h // group + 1
    rng = np.random.default_rng(3)
    hkv, group, L, d = 3, 4, 5, 8
    k = _rand(rng, hkv, L, d)
    v = np.broadcast_to((np.arange(hkv) + 1.0)[:, None, None], (hkv, L, d))
    out, _ = oracle.decode_attention(_rand(rng, hkv * group, d), k, v, 0.3)
    assert np.allclose(out, (np.arange(hkv * group) // group + 1.0)[:, None], rtol=1e-14, atol=0)


def test_attention_token_order_does_not_matter_and_scale_folds_into_q():
    rng = np.random.default_rng(4)
    q, k, v = _rand(rng, 2, 16), _rand(rng, 1, 9, 16), _rand(rng, 1, 9, 16)
    perm = rng.permutation(9)
    a, _ = oracle.decode_attention(q, k, v, 0.2)
    b, _ = oracle.decode_attention(q, k[:, perm], v[:, perm], 0.2)
    c, _ = oracle.decode_attention(0.2 * q, k, v, 1.0)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15) and np.allclose(a, c, rtol=1e-13, atol=1e-15)


def test_attention_large_scores_do_not_overflow_and_pick_the_maximum():
    # one score far above the rest: the output is that token's value (softmax is shift-free)
    q = np.array([[100.0, 0.0]])
    k = np.array([[[10.0, 0.0], [9.0, 0.0], [-10.0, 0.0]]])
    v = np.array([[[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]]])
    out, _ = oracle.decode_attention(q, k, v, 1.0)
    assert np.all(np.isfinite(out)) and np.allclose(out[0], [1.0, 2.0], rtol=0, atol=1e-40)


def _sylvester(d):
    h = np.array([[1.0]])
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def test_hadamard_rotate_matches_the_matrix_and_is_its_own_inverse():
    rng = np.random.default_rng(7)
    for d in (64, 128, 256):
        # small integers: every sum is exact, so the fast transform equals the matrix product
        x = rng.integers(-50, 51, size=(3, d)).astype(np.float64)
        want = x @ _sylvester(d).T * oracle.attn.INV_SQRT[d]
        assert np.array_equal(oracle.hadamard_rotate(x), want)
        y = rng.standard_normal((4, d))
        r = oracle.hadamard_rotate(y)
        assert np.allclose(np.linalg.norm(r, axis=1), np.linalg.norm(y, axis=1), rtol=1e-14)
        assert np.allclose(oracle.hadamard_rotate(r), y, rtol=0, atol=1e-13)
    # a one-hot input gives a constant-magnitude column of H: the rotation spreads an outlier
    e = np.zeros((1, 256)); e[0, 37] = 1.0
    assert np.allclose(np.abs(oracle.hadamard_rotate(e)), 1.0 / 16)
    # each constant is the double nearest 1/sqrt(d): of it and its two neighbours, its square
    # times d is closest to 1 (exact rational arithmetic)
    for d, c in oracle.attn.INV_SQRT.items():
        err = [abs(Fraction(v) ** 2 * d - 1) for v in (math.nextafter(c, 0), c, math.nextafter(c, 1))]
        assert err[1] < err[0] and err[1] < err[2], d


def test_rotated_v_rows_are_bfp4_of_the_rounded_rotation():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 2, 128)).astype(np.float32)
    exp, code = oracle.kv_encode_rotated(x)
    assert exp.shape == (2, 3, 8) and code.shape == (2, 3, 64)
    r = oracle.hadamard_rotate(x).astype(np.float32)
    e2, c2 = oracle.kv_encode(r, oracle.BFP4)
    assert np.array_equal(exp, e2) and np.array_equal(code, c2)
    # attention is linear in v: attention over the rotated values, rotated back, is attention
    # over the values the rotated cache stands for
    q = rng.standard_normal((4, 128))
    k = oracle.kv_decode(*oracle.kv_encode(x), BFP8, 128)
    vr = oracle.kv_decode(exp, code, oracle.BFP4, 128)
    out_r, _ = oracle.decode_attention(q, k, vr, 0.1)
    out, _ = oracle.decode_attention(q, k, oracle.hadamard_rotate(vr), 0.1)
    assert np.allclose(oracle.hadamard_rotate(out_r), out, rtol=0, atol=1e-12)



def test_rotated_cache_bytes_per_token_match_the_card():
    """The 27B card ("Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ)", changes in s27-20261005,
    DFlash2 at 262K) gives 26,624 bytes per token for the BFP8-K / 4-bit-V cache against 34,816
    for the BFP8 KV cache. Both follow from the 16-value block layout with one exponent byte per
    block, for a model whose cached head dimensions add up to 16,384 per token: BFP8 rows cost
    17/16 bytes per value, BFP4 rows 9/16."""
    rng = np.random.default_rng(10)
    x = rng.standard_normal((1, 64, 256)).astype(np.float32)          # one token, 64 x 256 = 16,384
    ek, ck = oracle.kv_encode(x)
    ev, cv = oracle.kv_encode_rotated(x)
    assert ek.nbytes + ck.nbytes + ev.nbytes + cv.nbytes == 26624
    ev8, cv8 = oracle.kv_encode(x)
    assert ek.nbytes + ck.nbytes + ev8.nbytes + cv8.nbytes == 34816
