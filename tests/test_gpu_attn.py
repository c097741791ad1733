"""GPU BFP KV cache (bfp_kv_append) and decode attention (bfp_attn_decode) against the oracle.

Append: the cache bytes of the appended slots equal the oracle's encoding bit for bit (the
weights' rounding); other slots are untouched. Attention: every output within 2e-3 of
sum_t p_t |v_t| (the oracle's fp64 attention over the oracle-decoded cache), plus the fp32
floor of the probabilities: the GPU's p_t = exp(s_t - max s) are fp32, so those below 2^-126
may flush to zero, dropping at most L * 2^-126 * max_t |v_t| from an output. One cached
token returns its value exactly.

Rotated 4-bit V cache (KV_V_BFP4_HADAMARD): K bytes as above, V bytes equal the oracle's
rotated BFP4 encoding bit for bit. The output is rotated back from attention over the rotated
values; the rotation is orthonormal, so with the oracle's rotated-domain attention o_r and its
normaliser n_r = sum_t p_t |v_r,t|, (1) every output is within 2e-3 * sum_j n_r,j / sqrt(d) of
the oracle's rotated-back output (the rotated-domain bound carried through H / sqrt(d)), and (2)
the GPU output rotated by the oracle's fp64 transform is within 2e-3 n_r plus the fp32
rounding of the GPU's back rotation, at most (log2 d + 1) 2^-24 sum_j n_r,j, of o_r.
"""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import oracle
import synth
from oracle import BFP4, BFP8
from gpu_util import assert_within, dev_bf16, dev_f32, note

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _check(out, ref, norm, vd, group, what):
    """assert_within with the fp32 probability floor of each query head's KV head."""
    L = vd.shape[1]
    vmax = np.abs(vd).max(axis=(1, 2))[np.arange(out.shape[0]) // group]
    assert_within(out, ref, norm, TOL, extra=(L * 2.0 ** -126 * vmax)[:, None], what=what)


def _cache_bytes(cache, g, t0, t1):
    hd, T = cache.head_dim, cache.max_tokens
    nb = hd // 16
    ke = cache.k_exp.view(cache.kv_heads, T, nb)[g, t0:t1].cpu().numpy()
    kc = cache.k_code.view(cache.kv_heads, T, hd)[g, t0:t1].cpu().numpy()
    ve = cache.v_exp.view(cache.kv_heads, T, nb)[g, t0:t1].cpu().numpy()
    vc = cache.v_code.view(cache.kv_heads, T, -1)[g, t0:t1].cpu().numpy()
    return ke, kc, ve, vc


def _fill(kvh, hd, L, seed, dtype="f32", max_tokens=None, kscale=1.0, v_format=bfq.KV_V_BFP8):
    """A cache holding L tokens of N(0, 1) keys (times kscale) and values, appended in three
    calls; returns the cache and the oracle's decoded K, V [kvh][L][hd]."""
    rng = np.random.default_rng(seed)
    k = (rng.standard_normal((L, kvh, hd)) * kscale).astype(np.float32)
    v = rng.standard_normal((L, kvh, hd)).astype(np.float32)
    if dtype == "bf16":
        kb, vb = synth.bf16_bits(k), synth.bf16_bits(v)
        k, v = synth.bf16_values(kb).astype(np.float32), synth.bf16_values(vb).astype(np.float32)
        kd, vd = dev_bf16(kb.reshape(L, kvh, hd)), dev_bf16(vb.reshape(L, kvh, hd))
    else:
        kd, vd = dev_f32(k), dev_f32(v)
    cache = bfq.KvCache.empty(kvh, hd, max_tokens or L, v_format=v_format)
    cuts = sorted({0, L // 3, (2 * L) // 3, L})
    for a, b in zip(cuts[:-1], cuts[1:]):
        bfq.bfp_kv_append(cache, kd[a:b].contiguous(), vd[a:b].contiguous(), a)
    ek, ck = oracle.kv_encode(k)
    if v_format == bfq.KV_V_BFP4_HADAMARD:
        ev, cv = oracle.kv_encode_rotated(v)
        return cache, oracle.kv_decode(ek, ck, BFP8, hd), oracle.kv_decode(ev, cv, BFP4, hd), (ek, ck, ev, cv)
    ev, cv = oracle.kv_encode(v)
    return cache, oracle.kv_decode(ek, ck, BFP8, hd), oracle.kv_decode(ev, cv, BFP8, hd), (ek, ck, ev, cv)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_append_bit_exact(dtype):
    note(f"kv append {dtype}")
    kvh, hd, L, T = 2, 256, 37, 50
    cache, _, _, (ek, ck, ev, cv) = _fill(kvh, hd, L, seed=1, dtype=dtype, max_tokens=T)
    for g in range(kvh):
        ke, kc, ve, vc = _cache_bytes(cache, g, 0, L)
        assert np.array_equal(ke, ek[g]) and np.array_equal(kc, ck[g])
        assert np.array_equal(ve, ev[g]) and np.array_equal(vc, cv[g])
        rest = _cache_bytes(cache, g, L, T)
        assert all(not r.any() for r in rest), "slots past the appended tokens were written"


# group 8 runs on the matrix cores, smaller groups on the vector ALUs
@pytest.mark.parametrize("kvh,group,hd,L", [(2, 8, 256, 1), (2, 8, 256, 5), (2, 8, 256, 257), (2, 8, 256, 3000),
                                            (1, 8, 64, 300), (3, 8, 128, 777), (1, 8, 64, 70000),
                                            (1, 1, 64, 100), (4, 2, 128, 1000), (2, 4, 256, 10000),
                                            (8, 1, 128, 64)])
@pytest.mark.parametrize("qdt", ["f32", "bf16"])
def test_attn_decode_matches_oracle(kvh, group, hd, L, qdt):
    note(f"attn kvh={kvh} group={group} hd={hd} L={L} q={qdt}")
    cache, kd, vd, _ = _fill(kvh, hd, L, seed=L + hd + group)
    rng = np.random.default_rng(L)
    q = rng.standard_normal((kvh * group, hd)).astype(np.float32)
    if qdt == "bf16":
        qb = synth.bf16_bits(q)
        q64, qt = oracle.bf16_to_f64(qb), dev_bf16(qb)
    else:
        q64, qt = q.astype(np.float64), dev_f32(q)
    scale = 1.0 / np.sqrt(hd)
    out = bfq.bfp_attn_decode(cache, qt, L, scale).cpu().numpy()
    ref, norm = oracle.decode_attention(q64, kd, vd, scale)
    _check(out, ref, norm, vd, group, f"attn L={L}")
    if L == 1:
        assert np.array_equal(out, vd[np.arange(kvh * group) // group, 0].astype(np.float32))


def test_attn_decode_peaked_scores_and_prefix():
    """Large scores (softmax close to one-hot, no overflow) and attention over a prefix of a
    longer cache (tokens past seq_len are ignored)."""
    note("attn peaked / prefix")
    kvh, group, hd, L = 2, 8, 128, 700
    cache, kd, vd, _ = _fill(kvh, hd, L, seed=9, kscale=8.0)
    q = np.random.default_rng(3).standard_normal((kvh * group, hd)).astype(np.float32) * 4
    for n in (700, 333):
        out = bfq.bfp_attn_decode(cache, dev_f32(q), n, 1.0).cpu().numpy()
        ref, norm = oracle.decode_attention(q.astype(np.float64), kd[:, :n], vd[:, :n], 1.0)
        assert np.all(np.isfinite(out))
        _check(out, ref, norm, vd[:, :n], group, f"attn peaked n={n}")


def test_attn_decode_deterministic():
    note("attn deterministic")
    cache, _, _, _ = _fill(2, 256, 5000, seed=4)
    q = dev_f32(np.random.default_rng(4).standard_normal((16, 256)).astype(np.float32))
    a = bfq.bfp_attn_decode(cache, q, 5000, 0.0625)
    b = bfq.bfp_attn_decode(cache, q, 5000, 0.0625)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_workload_attn_decode_128k():
    """35B-class attention layer at 131,072 cached tokens: 2 KV heads x 256, 16 query heads."""
    note("workload: attn decode L=131072")
    kvh, group, hd, L = 2, 8, 256, 131072
    cache, kd, vd, _ = _fill(kvh, hd, L, seed=128)
    q = np.random.default_rng(5).standard_normal((kvh * group, hd)).astype(np.float32)
    out = bfq.bfp_attn_decode(cache, dev_f32(q), L, 1.0 / 16).cpu().numpy()
    ref, norm = oracle.decode_attention(q.astype(np.float64), kd, vd, 1.0 / 16)
    _check(out, ref, norm, vd, group, "attn 128K")


# ---- rotated 4-bit V ----------------------------------------------------------------------

V4R = bfq.KV_V_BFP4_HADAMARD


def _check_rot(out, q64, kd, vrd, scale, group, what):
    """Bounds (1) and (2) of the module notes; vrd: oracle-decoded rotated values."""
    hd = kd.shape[2]
    o_r, n_r = oracle.decode_attention(q64, kd, vrd, scale)
    L = vrd.shape[1]
    floor = (L * 2.0 ** -126 * np.abs(vrd).max(axis=(1, 2)))[np.arange(out.shape[0]) // group]
    tot = n_r.sum(axis=1) + hd * floor                                   # sum_j of the per-dim bound
    wide = np.repeat((tot / np.sqrt(hd))[:, None], hd, axis=1)
    assert_within(out, oracle.hadamard_rotate(o_r), wide, TOL, what=what + " (output)")
    back = oracle.hadamard_rotate(out.astype(np.float64))
    rnd = (np.log2(hd) + 1) * 2.0 ** -24 * tot
    assert_within(back, o_r, n_r, TOL, extra=floor[:, None] + rnd[:, None], what=what + " (rotated)")


@pytest.mark.parametrize("hd", [64, 128, 256])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_kv_append_v4r_bit_exact(hd, dtype):
    note(f"kv append v4r hd={hd} {dtype}")
    kvh, L, T = 3, 29, 40
    cache, _, _, (ek, ck, ev, cv) = _fill(kvh, hd, L, seed=hd + 2, dtype=dtype, max_tokens=T, v_format=V4R)
    assert cache.v_code.numel() == kvh * T * hd // 2
    for g in range(kvh):
        ke, kc, ve, vc = _cache_bytes(cache, g, 0, L)
        assert np.array_equal(ke, ek[g]) and np.array_equal(kc, ck[g])
        assert np.array_equal(ve, ev[g]) and np.array_equal(vc, cv[g])
        rest = _cache_bytes(cache, g, L, T)
        assert all(not r.any() for r in rest), "slots past the appended tokens were written"


def test_kv_append_v4r_outliers_and_tiny_values():
    """Rows with one huge channel, rows of subnormal-range values and zero rows: the fp64
    transform, its fp32 rounding (subnormals kept) and the BFP4 encoding match bit for bit."""
    note("kv append v4r outliers / tiny")
    kvh, hd, L = 2, 128, 12
    rng = np.random.default_rng(11)
    v = rng.standard_normal((L, kvh, hd)).astype(np.float32)
    v[0, 0, 5] = 3.0e4
    v[1, 1] *= np.float32(1e-38)
    v[2] = 0.0
    v[3, 0] = np.float32(1.4e-45)
    v[4, 1, 7] = -2.0 ** -149
    k = rng.standard_normal((L, kvh, hd)).astype(np.float32)
    cache = bfq.KvCache.empty(kvh, hd, L, v_format=V4R)
    bfq.bfp_kv_append(cache, dev_f32(k), dev_f32(v), 0)
    ev, cv = oracle.kv_encode_rotated(v)
    for g in range(kvh):
        _, _, ve, vc = _cache_bytes(cache, g, 0, L)
        assert np.array_equal(ve, ev[g]) and np.array_equal(vc, cv[g]), f"head {g}"


@pytest.mark.parametrize("kvh,group,hd,L", [(2, 8, 256, 1), (2, 8, 256, 257), (2, 8, 256, 3000),
                                            (1, 8, 64, 300), (3, 8, 128, 777),
                                            (1, 1, 64, 100), (4, 2, 128, 1000), (2, 4, 256, 10000),
                                            (8, 1, 128, 64)])
@pytest.mark.parametrize("qdt", ["f32", "bf16"])
def test_attn_decode_v4r_matches_oracle(kvh, group, hd, L, qdt):
    note(f"attn v4r kvh={kvh} group={group} hd={hd} L={L} q={qdt}")
    cache, kd, vrd, _ = _fill(kvh, hd, L, seed=L + hd + group + 1, v_format=V4R)
    rng = np.random.default_rng(L + 1)
    q = rng.standard_normal((kvh * group, hd)).astype(np.float32)
    if qdt == "bf16":
        qb = synth.bf16_bits(q)
        q64, qt = oracle.bf16_to_f64(qb), dev_bf16(qb)
    else:
        q64, qt = q.astype(np.float64), dev_f32(q)
    scale = 1.0 / np.sqrt(hd)
    out = bfq.bfp_attn_decode(cache, qt, L, scale).cpu().numpy()
    _check_rot(out, q64, kd, vrd, scale, group, f"attn v4r L={L}")


def test_attn_decode_v4r_peaked_and_prefix():
    note("attn v4r peaked / prefix")
    kvh, group, hd, L = 2, 8, 256, 900
    cache, kd, vrd, _ = _fill(kvh, hd, L, seed=19, kscale=8.0, v_format=V4R)
    q = np.random.default_rng(13).standard_normal((kvh * group, hd)).astype(np.float32) * 4
    for n in (900, 401):
        out = bfq.bfp_attn_decode(cache, dev_f32(q), n, 1.0).cpu().numpy()
        assert np.all(np.isfinite(out))
        _check_rot(out, q.astype(np.float64), kd[:, :n], vrd[:, :n], 1.0, group, f"attn v4r peaked n={n}")


def test_attn_decode_v4r_deterministic():
    note("attn v4r deterministic")
    cache, _, _, _ = _fill(2, 256, 5000, seed=14, v_format=V4R)
    q = dev_f32(np.random.default_rng(14).standard_normal((16, 256)).astype(np.float32))
    a = bfq.bfp_attn_decode(cache, q, 5000, 0.0625)
    b = bfq.bfp_attn_decode(cache, q, 5000, 0.0625)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_workload_attn_decode_v4r_262k():
    """The long-context cache at 262,144 cached tokens, 35B-class layer shape (2 KV heads x 256,
    16 query heads)."""
    note("workload: attn decode v4r L=262144")
    kvh, group, hd, L = 2, 8, 256, 262144
    cache, kd, vrd, _ = _fill(kvh, hd, L, seed=262, v_format=V4R)
    q = np.random.default_rng(6).standard_normal((kvh * group, hd)).astype(np.float32)
    out = bfq.bfp_attn_decode(cache, dev_f32(q), L, 1.0 / 16).cpu().numpy()
    _check_rot(out, q.astype(np.float64), kd, vrd, 1.0 / 16, group, "attn v4r 262K")
