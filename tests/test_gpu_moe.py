"""GPU MoE routing, dispatch and layer forward against the oracle.

Routing and dispatch are integer decisions and must match bit for bit (expert ids and
their order, counts, offsets, permutation). Routing weights and the shared gate are fp32
outputs of fp64 computations (within 1e-6 relative). The layer output y is within 2e-3 of
the oracle's, relative to the oracle's sum of |w_j| * sum_k |h_k Wd_k| (+ the shared term).
"""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import oracle
import synth
from gpu_util import assert_within, dev_bf16, dev_f32, note
from moe_util import LazyBank, device_layer

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _router_only_layer(seed, bias=None):
    router, shg = synth.moe_router(seed)
    dummy = bfq.BfpMatrix(4, 1, 32, torch.zeros(16, dtype=torch.uint8, device="cuda"),
                          torch.zeros(16, dtype=torch.uint8, device="cuda"))
    lay = bfq.MoeLayer(256, 8, synth.HIDDEN, synth.INTER, dev_bf16(router),
                       dev_f32(bias) if bias is not None else None, dummy, dummy, dummy, None, None, None,
                       dev_bf16(shg))
    return lay, router, shg


@pytest.mark.parametrize("m,with_bias", [(1, False), (8, False), (16, False), (32, False), (2048, True)])
def test_route_matches_oracle(m, with_bias):
    note(f"route m={m} bias={with_bias}")
    bias = synth.router_bias(0) if with_bias else None
    lay, router, shg = _router_only_layer(0, bias)
    x = synth.moe_tokens(m, 0, cfg_id=5 if with_bias else 4)
    ids, w, g = bfq.bfp_moe_route(lay, dev_bf16(x))
    ref = oracle.route(x, router, 8, bias=bias, sh_gate_bits=shg)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.allclose(w.cpu().numpy(), ref["r"], rtol=1e-6, atol=0)
    assert np.allclose(g.cpu().numpy(), ref["g"], rtol=1e-6, atol=0)


def test_route_special_cases():
    """All-zero router: every logit ties, experts 0..7 in order, weights exactly 1/8."""
    note("route special cases")
    lay, router, shg = _router_only_layer(0)
    lay.router_w = torch.zeros_like(lay.router_w)
    lay.sh_gate_w = torch.zeros_like(lay.sh_gate_w)
    x = dev_bf16(synth.moe_tokens(3, 1))
    ids, w, g = bfq.bfp_moe_route(lay, x)
    assert ids.cpu().tolist() == [list(range(8))] * 3
    assert torch.all(w == 0.125) and torch.all(g == 0.5)
    # a +100 bias on chosen experts forces them, ordered by bias
    bias = np.zeros(256, np.float32)
    chosen = [200, 3, 77, 150, 9, 31, 255, 128]
    for r_, e in enumerate(chosen):
        bias[e] = 100.0 + 8 - r_
    lay2, _, _ = _router_only_layer(0, bias)
    lay2.router_w = torch.zeros_like(lay2.router_w)
    ids, w, g = bfq.bfp_moe_route(lay2, x)
    assert ids.cpu().tolist() == [chosen] * 3


@pytest.mark.parametrize("m", [1, 7, 32, 33, 300, 2048, 5000])
def test_dispatch_bit_exact(m):
    note(f"dispatch m={m}")
    rng = np.random.default_rng(m)
    # skewed expert popularity, distinct experts per token
    p = rng.dirichlet(np.full(256, 0.1))
    ids = np.stack([rng.choice(256, 8, replace=False, p=p) for _ in range(m)]).astype(np.int32)
    counts, offsets, perm = bfq.bfp_moe_dispatch(torch.from_numpy(ids).cuda(), 256)
    ref = oracle.dispatch(ids, 256)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(perm.cpu().numpy(), ref["perm"])


@pytest.fixture(scope="module")
def moe_full():
    note("building the 256-expert MoE layer")
    layer = synth.moe_layer(0)
    dev = device_layer(layer)
    return layer, dev, LazyBank(layer)


@pytest.mark.parametrize("m", [1, 3, 8, 16])
def test_moe_decode_matches_oracle(moe_full, m):
    layer, dev, bank = moe_full
    note(f"moe decode m={m}")
    x = synth.moe_tokens(m, 0)
    ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((m, 8), dtype=torch.float32, device="cuda")
    y = bfq.bfp_moe_forward(dev, dev_bf16(x), topk_ids=ids, topk_w=w).cpu().numpy()
    rt = oracle.route(x, layer["router"], 8, sh_gate_bits=layer["sh_gate_w"])
    assert np.array_equal(ids.cpu().numpy(), rt["ids"])
    assert np.allclose(w.cpu().numpy(), rt["r"], rtol=1e-6, atol=0)
    ref, norm = oracle.moe_decode(bank, x, rt)
    assert_within(y, ref, norm, TOL, what=f"moe decode m={m}")


def test_moe_decode_crowded_experts(moe_full):
    """Decode with every token routed to the same 8 experts (a large router bias on them):
    each group holds all 32 pairs and is cut into many row tiles; the shared group too."""
    layer, dev, bank = moe_full
    note("moe decode m=32 crowded")
    m = 32
    bias = np.zeros(256, np.float32)
    bias[[3, 17, 42, 64, 99, 128, 200, 255]] = 40.0 + np.arange(8, dtype=np.float32)
    devb = bfq.MoeLayer(**{**dev.__dict__, "router_bias": dev_f32(bias)})
    x = synth.moe_tokens(m, 5)
    ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
    y = bfq.bfp_moe_forward(devb, dev_bf16(x), topk_ids=ids).cpu().numpy()
    rt = oracle.route(x, layer["router"], 8, bias=bias, sh_gate_bits=layer["sh_gate_w"])
    assert np.array_equal(ids.cpu().numpy(), rt["ids"])
    assert set(np.unique(rt["ids"])) == {3, 17, 42, 64, 99, 128, 200, 255}
    ref, norm = oracle.moe_decode(bank, x, rt)
    assert_within(y, ref, norm, TOL, what="moe decode crowded")


@pytest.mark.parametrize("m", [2, 5])
def test_moe_decode_small_odd_batches(moe_full, m):
    """Row tiles of two pairs with a one-pair tail (odd m: the shared group)."""
    layer, dev, bank = moe_full
    note(f"moe decode m={m}")
    x = synth.moe_tokens(m, 9)
    y = bfq.bfp_moe_forward(dev, dev_bf16(x)).cpu().numpy()
    rt = oracle.route(x, layer["router"], 8, sh_gate_bits=layer["sh_gate_w"])
    ref, norm = oracle.moe_decode(bank, x, rt)
    assert_within(y, ref, norm, TOL, what=f"moe decode m={m}")


def test_moe_decode_deterministic_and_row_invariant(moe_full):
    """Same input, same bits; and token t's output is the same bits whatever the batch it is
    in (1..32 tokens): routing, expert sums and the combine are per token, in an order that
    does not depend on the batch."""
    layer, dev, bank = moe_full
    note("moe decode determinism")
    x = dev_bf16(synth.moe_tokens(4, 3))
    a = bfq.bfp_moe_forward(dev, x)
    b = bfq.bfp_moe_forward(dev, x)
    assert torch.equal(a, b)
    note("moe decode batch invariance")
    x32 = dev_bf16(synth.moe_tokens(32, 4))
    y32 = bfq.bfp_moe_forward(dev, x32).view(torch.int32)
    for lo, hi in [(0, 1), (13, 14), (31, 32), (4, 12), (0, 16), (16, 32), (5, 7)]:
        y = bfq.bfp_moe_forward(dev, x32[lo:hi].contiguous()).view(torch.int32)
        assert torch.equal(y, y32[lo:hi]), f"tokens {lo}:{hi} differ from the 32-token call"


def _prefill_check(layer, dev, bank, x, bias, sample):
    m = x.shape[0]
    ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
    y = bfq.bfp_moe_forward(dev, dev_bf16(x), topk_ids=ids).cpu().numpy()
    rt_all = oracle.route(x, layer["router"], 8, bias=bias, sh_gate_bits=layer["sh_gate_w"])
    assert np.array_equal(ids.cpu().numpy(), rt_all["ids"])
    xs = x[sample]
    rt = {k: v[sample] for k, v in rt_all.items()}
    ref, norm = oracle.moe_prefill(bank, xs, rt)
    return assert_within(y[sample], ref, norm, TOL, what=f"moe prefill m={m}")


def test_moe_prefill_small(moe_full):
    layer, dev, bank = moe_full
    note("moe prefill m=40")
    x = synth.moe_tokens(40, 7)
    _prefill_check(layer, dev, bank, x, None, np.arange(40))


@pytest.mark.parametrize("crowded", [False, True])
def test_moe_prefill_multi_chunk_dispatch(moe_full, crowded):
    """300 tokens: the many-token dispatch runs over three token chunks (128, 128, 44), so each
    expert's pairs are ranked across chunks; with crowded experts (a +40 bias on eight
    experts) every chunk feeds the same groups. Every token is checked."""
    layer, dev, bank = moe_full
    note(f"moe prefill m=300 crowded={crowded}")
    bias = None
    devb = dev
    if crowded:
        bias = np.zeros(256, dtype=np.float32)
        bias[[3, 17, 42, 64, 99, 128, 200, 255]] = 40.0
        devb = bfq.MoeLayer(**{**dev.__dict__, "router_bias": dev_f32(bias)})
    x = synth.moe_tokens(300, 21)
    _prefill_check(layer, devb, bank, x, bias, np.arange(300))


def test_moe_prefill_chunk_2048(moe_full):
    """The 2,048-token prefill chunk with a skewed N(0, 1.5) per-expert router bias: every
    output of every token."""
    layer, dev, bank = moe_full
    note("moe prefill m=2048 with bias")
    bias = synth.router_bias(0)
    devb = bfq.MoeLayer(**{**dev.__dict__, "router_bias": dev_f32(bias)})
    x = synth.moe_tokens(2048, 0, cfg_id=5)
    _prefill_check(layer, devb, bank, x, bias, np.arange(2048))


def test_moe_prefill_repeatable(moe_full):
    """The 2,048-token chunk run 24 times, each over a workspace filled with other random
    bytes: every output bit for bit the same. Guards the LDS ring of the grouped GEMMs (a
    slot refilled while another wave's reads of it were still queued once changed a few
    outputs of one wave's columns in rare runs) and any read of workspace not written."""
    layer, dev, bank = moe_full
    note("moe prefill m=2048 repeatability")
    devb = bfq.MoeLayer(**{**dev.__dict__, "router_bias": dev_f32(synth.router_bias(0))})
    m = 2048
    x = dev_bf16(synth.moe_tokens(m, 0, cfg_id=5))
    ws = torch.empty((bfq.bfp_moe_workspace_bytes(devb, m),), dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda")
    first = None
    for r in range(24):
        gen.manual_seed(1000 + r)
        ws.random_(0, 256, generator=gen)
        y = bfq.bfp_moe_forward(devb, x, workspace=ws)
        if first is None:
            first = y.clone()
        else:
            bad = (y != first).any(1).nonzero().flatten().tolist()
            assert not bad, f"run {r}: tokens {bad[:8]} differ from the first run"


def test_moe_prefill_and_decode_agree(moe_full):
    """The same 33 tokens through the prefill path and through 33 single-token decodes:
    identical routing, outputs equal up to the bf16 rounding of h in prefill."""
    layer, dev, bank = moe_full
    note("moe prefill vs decode")
    x = synth.moe_tokens(33, 11)
    yp = bfq.bfp_moe_forward(dev, dev_bf16(x)).cpu().numpy()
    yd = np.concatenate([bfq.bfp_moe_forward(dev, dev_bf16(x[i:i + 1])).cpu().numpy() for i in range(33)])
    rt = oracle.route(x, layer["router"], 8, sh_gate_bits=layer["sh_gate_w"])
    _, norm = oracle.moe_decode(bank, x, rt)
    assert np.all(np.abs(yp - yd) <= 2.0 ** -7 * norm)


def _small_layer(seed, gate_scale=1.0, x_scale=1.0, n_exp=16, hidden=256, inter=64, top_k=4):
    """A small layer (fp32 weights, oracle-encodable) with the workload's distributions; gate and
    up of every expert (and the shared one) scaled by gate_scale."""
    rng = np.random.default_rng(seed)

    def mat(r, c, s=1.0):
        return (rng.standard_normal((r, c)) * 0.02 * s).astype(np.float32)
    return {
        "fmt": 4, "n_experts": n_exp, "top_k": top_k, "hidden": hidden, "inter": inter,
        "router": synth.normal_bf16(rng, (n_exp, hidden), std=0.02 / x_scale),
        "sh_gate_w": synth.normal_bf16(rng, (hidden,), std=0.02 / x_scale),
        "gate": mat(n_exp * inter, hidden, gate_scale), "up": mat(n_exp * inter, hidden, gate_scale),
        "down": mat(n_exp * hidden, inter),
        "sh_gate": mat(inter, hidden, gate_scale), "sh_up": mat(inter, hidden, gate_scale),
        "sh_down": mat(hidden, inter),
    }


@pytest.mark.parametrize("m", [1, 4])
def test_moe_decode_extreme_exponents(m):
    """Gate and up weights near 2^123 (shared exponents up to ~252) with activations near
    2^-112 (products stay normal fp32 numbers): the decode expert kernels apply the BFP4 block
    scale exactly for every exponent."""
    note(f"moe decode extreme exponents m={m}")
    layer = _small_layer(31, gate_scale=2.0 ** 128, x_scale=2.0 ** -112)
    e, _ = oracle.encode(layer["gate"], 4)
    assert e.max() >= 248
    dev = device_layer(layer)
    rng = np.random.default_rng(32)
    x = synth.bf16_bits((rng.standard_normal((m, layer["hidden"])) * 2.0 ** -112).astype(np.float32))
    ids = torch.empty((m, layer["top_k"]), dtype=torch.int32, device="cuda")
    y = bfq.bfp_moe_forward(dev, dev_bf16(x), topk_ids=ids).cpu().numpy()
    rt = oracle.route(x, layer["router"], layer["top_k"], sh_gate_bits=layer["sh_gate_w"])
    assert np.array_equal(ids.cpu().numpy(), rt["ids"])
    ref, norm = oracle.moe_decode(LazyBank(layer), x, rt)
    assert np.all(np.isfinite(y))
    assert_within(y, ref, norm, TOL, what="moe decode extreme exponents")


# (experts, top_k, hidden, inter, shared): lanes per row 4 / 8 / 16 in the gate/up and down
# kernels, a half-filled last row tile (inter 96), a one-unit second group (inter 1056), no
# shared expert, top-1, an intermediate size past the per-token kernels' limit (2080), and
# the largest one they take with nine slots (83 KB of staged h per down workgroup)
_ONE_TOKEN_SHAPES = [(16, 4, 256, 96, True), (32, 8, 1024, 640, False), (4, 2, 2080, 1056, True),
                     (8, 1, 128, 2080, True), (6, 3, 512, 512, False), (8, 8, 256, 2048, True)]


@pytest.mark.parametrize("n_exp,top_k,hidden,inter,shared", _ONE_TOKEN_SHAPES)
def test_moe_one_token_shapes(n_exp, top_k, hidden, inter, shared):
    """One token against the oracle (ids, weights, gate, y), and the same bits as that token's
    row of a 3-token call (per-token kernels) and of a 6-token call (grouped kernels)."""
    note(f"moe one token E={n_exp} k={top_k} H={hidden} F={inter} shared={shared}")
    layer = _small_layer(50 + top_k, n_exp=n_exp, hidden=hidden, inter=inter, top_k=top_k)
    if not shared:
        for name in ("sh_gate", "sh_up", "sh_down"):
            layer[name] = np.zeros_like(layer[name])
    dev = device_layer(layer, shared=shared)
    rng = np.random.default_rng(51)
    x = synth.bf16_bits(rng.standard_normal((6, hidden)).astype(np.float32))
    xd = dev_bf16(x)
    ids = torch.empty((1, top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, top_k), dtype=torch.float32, device="cuda")
    y1 = bfq.bfp_moe_forward(dev, xd[1:2].contiguous(), topk_ids=ids, topk_w=w)
    rt = oracle.route(x[1:2], layer["router"], top_k, sh_gate_bits=layer["sh_gate_w"] if shared else None)
    assert np.array_equal(ids.cpu().numpy(), rt["ids"])
    assert np.allclose(w.cpu().numpy(), rt["r"], rtol=1e-6, atol=0)
    if not shared:
        rt["g"] = np.zeros(1)              # no shared term (its weights are zero as well)
    ref, norm = oracle.moe_decode(LazyBank(layer), x[1:2], rt)
    assert_within(y1.cpu().numpy(), ref, norm, TOL, what="moe one token")
    y3 = bfq.bfp_moe_forward(dev, xd[:3].contiguous())
    assert torch.equal(y1.view(torch.int32), y3[1:2].view(torch.int32))
    y6 = bfq.bfp_moe_forward(dev, xd)
    assert torch.equal(y1.view(torch.int32), y6[1:2].view(torch.int32))


@pytest.mark.parametrize("m", [4, 40])
def test_route_nan_token(m):
    """A token whose activations hold NaN (so every logit is NaN) still gets top-k distinct
    experts in range: NaN ranks below every number, ties go to the lower index, so it takes
    experts 0..7. The other tokens route as the oracle does (decode path at m = 4, the
    certified many-token path at m = 40)."""
    note(f"route NaN token m={m}")
    lay, router, shg = _router_only_layer(0)
    x = synth.moe_tokens(m, 2)
    bad = 1
    x[bad, 7] = 0x7FC0                      # bf16 quiet NaN
    ids, w, g = bfq.bfp_moe_route(lay, dev_bf16(x))
    ids = ids.cpu().numpy()
    assert ids[bad].tolist() == list(range(8))
    ok = np.array([t for t in range(m) if t != bad])
    ref = oracle.route(x[ok], router, 8, sh_gate_bits=shg)
    assert np.array_equal(ids[ok], ref["ids"])
    assert np.allclose(w.cpu().numpy()[ok], ref["r"], rtol=1e-6, atol=0)


@pytest.mark.parametrize("m", [4, 40])
def test_moe_forward_nan_token(moe_full, m):
    """A NaN token through the whole layer (decode at m = 4, prefill at m = 40): its expert
    ids stay valid, so the dispatch and the expert kernels read only real rows, and every other
    token's output matches the oracle."""
    layer, dev, bank = moe_full
    note(f"moe forward NaN token m={m}")
    x = synth.moe_tokens(m, 6)
    bad = m - 2
    x[bad, 100] = 0x7FC0
    ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
    y = bfq.bfp_moe_forward(dev, dev_bf16(x), topk_ids=ids).cpu().numpy()
    assert ids.cpu().numpy()[bad].tolist() == list(range(8))
    ok = np.array([t for t in range(m) if t != bad])
    rt = oracle.route(x[ok], layer["router"], 8, sh_gate_bits=layer["sh_gate_w"])
    assert np.array_equal(ids.cpu().numpy()[ok], rt["ids"])
    fn = oracle.moe_decode if m <= 32 else oracle.moe_prefill
    ref, norm = fn(bank, x[ok], rt)
    assert_within(y[ok], ref, norm, TOL, what=f"moe forward with a NaN token m={m}")


def test_route_many_tokens_with_exact_ties():
    """Many-token routing (certified matrix-core logits + exact re-check) with planted exact
    ties: duplicated router rows must rank by expert index, as the oracle does."""
    note("route m=300 with duplicated router rows")
    router, shg = synth.moe_router(3)
    for a, b in ((5, 17), (40, 41), (100, 200), (7, 255)):
        router[b] = router[a]
    lay, _, _ = _router_only_layer(3)
    lay.router_w = dev_bf16(router)
    x = synth.moe_tokens(300, 3)
    ids, w, g = bfq.bfp_moe_route(lay, dev_bf16(x))
    ref = oracle.route(x, router, 8, sh_gate_bits=shg)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.allclose(w.cpu().numpy(), ref["r"], rtol=1e-6, atol=0)
    assert np.allclose(g.cpu().numpy(), ref["g"], rtol=1e-6, atol=0)
