"""Pins for the oracle's router, MoE and dispatch (CPU only)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from oracle import BFP4
from oracle.moe import ExpertBank, encode_layer


def _tiny_layer(rng, n_exp=8, hidden=32, inter=16, identical=False):
    def mat(r, c):
        return (rng.standard_normal((r, c)) * 0.2).astype(np.float32)
    g1, u1, d1 = mat(inter, hidden), mat(inter, hidden), mat(hidden, inter)
    gate = np.concatenate([g1 if identical else mat(inter, hidden) for _ in range(n_exp)])
    up = np.concatenate([u1 if identical else mat(inter, hidden) for _ in range(n_exp)])
    down = np.concatenate([d1 if identical else mat(hidden, inter) for _ in range(n_exp)])
    return {
        "fmt": BFP4, "n_experts": n_exp, "hidden": hidden, "inter": inter,
        "router": synth.bf16_bits((rng.standard_normal((n_exp, hidden)) * 0.3).astype(np.float32)),
        "sh_gate_w": synth.bf16_bits((rng.standard_normal(hidden) * 0.3).astype(np.float32)),
        "gate": gate, "up": up, "down": down,
        "sh_gate": mat(inter, hidden), "sh_up": mat(inter, hidden), "sh_down": mat(hidden, inter),
    }


def test_router_all_zero_weights():
    x = synth.normal_bf16(np.random.default_rng(0), (3, 64))
    wr = np.zeros((256, 64), np.uint16)
    out = oracle.route(x, wr, 8, sh_gate_bits=np.zeros(64, np.uint16))
    assert out["ids"].tolist() == [list(range(8))] * 3
    assert np.all(out["r"] == 0.125)
    assert np.all(out["g"] == 0.5)


def test_router_bias_forces_selection_and_order():
    rng = np.random.default_rng(1)
    x = synth.normal_bf16(rng, (4, 64))
    wr = synth.normal_bf16(rng, (256, 64), std=0.02)
    bias = np.zeros(256, np.float32)
    chosen = [200, 3, 77, 150, 9, 31, 255, 128]
    for rank, e in enumerate(chosen):
        bias[e] = 100.0 + 8 - rank
    out = oracle.route(x, wr, 8, bias=bias)
    assert out["ids"].tolist() == [chosen] * 4
    assert np.allclose(out["r"].sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(out["r"], axis=1) < 0)


def test_router_shared_gate_values():
    """The shared gate g = sigmoid(x . g_s) against tabulated logistic values: a one-hot x
    makes x . g_s one exact bf16 value z, and sigma(1), sigma(-2) are the constants
    e/(1+e) and 1/(1+e^2) (50-digit decimal arithmetic)."""
    x = np.zeros((2, 64), np.uint16)
    x[0, 5] = synth.bf16_bits(np.array([1.0], np.float32))[0]
    x[1, 40] = synth.bf16_bits(np.array([-0.5], np.float32))[0]
    gs = np.zeros(64, np.uint16)
    gs[5] = synth.bf16_bits(np.array([1.0], np.float32))[0]
    gs[40] = synth.bf16_bits(np.array([4.0], np.float32))[0]
    wr = synth.normal_bf16(np.random.default_rng(0), (16, 64), std=0.02)
    g = oracle.route(x, wr, 4, sh_gate_bits=gs)["g"]
    assert abs(g[0] - 0.73105857863000487925) <= 2.3e-16
    assert abs(g[1] - 0.11920292202211755594) <= 2.3e-16 * 0.12


def test_router_near_tie_settled_exactly():
    """Two logits whose fp64 sums come out in the wrong order: expert 0's exact logit is
    2^60 + 1000 * 1 - 2^60 = 1000, expert 1's is 999 + 0.5 = 999.5. Summed in fp64 the ones
    next to 2^60 are lost (the ulp there is 256), so a plain fp64 matmul ranks expert 1 first;
    the oracle's error intervals overlap, it recomputes the logits exactly and ranks expert 0
    first, with the weights of the exact logits (sigma(0.5) and 1 - sigma(0.5))."""
    h = 1024
    one, big, half = (synth.bf16_bits(np.array([v], np.float32))[0] for v in (1.0, 2.0 ** 30, 0.5))
    nbig = synth.bf16_bits(np.array([-2.0 ** 30], np.float32))[0]
    x = np.zeros((1, h), np.uint16)
    x[0, 0], x[0, 1:1001], x[0, 1001] = big, one, big
    wr = np.zeros((4, h), np.uint16)
    wr[0, 0], wr[0, 1:1001], wr[0, 1001] = big, one, nbig
    wr[1, 1:1000], wr[1, 1000] = one, half
    plain = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(wr).T
    assert plain[0, 1] > plain[0, 0], "the construction must fool a plain fp64 sum"
    out = oracle.route(x, wr, 2)
    assert out["exact"].tolist() == [True]
    assert out["ids"].tolist() == [[0, 1]]
    assert out["logits"][0, 0] == 1000.0 and out["logits"][0, 1] == 999.5
    assert abs(out["r"][0, 0] - 0.62245933120185456464) <= 4e-16
    assert abs(out["r"][0, 1] - 0.37754066879814543536) <= 4e-16
    # with a fp32 bias of +0.75 on expert 1 the exact order flips (1000 < 1000.25)
    bias = np.array([0.0, 0.75, 0.0, 0.0], np.float32)
    out = oracle.route(x, wr, 2, bias=bias)
    assert out["ids"].tolist() == [[1, 0]] and out["logits"][0, 1] == 1000.25


def test_router_random_data_needs_no_recheck():
    """On the workload's router draws the fp64 error intervals never overlap at the
    selection, so the recheck leaves the plain fp64 ranking in place."""
    router, shg = synth.moe_router(0)
    x = synth.moe_tokens(64, 0)
    out = oracle.route(x, router, 8, sh_gate_bits=shg)
    assert not out["exact"].any()
    plain = oracle.bf16_to_f64(x) @ oracle.bf16_to_f64(router).T
    want = np.argsort(-plain, axis=1, kind="stable")[:, :8]
    assert np.array_equal(out["ids"], want)


def test_router_tiny_vs_exact():
    rng = np.random.default_rng(2)
    m, n_exp, h = 5, 12, 24
    x = synth.normal_bf16(rng, (m, h))
    wr = synth.normal_bf16(rng, (n_exp, h), std=0.3)
    wr[3] = wr[7]                      # an exact tie: lower index must rank first
    out = oracle.route(x, wr, 4)
    xv = synth.bf16_values(x)
    wv = synth.bf16_values(wr)
    for t in range(m):
        logit = [sum(Fraction(float(xv[t, k])) * Fraction(float(wv[e, k])) for k in range(h)) for e in range(n_exp)]
        # brute force: rank = number of experts strictly better, ties broken by index
        rank = [sum(1 for f in range(n_exp) if logit[f] > logit[e] or (logit[f] == logit[e] and f < e))
                for e in range(n_exp)]
        want = [rank.index(i) for i in range(4)]
        assert out["ids"][t].tolist() == want
        if 3 in want and 7 in want:
            assert want.index(3) < want.index(7)
        lm = max(float(v) for v in logit)
        ex = [math.exp(float(logit[e]) - lm) for e in want]
        for j in range(4):
            assert abs(out["r"][t, j] - ex[j] / math.fsum(ex)) < 1e-14


def _scalar_moe(layer, x_bits, ids, r, g, round_h):
    """Per-token, per-slot loops with Python floats: the layer written out one sum at a time."""
    q = encode_layer(layer)
    h_, f_ = layer["hidden"], layer["inter"]

    def dec(role, r0, r1, k):
        exp, code = q[role]
        return oracle.decode(exp[r0:r1], code[r0:r1], BFP4, r1 - r0, k)

    def expert(e):
        if e < 0:
            return dec("sh_gate", 0, f_, h_), dec("sh_up", 0, f_, h_), dec("sh_down", 0, h_, f_)
        return (dec("gate", e * f_, (e + 1) * f_, h_), dec("up", e * f_, (e + 1) * f_, h_),
                dec("down", e * h_, (e + 1) * h_, f_))

    def mlp(xv, e):
        wg, wu, wd = expert(e)
        h = []
        for n in range(f_):
            a = math.fsum(xv[k] * wg[n, k] for k in range(h_))
            b = math.fsum(xv[k] * wu[n, k] for k in range(h_))
            hv = a / (1.0 + math.exp(-a)) * b
            if round_h:
                hv = float(oracle.bf16_round(np.array([hv]))[0])
            h.append(hv)
        return [math.fsum(h[k] * wd[n, k] for k in range(f_)) for n in range(h_)]

    xs = synth.bf16_values(x_bits).astype(np.float64)
    y = np.zeros((x_bits.shape[0], h_))
    for t in range(x_bits.shape[0]):
        acc = [0.0] * h_
        for j in range(ids.shape[1]):
            o = mlp(list(xs[t]), int(ids[t, j]))
            acc = [acc[n] + r[t, j] * o[n] for n in range(h_)]
        s = mlp(list(xs[t]), -1)
        y[t] = [acc[n] + g[t] * s[n] for n in range(h_)]
    return y


@pytest.mark.parametrize("round_h", [False, True])
def test_moe_tiny_vs_scalar_loops(round_h):
    rng = np.random.default_rng(3)
    layer = _tiny_layer(rng)
    x = synth.normal_bf16(rng, (3, layer["hidden"]))
    rt = oracle.route(x, layer["router"], 2, sh_gate_bits=layer["sh_gate_w"])
    bank = ExpertBank(layer, encode_layer(layer))
    fn = oracle.moe_prefill if round_h else oracle.moe_decode
    y, norm = fn(bank, x, rt)
    ys = _scalar_moe(layer, x, rt["ids"], rt["r"], rt["g"], round_h)
    assert np.all(np.abs(y - ys) <= 1e-12 * norm)


def test_moe_identical_experts_reduce_to_dense_mlp():
    rng = np.random.default_rng(4)
    layer = _tiny_layer(rng, identical=True)
    x = synth.normal_bf16(rng, (4, layer["hidden"]))
    rt = oracle.route(x, layer["router"], 3, sh_gate_bits=layer["sh_gate_w"])
    bank = ExpertBank(layer, encode_layer(layer))
    y, norm = oracle.moe_decode(bank, x, rt)
    # every routed expert is the same MLP, so MoE(x) = (sum r) * MLP(x) + g * Shared(x)
    xf = oracle.bf16_to_f64(x)
    f_, h_ = layer["inter"], layer["hidden"]
    q = encode_layer(layer)
    wg = oracle.decode(q["gate"][0][:f_], q["gate"][1][:f_], BFP4, f_, h_)
    wu = oracle.decode(q["up"][0][:f_], q["up"][1][:f_], BFP4, f_, h_)
    wd = oracle.decode(q["down"][0][:h_], q["down"][1][:h_], BFP4, h_, f_)
    mlp = oracle.gemm(oracle.swiglu(oracle.gemm(xf, wg), oracle.gemm(xf, wu)), wd)
    sg, su, sd = (oracle.decode(*q[k], BFP4, *shape) for k, shape in
                  (("sh_gate", (f_, h_)), ("sh_up", (f_, h_)), ("sh_down", (h_, f_))))
    sh = oracle.gemm(oracle.swiglu(oracle.gemm(xf, sg), oracle.gemm(xf, su)), sd)
    want = rt["r"].sum(axis=1, keepdims=True) * mlp + rt["g"][:, None] * sh
    assert np.all(np.abs(y - want) <= 1e-12 * norm)


def test_prefill_vs_decode_differ_only_by_h_rounding():
    rng = np.random.default_rng(5)
    layer = _tiny_layer(rng)
    x = synth.normal_bf16(rng, (6, layer["hidden"]))
    rt = oracle.route(x, layer["router"], 2, sh_gate_bits=layer["sh_gate_w"])
    bank = ExpertBank(layer, encode_layer(layer))
    yd, nd = oracle.moe_decode(bank, x, rt)
    yp, npf = oracle.moe_prefill(bank, x, rt)
    # rounding h to bf16 moves each term by at most 2**-9 of its size
    assert np.all(np.abs(yd - yp) <= 2.0 ** -8 * nd)
    assert not np.array_equal(yd, yp)


def test_dispatch_structure():
    rng = np.random.default_rng(6)
    m, k, n_exp = 300, 8, 64
    ids = np.stack([rng.choice(n_exp, k, replace=False, p=None) for _ in range(m)]).astype(np.int32)
    d = oracle.dispatch(ids, n_exp)
    assert d["counts"].sum() == m * k
    assert d["offsets"][0] == 0 and d["offsets"][-1] == m * k
    assert np.all(np.diff(d["offsets"]) == d["counts"])
    assert sorted(d["perm"].tolist()) == list(range(m * k))
    e_of = ids.ravel()[d["perm"]]
    t_of = d["perm"] // k
    want = np.lexsort((t_of, e_of))
    assert np.array_equal(want, np.arange(m * k))             # (e, t) nondecreasing
    for e in range(n_exp):
        seg = d["perm"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(ids.ravel()[seg] == e)
        assert len(seg) == int(np.sum(ids == e))
