"""Pins for the oracle's BFP encoder/decoder (CPU only).

Each pin is something other than the oracle itself: a block worked by hand
(tests/golden/hand_block.json), byte counts printed on the pages
(tests/golden/byte_pins.json), a brute-force nearest-grid search in exact rational
arithmetic, and invariants the pages state (values already representable re-encode
bit for bit: "Qwen3.8-27B ... gptq-ctx2-20261002", "What changed in this release").
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import BFP4, BFP8

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f32(bits_hex):
    return np.array([int(b, 16) for b in bits_hex], np.uint32).view(np.float32)


def _dec(strings):
    out = []
    for s in strings:
        out.append(-0.0 if s == "-0" else float(s))
    return np.array(out)


@pytest.mark.parametrize("fmt,key", [(BFP8, "bfp8"), (BFP4, "bfp4")])
def test_hand_worked_block(fmt, key):
    g = _load("hand_block.json")
    w = _f32(g["inputs_f32_bits"]).reshape(1, 16)
    exp, code = oracle.encode(w, fmt)
    assert exp.tolist() == [g[key]["exp"]]
    assert [f"{b:02x}" for b in code.ravel()] == g[key]["code_hex"]
    v = oracle.decode(exp, code, fmt, 1, 16).ravel()
    want = _dec(g[key]["decoded"])
    assert np.array_equal(v, want)
    # signed zeros are part of the pin
    assert np.array_equal(np.signbit(v), np.signbit(want))


def test_bfp4_nibble_order():
    g = _load("hand_block.json")["bfp4"]
    w = _f32(_load("hand_block.json")["inputs_f32_bits"]).reshape(1, 16)
    _, code = oracle.encode(w, BFP4)
    sign, mag = oracle.unpack_codes(code, BFP4, 1, 16)
    nib = (sign << 3 | mag).ravel()
    assert [f"{n:x}" for n in nib] == g["nibbles_hex"]


def test_page_byte_pins():
    pins = _load("byte_pins.json")["pins"]
    kv = pins[0]
    vals = kv["bf16_bytes_per_token"] // 2
    b8 = oracle.storage_bytes(BFP8, vals)
    assert round(b8 / 1024, kv["printed_decimals"]) == kv["bfp8_kib_per_token_printed"]
    assert b8 == vals * 17 // 16
    full = pins[1]
    total = full["tokens"] * oracle.storage_bytes(BFP8, full["bf16_bytes_per_token"] // 2)
    assert round(total / 2 ** 30, full["printed_decimals"]) == full["bfp8_gib_printed"]
    v4 = pins[2]
    # find the per-token value count that makes K and V in BFP8 take the printed bytes
    n = [n for n in range(16, 40000, 16) if 2 * oracle.storage_bytes(BFP8, n) == v4["bfp8_k_plus_bfp8_v_bytes"]]
    assert n == [16384]
    assert oracle.storage_bytes(BFP8, n[0]) + oracle.storage_bytes(BFP4, n[0]) == v4["bfp8_k_plus_bfp4_v_bytes"]


def _brute_mag(v: np.float32, s: int, m: int) -> int:
    """Nearest grid point mag*2**s (mag in 0..2**m-1) to |v| in exact rationals, ties to even."""
    a = abs(Fraction(float(v)))
    step = Fraction(2) ** s
    best, best_d = None, None
    for mag in range(2 ** m):
        d = abs(a - mag * step)
        if best is None or d < best_d or (d == best_d and mag % 2 == 0):
            best, best_d = mag, d
    return best


def _brute_block(vals: np.ndarray, m: int):
    bits = vals.view(np.uint32)
    big_e = int(((bits >> 23) & 0xFF).max())
    s = big_e - 127 - (m - 1)
    mags = [_brute_mag(v, s, m) for v in vals]
    signs = [int(b >> 31) for b in bits]
    return big_e, mags, signs


def _random_blocks(rng, nblk):
    out = []
    for i in range(nblk):
        kind = i % 5
        if kind == 0:
            v = rng.standard_normal(16).astype(np.float32) * np.float32(0.02)
        elif kind == 1:   # wide dynamic range inside one block
            v = (rng.standard_normal(16) * np.exp2(rng.integers(-30, 5, 16))).astype(np.float32)
        elif kind == 2:   # exact ties at the BFP4 and BFP8 grids
            e = rng.integers(-3, 4)
            v = (rng.integers(0, 32, 16) / 2.0 * 2.0 ** (e - 4)).astype(np.float32)
            v[0] = np.float32(2.0 ** e)
        elif kind == 3:   # subnormal and tiny
            v = (rng.integers(0, 1 << 23, 16).astype(np.uint32)).view(np.float32).copy()
            v[rng.random(16) < 0.5] *= -1
        else:             # values just below a power of two (rounding carries)
            v = (np.float32(1.0) - rng.integers(0, 8, 16).astype(np.float32) * np.float32(2.0 ** -24))
            v *= np.float32(2.0 ** rng.integers(-5, 5))
        out.append(v)
    return np.stack(out).astype(np.float32)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_brute_force_nearest(fmt):
    m = oracle.mantissa_bits(fmt)
    rng = np.random.default_rng(1234 + fmt)
    blocks = _random_blocks(rng, 60)
    exp, code = oracle.encode(blocks, fmt)
    sign, mag = oracle.unpack_codes(code, fmt, blocks.shape[0], 16)
    for i, blk in enumerate(blocks):
        big_e, mags, signs = _brute_block(blk, m)
        assert exp[i, 0] == big_e
        assert mag[i].tolist() == mags, (i, blk)
        assert sign[i].tolist() == signs


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_all_codes_decode_and_reencode(fmt):
    """Every (E, code) pair that the encoder can emit re-encodes to itself.

    A block the encoder emits always holds at least one magnitude in [2**(m-1), 2**m)
    (the element that set E), so the decoded max keeps exponent field E. Here every
    magnitude and sign is exercised at several exponents, with that lead element fixed.
    """
    m = oracle.mantissa_bits(fmt)
    rng = np.random.default_rng(7)
    for big_e in (0, 1, 2, 60, 127, 200, 254):
        codes = np.arange(2 ** (m + 1), dtype=np.uint8)
        per_block = []
        for start in range(0, len(codes), 15):
            chunk = list(codes[start:start + 15])
            chunk += list(rng.integers(0, 2 ** (m + 1), 15 - len(chunk)).astype(np.uint8))
            lead = np.uint8((rng.integers(0, 2) << m) | rng.integers(2 ** (m - 1), 2 ** m))
            per_block.append([lead] + chunk)
        per_value = np.array(per_block, np.uint8)
        nb = per_value.shape[0]
        if fmt == BFP4:
            code = (per_value[:, 0::2] | (per_value[:, 1::2] << 4)).astype(np.uint8)
        else:
            code = per_value
        exp = np.full((nb, 1), big_e, np.uint8)
        v = oracle.decode(exp, code, fmt, nb, 16).astype(np.float32)
        exp2, code2 = oracle.encode(v, fmt)
        assert np.array_equal(exp2, exp)
        assert np.array_equal(code2, code)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_idempotent(fmt):
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((40, 256)) * np.exp2(rng.integers(-20, 20, (40, 1)))).astype(np.float32)
    exp, code = oracle.encode(w, fmt)
    v = oracle.decode(exp, code, fmt, 40, 256)
    exp2, code2 = oracle.encode(v.astype(np.float32), fmt)
    assert np.array_equal(exp2, exp) and np.array_equal(code2, code)
    v2 = oracle.decode(exp2, code2, fmt, 40, 256)
    assert np.array_equal(v, v2)


def test_edge_cases():
    # rounding carry at the top is clamped, E stays the max exponent
    w = np.zeros((1, 16), np.float32)
    w[0, 0] = np.float32(1.9999)
    exp, code = oracle.encode(w, BFP8)
    assert exp[0, 0] == 127 and code[0, 0] == 127
    # an all-subnormal block: E = 0, s = -133 (BFP8) / -129 (BFP4)
    sub = np.zeros(16, np.uint32)
    sub[:3] = [0x007FFFFF, 0x00400000, 0x00000001]
    w = sub.view(np.float32).reshape(1, 16)
    exp, code = oracle.encode(w, BFP8)
    assert exp[0, 0] == 0
    assert code[0, :3].tolist() == [127, 64, 0]
    exp, code = oracle.encode(w, BFP4)
    _, mag = oracle.unpack_codes(code, BFP4, 1, 16)
    assert exp[0, 0] == 0 and mag[0, :3].tolist() == [7, 4, 0]
    # all zeros
    exp, code = oracle.encode(np.zeros((2, 32), np.float32), BFP4)
    assert not exp.any() and not code.any()
    # non-finite input is rejected
    for bad in (np.inf, -np.inf, np.nan):
        w = np.ones((1, 16), np.float32)
        w[0, 5] = bad
        with pytest.raises(oracle.NonFiniteError):
            oracle.encode(w, BFP8)
    with pytest.raises(ValueError):
        oracle.encode(np.ones((1, 24), np.float32), BFP8)


@pytest.mark.parametrize("fmt", [BFP8, BFP4])
def test_decoded_values_are_bf16_exact(fmt):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((16, 128)) * np.exp2(rng.integers(-140, 120, (16, 1)))).astype(np.float32)
    exp, code = oracle.encode(w, fmt)
    v = oracle.decode(exp, code, fmt, 16, 128)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v)          # exact in fp32
    assert not np.any(f.view(np.uint32) & 0xFFFF)           # and in bf16 (low half zero)


def test_storage_size_formula():
    for fmt, num in ((BFP8, 17), (BFP4, 9)):
        for n, k in ((3, 16), (7, 2048), (2, 17408)):
            w = np.ones((n, k), np.float32)
            exp, code = oracle.encode(w, fmt)
            assert exp.nbytes + code.nbytes == n * k * num // 16
            assert exp.nbytes == oracle.exp_bytes(n, k)
            assert code.nbytes == oracle.code_bytes(fmt, n, k)
