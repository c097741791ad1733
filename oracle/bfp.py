"""Block floating point (BFP4 / BFP8) encode and decode, fp64, written for reading.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Format
------
A matrix stored ``[N][K]`` (N output rows, reduction dimension K) is cut along K into
16-value blocks ("Qwen3.8-27B ... gptq-ctx2-20261002", "What changed in this release",
GPTQ bullet: error compensation inside the 16-value BFP4 blocks). Each block keeps one
shared 8-bit exponent; each value keeps a sign bit and an ``m``-bit magnitude:

* BFP8: m = 7 (1 + 7 bits per value + 8/16 of the exponent = 8.5 bits per value),
* BFP4: m = 3 (1 + 3 + 0.5 = 4.5 bits per value).

The encoding, step by step (reading taken where the pages say only "block floating
point" and "round to nearest"):

1. ``e_i`` = the 8-bit exponent field of each fp32 value ``v_i`` of the block.
2. ``E`` = max_i e_i  (the shared exponent; 0 for a block of zeros/subnormals).
3. ``s`` = E - 127 - (m - 1): the block's scale is 2**s, so the block's largest value
   lands in [2**(m-1), 2**m) and its leading 1 is an explicit magnitude bit.
4. ``q_i`` = |v_i| * 2**-s rounded to the nearest integer, ties to even.
5. ``mag_i`` = min(q_i, 2**m - 1)   (a carry out of the top is clamped, E never grows).
6. ``sign_i`` = the sign bit of v_i (copied even when mag_i is 0, so -0.0 survives).
7. code_i = sign_i << m | mag_i; the block stores E.

Decode: v'_i = (-1)**sign_i * mag_i * 2**s. This is exact in fp32 and in bf16 (mag has
at most 8 significant bits and 2**s >= 2**-133, the smallest bf16 subnormal).

Inf and NaN have no finite block scale and are rejected (``NonFiniteError``).

Byte layout (ours; the pages do not give TT's tile layout): two planes, row-major in
``[N][K/16]`` block order. ``exp`` is ``uint8[N][K/16]``. For BFP8 ``code`` is
``uint8[N][K]``, one ``sign<<7 | mag`` byte per value. For BFP4 ``code`` is
``uint8[N][K/2]``: value 2j sits in the low nibble and value 2j+1 in the high nibble of
byte j, each nibble ``sign<<3 | mag``.
"""
from __future__ import annotations

import numpy as np

BFP4 = 4
BFP8 = 8
BLOCK = 16


class NonFiniteError(ValueError):
    """Raised for Inf/NaN input: no finite shared exponent exists for that block."""


def mantissa_bits(fmt: int) -> int:
    """Magnitude bits per value: 7 for BFP8, 3 for BFP4."""
    if fmt == BFP8:
        return 7
    if fmt == BFP4:
        return 3
    raise ValueError(f"unknown BFP format {fmt}")


def exp_bytes(n: int, k: int) -> int:
    """Bytes of the shared-exponent plane: one byte per 16-value block."""
    return n * (k // BLOCK)


def code_bytes(fmt: int, n: int, k: int) -> int:
    """Bytes of the code plane: one byte per value (BFP8) or one per two values (BFP4)."""
    return n * k if fmt == BFP8 else n * k // 2


def storage_bytes(fmt: int, n_values: int) -> int:
    """Total bytes for ``n_values`` values (a multiple of 16) in one row."""
    return exp_bytes(1, n_values) + code_bytes(fmt, 1, n_values)


def encode(w: np.ndarray, fmt: int) -> tuple[np.ndarray, np.ndarray]:
    """fp32 ``[N][K]`` -> (exp uint8 ``[N][K/16]``, code uint8 per the byte layout).

    Follows steps 1-7 of the module docstring. The scaling |v| * 2**-s is exact in fp64
    (|v| >= 2**-149 and -s <= 133 stay far inside fp64's range) and ``np.rint`` rounds
    half to even, so q is the exactly rounded integer.
    """
    m = mantissa_bits(fmt)
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("expected a 2-D [N][K] matrix")
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 16")
    if not np.all(np.isfinite(w)):
        raise NonFiniteError("Inf/NaN cannot be encoded")
    bits = w.view(np.uint32).reshape(n, k // BLOCK, BLOCK)
    e = ((bits >> 23) & 0xFF).astype(np.int64)            # step 1
    big_e = e.max(axis=2)                                   # step 2
    s = big_e - 127 - (m - 1)                               # step 3
    a = np.abs(w.astype(np.float64)).reshape(n, k // BLOCK, BLOCK)
    q = np.rint(np.ldexp(a, -s[:, :, None]))                # step 4 (exact, ties to even)
    mag = np.minimum(q, 2 ** m - 1).astype(np.uint8)        # step 5
    sign = (bits >> 31).astype(np.uint8)                    # step 6
    code = (sign << m) | mag                                # step 7
    exp = big_e.astype(np.uint8)
    code = code.reshape(n, k)
    if fmt == BFP4:
        code = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return exp, np.ascontiguousarray(code)


def unpack_codes(code: np.ndarray, fmt: int, n: int, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Code plane -> (sign uint8 [N][K], mag uint8 [N][K])."""
    m = mantissa_bits(fmt)
    code = np.asarray(code, dtype=np.uint8).reshape(n, -1)
    if fmt == BFP4:
        per_value = np.empty((n, k), np.uint8)
        per_value[:, 0::2] = code & 0x0F
        per_value[:, 1::2] = code >> 4
    else:
        per_value = code.reshape(n, k)
    return per_value >> m, per_value & ((1 << m) - 1)


def decode(exp: np.ndarray, code: np.ndarray, fmt: int, n: int, k: int) -> np.ndarray:
    """(exp, code) -> fp64 ``[N][K]`` of v' = (-1)**sign * mag * 2**s, exact.

    The result holds only fp32/bf16-representable values; ``.astype(np.float32)`` is
    exact. Signed zeros are kept (a sign bit with magnitude 0 decodes to -0.0).
    """
    m = mantissa_bits(fmt)
    sign, mag = unpack_codes(code, fmt, n, k)
    s = np.asarray(exp, dtype=np.int64).reshape(n, k // BLOCK) - 127 - (m - 1)
    s = np.repeat(s, BLOCK, axis=1)
    v = np.ldexp(mag.astype(np.float64), s)
    return np.where(sign == 1, -v, v)
