"""Helpers for the GPU parity tests: move seeded numpy inputs to the device and compare
GPU results with the oracle's."""
import sys

import numpy as np
import torch

import block_float_quantized_amd as bfq
import oracle

DEV = "cuda"


def note(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(msg, file=sys.stderr, flush=True)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).to(DEV)
    return t.view(torch.bfloat16)


def host_bits_bf16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def matrix_from_oracle(fmt: int, exp: np.ndarray, code: np.ndarray, n: int, k: int) -> bfq.BfpMatrix:
    e = torch.from_numpy(np.ascontiguousarray(exp).reshape(-1)).to(DEV)
    c = torch.from_numpy(np.ascontiguousarray(code).reshape(-1)).to(DEV)
    return bfq.BfpMatrix(fmt, n, k, e, c)


def quantize_on_gpu(fmt: int, w: np.ndarray) -> bfq.BfpMatrix:
    return bfq.bfp_quantize(fmt, dev_f32(w))


def assert_within(y_gpu: np.ndarray, y_ref: np.ndarray, norm: np.ndarray, tol: float, extra=None, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    bound = tol * norm
    if extra is not None:
        bound = bound + extra
    d = np.abs(y_gpu - y_ref)
    bad = d > bound
    if np.any(bad):
        i = np.argwhere(bad)[0]
        idx = tuple(i)
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; first at {idx}: gpu={y_gpu[idx]!r} "
                             f"oracle={y_ref[idx]!r} norm={norm[idx]!r} rel={d[idx] / max(norm[idx], 1e-300):.3e}")
    return float(np.max(np.where(norm > 0, d / np.where(norm > 0, norm, 1), 0)))
