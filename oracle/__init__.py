"""CPU oracle for BFP4/BFP8 block-floating-point matmuls — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct fp64 implementation (Python + numpy) of what the
weight-streaming matmul path computes. Only the test suite, the smoke check and the
bench's CPU-baseline leg may import it. The GPU library never imports, links or calls
anything here, and this package imports nothing from the GPU library: the two share no
code, headers, tables or constants. Its only shared dependency is the ``synth`` input
generator, which draws random numbers and holds none of the method's arithmetic.

Sources (the model-card pages on the TT-native mixed BFP4/BFP8 Qwen checkpoints):

* "Qwen3.8-27B — TT-native mixed BFP4/BFP8 (GPTQ), single P150", revision
  gptq-ctx2-20261002, section "What changed in this release", GPTQ bullet: BFP4
  matrices are made of 16-value blocks; values already representable in BFP4 are
  reproduced bit for bit by a re-conversion.
* "Qwen3.6-35B-A3B — TT-native mixed BFP4/BFP8 (GPTQ experts), single P150",
  sections "What is in this release" and "Precision as served" (experts BFP4; dense
  projections and LM head BFP8, round to nearest; router BF16) and "Verification",
  Checkpoint bullet (BFP tensors re-derived on CPU as the bit-exact round-to-nearest
  conversion).
* "qwen3.6-a3b-blackhole" bundle page, introduction: each layer has a 256-expert MoE
  with top-8 routing plus a shared expert.

Where the pages leave a step open (the meaning of the magnitude bits, ties, clamping,
signed zero, subnormals, the byte layout, where activations are rounded), the oracle
takes one stated reading; each function says which.

Modules: ``bfp`` (encode/decode/storage sizes), ``linalg`` (bf16 rounding, GEMM,
SwiGLU, greedy pick, error normaliser), ``moe`` (router, top-k, decode and prefill MoE, dispatch),
``attn`` (BFP8 KV cache rows, the rotated 4-bit V, single-token decode attention).
Every function here is pinned by ``tests/test_oracle_*.py`` against hand-worked values,
brute force, exact rational arithmetic, invariants or byte counts printed on the pages.
"""
from . import attn, bfp, linalg, moe  # noqa: F401
from .bfp import (BFP4, BFP8, NonFiniteError, code_bytes, decode, encode, exp_bytes,  # noqa: F401
                  mantissa_bits, storage_bytes, unpack_codes)
from .linalg import (bf16_round, bf16_to_f64, gemm, greedy_pick, normaliser, rel_err, silu,  # noqa: F401
                     swiglu)
from .moe import dispatch, moe_decode, moe_prefill, route  # noqa: F401
from .attn import decode_attention, hadamard_rotate, kv_decode, kv_encode, kv_encode_rotated  # noqa: F401
