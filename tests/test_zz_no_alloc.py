"""bfp_moe_forward_noalloc (decode MoE on the library's static device scratch) against
bfp_moe_forward with a caller workspace: same kernels, so the same bits, on two calls in a
row, the second with fewer tokens (the scratch keeps the first call's contents)."""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import synth
from gpu_util import dev_bf16, note
from moe_util import device_layer

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer_dev():
    note("no-alloc: building the 256-expert MoE layer")
    return device_layer(synth.moe_layer(0))


def _reference(dev, x):
    m = x.shape[0]
    ids = torch.empty((m, 8), dtype=torch.int32, device="cuda")
    w = torch.empty((m, 8), dtype=torch.float32, device="cuda")
    y = bfq.bfp_moe_forward(dev, x, topk_ids=ids, topk_w=w)
    return y, ids, w


def test_noalloc_matches_workspace_call_twice(layer_dev):
    # 16 tokens: grouped kernels; 8: grouped gate/up, per-token down; 3: per-token kernels
    for m, seed in ((16, 40), (8, 42), (3, 41)):
        note(f"no-alloc moe decode m={m}")
        x = dev_bf16(synth.moe_tokens(m, seed))
        y_ref, ids_ref, w_ref = _reference(layer_dev, x)
        y = torch.full((m, 2048), float("nan"), dtype=torch.float32, device="cuda")
        ids = torch.full((m, 8), -1, dtype=torch.int32, device="cuda")
        w = torch.zeros((m, 8), dtype=torch.float32, device="cuda")
        bfq.bfp_moe_forward_noalloc(layer_dev, x, y, topk_ids=ids, topk_w=w)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref), f"m={m}: expert ids differ"
        assert torch.equal(w.view(torch.int32), w_ref.view(torch.int32)), f"m={m}: routing weights differ"
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), f"m={m}: outputs differ"


def test_noalloc_rejects_prefill_sizes(layer_dev):
    note("no-alloc: host-side refusals")
    x = dev_bf16(synth.moe_tokens(33, 1))
    y = torch.empty((33, 2048), dtype=torch.float32, device="cuda")
    with pytest.raises(bfq.BfpError) as e:
        bfq.bfp_moe_forward_noalloc(layer_dev, x, y)
    assert e.value.status == 7
    assert bfq.bfp_moe_workspace_bytes(layer_dev, 32) <= bfq.MOE_NOALLOC_SCRATCH_BYTES
