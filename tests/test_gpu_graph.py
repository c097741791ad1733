"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph on the current stream):
a dense BFP4 gate/up + SwiGLU and BFP8 down GEMV, an MoE decode step and a rotated-V decode
attention call are captured into one graph; each of several replays, every one following eager
work (the outputs zeroed) and a synchronisation, leaves every output bit-identical to the eager
calls. The calls allocate nothing and never synchronise, so they can be captured."""
import numpy as np
import pytest
import torch

import block_float_quantized_amd as bfq
import synth
from gpu_util import dev_bf16, dev_f32, note, quantize_on_gpu
from moe_util import device_layer

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager_calls():
    note("graph capture: gemv + moe decode + attention")
    rng = np.random.default_rng(31)
    n, k = 3008, 2048
    g = quantize_on_gpu(4, (rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    u = quantize_on_gpu(4, (rng.standard_normal((n, k)) * 0.02).astype(np.float32))
    d = quantize_on_gpu(8, (rng.standard_normal((k, n)) * 0.02).astype(np.float32))
    x = dev_bf16(synth.bf16_bits(rng.standard_normal((2, k)).astype(np.float32)))
    h = torch.empty((2, n), dtype=torch.float32, device="cuda")
    y = torch.empty((2, k), dtype=torch.float32, device="cuda")
    ws_gu = torch.empty((max(bfq.bfp_gemm_workspace_bytes(g, 2, u), 16),), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty((max(bfq.bfp_gemm_workspace_bytes(d, 2), 16),), dtype=torch.uint8, device="cuda")

    layer = device_layer(synth.moe_layer(0))
    xm = dev_bf16(synth.moe_tokens(4, 0))
    ym = torch.empty((4, 2048), dtype=torch.float32, device="cuda")
    ws_m = torch.empty((bfq.bfp_moe_workspace_bytes(layer, 4),), dtype=torch.uint8, device="cuda")
    xm8 = dev_bf16(synth.moe_tokens(8, 1))              # grouped gate/up, per-token down
    ym8 = torch.empty((8, 2048), dtype=torch.float32, device="cuda")
    ws_m8 = torch.empty((bfq.bfp_moe_workspace_bytes(layer, 8),), dtype=torch.uint8, device="cuda")

    kvh, hd, L = 2, 256, 3000
    cache = bfq.KvCache.empty(kvh, hd, L, v_format=bfq.KV_V_BFP4_HADAMARD)
    bfq.bfp_kv_append(cache, dev_f32(rng.standard_normal((L, kvh, hd)).astype(np.float32)),
                      dev_f32(rng.standard_normal((L, kvh, hd)).astype(np.float32)), 0)
    q = dev_f32(rng.standard_normal((16, hd)).astype(np.float32))
    ya = torch.empty((16, hd), dtype=torch.float32, device="cuda")
    ws_a = torch.empty((bfq.bfp_attn_decode_workspace_bytes(cache, 16, L),), dtype=torch.uint8, device="cuda")

    def calls():
        bfq.bfp_gemm(g, x, w_up=u, out=h, workspace=ws_gu)
        bfq.bfp_gemm(d, h, out=y, workspace=ws_d)
        bfq.bfp_moe_forward(layer, xm, out=ym, workspace=ws_m)
        bfq.bfp_moe_forward(layer, xm8, out=ym8, workspace=ws_m8)
        bfq.bfp_attn_decode(cache, q, L, 1.0 / 16, out=ya, workspace=ws_a)

    outs = [h, y, ym, ym8, ya]
    calls()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}, output {i}"
    # eager calls after the replays still give the same results
    calls()
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o.view(torch.uint8), r.view(torch.uint8))
    del graph
