"""Helpers shared by the MoE GPU tests: device copies of a layer and an oracle expert bank
that encodes (with the oracle's own encoder) only the experts a test routes to."""
import numpy as np
import torch

import block_float_quantized_amd as bfq
import oracle
from oracle.moe import ExpertBank
from gpu_util import dev_bf16, dev_f32


class LazyBank(ExpertBank):
    """Oracle expert weights, encoded and decoded on demand from the fp32 layer."""

    def __init__(self, layer):
        self.fmt = layer["fmt"]
        self.hidden = layer["hidden"]
        self.inter = layer["inter"]
        self.layer = layer
        self._cache = {}

    def _dec(self, w):
        e, c = oracle.encode(w, self.fmt)
        return oracle.decode(e, c, self.fmt, *w.shape)

    def expert(self, e):
        if e in self._cache:
            return self._cache[e]
        h, f, L = self.hidden, self.inter, self.layer
        if e < 0:
            w = (self._dec(L["sh_gate"]), self._dec(L["sh_up"]), self._dec(L["sh_down"]))
        else:
            w = (self._dec(L["gate"][e * f:(e + 1) * f]), self._dec(L["up"][e * f:(e + 1) * f]),
                 self._dec(L["down"][e * h:(e + 1) * h]))
        self._cache[e] = w
        return w


def device_layer(layer, bias=None, shared=True) -> bfq.MoeLayer:
    def q(name):
        t = dev_f32(layer[name])
        m = bfq.bfp_quantize(layer["fmt"], t)
        del t
        return m
    return bfq.MoeLayer(
        n_experts=layer["n_experts"], top_k=layer["top_k"], hidden=layer["hidden"], inter=layer["inter"],
        router_w=dev_bf16(layer["router"]),
        router_bias=dev_f32(bias) if bias is not None else None,
        gate=q("gate"), up=q("up"), down=q("down"),
        sh_gate=q("sh_gate") if shared else None, sh_up=q("sh_up") if shared else None,
        sh_down=q("sh_down") if shared else None,
        sh_gate_w=dev_bf16(layer["sh_gate_w"]) if shared else None)
