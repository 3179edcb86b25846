"""Materialise a synthetic workload on the GPU (torch provides the memory).

Weights of all E experts are allocated contiguously, as a serving engine would
hold them. Experts are either all drawn (`experts=None`) or only a given set,
with the others filled with NaN (bf16 0xFFFF, e4m3 0xFF) so that reading an
unselected expert poisons the output. Draws use the device fill of the
generator, which writes the same bytes as the host fill.
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from moe_decode_02_amd import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, moe_layer_desc,
                               moe_layer_weights)

_TORCH = {synth.F32: torch.float32, synth.BF16: torch.bfloat16, synth.FP8: torch.uint8}
_MOE = {synth.F32: MOE_F32, synth.BF16: MOE_BF16, synth.FP8: MOE_FP8_E4M3}


def desc_of(w: synth.Workload) -> moe_layer_desc:
    return moe_layer_desc(w.H, w.E, w.k, w.I, w.Is, w.eps, _MOE[w.act], _MOE[w.router],
                          _MOE[w.expert], _MOE[w.shared], w.scale_group if w.expert == synth.FP8 else 0)


def to_device(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(a.view(np.int16).copy()).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def act_tensor(w: synth.Workload, B: int, device) -> torch.Tensor:
    return torch.zeros((B, w.H), dtype=_TORCH[w.act], device=device)


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DeviceLayer:
    """One layer of workload w on `device`; .weights is the moe_layer_weights struct."""

    def __init__(self, w: synth.Workload, layer: int = 0, device="cuda:0", experts=None,
                 random_gamma: bool = False, host_router=None, host_gamma=None):
        self.w, self.layer, self.device = w, layer, torch.device(device)
        dev = self.device
        g = host_gamma if host_gamma is not None else synth.gamma(w, random=random_gamma, layer=layer)
        self.gamma = to_device(g, dev)
        r = host_router if host_router is not None else synth.router_w(w, layer)
        self.router_w = to_device(r, dev)
        b = synth.router_bias(w, layer)
        self.router_bias = to_device(b, dev) if b is not None else None
        et = _TORCH[w.expert]
        self.egu = torch.empty((w.E, 2 * w.I, w.H), dtype=et, device=dev)
        self.ed = torch.empty((w.E, w.H, w.I), dtype=et, device=dev)
        self.egus = self.eds = None
        if w.expert == synth.FP8:
            self.egus = torch.zeros((w.E, 2 * w.I // 128), dtype=torch.bfloat16, device=dev)
            self.eds = torch.zeros((w.E, w.H // 128), dtype=torch.bfloat16, device=dev)
        ids = range(w.E) if experts is None else sorted(set(int(e) for e in np.ravel(experts)))
        if experts is not None:
            self._poison()
        self.fill_experts(ids)
        self.sgu = self.sd = None
        if w.Is > 0:
            self.sgu = torch.empty((2 * w.Is, w.H), dtype=_TORCH[w.shared], device=dev)
            self.sd = torch.empty((w.H, w.Is), dtype=_TORCH[w.shared], device=dev)
            synth.fill_device(self.sgu, synth.key(w.seed, layer, synth.T_SHARED_GU), w.shared, synth.WEIGHT_SIGMA)
            synth.fill_device(self.sd, synth.key(w.seed, layer, synth.T_SHARED_D), w.shared, synth.WEIGHT_SIGMA)
        self.weights = self._struct()

    def _poison(self):
        if self.w.expert == synth.FP8:
            self.egu.fill_(0xFF)
            self.ed.fill_(0xFF)
        elif self.w.expert == synth.BF16:  # 0xFFFF is a bf16 NaN
            self.egu.view(torch.int16).fill_(-1)
            self.ed.view(torch.int16).fill_(-1)
        else:
            self.egu.fill_(float("nan"))
            self.ed.fill_(float("nan"))

    def fill_experts(self, ids):
        w, L = self.w, self.layer
        for e in ids:
            kgu = synth.key(w.seed, L, synth.T_EXPERT_GU, e)
            kd = synth.key(w.seed, L, synth.T_EXPERT_D, e)
            if w.expert == synth.FP8:
                s1 = synth.fill_device_fp8(self.egu[e], 2 * w.I, w.H, kgu, synth.key(w.seed, L, synth.T_SCALE_GU, e),
                                           synth.WEIGHT_SIGMA)
                s2 = synth.fill_device_fp8(self.ed[e], w.H, w.I, kd, synth.key(w.seed, L, synth.T_SCALE_D, e),
                                           synth.WEIGHT_SIGMA)
                self.egus[e] = to_device(s1, self.device)
                self.eds[e] = to_device(s2, self.device)
            else:
                synth.fill_device(self.egu[e], kgu, w.expert, synth.WEIGHT_SIGMA)
                synth.fill_device(self.ed[e], kd, w.expert, synth.WEIGHT_SIGMA)

    def _struct(self) -> moe_layer_weights:
        def a(t):
            return None if t is None else t.data_ptr()
        return moe_layer_weights(a(self.gamma), a(self.router_w), a(self.router_bias), a(self.egu), a(self.ed),
                                 a(self.egus), a(self.eds), a(self.sgu), a(self.sd))

    def touched_bytes(self, experts) -> int:
        """Weight bytes one step reads: router + shared + gamma + the touched experts (+ scales)."""
        w = self.w
        esz = {synth.F32: 4, synth.BF16: 2, synth.FP8: 1}
        per_expert = 3 * w.I * w.H * esz[w.expert]
        if w.expert == synth.FP8:
            per_expert += (2 * w.I // 128 + w.H // 128) * 2
        return (w.E * w.H * esz[w.router] + 3 * w.Is * w.H * esz[w.shared] + w.H * esz[w.act]
                + len(set(int(e) for e in np.ravel(experts))) * per_expert)


def workspace(desc: moe_layer_desc, max_tokens: int, layers: int, device) -> torch.Tensor:
    from moe_decode_02_amd import moe_workspace_bytes
    n = moe_workspace_bytes(desc, max_tokens, layers)
    if n == 0:
        raise ValueError("descriptor outside the library's envelope")
    return torch.zeros(n, dtype=torch.uint8, device=device)
