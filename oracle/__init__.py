"""ctypes wrapper of the plain CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline of the benchmark; the product path never imports it. The arithmetic
lives in moe_oracle.c; this file only marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from functools import lru_cache
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(_HERE, "libmoe_oracle.so")

F32, BF16, FP8 = 0, 1, 2


def build(force: bool = False) -> None:
    if force or not os.path.exists(SO):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-shared", "-fPIC", "-o", SO,
                               os.path.join(_HERE, "moe_oracle.c"), "-lm"])


class OrcDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("act", ctypes.c_int32), ("router", ctypes.c_int32), ("expert", ctypes.c_int32),
                ("shared", ctypes.c_int32), ("scale_group", ctypes.c_int32)]


class OrcWeights(ctypes.Structure):
    _fields_ = [("rms_gamma", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("expert_gate_up", ctypes.c_void_p),
                ("expert_down", ctypes.c_void_p), ("expert_gate_up_scale", ctypes.c_void_p),
                ("expert_down_scale", ctypes.c_void_p), ("shared_gate_up", ctypes.c_void_p),
                ("shared_down", ctypes.c_void_p)]


@lru_cache(maxsize=None)
def lib():
    if not os.path.exists(SO):
        build()
    L = ctypes.CDLL(SO)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    L.orc_bf16_value.argtypes = [ctypes.c_uint16]
    L.orc_bf16_value.restype = ctypes.c_double
    L.orc_bf16_round.argtypes = [ctypes.c_double]
    L.orc_bf16_round.restype = ctypes.c_uint16
    L.orc_e4m3_value.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_value.restype = ctypes.c_double
    L.orc_rmsnorm.argtypes = [vp, vp, vp, vp, vp]
    L.orc_router_logits.argtypes = [vp, vp, vp, vp]
    L.orc_route.argtypes = [vp, vp, vp, vp]
    L.orc_route_weights.argtypes = [vp, vp, vp, vp]
    L.orc_layer_token_given.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.orc_ffn.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp, vp, vp]
    L.orc_layer_token.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    L.orc_layer.argtypes = [vp, vp, vp, i32, vp, vp, vp, vp]
    L.orc_stack.argtypes = [vp, vp, i32, vp, i32, vp, vp, vp, vp]
    L.orc_error_string.argtypes = [ctypes.c_int]
    L.orc_error_string.restype = ctypes.c_char_p
    return L


def _p(a) -> Optional[int]:
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _check(rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"oracle error {rc}: {lib().orc_error_string(rc).decode()}")


@dataclasses.dataclass
class Layer:
    """Host weights of one layer. Experts are dicts {expert id: array}; experts
    that are absent must not be selected (the oracle reports it)."""
    gamma: np.ndarray
    router_w: np.ndarray
    router_bias: Optional[np.ndarray]
    gate_up: Dict[int, np.ndarray]
    down: Dict[int, np.ndarray]
    gate_up_scale: Dict[int, np.ndarray] = dataclasses.field(default_factory=dict)
    down_scale: Dict[int, np.ndarray] = dataclasses.field(default_factory=dict)
    shared_gate_up: Optional[np.ndarray] = None
    shared_down: Optional[np.ndarray] = None


def desc(H, E, k, I, Is, act, router, expert, shared, eps=1e-6, scale_group=128) -> OrcDesc:
    return OrcDesc(H, E, k, I, Is, eps, act, router, expert, shared, scale_group)


def desc_of(w) -> OrcDesc:
    """Descriptor of a synth.Workload."""
    return desc(w.H, w.E, w.k, w.I, w.Is, w.act, w.router, w.expert, w.shared, w.eps, w.scale_group)


class _Pinned:
    """Keeps the ctypes arrays alive while the oracle runs."""

    def __init__(self, d: OrcDesc, layer: Layer):
        E = d.num_experts
        self.gu = (ctypes.c_void_p * E)(*[_p(layer.gate_up.get(e)) for e in range(E)])
        self.dn = (ctypes.c_void_p * E)(*[_p(layer.down.get(e)) for e in range(E)])
        self.gus = (ctypes.c_void_p * E)(*[_p(layer.gate_up_scale.get(e)) for e in range(E)])
        self.dns = (ctypes.c_void_p * E)(*[_p(layer.down_scale.get(e)) for e in range(E)])
        if layer.router_bias is not None:
            assert layer.router_bias.dtype == np.float32
        self.w = OrcWeights(_p(layer.gamma), _p(layer.router_w), _p(layer.router_bias),
                            ctypes.cast(self.gu, ctypes.c_void_p), ctypes.cast(self.dn, ctypes.c_void_p),
                            ctypes.cast(self.gus, ctypes.c_void_p), ctypes.cast(self.dns, ctypes.c_void_p),
                            _p(layer.shared_gate_up), _p(layer.shared_down))
        self.layer = layer


def _act_np(d: OrcDesc):
    return np.uint16 if d.act == BF16 else np.float32


def rmsnorm(d: OrcDesc, x_t: np.ndarray, gamma: np.ndarray):
    xhat = np.zeros(d.hidden, np.float32)
    xact = np.zeros(d.hidden, np.float32)
    _check(lib().orc_rmsnorm(ctypes.byref(d), _p(x_t), _p(gamma), _p(xhat), _p(xact)))
    return xhat, xact


def router_logits(d: OrcDesc, layer: Layer, xhat: np.ndarray) -> np.ndarray:
    pin = _Pinned(d, layer)
    out = np.zeros(d.num_experts, np.float32)
    _check(lib().orc_router_logits(ctypes.byref(d), ctypes.byref(pin.w), _p(xhat), _p(out)))
    return out


def route(d: OrcDesc, logits: np.ndarray):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    idx = np.zeros(d.top_k, np.int32)
    w = np.zeros(d.top_k, np.float32)
    _check(lib().orc_route(ctypes.byref(d), _p(logits), _p(idx), _p(w)))
    return idx, w


def route_weights(d: OrcDesc, logits: np.ndarray, idx) -> np.ndarray:
    """Weights of a given selection idx [k]: the restricted, renormalised softmax."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    w = np.zeros(d.top_k, np.float32)
    _check(lib().orc_route_weights(ctypes.byref(d), _p(logits), _p(idx), _p(w)))
    return w


def ffn(d: OrcDesc, dtype: int, inter: int, gate_up, down, xact, gate_up_scale=None, down_scale=None):
    h = np.zeros(inter, np.float32)
    out = np.zeros(d.hidden, np.float32)
    _check(lib().orc_ffn(ctypes.byref(d), dtype, inter, _p(gate_up), _p(down), _p(gate_up_scale),
                         _p(down_scale), _p(np.ascontiguousarray(xact, np.float32)), _p(h), _p(out)))
    return h, out


def layer(d: OrcDesc, L: Layer, x: np.ndarray):
    """x [B][H] (act dtype) -> (y [B][H], idx [B][k], w [B][k], logits [B][E])."""
    x = np.ascontiguousarray(x)
    B = x.shape[0]
    y = np.zeros_like(x)
    idx = np.zeros((B, d.top_k), np.int32)
    w = np.zeros((B, d.top_k), np.float32)
    logits = np.zeros((B, d.num_experts), np.float32)
    pin = _Pinned(d, L)
    _check(lib().orc_layer(ctypes.byref(d), ctypes.byref(pin.w), _p(x), B, _p(y), _p(idx), _p(w),
                           _p(logits)))
    return y, idx, w, logits


def layer_given(d: OrcDesc, L: Layer, x_t: np.ndarray, idx):
    """One token x_t [H] through the layer with the selection idx [k] (rank order)
    in place of the top-k -> (y [H], w [k], logits [E])."""
    x_t = np.ascontiguousarray(x_t)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    y = np.zeros_like(x_t)
    w = np.zeros(d.top_k, np.float32)
    logits = np.zeros(d.num_experts, np.float32)
    pin = _Pinned(d, L)
    _check(lib().orc_layer_token_given(ctypes.byref(d), ctypes.byref(pin.w), _p(x_t), _p(idx), _p(y), _p(w),
                                       _p(logits)))
    return y, w, logits


def stack(d: OrcDesc, layers, x: np.ndarray):
    """x [B][H] -> (y [B][H], idx [L][B][k], w [L][B][k], logits [L][B][E])."""
    x = np.ascontiguousarray(x)
    B, Ln = x.shape[0], len(layers)
    pins = [_Pinned(d, L) for L in layers]
    arr = (OrcWeights * Ln)(*[p.w for p in pins])
    y = np.zeros_like(x)
    idx = np.zeros((Ln, B, d.top_k), np.int32)
    w = np.zeros((Ln, B, d.top_k), np.float32)
    logits = np.zeros((Ln, B, d.num_experts), np.float32)
    _check(lib().orc_stack(ctypes.byref(d), arr, Ln, _p(x), B, _p(y), _p(idx), _p(w), _p(logits)))
    return y, idx, w, logits


def bf16_value(bits: int) -> float:
    return lib().orc_bf16_value(bits)


def bf16_round(v: float) -> int:
    return lib().orc_bf16_round(v)


def e4m3_value(code: int) -> float:
    return lib().orc_e4m3_value(code)
