"""Seeded synthetic inputs for the MoE decode layer.

This module holds no arithmetic of the layer. It draws the inputs both sides
use: the plain CPU oracle (tests, smoke check, CPU baseline) and the HIP path
(tests, benchmark). Every draw is counter-based (synth_core.h): the host fill
(synth_host.c) and the device fill (synth_dev.hip) produce the same bytes.

The workloads (``WORKLOADS``) are the five synthetic decode-layer
configurations; their shapes follow the 16-of-896-expert Kimi K3 MoE
(aiposthub.com article, section on what the K3 decode path changed) at one
GPU's tensor-parallel share, and batch 1-64 (same section; smzdm.com post,
section on who can use it).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from functools import lru_cache

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(_HERE, "libsynth_host.so")
DEV_SO = os.path.join(_HERE, "libsynth_dev.so")

TABLE_SIZE = 1 << 14
T_X, T_GAMMA, T_ROUTER, T_EXPERT_GU, T_EXPERT_D, T_SHARED_GU, T_SHARED_D = 1, 2, 3, 4, 5, 6, 7
T_BIAS_PERM, T_SCALE_GU, T_SCALE_D = 8, 9, 10
T_SPEC = 11  # draft-token perturbations of the speculative-decoding verify workload

F32, BF16, FP8 = 0, 1, 2
WEIGHT_SIGMA = 0.02
INPUT_SIGMA = 1.0


def hip_flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(force: bool = False, device: bool = True) -> None:
    """Compile the host generator (gcc) and, if asked, the device fill (hipcc)."""
    if force or not os.path.exists(HOST_SO):
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", HOST_SO,
                               os.path.join(_HERE, "synth_host.c"), "-lm", "-lpthread"])
    if device and (force or not os.path.exists(DEV_SO)):
        subprocess.check_call(["/opt/rocm/bin/hipcc", *hip_flags(), "-o", DEV_SO,
                               os.path.join(_HERE, "synth_dev.hip")])


@lru_cache(maxsize=None)
def _host():
    if not os.path.exists(HOST_SO):
        build(device=False)
    lib = ctypes.CDLL(HOST_SO)
    u64, u32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
    lib.synth_normal_table.argtypes = [vp]
    lib.synth_value_table.argtypes = [vp, ctypes.c_double, ctypes.c_int, vp]
    lib.synth_fp8_scale_bits.argtypes = [vp, ctypes.c_double, ctypes.c_int]
    lib.synth_fp8_scale_bits.restype = ctypes.c_uint16
    lib.synth_fp8_code_table.argtypes = [vp, ctypes.c_double, ctypes.c_int, vp]
    lib.synth_fill.argtypes = [vp, u64, u64, vp, ctypes.c_int, ctypes.c_int]
    lib.synth_fill_fp8.argtypes = [vp, u64, u64, u64, u64, vp, vp, vp]
    lib.synth_key_c.argtypes = [u64, u32, u32, u32, u32]
    lib.synth_key_c.restype = u64
    lib.synth_index_c.argtypes = [u64, u64]
    lib.synth_index_c.restype = u32
    lib.synth_scale_class.argtypes = [u64, u64]
    lib.synth_scale_class.restype = u32
    lib.synth_zipf_bias.argtypes = [u64, ctypes.c_int, ctypes.c_double, vp]
    return lib


@lru_cache(maxsize=None)
def _dev():
    if not os.path.exists(DEV_SO):
        raise RuntimeError(f"{DEV_SO} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(DEV_SO)
    u64, vp = ctypes.c_uint64, ctypes.c_void_p
    lib.synth_dev_fill.argtypes = [vp, u64, u64, vp, ctypes.c_int, vp]
    lib.synth_dev_fill.restype = ctypes.c_int
    lib.synth_dev_fill_fp8.argtypes = [vp, u64, u64, u64, u64, vp, vp]
    lib.synth_dev_fill_fp8.restype = ctypes.c_int
    return lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


NTHREADS = max(1, min(16, os.cpu_count() or 1))


# ---- tables ---------------------------------------------------------------

@lru_cache(maxsize=None)
def normal_table() -> np.ndarray:
    """z_i = Phi^-1((i + 0.5) / 2^14), i < 2^14 (float64)."""
    z = np.zeros(TABLE_SIZE, dtype=np.float64)
    _host().synth_normal_table(_ptr(z))
    return z


@lru_cache(maxsize=None)
def value_table(sigma: float, dtype: int) -> np.ndarray:
    """Storage bytes of z * sigma: float32 entries (dtype F32) or bf16 bit patterns (BF16)."""
    z = normal_table()
    if dtype == F32:
        out = np.zeros(TABLE_SIZE, dtype=np.float32)
    elif dtype == BF16:
        out = np.zeros(TABLE_SIZE, dtype=np.uint16)
    else:
        raise ValueError(dtype)
    _host().synth_value_table(_ptr(z), sigma, dtype, _ptr(out))
    return out


@lru_cache(maxsize=None)
def fp8_tables(sigma: float):
    """(codes [4][2^14] uint8, scale bits [4] uint16): one code table per scale class."""
    z = normal_table()
    codes = np.zeros((4, TABLE_SIZE), dtype=np.uint8)
    scales = np.zeros(4, dtype=np.uint16)
    for c in range(4):
        scales[c] = _host().synth_fp8_scale_bits(_ptr(z), sigma, c)
        _host().synth_fp8_code_table(_ptr(z), sigma, c, _ptr(codes[c]))
    return codes, scales


def key(seed: int, layer: int, tensor: int, sub: int = 0, attempt: int = 0) -> int:
    return int(_host().synth_key_c(seed, layer, tensor, sub, attempt))


def index(k: int, i: int) -> int:
    return int(_host().synth_index_c(k, i))


def scale_class(class_key: int, g: int) -> int:
    return int(_host().synth_scale_class(class_key, g))


# ---- host fills -------------------------------------------------------------

def _np_dtype(dtype: int):
    return {F32: np.float32, BF16: np.uint16, FP8: np.uint8}[dtype]


def fill_host(shape, k: int, dtype: int, sigma: float) -> np.ndarray:
    """Array of the given shape: element i = value_table(sigma, dtype)[index(k, i)]."""
    table = value_table(sigma, dtype)
    out = np.empty(shape, dtype=_np_dtype(dtype))
    _host().synth_fill(_ptr(out), out.size, k, _ptr(table), out.itemsize, NTHREADS)
    return out


def fill_host_fp8(rows: int, cols: int, k: int, class_key: int, sigma: float):
    """(codes [rows][cols] uint8, scales [rows/128] bf16 bits)."""
    codes, scale_bits = fp8_tables(sigma)
    out = np.empty((rows, cols), dtype=np.uint8)
    scales = np.empty(rows // 128, dtype=np.uint16)
    _host().synth_fill_fp8(_ptr(out), rows, cols, k, class_key, _ptr(codes), _ptr(scale_bits),
                           _ptr(scales))
    return out, scales


def zipf_bias(seed: int, E: int, s: float) -> np.ndarray:
    out = np.zeros(E, dtype=np.float32)
    _host().synth_zipf_bias(seed, E, s, _ptr(out))
    return out


# ---- workloads ---------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    H: int
    E: int
    k: int
    I: int
    Is: int
    act: int
    router: int
    expert: int
    shared: int
    seed: int
    batches: tuple
    layers: int = 1
    zipf_s: float = 0.0       # router bias = log-Zipf(s) when > 0
    eps: float = 1e-6
    scale_group: int = 128
    # speculative-decoding verify step: each request contributes its base
    # token and spec_drafts draft tokens, x_draft = act(x_base + spec_delta * z)
    spec_drafts: int = 0
    spec_delta: float = 0.0

    @property
    def B(self) -> int:
        return self.batches[0]


WORKLOADS = {
    # tiny fp32 layer the oracle finishes in well under a second
    "tiny_f32": Workload("tiny_f32", H=256, E=32, k=4, I=128, Is=128, act=F32, router=F32,
                         expert=F32, shared=F32, seed=0, batches=(1,)),
    # one GPU's share of a K3-scale layer (I = 1024 tensor-parallel slice)
    "k3_b1": Workload("k3_b1", H=7168, E=896, k=16, I=1024, Is=2048, act=BF16, router=F32,
                      expert=BF16, shared=BF16, seed=1, batches=(1,)),
    "k3_b8": Workload("k3_b8", H=7168, E=896, k=16, I=1024, Is=2048, act=BF16, router=F32,
                      expert=BF16, shared=BF16, seed=2, batches=(8,)),
    "k3_b64_zipf": Workload("k3_b64_zipf", H=7168, E=896, k=16, I=1024, Is=2048, act=BF16,
                            router=F32, expert=BF16, shared=BF16, seed=3, batches=(64,),
                            zipf_s=1.1),
    "k3_stack4_fp8": Workload("k3_stack4_fp8", H=7168, E=896, k=16, I=1024, Is=2048, act=BF16,
                              router=BF16, expert=FP8, shared=BF16, seed=4,
                              batches=(1, 2, 4, 16, 64), layers=4),
    # the verify step of speculative decoding on the K3 share: R requests of
    # 1 + 7 tokens (R = 1 and 8), drafts perturbing their request's base token
    "k3_spec_verify": Workload("k3_spec_verify", H=7168, E=896, k=16, I=1024, Is=2048, act=BF16,
                               router=F32, expert=BF16, shared=BF16, seed=5, batches=(8, 64),
                               spec_drafts=7, spec_delta=0.5),
}


def token_row(w: Workload, t: int, attempts=None, layer: int = 0) -> np.ndarray:
    """Token t of a layer input [H] in the activation dtype (redraw attempts[t]).
    Verify-step workloads (spec_drafts > 0): token t = r * (1 + drafts) + d is
    request r's base token (d = 0, an N(0, 1) draw) or a draft, the base plus
    spec_delta * N(0, 1) in fp32, stored in the activation dtype; a draft's
    attempt redraws its perturbation, the base's attempt the whole request."""
    a = 0 if attempts is None else int(attempts[t])
    if w.spec_drafts <= 0:
        return fill_host((w.H,), key(w.seed, layer, T_X, t, a), w.act, INPUT_SIGMA)
    g = 1 + w.spec_drafts
    t0 = (t // g) * g
    a0 = 0 if attempts is None else int(attempts[t0])
    x = fill_host((w.H,), key(w.seed, layer, T_X, t0, a0), F32, INPUT_SIGMA)
    if t != t0:
        x = x + fill_host((w.H,), key(w.seed, layer, T_SPEC, t, a), F32, w.spec_delta)
    return x.astype(np.float32) if w.act == F32 else _bf16_bits_of(x)


def x_tokens(w: Workload, B: int, attempts=None, layer: int = 0) -> np.ndarray:
    """Layer input [B][H] in the activation dtype; token t uses redraw attempts[t]."""
    rows = [token_row(w, t, attempts, layer) for t in range(B)]
    return np.stack(rows) if rows else np.zeros((0, w.H), dtype=_np_dtype(w.act))


def gamma(w: Workload, random: bool = False, layer: int = 0) -> np.ndarray:
    """RMSNorm gain: ones (the workloads), or a random N(1, 0.25) gain for pins."""
    if not random:
        one = np.ones(w.H, dtype=np.float32)
        return one if w.act == F32 else (one.view(np.uint32) >> 16).astype(np.uint16)
    g = fill_host((w.H,), key(w.seed, layer, T_GAMMA), F32, 0.25) + np.float32(1.0)
    if w.act == F32:
        return g.astype(np.float32)
    return _bf16_bits_of(g)


def _bf16_bits_of(f: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def router_w(w: Workload, layer: int = 0) -> np.ndarray:
    return fill_host((w.E, w.H), key(w.seed, layer, T_ROUTER), w.router, WEIGHT_SIGMA)


def router_bias(w: Workload, layer: int = 0):
    if w.zipf_s <= 0:
        return None
    return zipf_bias(w.seed * 1000 + layer, w.E, w.zipf_s)


def shared_gate_up(w: Workload, layer: int = 0) -> np.ndarray:
    return fill_host((2 * w.Is, w.H), key(w.seed, layer, T_SHARED_GU), w.shared, WEIGHT_SIGMA)


def shared_down(w: Workload, layer: int = 0) -> np.ndarray:
    return fill_host((w.H, w.Is), key(w.seed, layer, T_SHARED_D), w.shared, WEIGHT_SIGMA)


def expert_gate_up(w: Workload, e: int, layer: int = 0):
    """[2I][H] weights of expert e (and bf16 scales [2I/128] for fp8, else None)."""
    k = key(w.seed, layer, T_EXPERT_GU, e)
    if w.expert == FP8:
        return fill_host_fp8(2 * w.I, w.H, k, key(w.seed, layer, T_SCALE_GU, e), WEIGHT_SIGMA)
    return fill_host((2 * w.I, w.H), k, w.expert, WEIGHT_SIGMA), None


def expert_down(w: Workload, e: int, layer: int = 0):
    """[H][I] weights of expert e (and bf16 scales [H/128] for fp8, else None)."""
    k = key(w.seed, layer, T_EXPERT_D, e)
    if w.expert == FP8:
        return fill_host_fp8(w.H, w.I, k, key(w.seed, layer, T_SCALE_D, e), WEIGHT_SIGMA)
    return fill_host((w.H, w.I), k, w.expert, WEIGHT_SIGMA), None


# ---- device fills (torch tensors; torch only provides the memory and stream) ----

def _dev_table(sigma: float, dtype: int, device):
    import torch
    cache = _dev_table.__dict__.setdefault("cache", {})
    ck = (sigma, dtype, str(device))
    if ck not in cache:
        if dtype == FP8:
            codes, _ = fp8_tables(sigma)
            cache[ck] = torch.from_numpy(codes.copy()).to(device)
        else:
            cache[ck] = torch.from_numpy(value_table(sigma, dtype).copy()).to(device)
    return cache[ck]


def fill_device(t, k: int, dtype: int, sigma: float) -> None:
    """Fill a contiguous device tensor with the draws fill_host would produce."""
    import torch
    assert t.is_contiguous()
    table = _dev_table(sigma, dtype, t.device)
    itemsize = {F32: 4, BF16: 2, FP8: 1}[dtype]
    assert t.numel() * t.element_size() % itemsize == 0
    n = t.numel() * t.element_size() // itemsize
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = _dev().synth_dev_fill(t.data_ptr(), n, k, table.data_ptr(), itemsize, stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill failed: hip error {rc}")


def fill_device_fp8(t, rows: int, cols: int, k: int, class_key: int, sigma: float) -> np.ndarray:
    """Fill fp8 codes [rows][cols] on the device; returns the bf16 scale bits [rows/128]."""
    import torch
    assert t.is_contiguous() and t.numel() * t.element_size() == rows * cols
    codes = _dev_table(sigma, FP8, t.device)
    stream = torch.cuda.current_stream(t.device).cuda_stream
    rc = _dev().synth_dev_fill_fp8(t.data_ptr(), rows, cols, k, class_key, codes.data_ptr(), stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill_fp8 failed: hip error {rc}")
    _, scale_bits = fp8_tables(sigma)
    return np.array([scale_bits[scale_class(class_key, g)] for g in range(rows // 128)],
                    dtype=np.uint16)
