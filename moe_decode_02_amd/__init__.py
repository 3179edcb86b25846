"""Thin ctypes binding of libmoedecode (include/moedecode.h).

Argument marshalling only: every step of the MoE decode layer runs in the HIP
kernels of csrc/moedecode.hip. The functions keep the C names; device buffers
may be passed as torch tensors (their data_ptr() is used) or as integer
device addresses, streams as torch streams, raw hipStream_t integers or None
(the default stream). There is no fallback: if the library is not built, the
import of a function fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from functools import lru_cache

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_PATH = os.path.join(_HERE, "libmoedecode.so")
# the ordering-stress build (same source, -DMOE_DEBUG_DELAY; include/moedecode_debug.h)
DELAY_PATH = os.path.join(_HERE, "libmoedecode_delay.so")
SOURCES = [os.path.join(_HERE, "csrc", "moedecode.hip")]
INCLUDE = os.path.join(_ROOT, "include")
HEADER = os.path.join(INCLUDE, "moedecode.h")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED = 0, 1, 2
MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_DEVICE, MOE_ERR_TIMEOUT = 3, 4, 5
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_UF_SHARED_SIDE, MOE_UF_PREFETCH_SIDE = 1, 2

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC", "-shared",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


PROBE_PATH = os.path.join(_HERE, "libmoeprobe.so")
PROBE_SOURCES = [os.path.join(_HERE, "csrc", "bench_probe.hip")]


def build(force: bool = True) -> str:
    """Compile libmoedecode.so, its ordering-stress build and the benchmark's
    probe library in-tree for gfx950 (hipcc cross-compiles without a GPU); the
    compilers run side by side."""
    jobs = []
    for path, srcs, extra in ((LIB_PATH, SOURCES, []), (DELAY_PATH, SOURCES, ["-DMOE_DEBUG_DELAY"]),
                              (PROBE_PATH, PROBE_SOURCES, [])):
        if force or not os.path.exists(path):
            tmp = path + ".tmp"
            cmd = ["/opt/rocm/bin/hipcc", *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-o", tmp, *srcs]
            jobs.append((subprocess.Popen(cmd), cmd, tmp, path))
    for proc, cmd, tmp, path in jobs:
        if proc.wait() != 0:
            raise subprocess.CalledProcessError(proc.returncode, cmd)
        os.replace(tmp, path)
    return LIB_PATH


@lru_cache(maxsize=None)
def probe_lib():
    """Measurement helpers of the benchmark (csrc/bench_probe.hip); not the decode path."""
    if not os.path.exists(PROBE_PATH):
        raise RuntimeError(f"{PROBE_PATH} is not built: run __graft_entry__.build()")
    L = ctypes.CDLL(PROBE_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    L.moe_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
    L.moe_probe_stream_read.restype = ctypes.c_int
    L.moe_probe_stream_read_u.argtypes = [vp, sz, vp, i32, i32, vp]
    L.moe_probe_stream_read_u.restype = ctypes.c_int
    L.moe_probe_copy.argtypes = [vp, vp, sz, i32, vp]
    L.moe_probe_copy.restype = ctypes.c_int
    return L


class moe_layer_desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("expert_inter", ctypes.c_int32),
                ("shared_inter", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("act", ctypes.c_int), ("router", ctypes.c_int), ("expert", ctypes.c_int),
                ("shared", ctypes.c_int), ("scale_group", ctypes.c_int32)]


class moe_layer_weights(ctypes.Structure):
    _fields_ = [("rms_gamma", ctypes.c_void_p), ("router_w", ctypes.c_void_p),
                ("router_bias", ctypes.c_void_p), ("expert_gate_up", ctypes.c_void_p),
                ("expert_down", ctypes.c_void_p), ("expert_gate_up_scale", ctypes.c_void_p),
                ("expert_down_scale", ctypes.c_void_p), ("shared_gate_up", ctypes.c_void_p),
                ("shared_down", ctypes.c_void_p)]


EXPORTS = ("moe_workspace_bytes", "moe_route", "moe_decode_layer", "moe_decode_layer_static", "moe_decode_stack",
           "moe_unfused_workspace_bytes", "moe_decode_layer_unfused",
           "moe_unfused_stack_workspace_bytes", "moe_decode_stack_unfused",
           "moe_check_workspace", "moe_set_watchdog_ticks", "moe_status_string", "moe_last_error")


@lru_cache(maxsize=None)
def lib():
    """The production library."""
    return _bind(LIB_PATH)


@lru_cache(maxsize=None)
def delay_lib():
    """The ordering-stress build: the same entry points plus moe_debug_set_delay."""
    L = _bind(DELAY_PATH)
    L.moe_debug_set_delay.argtypes = [ctypes.c_uint64, ctypes.c_int32]
    L.moe_debug_set_delay.restype = None
    return L


def _bind(path):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() (no fallback exists)")
    L = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    D, Wt = ctypes.POINTER(moe_layer_desc), ctypes.POINTER(moe_layer_weights)
    L.moe_workspace_bytes.argtypes = [D, i32, i32]
    L.moe_workspace_bytes.restype = sz
    L.moe_route.argtypes = [D, Wt, vp, i32, vp, vp, vp, vp, sz, vp]
    L.moe_route.restype = ctypes.c_int
    L.moe_decode_layer.argtypes = [D, Wt, vp, vp, i32, vp, vp, vp, sz, vp]
    L.moe_decode_layer.restype = ctypes.c_int
    L.moe_decode_layer_static.argtypes = [D, Wt, vp, vp, i32, vp, vp, vp]
    L.moe_decode_layer_static.restype = ctypes.c_int
    L.moe_decode_stack.argtypes = [D, Wt, i32, vp, vp, i32, vp, vp, vp, sz, vp]
    L.moe_decode_stack.restype = ctypes.c_int
    L.moe_unfused_workspace_bytes.argtypes = [D, i32]
    L.moe_unfused_workspace_bytes.restype = sz
    L.moe_decode_layer_unfused.argtypes = [D, Wt, vp, vp, i32, vp, vp, vp, sz, vp]
    L.moe_decode_layer_unfused.restype = ctypes.c_int
    L.moe_unfused_stack_workspace_bytes.argtypes = [D, i32, i32]
    L.moe_unfused_stack_workspace_bytes.restype = sz
    L.moe_decode_stack_unfused.argtypes = [D, Wt, i32, vp, vp, i32, vp, vp, vp, sz, vp, vp, ctypes.c_uint32]
    L.moe_decode_stack_unfused.restype = ctypes.c_int
    L.moe_check_workspace.argtypes = [vp, sz, vp]
    L.moe_check_workspace.restype = ctypes.c_int
    L.moe_set_watchdog_ticks.argtypes = [ctypes.c_int64]
    L.moe_set_watchdog_ticks.restype = None
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    L.moe_last_error.argtypes = []
    L.moe_last_error.restype = ctypes.c_char_p
    return L


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{moe_status_string(status)}: {detail}")
        self.status = status


def _addr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(s):
    if s is None:
        return None
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _bytes(t):
    return t.numel() * t.element_size()


def _check(status: int, library=None) -> None:
    if status != MOE_OK:
        raise MoeError(status, (library or lib()).moe_last_error().decode())


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_workspace_bytes(desc: moe_layer_desc, max_tokens: int, num_layers: int = 1) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), max_tokens, num_layers))


def moe_route(desc, weights, x, B, topk_idx, topk_w, logits, ws, ws_bytes=None, stream=None, check=True,
              library=None):
    st = (library or lib()).moe_route(ctypes.byref(desc), ctypes.byref(weights), _addr(x), B, _addr(topk_idx),
                         _addr(topk_w), _addr(logits), _addr(ws),
                         _bytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    if check:
        _check(st, library)
    return st


def moe_decode_layer(desc, weights, x, y, B, topk_idx, topk_w, ws, ws_bytes=None, stream=None, check=True,
                     library=None):
    st = (library or lib()).moe_decode_layer(ctypes.byref(desc), ctypes.byref(weights), _addr(x), _addr(y), B,
                                _addr(topk_idx), _addr(topk_w), _addr(ws),
                                _bytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    if check:
        _check(st, library)
    return st


def moe_decode_layer_static(desc, weights, x, y, B, topk_idx, topk_w, stream=None, check=True, library=None):
    st = (library or lib()).moe_decode_layer_static(ctypes.byref(desc), ctypes.byref(weights), _addr(x), _addr(y), B,
                                                    _addr(topk_idx), _addr(topk_w), _stream(stream))
    if check:
        _check(st, library)
    return st


def moe_decode_stack(desc, layers, x, y, B, topk_idx, topk_w, ws, ws_bytes=None, stream=None, check=True,
                     library=None):
    arr = (moe_layer_weights * len(layers))(*layers)
    st = (library or lib()).moe_decode_stack(ctypes.byref(desc), arr, len(layers), _addr(x), _addr(y), B,
                                _addr(topk_idx), _addr(topk_w), _addr(ws),
                                _bytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    if check:
        _check(st, library)
    return st


def moe_unfused_workspace_bytes(desc: moe_layer_desc, max_tokens: int) -> int:
    return lib().moe_unfused_workspace_bytes(ctypes.byref(desc), max_tokens)


def moe_decode_layer_unfused(desc, weights, x, y, B, topk_idx, topk_w, ws, ws_bytes=None, stream=None, check=True,
                             library=None):
    st = (library or lib()).moe_decode_layer_unfused(ctypes.byref(desc), ctypes.byref(weights), _addr(x), _addr(y), B,
                                        _addr(topk_idx), _addr(topk_w), _addr(ws),
                                        _bytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
    if check:
        _check(st, library)
    return st


def moe_unfused_stack_workspace_bytes(desc: moe_layer_desc, max_tokens: int, num_layers: int) -> int:
    return lib().moe_unfused_stack_workspace_bytes(ctypes.byref(desc), max_tokens, num_layers)


def moe_decode_stack_unfused(desc, layers, x, y, B, topk_idx, topk_w, ws, ws_bytes=None, stream=None,
                             side_stream=None, flags=0, check=True, library=None):
    arr = (moe_layer_weights * len(layers))(*layers)
    st = (library or lib()).moe_decode_stack_unfused(ctypes.byref(desc), arr, len(layers), _addr(x), _addr(y), B,
                                                     _addr(topk_idx), _addr(topk_w), _addr(ws),
                                                     _bytes(ws) if ws_bytes is None else ws_bytes, _stream(stream),
                                                     _stream(side_stream), flags)
    if check:
        _check(st, library)
    return st


def moe_set_watchdog_ticks(ticks: int, library=None) -> None:
    (library or lib()).moe_set_watchdog_ticks(ticks)


def moe_check_workspace(ws, ws_bytes=None, stream=None, library=None) -> int:
    return (library or lib()).moe_check_workspace(_addr(ws), _bytes(ws) if ws_bytes is None else ws_bytes, _stream(stream))
