"""C ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented statuses before
any HIP call."""
import ctypes
import re

import pytest

import moe_decode_02_amd as md
import synth
from synth.device import desc_of


@pytest.fixture(scope="module")
def lib():
    md.build(force=False)
    return md.lib()


def header_functions():
    text = open(md.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(lib):
    names = header_functions()
    assert set(names) == set(md.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_stress_build_exports(lib):
    """The ordering-stress build exports every entry point of moedecode.h plus
    the call of moedecode_debug.h; the production library does not export it."""
    md.build(force=False)
    L = md.delay_lib()
    for n in header_functions():
        assert hasattr(L, n), n
    text = re.sub(r"/\*.*?\*/", "", open(md.HEADER.replace("moedecode.h", "moedecode_debug.h")).read(), flags=re.S)
    dbg = sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))
    assert dbg == ["moe_debug_set_delay"] and hasattr(L, dbg[0])
    with pytest.raises(AttributeError):
        getattr(lib, "moe_debug_set_delay")


def test_status_strings(lib):
    for code, name in [(0, "MOE_OK"), (1, "MOE_ERR_INVALID_ARGUMENT"), (2, "MOE_ERR_UNSUPPORTED"),
                       (3, "MOE_ERR_WORKSPACE_TOO_SMALL"), (4, "MOE_ERR_DEVICE"), (5, "MOE_ERR_TIMEOUT")]:
        assert md.moe_status_string(code) == name


def test_workspace_bytes_and_envelope(lib):
    d = desc_of(synth.WORKLOADS["k3_b1"])
    n1 = md.moe_workspace_bytes(d, 1, 1)
    n64 = md.moe_workspace_bytes(d, 64, 1)
    n64s = md.moe_workspace_bytes(d, 64, 4)
    assert 0 < n1 < n64 < n64s
    assert md.moe_workspace_bytes(d, 0, 1) == 0
    assert md.moe_workspace_bytes(d, 65, 1) == 0
    assert md.moe_workspace_bytes(d, 1, 9) == 0
    bad = desc_of(synth.WORKLOADS["k3_b1"])
    bad.hidden = 7000
    assert md.moe_workspace_bytes(bad, 1, 1) == 0
    bad = desc_of(synth.WORKLOADS["k3_b1"])
    bad.act = md.MOE_F32  # fp32 activations with bf16 experts: not a supported set
    assert md.moe_workspace_bytes(bad, 1, 1) == 0


@pytest.mark.parametrize("field,value,ok", [
    ("hidden", 4224, True), ("hidden", 128, True), ("hidden", 16384, True), ("hidden", 16512, False),
    ("hidden", 4160, False), ("expert_inter", 384, True), ("expert_inter", 4224, False),
    ("expert_inter", 192, False), ("shared_inter", 0, True), ("shared_inter", 384, True),
    ("shared_inter", 8192, True), ("shared_inter", 8320, False), ("shared_inter", 200, False),
    ("top_k", 32, True), ("top_k", 33, False), ("num_experts", 1024, True), ("num_experts", 1025, False),
])
def test_envelope_edges_abi(lib, field, value, ok):
    """The envelope: H, I and Is multiples of 128 (Is need not be a multiple of
    I), H <= 16384, I <= 4096, Is <= 8192, k <= 32, E <= 1024."""
    d = desc_of(synth.WORKLOADS["k3_b1"])
    setattr(d, field, value)
    assert (md.moe_workspace_bytes(d, 4, 1) > 0) == ok
    assert (md.moe_unfused_workspace_bytes(d, 4) > 0) == ok


FAKE = 1 << 40  # a 16-byte aligned address; validation fails before anything touches it


def _weights():
    return md.moe_layer_weights(FAKE, FAKE, None, FAKE, FAKE, None, None, FAKE, FAKE)


@pytest.mark.parametrize("case,status", [
    ("batch0", md.MOE_ERR_UNSUPPORTED), ("batch65", md.MOE_ERR_UNSUPPORTED),
    ("misaligned_x", md.MOE_ERR_INVALID_ARGUMENT), ("null_x", md.MOE_ERR_INVALID_ARGUMENT),
    ("small_ws", md.MOE_ERR_WORKSPACE_TOO_SMALL), ("partial_overlap", md.MOE_ERR_INVALID_ARGUMENT),
    ("bad_hidden", md.MOE_ERR_UNSUPPORTED), ("fp8_no_scales", md.MOE_ERR_INVALID_ARGUMENT),
    ("k_too_big", md.MOE_ERR_UNSUPPORTED), ("null_desc", md.MOE_ERR_INVALID_ARGUMENT),
])
@pytest.mark.parametrize("entry", ["fused", "unfused"])
def test_layer_argument_errors(lib, case, status, entry):
    w = synth.WORKLOADS["k3_b1"]
    d = desc_of(w)
    wt = _weights()
    B, x, y = 1, FAKE + (1 << 30), FAKE + (2 << 30)
    ws = FAKE + (3 << 30)
    wsb = md.moe_workspace_bytes(d, 64, 1) if entry == "fused" else md.moe_unfused_workspace_bytes(d, 64)
    if case == "batch0":
        B = 0
    elif case == "batch65":
        B = 65
    elif case == "misaligned_x":
        x += 2
    elif case == "null_x":
        x = None
    elif case == "small_ws":
        wsb = 1024
    elif case == "partial_overlap":
        y = x + 16
    elif case == "bad_hidden":
        d.hidden = 7000
    elif case == "fp8_no_scales":
        d = desc_of(synth.WORKLOADS["k3_stack4_fp8"])
    elif case == "k_too_big":
        d.top_k = 33
    fused = entry == "fused"
    if case == "null_desc":
        fn = lib.moe_decode_layer if fused else lib.moe_decode_layer_unfused
        st = fn(None, ctypes.byref(wt), x, y, B, None, None, ws, wsb, None)
    else:
        fn = md.moe_decode_layer if fused else md.moe_decode_layer_unfused
        st = fn(d, wt, x, y, B, None, None, ws, wsb, check=False)
    assert st == status, (case, md.moe_last_error())
    assert md.moe_last_error()


def test_route_and_stack_argument_errors(lib):
    w = synth.WORKLOADS["k3_b1"]
    d = desc_of(w)
    wt = _weights()
    ws, wsb = FAKE + (3 << 30), md.moe_workspace_bytes(d, 64, 4)
    x = FAKE + (1 << 30)
    assert md.moe_route(d, wt, x, 1, None, FAKE, None, ws, wsb, check=False) == md.MOE_ERR_INVALID_ARGUMENT
    assert md.moe_decode_stack(d, [wt] * 9, x, x, 1, None, None, ws, wsb, check=False) == md.MOE_ERR_UNSUPPORTED
    assert md.moe_decode_stack(d, [wt, wt], x, x, 1, None, None, ws, 4096, check=False) == \
        md.MOE_ERR_WORKSPACE_TOO_SMALL
    assert md.moe_check_workspace(None, 0) == md.MOE_ERR_INVALID_ARGUMENT


def test_unfused_workspace_bytes(lib):
    d = desc_of(synth.WORKLOADS["k3_b1"])
    n1, n64 = md.moe_unfused_workspace_bytes(d, 1), md.moe_unfused_workspace_bytes(d, 64)
    # at least the fp32 gate/up and down outputs of every (token, expert) pair
    assert n64 >= 64 * 16 * (2 * 1024 + 7168) * 4 > n1 > 0
    assert md.moe_unfused_workspace_bytes(d, 0) == 0 and md.moe_unfused_workspace_bytes(d, 65) == 0


def test_unfused_stack_workspace_and_argument_errors(lib):
    """moe_decode_stack_unfused: workspace size, layer count, flag and side-stream
    checks, all returned before any HIP call."""
    d = desc_of(synth.WORKLOADS["k3_b1"])
    wt = _weights()
    one = md.moe_unfused_stack_workspace_bytes(d, 8, 1)
    assert one == md.moe_unfused_workspace_bytes(d, 8)
    four = md.moe_unfused_stack_workspace_bytes(d, 8, 4)
    assert four >= one + 2 * 8 * 7168 * 2  # two bf16 [B][H] buffers between layers
    assert md.moe_unfused_stack_workspace_bytes(d, 8, 0) == 0 and md.moe_unfused_stack_workspace_bytes(d, 8, 9) == 0
    x, ws = FAKE + (1 << 30), FAKE + (3 << 30)
    side = FAKE + (5 << 30)  # never used: every case fails validation first

    def call(layers, wsb, side_stream, flags):
        return md.moe_decode_stack_unfused(d, layers, x, x, 8, None, None, ws, wsb, side_stream=side_stream,
                                           flags=flags, check=False)

    assert call([wt] * 9, four, None, 0) == md.MOE_ERR_UNSUPPORTED
    assert call([wt] * 4, one, None, 0) == md.MOE_ERR_WORKSPACE_TOO_SMALL
    assert call([wt] * 4, four, None, md.MOE_UF_SHARED_SIDE) == md.MOE_ERR_INVALID_ARGUMENT
    assert call([wt] * 4, four, None, md.MOE_UF_PREFETCH_SIDE) == md.MOE_ERR_INVALID_ARGUMENT
    assert call([wt] * 4, four, side, 4) == md.MOE_ERR_INVALID_ARGUMENT
    assert "flags" in md.moe_last_error()
    assert lib.moe_decode_stack_unfused(ctypes.byref(d), None, 1, x, x, 8, None, None, ws, four, None, None, 0) == \
        md.MOE_ERR_INVALID_ARGUMENT
