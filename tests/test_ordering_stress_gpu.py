"""Ordering stress on the GPU.

The ordering-stress build of the library (libmoedecode_delay.so, the same
source compiled with -DMOE_DEBUG_DELAY; include/moedecode_debug.h) injects
seeded pauses of up to ~55 us before barrier arrivals, published router
logits, expert gate/up tasks, output-row units, routing and the combine,
permutes which hardware workgroup takes which work share, and can run a grid
smaller than one workgroup per CU. Fixed-timing kernel tests can miss
ordering bugs that long runs expose (aiposthub.com article, section on how
vLLM verifies AI-written kernels); these runs change the timing and the
placement of every share while the work itself stays the same.

Bars, per case: the undelayed run of the stress build at the full grid is
bit-identical to the production library; every delayed run (3 seeds, at the
full grid and at 120 and 255 workgroups) is bit-identical to the undelayed
run at its grid, with no watchdog stop; the undelayed results match the
oracle (layers: every token at the parity bar; the stack: the oracle's own
stack, routing equal at every layer and the composed bar).
"""
import numpy as np
import pytest
import torch

import moe_decode_02_amd as md
import oracle
import synth
from helpers import (add_experts, draw_tokens_with_margin, drop_experts, host_layer, max_rel_err,
                     oracle_layer_tokens, pmap, to_f64)
from synth.device import DeviceLayer, act_tensor, desc_of, to_device, to_host, workspace

pytestmark = pytest.mark.gpu

SEEDS = [0x9E3779B97F4A7C15 * s & 0xFFFFFFFFFFFFFFFF for s in (1, 2, 3)]
GRIDS = [0, 120, 255]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    md.lib()
    md.delay_lib()
    return torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)


def run(w, layers, x, B, dev, library):
    d = desc_of(w)
    L = len(layers)
    xd, yd = to_device(x, dev), act_tensor(w, B, dev)
    idx = torch.full((L, B, w.k), -7, dtype=torch.int32, device=dev)
    wts = torch.zeros((L, B, w.k), dtype=torch.float32, device=dev)
    ws = workspace(d, B, L, dev)
    md.moe_decode_stack(d, [dl.weights for dl in layers], xd, yd, B, idx, wts, ws, library=library)
    torch.cuda.synchronize()
    assert md.moe_check_workspace(ws, library=library) == md.MOE_OK, "watchdog stop"
    return to_host(yd), idx.cpu().numpy(), wts.cpu().numpy()


def same(a, b):
    return all(np.array_equal(u, v) for u, v in zip(a, b))


def stress(w, layers, x, B, dev):
    """Production run, then the stress build undelayed and delayed at every
    grid; returns the production result."""
    lib_d = md.delay_lib()
    prod = run(w, layers, x, B, dev, md.lib())
    base = {}
    try:
        for g in GRIDS:
            lib_d.moe_debug_set_delay(0, g)
            base[g] = run(w, layers, x, B, dev, lib_d)
            if g == 0:
                assert same(base[0], prod), "stress build, undelayed, differs from the production library"
            for s in SEEDS:
                log(f"stress {w.name} B={B} layers={len(layers)} grid={g or 'per-CU'} seed={s:#x}")
                lib_d.moe_debug_set_delay(s, g)
                got = run(w, layers, x, B, dev, lib_d)
                assert same(got, base[g]), (g, s)
    finally:
        lib_d.moe_debug_set_delay(0, 0)
    log(f"stress {w.name} B={B}: every delayed run bit-identical; grids give identical bits: "
        f"{all(same(base[g], base[0]) for g in GRIDS)}")
    return prod


@pytest.mark.parametrize("name,B", [("k3_b1", 1), ("k3_b1", 4), ("k3_b8", 8), ("tiny_f32", 2), ("tiny_f32", 9)])
def test_layer_under_delays(dev, name, B):
    w = synth.WORKLOADS[name]
    Lh = host_layer(w, experts=[])
    x, _ = draw_tokens_with_margin(w, B, [Lh])
    dl = DeviceLayer(w, device=dev)
    y, idx, wts = stress(w, [dl], x, B, dev)
    d = oracle.desc_of(w)
    lg = np.stack([oracle.router_logits(d, Lh, oracle.rmsnorm(d, x[t], Lh.gamma)[0]) for t in range(B)])
    add_experts(w, Lh, [oracle.route(d, lg[t])[0] for t in range(B)])
    y_ref, idx_ref, w_ref, _ = oracle_layer_tokens(d, Lh, x)
    assert np.array_equal(idx[0], idx_ref)
    assert np.allclose(wts[0], w_ref, rtol=1e-4, atol=1e-6)
    tol = 1e-4 if w.act == synth.F32 else 2e-2
    errs = [max_rel_err(to_f64(y[t], w.act), to_f64(y_ref[t], w.act)) for t in range(B)]
    assert max(errs) <= tol, errs
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,B,L", [("k3_stack4_fp8", 2, 4), ("tiny_f32", 3, 3)])
def test_stack_under_delays(dev, name, B, L):
    w = synth.WORKLOADS[name]
    hosts = [host_layer(w, experts=[], layer=l % w.layers) for l in range(L)]
    x, _ = draw_tokens_with_margin(w, B, [hosts[0]])
    dls = [DeviceLayer(w, layer=l % w.layers, device=dev) for l in range(L)]
    y, idx, wts = stress(w, dls, x, B, dev)
    # the oracle's own stack, layer by layer with the experts each layer needs
    d = oracle.desc_of(w)
    cur = x.copy()
    agree = np.ones(B, bool)
    for l in range(L):
        Lh = hosts[l]
        lg = np.stack([oracle.router_logits(d, Lh, oracle.rmsnorm(d, cur[t], Lh.gamma)[0]) for t in range(B)])
        add_experts(w, Lh, [oracle.route(d, lg[t])[0] for t in range(B)], layer=l % w.layers)
        cur, i_r, w_r, _ = oracle_layer_tokens(d, Lh, cur)
        agree &= np.all(i_r == idx[l], axis=1)
        drop_experts(Lh)
    errs = [max_rel_err(to_f64(y[t], w.act), to_f64(cur[t], w.act)) for t in range(B)]
    log(f"stack {name} B={B} L={L}: routing equal to the oracle's at every layer for {int(agree.sum())}/{B} "
        f"tokens, free-running max rel err {max(errs):.2e}")
    assert agree[0]  # layer 0 is drawn with margin; deeper near-ties may legitimately differ
    tol = 1e-4 if w.act == synth.F32 else 2e-2
    for t in range(B):
        if agree[t]:
            assert errs[t] <= L * tol, (t, errs[t])
    del dls
    torch.cuda.empty_cache()
