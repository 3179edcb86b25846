"""GPU parity of the multi-launch path (moe_decode_layer_unfused, eleven
kernel launches with every intermediate in device memory) against the CPU oracle,
with the bars of the fused kernel: expert indices bit-exact on tokens whose
router margin is >= 1e-3, routing weights within 1e-4 relative, outputs within
max relative error 2e-2 (bf16 / fp8 weights) or 1e-4 (fp32)."""
import numpy as np
import pytest
import torch

import moe_decode_02_amd as md
import oracle
import synth
from helpers import (add_experts, draw_tokens_with_margin, drop_experts, host_layer, margin, max_rel_err,
                     oracle_layer_tokens, oracle_logits_tokens, pmap, small_workload, to_f64, valid_selection)
from synth.device import DeviceLayer, act_tensor, desc_of, to_device, to_host

pytestmark = pytest.mark.gpu

TOL = {synth.F32: 1e-4, synth.BF16: 2e-2}


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    md.build(force=False)
    synth.build(force=False, device=True)
    md.lib()
    return torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)


def unfused_layer(w, dl, x, B, dev):
    d = desc_of(w)
    xd = to_device(x, dev)
    yd = act_tensor(w, B, dev)
    idx = torch.full((B, w.k), -1, dtype=torch.int32, device=dev)
    wts = torch.zeros((B, w.k), dtype=torch.float32, device=dev)
    ws = torch.empty(md.moe_unfused_workspace_bytes(d, B), dtype=torch.uint8, device=dev)
    ws.fill_(0xA5)  # no zero fill needed: every call writes what it reads
    md.moe_decode_layer_unfused(d, dl.weights, xd, yd, B, idx, wts, ws)
    torch.cuda.synchronize()
    return {"y": to_host(yd), "idx": idx.cpu().numpy(), "w": wts.cpu().numpy()}


def parity(w, B, dev, random_gamma=False):
    """Every token of a B-token batch against the oracle; unselected experts
    hold NaN, so a wrong gather poisons the output."""
    Lh = host_layer(w, experts=[], random_gamma=random_gamma)
    x, _ = draw_tokens_with_margin(w, B, [Lh])
    d = oracle.desc_of(w)
    idx_r = np.zeros((B, w.k), np.int32)
    for t in range(B):
        xhat, _ = oracle.rmsnorm(d, x[t], Lh.gamma)
        idx_r[t], _ = oracle.route(d, oracle.router_logits(d, Lh, xhat))
    tok = list(range(B))
    add_experts(w, Lh, idx_r)
    y_ref, idx_o, w_o, _ = oracle_layer_tokens(d, Lh, x)
    log(f"gpu unfused: {w.name} B={B}")
    dl = DeviceLayer(w, device=dev, experts=idx_r, random_gamma=random_gamma)
    got = unfused_layer(w, dl, x, B, dev)
    assert np.array_equal(got["idx"], idx_r)
    errs = []
    for j, t in enumerate(tok):
        assert np.array_equal(got["idx"][t], idx_o[j])
        assert np.allclose(got["w"][t], w_o[j], rtol=1e-4, atol=1e-6), t
        errs.append(max_rel_err(to_f64(got["y"][t], w.act), to_f64(y_ref[j], w.act)))
        assert errs[-1] <= TOL[w.act], (t, errs[-1])
    assert np.all(np.isfinite(to_f64(got["y"], w.act)))
    del dl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log(f"  max rel err {max(errs):.2e}")
    return max(errs)


@pytest.mark.parametrize("B", [1, 3, 64])
def test_unfused_tiny_f32(dev, B):
    parity(synth.WORKLOADS["tiny_f32"], B, dev)


def test_unfused_small_bf16_zipf_random_gamma(dev):
    w = small_workload(name="small_bf16", H=512, E=40, k=6, I=256, Is=512, act=synth.BF16, router=synth.F32,
                       expert=synth.BF16, shared=synth.BF16, zipf_s=1.1, seed=21)
    for B in (1, 5, 33):
        parity(w, B, dev, random_gamma=True)


def test_unfused_fp8_bf16_router(dev):
    w = small_workload(name="small_fp8", H=1024, E=24, k=4, I=256, Is=256, act=synth.BF16, router=synth.BF16,
                       expert=synth.FP8, shared=synth.BF16, seed=61)
    for B in (1, 7):
        parity(w, B, dev)


def test_unfused_k3_b1(dev):
    parity(synth.WORKLOADS["k3_b1"], 1, dev)


def test_unfused_k3_b8(dev):
    parity(synth.WORKLOADS["k3_b8"], 8, dev)


def _unfused_chain(w, dls, x, B, dev):
    """The layers one call of moe_decode_layer_unfused at a time, on one stream:
    (input of each layer, output, idx [L][B][k], w [L][B][k])."""
    ins, idxs, ws_ = [x], [], []
    for dl in dls:
        got = unfused_layer(w, dl, ins[-1], B, dev)
        ins.append(got["y"])
        idxs.append(got["idx"])
        ws_.append(got["w"])
    return ins[:-1], ins[-1], np.stack(idxs), np.stack(ws_)


def _unfused_stack(w, dls, x, B, dev, flags, side):
    d = desc_of(w)
    L = len(dls)
    xd = to_device(x, dev)
    yd = act_tensor(w, B, dev)
    idx = torch.full((L, B, w.k), -1, dtype=torch.int32, device=dev)
    wts = torch.zeros((L, B, w.k), dtype=torch.float32, device=dev)
    ws = torch.empty(md.moe_unfused_stack_workspace_bytes(d, B, L), dtype=torch.uint8, device=dev)
    ws.fill_(0xA5)
    md.moe_decode_stack_unfused(d, [dl.weights for dl in dls], xd, yd, B, idx, wts, ws,
                                stream=torch.cuda.current_stream(dev), side_stream=side, flags=flags)
    torch.cuda.synchronize()
    return to_host(yd), idx.cpu().numpy(), wts.cpu().numpy()


@pytest.mark.parametrize("name,B,layers,check_oracle", [("tiny_f32", 3, 3, True), ("k3_stack4_fp8", 2, 4, True),
                                                          ("k3_stack4_fp8", 16, 4, False)])
def test_unfused_stack_side_streams(dev, name, B, layers, check_oracle):
    """moe_decode_stack_unfused, with the shared expert and / or the next
    layer's prefetch on a second stream (every flag set, each run twice), is
    bit-identical to the same layers chained through moe_decode_layer_unfused
    on one stream: the same kernels on the same data, ordered by events. Each
    layer of the chain is checked against the oracle teacher-forced (the
    oracle's layer l on the GPU's input of layer l), every token, with the
    fused stack's bar: routing bit-exact where the margin is >= 1e-3, else a
    valid near-tie selection checked on the oracle evaluated on it."""
    w = synth.WORKLOADS[name]
    log(f"gpu unfused stack: {name} B={B} layers={layers}")
    dls = [DeviceLayer(w, layer=l, device=dev) for l in range(layers)]
    hosts = [host_layer(w, experts=[], layer=l) for l in range(layers)]
    x, _ = draw_tokens_with_margin(w, B, [hosts[0]])
    ins, y0, i0, w0 = _unfused_chain(w, dls, x, B, dev)
    assert np.all(np.isfinite(to_f64(y0, w.act)))
    side = torch.cuda.Stream(device=dev)  # default priority, as the header asks
    for flags in (0, md.MOE_UF_SHARED_SIDE, md.MOE_UF_PREFETCH_SIDE, md.MOE_UF_SHARED_SIDE | md.MOE_UF_PREFETCH_SIDE):
        for rep in range(2):
            y, i, ww = _unfused_stack(w, dls, x, B, dev, flags, side if flags else None)
            assert np.array_equal(i, i0), (flags, rep)
            assert np.array_equal(ww.view(np.uint32), w0.view(np.uint32)), (flags, rep)
            assert np.array_equal(y, y0), (flags, rep)
    log(f"  flags 0..3, twice each: bit-identical to the chained single-stream layers")
    if check_oracle:
        d = oracle.desc_of(w)
        tol = TOL[w.act]
        for l in range(layers):
            Lh = hosts[l]
            lg = oracle_logits_tokens(d, Lh, ins[l])
            add_experts(w, Lh, np.concatenate([i0[l].ravel(),
                                               np.stack([oracle.route(d, lg[t])[0] for t in range(B)]).ravel()]),
                        layer=l)

            def check(t):
                xt = np.ascontiguousarray(ins[l][t])
                if margin(lg[t], w.k) >= 1e-3:
                    yr, ir, wr, _ = oracle.layer(d, Lh, xt[None, :])
                    yr, wr = yr[0], wr[0]
                    assert np.array_equal(i0[l, t], ir[0]), (t, l)
                else:
                    assert valid_selection(lg[t], i0[l, t], w.k, 4e-4), (t, l)
                    yr, wr, _ = oracle.layer_given(d, Lh, xt, i0[l, t])
                assert np.allclose(w0[l, t], wr, rtol=1e-4, atol=1e-6), (t, l)
                out = ins[l + 1][t] if l + 1 < layers else y0[t]
                err = max_rel_err(to_f64(out, w.act), to_f64(yr, w.act))
                assert err <= tol, (t, l, err)
                return err

            errs = pmap(check, range(B))
            log(f"  layer {l} teacher-forced: max rel err {max(errs):.2e}")
            drop_experts(Lh)
    del dls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
