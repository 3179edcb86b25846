"""Pins of the CPU oracle to things other than itself: the number formats'
definitions (checked against torch's casts), closed forms, brute force on tiny
inputs, invariants of the layer, and an independent float64 torch composition.
"""
import itertools

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth
from helpers import host_layer, max_rel_err, small_workload, to_f64
import torch_ref

F32, BF16, FP8 = synth.F32, synth.BF16, synth.FP8


# ---- number formats -----------------------------------------------------------

def test_bf16_value_exhaustive_vs_torch():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_value(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20, 3.3895313892515355e38,
                  3.39e38, 1e-40, -1e-40, 0.0, -0.0, 65504.0, 2 ** -126], dtype=np.float32)])
    vals = vals[np.isfinite(vals)]
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_round(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, ref)
    assert oracle.bf16_round(1 + 2 ** -8) == 0x3F80  # tie to even: down
    assert oracle.bf16_round(1 + 3 * 2 ** -8) == 0x3F82  # tie to even: up


def test_e4m3_all_codes_vs_torch_and_format():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


# ---- RMSNorm -------------------------------------------------------------------

@pytest.mark.parametrize("c", [1e-3, 0.5, 3.0])
def test_rmsnorm_constant_vector_closed_form(c):
    d = oracle.desc(8, 2, 1, 128, 0, F32, F32, F32, F32, eps=1e-6)
    x = np.full(8, c, np.float32)
    g = np.linspace(0.5, 2.0, 8).astype(np.float32)
    xhat, xact = oracle.rmsnorm(d, x, g)
    cf = float(np.float32(c))
    expect = cf / np.sqrt(cf * cf + float(np.float32(1e-6))) * g.astype(np.float64)
    assert np.allclose(xhat, expect, rtol=1e-7, atol=0)
    assert np.array_equal(xhat, xact)


def test_rmsnorm_vs_torch_rms_norm_bf16():
    w = small_workload(H=512, act=BF16)
    x = synth.x_tokens(w, 1)[0]
    g = synth.gamma(w, random=True)
    d = oracle.desc_of(w)
    xhat, xact = oracle.rmsnorm(d, x, g)
    xt = torch_ref.decode(x, BF16)
    ref = torch.nn.functional.rms_norm(xt, (512,), weight=torch_ref.decode(g, BF16), eps=float(np.float32(1e-6)))
    assert np.allclose(xhat, ref.numpy(), rtol=2e-7, atol=1e-30)
    assert np.array_equal(xact, torch.from_numpy(xhat).to(torch.bfloat16).to(torch.float32).numpy())


# ---- router ---------------------------------------------------------------------

@pytest.mark.parametrize("rdt", [F32, BF16])
def test_router_vs_matmul_with_bias(rdt):
    w = small_workload(H=384, E=24, router=rdt, act=BF16, zipf_s=1.1)
    L = host_layer(w, experts=[])
    d = oracle.desc_of(w)
    xhat = np.random.default_rng(1).standard_normal(384).astype(np.float32)
    got = oracle.router_logits(d, L, xhat)
    ref = (torch_ref.decode(L.router_w, rdt) @ torch.from_numpy(xhat).to(torch.float64)).to(torch.float32)
    ref = ref + torch.from_numpy(L.router_bias)
    assert np.array_equal(got, ref.numpy())  # one fp32 rounding of an fp64 sum, then one fp32 add


def test_router_identity_rows():
    H, E = 64, 16
    d = oracle.desc(H, E, 2, 128, 0, F32, F32, F32, F32)
    Wr = np.zeros((E, H), np.float32)
    cols = np.arange(E) * 3 + 1
    Wr[np.arange(E), cols] = 1.0
    L = oracle.Layer(gamma=np.ones(H, np.float32), router_w=Wr, router_bias=None, gate_up={}, down={})
    xhat = np.random.default_rng(2).standard_normal(H).astype(np.float32)
    assert np.array_equal(oracle.router_logits(d, L, xhat), xhat[cols])


# ---- softmax + top-k + renormalisation ---------------------------------------------

@pytest.mark.parametrize("E", [1, 2, 3, 4, 5, 6])
def test_topk_brute_force_with_ties(E):
    for vals in itertools.product([0.0, 1.0, 2.0], repeat=E):
        lg = np.array(vals, np.float32)
        # rank(e) = #{j : l_j > l_e or (l_j == l_e and j < e)}
        rank = [sum(1 for j in range(E) if lg[j] > lg[e] or (lg[j] == lg[e] and j < e)) for e in range(E)]
        for k in range(1, E + 1):
            d = oracle.desc(8, E, k, 128, 0, F32, F32, F32, F32)
            idx, w = oracle.route(d, lg)
            assert [rank[e] for e in idx] == list(range(k))
            assert abs(float(np.sum(w, dtype=np.float64)) - 1.0) < 1e-6


def test_topk_matches_stable_argsort_and_restricted_softmax():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal(896).astype(np.float32) * 2
    lg[100] = lg[200] = lg[np.argmax(lg)]  # exact ties at the top
    d = oracle.desc(8, 896, 16, 128, 0, F32, F32, F32, F32)
    idx, w = oracle.route(d, lg)
    assert np.array_equal(idx, np.argsort(-lg, kind="stable")[:16])
    ref = scipy.special.softmax(lg[idx].astype(np.float64))
    assert np.allclose(w, ref, rtol=1e-6, atol=0)


def test_route_special_cases():
    lg = np.array([0.5, 3.0, 3.0, 3.0, -1.0], np.float32)
    d1 = oracle.desc(8, 5, 1, 128, 0, F32, F32, F32, F32)
    idx, w = oracle.route(d1, lg)
    assert idx.tolist() == [1] and w.tolist() == [1.0]
    d3 = oracle.desc(8, 5, 3, 128, 0, F32, F32, F32, F32)
    idx, w = oracle.route(d3, lg)
    assert idx.tolist() == [1, 2, 3] and np.allclose(w, 1 / 3, rtol=1e-7)
    d5 = oracle.desc(8, 5, 5, 128, 0, F32, F32, F32, F32)
    idx, w = oracle.route(d5, lg)
    full = scipy.special.softmax(lg.astype(np.float64))
    assert np.allclose(w, full[idx], rtol=1e-6)


# ---- SwiGLU FFN ----------------------------------------------------------------------

@pytest.mark.parametrize("dt", [F32, BF16])
def test_ffn_vs_torch_swiglu(dt):
    w = small_workload(H=320, I=192, Is=0, act=dt, expert=dt, shared=dt)
    d = oracle.desc_of(w)
    gu, _ = synth.expert_gate_up(w, 3)
    dn, _ = synth.expert_down(w, 3)
    xa = torch_ref.round_act(torch.from_numpy(np.random.default_rng(4).standard_normal(320)), dt).numpy().astype(np.float32)
    h, out = oracle.ffn(d, dt, 192, gu, dn, xa)
    ref, href = torch_ref.ffn(torch_ref.decode(gu, dt), torch_ref.decode(dn, dt), torch.from_numpy(xa).to(torch.float64), dt)
    assert np.mean(h == href.numpy().astype(np.float32)) > 0.99
    assert max_rel_err(out, ref.numpy()) < (1e-6 if dt == F32 else 1e-3)


def test_ffn_zero_gate_or_up_gives_zero():
    w = small_workload(H=256, I=128, Is=0)
    d = oracle.desc_of(w)
    gu, _ = synth.expert_gate_up(w, 0)
    dn, _ = synth.expert_down(w, 0)
    xa = np.random.default_rng(6).standard_normal(256).astype(np.float32)
    for rows in (slice(0, 128), slice(128, 256)):
        z = gu.copy()
        z[rows] = 0
        _, out = oracle.ffn(d, F32, 128, z, dn, xa)
        assert not np.any(out)


def test_ffn_fp8_dequant_and_power_of_two_scale():
    w = small_workload(H=256, I=128, Is=0, act=BF16, expert=FP8)
    d = oracle.desc_of(w)
    gu, gus = synth.expert_gate_up(w, 5)
    dn, dns = synth.expert_down(w, 5)
    xa = torch_ref.round_act(torch.from_numpy(np.random.default_rng(7).standard_normal(256)), BF16).numpy().astype(np.float32)
    h, out = oracle.ffn(d, FP8, 128, gu, dn, xa, gus, dns)
    ref, _ = torch_ref.ffn(torch_ref.decode(gu, FP8, gus), torch_ref.decode(dn, FP8, dns), torch.from_numpy(xa).to(torch.float64), BF16)
    assert max_rel_err(out, ref.numpy()) < 1e-3
    # multiplying the down scales of one row group by 2^3 multiplies those outputs by exactly 8
    dns2 = dns.copy()
    dns2[1] = oracle.bf16_round(oracle.bf16_value(int(dns[1])) * 8)
    _, out2 = oracle.ffn(d, FP8, 128, gu, dn, xa, gus, dns2)
    assert np.array_equal(out2[128:256], out[128:256] * 8)
    assert np.array_equal(out2[:128], out[:128])


# ---- the whole layer -----------------------------------------------------------------

def _layer_vs_torch(w, L, x, rtol):
    d = oracle.desc_of(w)
    y, idx, wts, _ = oracle.layer(d, L, x)
    for t in range(x.shape[0]):
        ry, ridx, rw = torch_ref.layer_token(d, L, x[t])
        assert np.array_equal(idx[t], ridx)
        assert np.allclose(wts[t], rw, rtol=1e-6)
        assert max_rel_err(to_f64(y[t], w.act), ry.numpy()) <= rtol
    return y, idx, wts


def test_layer_tiny_f32_vs_torch():
    w = synth.WORKLOADS["tiny_f32"]
    L = host_layer(w)
    x = synth.x_tokens(w, 3)
    _layer_vs_torch(w, L, x, 1e-6)


def test_layer_bf16_zipf_random_gamma_vs_torch():
    w = small_workload(H=512, E=24, k=6, I=128, Is=256, act=BF16, router=F32, expert=BF16, shared=BF16, zipf_s=1.1)
    L = host_layer(w, random_gamma=True)
    x = synth.x_tokens(w, 2)
    _layer_vs_torch(w, L, x, 8e-3)  # one bf16 ulp of the output where a rounding flips


def test_layer_fp8_vs_torch():
    w = small_workload(H=256, E=12, k=3, I=128, Is=128, act=BF16, router=BF16, expert=FP8, shared=BF16)
    L = host_layer(w)
    _layer_vs_torch(w, L, synth.x_tokens(w, 2), 8e-3)


@pytest.mark.parametrize("dt", [F32, BF16])
def test_layer_with_given_selection_vs_torch(dt):
    """A layer evaluated on a selection that is not the top-k (the k-th expert
    swapped with the (k+1)-th, the order reversed): weights are the softmax
    restricted to that selection, the output the torch composition with it."""
    w = small_workload(H=384, E=20, k=5, I=128, Is=256, act=dt, router=F32, expert=dt, shared=dt, zipf_s=1.1)
    L = host_layer(w, random_gamma=True)
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 2)
    y, idx, wts, lg = oracle.layer(d, L, x)
    # the top-k itself gives the layer's result bit for bit
    y0, w0, l0 = oracle.layer_given(d, L, x[0], idx[0])
    assert np.array_equal(y0, y[0]) and np.array_equal(w0, wts[0]) and np.array_equal(l0, lg[0])
    for t in range(2):
        order = np.argsort(-lg[t], kind="stable")
        sel = np.concatenate([order[: w.k - 1], order[w.k: w.k + 1]])[::-1].astype(np.int32)
        yg, wg, _ = oracle.layer_given(d, L, x[t], sel)
        ry, ridx, rw = torch_ref.layer_token(d, L, x[t], given=sel)
        assert np.array_equal(ridx, sel)
        assert np.allclose(wg, rw, rtol=1e-6)
        p = scipy.special.softmax(lg[t].astype(np.float64))
        assert np.allclose(wg, p[sel] / p[sel].sum(), rtol=1e-6)
        assert max_rel_err(to_f64(yg, w.act), ry.numpy()) <= (1e-6 if dt == F32 else 8e-3)
        assert max_rel_err(to_f64(yg, w.act), to_f64(y[t], w.act)) > 1e-4  # a different expert set
    with pytest.raises(RuntimeError, match="invalid"):
        oracle.layer_given(d, L, x[0], np.array([0, 0, 1, 2, 3], np.int32))  # repeated expert
    with pytest.raises(RuntimeError, match="invalid"):
        oracle.layer_given(d, L, x[0], np.array([0, 1, 2, 3, w.E], np.int32))  # out of range


def test_identical_experts_collapse_to_dense_ffn():
    w = small_workload(H=256, E=8, k=3, I=128, Is=128)
    L = host_layer(w)
    for e in range(w.E):
        L.gate_up[e], L.down[e] = L.gate_up[0], L.down[0]
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 4)
    y, idx, _, _ = oracle.layer(d, L, x)
    assert len({tuple(r) for r in idx.tolist()}) > 1  # routing differs between tokens
    for t in range(4):
        xt = torch_ref.decode(x[t], F32)
        xhat = (xt * torch.rsqrt((xt * xt).mean() + float(np.float32(1e-6)))).to(torch.float32).to(torch.float64)
        dense, _ = torch_ref.ffn(torch_ref.decode(L.gate_up[0], F32), torch_ref.decode(L.down[0], F32), xhat, F32)
        sh, _ = torch_ref.ffn(torch_ref.decode(L.shared_gate_up, F32), torch_ref.decode(L.shared_down, F32), xhat, F32)
        assert max_rel_err(y[t], (xt + sh + dense).numpy()) < 1e-6


def test_zero_experts_give_shared_plus_residual():
    w = small_workload(H=256, E=8, k=3, I=128, Is=128)
    L = host_layer(w)
    for e in range(w.E):
        L.gate_up[e] = np.zeros_like(L.gate_up[e])
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 2)
    y, _, _, _ = oracle.layer(d, L, x)
    for t in range(2):
        xt = torch_ref.decode(x[t], F32)
        xhat = (xt * torch.rsqrt((xt * xt).mean() + float(np.float32(1e-6)))).to(torch.float32).to(torch.float64)
        sh, _ = torch_ref.ffn(torch_ref.decode(L.shared_gate_up, F32), torch_ref.decode(L.shared_down, F32), xhat, F32)
        assert np.array_equal(y[t], (xt + sh).to(torch.float32).numpy())


def test_single_expert_is_dense_swiglu_block():
    w = small_workload(H=256, E=1, k=1, I=128, Is=0)
    L = host_layer(w)
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 2)
    y, idx, wts, _ = oracle.layer(d, L, x)
    assert idx.tolist() == [[0], [0]] and wts.tolist() == [[1.0], [1.0]]
    for t in range(2):
        xt = torch_ref.decode(x[t], F32)
        xhat = (xt * torch.rsqrt((xt * xt).mean() + float(np.float32(1e-6)))).to(torch.float32).to(torch.float64)
        dense, _ = torch_ref.ffn(torch_ref.decode(L.gate_up[0], F32), torch_ref.decode(L.down[0], F32), xhat, F32)
        assert np.array_equal(y[t], (xt + dense).to(torch.float32).numpy())


def test_batch_invariance_and_missing_expert():
    w = small_workload(H=256, E=16, k=4, act=BF16, expert=BF16, shared=BF16, router=F32)
    L = host_layer(w)
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 5)
    y, idx, wts, lg = oracle.layer(d, L, x)
    for t in range(5):
        y1, i1, w1, l1 = oracle.layer(d, L, x[t:t + 1])
        assert np.array_equal(y1[0], y[t]) and np.array_equal(i1[0], idx[t]) and np.array_equal(l1[0], lg[t])
    L2 = host_layer(w, experts=[e for e in range(w.E) if e != idx[0, 0]])
    with pytest.raises(RuntimeError, match="no weights"):
        oracle.layer(d, L2, x[:1])


def test_expert_permutation_equivariance():
    w = small_workload(H=256, E=16, k=4, act=BF16, expert=BF16, shared=BF16, router=F32, zipf_s=1.1)
    L = host_layer(w)
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 3)
    y, idx, wts, _ = oracle.layer(d, L, x)
    perm = np.random.default_rng(8).permutation(w.E)  # new id of old expert e is perm[e]
    inv = np.argsort(perm)
    P = oracle.Layer(gamma=L.gamma, router_w=np.ascontiguousarray(L.router_w[inv]),
                     router_bias=np.ascontiguousarray(L.router_bias[inv]),
                     gate_up={int(perm[e]): L.gate_up[e] for e in range(w.E)},
                     down={int(perm[e]): L.down[e] for e in range(w.E)},
                     shared_gate_up=L.shared_gate_up, shared_down=L.shared_down)
    y2, idx2, wts2, _ = oracle.layer(d, P, x)
    assert np.array_equal(y2, y)
    assert np.array_equal(idx2, perm[idx]) and np.array_equal(wts2, wts)


def test_stack_is_successive_layers():
    w = small_workload(H=256, E=16, k=4, act=BF16, expert=FP8, shared=BF16, router=BF16, layers=3)
    Ls = [host_layer(w, layer=l) for l in range(3)]
    d = oracle.desc_of(w)
    x = synth.x_tokens(w, 2)
    y, idx, wts, lg = oracle.stack(d, Ls, x)
    cur = x
    for l in range(3):
        cur, i, ww, g = oracle.layer(d, Ls[l], cur)
        assert np.array_equal(i, idx[l]) and np.array_equal(ww, wts[l]) and np.array_equal(g, lg[l])
    assert np.array_equal(cur, y)
    y1, i1, _, _ = oracle.stack(d, Ls[:1], x)
    y0, i0, _, _ = oracle.layer(d, Ls[0], x)
    assert np.array_equal(y1, y0) and np.array_equal(i1[0], i0)
