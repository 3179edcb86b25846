"""Pins of the seeded input generator (no GPU)."""
import numpy as np
import scipy.special
import torch

import synth


def test_normal_table_matches_ndtri():
    z = synth.normal_table()
    p = (np.arange(synth.TABLE_SIZE) + 0.5) / synth.TABLE_SIZE
    assert np.max(np.abs(z - scipy.special.ndtri(p))) < 1e-9
    assert np.array_equal(z, -z[::-1])
    assert np.all(np.diff(z) > 0)


def test_value_tables_are_torch_casts():
    z = synth.normal_table()
    f = (z * 0.02).astype(np.float32)
    assert np.array_equal(synth.value_table(0.02, synth.F32), f)
    bf = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.value_table(0.02, synth.BF16), bf)


def test_fp8_code_tables_and_scales():
    z = synth.normal_table()
    codes, scales = synth.fp8_tables(0.02)
    for c in range(4):
        s = torch.from_numpy(scales[c:c + 1].view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).item()
        assert abs(s / (0.02 * z[-1] / 448 * (1 + c / 4)) - 1) < 2 ** -8
        v = torch.from_numpy(z * 0.02 / s)
        ref = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.mean(ref == codes[c]) > 0.999  # torch rounds via fp32 first: rare double-rounding ties
        deq = torch.from_numpy(codes[c].copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s
        assert np.max(np.abs(deq - z * 0.02)) <= 0.02 * z[-1] * (1 + c / 4) / 16  # within half an fp8 step of the top binade


def test_draws_are_deterministic_and_streams_distinct():
    k = synth.key(1, 0, synth.T_EXPERT_GU, 7)
    a = synth.fill_host((1000,), k, synth.BF16, 0.02)
    b = synth.fill_host((1000,), k, synth.BF16, 0.02)
    assert np.array_equal(a, b)
    others = [synth.key(2, 0, synth.T_EXPERT_GU, 7), synth.key(1, 1, synth.T_EXPERT_GU, 7),
              synth.key(1, 0, synth.T_EXPERT_D, 7), synth.key(1, 0, synth.T_EXPERT_GU, 8),
              synth.key(1, 0, synth.T_EXPERT_GU, 7, 1)]
    assert len(set(others + [k])) == 6
    for o in others:
        assert np.mean(synth.fill_host((1000,), o, synth.BF16, 0.02) == a) < 0.05
    # the fill is element-wise: a prefix of a longer fill equals the shorter fill
    assert np.array_equal(synth.fill_host((5003,), k, synth.BF16, 0.02)[:1000], a)
    table = synth.value_table(0.02, synth.BF16)
    assert all(table[synth.index(k, i)] == a[i] for i in range(64))


def test_moments_of_weight_draws():
    v = synth.fill_host((1 << 20,), synth.key(9, 0, synth.T_ROUTER), synth.F32, 0.02).astype(np.float64)
    assert abs(v.mean()) < 0.02 * 5e-3
    assert abs(v.std() / 0.02 - 1) < 5e-3
    idx = np.array([synth.index(synth.key(9, 0, synth.T_ROUTER), i) for i in range(40000)])
    hist = np.bincount(idx >> 10, minlength=16)
    assert hist.min() > 2200 and hist.max() < 2800  # 16 bins of 2500 expected


def test_zipf_bias_is_log_of_normalised_zipf():
    b = synth.zipf_bias(3, 896, 1.1)
    p = np.exp(b.astype(np.float64))
    assert abs(p.sum() - 1) < 1e-5
    ranks = np.arange(1, 897, dtype=np.float64)
    ref = ranks ** -1.1 / np.sum(ranks ** -1.1)
    assert np.allclose(np.sort(p)[::-1], ref, rtol=1e-5)
    assert not np.all(np.diff(p) <= 0)  # permuted, not sorted by expert id


def test_fp8_fill_uses_scale_class_per_group():
    codes, scales = synth.fill_host_fp8(512, 64, synth.key(4, 0, synth.T_EXPERT_D, 1),
                                        synth.key(4, 0, synth.T_SCALE_D, 1), 0.02)
    _, sb = synth.fp8_tables(0.02)
    classes = [synth.scale_class(synth.key(4, 0, synth.T_SCALE_D, 1), g) for g in range(4)]
    assert scales.tolist() == [int(sb[c]) for c in classes]
    assert codes.shape == (512, 64)


def test_workload_shapes():
    w = synth.WORKLOADS["k3_b1"]
    assert (w.H, w.E, w.k, w.I, w.Is) == (7168, 896, 16, 1024, 2048)
    x = synth.x_tokens(w, 2)
    assert x.shape == (2, 7168) and x.dtype == np.uint16
    t = synth.WORKLOADS["tiny_f32"]
    assert synth.router_w(t).shape == (32, 256) and synth.router_w(t).dtype == np.float32


def test_spec_verify_tokens():
    """Verify-step tokens: request r's base token is an N(0, 1) draw stored in
    bf16; each of its 7 drafts is bf16(base + 0.5 z) with z drawn under its own
    key, so a draft correlates with its base (~1/sqrt(1.25)) and requests are
    independent; a draft's redraw changes only that draft."""
    w = synth.WORKLOADS["k3_spec_verify"]
    g = 1 + w.spec_drafts
    x = synth.x_tokens(w, 2 * g)
    f = lambda a: (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    base = synth.fill_host((w.H,), synth.key(w.seed, 0, synth.T_X, 0), synth.F32, 1.0)
    assert np.array_equal(x[0], synth._bf16_bits_of(base))
    z = synth.fill_host((w.H,), synth.key(w.seed, 0, synth.T_SPEC, 3), synth.F32, w.spec_delta)
    assert np.array_equal(x[3], synth._bf16_bits_of(base + z))
    c_in = np.corrcoef(f(x[0]), f(x[5]))[0, 1]
    c_out = np.corrcoef(f(x[0]), f(x[g]))[0, 1]
    assert abs(c_in - 1 / np.sqrt(1 + w.spec_delta ** 2)) < 0.02 and abs(c_out) < 0.05
    att = np.zeros(2 * g, np.int64)
    att[3] = 1
    y = synth.x_tokens(w, 2 * g, att)
    assert not np.array_equal(y[3], x[3]) and np.array_equal(np.delete(y, 3, 0), np.delete(x, 3, 0))
    att[:] = 0
    att[g] = 1  # the second request's base: all its tokens move
    y = synth.x_tokens(w, 2 * g, att)
    assert np.array_equal(y[:g], x[:g]) and not any(np.array_equal(y[t], x[t]) for t in range(g, 2 * g))
