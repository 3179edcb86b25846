"""Shared test helpers: host layers from the seeded generator, the error metric,
and the router-margin redraw. Imports the oracle (test infrastructure)."""
import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth


def small_workload(name="small", H=256, E=16, k=4, I=128, Is=128, act=synth.F32, router=synth.F32,
                   expert=synth.F32, shared=synth.F32, seed=11, B=1, zipf_s=0.0, layers=1):
    return synth.Workload(name, H=H, E=E, k=k, I=I, Is=Is, act=act, router=router, expert=expert,
                          shared=shared, seed=seed, batches=(B,), zipf_s=zipf_s, layers=layers)


def host_layer(w, experts=None, layer=0, random_gamma=False) -> oracle.Layer:
    """Host weights of one layer of workload w; experts = ids to materialise (default all)."""
    ids = range(w.E) if experts is None else sorted(set(int(e) for e in experts))
    L = oracle.Layer(gamma=synth.gamma(w, random=random_gamma, layer=layer),
                     router_w=synth.router_w(w, layer), router_bias=synth.router_bias(w, layer),
                     gate_up={}, down={})
    for e in ids:
        gu, gus = synth.expert_gate_up(w, e, layer)
        dn, dns = synth.expert_down(w, e, layer)
        L.gate_up[e], L.down[e] = gu, dn
        if gus is not None:
            L.gate_up_scale[e], L.down_scale[e] = gus, dns
    if w.Is > 0:
        L.shared_gate_up = synth.shared_gate_up(w, layer)
        L.shared_down = synth.shared_down(w, layer)
    return L


def to_f64(a: np.ndarray, act: int) -> np.ndarray:
    if act == synth.BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def max_rel_err(a: np.ndarray, r: np.ndarray) -> float:
    """max_i |a_i - r_i| / max(|r_i|, rms(r)): elementwise relative above the RMS
    of the reference, RMS-normalised absolute below it."""
    a = np.asarray(a, np.float64).ravel()
    r = np.asarray(r, np.float64).ravel()
    if r.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(r * r)))
    den = np.maximum(np.abs(r), rms if rms > 0 else 1.0)
    return float(np.max(np.abs(a - r) / den))


def margin(logits: np.ndarray, k: int) -> float:
    """Gap between the k-th and (k+1)-th largest logit (inf when k == E)."""
    s = np.sort(np.asarray(logits, np.float64))[::-1]
    return float("inf") if k >= s.size else float(s[k - 1] - s[k])


def draw_tokens_with_margin(w, B, layers_host, min_margin=1e-3, max_attempts=64, check_tokens=None):
    """Draw x [B][H] (redrawing a token with a new attempt number until the
    oracle's router margin is >= min_margin in every layer of layers_host).
    For more than one layer this runs the oracle stack per checked token.
    check_tokens limits the margin checks (others keep attempt 0).
    Returns (x, attempts)."""
    d = oracle.desc_of(w)
    attempts = np.zeros(B, np.int64)
    toks = range(B) if check_tokens is None else check_tokens
    for t in toks:
        for a in range(max_attempts):
            attempts[t] = a
            xt = synth.token_row(w, t, attempts)[None, :]
            ok = True
            if len(layers_host) == 1:
                xhat, _ = oracle.rmsnorm(d, xt[0], layers_host[0].gamma)
                lg = oracle.router_logits(d, layers_host[0], xhat)
                ok = margin(lg, w.k) >= min_margin
            else:
                _, _, _, lg = oracle.stack(d, layers_host, xt)
                ok = all(margin(lg[l, 0], w.k) >= min_margin for l in range(len(layers_host)))
            if ok:
                break
        else:
            raise RuntimeError(f"token {t}: no draw with margin >= {min_margin}")
    return synth.x_tokens(w, B, attempts), attempts


# The oracle is plain single-threaded C called through ctypes, which releases
# the GIL: independent tokens run side by side in threads, each through the
# unchanged oracle functions.
WORKERS = max(1, min(16, os.cpu_count() or 1))


def pmap(fn, items):
    items = list(items)
    if len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(min(WORKERS, len(items))) as ex:
        return list(ex.map(fn, items))


def oracle_layer_tokens(d, L, x):
    """oracle.layer on every token of x [B][H], tokens in parallel threads ->
    (y [B][H], idx [B][k], w [B][k], logits [B][E])."""
    outs = pmap(lambda t: oracle.layer(d, L, np.ascontiguousarray(x[t:t + 1])), range(x.shape[0]))
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(4))


def oracle_logits_tokens(d, L, x):
    """Router logits [B][E] of every token of x (RMSNorm + router)."""
    def one(t):
        xhat, _ = oracle.rmsnorm(d, np.ascontiguousarray(x[t]), L.gamma)
        return oracle.router_logits(d, L, xhat)
    return np.stack(pmap(one, range(x.shape[0])))


def add_experts(w, L, ids, layer=0):
    """Materialise the experts `ids` of layer `layer` in L (host generator)."""
    new = [e for e in sorted(set(int(i) for i in np.ravel(ids))) if e not in L.gate_up]
    gen = lambda e: (synth.expert_gate_up(w, e, layer), synth.expert_down(w, e, layer))
    # fp8 fills are single-threaded C: run them in the pool; bf16/fp32 fills thread internally
    outs = pmap(gen, new) if w.expert == synth.FP8 else [gen(e) for e in new]
    for e, ((gu, gus), (dn, dns)) in zip(new, outs):
        L.gate_up[e], L.down[e] = gu, dn
        if gus is not None:
            L.gate_up_scale[e], L.down_scale[e] = gus, dns


def drop_experts(L):
    L.gate_up.clear(); L.down.clear(); L.gate_up_scale.clear(); L.down_scale.clear()


def valid_selection(logits, sel, k, tol):
    """sel is a top-k of some logit vector within tol of `logits`: k distinct
    experts in range, none below the k-th largest logit by more than tol, none
    left out above it by more than tol, and in non-increasing order up to 2 tol."""
    lg = np.asarray(logits, np.float64)
    sel = np.asarray(sel)
    if len(set(sel.tolist())) != k or sel.min() < 0 or sel.max() >= lg.size:
        return False
    kth = np.sort(lg)[::-1][k - 1]
    rest = np.setdiff1d(np.arange(lg.size), sel)
    if np.any(lg[sel] < kth - tol) or (rest.size and np.any(lg[rest] > kth + tol)):
        return False
    return bool(np.all(np.diff(lg[sel]) <= 2 * tol))
