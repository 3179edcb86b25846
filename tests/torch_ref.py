"""An independent float64 PyTorch (CPU) composition of the MoE decode layer,
used only to pin the C oracle. It is written from the same definition (RMSNorm,
router, softmax + top-k + renormalisation, SwiGLU experts, shared expert,
residual) with library routines (torch.matmul, torch.softmax, F.silu,
torch.argsort(stable=True), torch's bf16 / fp8 casts) and the same rounding
points; it shares no code with the oracle.
"""
import numpy as np
import torch
import torch.nn.functional as F

F32, BF16, FP8 = 0, 1, 2


def decode(a: np.ndarray, dtype: int, scales: np.ndarray = None, group: int = 128) -> torch.Tensor:
    """Storage array -> float64 tensor (fp8: code * bf16 scale of its row group)."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == F32:
        return t.to(torch.float64)
    if dtype == BF16:
        return t.view(torch.int16).view(torch.bfloat16).to(torch.float64)
    v = t.view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(np.ascontiguousarray(scales)).view(torch.int16).view(torch.bfloat16).to(torch.float64)
    return v * s.repeat_interleave(group)[:, None]


def round_act(v: torch.Tensor, act: int) -> torch.Tensor:
    v = v.to(torch.float32)
    if act == BF16:
        v = v.to(torch.bfloat16)
    return v.to(torch.float64)


def ffn(gate_up: torch.Tensor, down: torch.Tensor, xa: torch.Tensor, act: int):
    inter = gate_up.shape[0] // 2
    g = (gate_up[:inter] @ xa).to(torch.float32).to(torch.float64)
    u = (gate_up[inter:] @ xa).to(torch.float32).to(torch.float64)
    h = round_act(F.silu(g) * u, act)
    return (down @ h).to(torch.float32).to(torch.float64), h


def layer_token(d, L, x_t: np.ndarray, given=None):
    """d: oracle.OrcDesc-like (attributes); L: oracle.Layer. Returns (y float64, idx, w).
    given: a selection (k expert ids in rank order) used in place of the top-k."""
    act = d.act
    x = decode(x_t, act)
    gamma = decode(L.gamma, act)
    xhat = (x * torch.rsqrt((x * x).mean() + float(np.float32(d.rms_eps))) * gamma).to(torch.float32).to(torch.float64)
    xa = round_act(xhat, act)
    logits = (decode(L.router_w, d.router) @ xhat).to(torch.float32)
    if L.router_bias is not None:
        logits = logits + torch.from_numpy(L.router_bias)
    p = torch.softmax(logits.to(torch.float64), dim=0)
    order = torch.argsort(-logits, stable=True)[: d.top_k]
    if given is not None:
        order = torch.as_tensor(np.asarray(given, np.int64))
    w = (p[order] / p[order].sum()).to(torch.float32)
    routed = torch.zeros_like(x)
    for i, e in enumerate(order.tolist()):
        gu = decode(L.gate_up[e], d.expert, L.gate_up_scale.get(e), d.scale_group)
        dn = decode(L.down[e], d.expert, L.down_scale.get(e), d.scale_group)
        de, _ = ffn(gu, dn, xa, act)
        routed += float(w[i]) * de
    sh = torch.zeros_like(x)
    if d.shared_inter > 0:
        sh, _ = ffn(decode(L.shared_gate_up, d.shared), decode(L.shared_down, d.shared), xa, act)
    y = round_act(x + sh + routed, act)
    return y, order.numpy().astype(np.int32), w.numpy()
