"""Library-built fp64 references used to pin the oracle (tests only).

Each step is one torch library routine in float64: rms_norm, matmul, softmax,
gelu(approximate="tanh"). The dense reference evaluates EVERY expert on every
token and weights them with a dense vector that is zero off the selected set,
so it has no permutation, no gather and no per-slot loop: a different
algorithm from the oracle's sparse one.
"""
import numpy as np
import torch
import torch.nn.functional as F


def bits_to_f64(a):
    """numpy array (float32, or uint16 holding bf16 bits) -> torch float64."""
    if a.dtype == np.uint16:
        return torch.from_numpy(a.astype(np.int16)).view(torch.bfloat16).to(torch.float64)
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rms_norm_plus_one(x, gamma, eps):
    """(1 + gamma) RMSNorm through torch's rms_norm."""
    return F.rms_norm(x, (x.shape[-1],), weight=1.0 + gamma, eps=eps)


def logits_fp64(x, router_w, gamma_r, bias, eps):
    z = rms_norm_plus_one(x, gamma_r, eps)
    lg = z @ router_w.T
    if bias is not None:
        lg = lg + bias
    return lg


def dense_ffn_fp64(h, w_gate, w_up, w_down):
    """W_down (gelu_tanh(W_gate h) * (W_up h)) for rows of h."""
    return (F.gelu(h @ w_gate.T, approximate="tanh") * (h @ w_up.T)) @ w_down.T


def dense_moe_fp64(x, w, k, eps, dense_weights=None):
    """Dense all-experts MoE in fp64.

    x [T, D] float64; w dict of float64 tensors router_w [E,D], router_gamma [D], router_bias [E]|None,
    ffn_gamma [D], w_gate_up [E,2F,D], w_down [E,D,F]. The dense weight matrix is the full softmax
    masked to the k largest logits (torch.topk) and renormalised, unless given.
    """
    lg = logits_fp64(x, w["router_w"], w["router_gamma"], w.get("router_bias"), eps)
    if dense_weights is None:
        p = torch.softmax(lg, dim=-1)
        top = torch.topk(lg, k, dim=-1).indices
        mask = torch.zeros_like(p).scatter_(1, top, 1.0)
        pm = p * mask
        dense_weights = pm / pm.sum(dim=-1, keepdim=True)
    h = rms_norm_plus_one(x, w["ffn_gamma"], eps)
    E = w["router_w"].shape[0]
    Fd = w["w_gate_up"].shape[1] // 2
    out = torch.zeros_like(x)
    for e in range(E):
        y = dense_ffn_fp64(h, w["w_gate_up"][e, :Fd], w["w_gate_up"][e, Fd:], w["w_down"][e])
        out = out + dense_weights[:, e:e + 1] * y
    return out, lg, dense_weights
