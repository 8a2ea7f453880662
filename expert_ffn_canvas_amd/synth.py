"""Seeded synthetic inputs for the MoE feed-forward layer.

This module only draws and lays out inputs: it holds none of the layer's
arithmetic, and both the GPU path and the CPU oracle consume what it returns.

Workloads (sizes from the pages: 128 experts / 8 active, d_model 2816,
expert d_ff 704, a 256-token canvas, a 2048-token prompt encoded together with
the canvas, two canvases, 30 MoE layers):

  canvas32   T=32,   fp32 hidden states, fp32 router weight, bf16 experts
  canvas256  T=256,  all bf16, router bias -1.1*ln(e+1) (Zipf s=1.1 skew)
  encode2304 T=2304, all bf16, no router bias
  int4       T=256,  bf16 activations, int4-g128 experts (zero point 8)
  q8         T=256,  bf16 activations, Q8_0 experts (blocks of 32, fp16 scale)
  mxfp4      T=256,  bf16 activations, MXFP4 experts (blocks of 32 E2M1 codes, E8M0 scale)
  mxfp8      T=256,  bf16 activations, MXFP8 experts (blocks of 32 E4M3 codes, E8M0 scale)
  stack30    T=512,  30 layers with their own bf16 weights, Zipf skew,
             a N(0, 0.5) offset [T, D] added after each layer

Canvas output stage (tied LM head + entropy), a workload of its own:

  head256    T=256 canvas positions, vocab 262144, d_model 2816, bf16 hidden
             states and embedding table; each position leans towards a random
             token by a logit margin drawn uniformly from [0, 24], so the
             per-position entropies span near zero to near ln(vocab)

Draw order from one torch generator seeded with the workload's seed:
x, then per layer: router weight, router gamma, expert-norm gamma, gate_up,
down (then, for the stack, the offset of that layer). Normal draws are fp32
and are rounded to bf16 (round-to-nearest-even) where the tensor is bf16.
Gammas and the bias stay fp32 tensors; in the all-bf16 workloads their values
are rounded to bf16-representable numbers. The generator runs on the device
the tensors are made on, so values depend on (seed, device type); every check
hands the oracle the exact tensors the GPU saw.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

N_EXPERTS = 128
TOP_K = 8
D_MODEL = 2816
D_FF = 704
RMS_EPS = 1e-6
GROUP = 128  # int4 group size along the input dimension


@dataclass
class Workload:
    name: str
    T: int
    act: str            # "f32" | "bf16"
    router_w: str       # "f32" | "bf16"
    experts: str        # "bf16" | "i4g128" | "q8_0" | "mxfp4" | "mxfp8"
    bias: str | None    # None | "zipf"
    seed: int
    layers: int = 1
    delta_std: float = 0.0
    E: int = N_EXPERTS
    K: int = TOP_K
    D: int = D_MODEL
    F: int = D_FF
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    "canvas32": Workload("canvas32", 32, "f32", "f32", "bf16", None, 0),
    "canvas256": Workload("canvas256", 256, "bf16", "bf16", "bf16", "zipf", 1),
    "encode2304": Workload("encode2304", 2304, "bf16", "bf16", "bf16", None, 2),
    "int4": Workload("int4", 256, "bf16", "bf16", "i4g128", None, 3),
    "q8": Workload("q8", 256, "bf16", "bf16", "q8_0", None, 5),
    "mxfp4": Workload("mxfp4", 256, "bf16", "bf16", "mxfp4", None, 6),
    "mxfp8": Workload("mxfp8", 256, "bf16", "bf16", "mxfp8", None, 7),
    "stack30": Workload("stack30", 512, "bf16", "bf16", "bf16", "zipf", 4, layers=30, delta_std=0.5),
}


def _randn(shape, std, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def _as_bf16_valued(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16).to(torch.float32)


def zipf_bias(E: int, s: float = 1.1) -> torch.Tensor:
    """Log of the unnormalised Zipf pmf over expert ids: b_e = -s * ln(e + 1)."""
    return torch.tensor([-s * math.log(e + 1) for e in range(E)], dtype=torch.float32)


def quantize_i4g128(w: torch.Tensor):
    """Symmetric int4 codes with zero point 8, groups of 128 along the last dim.

    w: fp32 [..., K]. Per (row, group): s = fp16(2 * amax / 15) and
    q = clamp(round_half_even(w / s) + 8, 0, 15). The last group of a row holds
    whatever remains when K is not a multiple of 128.
    Returns (packed uint8 [..., ceil(K/2)] with even k in the low nibble,
    scales as fp16 [..., ceil(K/128)]).
    """
    K = w.shape[-1]
    G = (K + GROUP - 1) // GROUP
    pad = G * GROUP - K
    wp = torch.nn.functional.pad(w, (0, pad)) if pad else w
    wg = wp.reshape(*w.shape[:-1], G, GROUP)
    amax = wg.abs().amax(dim=-1)
    s16 = (2.0 * amax / 15.0).clamp_min(1e-8).to(torch.float16)
    q = torch.round(wg / s16.to(torch.float32).unsqueeze(-1)) + 8.0
    q = q.clamp(0, 15).to(torch.uint8).reshape(*w.shape[:-1], G * GROUP)[..., :K]
    if K % 2:
        q = torch.nn.functional.pad(q, (0, 1))
    packed = (q[..., 0::2] | (q[..., 1::2] << 4)).contiguous()
    return packed, s16.contiguous()


def quantize_q8_0(w: torch.Tensor) -> torch.Tensor:
    """Q8_0 blocks of 32 consecutive inputs along the last dim (K % 32 == 0), the
    public ggml reference rule: d = amax / 127 (stored as fp16), q = the int8
    nearest to w / d with halves away from zero (0 where the block is all zero).
    Returns uint8 [..., K/32, 34]: per block the fp16 d (little endian), then the
    32 codes as two's-complement bytes.
    """
    K = w.shape[-1]
    assert K % 32 == 0
    wb = w.reshape(*w.shape[:-1], K // 32, 32).to(torch.float32)
    d = wb.abs().amax(dim=-1) / 127.0
    inv = torch.where(d > 0, 1.0 / d, torch.zeros_like(d))
    v = wb * inv.unsqueeze(-1)
    q = (torch.sign(v) * torch.floor(v.abs() + 0.5)).clamp(-127, 127).to(torch.int8)
    d16 = d.to(torch.float16).contiguous().view(torch.uint8).reshape(*d.shape, 2)
    return torch.cat([d16, q.view(torch.uint8)], dim=-1).contiguous()


E2M1_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # magnitudes of E2M1 codes 0..7 (OCP Microscaling)


def quantize_mxfp4(w: torch.Tensor) -> torch.Tensor:
    """MXFP4 blocks of 32 consecutive inputs along the last dim (K % 32 == 0), the
    OCP Microscaling conversion: shared exponent X = floor(log2(amax)) - 2 (the
    largest E2M1 power is 2^2), clamped to [-127, 127] (-127 for an all-zero
    block); each input the E2M1 code nearest to w / 2^X, ties to the even code,
    magnitudes above 6 saturating. Returns uint8 [..., K/32, 17]: per block the
    E8M0 byte X + 127, then 16 bytes holding input j in the low nibble of byte j
    (j < 16) or the high nibble of byte j - 16.
    """
    K = w.shape[-1]
    assert K % 32 == 0
    wb = w.reshape(*w.shape[:-1], K // 32, 32).to(torch.float32)
    amax = wb.abs().amax(dim=-1)
    _, ex = torch.frexp(amax)  # amax = m 2^ex with m in [0.5, 1): floor(log2(amax)) = ex - 1
    X = torch.where(amax > 0, ex.to(torch.float32) - 1 - 2, torch.full_like(amax, -127.0)).clamp(-127, 127)
    v = wb / torch.exp2(X).unsqueeze(-1)
    grid = torch.tensor(E2M1_GRID, dtype=torch.float32, device=w.device)
    dist = (v.abs().clamp(max=6.0).unsqueeze(-1) - grid).abs()
    best = dist.min(dim=-1, keepdim=True).values
    even = (torch.arange(8, device=w.device) % 2 == 0).to(torch.float32)
    idx = ((dist == best).to(torch.float32) * (1.0 + even)).argmax(dim=-1)  # ties -> the even code
    code = (idx | torch.where((v < 0) & (idx > 0), 8, 0)).to(torch.uint8)
    packed = code[..., :16] | (code[..., 16:] << 4)
    e8 = (X + 127).to(torch.uint8).unsqueeze(-1)
    return torch.cat([e8, packed], dim=-1).contiguous()


E4M3_MAX = 448.0  # largest E4M3 magnitude (OCP 8-bit floating point, E4M3 with no infinities)


def quantize_mxfp8(w: torch.Tensor) -> torch.Tensor:
    """MXFP8 (E4M3) blocks of 32 consecutive inputs along the last dim (K % 32 == 0),
    the OCP Microscaling conversion: shared exponent X = floor(log2(amax)) - 8 (the
    largest E4M3 power is 2^8), clamped to [-127, 127] (-127 for an all-zero block);
    each input the E4M3 value nearest to w / 2^X (three mantissa bits below the
    input's own power of two, a fixed 2^-9 step under 2^-6), ties to the even
    code, magnitudes above 448 saturating. Returns uint8 [..., K/32, 33]: per block
    the E8M0 byte X + 127, then the 32 codes in input order.
    """
    K = w.shape[-1]
    assert K % 32 == 0
    out = torch.empty((*w.shape[:-1], K // 32, 33), dtype=torch.uint8, device=w.device)
    flat_w = w.reshape(-1, K)
    flat_o = out.view(-1, K // 32, 33)
    step = max(1, (1 << 24) // K)  # rows per chunk: a few hundred MB of temporaries at most
    for r0 in range(0, flat_w.shape[0], step):
        wb = flat_w[r0:r0 + step].reshape(-1, K // 32, 32).to(torch.float32)
        amax = wb.abs().amax(dim=-1)
        _, ex = torch.frexp(amax)  # floor(log2(amax)) = ex - 1
        X = torch.where(amax > 0, ex.to(torch.float32) - 1 - 8, torch.full_like(amax, -127.0)).clamp(-127, 127)
        a = (wb / torch.exp2(X).unsqueeze(-1)).abs()
        _, ea = torch.frexp(a)  # a in [2^(ea-1), 2^ea)
        quantum = torch.exp2((ea.to(torch.float32) - 1 - 3).clamp(min=-9.0))
        q = (torch.round(a / quantum) * quantum).clamp(max=E4M3_MAX)  # torch.round: half to even
        # q is now an E4M3 magnitude; its code: under 2^-6 the subnormal m 2^-9
        # (m = 8 is 2^-6, code 0x08, the first normal), else exponent and mantissa
        _, eq = torch.frexp(q)
        e_f = (eq - 1 + 7).to(torch.float32)
        normal = q >= 2.0 ** -6
        mant = torch.where(normal, q / torch.exp2(eq.to(torch.float32) - 1) * 8 - 8, q * 512)
        code = torch.where(normal, e_f * 8 + mant, mant).to(torch.int32)
        code = code | torch.where((wb < 0) & (code > 0), 0x80, 0)
        flat_o[r0:r0 + step, :, 0] = (X + 127).to(torch.uint8)
        flat_o[r0:r0 + step, :, 1:] = code.to(torch.uint8)
    return out


def make_layer_weights(wl: Workload, gen: torch.Generator, device) -> dict:
    """Weights of one layer, drawn in the fixed order (router W, gammas, gate_up, down)."""
    E, D, F = wl.E, wl.D, wl.F
    w = {}
    rw = _randn((E, D), 0.02, gen, device)
    w["router_w"] = rw.to(torch.bfloat16) if wl.router_w == "bf16" else rw
    g_r = _randn((D,), 0.1, gen, device)
    g_e = _randn((D,), 0.1, gen, device)
    if wl.act == "bf16":
        g_r, g_e = _as_bf16_valued(g_r), _as_bf16_valued(g_e)
    w["router_gamma"], w["ffn_gamma"] = g_r, g_e
    if wl.bias == "zipf":
        b = zipf_bias(E).to(device)
        w["router_bias"] = _as_bf16_valued(b) if wl.act == "bf16" else b
    else:
        w["router_bias"] = None
    gu = _randn((E, 2 * F, D), 0.02, gen, device)
    if wl.experts == "i4g128":
        w["q_gate_up"], w["s_gate_up"] = quantize_i4g128(gu)
        del gu
        dn = _randn((E, D, F), 0.02, gen, device)
        w["q_down"], w["s_down"] = quantize_i4g128(dn)
        del dn
    elif wl.experts == "q8_0":
        w["q8_gate_up"] = quantize_q8_0(gu)
        del gu
        w["q8_down"] = quantize_q8_0(_randn((E, D, F), 0.02, gen, device))
    elif wl.experts == "mxfp4":
        w["mx4_gate_up"] = quantize_mxfp4(gu)
        del gu
        w["mx4_down"] = quantize_mxfp4(_randn((E, D, F), 0.02, gen, device))
    elif wl.experts == "mxfp8":
        w["mx8_gate_up"] = quantize_mxfp8(gu)
        del gu
        w["mx8_down"] = quantize_mxfp8(_randn((E, D, F), 0.02, gen, device))
    else:
        w["w_gate_up"] = gu.to(torch.bfloat16)
        del gu
        w["w_down"] = _randn((E, D, F), 0.02, gen, device).to(torch.bfloat16)
    return w


def make_inputs(wl: Workload, device="cpu", layers: int | None = None, T: int | None = None):
    """Generate x and the weights of the first `layers` layers (default: all).

    Returns dict(x, layers=[weights...], deltas=[...] for stacks).
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed)
    T = wl.T if T is None else T
    x = _randn((T, wl.D), 1.0, gen, device)
    x = x.to(torch.bfloat16) if wl.act == "bf16" else x
    n_layers = wl.layers if layers is None else layers
    out = {"x": x, "layers": [], "deltas": []}
    for _ in range(n_layers):
        out["layers"].append(make_layer_weights(wl, gen, device))
        if wl.delta_std > 0:
            d = _randn((T, wl.D), wl.delta_std, gen, device)
            out["deltas"].append(d.to(torch.bfloat16) if wl.act == "bf16" else d)
    return out


@dataclass
class HeadWorkload:
    name: str
    T: int
    V: int
    D: int
    seed: int
    max_margin: float = 24.0


HEAD_WORKLOADS = {
    "head256": HeadWorkload("head256", 256, 262144, D_MODEL, 8),
}


def make_head_inputs(hw: HeadWorkload, device="cpu"):
    """Embedding table emb [V, D] ~ N(0, 0.02) and canvas hidden states h [T, D], both bf16.

    Draw order from one generator seeded with hw.seed: emb, then z ~ N(0, 1) [T, D], then a target
    token y_t and a margin L_t ~ U(0, max_margin) per position (position 0 gets margin 0 and the last
    position max_margin). h_t = z_t + L_t emb[y_t] / |emb[y_t]|^2, so the target's logit is raised
    by about L_t over the rest. Returns dict(emb, h, target, margin).
    """
    gen = torch.Generator(device=device).manual_seed(hw.seed)
    emb = _randn((hw.V, hw.D), 0.02, gen, device).to(torch.bfloat16)
    z = torch.randn((hw.T, hw.D), generator=gen, device=device, dtype=torch.float32)
    y = torch.randint(0, hw.V, (hw.T,), generator=gen, device=device)
    L = torch.rand((hw.T,), generator=gen, device=device, dtype=torch.float32) * hw.max_margin
    if hw.T > 0:
        L[0] = 0.0
        L[-1] = hw.max_margin
    ey = emb[y].to(torch.float32)
    h = (z + L.unsqueeze(1) * ey / (ey * ey).sum(dim=1, keepdim=True)).to(torch.bfloat16)
    return {"emb": emb, "h": h, "target": y, "margin": L}


def small_workload(name="tiny", T=16, E=6, K=2, D=128, F=64, act="bf16", router_w="bf16",
                   experts="bf16", bias=None, seed=0) -> Workload:
    """A shrunken workload with the same recipe, for tests the oracle finishes quickly."""
    return Workload(name, T, act, router_w, experts, bias, seed, E=E, K=K, D=D, F=F)


def to_numpy_bits(t: torch.Tensor | None):
    """Host numpy view for the oracle: bf16 -> uint16 bits, fp16 -> uint16 bits, others as is."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16 or t.dtype == torch.float16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def weights_to_numpy(w: dict) -> dict:
    return {k: to_numpy_bits(v) for k, v in w.items()}
