"""Pins of the CPU oracle against things other than itself (CPU only).

Each test ties one part of the oracle to brute force, a torch/numpy/scipy
library routine, a closed form or an invariant, chosen so that a plausible
mistake (dropped (1+gamma), eps outside the root, transposed operand, gate and
up swapped, wrong tie order, wrong nibble order or zero point, wrong softmax
normalisation) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax as scipy_softmax

import oracle
from expert_ffn_canvas_amd import synth
from tests.ref_lib import bits_to_f64, dense_ffn_fp64, dense_moe_fp64, logits_fp64, rms_norm_plus_one

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
EPS = 1e-6


def small(T=16, E=6, K=2, D=128, F=64, seed=0, act="bf16", router_w="bf16", experts="bf16", bias=None):
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, act=act, router_w=router_w, experts=experts,
                              bias=bias, seed=seed)
    inp = synth.make_inputs(wl, device="cpu")
    return wl, inp["x"], inp["layers"][0]


def np_inputs(x, w):
    return synth.to_numpy_bits(x), synth.weights_to_numpy(w)


def f64_weights(wn):
    out = {}
    for k, v in wn.items():
        out[k] = None if v is None else bits_to_f64(v)
    return out


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


# ----------------------------------------------------------------------------- scalar helpers

def test_gelu_tanh_pins():
    # gelu(0) = 0, and the tanh form satisfies gelu(z) - gelu(-z) = z exactly in real arithmetic.
    assert oracle.gelu_tanh_f64(0.0) == 0.0
    assert oracle.gelu_tanh_f32(0.0) == 0.0
    zs = np.linspace(-9.0, 9.0, 721)
    for z in zs:
        g64 = oracle.gelu_tanh_f64(z)
        assert abs((g64 - oracle.gelu_tanh_f64(-z)) - z) <= 1e-14 * max(1.0, abs(z))
        g32 = oracle.gelu_tanh_f32(np.float32(z))
        assert abs((g32 - oracle.gelu_tanh_f32(np.float32(-z))) - np.float32(z)) <= 2e-6 * max(1.0, abs(z))
    # library routine: torch's tanh-approximate GELU in fp64
    zt = torch.tensor(zs, dtype=torch.float64)
    lib = F.gelu(zt, approximate="tanh").numpy()
    ours64 = np.array([oracle.gelu_tanh_f64(z) for z in zs])
    ours32 = np.array([oracle.gelu_tanh_f32(np.float32(z)) for z in zs])
    assert np.max(np.abs(ours64 - lib)) <= 1e-14
    assert np.max(np.abs(ours32 - lib) / np.maximum(np.abs(lib), 1.0)) <= 2e-6
    # textbook: the tanh form stays within 5e-4 of the exact x * Phi(x) GELU
    exact = 0.5 * zt * (1.0 + torch.erf(zt / math.sqrt(2.0)))
    assert np.max(np.abs(ours64 - exact.numpy())) <= 5e-4
    # asymptotes
    assert abs(oracle.gelu_tanh_f64(30.0) - 30.0) < 1e-12
    assert abs(oracle.gelu_tanh_f64(-30.0)) < 1e-12


def test_half_to_float_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    lib = bits.view(np.float16).astype(np.float32)
    ours = np.array([oracle.half_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan].view(np.uint32), lib[~nan].view(np.uint32))


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10,
        # exact ties: low half 0x8000 with even and odd upper halves
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, np.inf, -np.inf], dtype=np.float32),
    ])
    lib = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.float_to_bf16_bits(v) for v in vals], dtype=np.uint16)
    assert np.array_equal(ours, lib)


# ----------------------------------------------------------------------------- router

@pytest.mark.parametrize("act,rw", [("bf16", "bf16"), ("f32", "f32")])
def test_router_logits_match_library_fp64(act, rw):
    wl, x, w = small(T=24, E=10, K=3, D=256, act=act, router_w=rw, bias="zipf", seed=3)
    xn, wn = np_inputs(x, w)
    r = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn["router_bias"], 3, EPS)
    lg = logits_fp64(bits_to_f64(xn), bits_to_f64(wn["router_w"]), bits_to_f64(wn["router_gamma"]),
                     bits_to_f64(wn["router_bias"]), EPS).numpy()
    assert np.max(np.abs(r["logits"] - lg)) <= 1e-12
    # r = 1/sqrt(mean(x^2) + eps): torch rms_norm of x with unit weight divided by x
    xt = bits_to_f64(xn)
    ref_r = (F.rms_norm(xt, (xt.shape[1],), eps=EPS) / xt)[:, 0].numpy()
    assert np.allclose(r["r"], ref_r, rtol=1e-12, atol=0)


def test_eps_sits_inside_the_root():
    # tiny residual: mean(x^2) ~ 1e-8 << eps, so r is dominated by eps.
    wl, x, w = small(T=8, E=6, K=2, D=128, act="f32", router_w="f32", seed=4)
    xs = (x * 1e-4).contiguous()
    xn, wn = np_inputs(xs, w)
    r = oracle.route(xn, wn["router_w"], wn["router_gamma"], None, 2, EPS)
    xt = bits_to_f64(xn)
    ref_r = (F.rms_norm(xt, (xt.shape[1],), eps=EPS) / xt)[:, 0].numpy()
    assert np.allclose(r["r"], ref_r, rtol=1e-12, atol=0)
    assert np.all(r["r"] < 1.0 / math.sqrt(EPS) * 1.0001)


@pytest.mark.parametrize("E,K", [(10, 3), (7, 1), (9, 2), (6, 6)])
def test_topk_equals_subset_enumeration(E, K):
    wl, x, w = small(T=40, E=E, K=K, D=128, seed=E * 10 + K)
    xn, wn = np_inputs(x, w)
    r = oracle.route(xn, wn["router_w"], wn["router_gamma"], None, K, EPS)
    lg = logits_fp64(bits_to_f64(xn), bits_to_f64(wn["router_w"]), bits_to_f64(wn["router_gamma"]), None,
                     EPS).numpy()
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(E), K), key=lambda s: sum(lg[t, list(s)]))
        assert sorted(r["idx"][t].tolist()) == sorted(best)
        # slots ordered by logit descending
        assert np.all(np.diff(lg[t, r["idx"][t]]) <= 0)
        if K < E:
            srt = np.sort(lg[t])[::-1]
            assert abs(r["gap"][t] - (srt[K - 1] - srt[K])) <= 1e-12


def test_exact_ties_go_to_lower_expert_id():
    # x = 0 makes every normalised router input 0, so the logits are exactly the bias.
    E, K, D = 8, 3, 128
    x = np.zeros((3, D), dtype=np.float32)
    rw = np.random.default_rng(0).standard_normal((E, D)).astype(np.float32)
    gam = np.zeros(D, dtype=np.float32)
    bias = np.array([[0.5, 1.0, 1.0, 0.2, 1.0, 1.0, 0.9, 0.1],
                     [2.0, 2.0, 2.0, 2.0, 2.0, 2.0, 2.0, 2.0],
                     [0.0, 0.3, 0.3, 0.7, 0.7, 0.7, 0.7, 0.1]], dtype=np.float32)
    want = [[1, 2, 4], [0, 1, 2], [3, 4, 5]]
    for row, exp in zip(bias, want):
        r = oracle.route(x[:1].copy(), rw, gam, row.copy(), K, EPS)
        assert r["idx"][0].tolist() == exp


def test_weights_are_renormalised_softmax():
    wl, x, w = small(T=32, E=12, K=4, D=128, seed=7, bias="zipf")
    xn, wn = np_inputs(x, w)
    r = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn["router_bias"], 4, EPS)
    assert np.max(np.abs(r["w"].sum(axis=1) - 1.0)) <= 1e-12
    full = scipy_softmax(r["logits"], axis=1)
    for t in range(32):
        sel = full[t, r["idx"][t]]
        assert np.allclose(r["w"][t], sel / sel.sum(), rtol=1e-12, atol=0)
    # k = E: the renormalised weights are the plain softmax (library routine)
    rE = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn["router_bias"], 12, EPS)
    for t in range(32):
        assert np.allclose(rE["w"][t], full[t, rE["idx"][t]], rtol=1e-12, atol=1e-300)
    # E = 1, k = 1: weight exactly 1
    r1 = oracle.route(xn, np.ascontiguousarray(wn["router_w"][:1]), wn["router_gamma"], None, 1, EPS)
    assert np.all(r1["w"] == 1.0) and np.all(r1["idx"] == 0)


def test_router_full_shape_matches_library_topk():
    wl = synth.WORKLOADS["canvas256"]
    gen = torch.Generator().manual_seed(11)
    x = torch.randn((64, wl.D), generator=gen).to(torch.bfloat16)
    rw = (torch.randn((wl.E, wl.D), generator=gen) * 0.02).to(torch.bfloat16)
    g = (torch.randn((wl.D,), generator=gen) * 0.1).to(torch.bfloat16).float()
    b = synth.zipf_bias(wl.E)
    xn, rwn = synth.to_numpy_bits(x), synth.to_numpy_bits(rw)
    r = oracle.route(xn, rwn, g.numpy(), b.numpy(), wl.K, EPS)
    lg = logits_fp64(bits_to_f64(xn), bits_to_f64(rwn), g.double(), b.double(), EPS)
    top = torch.topk(lg, wl.K + 1, dim=1)
    for t in range(64):
        gap = (top.values[t, wl.K - 1] - top.values[t, wl.K]).item()
        assert abs(gap - r["gap"][t]) <= 1e-12
        if gap > 1e-9:
            assert r["idx"][t].tolist() == top.indices[t, :wl.K].tolist()


# ----------------------------------------------------------------------------- permutation

def test_permutation_matches_stable_argsort():
    rng = np.random.default_rng(1)
    T, K, E = 300, 8, 128
    # skewed routing with distinct experts per token, some experts empty
    p = np.exp(-1.1 * np.log(np.arange(E) + 1.0))
    p /= p.sum()
    idx = np.stack([rng.choice(E, size=K, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    pm = oracle.permute(idx, E)
    assert pm["counts"].sum() == K * T
    assert np.array_equal(pm["counts"], np.bincount(idx.ravel(), minlength=E))
    assert np.array_equal(pm["offsets"], np.concatenate([[0], np.cumsum(pm["counts"])]))
    order = np.argsort(idx.ravel(), kind="stable")  # library stable sort over slots
    assert np.array_equal(pm["sorted_token"], order // K)
    inv = np.empty_like(order)
    inv[order] = np.arange(T * K)
    assert np.array_equal(pm["row_of_slot"], inv)
    # every token appears exactly K times
    assert np.array_equal(np.bincount(pm["sorted_token"], minlength=T), np.full(T, K))
    assert np.any(pm["counts"] == 0)


# ----------------------------------------------------------------------------- whole layer

def test_dense_all_experts_bruteforce():
    wl, x, w = small(T=16, E=6, K=2, D=128, F=64, seed=21, bias="zipf")
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 2, EPS)
    ref, lg, dw = dense_moe_fp64(bits_to_f64(xn), f64_weights(wn), 2, EPS)
    assert rel_err(o["out"], ref.numpy()) <= 2e-5
    # the oracle's weights equal the dense masked-softmax weights on its selection
    for t in range(16):
        assert np.allclose(o["w"][t], dw[t, o["idx"][t]].numpy(), rtol=1e-12)


def test_dense_bruteforce_fp32_activations():
    wl, x, w = small(T=12, E=5, K=3, D=256, F=128, seed=22, act="f32", router_w="f32")
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 3, EPS)
    ref, _, _ = dense_moe_fp64(bits_to_f64(xn), f64_weights(wn), 3, EPS)
    assert rel_err(o["out"], ref.numpy()) <= 2e-5


def test_single_expert_closed_form():
    # E = 1, k = 1: out = W_down (gelu_tanh(W_gate h) * W_up h), with D != F so a transposed
    # operand cannot pass.
    wl, x, w = small(T=10, E=1, K=1, D=256, F=64, seed=23)
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 1, EPS)
    wf = f64_weights(wn)
    h = rms_norm_plus_one(bits_to_f64(xn), wf["ffn_gamma"], EPS)
    ref = dense_ffn_fp64(h, wf["w_gate_up"][0, :64], wf["w_gate_up"][0, 64:], wf["w_down"][0])
    assert rel_err(o["out"], ref.numpy()) <= 2e-5
    assert np.all(o["w"] == 1.0)
    # gate and up swapped gives a clearly different answer (the pin can see that mistake)
    swapped = dense_ffn_fp64(h, wf["w_gate_up"][0, 64:], wf["w_gate_up"][0, :64], wf["w_down"][0])
    assert rel_err(swapped.numpy(), ref.numpy()) > 0.1


def test_forced_expert_by_bias():
    E, K = 8, 3
    wl, x, w = small(T=20, E=E, K=K, D=128, F=64, seed=24)
    j = 5
    b = torch.zeros(E)
    b[j] = 30.0
    w["router_bias"] = b
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 1, EPS)
    assert np.all(o["idx"][:, 0] == j)
    wf = f64_weights(wn)
    h = rms_norm_plus_one(bits_to_f64(xn), wf["ffn_gamma"], EPS)
    ref = dense_ffn_fp64(h, wf["w_gate_up"][j, :64], wf["w_gate_up"][j, 64:], wf["w_down"][j])
    assert rel_err(o["out"], ref.numpy()) <= 2e-5
    # with k = 3 the forced expert takes weight 1 - O(e^-20)
    o3 = oracle.moe_forward(wn, xn, K, EPS)
    assert np.all(o3["idx"][:, 0] == j)
    assert np.all(o3["w"][:, 0] > 1 - 1e-8)
    assert rel_err(o3["out"], ref.numpy()) <= 2e-5


def test_identical_experts_make_routing_irrelevant():
    E, K = 8, 3
    wl, x, w = small(T=24, E=E, K=K, D=128, F=64, seed=25, bias="zipf")
    w["w_gate_up"] = w["w_gate_up"][:1].expand(E, -1, -1).contiguous()
    w["w_down"] = w["w_down"][:1].expand(E, -1, -1).contiguous()
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, K, EPS)
    wf = f64_weights(wn)
    h = rms_norm_plus_one(bits_to_f64(xn), wf["ffn_gamma"], EPS)
    ref = dense_ffn_fp64(h, wf["w_gate_up"][0, :64], wf["w_gate_up"][0, 64:], wf["w_down"][0])
    assert rel_err(o["out"], ref.numpy()) <= 2e-5


def test_fold_invariance_is_exact():
    # Fold a power-of-two scale s_d out of the expert norm and into gate_up's input columns:
    # (1 + g') = (1 + g) / s, W' = W * s. The router reads the raw residual through its own norm, so
    # routing cannot move; with powers of two every product is unchanged, so the output is identical.
    E, K, D = 8, 3, 128
    wl, x, w = small(T=16, E=E, K=K, D=D, F=64, seed=26, bias="zipf")
    gen = torch.Generator().manual_seed(3)
    g = (torch.randint(-256, 256, (D,), generator=gen).float() / 1024.0)  # exact in fp32
    w["ffn_gamma"] = g
    s = torch.tensor([0.5, 1.0, 2.0])[torch.randint(0, 3, (D,), generator=gen)]
    w2 = dict(w)
    w2["ffn_gamma"] = (1.0 + g) / s - 1.0
    assert torch.equal(1.0 + w2["ffn_gamma"].double(), (1.0 + g.double()) / s.double())
    w2["w_gate_up"] = (w["w_gate_up"].float() * s).to(torch.bfloat16)
    xn, wn = np_inputs(x, w)
    _, wn2 = np_inputs(x, w2)
    o1 = oracle.moe_forward(wn, xn, K, EPS)
    o2 = oracle.moe_forward(wn2, xn, K, EPS)
    assert np.array_equal(o1["idx"], o2["idx"])
    assert np.array_equal(o1["w"], o2["w"])
    assert np.array_equal(o1["out"], o2["out"])
    # and a mistake that lets the expert norm leak into routing would be visible: the fold does change h
    assert not np.array_equal(wn["ffn_gamma"], wn2["ffn_gamma"])


def test_forced_selection_and_token_subset():
    wl, x, w = small(T=20, E=10, K=3, D=128, F=64, seed=27)
    xn, wn = np_inputs(x, w)
    full = oracle.moe_forward(wn, xn, 3, EPS)
    sub = oracle.moe_forward(wn, xn, 3, EPS, tokens=np.array([19, 0, 7]))
    assert np.array_equal(sub["out"], full["out"][[19, 0, 7]])
    # forcing the oracle's own selection reproduces it; forcing another set follows the dense reference
    same = oracle.moe_forward(wn, xn, 3, EPS, forced=full["idx"])
    assert np.array_equal(same["out"], full["out"])
    forced = np.tile(np.array([[9, 4, 1]], dtype=np.int32), (20, 1))
    of = oracle.moe_forward(wn, xn, 3, EPS, forced=forced)
    wf = f64_weights(wn)
    xt = bits_to_f64(xn)
    lg = logits_fp64(xt, wf["router_w"], wf["router_gamma"], None, EPS)
    dw = torch.zeros_like(lg)
    sel = torch.softmax(lg[:, [9, 4, 1]], dim=1)
    dw[:, [9, 4, 1]] = sel
    ref, _, _ = dense_moe_fp64(xt, wf, 3, EPS, dense_weights=dw)
    assert rel_err(of["out"], ref.numpy()) <= 2e-5


def test_residual_and_addend():
    wl, x, w = small(T=8, E=6, K=2, D=128, F=64, seed=28)
    xn, wn = np_inputs(x, w)
    add = synth.to_numpy_bits((torch.randn(x.shape) * 0.5).to(torch.bfloat16))
    base = oracle.moe_forward(wn, xn, 2, EPS)
    both = oracle.moe_forward(wn, xn, 2, EPS, add_input=True, addend=add)
    xf = bits_to_f64(xn).float().numpy()
    af = bits_to_f64(add).float().numpy()
    assert np.array_equal(both["out"], (base["out"] + xf) + af)


# ----------------------------------------------------------------------------- int4 codec

def test_int4_codec_roundtrip_and_layout():
    gen = torch.Generator().manual_seed(9)
    for K in (2816, 704, 320):
        w = torch.randn((6, K), generator=gen) * 0.02
        # a recognisable pattern in the tail group
        w[0, -1] = 0.3
        q, s = synth.quantize_i4g128(w)
        G = (K + 127) // 128
        assert q.shape == (6, (K + 1) // 2) and s.shape == (6, G) and s.dtype == torch.float16
        deq = oracle.dequant_i4(q.numpy(), s.view(torch.int16).numpy().view(np.uint16), K)
        # numpy unpack of the layout: even k in the low nibble
        qb = q.numpy()
        codes = np.empty((6, K), dtype=np.int32)
        codes[:, 0::2] = (qb & 0x0F)[:, : (K + 1) // 2][:, : codes[:, 0::2].shape[1]]
        codes[:, 1::2] = (qb >> 4)[:, : codes[:, 1::2].shape[1]]
        sf = s.float().numpy()
        ref = (codes - 8).astype(np.float32) * np.repeat(sf, 128, axis=1)[:, :K]
        assert np.array_equal(deq, ref)  # (q - 8) * s is exact in fp32
        # round trip: within half a step of the original weight. The fp16 rounding of the scale
        # (relative 2^-11) can push the group's largest weight up to 7.5 * 2^-11 steps further.
        step = np.repeat(sf, 128, axis=1)[:, :K]
        assert np.all(np.abs(deq - w.numpy()) <= step * (0.5 + 7.5 * 2 ** -11) + 1e-12)
        # the largest magnitude of each group maps to code 0 or 15 (full range used)
        assert np.all((codes.min(axis=1) == 0) | (codes.max(axis=1) == 15))
        assert abs(deq[0, -1] - 0.3) <= step[0, -1] * (0.5 + 7.5 * 2 ** -11)


def test_int4_layer_matches_dense_reference_of_dequantised_weights():
    wl, x, w = small(T=12, E=6, K=2, D=256, F=192, seed=29, experts="i4g128")
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 2, EPS)
    wf = f64_weights({k: v for k, v in wn.items() if k in ("router_w", "router_gamma", "ffn_gamma")})
    wf["router_bias"] = None
    E, D, Fd = 6, 256, 192
    gu = oracle.dequant_i4(wn["q_gate_up"].reshape(E * 2 * Fd, -1), wn["s_gate_up"].reshape(E * 2 * Fd, -1), D)
    dn = oracle.dequant_i4(wn["q_down"].reshape(E * D, -1), wn["s_down"].reshape(E * D, -1), Fd)
    wf["w_gate_up"] = torch.from_numpy(gu.reshape(E, 2 * Fd, D)).double()
    wf["w_down"] = torch.from_numpy(dn.reshape(E, D, Fd)).double()
    ref, _, _ = dense_moe_fp64(bits_to_f64(xn), wf, 2, EPS)
    assert rel_err(o["out"], ref.numpy()) <= 2e-5


def test_q8_0_block_layout_and_roundtrip():
    # A hand-made block: fp16 scale 0.5 stored little endian (0x3800 -> bytes 00 38), then 32 int8
    # codes in two's complement; each weight is code * 0.5 exactly.
    codes = [-128, -127, -1, 0, 1, 2, 63, 127] + list(range(-12, 12))
    blk = np.array([0x00, 0x38] + [c & 0xFF for c in codes], dtype=np.uint8)
    assert blk.size == 34
    deq = oracle.dequant_q8_0(blk.reshape(1, 34), 32)
    assert np.array_equal(deq[0], np.array(codes, dtype=np.float32) * 0.5)
    # Two blocks per row, two rows: the scale of block b covers inputs 32 b .. 32 b + 31 of its row.
    two = np.zeros((2, 2, 34), dtype=np.uint8)
    two[:, :, 0:2] = [[[0x00, 0x3C], [0x00, 0x40]], [[0x00, 0xBC], [0x00, 0x00]]]  # 1, 2, -1, 0
    two[:, :, 2:] = 3
    d2 = oracle.dequant_q8_0(two.reshape(2, 68), 64)
    assert np.array_equal(d2, np.array([[3.0] * 32 + [6.0] * 32, [-3.0] * 32 + [0.0] * 32], dtype=np.float32))
    # Round trip of the quantiser of the inputs: within half a step of the original weight, where the
    # fp16 rounding of the scale (relative 2^-11) can move the largest code (127) by 127 * 2^-11 steps.
    gen = torch.Generator().manual_seed(11)
    w = torch.randn((5, 2816), generator=gen) * 0.02
    w[1, 64:96] = 0.0  # an all-zero block: scale 0, codes 0
    b = synth.quantize_q8_0(w)
    assert b.shape == (5, 88, 34) and b.dtype == torch.uint8
    deq = oracle.dequant_q8_0(b.numpy().reshape(5, -1), 2816)
    step = np.repeat((w.reshape(5, 88, 32).abs().amax(-1) / 127.0).numpy(), 32, axis=1)
    assert np.all(np.abs(deq - w.numpy()) <= step * (0.5 + 127 * 2 ** -11) + 1e-12)
    assert np.all(deq[1, 64:96] == 0.0) and np.all(b[1, 2, :].numpy() == 0)
    # the largest magnitude of every non-zero block maps to code +-127 (full range used)
    q = b[..., 2:].numpy().view(np.int8).astype(np.int32)
    nz = step[:, ::32] > 0
    assert np.all(np.abs(q).max(axis=-1)[nz] == 127)


def test_q8_0_layer_matches_dense_reference_of_dequantised_weights():
    wl, x, w = small(T=12, E=6, K=2, D=256, F=192, seed=31, experts="q8_0")
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 2, EPS)
    wf = f64_weights({k: v for k, v in wn.items() if k in ("router_w", "router_gamma", "ffn_gamma")})
    wf["router_bias"] = None
    E, D, Fd = 6, 256, 192
    gu = oracle.dequant_q8_0(wn["q8_gate_up"].reshape(E * 2 * Fd, -1), D)
    dn = oracle.dequant_q8_0(wn["q8_down"].reshape(E * D, -1), Fd)
    wf["w_gate_up"] = torch.from_numpy(gu.reshape(E, 2 * Fd, D)).double()
    wf["w_down"] = torch.from_numpy(dn.reshape(E, D, Fd)).double()
    ref, _, _ = dense_moe_fp64(bits_to_f64(xn), wf, 2, EPS)
    assert rel_err(o["out"], ref.numpy()) <= 2e-5


# E2M1 values of codes 0..15 as the OCP Microscaling specification tabulates them (sign bit 3; exponent
# bits 2..1 with bias 1, code 0b001 the subnormal 0.5; mantissa bit 0).
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_mxfp4_codes_scales_and_layout():
    # One block with scale byte 127 (2^0): inputs 0..15 carry codes 0..15 in the low nibbles, inputs
    # 16..31 carry codes 15..0 in the high nibbles of the same 16 bytes.
    lo = np.arange(16, dtype=np.uint8)
    hi = lo[::-1]
    blk = np.concatenate([[127], lo | (hi << 4)]).astype(np.uint8)
    deq = oracle.dequant_mxfp4(blk.reshape(1, 17), 32)[0]
    spec = np.array(E2M1_SPEC, dtype=np.float32)
    assert np.array_equal(deq[:16], spec) and np.array_equal(deq[16:], spec[::-1])
    assert np.array_equal(np.signbit(deq[:16]), np.signbit(spec))
    # E8M0: byte e scales by 2^(e - 127), down to 2^-127 (an fp32 subnormal); 255 is NaN.
    for e, scale in [(128, 2.0), (126, 0.5), (120, 2.0 ** -7), (0, 2.0 ** -127), (200, 2.0 ** 73)]:
        b = blk.copy()
        b[0] = e
        d = oracle.dequant_mxfp4(b.reshape(1, 17), 32)[0]
        assert np.array_equal(d, (spec.astype(np.float64) * scale).astype(np.float32)[np.r_[0:16, 15:-1:-1]]), e
    b = blk.copy()
    b[0] = 255
    assert np.all(np.isnan(oracle.dequant_mxfp4(b.reshape(1, 17), 32)))
    # Two blocks per row: block b covers inputs 32 b .. 32 b + 31 of its row.
    two = np.zeros((1, 2, 17), dtype=np.uint8)
    two[0, 0, 0], two[0, 1, 0] = 127, 129  # 1 and 4
    two[0, :, 1:] = 0x72  # inputs j < 16: code 2 (1.0); j >= 16: code 7 (6.0)
    d2 = oracle.dequant_mxfp4(two.reshape(1, 34), 64)[0]
    assert np.array_equal(d2, np.array([1.0] * 16 + [6.0] * 16 + [4.0] * 16 + [24.0] * 16, dtype=np.float32))


def test_mxfp4_quantiser_roundtrip():
    gen = torch.Generator().manual_seed(12)
    w = torch.randn((5, 2816), generator=gen) * 0.02
    w[2, 32:64] = 0.0  # an all-zero block
    w[3, 0:32] = torch.tensor([6.0, -2.5, 1.25, 0.25] + [0.0] * 28)  # ties at scale 1 (amax 6 -> X = 0)
    b = synth.quantize_mxfp4(w)
    assert b.shape == (5, 88, 17) and b.dtype == torch.uint8
    deq = oracle.dequant_mxfp4(b.numpy().reshape(5, -1), 2816)
    wn = w.numpy()
    amax = np.abs(wn.reshape(5, 88, 32)).max(-1)
    X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    scale = np.repeat(2.0 ** X, 32, axis=1)
    # the block's largest magnitude lands in [4, 8) scale units; rounding is within half a grid gap
    # (a quarter of the value, or a quarter of the scale near zero), saturation above 6 within 2 units
    err = np.abs(deq - wn)
    assert np.all(err <= np.maximum(0.25 * scale, 0.25 * np.abs(wn)) + 1e-12)
    assert np.all(deq[2, 32:64] == 0.0) and b[2, 1, 0].item() == 0
    # ties go to the even code: 2.5 -> 2, 1.25 -> 1, 0.25 -> 0; 6 stays 6
    assert b[3, 0, 0].item() == 127
    assert np.array_equal(deq[3, :4], np.array([6.0, -2.0, 1.0, 0.0], dtype=np.float32))
    # the scale uses the largest power of two that keeps every block's maximum within E2M1 range
    top = np.abs(deq.reshape(5, 88, 32)).max(-1)
    nz = amax > 0
    assert np.all(top[nz] >= 4 * (2.0 ** X[nz]) - 1e-30)


def test_mxfp4_layer_matches_dense_reference_of_dequantised_weights():
    wl, x, w = small(T=12, E=6, K=2, D=256, F=192, seed=33, experts="mxfp4")
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 2, EPS)
    wf = f64_weights({k: v for k, v in wn.items() if k in ("router_w", "router_gamma", "ffn_gamma")})
    wf["router_bias"] = None
    E, D, Fd = 6, 256, 192
    gu = oracle.dequant_mxfp4(wn["mx4_gate_up"].reshape(E * 2 * Fd, -1), D)
    dn = oracle.dequant_mxfp4(wn["mx4_down"].reshape(E * D, -1), Fd)
    wf["w_gate_up"] = torch.from_numpy(gu.reshape(E, 2 * Fd, D)).double()
    wf["w_down"] = torch.from_numpy(dn.reshape(E, D, Fd)).double()
    ref, _, _ = dense_moe_fp64(bits_to_f64(xn), wf, 2, EPS)
    assert rel_err(o["out"], ref.numpy()) <= 2e-5


# E4M3 values fixed by the 8-bit floating-point format's definition (OCP): bias 7, three mantissa bits,
# exponent field 0 subnormal with step 2^-9, the smallest normal 2^-6, the largest 448, and the all-ones
# pattern NaN (no infinities).
E4M3_SPEC = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}


def test_mxfp8_codes_scales_and_layout():
    codes = np.arange(256, dtype=np.uint8)
    rows = np.zeros((8, 33), dtype=np.uint8)
    rows[:, 0] = 127
    rows[:, 1:] = codes.reshape(8, 32)
    deq = oracle.dequant_mxfp8(rows, 32).reshape(-1)
    for c, v in E4M3_SPEC.items():
        assert deq[c] == v and np.signbit(deq[c]) == np.signbit(v), hex(c)
    assert np.isnan(deq[0x7F]) and np.isnan(deq[0xFF])
    # every code against torch's own E4M3 decoder (a library routine of the same format)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    ok = ~np.isnan(lib)
    assert np.array_equal(np.isnan(deq), np.isnan(lib))
    assert np.array_equal(deq[ok], lib[ok]) and np.array_equal(np.signbit(deq[ok]), np.signbit(lib[ok]))
    # E8M0: byte e scales by 2^(e - 127); even 2^-127 times the smallest code stays exact in fp32
    for e, scale in [(128, 2.0), (126, 0.5), (120, 2.0 ** -7), (0, 2.0 ** -127), (200, 2.0 ** 73)]:
        r = rows.copy()
        r[:, 0] = e
        d = oracle.dequant_mxfp8(r, 32).reshape(-1)
        assert np.array_equal(d[ok], (lib[ok].astype(np.float64) * scale).astype(np.float32)), e
    r = rows.copy()
    r[:, 0] = 255
    assert np.all(np.isnan(oracle.dequant_mxfp8(r, 32)))
    # two blocks per row: block b covers inputs 32 b .. 32 b + 31, byte j of a block is input j
    two = np.zeros((1, 2, 33), dtype=np.uint8)
    two[0, 0, 0], two[0, 1, 0] = 127, 130  # 1 and 8
    two[0, :, 1:] = 0x38  # 1.0
    two[0, 1, 32] = 0xC0  # block 1, input 31: -2.0
    d2 = oracle.dequant_mxfp8(two.reshape(1, 66), 64)[0]
    assert np.array_equal(d2, np.array([1.0] * 32 + [8.0] * 31 + [-16.0], dtype=np.float32))


def test_mxfp8_quantiser_roundtrip():
    gen = torch.Generator().manual_seed(13)
    w = torch.randn((5, 2816), generator=gen) * 0.02
    w[2, 32:64] = 0.0  # an all-zero block
    # at scale 2^0 (amax 460 -> X = 8 - 8): 460 saturates to 448; -1.0625 and 1.1875 are ties between
    # neighbours 1/8 apart (-> the even mantissa: -1.0, 1.25); 2^-10 and 3 2^-10 are ties on the
    # subnormal grid (-> 0 and 2^-8); 300 rounds to 288 (step 32 above 256)
    w[3, 0:32] = torch.tensor([460.0, -1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 300.0] + [0.0] * 26)
    b = synth.quantize_mxfp8(w)
    assert b.shape == (5, 88, 33) and b.dtype == torch.uint8
    deq = oracle.dequant_mxfp8(b.numpy().reshape(5, -1), 2816)
    assert b[3, 0, 0].item() == 127
    assert np.array_equal(deq[3, :6], np.array([448.0, -1.0, 1.25, 0.0, 2.0 ** -8, 288.0], dtype=np.float32))
    assert np.all(deq[2, 32:64] == 0.0) and b[2, 1, 0].item() == 0
    wn = w.numpy()
    amax = np.abs(wn.reshape(5, 88, 32)).max(-1)
    X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127)
    assert np.array_equal(b[..., 0].numpy().astype(np.int64), (X + 127).astype(np.int64))
    # the codes are torch's round-to-nearest-even E4M3 conversion of w / 2^X clamped to +-448 (the
    # sign of a zero aside)
    v = torch.from_numpy(wn.reshape(5, 88, 32) / np.exp2(X)[..., None]).clamp(-448.0, 448.0)
    lib = v.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = b[..., 1:].numpy()
    assert np.array_equal(np.where(lib == 0x80, 0, lib), np.where(mine == 0x80, 0, mine))
    # error: at most half a step, 2^-4 of the magnitude (2^-10 of the scale near zero), unless saturated
    scale = np.repeat(2.0 ** X, 32, axis=1)
    sat = np.abs(wn) > 448 * scale
    err = np.abs(deq - wn)
    assert np.all(err[~sat] <= np.maximum(2.0 ** -4 * np.abs(wn), 2.0 ** -10 * scale)[~sat] + 1e-30)
    assert np.all(np.abs(deq[sat]) == (448 * scale)[sat])


def test_mxfp8_layer_matches_dense_reference_of_dequantised_weights():
    wl, x, w = small(T=12, E=6, K=2, D=256, F=192, seed=34, experts="mxfp8")
    xn, wn = np_inputs(x, w)
    o = oracle.moe_forward(wn, xn, 2, EPS)
    wf = f64_weights({k: v for k, v in wn.items() if k in ("router_w", "router_gamma", "ffn_gamma")})
    wf["router_bias"] = None
    E, D, Fd = 6, 256, 192
    gu = oracle.dequant_mxfp8(wn["mx8_gate_up"].reshape(E * 2 * Fd, -1), D)
    dn = oracle.dequant_mxfp8(wn["mx8_down"].reshape(E * D, -1), Fd)
    wf["w_gate_up"] = torch.from_numpy(gu.reshape(E, 2 * Fd, D)).double()
    wf["w_down"] = torch.from_numpy(dn.reshape(E, D, Fd)).double()
    ref, _, _ = dense_moe_fp64(bits_to_f64(xn), wf, 2, EPS)
    assert rel_err(o["out"], ref.numpy()) <= 2e-5


# ----------------------------------------------------------------------------- canvas output stage


def _head_small(T=7, V=600, D=96, seed=5, max_margin=24.0):
    hw = synth.HeadWorkload("t", T, V, D, seed, max_margin)
    inp = synth.make_head_inputs(hw)
    return synth.to_numpy_bits(inp["h"]), synth.to_numpy_bits(inp["emb"])


def test_output_stage_workload_from_the_pages():
    with open(os.path.join(GOLDEN, "output_stage.json")) as f:
        g = json.load(f)
    with open(os.path.join(GOLDEN, "expert_shapes.json")) as f:
        e = json.load(f)
    hw = synth.HEAD_WORKLOADS["head256"]
    # the tied head reads the token embedding [vocab, d_model] at 16 bits and writes fp32 logits for the
    # whole canvas
    assert g["tie_word_embeddings"] and g["embed_tokens_bits"] == 16 and g["logits_dtype"] == "f32"
    assert (hw.T, hw.V, hw.D) == (g["canvas_length"], g["vocab"], e["expert_linears"]["gate_proj"]["in_features"])
    assert g["canvas_length"] == e["canvas_length"]
    inp = synth.make_head_inputs(synth.HeadWorkload("t", 4, 512, 64, 1))
    assert inp["emb"].dtype == torch.bfloat16 and inp["h"].dtype == torch.bfloat16


def test_canvas_head_logits_match_a_library_matmul():
    h, emb = _head_small()
    r = oracle.canvas_head(h, emb, want_logits=True)
    ref = (bits_to_f64(h) @ bits_to_f64(emb).T).numpy()  # a library fp64 matmul of the exact bf16 values
    assert np.max(np.abs(r["logits"] - ref)) <= 1e-12 * np.max(np.abs(ref))
    # argmax (lowest id on ties) and the top-1 / top-2 gap against numpy
    assert np.array_equal(r["argmax"], np.argmax(ref, axis=1))
    srt = np.sort(ref, axis=1)
    assert np.allclose(r["gap"], srt[:, -1] - srt[:, -2], rtol=0, atol=1e-12)


@pytest.mark.parametrize("beta", [1.0, 1 / 0.8, 1 / 0.4])
def test_canvas_head_entropy_matches_library_routines(beta):
    from scipy.special import softmax
    from scipy.stats import entropy
    h, emb = _head_small(seed=6)
    r = oracle.canvas_head(h, emb, beta=beta, want_logits=True)
    ref = entropy(softmax(beta * r["logits"], axis=1), axis=1)  # nats
    assert np.max(np.abs(r["entropy"] - ref)) <= 1e-10
    assert np.all(r["entropy"] >= 0) and np.all(r["entropy"] <= np.log(600) + 1e-12)


def test_canvas_head_closed_forms():
    D, V = 64, 50
    gen = torch.Generator().manual_seed(9)
    emb = torch.randn((V, D), generator=gen).to(torch.bfloat16)
    # h = 0: every logit is 0, the softmax is uniform, H = ln V, the argmax is id 0, the gap 0
    h0 = torch.zeros((1, D), dtype=torch.bfloat16)
    r = oracle.canvas_head(synth.to_numpy_bits(h0), synth.to_numpy_bits(emb))
    assert abs(r["entropy"][0] - math.log(V)) <= 1e-12 and r["argmax"][0] == 0 and r["gap"][0] == 0.0
    # two tokens only, logits 0 and a: H = ln(1 + e^-a) + a e^-a / (1 + e^-a)
    e2 = torch.zeros((2, D), dtype=torch.bfloat16)
    e2[1, 0] = 1.0
    for a in [0.5, 2.0, 7.25]:
        h = torch.zeros((1, D), dtype=torch.bfloat16)
        h[0, 0] = a
        r = oracle.canvas_head(synth.to_numpy_bits(h), synth.to_numpy_bits(e2))
        want = math.log1p(math.exp(-a)) + a * math.exp(-a) / (1 + math.exp(-a))
        assert abs(r["entropy"][0] - want) <= 1e-12 and r["argmax"][0] == 1 and r["gap"][0] == a
    # two equal maxima far above the rest: H -> ln 2, the argmax the lower id
    e3 = torch.zeros((V, D), dtype=torch.bfloat16)
    e3[17, 1] = 1.0
    e3[9, 1] = 1.0
    h = torch.zeros((1, D), dtype=torch.bfloat16)
    h[0, 1] = 60.0
    r = oracle.canvas_head(synth.to_numpy_bits(h), synth.to_numpy_bits(e3))
    assert abs(r["entropy"][0] - math.log(2)) <= 1e-12 and r["argmax"][0] == 9 and r["gap"][0] == 0.0
    # one logit 80 above the rest: H ~ 0, and beta scales the margin
    e3[9, 1] = 0.0
    r = oracle.canvas_head(synth.to_numpy_bits(h), synth.to_numpy_bits(e3), beta=0.1)
    # logits: 60 on id 17, 0 elsewhere; at beta 0.1 the margin is 6 over V - 1 equal others
    p1 = 1 / (1 + (V - 1) * math.exp(-6.0))
    q = (1 - p1) / (V - 1)
    want = -(p1 * math.log(p1) + (V - 1) * q * math.log(q))
    assert abs(r["entropy"][0] - want) <= 1e-12 and r["argmax"][0] == 17


def test_canvas_head_input_recipe():
    # the margin puts the target on top once it clears the rest, and the entropies spread out
    hw = synth.HeadWorkload("t", 24, 4096, 256, 11)
    inp = synth.make_head_inputs(hw)
    r = oracle.canvas_head(synth.to_numpy_bits(inp["h"]), synth.to_numpy_bits(inp["emb"]))
    big = inp["margin"].numpy() > 16
    assert np.all(r["argmax"][big] == inp["target"].numpy()[big])
    assert r["entropy"][0] > 0.8 * math.log(4096) and r["entropy"][-1] < 1e-3
    assert np.min(r["entropy"]) < 0.1 and np.max(r["entropy"]) > 7.0


# ----------------------------------------------------------------------------- shapes printed on the pages

def test_shapes_from_the_pages():
    with open(os.path.join(GOLDEN, "expert_shapes.json")) as f:
        g = json.load(f)
    lin = g["expert_linears"]
    D = lin["gate_proj"]["in_features"]
    Fd = lin["gate_proj"]["out_features"]
    assert (lin["up_proj"]["in_features"], lin["up_proj"]["out_features"]) == (D, Fd)
    assert (lin["down_proj"]["in_features"], lin["down_proj"]["out_features"]) == (Fd, D)
    for wl in synth.WORKLOADS.values():
        assert (wl.E, wl.K, wl.D, wl.F) == (g["n_experts"], g["active_experts"], D, Fd)
    assert g["moe_modules_over_both_tied_stacks"] // 2 == synth.WORKLOADS["stack30"].layers
    assert synth.WORKLOADS["canvas256"].T == g["canvas_length"]
    assert g["quantization_config"]["group_size"] == synth.GROUP
    # parameters per expert: fused gate_up [2F, D] + down [D, F]
    assert 2 * Fd * D + D * Fd == 5_947_392
    # int4 storage per expert: nibbles + fp16 scales (the last down group is 64 wide)
    nib = (2 * Fd * D + D * Fd) // 2
    scales = 2 * (2 * Fd * (D // 128) + D * math.ceil(Fd / 128))
    assert nib + scales == 3_069_440
