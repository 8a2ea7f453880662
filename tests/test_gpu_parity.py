"""GPU parity of the HIP MoE layer against the CPU oracle, through the C ABI (MI355X only).

Every case prints what it runs before touching the GPU, so a failing run names its case.
"""
import numpy as np
import pytest
import torch

from expert_ffn_canvas_amd import synth
from tests.conftest import gpu_available
from tests.parity_util import OUT_TOL, host, layer_parity, oracle_weights, rel_max_err, to_f32

pytestmark = pytest.mark.gpu

if gpu_available():
    from expert_ffn_canvas_amd import dgmoe
    import oracle


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _layer(w, max_tokens, act, K=8, pack=False):
    return dgmoe.MoELayer(w, max_tokens=max_tokens, act_dtype=act, top_k=K, pack=pack)


def _act(wl):
    return torch.float32 if wl.act == "f32" else torch.bfloat16


@pytest.fixture(scope="module")
def canvas256():
    wl = synth.WORKLOADS["canvas256"]
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    return wl, inp["x"], w, oracle_weights(w)


# ----------------------------------------------------------------------------- small shapes

@pytest.mark.parametrize("E,K,D,F,T,act,rw", [
    (6, 2, 128, 64, 37, "bf16", "bf16"),
    (16, 4, 256, 128, 70, "f32", "f32"),
    (40, 8, 384, 192, 129, "bf16", "f32"),
    # many rows per expert (at least 64 on average: the tall-tile GEMMs), down K = 192 and K = 64
    (8, 4, 384, 192, 300, "bf16", "bf16"),
    (6, 2, 256, 64, 400, "bf16", "f32"),
    # about 350 rows per expert on average: about three tall tiles each
    (4, 2, 256, 128, 700, "bf16", "bf16"),
    # every token to both experts: 600 rows each, five tall tiles of 120 rows
    (2, 2, 256, 128, 600, "bf16", "bf16"),
    # just past the tall-tile threshold with a skewed load: tiles of every height
    (16, 8, 256, 128, 130, "bf16", "bf16"),
])
@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_small_shapes(E, K, D, F, T, act, rw, pack):
    _say(f"small E={E} K={K} D={D} F={F} T={T} act={act} router={rw} pack={pack}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, act=act, router_w=rw, bias="zipf", seed=E + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, _act(wl), K=K, pack=pack)
    r = layer_parity(layer, inp["x"], oracle_weights(w), K)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


@pytest.mark.parametrize("E,K,D,F,T", [
    (256, 8, 256, 128, 300),    # the most experts a layer may have
    (16, 8, 256, 128, 3000),    # k T = 24000 slots: past what the permutation stages in LDS; tall tiles
    (8, 2, 1024, 4096, 40),     # the largest d_ff: 64 gate_up column blocks, down over K = 4096
    (4, 1, 16384, 64, 20),      # the largest d_model: 128 router chunks, gate_up over K = 16384
])
def test_shape_limits(E, K, D, F, T):
    _say(f"limits E={E} K={K} D={D} F={F} T={T}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, bias="zipf", seed=80 + E)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    r = layer_parity(layer, inp["x"], oracle_weights(w), K)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")
    layer.close()


def test_single_expert_closed_form():
    _say("E=1 k=1 D=256 F=128 T=33")
    wl = synth.small_workload(T=33, E=1, K=1, D=256, F=128, seed=5)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, 33, torch.bfloat16, K=1)
    r = layer_parity(layer, inp["x"], oracle_weights(w), 1)
    assert np.all(r["dbg"]["topk_w"].cpu().numpy() == 1.0)


# ----------------------------------------------------------------------------- the five workloads

def test_canvas32_fp32():
    wl = synth.WORKLOADS["canvas32"]
    _say(f"{wl.name} T={wl.T}")
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, wl.T, torch.float32)
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


def test_canvas256_zipf(canvas256):
    wl, x, w, wn = canvas256
    _say(f"{wl.name} T={wl.T}")
    layer = _layer(w, wl.T, torch.bfloat16)
    r = layer_parity(layer, x, wn, wl.K)
    counts = r["dbg"]["counts"].cpu().numpy()
    print(f"err {r['err']:.3e} near-ties {r['near_ties']} touched {int((counts > 0).sum())} max {counts.max()}")
    assert (counts > 0).sum() < wl.E  # the skew leaves experts empty


def test_encode2304_sampled():
    wl = synth.WORKLOADS["encode2304"]
    _say(f"{wl.name} T={wl.T}")
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, wl.T, torch.bfloat16)
    rng = np.random.default_rng(0)
    tok = np.unique(np.concatenate([[0, 1, wl.T - 1], rng.choice(wl.T, 125, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_int4_g128(pack):
    wl = synth.WORKLOADS["int4"]
    _say(f"{wl.name} T={wl.T} pack={pack}")
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, wl.T, torch.bfloat16, pack=pack)
    rng = np.random.default_rng(1)
    tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 100, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


@pytest.mark.parametrize("E,K,T", [(12, 3, 50), (8, 4, 200)])
@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_int4_small_tail_group(E, K, T, pack):
    # d_ff = 192 = 128 + 64: the down projection's last scale group is 64 wide;
    # T = 200 on 8 experts fills tiles of up to 64 rows
    _say(f"int4 small E={E} K={K} D=256 F=192 T={T} pack={pack}")
    wl = synth.small_workload(T=T, E=E, K=K, D=256, F=192, experts="i4g128", seed=8 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=pack)
    layer_parity(layer, inp["x"], oracle_weights(w), K)


def test_q8_0():
    wl = synth.WORKLOADS["q8"]
    _say(f"{wl.name} T={wl.T} pack=True")
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, wl.T, torch.bfloat16, pack=True)
    rng = np.random.default_rng(2)
    tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 100, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


@pytest.mark.parametrize("E,K,D,F,T", [
    (12, 3, 256, 192, 50),   # down K = 192: a last 128-input step holding two Q8_0 blocks
    (8, 4, 256, 192, 200),   # tiles of up to 64 rows
    (6, 2, 128, 64, 37),     # gate_up K = 128 (one step), down K = 64 (a lone short step)
    (4, 2, 384, 320, 300),   # gate_up three steps, down two full steps and a short one
    (16, 8, 256, 192, 1),    # one token: eight one-row tiles, every other expert empty
])
def test_q8_0_small(E, K, D, F, T):
    _say(f"q8_0 small E={E} K={K} D={D} F={F} T={T}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, experts="q8_0", bias="zipf", seed=20 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    r = layer_parity(layer, inp["x"], oracle_weights(w), K)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


def test_mxfp4():
    wl = synth.WORKLOADS["mxfp4"]
    _say(f"{wl.name} T={wl.T} pack=True")
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, wl.T, torch.bfloat16, pack=True)
    rng = np.random.default_rng(3)
    tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 100, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


@pytest.mark.parametrize("E,K,D,F,T", [
    (12, 3, 256, 192, 50),   # down K = 192: a last 128-input step holding two blocks
    (8, 4, 256, 192, 200),   # tiles of up to 64 rows
    (6, 2, 128, 64, 37),     # gate_up K = 128 (one step), down K = 64 (a lone short step)
    (4, 2, 384, 320, 300),   # gate_up three steps, down two full steps and a short one
    (16, 8, 256, 192, 1),    # one token: eight one-row tiles, every other expert empty
])
def test_mxfp4_small(E, K, D, F, T):
    _say(f"mxfp4 small E={E} K={K} D={D} F={F} T={T}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, experts="mxfp4", bias="zipf", seed=40 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    r = layer_parity(layer, inp["x"], oracle_weights(w), K)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


def test_mxfp8():
    wl = synth.WORKLOADS["mxfp8"]
    _say(f"{wl.name} T={wl.T} pack=True")
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, wl.T, torch.bfloat16, pack=True)
    rng = np.random.default_rng(4)
    tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 100, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


@pytest.mark.parametrize("E,K,D,F,T,jitter", [
    (12, 3, 256, 192, 50, 0),   # down K = 192: a last 128-input step holding two blocks
    (8, 4, 256, 192, 200, 6),   # tiles of up to 64 rows; every block's scale byte moved by -6..6
    (6, 2, 128, 64, 37, 0),     # gate_up K = 128 (one step), down K = 64 (a lone short step)
    (4, 2, 384, 320, 300, 3),   # gate_up three steps, down two full steps and a short one
    (16, 8, 256, 192, 1, 0),    # one token: eight one-row tiles, every other expert empty
])
def test_mxfp8_small(E, K, D, F, T, jitter):
    _say(f"mxfp8 small E={E} K={K} D={D} F={F} T={T} jitter={jitter}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, experts="mxfp8", bias="zipf", seed=60 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    if jitter:  # per-block scales far apart, so a block read with another block's scale shows
        gen = torch.Generator(device="cpu").manual_seed(T)
        for key in ("mx8_gate_up", "mx8_down"):
            sc = w[key][..., 0].to(torch.int32)
            off = torch.randint(-jitter, jitter + 1, sc.shape, generator=gen).to(sc.device)
            w[key][..., 0] = (sc + off).clamp(1, 254).to(torch.uint8)
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    r = layer_parity(layer, inp["x"], oracle_weights(w), K)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")


# ----------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("T", [1, 15, 17, 255, 257])
def test_ragged_token_counts(canvas256, T):
    wl, x, w, wn = canvas256
    _say(f"ragged T={T}")
    gen = torch.Generator(device="cuda").manual_seed(100 + T)
    xt = torch.randn((T, wl.D), generator=gen, device="cuda").to(torch.bfloat16)
    layer = _layer(w, 300, torch.bfloat16)
    layer_parity(layer, xt, wn, wl.K)


def test_zero_tokens_is_a_no_op(canvas256):
    wl, x, w, wn = canvas256
    _say("T=0")
    layer = _layer(w, 16, torch.bfloat16)
    out = torch.full((1, wl.D), 7.0, dtype=torch.bfloat16, device="cuda")
    st = dgmoe.dg_moe_forward(layer.handle, x.data_ptr(), out.data_ptr(), 0, None, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert st == dgmoe.DG_OK
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_all_tokens_forced_to_one_expert(canvas256):
    # bias +30 on one expert: every token picks it first with weight ~1, it receives all T rows
    # (three tiles), and most experts stay empty.
    wl, x, w, wn = canvas256
    T = 300
    _say(f"forced expert 7, T={T}")
    w2 = dict(w)
    b = torch.zeros(wl.E, device="cuda")
    b[7] = 30.0
    w2["router_bias"] = b
    gen = torch.Generator(device="cuda").manual_seed(7)
    xt = torch.randn((T, wl.D), generator=gen, device="cuda").to(torch.bfloat16)
    layer = _layer(w2, T, torch.bfloat16, K=1)
    wn2 = dict(wn)
    wn2["router_bias"] = host(b)
    r = layer_parity(layer, xt, wn2, 1)
    counts = r["dbg"]["counts"].cpu().numpy()
    assert counts[7] == T and counts.sum() == T
    # identity: with k = 1 the output is that expert's FFN of the normalised input
    assert np.all(r["dbg"]["topk_w"].cpu().numpy() == 1.0)


def test_identical_experts_any_routing():
    # all experts share one weight set: the output is the dense FFN whatever the routing
    _say("identical experts E=16 K=4 D=2816 F=704 T=96")
    wl = synth.small_workload(T=96, E=16, K=4, D=2816, F=704, bias="zipf", seed=9)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    w["w_gate_up"] = w["w_gate_up"][:1].expand(16, -1, -1).contiguous()
    w["w_down"] = w["w_down"][:1].expand(16, -1, -1).contiguous()
    layer = _layer(w, 96, torch.bfloat16, K=4)
    out = to_f32(layer.forward(inp["x"]))
    wn = oracle_weights(w)
    xn = host(inp["x"])
    # closed form: expert 0 alone, through the oracle's single-expert FFN on the normalised input
    rt = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn["router_bias"], 4, synth.RMS_EPS)
    h = (xn.view(np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64) * rt["r"][:, None] \
        * (1.0 + wn["ffn_gamma"].astype(np.float64))
    ref = oracle.expert_ffn(wn, 0, h.astype(np.float32))
    assert rel_max_err(out, ref) <= OUT_TOL


def test_determinism(canvas256):
    wl, x, w, wn = canvas256
    _say("determinism")
    layer = _layer(w, wl.T, torch.bfloat16)
    a = layer.forward(x).clone()
    b = layer.forward(x).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_fold_invariance_bit_exact(canvas256):
    # moving a power-of-two scale from the expert norm into gate_up's input columns leaves the routing and
    # (with exact powers of two) every product unchanged
    wl, x, w, wn = canvas256
    _say("fold invariance")
    gen = torch.Generator(device="cuda").manual_seed(3)
    g = torch.randint(-256, 256, (wl.D,), generator=gen, device="cuda").float() / 1024.0
    s = torch.tensor([0.5, 1.0, 2.0], device="cuda")[torch.randint(0, 3, (wl.D,), generator=gen, device="cuda")]
    w1 = dict(w)
    w1["ffn_gamma"] = g
    w2 = dict(w)
    w2["ffn_gamma"] = (1.0 + g) / s - 1.0
    w2["w_gate_up"] = (w["w_gate_up"].float() * s).to(torch.bfloat16)
    l1 = _layer(w1, wl.T, torch.bfloat16)
    l2 = _layer(w2, wl.T, torch.bfloat16)
    d1 = l1.forward_debug(x)
    d2 = l2.forward_debug(x)
    torch.cuda.synchronize()
    assert torch.equal(d1["topk_idx"], d2["topk_idx"])
    assert torch.equal(d1["topk_w"], d2["topk_w"])
    assert torch.equal(d1["out"].view(torch.int16), d2["out"].view(torch.int16))


def test_pack_equals_borrow(canvas256):
    # Packing changes the weight layout only, except that with bf16 activations the packed gate_up also
    # carries the expert norm's (1 + gamma), rounded to bf16 with the weight (h is then never formed). The
    # routing does not depend on the experts' storage; with fp32 activations nothing is folded and the
    # outputs are bit-identical; with bf16 ones the two roundings differ by a few bf16 ulps.
    wl, x, w, wn = canvas256
    _say("pack vs borrow")
    a = _layer(w, wl.T, torch.bfloat16).forward_debug(x)
    b = _layer(w, wl.T, torch.bfloat16, pack=True).forward_debug(x)
    x32 = x.float()
    a32 = _layer(w, wl.T, torch.float32).forward(x32)
    b32 = _layer(w, wl.T, torch.float32, pack=True).forward(x32)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_w", "sorted_slot", "row_of_slot"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a32.view(torch.int32), b32.view(torch.int32))
    err = rel_max_err(to_f32(b["out"]), to_f32(a["out"]))
    print(f"folded vs materialised expert input: max|d|/max|ref| = {err:.3e}")
    assert err <= 1e-2


def test_residual_and_addend(canvas256):
    wl, x, w, wn = canvas256
    _say("residual + addend")
    gen = torch.Generator(device="cuda").manual_seed(11)
    add = (torch.randn(x.shape, generator=gen, device="cuda") * 0.5).to(torch.bfloat16)
    layer = _layer(w, wl.T, torch.bfloat16)
    moe = to_f32(layer.forward(x))
    full = to_f32(layer.forward(x, addend=add, add_input=True))
    tok = np.arange(0, wl.T, 4)
    ref = oracle.moe_forward(wn, host(x), wl.K, synth.RMS_EPS, tokens=tok)["out"]
    exact = ref + to_f32(x)[tok] + to_f32(add)[tok]
    # bf16 rounding of the sum can move by one ulp of the sum when the MoE part differs within tolerance
    ulp = np.abs(exact) * 2.0 ** -7
    assert np.all(np.abs(full[tok] - exact) <= ulp + OUT_TOL * np.max(np.abs(ref)))
    assert rel_max_err(moe[tok], ref) <= OUT_TOL


def test_error_paths_on_device(canvas256):
    wl, x, w, wn = canvas256
    _say("error paths")
    layer = _layer(w, 64, torch.bfloat16)
    out = torch.empty((128, wl.D), dtype=torch.bfloat16, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    assert dgmoe.dg_moe_forward(layer.handle, x.data_ptr(), out.data_ptr(), 65, None, 0, sp) == dgmoe.DG_ERR_SHAPE
    assert "max_tokens" in dgmoe.dg_moe_last_error()
    assert dgmoe.dg_moe_forward(layer.handle, x.data_ptr(), x.data_ptr(), 8, None, 0, sp) == dgmoe.DG_ERR_INVALID_ARG
    assert dgmoe.dg_moe_forward(layer.handle, x.data_ptr(), out.data_ptr(), 8, None, 0x10, sp) == \
        dgmoe.DG_ERR_INVALID_ARG
    assert dgmoe.dg_moe_forward(layer.handle, x.data_ptr() + 2, out.data_ptr(), 8, None, 0, sp) == dgmoe.DG_ERR_ALIGN


def test_stack30_teacher_forced():
    # 30 layers with their own weights (45.7 GB of bf16 experts resident), T = 512 (two canvases):
    # x_{l+1} = bf16(x_l + MoE_l(x_l) + delta_l). Each checked layer is compared on its own GPU input.
    wl = synth.WORKLOADS["stack30"]
    _say(f"{wl.name} T={wl.T} layers={wl.layers}")
    inp = synth.make_inputs(wl, device="cuda")
    layers = [_layer(w, wl.T, torch.bfloat16) for w in inp["layers"]]
    xs = [inp["x"]]
    for l in range(wl.layers):
        xs.append(layers[l].forward(xs[l], addend=inp["deltas"][l], add_input=True))
    torch.cuda.synchronize()
    assert all(torch.isfinite(t.float()).all() for t in xs)
    rng = np.random.default_rng(4)
    for l in (0, 13, 29):
        _say(f"{wl.name} layer {l}")
        wn = oracle_weights(inp["layers"][l])
        tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 40, replace=False)]))
        r = layer_parity(layers[l], xs[l], wn, wl.K, tokens=tok)
        # the residual path of the same layer: bf16(x + MoE + delta) within one bf16 ulp of the sum
        exact = r["ref"]["out"] + to_f32(xs[l])[tok] + to_f32(inp["deltas"][l])[tok]
        got = to_f32(xs[l + 1])[tok]
        ulp = np.abs(exact) * 2.0 ** -7
        assert np.all(np.abs(got - exact) <= ulp + OUT_TOL * np.max(np.abs(r["ref"]["out"])))
        print(f"layer {l}: err {r['err']:.3e} near-ties {r['near_ties']} "
              f"touched {(r['dbg']['counts'].cpu().numpy() > 0).sum()}")
    for layer in layers:
        layer.close()


def test_profiled_forward_times_each_kernel(canvas256):
    import ctypes
    wl, x, w, wn = canvas256
    _say("profiled forward: 12 dispatch-stamped events")
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(12):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    layer = _layer(w, wl.T, torch.bfloat16)
    out = torch.empty_like(x)
    sp = torch.cuda.current_stream().cuda_stream
    ref = layer.forward(x)
    st = dgmoe.dg_moe_forward_profiled(layer.handle, x.data_ptr(), out.data_ptr(), wl.T, None, 0, evs, sp)
    assert st == 0, dgmoe.dg_moe_last_error()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    ms = []
    for k in range(6):
        t = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(t), evs[2 * k], evs[2 * k + 1]) == 0
        ms.append(t.value)
    print("kernel ms", [round(v, 4) for v in ms])
    # the norm (folded here) and the down GEMM (fused with gate_up for bf16 experts) bracket no launch of
    # their own: their pairs are recorded back to back
    assert all(v >= 0 for v in ms)
    assert all(ms[k] > 0 for k in (1, 2, 3, 5))
    # a NULL event is rejected before anything is launched
    bad = list(evs)
    bad[7] = None
    assert dgmoe.dg_moe_forward_profiled(layer.handle, x.data_ptr(), out.data_ptr(), wl.T, None, 0, bad, sp) == \
        dgmoe.DG_ERR_INVALID_ARG
    for e in evs:
        hip.hipEventDestroy(e)
