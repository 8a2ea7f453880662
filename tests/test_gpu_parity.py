"""GPU parity of the HIP MoE layer against the CPU oracle, through the C ABI (MI355X only).

Every case prints what it runs before touching the GPU, so a failing run names its case.
"""
import numpy as np
import pytest
import torch

from expert_ffn_canvas_amd import synth
from tests.conftest import gpu_available
from tests.parity_util import (OUT_TOL, check_device_state, check_permutation, check_routing_many, host,
                               layer_parity, oracle_weights, rel_max_err, to_f32)

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
    (16, 8, 256, 128, 3000),    # eight scatter workgroups of 375 tokens (ranges off the 1024-token
                                # chunks, staged in LDS); wide tiles
    (16, 8, 256, 128, 24000),   # eight scatter workgroups of 3000 tokens (three chunks, the last one
                                # partial): 24000 slots of a range, past what one stages in LDS, so
                                # written directly
    (8, 2, 1024, 4096, 40),     # the largest d_ff: 64 gate_up column blocks, down over K = 4096
    (4, 1, 16384, 64, 20),      # the largest d_model: 128 router chunks, gate_up over K = 16384
])
def test_shape_limits(E, K, D, F, T):
    _say(f"limits E={E} K={K} D={D} F={F} T={T}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, bias="zipf", seed=80 + E)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    # routing and permutation are checked for every token; outputs on a sample past 10000 tokens
    tok = None if T <= 10000 else np.unique(np.concatenate(
        [np.arange(0, T, 997), np.arange(T - 40, T), np.random.default_rng(T).choice(T, 200, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")
    layer.close()


def test_max_tokens():
    # the largest token count a layer accepts (max_tokens = 2^20), with K T D = 2^32 expert-output elements
    # and K T F = 2^32 gated activations, so every offset into y and act needs 64 bits; wide tiles (524288
    # rows per expert, 3277 tiles each). Routing and permutation over all tokens, outputs on a sample.
    T, E, K, D, F = 1 << 20, 16, 8, 512, 512
    _say(f"max tokens E={E} K={K} D={D} F={F} T={T}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, bias="zipf", seed=97)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    dbg = layer.forward_debug(inp["x"])
    torch.cuda.synchronize()
    xn, wn = host(inp["x"]), oracle_weights(w)
    orc = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn.get("router_bias"), K, synth.RMS_EPS)
    gidx = dbg["topk_idx"].cpu().numpy()
    check_routing_many(gidx, dbg["topk_w"].cpu().numpy(), orc, K, T)
    check_permutation(dbg, K, E, T)
    check_device_state(dbg, K, E, T, D, F, balanced=layer.gemms_fused)
    tok = np.unique(np.concatenate([[0, 1, T - 1], np.arange(0, T, 8191),
                                    np.random.default_rng(97).choice(T, 200, replace=False)]))
    ref = oracle.moe_forward(wn, xn, K, synth.RMS_EPS, forced=gidx, tokens=tok)
    gout = dbg["out"][torch.from_numpy(tok).to(dbg["out"].device)].float().cpu().numpy()
    err = rel_max_err(gout, ref["out"])
    print(f"{len(tok)} tokens: err {err:.3e}")
    assert np.all(np.isfinite(gout))
    assert err <= OUT_TOL, f"max|d|/max|ref| = {err:.3e} > {OUT_TOL}"
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


# pack=True is the path the benchmark times: packed fragment-order experts with the expert norm's (1 + gamma)
# folded into gate_up (the GEMM reads x and scales its sums by r); pack=False materialises h and reads the
# caller's row-major weights.
@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_canvas256_zipf(canvas256, pack):
    wl, x, w, wn = canvas256
    _say(f"{wl.name} T={wl.T} pack={pack}")
    layer = _layer(w, wl.T, torch.bfloat16, pack=pack)
    r = layer_parity(layer, x, wn, wl.K)
    counts = r["dbg"]["counts"].cpu().numpy()
    print(f"err {r['err']:.3e} near-ties {r['near_ties']} touched {int((counts > 0).sum())} max {counts.max()}")
    assert (counts > 0).sum() < wl.E  # the skew leaves experts empty
    layer.close()


@pytest.fixture(scope="module")
def encode2304():
    wl = synth.WORKLOADS["encode2304"]
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    return wl, inp["x"], w, oracle_weights(w)


@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_encode2304_sampled(encode2304, pack):
    wl, x, w, wn = encode2304
    _say(f"{wl.name} T={wl.T} pack={pack}")
    layer = _layer(w, wl.T, torch.bfloat16, pack=pack)
    rng = np.random.default_rng(0)
    tok = np.unique(np.concatenate([[0, 1, wl.T - 1], rng.choice(wl.T, 125, replace=False)]))
    r = layer_parity(layer, x, wn, wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")
    layer.close()


# The router's kernel variant depends on T, the number of experts, the CU count and the activation type:
# 16, 32, 64 or 80 tokens per workgroup (the height that fills the CUs in the fewest rounds for the bytes
# each workgroup reads), two workgroups per expert tile when the 16-token tiles give at most 64, fp32 rows
# held in registers (at most 32 tokens). These cases reach each variant at the model's E = 128 and d_model
# on a 256-CU device, with a ragged last token tile.
@pytest.mark.parametrize("T,act,variant", [
    (1000, "bf16", "bf16 x, 32-token workgroups, ragged last tile (1000 = 31 x 32 + 8)"),
    (1500, "bf16", "bf16 x, 64-token workgroups, ragged last tile (1500 = 23 x 64 + 28)"),
    (2200, "bf16", "bf16 x, 80-token workgroups, ragged last tile (2200 = 27 x 80 + 40)"),
    (256, "f32", "fp32 x, 16-token workgroups, one per expert tile"),
    (1500, "f32", "fp32 x, 32-token workgroups, ragged last tile"),
    (40, "f32", "fp32 x, 16-token workgroups, two per expert tile, ragged"),
    (40, "bf16", "bf16 x, 16-token workgroups, two per expert tile, ragged"),
])
def test_router_variants(T, act, variant):
    _say(f"router variant T={T} act={act}: {variant}")
    wl = synth.small_workload(T=T, E=128, K=8, D=2816, F=704, act=act, router_w="bf16", bias="zipf",
                              seed=200 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, _act(wl), pack=True)
    rng = np.random.default_rng(T)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, min(T, 60), replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")
    layer.close()


# Tiles of 64 or 80 tokens whose launch fits the CUs at once share the top-k selection out among their
# workgroups (each waits, a bounded number of polls, for the tile's last logits, then selects for its share);
# a workgroup that stops waiting leaves its share to the last arriver. DG_FWD_ROUTER_NO_WAIT makes every
# workgroup stop at once. Both paths must give the same bits, run right after a forward of other input, so
# that a share nobody selected would keep that forward's routing and show.
@pytest.mark.parametrize("T,E,D,F,case", [
    (2200, 128, 512, 128, "80-token tiles, 8 shares of 10 tokens"),
    (1500, 128, 512, 128, "64-token tiles, 8 shares of 8 tokens, ragged last tile"),
    (3000, 40, 512, 128, "64-token tiles, 3 shares of 21-22 tokens, ragged last tile"),
])
def test_router_shared_selection(T, E, D, F, case):
    _say(f"router shared selection T={T} E={E}: {case}")
    wl = synth.small_workload(T=T, E=E, K=8, D=D, F=F, act="bf16", router_w="bf16", bias="zipf", seed=300 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    x2 = inp["x"]
    x1 = torch.roll(x2, shifts=7, dims=0).contiguous()
    layer = _layer(w, T, torch.bfloat16, pack=True)
    o1 = layer.forward(x1).clone()
    o_nowait = layer.forward(x2, router_no_wait=True).clone()
    o_wait = layer.forward(x2).clone()
    o1b = layer.forward(x1).clone()
    o_nowait2 = layer.forward(x2, router_no_wait=True).clone()
    torch.cuda.synchronize()
    assert not torch.equal(o1.view(torch.int16), o_wait.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o1b.view(torch.int16))
    assert torch.equal(o_nowait.view(torch.int16), o_wait.view(torch.int16))
    assert torch.equal(o_nowait2.view(torch.int16), o_wait.view(torch.int16))
    rng = np.random.default_rng(T)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 40, replace=False)]))
    r = layer_parity(layer, x2, oracle_weights(w), wl.K, tokens=tok)
    print(f"err {r['err']:.3e} near-ties {r['near_ties']}")
    layer.close()


def test_adversarial_expert_loads():
    # Six experts take every token (bias +30) and 24 more most of the other two slots (bias +3), at expert
    # ids placed so that dealing the larger experts in id order would stack three of the six on one queue;
    # the rest (bias +1) get a few rows each. The deal by size keeps the queues within the balance bound,
    # every task runs, and the output meets the oracle.
    T, E = 1000, 128
    _say(f"adversarial expert loads E={E} T={T}")
    wl = synth.small_workload(T=T, E=E, K=8, D=2816, F=704, act="bf16", router_w="bf16", seed=31)
    inp = synth.make_inputs(wl, device="cuda")
    w = dict(inp["layers"][0])
    heavy = [0, 1, 14, 15, 16, 17]
    b = torch.full((E,), 1.0)
    b[:30] = 3.0
    b[heavy] = 30.0
    w["router_bias"] = b.to("cuda")
    layer = _layer(w, T, torch.bfloat16, pack=True)
    rng = np.random.default_rng(5)
    tok = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 60, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), wl.K, tokens=tok)
    counts = r["dbg"]["counts"].cpu().numpy()
    assert np.all(counts[heavy] == T)
    ql = r["dbg"]["queue_len"].cpu().numpy()
    print(f"err {r['err']:.3e} gate_up queues {ql[:8]} down queues {ql[8:16]} capacity {ql[16:]}")
    layer.close()


def _routed_inputs(T, E, D, choices, seed):
    """A layer whose router picks exactly choices[t] (k expert ids, in slot order) for every token t: the router
    weight is the identity on the first E inputs, x[t] holds 3 + k - j at input choices[t][j] and 0 elsewhere,
    and gamma_r = 0, so logit_e = r x[t, e] with every chosen logit at least 2 above every other."""
    K = len(choices[0])
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=64, act="bf16", router_w="bf16", seed=seed)
    inp = synth.make_inputs(wl, device="cuda")
    w = dict(inp["layers"][0])
    rw = torch.zeros((E, D), dtype=torch.float32)
    rw[torch.arange(E), torch.arange(E)] = 1.0
    w["router_w"] = rw.to(torch.bfloat16).to("cuda")
    w["router_gamma"] = torch.zeros(D, device="cuda")
    x = torch.zeros((T, D), dtype=torch.float32)
    for t, ch in enumerate(choices):
        for j, e in enumerate(ch):
            x[t, e] = 3.0 + K - j
    return wl, x.to(torch.bfloat16).to("cuda"), w


def test_deal_falls_back_to_size_order():
    # Exact routing (no near ties): 5 experts take every token (16 tiles of 64 rows each), 28 take 65 rows
    # (2 tiles), 95 share the rest (1 tile each). The larger experts dealt in id order would put the five big
    # ones (ids 0, 15, 16, 31, 32: snake positions that all land on queue 0) on one queue, 80 tiles against a
    # capacity of 64; the permutation sees that and deals the larger experts again in order of size. Every
    # task runs (no overflow), the queues stay within the balance bound, and the output meets the oracle.
    T, E, D, K = 1000, 128, 256, 8
    _say(f"deal fallback E={E} T={T}: five experts take every token")
    big = [0, 15, 16, 31, 32]
    mid = [e for e in range(33) if e not in big]
    rest = list(range(33, 128))
    seq = [mid[i % 28] for i in range(28 * 65)]
    seq += [rest[i % 95] for i in range(3 * T - len(seq))]
    choices = [big + seq[3 * t:3 * t + 3] for t in range(T)]
    wl, x, w = _routed_inputs(T, E, D, choices, seed=77)
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    r = layer_parity(layer, x, oracle_weights(w), K)
    counts = r["dbg"]["counts"].cpu().numpy()
    assert np.all(counts[big] == T) and np.all(counts[mid] == 65) and np.all(counts[rest] <= 64)
    ql = r["dbg"]["queue_len"].cpu().numpy()
    print(f"gate_up queue tiles {ql[:8]}, capacity {ql[16]}")
    assert ql[:8].max() < 5 * 16  # the five big experts are not on one queue
    layer.close()


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


@pytest.mark.parametrize("E,K,T,bias", [(12, 3, 50, None), (8, 4, 200, None), (16, 2, 150, "zipf")])
@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_int4_small_tail_group(E, K, T, bias, pack):
    # d_ff = 192 = 128 + 64: the down projection's last scale group is 64 wide. Packed, up to 20 rows per
    # expert on average run in 32-row tiles (T = 50 on 12 experts; T = 150 on 16 with a skew that puts some
    # experts in two of them), more in 64-row tiles (T = 200 on 8 experts)
    _say(f"int4 small E={E} K={K} D=256 F=192 T={T} bias={bias} pack={pack}")
    wl = synth.small_workload(T=T, E=E, K=K, D=256, F=192, experts="i4g128", bias=bias, seed=8 + T)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=pack)
    layer_parity(layer, inp["x"], oracle_weights(w), K)


@pytest.mark.parametrize("pack", [False, True], ids=["borrow", "pack"])
def test_int4_long_rows(pack):
    # d_model 8192: 64 scale groups per gate_up row, more than the packed kernel keeps in LDS, so its gate_up
    # loads each group's scales with the codes, while its down GEMM (d_ff 192: two groups, the last 64 wide)
    # keeps them in LDS
    T, E, K, D, F = 40, 6, 2, 8192, 192
    _say(f"int4 long rows E={E} K={K} D={D} F={F} T={T} pack={pack}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, experts="i4g128", bias="zipf", seed=71)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=pack)
    r = layer_parity(layer, inp["x"], oracle_weights(w), K)
    print(f"err {r['err']:.3e}")
    layer.close()


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


@pytest.mark.parametrize("experts", ["i4g128", "q8_0", "mxfp4", "mxfp8"])
def test_quantised_many_tiles(experts):
    # T = 32768 over 16 experts (Zipf): 64-row tiles, about 256 of them per expert, so every weight block is
    # read through the caches by many tiles; d_ff 192 gives the down GEMM a 64-input last step. Routing and
    # permutation on every token, outputs on a sample.
    T, E, K, D, F = 32768, 16, 8, 256, 192
    _say(f"{experts} many tiles E={E} K={K} D={D} F={F} T={T}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, experts=experts, bias="zipf", seed=61)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    layer = _layer(w, T, torch.bfloat16, K=K, pack=True)
    tok = np.unique(np.concatenate([[0, T - 1], np.arange(0, T, 997), np.random.default_rng(61).choice(T, 150, replace=False)]))
    r = layer_parity(layer, inp["x"], oracle_weights(w), K, tokens=tok)
    counts = r["dbg"]["counts"].cpu().numpy()
    assert counts.max() >= 64 * 64, "the largest expert should span many 64-row tiles"
    print(f"err {r['err']:.3e} near-ties {r['near_ties']} largest expert {counts.max()} rows")
    layer.close()


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


def test_device_status_word_stays_clear(canvas256):
    # 50 forwards of the benchmarked path: no workgroup ran off its XCD, no queue overflowed, no down task
    # timed out (the word is sticky, so one read after all of them covers every forward)
    wl, x, w, wn = canvas256
    _say("device status word over 50 forwards")
    layer = _layer(w, wl.T, torch.bfloat16, pack=True)
    for _ in range(50):
        layer.forward(x)
    dbg = layer.forward_debug(x)
    torch.cuda.synchronize()
    assert int(dbg["dev_flags"].cpu()[0]) == 0
    layer.close()


@pytest.mark.parametrize("experts,act", [("bf16", "bf16"), ("i4g128", "bf16"), ("mxfp4", "bf16"), ("bf16", "f32")])
def test_down_wait_timeout_reaches_the_host(experts, act):
    # The fused launch's down tasks forced (from the host) to give up their bounded wait at once: every one
    # writes NaN for its outputs and raises DG_DEV_WAIT_TIMEOUT, which the host reads back; every kernel ends
    # normally, another handle is untouched, and a forward of the same handle without the flag is correct
    # again (the bit stays set: the word is sticky).
    T, E, K, D, F = 96, 16, 4, 256, 128
    _say(f"down wait timeout {experts} act={act}")
    wl = synth.small_workload(T=T, E=E, K=K, D=D, F=F, act=act, router_w=act, experts=experts, seed=33)
    inp = synth.make_inputs(wl, device="cuda")
    w, x = inp["layers"][0], inp["x"]
    adt = _act(wl)
    forced = _layer(w, T, adt, K=K, pack=True)
    other = _layer(w, T, adt, K=K, pack=True)
    sp = torch.cuda.current_stream().cuda_stream
    out = torch.empty((T, D), dtype=adt, device="cuda")
    assert dgmoe.dg_moe_forward(forced.handle, x.data_ptr(), out.data_ptr(), T, None, dgmoe.DG_FWD_GEMM_NO_WAIT,
                                sp) == 0
    torch.cuda.synchronize()
    assert not torch.isfinite(out.float()).any(), "every output should be NaN once every down task gave up"
    r = layer_parity(forced, x, oracle_weights(w), K, check_state=False)  # the same handle, normal forward
    flags = int(r["dbg"]["dev_flags"].cpu()[0])
    assert flags == dgmoe.DG_DEV_WAIT_TIMEOUT, f"device status word 0x{flags:x}"
    r2 = layer_parity(other, x, oracle_weights(w), K)
    assert int(r2["dbg"]["dev_flags"].cpu()[0]) == 0
    forced.close()
    other.close()


def test_create_out_of_memory():
    # a workspace larger than the device (max_tokens 2^20 at d_model 16384, d_ff 4096: act and the per-slot
    # outputs alone need 8 * 2^20 * (4096 + 16384) * 2 bytes = 344 GB) is refused with DG_ERR_OOM at create
    _say("create: workspace beyond the device's memory")
    cfg = dgmoe.make_config(E=8, K=8, D=16384, F=4096, max_tokens=1 << 20)
    need = dgmoe.dg_moe_workspace_bytes(cfg)
    free, total = torch.cuda.mem_get_info()
    assert need > total
    wl = synth.small_workload(T=4, E=8, K=8, D=16384, F=64, seed=3)
    inp = synth.make_inputs(wl, device="cuda")
    w = inp["layers"][0]
    gu = torch.zeros((8, 2 * 4096, 128), dtype=torch.bfloat16, device="cuda")  # never read: create fails first
    wts = dgmoe.dg_moe_weights(w["router_w"].data_ptr(), w["router_gamma"].data_ptr(), 0,
                               w["ffn_gamma"].data_ptr(), gu.data_ptr(), gu.data_ptr(), 0, 0)
    st, h = dgmoe.dg_moe_create(cfg, wts, torch.cuda.current_stream().cuda_stream)
    assert st == dgmoe.DG_ERR_OOM, dgmoe.dg_moe_last_error()
    assert not h.value
    assert "workspace" in dgmoe.dg_moe_last_error()
    # the device is still usable
    layer = _layer(w, 4, torch.bfloat16)
    layer.forward(inp["x"])
    torch.cuda.synchronize()
    layer.close()


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
    # 30 layers with their own weights (45.7 GB of bf16 experts, packed at create as the benchmark runs them),
    # T = 512 (two canvases): x_{l+1} = bf16(x_l + MoE_l(x_l) + delta_l). Every layer is compared on its own
    # GPU input (teacher-forced) on sampled tokens; then the end of the stack is compared with the oracle
    # running all 30 layers on its own trajectory for a few tokens (the layer treats tokens independently).
    wl = synth.WORKLOADS["stack30"]
    _say(f"{wl.name} T={wl.T} layers={wl.layers} pack=True")
    inp = synth.make_inputs(wl, device="cuda")
    layers = [_layer(w, wl.T, torch.bfloat16, pack=True) for w in inp["layers"]]
    xs = [inp["x"]]
    for l in range(wl.layers):
        xs.append(layers[l].forward(xs[l], addend=inp["deltas"][l], add_input=True))
    torch.cuda.synchronize()
    assert all(torch.isfinite(t.float()).all() for t in xs)
    rng = np.random.default_rng(4)
    wns = []
    for l in range(wl.layers):
        _say(f"{wl.name} layer {l}")
        wn = oracle_weights(inp["layers"][l])
        wns.append(wn)
        tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 14, replace=False)]))
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
    # end of the stack: the oracle's own trajectory (fp32 residual rounded to bf16 after each layer, as the
    # stack defines it) for 16 tokens, against the GPU's x_30
    _say(f"{wl.name} end of stack")
    tok = np.unique(np.concatenate([[0, wl.T - 1], rng.choice(wl.T, 14, replace=False)]))
    xo = host(xs[0])[tok].copy()
    near_any = np.zeros(len(tok), dtype=bool)
    for l in range(wl.layers):
        d = host(inp["deltas"][l])[tok].copy()
        ref = oracle.moe_forward(wns[l], xo, wl.K, synth.RMS_EPS, add_input=True, addend=d)
        near_any |= ref["gap"] < 1e-4
        xo = synth.to_numpy_bits(torch.from_numpy(ref["out"]).to(torch.bfloat16))
    gpu_end = to_f32(xs[-1])[tok]
    ref_end = (xo.astype(np.uint32) << 16).view(np.float32)
    keep = ~near_any
    err = rel_max_err(gpu_end[keep], ref_end[keep])
    moe_err = float(np.max(np.abs(gpu_end[keep] - ref_end[keep])))
    print(f"end of stack: {keep.sum()} of {len(tok)} tokens without a near tie on the way; "
          f"max|x30 gpu - x30 oracle| = {moe_err:.3e} ({err:.3e} of max|x30|)")
    # Reported, not held to the layer's tolerance: where the two MoE outputs differ (within it), the bf16
    # rounding of the residual can land one ulp apart, and such steps accumulate over 30 layers (an ulp is
    # 2^-8 relative). A broken layer would put the trajectories O(1) apart.
    assert np.all(np.isfinite(gpu_end))
    assert err <= 0.1


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
