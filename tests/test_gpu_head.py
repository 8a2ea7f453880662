"""GPU parity of the canvas output stage (tied LM head + softmax entropy) against the CPU oracle,
through the C ABI (MI355X only).

Tolerances, derived from the arithmetic:
- logits: each product of two bf16 values is exact in fp32, so the only error is the fp32 summation
  of D terms, bounded for any order by D 2^-24 sum_d |h_d e_d| (the standard recursive-summation
  bound); the test checks every logit against that bound computed from the same inputs;
- entropy: H = ln s - u / s from fp32 partial sums of e^(x - m) and e^(x - m)(x - m) merged in
  trees, plus the logit error above (at most ~1e-3 in x for these inputs) propagated through
  dH/dx_v = -p_v (ln p_v + H): 2e-3 nats absolute;
- argmax: the oracle's id wherever its top-1 / top-2 gap exceeds twice the logit bound; elsewhere
  any id whose oracle logit is within that bound of the maximum;
- the mean: the GPU's own entropies averaged (1e-6 relative), and the oracle's mean within the
  entropy tolerance.
Every case prints what it runs before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

from expert_ffn_canvas_amd import synth
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    from expert_ffn_canvas_amd import dgmoe
    import oracle

H_TOL = 2e-3


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _bits(t):
    return synth.to_numpy_bits(t.cpu() if t.is_cuda else t)


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_head(h, emb, beta, tokens=None, want_logits=True):
    """Run the stage on the GPU and compare positions `tokens` (all if None) with the oracle."""
    T = h.shape[0]
    head = dgmoe.CanvasHead(emb, max_tokens=T)
    r = head.forward(h, beta=beta, want_logits=want_logits)
    torch.cuda.synchronize()
    hb, eb = _bits(h), _bits(emb)
    ref = oracle.canvas_head(hb, eb, beta=beta, tokens=tokens, want_logits=True)
    idx = np.arange(T) if tokens is None else np.asarray(tokens)
    D = h.shape[1]
    # the summation bound per logit, from |h| |e|^T (fp32 products of fp32 magnitudes, 1% margin for
    # their own rounding)
    habs = np.abs(_f64(hb[idx])).astype(np.float32)
    eabs = np.abs((eb.astype(np.uint32) << 16).view(np.float32))
    bound = 1.01 * D * 2.0 ** -24 * (habs @ eabs.T).astype(np.float64) + 1e-30
    del eabs
    ent = r["entropy"].cpu().numpy().astype(np.float64)
    am = r["argmax"].cpu().numpy()
    if want_logits:
        lg = r["logits"].cpu().numpy().astype(np.float64)[idx]
        err = np.abs(lg - ref["logits"])
        assert np.all(err <= bound), f"logit error {err.max():.3e} above its bound at {np.unravel_index((err - bound).argmax(), err.shape)}"
    dH = np.abs(ent[idx] - ref["entropy"])
    assert dH.max() <= H_TOL, f"entropy error {dH.max():.3e}"
    bmax = bound.max(axis=1)
    clear = ref["gap"] > 2 * bmax
    assert np.array_equal(am[idx][clear], ref["argmax"][clear])
    for j in np.nonzero(~clear)[0]:  # near ties: any id within the bound of the maximum
        lg_row = ref["logits"][j]
        assert lg_row[am[idx[j]]] >= lg_row.max() - 2 * bmax[j]
    mean = r["mean_entropy"].cpu().item()
    assert abs(mean - ent.mean()) <= 1e-6 * max(1.0, abs(ent.mean()))
    assert np.all(ent >= -H_TOL) and np.all(ent <= math.log(emb.shape[0]) + H_TOL)
    head.close()
    return r, ref, dH.max()


@pytest.mark.parametrize("T,V,D,beta", [
    (37, 1000, 128, 1.0),     # three full vocabulary tiles and a ragged one
    (300, 2048, 256, 1.0),    # two position blocks, the second ragged
    (1, 257, 64, 2.5),        # one position, a lone vocabulary row in the last tile
    (256, 4096, 2816, 1.25),  # the model's d_model: 44 stages per tile
    (64, 512, 2816, 1.0),
    (5, 300, 64, 1.0),        # one stage per tile
    (3, 700, 128, 1.0),       # two stages per tile: the pipeline's prologue and tail only
    (16, 70000, 64, 1.0),     # 274 tiles: some workgroups run two tiles back to back
    (16, 700, 16384, 1.0),    # the largest d_model: 256 stages per tile
])
def test_head_small(T, V, D, beta):
    _say(f"head small T={T} V={V} D={D} beta={beta}")
    hw = synth.HeadWorkload("t", T, V, D, seed=T + V)
    inp = synth.make_head_inputs(hw, device="cuda")
    _, _, e = check_head(inp["h"], inp["emb"], beta)
    print(f"max entropy error {e:.3e}")


def test_head_without_logits_matches_with_logits():
    _say("head T=96 V=3000 D=320: logits NULL against written, and bit-reproducible")
    hw = synth.HeadWorkload("t", 96, 3000, 320, seed=5)
    inp = synth.make_head_inputs(hw, device="cuda")
    head = dgmoe.CanvasHead(inp["emb"], max_tokens=128)
    a = head.forward(inp["h"], want_logits=True)
    b = head.forward(inp["h"], want_logits=False)
    c = head.forward(inp["h"], want_logits=True)
    torch.cuda.synchronize()
    for k in ("entropy", "argmax", "mean_entropy"):
        assert torch.equal(a[k], b[k]) and torch.equal(a[k], c[k]), k
    assert torch.equal(a["logits"], c["logits"])
    head.close()


def test_head_zero_tokens_and_bad_arguments():
    _say("head T=0 and argument errors")
    emb = torch.zeros((512, 64), dtype=torch.bfloat16, device="cuda")
    head = dgmoe.CanvasHead(emb, max_tokens=8)
    h = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    ent = torch.empty(8, device="cuda")
    am = torch.empty(8, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert dgmoe.dg_head_forward(head.handle, h.data_ptr(), 0, 1.0, None, ent.data_ptr(), am.data_ptr(), None,
                                 s) == dgmoe.DG_OK
    assert dgmoe.dg_head_forward(head.handle, h.data_ptr(), 9, 1.0, None, ent.data_ptr(), am.data_ptr(), None,
                                 s) == dgmoe.DG_ERR_SHAPE
    assert dgmoe.dg_head_forward(head.handle, h.data_ptr(), 8, 0.0, None, ent.data_ptr(), am.data_ptr(), None,
                                 s) == dgmoe.DG_ERR_INVALID_ARG
    assert dgmoe.dg_head_forward(head.handle, h.data_ptr(), 8, 1.0, None, ent.data_ptr(), ent.data_ptr(), None,
                                 s) == dgmoe.DG_ERR_INVALID_ARG  # entropy and argmax overlap
    assert dgmoe.dg_head_forward(head.handle, h.data_ptr() + 8, 8, 1.0, None, ent.data_ptr(), am.data_ptr(), None,
                                 s) == dgmoe.DG_ERR_ALIGN
    # all-zero inputs: every logit 0, the entropy ln V, the argmax id 0
    r = head.forward(h)
    torch.cuda.synchronize()
    assert torch.all(r["logits"] == 0) and torch.all(r["argmax"] == 0)
    assert torch.allclose(r["entropy"], torch.full((8,), math.log(512), device="cuda"), atol=1e-5, rtol=0)
    head.close()


def test_head256_full_size_sampled():
    hw = synth.HEAD_WORKLOADS["head256"]
    _say(f"{hw.name} T={hw.T} V={hw.V} D={hw.D}: sampled positions against the oracle")
    inp = synth.make_head_inputs(hw, device="cuda")
    rng = np.random.default_rng(8)
    tok = np.unique(np.concatenate([[0, hw.T - 1], rng.choice(hw.T, 6, replace=False)]))
    r, ref, e = check_head(inp["h"], inp["emb"], 1.0, tokens=tok)
    print(f"max entropy error {e:.3e} at positions {tok.tolist()}")
    # properties at every position: a target pushed 16 or more above the rest is the argmax
    margin, target = inp["margin"].cpu().numpy(), inp["target"].cpu().numpy()
    am = r["argmax"].cpu().numpy()
    big = margin > 16
    assert np.all(am[big] == target[big])
