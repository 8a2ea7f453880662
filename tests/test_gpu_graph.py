"""A forward captured in a HIP graph (through torch's graph capture) replays bit-identically to the eager call.

dg_moe_forward and dg_head_forward allocate nothing and clear their own counters with kernels, so they can
be captured. Each graph is replayed several times with eager work on the same handle and buffers in
between, and every replay is compared with the eager result (both paths are deterministic). MI355X only.
"""
import pytest
import torch

from expert_ffn_canvas_amd import synth
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    from expert_ffn_canvas_amd import dgmoe


def _say(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("pack", [True, False], ids=["pack", "borrow"])
def test_moe_forward_graph_replays(pack):
    _say(f"graph: MoE forward T=64 E=16 K=4 D=256 F=128 pack={pack}")
    wl = synth.small_workload(T=64, E=16, K=4, D=256, F=128, bias="zipf", seed=3)
    inp = synth.make_inputs(wl, device="cuda")
    layer = dgmoe.MoELayer(inp["layers"][0], max_tokens=wl.T, act_dtype=torch.bfloat16, top_k=wl.K, pack=pack)
    x = inp["x"]
    ref = layer.forward(x).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = dgmoe.dg_moe_forward(layer.handle, x.data_ptr(), out.data_ptr(), wl.T, None, 0,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == dgmoe.DG_OK, dgmoe.dg_moe_last_error()
    x2 = torch.randn_like(x, dtype=torch.float32).to(torch.bfloat16)
    for i in range(4):
        out.fill_(0.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i}"
        other = layer.forward(x2)  # eager work on the same handle between replays
        torch.cuda.synchronize()
        assert not torch.equal(other, ref)
    layer.close()


def test_head_forward_graph_replays():
    _say("graph: output stage T=48 V=3000 D=192")
    hw = synth.HeadWorkload("t", 48, 3000, 192, seed=9)
    inp = synth.make_head_inputs(hw, device="cuda")
    head = dgmoe.CanvasHead(inp["emb"], max_tokens=hw.T)
    ref = {k: (None if v is None else v.clone()) for k, v in head.forward(inp["h"]).items()}
    torch.cuda.synchronize()
    out = {k: torch.empty_like(v) for k, v in ref.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st = dgmoe.dg_head_forward(head.handle, inp["h"].data_ptr(), hw.T, 1.0, out["logits"].data_ptr(),
                                   out["entropy"].data_ptr(), out["argmax"].data_ptr(),
                                   out["mean_entropy"].data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == dgmoe.DG_OK, dgmoe.dg_moe_last_error()
    h2 = torch.randn_like(inp["h"], dtype=torch.float32).to(torch.bfloat16)
    for i in range(4):
        for v in out.values():
            v.zero_()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(out[k], ref[k]), f"replay {i}: {k}"
        head.forward(h2)  # eager work on the same handle between replays
        torch.cuda.synchronize()
    head.close()
