"""The allocation-free entry point of the canvas output stage (dg_head_forward_noalloc), through the C ABI,
against the handle-based dg_head_forward on the same inputs, on two calls in a row, the second with fewer
positions and a smaller vocabulary: every output bit-identical, and the entropies and argmax within the
oracle's bounds. Runs alone in a fresh process or after the other tests."""
import numpy as np
import pytest
import torch

from expert_ffn_canvas_amd import synth
from tests.conftest import gpu_available

pytestmark = pytest.mark.gpu

if gpu_available():
    from expert_ffn_canvas_amd import dgmoe
    import oracle


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _outputs(T, V, dev="cuda"):
    return {"logits": torch.full((T, V), float("nan"), dtype=torch.float32, device=dev),
            "entropy": torch.full((T,), float("nan"), dtype=torch.float32, device=dev),
            "argmax": torch.full((T,), -1, dtype=torch.int32, device=dev),
            "mean_entropy": torch.full((1,), float("nan"), dtype=torch.float32, device=dev)}


def _ptrs(o):
    return o["logits"].data_ptr(), o["entropy"].data_ptr(), o["argmax"].data_ptr(), o["mean_entropy"].data_ptr()


@pytest.mark.parametrize("first,second", [
    ((300, 4096, 256), (37, 1000, 256)),        # ragged vocabulary and position blocks, then fewer of both
    ((256, 262144, 2816), (200, 262144, 2816)),  # the canvas at the model's vocabulary, then a shorter one
])
def test_noalloc_matches_handle(first, second):
    sp = torch.cuda.current_stream().cuda_stream
    for i, (T, V, D) in enumerate((first, second)):
        _say(f"no-alloc output stage call {i}: T={T} V={V} D={D}")
        hw = synth.HeadWorkload(f"noalloc{i}", T, V, D, seed=40 + i)
        inp = synth.make_head_inputs(hw, device="cuda")
        h, emb = inp["h"], inp["emb"]
        cfg = dgmoe.make_head_config(V, D, max_tokens=T)
        a, b = _outputs(T, V), _outputs(T, V)
        st = dgmoe.dg_head_forward_noalloc(cfg, emb.data_ptr(), h.data_ptr(), T, 1.25, *_ptrs(a), sp)
        assert st == dgmoe.DG_OK, dgmoe.dg_moe_last_error()
        head = dgmoe.CanvasHead(emb, max_tokens=T)
        st = dgmoe.dg_head_forward(head.handle, h.data_ptr(), T, 1.25, *_ptrs(b), sp)
        assert st == dgmoe.DG_OK, dgmoe.dg_moe_last_error()
        torch.cuda.synchronize()
        head.close()
        for k in a:
            assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k
        # and against the oracle on a few positions
        tok = np.unique(np.array([0, T // 2, T - 1]))
        ref = oracle.canvas_head(synth.to_numpy_bits(h), synth.to_numpy_bits(emb), beta=1.25, tokens=tok)
        ent = a["entropy"].cpu().numpy()[tok]
        assert np.max(np.abs(ent - ref["entropy"])) <= 2e-3
        am = a["argmax"].cpu().numpy()[tok]
        clear = ref["gap"] > 1e-3
        assert np.array_equal(am[clear], ref["argmax"][clear])


def test_noalloc_rejects_beyond_scratch():
    _say("no-alloc output stage: sizes beyond the static scratch, bad arguments")
    sp = torch.cuda.current_stream().cuda_stream
    V, D, T = 262144, 256, 410  # 5 * 410 * 1024 * 4 bytes > 8 MiB
    cfg = dgmoe.make_head_config(V, D, max_tokens=T)
    emb = torch.zeros((16, D), dtype=torch.bfloat16, device="cuda")  # never read: rejected first
    h = torch.zeros((T, D), dtype=torch.bfloat16, device="cuda")
    ent = torch.empty((T,), dtype=torch.float32, device="cuda")
    am = torch.empty((T,), dtype=torch.int32, device="cuda")
    st = dgmoe.dg_head_forward_noalloc(cfg, emb.data_ptr(), h.data_ptr(), T, 1.0, None, ent.data_ptr(),
                                       am.data_ptr(), None, sp)
    assert st == dgmoe.DG_ERR_SHAPE and "scratch" in dgmoe.dg_moe_last_error()
    st = dgmoe.dg_head_forward_noalloc(cfg, emb.data_ptr(), h.data_ptr(), T + 1, 1.0, None, ent.data_ptr(),
                                       am.data_ptr(), None, sp)
    assert st == dgmoe.DG_ERR_SHAPE
    st = dgmoe.dg_head_forward_noalloc(cfg, 0, h.data_ptr(), 8, 1.0, None, ent.data_ptr(), am.data_ptr(), None, sp)
    assert st == dgmoe.DG_ERR_INVALID_ARG
    st = dgmoe.dg_head_forward_noalloc(cfg, emb.data_ptr(), h.data_ptr(), 0, 1.0, None, ent.data_ptr(),
                                       am.data_ptr(), None, sp)
    assert st == dgmoe.DG_OK
