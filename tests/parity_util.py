"""Helpers of the GPU parity tests: run the HIP layer, run the oracle on the same tensors, and apply the
acceptance rules.

Acceptance rules:
  * routing: wherever the gap between the 8th and 9th largest oracle (fp64) logit is >= 1e-4, the GPU's
    expert set equals the oracle's exactly. Below that, several sets are correct: with A = experts whose
    logit exceeds the 8th largest by >= 1e-4 and B = experts within 1e-4 of it, any set S' with
    A <= S' <= A u B and |S'| = k is accepted, and that token's output is compared with the oracle re-run
    on S'. The GPU weights sum to 1 within 1e-6 and match the oracle's within 1e-5: the GPU logits are
    fp32 dot products over d_model = 2816 terms (error a few 1e-6), and a logit error d moves a weight
    w by about w * d, so 1e-5 bounds it with margin while a wrong softmax (missing renormalisation, a
    dropped term) is off by far more.
  * output: max|gpu - oracle| <= 2e-2 * max|oracle| over the compared tokens.
"""
import numpy as np
import torch

import oracle
from expert_ffn_canvas_amd import synth

TIE = 1e-4
OUT_TOL = 2e-2
W_TOL = 1e-5
SUM_TOL = 1e-6


def host(t):
    return synth.to_numpy_bits(t)


def oracle_weights(w):
    return synth.weights_to_numpy(w)


def check_routing(gpu_idx, gpu_w, orc, K, T):
    """gpu_idx/gpu_w: numpy [T,K]; orc: oracle.route(...) result. Returns the number of near-tie tokens."""
    lg = orc["logits"]
    near = 0
    max_dw = 0.0
    for t in range(T):
        s_gpu = set(gpu_idx[t].tolist())
        assert len(s_gpu) == K, f"token {t}: duplicate experts {gpu_idx[t]}"
        if orc["gap"][t] >= TIE:
            assert s_gpu == set(orc["idx"][t].tolist()), f"token {t}: set {sorted(s_gpu)} != oracle " \
                f"{sorted(orc['idx'][t].tolist())} (gap {orc['gap'][t]:.3g})"
            ow = dict(zip(orc["idx"][t].tolist(), orc["w"][t].tolist()))
            for j in range(K):
                dw = abs(gpu_w[t, j] - ow[int(gpu_idx[t, j])])
                max_dw = max(max_dw, dw)
                assert dw <= W_TOL, f"token {t} slot {j} weight off by {dw:.3g}"
        else:
            near += 1
            l8 = np.sort(lg[t])[::-1][K - 1]
            A = set(np.nonzero(lg[t] >= l8 + TIE)[0].tolist())
            B = set(np.nonzero(np.abs(lg[t] - l8) < TIE)[0].tolist())
            assert A <= s_gpu <= (A | B), f"token {t}: near-tie set {sorted(s_gpu)} not within A={A} B={B}"
        assert abs(float(np.sum(gpu_w[t], dtype=np.float64)) - 1.0) <= SUM_TOL
        # slots ordered by weight (logit) descending
        assert np.all(np.diff(gpu_w[t]) <= 1e-7), f"token {t}: slots not ordered {gpu_w[t]}"
    print(f"routing: near-tie tokens {near}, max |w_gpu - w_oracle| {max_dw:.3g}")
    return near


def check_permutation(dbg, K, E, T):
    """The GPU permutation equals the oracle's permutation of the GPU routing, integer-exact."""
    idx = dbg["topk_idx"].cpu().numpy().astype(np.int32)
    pm = oracle.permute(idx, E)
    assert np.array_equal(dbg["counts"].cpu().numpy(), pm["counts"])
    assert np.array_equal(dbg["offsets"].cpu().numpy(), pm["offsets"])
    slot = dbg["sorted_slot"].cpu().numpy()
    assert np.array_equal(slot // K, pm["sorted_token"])
    row_of_slot = dbg["row_of_slot"].cpu().numpy()
    assert np.array_equal(row_of_slot, pm["row_of_slot"])
    # the slot of each row routes to that row's expert, and gather after scatter is the identity
    row_expert = np.repeat(np.arange(E), pm["counts"])
    assert np.array_equal(idx.ravel()[slot], row_expert)
    assert np.array_equal(row_of_slot[slot], np.arange(K * T))
    assert int(pm["counts"].sum()) == K * T


def rel_max_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(gpu - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def to_f32(t):
    return t.detach().float().cpu().numpy()


def layer_parity(layer, x, wn, K, eps=synth.RMS_EPS, tokens=None, n_threads=0):
    """Run the GPU forward (debug) and compare routing, permutation and output with the oracle.

    tokens: indices of tokens whose outputs are compared (None = all). Returns a dict of measurements.
    """
    T = x.shape[0]
    dbg = layer.forward_debug(x)
    torch.cuda.synchronize()
    xn = host(x)
    orc = oracle.route(xn, wn["router_w"], wn["router_gamma"], wn.get("router_bias"), K, eps, n_threads=n_threads)
    gidx = dbg["topk_idx"].cpu().numpy()
    gw = dbg["topk_w"].cpu().numpy()
    near = check_routing(gidx, gw, orc, K, T)
    check_permutation(dbg, K, layer.E, T)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    ref = oracle.moe_forward(wn, xn, K, eps, forced=gidx, tokens=tok, n_threads=n_threads)
    gout = to_f32(dbg["out"])[tok]
    err = rel_max_err(gout, ref["out"])
    assert np.all(np.isfinite(gout))
    assert err <= OUT_TOL, f"max|d|/max|ref| = {err:.3e} > {OUT_TOL}"
    return dict(err=err, near_ties=near, dbg=dbg, ref=ref, tokens=tok)
