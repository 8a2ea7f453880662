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


def check_routing_many(gpu_idx, gpu_w, orc, K, T):
    """check_routing's acceptance rules for many tokens: vectorised over the tokens without a near tie, the
    near-tie tokens one by one through check_routing. Returns the number of near-tie tokens."""
    gi = np.asarray(gpu_idx).astype(np.int64)
    gw = np.asarray(gpu_w, dtype=np.float64)
    assert gi.shape == (T, K) and gw.shape == (T, K)
    srt = np.sort(gi, axis=1)
    assert np.all(np.diff(srt, axis=1) != 0), "a token with duplicate experts"
    clear = orc["gap"] >= TIE
    differ = clear & np.any(srt != np.sort(orc["idx"].astype(np.int64), axis=1), axis=1)
    assert not differ.any(), f"tokens {np.nonzero(differ)[0][:8]}: expert sets differ from the oracle's"
    wo = np.zeros(orc["logits"].shape, dtype=np.float64)
    np.put_along_axis(wo, orc["idx"].astype(np.int64), orc["w"], axis=1)
    dw = np.abs(gw - np.take_along_axis(wo, gi, axis=1))[clear]
    assert dw.size == 0 or float(dw.max()) <= W_TOL, f"a routing weight off by {float(dw.max()):.3g}"
    assert np.all(np.abs(gw.sum(axis=1) - 1.0) <= SUM_TOL)
    assert np.all(np.diff(np.asarray(gpu_w), axis=1) <= 1e-7), "slots not ordered by weight"
    near = np.nonzero(~clear)[0]
    if len(near):
        sub = {k: orc[k][near] for k in ("idx", "w", "logits", "gap")}
        check_routing(np.asarray(gpu_idx)[near], np.asarray(gpu_w)[near], sub, K, len(near))
    print(f"routing: {T} tokens, near-tie tokens {len(near)}, max |w_gpu - w_oracle| "
          f"{float(dw.max()) if dw.size else 0.0:.3g}")
    return len(near)


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


def snake(h):
    """Queue of the h-th expert dealt in snake order over the 8 queues (0..7, then 7..0, ...)."""
    return 7 - h % 8 if (h // 8) % 2 else h % 8


TILE_COST = 128  # the cost of a tile, in rows, for the deal of wide tiles
WIDE_ROWS = 160   # the height of wide tiles


def cost_snake_deal(ntile, counts):
    """The balanced deal of wide tiles: each expert with rows costs TILE_COST per tile plus its rows; the experts
    in order of cost (descending, ties to the lower id) go to the queues in snake order (0..7, then 7..0, ...).
    Returns a list (None for experts without rows)."""
    E = len(ntile)
    cost = [TILE_COST * int(ntile[e]) + int(counts[e]) if ntile[e] > 0 else 0 for e in range(E)]
    order = sorted(range(E), key=lambda e: (-cost[e], e))
    qof = [None] * E
    for r, e in enumerate(order):
        if ntile[e] > 0:
            qof[e] = snake(r)
    return qof


def balanced_deal(ntile, counts):
    """The queue of every expert under the permutation's balanced deal of whole experts, from the tile counts
    (ntile) and token counts of the experts, written out step by step as the deal is specified: the experts
    with more than the smallest nonzero tile count v1 are dealt in snake order by id; if the most loaded queue
    then exceeds an even share of all tiles by more than the largest tile count, they are dealt again in snake
    order of their rank by token count (descending, ties to the lower id); the experts of v1 tiles then fill
    the queues level by level (queue q at level load_q // v1), the i-th of them (in id order) taking the i-th
    smallest (level, queue) pair at or above each queue's level. Returns a list (None for experts without
    rows)."""
    ntile = [int(v) for v in ntile]
    E = len(ntile)
    nz = [v for v in ntile if v > 0]
    qof = [None] * E
    if not nz:
        return qof
    v1, total, a_max = min(nz), sum(ntile), max(ntile)
    heavy = [e for e in range(E) if ntile[e] > v1]
    tail = [e for e in range(E) if ntile[e] == v1]
    pos = {e: i for i, e in enumerate(heavy)}
    load = [0] * 8
    for e in heavy:
        load[snake(pos[e])] += ntile[e]
    if max(load) > (total + 7) // 8 + a_max:
        order = sorted(range(E), key=lambda e: (-int(counts[e]), e))
        pos = {e: r for r, e in enumerate(order) if e in pos}
        load = [0] * 8
        for e in heavy:
            load[snake(pos[e])] += ntile[e]
    for e in heavy:
        qof[e] = snake(pos[e])
    lv = [l // v1 for l in load]
    for i, e in enumerate(tail):
        lam = min(lv)
        while sum(max(0, lam + 1 - l) for l in lv) <= i:
            lam += 1
        j = i - sum(max(0, lam - l) for l in lv)
        qof[e] = [q for q in range(8) if lv[q] <= lam][j]
    return qof


def check_device_state(dbg, K, E, T, D, F, balanced=None):
    """The handle's sticky device status word is clear, and the per-XCD task queues hold their tasks within the
    capacity and within the balance the deal guarantees: no queue more than 2 tiles of the largest expert above
    an even share of all tiles (per column block of each GEMM), or, for the deal of wide tiles by cost, exactly
    the model's queues. balanced: the fused launch's balanced deal (its queues are compared with the model)."""
    flags = int(dbg["dev_flags"].cpu().numpy()[0])
    assert flags == 0, f"device status word 0x{flags:x}"
    ql = dbg["queue_len"].cpu().numpy()
    counts = dbg["counts"].cpu().numpy()
    lens, caps = ql[:16].reshape(2, 8), ql[16:18]
    # the tile height and column blocks the launch used: 32-, 64- or 128-row tiles with blocks of 64 gate_up
    # features and 128 down outputs, or 160-row tiles with blocks of 128 and 256 (the last one partial)
    shapes = [(32, (F // 64, D // 128)), (64, (F // 64, D // 128)), (128, (F // 64, D // 128)),
              (160, (-(-F // 128), -(-D // 256)))]
    match = [(R, nbs) for R, nbs in shapes
             if all(lens[g].sum() == nbs[g] * int(np.sum((counts + R - 1) // R)) for g in range(2))]
    assert match, f"queue lengths {lens} match no tile height"
    R, nbs = match[0]
    tiles = int(np.sum((counts + R - 1) // R))
    a_max = int((counts.max() + R - 1) // R)
    for g, nb in enumerate(nbs):
        assert np.all(lens[g] <= caps[g]), f"GEMM {g}: queue lengths {lens[g]} over capacity {caps[g]}"
        if not (balanced and R == WIDE_ROWS):
            bound = nb * (-(-tiles // 8) + 2 * a_max)
            assert lens[g].max() <= bound, f"GEMM {g}: queue {lens[g].max()} > balance bound {bound} ({lens[g]})"
    if balanced:
        # every queue holds exactly the tiles the balanced deal gives it (by cost for wide tiles)
        ntile = (counts + R - 1) // R
        qof = cost_snake_deal(ntile, counts) if R == WIDE_ROWS else balanced_deal(ntile, counts)
        want = np.zeros(8, dtype=np.int64)
        for e in range(E):
            if qof[e] is not None:
                want[qof[e]] += ntile[e]
        for g, nb in enumerate(nbs):
            assert np.array_equal(lens[g], nb * want), f"GEMM {g}: queue lengths {lens[g]}, deal gives {nb * want}"


def rel_max_err(gpu, ref):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(gpu - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def to_f32(t):
    return t.detach().float().cpu().numpy()


def layer_parity(layer, x, wn, K, eps=synth.RMS_EPS, tokens=None, n_threads=0, check_state=True):
    """Run the GPU forward (debug) and compare routing, permutation and output with the oracle.

    tokens: indices of tokens whose outputs are compared (None = all). check_state: also require a clear device
    status word and the queues the deal gives. Returns a dict of measurements.
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
    if check_state:
        check_device_state(dbg, K, layer.E, T, layer.D, layer.F, balanced=layer.gemms_fused)
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    ref = oracle.moe_forward(wn, xn, K, eps, forced=gidx, tokens=tok, n_threads=n_threads)
    gout = to_f32(dbg["out"])[tok]
    err = rel_max_err(gout, ref["out"])
    assert np.all(np.isfinite(gout))
    assert err <= OUT_TOL, f"max|d|/max|ref| = {err:.3e} > {OUT_TOL}"
    return dict(err=err, near_ties=near, dbg=dbg, ref=ref, tokens=tok)
