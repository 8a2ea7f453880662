"""The balanced deals of whole experts to the 8 per-XCD task queues, on the CPU: their balance guarantees, which
size the queues' capacity, over random, skewed and adversarial loads. By tiles: no queue more than twice the
largest expert's tile count above an even share of all tiles. By cost (wide tiles; TILE_COST per tile plus the
rows): no two queues more than the costliest expert apart, so no queue's tiles above the capacity's cost term.
The GPU tests check that the permutation kernel deals exactly as these models do (tests/parity_util.py,
check_device_state)."""
import numpy as np
import pytest

from parity_util import TILE_COST, balanced_deal, cost_snake_deal, snake


def queue_tiles(ntile, qof):
    q = np.zeros(8, dtype=np.int64)
    for e, x in enumerate(qof):
        if x is not None:
            q[x] += ntile[e]
    return q


def check_bound(counts, R):
    counts = np.asarray(counts, dtype=np.int64)
    ntile = (counts + R - 1) // R
    qof = balanced_deal(ntile, counts)
    assert all((x is None) == (t == 0) for x, t in zip(qof, ntile))
    q = queue_tiles(ntile, qof)
    assert q.sum() == ntile.sum()
    if ntile.sum():
        assert q.max() <= -(-int(ntile.sum()) // 8) + 2 * int(ntile.max()), (q, ntile.max())
    return q


def test_snake_order():
    assert [snake(h) for h in range(20)] == [0, 1, 2, 3, 4, 5, 6, 7, 7, 6, 5, 4, 3, 2, 1, 0, 0, 1, 2, 3]


def test_small_cases_by_hand():
    # four experts of one tile each: one per queue, in id order
    assert balanced_deal([1, 1, 1, 1], [5, 5, 5, 5]) == [0, 1, 2, 3]
    # one larger expert (3 tiles) on queue 0; the single-tile ones fill queues 1..7, then 1.. again at level 1
    # (queue 0 sits at level 3 and takes no more until level 3)
    q = balanced_deal([3] + [1] * 10, [300] + [10] * 10)
    assert q[0] == 0 and q[1:] == [1, 2, 3, 4, 5, 6, 7, 1, 2, 3]
    # no rows at all
    assert balanced_deal([0, 0], [0, 0]) == [None, None]


@pytest.mark.parametrize("seed", range(20))
def test_bound_random_zipf(seed):
    rng = np.random.default_rng(seed)
    E, K = 128, 8
    T = int(rng.choice([32, 256, 512, 2304, 4096, 8192]))
    p = 1.0 / np.arange(1, E + 1) ** rng.uniform(0.0, 1.5)
    p = p[rng.permutation(E)]
    p /= p.sum()
    counts = np.bincount(rng.choice(E, size=T * K, p=p), minlength=E)
    for R in (64, 128, 160):
        check_bound(counts, R)


@pytest.mark.parametrize("T", [4096, 8192, 65536])
def test_bound_adversarial(T):
    # a few experts take every token, at ids that dealt in id order stack on queue 0 (snake positions 0, 15,
    # 16, 31, 32, ...); the rest share the remaining slots evenly or not at all
    E, K = 128, 8
    for big in ([0, 15, 16, 31, 32], [0, 15, 16, 31, 32, 47, 48], [0, 1, 14, 15, 16, 17]):
        for rest_share in (0.0, 0.3, 1.0):
            counts = np.zeros(E, dtype=np.int64)
            counts[big] = T
            others = [e for e in range(E) if e not in big]
            n_rest = (K - len(big)) * T if len(big) < K else 0
            n_use = max(1, int(len(others) * rest_share))
            for i in range(n_rest):
                counts[others[i % n_use]] += 1
            for R in (64, 128, 160):
                check_bound(counts, R)


def capacity_tiles(T, K, E, R):
    """The library's queue capacity (launch.h max_queue_len) for one column block, in tiles."""
    max_tiles = -(-(K * T) // R) + E
    per_expert = -(-T // R)
    by_tiles = -(-max_tiles // 8) + 2 * per_expert
    by_cost = -(-max_tiles // 8) + per_expert + -(-(K * T + 8 * T) // (8 * TILE_COST)) + 1
    return max(by_tiles, by_cost)


def check_cost_bound(counts, T, K, R=160):
    counts = np.asarray(counts, dtype=np.int64)
    ntile = (counts + R - 1) // R
    qof = cost_snake_deal(ntile, counts)
    cost = np.where(ntile > 0, TILE_COST * ntile + counts, 0)
    load = np.zeros(8, dtype=np.int64)
    for e, x in enumerate(qof):
        if x is not None:
            load[x] += cost[e]
    assert load.sum() == cost.sum()
    assert load.max() - load.min() <= cost.max(), (load, cost.max())
    q = queue_tiles(ntile, qof)
    assert q.sum() == ntile.sum()
    assert q.max() <= capacity_tiles(T, K, len(counts), R), (q.max(), capacity_tiles(T, K, len(counts), R))
    return load


def test_cost_deal_by_hand():
    # costs 128 t + rows: 456, then 138 x 9; snake: ranks 0..7 to queues 0..7, ranks 8, 9 to queues 7, 6
    assert cost_snake_deal([2] + [1] * 9, [200] + [10] * 9) == [0, 1, 2, 3, 4, 5, 6, 7, 7, 6]


@pytest.mark.parametrize("seed", range(20))
def test_cost_bound_random(seed):
    rng = np.random.default_rng(100 + seed)
    E, K = 128, 8
    T = int(rng.choice([1536, 2304, 4096, 8192, 65536]))
    p = rng.dirichlet(np.ones(E) * rng.uniform(0.3, 30))
    counts = np.bincount(rng.choice(E, size=T * K, p=p), minlength=E)
    check_cost_bound(counts, T, K)


@pytest.mark.parametrize("T", [2304, 8192, 65536])
def test_cost_bound_adversarial(T):
    E, K = 128, 8
    for big in ([0, 15, 16, 31, 32], [0, 1, 2, 3, 4, 5, 6, 7]):
        counts = np.zeros(E, dtype=np.int64)
        counts[big] = T
        rest = [e for e in range(E) if e not in big]
        for i in range((K - len(big)) * T):
            counts[rest[i % len(rest)]] += 1
        check_cost_bound(counts, T, K)
    # one row each for all but one expert
    counts = np.ones(E, dtype=np.int64)
    counts[0] = K * T - (E - 1)
    counts[0] = min(counts[0], T)
    check_cost_bound(counts, T, K)
