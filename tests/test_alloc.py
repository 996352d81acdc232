"""Offline bitwidth allocation and channel reordering (host, no GPU).

The oracle (oracle.alloc) is pinned to what the ScaleBITS explainer page and
the arithmetic fix: closed forms at the ends of the budget range, the order
of blocks that are scaled copies of one another, exact block statistics, and
a lower objective than the uniform 3-bit start.  The library's C++ version
(gbb_allocate_bits, gbb_channel_order) must then reproduce the oracle's
decisions bit for bit.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import gemm_block_bit_amd as gbb
from oracle import alloc
from oracle import blockquant as bq

ALLOWED = (1, 2, 3, 4, 6, 8)


def rand_w(N, K, seed, scale=0.02):
    g = np.random.default_rng(seed)
    W = scale * g.standard_normal((N, K))
    W[g.random((N, K)) < 0.01] *= 8
    return W.astype(np.float16)


def outlier_mix(n, seed):
    """One block row of n blocks: dense Gaussian blocks of random scale and
    sparse blocks (0.2 % outliers on a small background), whose L1 norm and
    quantization error rank the blocks differently."""
    g = np.random.default_rng(seed)
    blocks = []
    for _ in range(n):
        if g.random() < 0.5:
            B = 0.01 * g.standard_normal((64, 128)) * np.exp(g.normal(0, 0.7))
        else:
            B = 0.001 * g.standard_normal((64, 128))
            m = g.random((64, 128)) < 0.002
            B[m] = g.normal(0, 0.3, m.sum())
        blocks.append(B)
    return np.hstack(blocks).astype(np.float16)


def brute_force_optimum(W, target):
    """min over every bitmap with sum(b) <= target * nblk of sum S_i e_i(b_i)."""
    S, E = alloc.block_stats(W)
    n = S.size
    combos = np.array(list(itertools.product(range(len(ALLOWED)), repeat=n)))
    total = np.array(ALLOWED)[combos].sum(axis=1)
    cost = (S.reshape(1, -1) * E.reshape(len(ALLOWED), -1)[combos, np.arange(n)]).sum(axis=1)
    return cost[total <= target * n].min()


def heterogeneous(nbr, nbc, seed):
    """Blocks of widely different magnitude and spread."""
    g = np.random.default_rng(seed)
    W = g.standard_normal((64 * nbr, 128 * nbc))
    amp = np.exp(g.normal(0.0, 1.0, (nbr, nbc)))
    W *= np.kron(amp, np.ones((64, 128))) * 0.01
    return W.astype(np.float16)


# ----------------------------------------------------------------------------
# pins of the oracle
# ----------------------------------------------------------------------------
def test_block_stats_exact():
    """S is the exact block L1 norm; e_b is the exact sum of squared RTN errors
    (rational arithmetic over the quantizer's outputs)."""
    W = rand_w(128, 256, 1)
    S, E = alloc.block_stats(W)
    w = W.astype(np.float64)
    for (br, bc) in [(0, 0), (1, 1)]:
        blk = W[64 * br:64 * br + 64, 128 * bc:128 * bc + 128]
        assert S[br, bc] == float(sum(Fraction(float(v)) for v in np.abs(blk.astype(np.float64)).ravel()))
        for t, b in enumerate(ALLOWED):
            q, s16, z16 = bq.quantize_blocks(blk, np.full((1, 1), b, np.uint8))
            wq = bq.dequant_fp32(q, s16, z16).astype(np.float64)
            exact = sum(Fraction(float(a)) ** 2 for a in (w[64 * br:64 * br + 64, 128 * bc:128 * bc + 128] - wq).ravel())
            assert abs(E[t, br, bc] - float(exact)) <= 1e-12 * float(exact)
    # more bits, less error on random data
    assert np.all(np.diff(E, axis=0) < 0)


@pytest.mark.parametrize("target,value", [(8.0, 8), (1.0, 1)])
def test_budget_extremes_are_uniform(target, value):
    W = heterogeneous(3, 4, 2)
    bits = alloc.allocate(W, target)
    assert np.all(bits == value)


@pytest.mark.parametrize("target", [1.05, 1.2, 1.5, 2.1, 2.5, 3.0, 3.1, 3.5, 4.25, 6.0])
def test_budget_met_with_allowed_bitwidths(target):
    W = heterogeneous(4, 5, 3)
    bits = alloc.allocate(W, target)
    assert set(np.unique(bits)) <= set(ALLOWED)
    assert bits.astype(np.int64).sum() <= target * bits.size
    # within one largest step (2 bits) of the budget: the greedy spends it
    assert bits.astype(np.int64).sum() > target * bits.size - 2 - 1e-9


def test_scaled_copies_get_monotone_bitwidths():
    """Blocks that are one pattern times 2^t (exact in fp16) have objectives
    scaled by 8^t at every bitwidth: a larger copy never gets fewer bits."""
    g = np.random.default_rng(4)
    P = 0.05 * g.standard_normal((64, 128))
    nbr, nbc = 2, 6
    t = np.arange(nbr * nbc).reshape(nbr, nbc) - 6
    W = np.kron(2.0 ** t, np.ones((64, 128))) * np.tile(P, (nbr, nbc))
    W = W.astype(np.float16)
    for target in (2.0, 3.0, 4.0):
        bits = alloc.allocate(W, target, gamma=0.1).ravel()
        order = np.argsort(t.ravel())
        assert np.all(np.diff(bits[order].astype(int)) >= 0), (target, bits[order])
        assert bits.min() < bits.max()


def test_objective_not_worse_than_uniform_start():
    W = heterogeneous(4, 6, 5)
    three = np.full((4, 6), 3, np.uint8)
    bits = alloc.allocate(W, 3.0)
    assert alloc.objective(W, bits) < alloc.objective(W, three)
    assert bits.astype(np.int64).sum() <= 3 * bits.size


def test_greedy_reaches_brute_force_optimum():
    """On five-block problems the greedy's result is compared with the best
    of all 6^5 bitmaps within the budget.  A batched greedy is a heuristic,
    so it need not always be optimal; this one is within 30 % of the optimum
    everywhere on this grid and exactly optimal in 51 of its 56 cases
    (dropping S from the gains, ranking by gain per step instead of per bit,
    reversing the lowering order or trading without comparing gain and cost
    each fall to 47 or fewer, up to 12x the optimum)."""
    exact, worst = 0, 0.0
    for seed in range(8):
        W = outlier_mix(5, seed)
        for target in (2.0, 2.6, 3.0, 3.4, 4.0, 4.8, 5.6):
            opt = brute_force_optimum(W, target)
            bits = alloc.allocate(W, target, gamma=0.2)
            assert bits.astype(np.int64).sum() <= target * bits.size
            rel = alloc.objective(W, bits) / opt - 1
            assert rel >= -1e-12
            exact += rel <= 1e-9
            worst = max(worst, rel)
    assert worst < 0.3 and exact >= 50, (exact, worst)


@pytest.mark.parametrize("target", [1.0, 1.5, 2.0, 2.5])
def test_low_budget_pair(target):
    """Two blocks, the second the first times 16 (exact in fp16), so its cost
    is 16^3 times the first's at every bitwidth: every spare bit goes to it,
    and no trade may overdraw the budget when nothing is left to lower."""
    g = np.random.default_rng(14)
    P = 0.01 * g.standard_normal((64, 128))
    W = np.hstack([P, 16 * P]).astype(np.float16)
    bits = alloc.allocate(W, target).ravel()
    assert bits.sum() <= 2 * target
    assert alloc.objective(W, bits.reshape(1, 2)) == brute_force_optimum(W, target)
    assert bits[0] == 1


def test_channel_order_pins():
    W = rand_w(70, 90, 6)
    W[13] *= 50               # a planted heavy row
    W[:, 41] *= 50            # and column
    W[20] = W[21]             # a tie, broken by index
    rows, cols = alloc.channel_order(W)
    assert sorted(rows.tolist()) == list(range(70)) and sorted(cols.tolist()) == list(range(90))
    assert rows[0] == 13 and cols[0] == 41
    a = np.abs(W.astype(np.float64))
    assert np.all(np.diff(a.sum(axis=1)[rows]) <= 0) and np.all(np.diff(a.sum(axis=0)[cols]) <= 0)
    assert list(rows).index(20) < list(rows).index(21)


# ----------------------------------------------------------------------------
# the library against the oracle
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("nbr,nbc,seed,target,gamma", [
    (4, 5, 3, 2.1, 0.05), (4, 5, 3, 3.1, 0.05), (3, 8, 7, 2.5, 0.1), (6, 6, 8, 3.5, 0.05),
    (2, 3, 9, 1.0, 0.05), (2, 3, 9, 8.0, 0.2), (5, 4, 10, 4.0, 1.0)])
def test_library_allocation_matches_oracle(nbr, nbc, seed, target, gamma):
    W = heterogeneous(nbr, nbc, seed)
    assert np.array_equal(gbb.allocate_bits(W, target, gamma), alloc.allocate(W, target, gamma))


@pytest.mark.parametrize("seed", range(4))
def test_library_allocation_matches_oracle_outliers(seed):
    W = np.hstack([outlier_mix(8, seed), outlier_mix(8, seed + 100)])
    W = np.vstack([W, W[:, ::-1]])
    for target in (2.0, 2.6, 3.0, 4.4, 5.6):
        assert np.array_equal(gbb.allocate_bits(W, target, 0.1), alloc.allocate(W, target, 0.1))


def test_library_allocation_on_gaussian_weights():
    W = rand_w(256, 1024, 11)
    assert np.array_equal(gbb.allocate_bits(W, 2.6), alloc.allocate(W, 2.6))


def test_library_channel_order_matches_oracle():
    W = rand_w(192, 384, 12)
    W[100] *= 30
    W[:, 7] = W[:, 8]
    for a, b in zip(gbb.channel_order(W), alloc.channel_order(W)):
        assert np.array_equal(a, b)


def test_library_allocation_errors():
    W = rand_w(64, 128, 13)
    with pytest.raises(gbb.GbbError):
        gbb.allocate_bits(W, 0.5)
    with pytest.raises(gbb.GbbError):
        gbb.allocate_bits(W, 3.0, gamma=0.0)
    with pytest.raises(gbb.GbbError):
        gbb.allocate_bits(rand_w(64, 100, 13), 3.0)
    Wn = W.copy()
    Wn[0, 0] = np.inf
    with pytest.raises(gbb.GbbError):
        gbb.allocate_bits(Wn, 3.0)
    with pytest.raises(gbb.GbbError):
        gbb.channel_order(Wn)


def test_library_allocation_matches_oracle_heavy_rows():
    """A 1024 x 4096 weight with heavy-tailed rows (512 blocks), reordered
    by the channel order first, at two budgets."""
    import synth
    W = synth.weight_heavy_rows(1024, 4096, synth.WL_LLAMA3_8B, 2)
    r, c = gbb.channel_order(W)
    rr, cc = alloc.channel_order(W)
    assert np.array_equal(r, rr) and np.array_equal(c, cc)
    Wr = np.ascontiguousarray(W[r][:, c])
    for target in (2.5, 3.5):
        assert np.array_equal(gbb.allocate_bits(Wr, target), alloc.allocate(Wr, target))
