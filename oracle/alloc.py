"""Offline bitwidth allocation and bidirectional channel reordering, with a
weight-magnitude proxy for the sensitivity.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (cited by page title and section):

* ScaleBITS explainer page, section 1.2.1 (bidirectional channel
  reordering): output channels (rows) and input channels (columns) are
  ordered by descending L1 sensitivity, gathering the sensitive weights in
  one corner before the block partition; done once, before quantization.
* Same page, section 2.2 (scalable greedy algorithm): minimise the loss
  subject to a mean-bitwidth budget, adjusting gamma * N blocks per round
  (gamma = 5 %) with first-order marginal gains; raise the most sensitive
  blocks while under the budget, otherwise trade raises of sensitive blocks
  for lowerings of insensitive ones.
* Same page, section 4.2: bitwidths {1,2,3,4,6,8}; start from 3 bits and
  lower the budget from there.

Readings where the pages are silent or garbled:

* The pages' sensitivity |grad L(w_Q) . dw_i| needs a model and calibration
  data.  The proxy objective of block i at bitwidth b is S_i * e_i(b): S_i
  is the block's L1 norm sum |w| and e_i(b) its RTN squared error
  sum (w - w'_b)^2 under the block quantizer of ``blockquant``.  S_i is exact
  in fp64 (fp16 values are multiples of 2^-24 and a block sums to less than
  2^29); e_i(b) is summed in fp64 in row-major order within the block.
* A step moves a block to the next bitwidth of the set.  Gains and costs
  are per bit: up_i = S_i (e_i(b) - e_i(b+)) / (b+ - b) and
  down_i = S_i (e_i(b-) - e_i(b)) / (b - b-), evaluated in that order.
* Every block starts at 3 bits; k = max(1, floor(gamma * nblk + 1/2)).
  A round: over the budget (sum of bits > target * nblk), lower the k
  blocks of least down (b > 1).  Within it, raise -- in order of largest
  up (b < 8) -- each of the first blocks whose step still fits the slack,
  at most k.  When none fits, take the h = max(1, k // 2) largest-up raises
  and pay for them with least-down lowerings of other blocks, in that
  order, until the bits freed cover the overshoot; trade if that lowers
  the objective (summed gains above summed costs, per step), otherwise
  stop.  At most 64 + floor(4 / gamma) rounds.
* Ties go to the lower block index (row-major over block rows, then block
  columns).  The channel orders use exact integer L1 norms (|w| * 2^24 in
  int64), ties to the lower index.
"""
from __future__ import annotations

import numpy as np

from . import blockquant as bq

ALLOWED = (1, 2, 3, 4, 6, 8)
STEP_UP = {1: 2, 2: 3, 3: 4, 4: 6, 6: 8}
STEP_DOWN = {2: 1, 3: 2, 4: 3, 6: 4, 8: 6}


def block_stats(W16: np.ndarray):
    """S [nbr][nbc]: block L1 norms; E [6][nbr][nbc]: RTN squared error of
    each block at each bitwidth of ALLOWED (ScaleBITS explainer, section
    2.2, with the proxy above)."""
    W16 = np.asarray(W16, np.float16)
    N, K = W16.shape
    if N % bq.BLOCK_ROWS or K % bq.GROUP:
        raise ValueError("N must be a multiple of 64 and K of 128")
    nbr, nbc = N // bq.BLOCK_ROWS, K // bq.GROUP
    w = W16.astype(np.float64)
    S = np.abs(w).reshape(nbr, 64, nbc, 128).sum(axis=(1, 3))   # exact in any order
    E = np.empty((len(ALLOWED), nbr, nbc))
    for t, b in enumerate(ALLOWED):
        q, s16, z16 = bq.quantize_blocks(W16, np.full((nbr, nbc), b, np.uint8))
        d2 = (w - bq.dequant_fp32(q, s16, z16).astype(np.float64)) ** 2
        blk = d2.reshape(nbr, 64, nbc, 128).transpose(0, 2, 1, 3).reshape(nbr, nbc, 64 * 128)
        E[t] = np.cumsum(blk, axis=2)[:, :, -1]                  # row-major, one by one
    return S, E


def allocate(W16: np.ndarray, target_bits: float, gamma: float = 0.05) -> np.ndarray:
    """Per-block bitwidths [N/64][K/128] with mean <= target_bits, by the
    batched greedy of the ScaleBITS explainer, section 2.2 (reading above)."""
    if not (1.0 <= target_bits <= 8.0) or not (0.0 < gamma <= 1.0):
        raise ValueError("target_bits in [1, 8] and gamma in (0, 1]")
    S, E = block_stats(W16)
    nbr, nbc = S.shape
    n = nbr * nbc
    Sf = S.reshape(-1)
    Ef = E.reshape(len(ALLOWED), -1)
    col = {b: t for t, b in enumerate(ALLOWED)}
    bits = [3] * n
    k = max(1, int(np.floor(gamma * n + 0.5)))
    budget = float(target_bits) * n

    def err(i, b):
        return float(Ef[col[b], i])

    def up(i):
        b = bits[i]
        b2 = STEP_UP[b]
        return float(Sf[i]) * (err(i, b) - err(i, b2)) / (b2 - b)

    def down(i):
        b = bits[i]
        b2 = STEP_DOWN[b]
        return float(Sf[i]) * (err(i, b2) - err(i, b)) / (b - b2)

    for _ in range(64 + int(np.floor(4.0 / gamma))):
        total = sum(bits)
        if total > budget:
            order = sorted((i for i in range(n) if bits[i] > 1), key=lambda i: (down(i), i))
            for i in order[:k]:
                bits[i] = STEP_DOWN[bits[i]]
            continue
        slack = budget - total
        ups = sorted((i for i in range(n) if bits[i] < 8), key=lambda i: (-up(i), i))
        raised = 0
        for i in ups:
            if raised == k:
                break
            step = STEP_UP[bits[i]] - bits[i]
            if step <= slack:
                bits[i] = STEP_UP[bits[i]]
                slack -= step
                raised += 1
        if raised:
            continue
        h = max(1, k // 2)
        chosen = ups[:h]
        taken = set(chosen)
        need = total + sum(STEP_UP[bits[i]] - bits[i] for i in chosen) - budget
        downs = []
        freed = 0
        for i in sorted((i for i in range(n) if bits[i] > 1), key=lambda i: (down(i), i)):
            if freed >= need:
                break
            if i not in taken:
                downs.append(i)
                freed += bits[i] - STEP_DOWN[bits[i]]
        gain = 0.0
        for i in chosen:
            gain += float(Sf[i]) * (err(i, bits[i]) - err(i, STEP_UP[bits[i]]))
        cost = 0.0
        for i in downs:
            cost += float(Sf[i]) * (err(i, STEP_DOWN[bits[i]]) - err(i, bits[i]))
        if not chosen or freed < need or not gain > cost:
            break
        for i in chosen:
            bits[i] = STEP_UP[bits[i]]
        for i in downs:
            bits[i] = STEP_DOWN[bits[i]]
    return np.array(bits, np.uint8).reshape(nbr, nbc)


def objective(W16: np.ndarray, bits: np.ndarray) -> float:
    """sum_i S_i e_i(b_i) of a bitmap (the proxy the allocation lowers)."""
    S, E = block_stats(W16)
    col = {b: t for t, b in enumerate(ALLOWED)}
    tot = 0.0
    for (r, c), b in np.ndenumerate(np.asarray(bits)):
        tot += float(S[r, c]) * float(E[col[int(b)], r, c])
    return tot


def channel_order(W16: np.ndarray):
    """(row_order, col_order): rows and columns by descending L1 norm, ties to
    the lower index (ScaleBITS explainer, section 1.2.1, with |W| as the
    sensitivity)."""
    a = (np.abs(np.asarray(W16, np.float16).astype(np.float64)) * 2.0 ** 24).astype(np.int64)
    rl1, cl1 = a.sum(axis=1), a.sum(axis=0)
    rows = np.lexsort((np.arange(rl1.size), -rl1)).astype(np.int32)
    cols = np.lexsort((np.arange(cl1.size), -cl1)).astype(np.int32)
    return rows, cols
