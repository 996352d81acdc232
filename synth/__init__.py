"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws inputs: weight matrices, per-block bitwidth maps,
activations and the salient-row lists of the output-feature mixed format.
It holds none of the quantization arithmetic (no scales, zeros, codes or
dequantization) -- those live separately in the oracle and in the library.

The sources describe Llama-3-8B / 70B layers and a single linear layer with
K = 4096 and N in {4096, 14336}; trained weights are not available, so every
tensor here is a random stand-in with those shapes and the value
distributions described below:

* "ScaleBITS: Scalable Bitwidth Search for Hardware-Aligned Mixed-Precision
  LLMs" (explainer page, sections 1.2.2 and 4.2): 64x128 blocks, bitwidths
  from {1,2,3,4,6,8}, mean budget around 2-3 bits.
* "MixLLM: LLM Quantization with Global Mixed-precision between
  Output-features ..." (section 3.1.1 and the experiment setup): 10 % of
  output rows at 8 bits, the rest at 4 bits; its salience search needs
  gradients, so the salient rows are stood in for by the rows with the
  largest L2 norm.

Every draw comes from ``numpy.random.default_rng(SeedSequence([0xB10C,
workload, projection, tensor]))`` so any tensor can be regenerated alone.
tensor ids: 0 = W, 1 = W outlier positions, 2 = bitmap shuffle, 3 = x,
4 = x outlier channels, 5 = row scales.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

BLOCK_ROWS = 64      # output rows per block
BLOCK_COLS = 128     # input columns per block (= quantization group)

# workload ids (only used to seed the generators)
WL_LINEAR_4096 = 1
WL_LLAMA3_8B = 2
WL_LLAMA3_70B = 3
WL_PREFILL_70B_MLP = 4
WL_W44A8 = 5

TENSOR_W, TENSOR_W_OUTLIER, TENSOR_BITMAP, TENSOR_X, TENSOR_X_OUTLIER, TENSOR_ROWSCALE = range(6)


def rng(workload: int, proj: int, tensor: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0xB10C, workload, proj, tensor]))


# ----------------------------------------------------------------------------
# weights
# ----------------------------------------------------------------------------
def weight_gauss_outliers(N: int, K: int, workload: int, proj: int,
                          sigma: float = 0.02, outlier_frac: float = 0.005,
                          outlier_mul: float = 10.0) -> np.ndarray:
    """fp16 [N][K]: sigma*N(0,1) drawn in fp32, then floor(frac*N*K) entries
    picked uniformly without replacement are multiplied by ``outlier_mul``;
    rounded to fp16 (round-to-nearest-even) at the end."""
    g = rng(workload, proj, TENSOR_W)
    w = g.standard_normal(N * K, dtype=np.float32)
    w *= np.float32(sigma)
    n_out = int(outlier_frac * N * K)
    if n_out:
        idx = rng(workload, proj, TENSOR_W_OUTLIER).choice(N * K, size=n_out, replace=False)
        w[idx] *= np.float32(outlier_mul)
    return w.astype(np.float16).reshape(N, K)


def weight_heavy_rows(N: int, K: int, workload: int, proj: int,
                      sigma: float = 0.015) -> np.ndarray:
    """fp16 [N][K]: sigma * r_n * N(0,1) with lognormal row scales
    r_n = exp(0.5*xi_n - 0.25), xi_n ~ N(0,1) (so E[r^2] = 1)."""
    xi = rng(workload, proj, TENSOR_ROWSCALE).standard_normal(N)
    r = np.exp(0.5 * xi - 0.25).astype(np.float32)
    w = rng(workload, proj, TENSOR_W).standard_normal(N * K, dtype=np.float32).reshape(N, K)
    w *= (np.float32(sigma) * r)[:, None]
    return w.astype(np.float16)


# ----------------------------------------------------------------------------
# bitwidth maps (one bitwidth per 64x128 block; the allocation search itself
# needs gradients, so these maps are drawn from quotas)
# ----------------------------------------------------------------------------
def quota_counts(fracs: Sequence[Tuple[int, float]], nblk: int) -> List[Tuple[int, int]]:
    """Largest-remainder split of nblk blocks over (bits, fraction) classes.
    Ties in the remainder go to the class listed first."""
    raw = [(b, f * nblk) for b, f in fracs]
    counts = [[b, int(np.floor(v))] for b, v in raw]
    left = nblk - sum(c for _, c in counts)
    order = sorted(range(len(raw)), key=lambda i: (-(raw[i][1] - np.floor(raw[i][1])), i))
    for i in order[:left]:
        counts[i][1] += 1
    return [(b, c) for b, c in counts]


def bitmap_shuffled(nbr: int, nbc: int, fracs, workload: int, proj: int) -> np.ndarray:
    """uint8 [nbr][nbc]: the quota multiset in a seeded random order."""
    vals = np.concatenate([np.full(c, b, np.uint8) for b, c in quota_counts(fracs, nbr * nbc)])
    rng(workload, proj, TENSOR_BITMAP).shuffle(vals)
    return vals.reshape(nbr, nbc)


def block_scores(W: np.ndarray, kind: str, block_cols: int = BLOCK_COLS) -> np.ndarray:
    """fp64 [nbr][nbc] block score of 64 x block_cols blocks: 'maxabs'
    (largest |w|) or 'l1' (sum |w|)."""
    N, K = W.shape
    nbr, nbc = N // BLOCK_ROWS, K // block_cols
    out = np.empty((nbr, nbc), np.float64)
    for r0 in range(0, nbr, 16):               # chunked to bound memory
        blk = np.abs(W[r0 * 64:(r0 + 16) * 64].astype(np.float64)).reshape(-1, 64, nbc, block_cols)
        out[r0:r0 + blk.shape[0]] = blk.max(axis=(1, 3)) if kind == "maxabs" else blk.sum(axis=(1, 3))
    return out


def bitmap_by_score(W: np.ndarray, fracs, kind: str, block_cols: int = BLOCK_COLS) -> np.ndarray:
    """uint8 [nbr][nbc]: blocks ranked by descending score (ties to the lower
    block index) take the classes in the order listed (widest first)."""
    sc = block_scores(W, kind, block_cols)
    nbr, nbc = sc.shape
    order = np.lexsort((np.arange(nbr * nbc), -sc.reshape(-1)))
    vals = np.empty(nbr * nbc, np.uint8)
    pos = 0
    for b, c in quota_counts(fracs, nbr * nbc):
        vals[order[pos:pos + c]] = b
        pos += c
    return vals.reshape(nbr, nbc)


def uniform_bitmap(N: int, K: int, b: int) -> np.ndarray:
    return np.full((N // BLOCK_ROWS, K // BLOCK_COLS), b, np.uint8)


def random_bitmap(N: int, K: int, choices: Sequence[int], seed: int) -> np.ndarray:
    g = np.random.default_rng(np.random.SeedSequence([0xB10C, 99, seed, TENSOR_BITMAP]))
    return g.choice(np.asarray(choices, np.uint8), size=(N // BLOCK_ROWS, K // BLOCK_COLS))


def random_bitmap64(N: int, K: int, choices: Sequence[int], seed: int) -> np.ndarray:
    """uint8 [N/64][K/64]: a random bitwidth per 64x64 block."""
    g = np.random.default_rng(np.random.SeedSequence([0xB10C, 98, seed, TENSOR_BITMAP]))
    return g.choice(np.asarray(choices, np.uint8), size=(N // BLOCK_ROWS, K // 64))


# ----------------------------------------------------------------------------
# activations and salient rows
# ----------------------------------------------------------------------------
def activations(M: int, K: int, workload: int, proj: int,
                outlier_chan_frac: float = 0.0, outlier_mul: float = 1.0) -> np.ndarray:
    """fp16 [M][K] ~ N(0,1); optionally floor(frac*K) channels (columns)
    multiplied by ``outlier_mul``."""
    x = rng(workload, proj, TENSOR_X).standard_normal((M, K), dtype=np.float32)
    n_ch = int(outlier_chan_frac * K)
    if n_ch:
        ch = rng(workload, proj, TENSOR_X_OUTLIER).choice(K, size=n_ch, replace=False)
        x[:, ch] *= np.float32(outlier_mul)
    return x.astype(np.float16)


def salient_rows_by_l2(W: np.ndarray, frac: float = 0.10) -> np.ndarray:
    """int32 ascending indices of the floor(frac*N + 0.5) rows with the
    largest L2 norm (fp64), ties broken towards the lower row index."""
    N = W.shape[0]
    n8 = int(np.floor(frac * N + 0.5))
    nrm = np.empty(N, np.float64)
    for r0 in range(0, N, 1024):
        blk = W[r0:r0 + 1024].astype(np.float64)
        nrm[r0:r0 + blk.shape[0]] = np.sqrt((blk * blk).sum(axis=1))
    order = np.lexsort((np.arange(N), -nrm))
    return np.sort(order[:n8]).astype(np.int32)


# ----------------------------------------------------------------------------
# named workloads (shapes of the layers the sources measure)
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Proj:
    name: str
    N: int           # output features
    K: int           # input features


LLAMA3_8B_LAYER = (Proj("q", 4096, 4096), Proj("k", 1024, 4096), Proj("v", 1024, 4096),
                   Proj("o", 4096, 4096), Proj("gate", 14336, 4096), Proj("up", 14336, 4096),
                   Proj("down", 4096, 14336))
LLAMA3_70B_LAYER = (Proj("q", 8192, 8192), Proj("k", 1024, 8192), Proj("v", 1024, 8192),
                    Proj("o", 8192, 8192), Proj("gate", 28672, 8192), Proj("up", 28672, 8192),
                    Proj("down", 8192, 28672))
LLAMA3_70B_MLP = (Proj("gate", 28672, 8192), Proj("down", 8192, 28672))

BITS_LINEAR = ((2, 0.25), (3, 0.40), (4, 0.35))
BITS_8B = ((8, 0.05), (6, 0.05), (4, 0.15), (3, 0.35), (2, 0.35), (1, 0.05))
BITS_70B = ((8, 0.02), (6, 0.02), (4, 0.05), (3, 0.11), (2, 0.49), (1, 0.31))
BITS_PREFILL = ((8, 0.04), (4, 0.20), (3, 0.46), (2, 0.30))


def linear_4096() -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Single 4096x4096 layer: W 0.02*N(0,1) with 0.5 % entries x10, bits
    {2,3,4} at 25/40/35 % in seeded random order, x [1][4096] ~ N(0,1)."""
    W = weight_gauss_outliers(4096, 4096, WL_LINEAR_4096, 0)
    bits = bitmap_shuffled(64, 32, BITS_LINEAR, WL_LINEAR_4096, 0)
    x = activations(1, 4096, WL_LINEAR_4096, 0)
    return W, bits, x


def llama3_8b_proj(i: int) -> Tuple[Proj, np.ndarray, np.ndarray]:
    """Projection i of a Llama-3-8B-shaped layer: W as for the single layer,
    bits from {1,2,3,4,6,8} ranked by block max|w| (widest 5 % at 8 bits)."""
    p = LLAMA3_8B_LAYER[i]
    W = weight_gauss_outliers(p.N, p.K, WL_LLAMA3_8B, i)
    return p, W, bitmap_by_score(W, BITS_8B, "maxabs")


def llama3_8b_proj64(i: int) -> Tuple[Proj, np.ndarray, np.ndarray]:
    """The same projection with 64x64 blocks: the same W, bits over
    [N/64][K/64] blocks ranked by block max|w| with the same quotas (mean
    3.10)."""
    p = LLAMA3_8B_LAYER[i]
    W = weight_gauss_outliers(p.N, p.K, WL_LLAMA3_8B, i)
    return p, W, bitmap_by_score(W, BITS_8B, "maxabs", 64)


def llama3_70b_proj(i: int) -> Tuple[Proj, np.ndarray, np.ndarray]:
    """Projection i of a Llama-3-70B-shaped layer: heavy-tailed rows, bits
    ranked by block L1 norm at mean 2.1."""
    p = LLAMA3_70B_LAYER[i]
    W = weight_heavy_rows(p.N, p.K, WL_LLAMA3_70B, i)
    return p, W, bitmap_by_score(W, BITS_70B, "l1")


def prefill_70b_mlp(i: int) -> Tuple[Proj, np.ndarray, np.ndarray]:
    """70B MLP matrix i (0 = gate 28672x8192, 1 = down 8192x28672), bits
    {2,3,4,8} ranked by block L1 norm at mean 3.1."""
    p = LLAMA3_70B_MLP[i]
    W = weight_heavy_rows(p.N, p.K, WL_PREFILL_70B_MLP, i)
    return p, W, bitmap_by_score(W, BITS_PREFILL, "l1")


def prefill_x(M: int, K: int, proj: int) -> np.ndarray:
    """Prefill activations: N(0,1) with 1 % of the K channels x20."""
    return activations(M, K, WL_PREFILL_70B_MLP, proj, 0.01, 20.0)


def w44a8_28672x8192() -> Tuple[np.ndarray, np.ndarray]:
    """Output-feature mixed layer: W 28672x8192 heavy-tailed rows and the
    2867 rows with the largest L2 norm as the 8-bit set."""
    W = weight_heavy_rows(28672, 8192, WL_W44A8, 0)
    return W, salient_rows_by_l2(W, 0.10)


def w44a8_8192x28672() -> Tuple[np.ndarray, np.ndarray]:
    """The same recipe at the down projection's shape (8192x28672): the
    819 rows with the largest L2 norm are the 8-bit set."""
    W = weight_heavy_rows(8192, 28672, WL_W44A8, 1)
    return W, salient_rows_by_l2(W, 0.10)


# Launch groups of a decoder layer: projections that read the same input are
# stacked along the output rows into one matrix, as serving stacks do
# (q|k|v and gate|up), so a layer is four products.
LAYER_LAUNCH_GROUPS = (("qkv", (0, 1, 2)), ("o", (3,)), ("gate_up", (4, 5)), ("down", (6,)))


def stacked_group(gen, idx) -> Tuple[int, int, np.ndarray, np.ndarray]:
    """(N, K, W, bits) of the projections gen(i), i in idx, stacked along the
    output rows (same K); the bitmaps are stacked the same way."""
    parts = [gen(i) for i in idx]
    K = parts[0][0].K
    W = np.concatenate([w for (_, w, _) in parts]) if len(parts) > 1 else parts[0][1]
    bits = np.concatenate([b for (_, _, b) in parts]) if len(parts) > 1 else parts[0][2]
    return W.shape[0], K, W, bits


def mean_bits(bits: np.ndarray) -> float:
    return float(np.asarray(bits, np.float64).mean())
