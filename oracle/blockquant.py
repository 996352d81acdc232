"""Block-wise mixed-bit weight-only quantization and the reference GEMM.

Sources (cited by page title and section):

* MixLLM page, section 2.1 "quantization principle": the affine map
  X_q = clamp(round(X / s) + z, range) and its inverse X' = (X_q - z) * s; a
  bitwidth b gives 2^b levels; scales and zeros may be per group.
* ScaleBITS explainer page, section 1.2.2 (hardware-aligned block partition):
  64x128 blocks with one bitwidth per block; section 4.2 gives the bitwidth
  set {1,2,3,4,6,8} and 64x64 as the other GPU block size; section 3.2 the
  fused dequantize-multiply kernel.
* SBVR page, section 4.1: groups of 128 run along the GEMV inner dimension.

Readings where the pages are silent:
* a block is 64 output rows x 128 input columns, so each (row, 128-column
  group) lies in one block and has one bitwidth; with 64x64 blocks the group
  is 64 columns for the same reason (``block_cols=64`` below);
* s and z are chosen by min/max: s = (max - min) / (2^b - 1) rounded to fp16,
  z = clamp(rint(-min / s), 0, 2^b - 1); rint is round-half-to-even and the
  code is rint(v / s) + z, then clamped -- the order of the formula;
* codes are computed with the fp16-rounded scale (the one that is stored);
* a constant group c gets s = |c| (1 if c = 0); an fp16 scale that would
  round to 0 becomes 2^-24;
* the decisions are taken in fp64; dequantization (q - z) * s is exact in
  fp32 (at most 8 + 11 significant bits).
"""
from __future__ import annotations

import numpy as np

BLOCK_ROWS = 64
GROUP = 128
ALLOWED_BITS = (1, 2, 3, 4, 6, 8)
FP16_MIN_SUBNORMAL = 2.0 ** -24


def fp16_rne(a) -> np.ndarray:
    """Round fp64/fp32 values to the nearest fp16 (ties to even)."""
    return np.asarray(a).astype(np.float16)


def group_bits(bits: np.ndarray, N: int, K: int, block_cols: int = GROUP) -> np.ndarray:
    """int64 [N][K/block_cols]: the bitwidth of each (row, group) -- its
    block's.  The group is the block's width (128, or 64 for 64x64 blocks)."""
    bits = np.asarray(bits)
    if block_cols not in (64, 128):
        raise ValueError("blocks are 64x128 or 64x64")
    if bits.shape != (N // BLOCK_ROWS, K // block_cols):
        raise ValueError(f"bitmap shape {bits.shape} != {(N // BLOCK_ROWS, K // block_cols)}")
    if not np.isin(bits, ALLOWED_BITS).all():
        raise ValueError("bitwidth outside {1,2,3,4,6,8}")
    return np.repeat(bits.astype(np.int64), BLOCK_ROWS, axis=0)


def choose_scale_zero(lo: np.ndarray, hi: np.ndarray, levels: np.ndarray):
    """Min/max scale and zero point of each group (fp64 decisions).

    Returns (s16, z) with s16 float16 and z float64 holding integers."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    levels = np.asarray(levels, np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        s16 = fp16_rne((hi - lo) / levels)
    s16 = np.where((hi > lo) & (s16 == 0), np.float16(FP16_MIN_SUBNORMAL), s16)
    const = hi == lo
    s16 = np.where(const & (lo != 0), fp16_rne(np.abs(lo)), s16)
    s16 = np.where(const & (lo == 0), np.float16(1.0), s16).astype(np.float16)
    s = s16.astype(np.float64)
    z = np.clip(np.rint(-lo / s), 0, levels)
    return s16, z


def quantize_blocks(W16: np.ndarray, bits: np.ndarray, block_cols: int = GROUP):
    """Asymmetric group-wise RTN of an fp16 [N][K] matrix, each (row, group)
    at the bitwidth of its 64 x block_cols block (groups of block_cols
    columns).

    Returns q uint8 [N][K], s16 float16 [N][G], z16 float16 [N][G] with
    G = K / block_cols."""
    W16 = np.asarray(W16, np.float16)
    N, K = W16.shape
    bc = block_cols
    if N % BLOCK_ROWS or K % bc:
        raise ValueError(f"N must be a multiple of 64 and K of {bc}")
    G = K // bc
    gb = group_bits(bits, N, K, bc)
    q = np.empty((N, K), np.uint8)
    s16 = np.empty((N, G), np.float16)
    z16 = np.empty((N, G), np.float16)
    for r0 in range(0, N, 1024):                       # row chunks bound memory
        v = W16[r0:r0 + 1024].astype(np.float64).reshape(-1, G, bc)
        levels = (2.0 ** gb[r0:r0 + 1024] - 1.0)
        sc, z = choose_scale_zero(v.min(axis=2), v.max(axis=2), levels)
        q[r0:r0 + 1024] = _codes(v, sc, z, levels).reshape(-1, K)
        s16[r0:r0 + 1024] = sc
        z16[r0:r0 + 1024] = z.astype(np.float16)
    return q, s16, z16


def _codes(v, s16, z, levels):
    """q = clamp(rint(v / s) + z, 0, levels) per group (fp64)."""
    s = np.asarray(s16, np.float16).astype(np.float64)[:, :, None]
    code = np.clip(np.rint(v / s) + np.asarray(z, np.float64)[:, :, None], 0, levels[:, :, None])
    return code.astype(np.uint8)


def codes_with(W16: np.ndarray, bits: np.ndarray, s16: np.ndarray, z16: np.ndarray,
               block_cols: int = GROUP) -> np.ndarray:
    """Codes of W for given per-(row, group) scales and zeros (for example
    scales from a clipping search), with the same rounding as quantize_blocks."""
    W16 = np.asarray(W16, np.float16)
    N, K = W16.shape
    gb = group_bits(bits, N, K, block_cols)
    v = W16.astype(np.float64).reshape(N, K // block_cols, block_cols)
    return _codes(v, s16, np.asarray(z16, np.float64), 2.0 ** gb - 1.0).reshape(N, K)


def dequant_fp32(q: np.ndarray, s16: np.ndarray, z16: np.ndarray) -> np.ndarray:
    """w' = (q - z) * s in fp32 (exact: |q - z| < 2^8 and s has 11 bits).
    The group size is K / (number of scale columns)."""
    N, K = q.shape
    g = K // s16.shape[1]
    qz = q.astype(np.float32).reshape(N, -1, g) - z16.astype(np.float32)[:, :, None]
    return (qz * s16.astype(np.float32)[:, :, None]).reshape(N, K)


def dequant_fp16(q, s16, z16) -> np.ndarray:
    return fp16_rne(dequant_fp32(q, s16, z16))


def gemm_fp64(x16: np.ndarray, w32: np.ndarray) -> np.ndarray:
    """y = x . W'^T in fp64 (x [M][K], W' [N][K])."""
    return np.asarray(x16, np.float64) @ np.asarray(w32, np.float64).T


def reference_gemm(x16, W16, bits, block_cols: int = GROUP) -> np.ndarray:
    """End-to-end reference: quantize, dequantize exactly, fp64 product."""
    q, s16, z16 = quantize_blocks(W16, bits, block_cols)
    return gemm_fp64(x16, dequant_fp32(q, s16, z16))


def reference_rows(x16, W16, bits, rows, block_cols: int = GROUP) -> np.ndarray:
    """Reference outputs y[:, rows] for selected rows only, for sampled checks
    at full size.  Each (row, group) is quantized on its own, so only the
    selected rows are quantized, with their blocks' bitwidths -- the same
    steps as quantize_blocks, then the exact dequantization and an fp64
    product."""
    rows = np.asarray(rows, np.int64)
    W16 = np.asarray(W16, np.float16)
    N, K = W16.shape
    bc = block_cols
    G = K // bc
    gb = group_bits(bits, N, K, bc)[rows]                   # [n][G]
    v = W16[rows].astype(np.float64).reshape(rows.size, G, bc)
    levels = 2.0 ** gb - 1.0
    sc, z = choose_scale_zero(v.min(axis=2), v.max(axis=2), levels)
    q = _codes(v, sc, z, levels).reshape(rows.size, K)
    w = dequant_fp32(q, sc, z.astype(np.float16))
    return gemm_fp64(x16, w)


def rel_inf_err(y, y_ref) -> float:
    """||y - y_ref||_inf / ||y_ref||_inf."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.abs(y_ref).max()
    return float(np.abs(y - y_ref).max() / (den if den > 0 else 1.0))
