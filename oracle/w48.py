"""Output-feature mixed precision W8(sym)/W4(asym) x A8(sym), group 128.

Sources (MixLLM page):
* section 3.1.1: salient output features get 8-bit weights, the others
  4-bit; each row set is an independent sub-problem and the outputs are
  gathered back to their original channels;
* section 3.1.2 and the experiment setup: 8-bit parts symmetric, 4-bit
  parts asymmetric, group size 128, activations 8-bit symmetric;
* section 2.1: symmetric quantization X_q = clamp(round(W / s), range),
  X' = X_q * s; asymmetric as in ``blockquant``;
* section 3.3: two-step dequantization -- per group, the integer product
  A_q (W_q - z) first, then the two scales s_a * s_w.

Readings where the pages are silent: the symmetric range is +-(2^(b-1) - 1), i.e.
+-127, with s = max|v| / 127 rounded to fp16 (1 if the group is all zero);
activations are quantized per token (the benchmark layer) or per 128-group
(the page's own choice); the activation decisions are taken in fp32, the
precision of the GPU kernel that makes them.
"""
from __future__ import annotations

import numpy as np

from .blockquant import FP16_MIN_SUBNORMAL, GROUP, choose_scale_zero, fp16_rne


def split_rows(N: int, rows8) -> tuple[np.ndarray, np.ndarray]:
    rows8 = np.asarray(rows8, np.int64)
    if rows8.size and (np.any(np.diff(rows8) <= 0) or rows8[0] < 0 or rows8[-1] >= N):
        raise ValueError("rows8 must be strictly ascending row indices")
    mask = np.ones(N, bool)
    mask[rows8] = False
    return rows8, np.nonzero(mask)[0]


def quant_sym8(W16: np.ndarray):
    """8-bit symmetric group-128 quantization of fp16 rows (fp64 decisions).
    Returns q int8 [n][K] in [-127, 127] and s16 float16 [n][K/128]."""
    n, K = W16.shape
    v = np.asarray(W16, np.float64).reshape(n, K // GROUP, GROUP)
    a = np.abs(v).max(axis=2)
    s16 = fp16_rne(a / 127.0)
    s16 = np.where((a > 0) & (s16 == 0), np.float16(FP16_MIN_SUBNORMAL), s16)
    s16 = np.where(a == 0, np.float16(1.0), s16).astype(np.float16)
    q = np.clip(np.rint(v / s16.astype(np.float64)[:, :, None]), -127, 127)
    return q.reshape(n, K).astype(np.int8), s16


def quant_asym4(W16: np.ndarray):
    """4-bit asymmetric group-128 quantization (min/max, as blockquant).
    Returns q uint8 [n][K] in [0, 15], s16 float16 [n][G], z uint8 [n][G]."""
    n, K = W16.shape
    v = np.asarray(W16, np.float64).reshape(n, K // GROUP, GROUP)
    levels = np.full(v.shape[:2], 15.0)
    s16, z = choose_scale_zero(v.min(axis=2), v.max(axis=2), levels)
    q = np.clip(np.rint(v / s16.astype(np.float64)[:, :, None]) + z[:, :, None], 0, 15)
    return q.reshape(n, K).astype(np.uint8), s16, z.astype(np.uint8)


def quant_act(x16: np.ndarray, group: int | None = None):
    """8-bit symmetric activations, per token (group=None) or per group of
    ``group`` columns.  fp32 decisions: s32 = max|x| / 127 (IEEE fp32 divide),
    s16 = fp16(s32) (1 if max|x| = 0, 2^-24 if it would round to 0),
    A_q = clamp(rint(x / s16), -127, 127) with an fp32 divide.
    Returns A_q int8 [M][K] and s16 float16 [M] or [M][K/group]."""
    x = np.asarray(x16, np.float16).astype(np.float32)
    M, K = x.shape
    g = K if group is None else group
    xv = x.reshape(M, K // g, g)
    a = np.abs(xv).max(axis=2)
    s16 = (a / np.float32(127.0)).astype(np.float32).astype(np.float16)
    s16 = np.where((a > 0) & (s16 == 0), np.float16(FP16_MIN_SUBNORMAL), s16)
    s16 = np.where(a == 0, np.float16(1.0), s16).astype(np.float16)
    qv = np.rint((xv / s16.astype(np.float32)[:, :, None]).astype(np.float32))
    A = np.clip(qv, -127, 127).reshape(M, K).astype(np.int8)
    return A, (s16[:, 0] if group is None else s16)


def group_acc(A_q: np.ndarray, Wz: np.ndarray) -> np.ndarray:
    """int64 [M][n][G]: acc[m, n, g] = sum_{k in g} A_q[m, k] * Wz[n, k]
    (Wz = W_q - z, integers).  One fp64 product per group; exact because
    every partial sum is an integer far below 2^53."""
    M, K = A_q.shape
    n = Wz.shape[0]
    G = K // GROUP
    out = np.empty((M, n, G), np.int64)
    A = A_q.astype(np.float64)
    W = Wz.astype(np.float64)
    for g in range(G):
        sl = slice(g * GROUP, (g + 1) * GROUP)
        out[:, :, g] = (A[:, sl] @ W[:, sl].T).astype(np.int64)
    return out


def two_step(A_q, s_a, Wz, s_w) -> np.ndarray:
    """y[m, n] = sum_g s_a[m(, g)] * s_w[n, g] * acc[m, n, g] in fp64."""
    acc = group_acc(A_q, Wz).astype(np.float64)
    sw = np.asarray(s_w, np.float64)[None, :, :]
    sa = np.asarray(s_a, np.float64)
    sa = sa[:, None, None] if sa.ndim == 1 else sa[:, None, :]
    return (acc * sa * sw).sum(axis=2)


def quantize_w48(W16: np.ndarray, rows8):
    """Both sub-problems of one layer: dict with rows8, rows4, q8, s8, q4,
    s4, z4 (quantized codes in ascending original-row order)."""
    N = W16.shape[0]
    r8, r4 = split_rows(N, rows8)
    q8, s8 = quant_sym8(W16[r8])
    q4, s4, z4 = quant_asym4(W16[r4])
    return dict(rows8=r8, rows4=r4, q8=q8, s8=s8, q4=q4, s4=s4, z4=z4)


def reference(x16, W16, rows8, act_group: int | None = None,
              quant: dict | None = None) -> np.ndarray:
    """fp64 y [M][N] of the W8/W4 x A8 layer, outputs scattered back to the
    original row order."""
    N, K = W16.shape
    qd = quant if quant is not None else quantize_w48(W16, rows8)
    A_q, s_a = quant_act(x16, act_group)
    y = np.zeros((A_q.shape[0], N), np.float64)
    if qd["rows8"].size:
        y[:, qd["rows8"]] = two_step(A_q, s_a, qd["q8"].astype(np.int64), qd["s8"])
    if qd["rows4"].size:
        Wz = qd["q4"].astype(np.int64) - np.repeat(qd["z4"].astype(np.int64), GROUP, axis=1)
        y[:, qd["rows4"]] = two_step(A_q, s_a, Wz, qd["s4"])
    return y


def dequant_rows(qd: dict, N: int, K: int) -> np.ndarray:
    """fp64 [N][K] dequantized weights in original row order (for identity
    checks: (q - z) * s, or q * s for the symmetric rows)."""
    W = np.zeros((N, K), np.float64)
    if qd["rows8"].size:
        W[qd["rows8"]] = qd["q8"].astype(np.float64) * np.repeat(qd["s8"].astype(np.float64), GROUP, axis=1)
    if qd["rows4"].size:
        qz = qd["q4"].astype(np.float64) - np.repeat(qd["z4"].astype(np.float64), GROUP, axis=1)
        W[qd["rows4"]] = qz * np.repeat(qd["s4"].astype(np.float64), GROUP, axis=1)
    return W
