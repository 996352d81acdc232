"""Pins of the oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: exact
rational arithmetic (fractions.Fraction), brute-force searches over all codes,
closed forms on grid-aligned inputs, invariants and the figures the MixLLM
page prints.  A plausible slip in the oracle (a dropped term, a wrong sign,
a transposed bitmap, a swapped pair in the unpacker) fails one of them.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import blockquant as bq
from oracle import image, model, w48

ALLOWED = (1, 2, 3, 4, 6, 8)


# ----------------------------------------------------------------------------
# exact helpers (independent of numpy's rounding)
# ----------------------------------------------------------------------------
def nearest_fp16(fr: Fraction) -> np.float16:
    """The fp16 closest to a rational, ties to the even bit pattern."""
    c = np.float16(float(fr))
    cands = {c, np.nextafter(c, np.float16(np.inf)), np.nextafter(c, np.float16(-np.inf))}
    cands = [h for h in cands if np.isfinite(h)]
    best = min(cands, key=lambda h: (abs(Fraction(float(h)) - fr), int(np.array(h).view(np.uint16)) & 1))
    return np.float16(best)


def nearest_code(v: Fraction, s: Fraction, z: int, L: int) -> int:
    """Brute force: the code q in [0, L] whose grid point (q - z) s is closest
    to v; on a tie the one with (q - z) even (round-half-even of v / s)."""
    return min(range(L + 1), key=lambda q: (abs(v - (q - z) * s), (q - z) % 2))


def brute_scale_zero(vals, b):
    lo, hi = min(vals), max(vals)
    L = 2 ** b - 1
    if hi > lo:
        s16 = nearest_fp16((hi - lo) / L)
        if s16 == 0:
            s16 = np.float16(2.0 ** -24)
    else:
        s16 = np.float16(abs(float(lo))) if lo != 0 else np.float16(1.0)
    s = Fraction(float(s16))
    z = min(max(round(-lo / s), 0), L)          # Python rounds Fractions half-even
    return s16, s, z


def small_matrix(N, K, seed, scale=0.02):
    g = np.random.default_rng(seed)
    W = (scale * g.standard_normal((N, K))).astype(np.float16)
    W[g.random((N, K)) < 0.01] *= np.float16(8)
    return W


# ----------------------------------------------------------------------------
# fp16 rounding used for scales
# ----------------------------------------------------------------------------
def test_fp16_rounding_is_nearest_even():
    g = np.random.default_rng(0)
    vals = np.concatenate([g.standard_normal(300) * 10.0 ** g.integers(-7, 4, 300),
                           g.random(50) * 2 ** -20])
    for v in vals:
        assert bq.fp16_rne(np.float64(v)) == nearest_fp16(Fraction(float(v)))
    # exact midpoints between neighbouring fp16 values go to the even one
    for h in np.float16([1.0, 0.0999, 3.14, 2 ** -14, 1000.0]):
        up = np.nextafter(h, np.float16(np.inf))
        mid = (Fraction(float(h)) + Fraction(float(up))) / 2
        got = bq.fp16_rne(np.float64(float(mid)))
        even = h if (int(np.array(h).view(np.uint16)) & 1) == 0 else up
        assert got == even


# ----------------------------------------------------------------------------
# affine group quantizer, block bitwidth map
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("b", ALLOWED)
def test_uniform_bitwidth_is_plain_group_rtn(b):
    """With one bitwidth everywhere the block quantizer is plain group-128
    RTN: scale, zero and every code agree with an exhaustive search."""
    N, K = 64, 256
    W = small_matrix(N, K, 10 + b)
    q, s16, z16 = bq.quantize_blocks(W, synth.uniform_bitmap(N, K, b))
    L = 2 ** b - 1
    for n in range(0, N, 7):
        for g in range(K // 128):
            vals = [Fraction(float(v)) for v in W[n, 128 * g:128 * g + 128]]
            s16_ref, s, z = brute_scale_zero(vals, b)
            assert s16[n, g] == s16_ref and z16[n, g] == z
            for k in range(0, 128, 3):
                assert q[n, 128 * g + k] == nearest_code(vals[k], s, z, L)


def test_mixed_bitmap_uses_the_block_of_each_group():
    """Mixed bitwidths: every (row, group) follows bits[row // 64][group]; a
    transposed or mis-indexed map changes the codes."""
    N, K = 192, 384
    W = small_matrix(N, K, 3)
    bits = np.array([[1, 8, 3], [6, 2, 4], [4, 3, 1]], np.uint8)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    for n in range(0, N, 5):
        for g in range(3):
            b = int(bits[n // 64, g])
            vals = [Fraction(float(v)) for v in W[n, 128 * g:128 * g + 128]]
            s16_ref, s, z = brute_scale_zero(vals, b)
            assert s16[n, g] == s16_ref and z16[n, g] == z
            assert q[n, 128 * g:128 * g + 128].max() <= 2 ** b - 1
            for k in (0, 17, 64, 101, 127):
                assert q[n, 128 * g + k] == nearest_code(vals[k], s, z, 2 ** b - 1)


def test_reconstruction_within_half_step_inside_clamp_range():
    N, K = 128, 512
    W = small_matrix(N, K, 5)
    bits = synth.random_bitmap(N, K, ALLOWED, 1)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    w = bq.dequant_fp32(q, s16, z16).astype(np.float64)
    s = np.repeat(s16.astype(np.float64), 128, axis=1)
    z = np.repeat(z16.astype(np.float64), 128, axis=1)
    L = np.repeat(np.repeat(2.0 ** bits.astype(np.float64) - 1, 64, 0), 128, 1)
    t = W.astype(np.float64) / s
    inside = (t >= -z - 0.5) & (t <= L - z + 0.5)
    assert inside.mean() > 0.99
    err = np.abs(W.astype(np.float64) - w)
    assert np.all(err[inside] <= s[inside] / 2 * (1 + 1e-12))
    assert np.all(q <= L)


def test_dequant_is_exact_in_fp32():
    N, K = 64, 256
    W = small_matrix(N, K, 6)
    q, s16, z16 = bq.quantize_blocks(W, np.array([[8, 3]], np.uint8))
    w = bq.dequant_fp32(q, s16, z16)
    assert w.dtype == np.float32
    for n in range(0, 64, 9):
        for k in range(0, 256, 11):
            exact = (int(q[n, k]) - Fraction(float(z16[n, k // 128]))) * Fraction(float(s16[n, k // 128]))
            assert Fraction(float(w[n, k])) == exact


@pytest.mark.parametrize("b", ALLOWED)
def test_grid_aligned_input_round_trips(b):
    """Closed form: a matrix already on a grid (q - z) * 2^-e with both end
    codes present in every group comes back with the same s, z and q."""
    g = np.random.default_rng(b)
    N, K = 64, 256
    L = 2 ** b - 1
    q0 = g.integers(0, L + 1, (N, K))
    q0[:, 0::128] = 0
    q0[:, 1::128] = L
    z0 = g.integers(0, L + 1, (N, K // 128))
    s0 = 2.0 ** -6
    W = ((q0 - np.repeat(z0, 128, 1)) * s0).astype(np.float16)
    assert np.array_equal(W.astype(np.float64), (q0 - np.repeat(z0, 128, 1)) * s0)
    q, s16, z16 = bq.quantize_blocks(W, synth.uniform_bitmap(N, K, b))
    assert np.all(s16 == np.float16(s0))
    assert np.array_equal(z16.astype(np.int64), z0)
    assert np.array_equal(q.astype(np.int64), q0)
    assert np.array_equal(bq.dequant_fp32(q, s16, z16), W.astype(np.float32))


def test_exact_ties_round_half_even_before_adding_zero():
    """Values exactly halfway between grid points: the code is
    rint(v / s) + z (ties to even on v / s, then the integer zero point), which
    differs from rint(v / s + z) when z is odd."""
    L = 15
    s0 = 2.0 ** -6
    W = np.zeros((64, 128), np.float64)
    W[:, 0] = -3 * s0                    # min -> z = 3 (odd)
    W[:, 1] = 12 * s0                    # max -> s = 15 s0 / 15 = s0
    W[:, 2:8] = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 4.5]) * s0
    W16 = W.astype(np.float16)
    q, s16, z16 = bq.quantize_blocks(W16, np.array([[4]], np.uint8))
    assert s16[0, 0] == np.float16(s0) and z16[0, 0] == 3
    assert list(q[0, 2:8]) == [0 + 3, 2 + 3, 2 + 3, 0 + 3, -2 + 3, 4 + 3]
    for k in range(2, 8):
        assert q[0, k] == nearest_code(Fraction(float(W16[0, k])), Fraction(s0), 3, L)


def test_degenerate_groups():
    W = np.zeros((64, 384), np.float16)
    W[:, 128:256] = np.float16(0.75)
    W[:, 256:384] = np.float16(-3.5)
    q, s16, z16 = bq.quantize_blocks(W, np.array([[1, 2, 8]], np.uint8))
    w = bq.dequant_fp32(q, s16, z16)
    assert np.array_equal(w, W.astype(np.float32))       # exact reconstruction
    assert np.all(s16[:, 0] == 1) and np.all(q[:, :128] == 0)
    # a group whose range is below the smallest fp16 scale keeps a nonzero s
    W2 = np.zeros((64, 128), np.float16)
    W2[:, 0] = np.float16(2.0 ** -24)
    _, s2, _ = bq.quantize_blocks(W2, np.array([[8]], np.uint8))
    assert np.all(s2 == np.float16(2.0 ** -24))


def test_shape_and_bitwidth_validation():
    with pytest.raises(ValueError):
        bq.quantize_blocks(np.zeros((64, 200), np.float16), np.ones((1, 1), np.uint8))
    with pytest.raises(ValueError):
        bq.quantize_blocks(np.zeros((64, 128), np.float16), np.array([[5]], np.uint8))
    with pytest.raises(ValueError):
        bq.quantize_blocks(np.zeros((128, 128), np.float16), np.ones((1, 2), np.uint8))


# ----------------------------------------------------------------------------
# the reference GEMM
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,M", [(64, 128, 1), (128, 256, 3), (192, 384, 5)])
def test_gemm_matches_exact_rational_dot_products(N, K, M):
    W = small_matrix(N, K, N + K)
    bits = synth.random_bitmap(N, K, ALLOWED, N)
    x = np.random.default_rng(M).standard_normal((M, K)).astype(np.float16)
    y = bq.reference_gemm(x, W, bits)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    for m in range(M):
        for n in range(0, N, 13):
            exact = sum(Fraction(float(x[m, k])) * (int(q[n, k]) - Fraction(float(z16[n, k // 128])))
                        * Fraction(float(s16[n, k // 128])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)


def test_gemm_closed_form_top_code():
    """All codes at 2^b - 1 with z = 0 and s = 1 give y = (2^b - 1) * sum(x)."""
    for b in ALLOWED:
        L = 2 ** b - 1
        W = np.full((64, 256), L, np.float16)
        W[:, 0::128] = 0                   # keeps min 0 so z = 0 and s = 1
        x = np.random.default_rng(b).standard_normal((2, 256)).astype(np.float16)
        q, s16, z16 = bq.quantize_blocks(W, synth.uniform_bitmap(64, 256, b))
        assert np.all(s16 == 1) and np.all(z16 == 0)
        y = bq.reference_gemm(x, W, synth.uniform_bitmap(64, 256, b))
        xs = x.astype(np.float64)
        expect = L * (xs.sum(axis=1) - xs[:, 0] - xs[:, 128])
        assert np.allclose(y, expect[:, None], rtol=1e-13, atol=1e-12)


def test_reference_rows_agrees_with_full_reference():
    N, K = 256, 384
    W = small_matrix(N, K, 9)
    bits = synth.random_bitmap(N, K, ALLOWED, 9)
    x = np.random.default_rng(2).standard_normal((3, K)).astype(np.float16)
    full = bq.reference_gemm(x, W, bits)
    rows = np.array([0, 63, 64, 130, 255])
    assert np.allclose(bq.reference_rows(x, W, bits, rows), full[:, rows], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------
# packed image: size identity and the oracle's reader
# ----------------------------------------------------------------------------
def test_packed_size_identity():
    _, bits, _ = synth.linear_4096()
    assert [(b, int((bits == b).sum())) for b in (2, 3, 4)] == [(2, 512), (3, 819), (4, 717)]
    codes = sum(64 * 128 * int(b) // 8 for b in bits.reshape(-1))
    assert codes == 6_501_376
    # by hand: 256 (header, padded) + 2048 (bitwidths) + 8448 (2049 offsets, padded)
    # + 524,288 (scale/zero records) + 6,501,376 (codes)
    assert image.block_image_size(bits) == 7_036_416


def _slow_block_image(q, s16, z16, bits):
    """Write a block image one code at a time from the format description."""
    N, K = q.shape
    nbr, nbc = N // 64, K // 128
    nblk = nbr * nbc
    al = lambda n: (n + 255) // 256 * 256
    bits_off = 256
    offs_off = al(bits_off + nblk)
    sz_off = al(offs_off + 4 * (nblk + 1))
    codes_off = sz_off + 256 * nblk
    total_kib = int(bits.astype(np.int64).sum())
    buf = bytearray(codes_off + 1024 * total_kib)
    hdr = np.array([0x31424247, 1, N, K, nbr, nbc], "<u4").tobytes()
    hdr += np.array([bits_off, offs_off, sz_off, codes_off, 1024 * total_kib], "<u8").tobytes()
    buf[:64] = hdr
    planes = {1: (1,), 2: (2,), 3: (2, 1), 4: (4,), 6: (4, 2), 8: (4, 4)}
    kib = 0
    for br in range(nbr):
        for bc in range(nbc):
            blk = br * nbc + bc
            b = int(bits[br, bc])
            buf[bits_off + blk] = b
            buf[offs_off + 4 * blk:offs_off + 4 * blk + 4] = int(kib).to_bytes(4, "little")
            for r in range(64):
                o = sz_off + 256 * blk + 4 * (4 * (r % 16) + r // 16)
                buf[o:o + 2] = np.float16(s16[64 * br + r, bc]).tobytes()
                buf[o + 2:o + 4] = np.float16(z16[64 * br + r, bc]).tobytes()
            base = codes_off + 1024 * kib
            shift = 0
            for w in planes[b]:
                npair = 16 // w
                words = [0] * (256 * w)          # u32 words of the plane
                # place each code: row tile rt, column tile kt, lane group g,
                # word c, half h; tile 4 kt + rt is field i of slot j
                for r in range(64):
                    for k in range(128):
                        rt, r16 = divmod(r, 16)
                        kt, g, c, h = k // 32, (k % 32) // 8, (k % 8) // 2, k % 2
                        j, i = divmod(4 * kt + rt, npair)
                        code = (int(q[64 * br + r, 128 * bc + k]) >> shift) & ((1 << w) - 1)
                        words[256 * j + 4 * (16 * g + r16) + c] |= code << (16 * h + w * i)
                for n, word in enumerate(words):
                    buf[base + 4 * n:base + 4 * n + 4] = word.to_bytes(4, "little")
                base += 1024 * w
                shift += w
            kib += b
    buf[offs_off + 4 * nblk:offs_off + 4 * nblk + 4] = int(kib).to_bytes(4, "little")
    return bytes(buf)


def test_oracle_reader_against_slow_writer():
    N, K = 128, 384
    g = np.random.default_rng(4)
    bits = np.array([[1, 2, 3], [4, 6, 8]], np.uint8)
    L = np.repeat(np.repeat(2 ** bits.astype(np.int64) - 1, 64, 0), 128, 1)
    q = (g.integers(0, 256, (N, K)) % (L + 1)).astype(np.uint8)
    s16 = g.standard_normal((N, 3)).astype(np.float16)
    z16 = (g.integers(0, 256, (N, 3)) % (np.repeat(2 ** bits.astype(np.int64), 64, 0))).astype(np.float16)
    img = _slow_block_image(q, s16, z16, bits)
    assert len(img) == image.block_image_size(bits)
    d = image.read_block_image(img)
    assert np.array_equal(d["bits"], bits)
    assert np.array_equal(d["q"], q)
    assert np.array_equal(d["s16"].view(np.uint16), s16.view(np.uint16))
    assert np.array_equal(d["z16"], z16)


# ----------------------------------------------------------------------------
# 64x64 blocks (groups of 64 columns)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("b", ALLOWED)
def test_64x64_uniform_bitwidth_is_plain_group64_rtn(b):
    """64x64 blocks with one bitwidth everywhere: plain group-64 RTN --
    scale, zero and codes agree with an exhaustive search per 64 columns."""
    N, K = 64, 256
    W = small_matrix(N, K, 20 + b)
    q, s16, z16 = bq.quantize_blocks(W, np.full((1, 4), b, np.uint8), block_cols=64)
    assert s16.shape == (N, 4)
    L = 2 ** b - 1
    for n in range(0, N, 9):
        for g in range(4):
            vals = [Fraction(float(v)) for v in W[n, 64 * g:64 * g + 64]]
            s16_ref, s, z = brute_scale_zero(vals, b)
            assert s16[n, g] == s16_ref and z16[n, g] == z
            for k in range(0, 64, 3):
                assert q[n, 64 * g + k] == nearest_code(vals[k], s, z, L)


def test_64x64_mixed_bitmap_uses_the_block_of_each_group():
    """Each (row, 64-column group) follows bits[row // 64][col // 64]; the same
    matrix with 64x128 blocks quantizes 128-column groups instead."""
    N, K = 128, 256
    W = small_matrix(N, K, 23)
    bits = np.array([[1, 8, 3, 6], [2, 4, 8, 1]], np.uint8)
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    for n in range(0, N, 7):
        for g in range(4):
            b = int(bits[n // 64, g])
            vals = [Fraction(float(v)) for v in W[n, 64 * g:64 * g + 64]]
            s16_ref, s, z = brute_scale_zero(vals, b)
            assert s16[n, g] == s16_ref and z16[n, g] == z
            for k in (0, 13, 31, 32, 63):
                assert q[n, 64 * g + k] == nearest_code(vals[k], s, z, 2 ** b - 1)
    with pytest.raises(ValueError):       # a 64x128 map does not fit 64x64 blocks
        bq.quantize_blocks(W, bits[:, :2], block_cols=64)


def test_64x64_gemm_matches_exact_rational_dot_products():
    N, K, M = 128, 192, 2
    W = small_matrix(N, K, 24)
    bits = synth.random_bitmap64(N, K, ALLOWED, 24)
    x = np.random.default_rng(5).standard_normal((M, K)).astype(np.float16)
    y = bq.reference_gemm(x, W, bits, block_cols=64)
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    for m in range(M):
        for n in range(0, N, 11):
            exact = sum(Fraction(float(x[m, k])) * (int(q[n, k]) - Fraction(float(z16[n, k // 64])))
                        * Fraction(float(s16[n, k // 64])) for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)
    rows = np.array([0, 63, 64, 127])
    assert np.allclose(bq.reference_rows(x, W, bits, rows, block_cols=64), y[:, rows], rtol=0, atol=1e-12)


def test_64x64_packed_size_identity():
    """Codes of a 64x64 block are 64 * 64 * b / 8 = 512 b bytes; by hand for a
    2 x 3 bitmap: 256 (header) + 256 (6 bitwidths, padded) + 256 (7 offsets,
    padded) + 1536 (scale/zero) + 512 * 24 (codes)."""
    bits = np.array([[1, 2, 3], [4, 6, 8]], np.uint8)
    assert sum(64 * 64 * int(b) // 8 for b in bits.reshape(-1)) == 12288
    assert image.block_image_size(bits, block_cols=64) == 256 + 256 + 256 + 1536 + 12288


def _slow_block_image_64(q, s16, z16, bits):
    """Write a 64x64-block image (version 2) one code at a time from the
    format description."""
    N, K = q.shape
    nbr, nbc = N // 64, K // 64
    nblk = nbr * nbc
    al = lambda n: (n + 255) // 256 * 256
    bits_off = 256
    offs_off = al(bits_off + nblk)
    sz_off = al(offs_off + 4 * (nblk + 1))
    codes_off = sz_off + 256 * nblk
    total = int(bits.astype(np.int64).sum())
    buf = bytearray(codes_off + 512 * total)
    hdr = np.array([0x31424247, 2, N, K, nbr, nbc], "<u4").tobytes()
    hdr += np.array([bits_off, offs_off, sz_off, codes_off, 512 * total], "<u8").tobytes()
    buf[:64] = hdr
    planes = {1: (1,), 2: (2,), 3: (2, 1), 4: (4,), 6: (4, 2), 8: (4, 4)}
    units = 0
    for br in range(nbr):
        for bc in range(nbc):
            blk = br * nbc + bc
            b = int(bits[br, bc])
            buf[bits_off + blk] = b
            buf[offs_off + 4 * blk:offs_off + 4 * blk + 4] = int(units).to_bytes(4, "little")
            for r in range(64):
                o = sz_off + 256 * blk + 4 * (4 * (r % 16) + r // 16)
                buf[o:o + 2] = np.float16(s16[64 * br + r, bc]).tobytes()
                buf[o + 2:o + 4] = np.float16(z16[64 * br + r, bc]).tobytes()
            base = codes_off + 512 * units
            shift = 0
            for w in planes[b]:
                per = 8 // w
                words = [0] * (128 * w)          # u32 words of the plane: [half-slot][lane][d]
                for r in range(64):
                    for k in range(64):
                        rt, r16 = divmod(r, 16)
                        kt, g, c, h = k // 32, (k % 32) // 8, (k % 8) // 2, k % 2
                        j, i = divmod(4 * kt + rt, per)
                        d, f = c // 2, (c % 2) * per + i
                        code = (int(q[64 * br + r, 64 * bc + k]) >> shift) & ((1 << w) - 1)
                        words[128 * j + 2 * (16 * g + r16) + d] |= code << (16 * h + w * f)
                for n, word in enumerate(words):
                    buf[base + 4 * n:base + 4 * n + 4] = word.to_bytes(4, "little")
                base += 512 * w
                shift += w
            units += b
    buf[offs_off + 4 * nblk:offs_off + 4 * nblk + 4] = int(units).to_bytes(4, "little")
    return bytes(buf)


def test_oracle_reader_64x64_against_slow_writer():
    N, K = 128, 192
    g = np.random.default_rng(6)
    bits = np.array([[1, 2, 3], [4, 6, 8]], np.uint8)
    L = np.repeat(np.repeat(2 ** bits.astype(np.int64) - 1, 64, 0), 64, 1)
    q = (g.integers(0, 256, (N, K)) % (L + 1)).astype(np.uint8)
    s16 = g.standard_normal((N, 3)).astype(np.float16)
    z16 = (g.integers(0, 256, (N, 3)) % (np.repeat(2 ** bits.astype(np.int64), 64, 0))).astype(np.float16)
    img = _slow_block_image_64(q, s16, z16, bits)
    assert len(img) == image.block_image_size(bits, block_cols=64)
    d = image.read_block_image(img)
    assert d["block_cols"] == 64
    assert np.array_equal(d["bits"], bits)
    assert np.array_equal(d["q"], q)
    assert np.array_equal(d["s16"].view(np.uint16), s16.view(np.uint16))
    assert np.array_equal(d["z16"], z16)


# ----------------------------------------------------------------------------
# output-feature mixed W8/W4 x A8
# ----------------------------------------------------------------------------
def test_sym8_brute_force():
    W = small_matrix(16, 256, 12)
    q, s16 = w48.quant_sym8(W)
    for n in range(16):
        for g in range(2):
            vals = [Fraction(float(v)) for v in W[n, 128 * g:128 * g + 128]]
            a = max(abs(v) for v in vals)
            assert s16[n, g] == nearest_fp16(a / 127)
            s = Fraction(float(s16[n, g]))
            for k in range(0, 128, 5):
                best = min(range(-127, 128), key=lambda c: (abs(vals[k] - c * s), c % 2))
                assert q[n, 128 * g + k] == best


def test_asym4_matches_block_quantizer_at_4_bits():
    W = small_matrix(64, 256, 13)
    q, s, z = w48.quant_asym4(W)
    q2, s2, z2 = bq.quantize_blocks(W, synth.uniform_bitmap(64, 256, 4))
    assert np.array_equal(q, q2) and np.array_equal(s, s2) and np.array_equal(z, z2.astype(np.uint8))


def test_act_quant_per_token_and_group():
    g = np.random.default_rng(7)
    x = g.standard_normal((5, 512)).astype(np.float16)
    x[2] = 0
    for group in (None, 128):
        A, s = w48.quant_act(x, group)
        gs = 512 if group is None else 128
        sa = (s[:, None] if group is None else s).astype(np.float64)
        sa = np.repeat(sa, gs, axis=1)
        xs = x.astype(np.float64)
        assert A.dtype == np.int8 and np.abs(A.astype(np.int64)).max() <= 127
        ok = np.abs(xs - A * sa) <= sa / 2 * (1 + 2 ** -20)
        assert ok.all()
        for m in (0, 1, 3, 4):                  # scale = fp16(fp32(max|x| / 127))
            for gi in range(512 // gs):
                seg = xs[m, gi * gs:(gi + 1) * gs]
                a = Fraction(float(np.abs(seg).max()))
                s32 = Fraction(float(np.float32(float(a)) / np.float32(127)))
                sv = s[m] if group is None else s[m, gi]
                assert sv == nearest_fp16(s32)
        assert np.all(A[2] == 0)


def test_two_step_identity_exact_in_rationals():
    """Two-step dequantization (integer group product, then both scales)
    equals the product of the dequantized operands, exactly."""
    g = np.random.default_rng(8)
    M, N, K = 3, 6, 256
    x = g.standard_normal((M, K)).astype(np.float16)
    W = small_matrix(N, K, 8)
    rows8 = np.array([1, 4])
    qd = w48.quantize_w48(W, rows8)
    A, sa = w48.quant_act(x, 128)
    Wd = w48.dequant_rows(qd, N, K)
    y = w48.reference(x, W, rows8, act_group=128, quant=qd)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(int(A[m, k])) * Fraction(float(sa[m, k // 128])) * Fraction(float(Wd[n, k]))
                        for k in range(K))
            assert abs(Fraction(float(y[m, n])) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)


def test_group_acc_unit_scales_is_int8_matmul():
    g = np.random.default_rng(9)
    A = g.integers(-127, 128, (4, 384)).astype(np.int8)
    Wz = g.integers(-127, 128, (5, 384)).astype(np.int64)
    acc = w48.group_acc(A, Wz)
    assert np.array_equal(acc.sum(axis=2), A.astype(np.int64) @ Wz.T)
    assert np.abs(acc).max() <= 127 * 127 * 128


@pytest.mark.parametrize("frac", [0.0, 0.1, 1.0])
def test_mixed_split_equals_unpartitioned_product(frac):
    """p0 (all 4-bit: W4A8), 10 % and p100 (all 8-bit: W8A8): the partitioned
    result, gathered back to original rows, equals the plain product of
    dequantized activations and weights."""
    g = np.random.default_rng(11)
    N, K, M = 48, 256, 4
    W = small_matrix(N, K, 11)
    x = g.standard_normal((M, K)).astype(np.float16)
    rows8 = synth.salient_rows_by_l2(W, frac) if frac < 1.0 else np.arange(N)
    qd = w48.quantize_w48(W, rows8)
    A, sa = w48.quant_act(x)
    plain = (A.astype(np.float64) * sa.astype(np.float64)[:, None]) @ w48.dequant_rows(qd, N, K).T
    y = w48.reference(x, W, rows8, quant=qd)
    assert np.allclose(y, plain, rtol=1e-12, atol=1e-12)
    if frac == 0.0:
        assert qd["rows8"].size == 0
    if frac == 1.0:
        assert qd["rows4"].size == 0


def test_salient_rows_are_the_largest_norms():
    W = small_matrix(640, 256, 14)
    r8 = synth.salient_rows_by_l2(W, 0.10)
    assert r8.size == 64 and np.all(np.diff(r8) > 0)
    nrm = np.linalg.norm(W.astype(np.float64), axis=1)
    rest = np.setdiff1d(np.arange(640), r8)
    assert nrm[r8].min() >= nrm[rest].max()
    assert int(np.floor(0.1 * 28672 + 0.5)) == 2867


# ----------------------------------------------------------------------------
# the page's intensity model (printed values)
# ----------------------------------------------------------------------------
def _golden(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    out = {}
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if line:
            k, v = line.split("=")
            out[k.strip()] = float(v)
    return out


def test_intensity_model_printed_values():
    gold = _golden("mixllm_intensity.txt")
    base = model.intensity(512, 4096, 4096, 1.0, 1.0)
    w4 = model.intensity(512, 4096, 4096, 1.0, 0.5)
    a4 = model.intensity(512, 4096, 4096, 0.5, 1.0)
    assert round(100 * (w4 / base - 1), 2) == gold["weight_8_to_4_gain_percent"]
    assert round(100 * (a4 / base - 1), 2) == gold["act_8_to_4_gain_percent"]


def _slow_w48_image(N, K, rows8, rows4, q8, s8, q4, s4, z4):
    """Write a W4/W8 image one element at a time from the format description."""
    n8, n4 = len(rows8), len(rows4)
    T8, T4 = (n8 + 15) // 16, (n4 + 15) // 16
    G, KT = K // 128, K // 64
    al = lambda n: (n + 255) // 256 * 256
    rows_off = 256
    s_off = al(rows_off + 4 * 16 * (T8 + T4))
    z_off = al(s_off + 2 * (T8 + T4) * G * 16)
    c8_off = al(z_off + T4 * G * 16)
    c4_off = al(c8_off + T8 * KT * 1024)
    buf = bytearray(c4_off + T4 * KT * 512)
    buf[:32] = np.array([0x38345747, 1, N, K, n8, n4, T8, T4], "<u4").tobytes()
    buf[32:72] = np.array([rows_off, s_off, z_off, c8_off, c4_off], "<u8").tobytes()
    packed_rows = [int(r) for r in rows8] + [-1] * (16 * T8 - n8) + [int(r) for r in rows4] + [-1] * (16 * T4 - n4)
    for i, r in enumerate(packed_rows):
        buf[rows_off + 4 * i:rows_off + 4 * i + 4] = int(r).to_bytes(4, "little", signed=True)
    for t in range(T8 + T4):
        for g in range(G):
            for r in range(16):
                if t < T8:
                    v = s8[16 * t + r, g] if 16 * t + r < n8 else np.float16(0)
                else:
                    j = 16 * (t - T8) + r
                    v = s4[j, g] if j < n4 else np.float16(0)
                o = s_off + 2 * ((t * G + g) * 16 + r)
                buf[o:o + 2] = np.float16(v).tobytes()
    for t in range(T4):
        for g in range(G):
            for r in range(16):
                j = 16 * t + r
                buf[z_off + (t * G + g) * 16 + r] = int(z4[j, g]) if j < n4 else 0
    for t in range(T8):
        for kt in range(KT):
            for lane in range(64):
                for e in range(16):
                    row, col = 16 * t + lane % 16, 64 * kt + 16 * (lane // 16) + e
                    v = int(q8[row, col]) if row < n8 else 0
                    buf[c8_off + (t * KT + kt) * 1024 + 16 * lane + e] = v & 0xFF
    for t in range(T4):
        for kt in range(KT):
            for lane in range(64):
                for j in range(2):
                    for i in range(4):
                        row = 16 * t + lane % 16
                        c0 = 64 * kt + 16 * (lane // 16) + 8 * j + i
                        lo = int(q4[row, c0]) if row < n4 else 0
                        hi = int(q4[row, c0 + 4]) if row < n4 else 0
                        buf[c4_off + (t * KT + kt) * 512 + 8 * lane + 4 * j + i] = lo | (hi << 4)
    return bytes(buf)


def test_oracle_w48_reader_against_slow_writer():
    g = np.random.default_rng(21)
    N, K = 40, 256
    rows8 = np.array([3, 17, 30])
    rows4 = np.setdiff1d(np.arange(N), rows8)
    q8 = g.integers(-127, 128, (3, K)).astype(np.int8)
    q4 = g.integers(0, 16, (N - 3, K)).astype(np.uint8)
    s8 = g.standard_normal((3, 2)).astype(np.float16)
    s4 = g.standard_normal((N - 3, 2)).astype(np.float16)
    z4 = g.integers(0, 16, (N - 3, 2)).astype(np.uint8)
    img = _slow_w48_image(N, K, rows8, rows4, q8, s8, q4, s4, z4)
    assert len(img) == image.w48_image_size(N, K, 3)
    d = image.read_w48_image(img)
    assert np.array_equal(d["rows8"], rows8) and np.array_equal(d["rows4"], rows4)
    assert np.array_equal(d["q8"], q8) and np.array_equal(d["q4"], q4)
    assert np.array_equal(d["s8"].view(np.uint16), s8.view(np.uint16))
    assert np.array_equal(d["s4"].view(np.uint16), s4.view(np.uint16))
    assert np.array_equal(d["z4"], z4)
    assert np.all(d["q8_pad"] == 0) and np.all(d["q4_pad"] == 0)


# ----------------------------------------------------------------------------
# the parity checker itself
# ----------------------------------------------------------------------------
def test_rel_inf_err_hand_cases():
    """||y - y_ref||_inf / ||y_ref||_inf on hand-computed cases: the maximum
    (not a mean) over every element, the reference's norm (not y's) below,
    an absolute error for an all-zero reference, and a failure for NaN or
    infinite outputs."""
    f = bq.rel_inf_err
    assert f([1.0, -4.0, 2.0], [1.0, -4.0, 2.0]) == 0.0
    assert f([1.5, -4.0, 2.0], [1.0, -4.0, 2.0]) == 0.125            # 0.5 / 4
    # the denominator is max|y_ref| = 2, not max|y| = 10 (which gives 0.8)
    assert f([1.0, 10.0], [1.0, 2.0]) == 4.0
    # a maximum, not a mean: one element off by 0.4 out of four (a mean gives 0.05)
    assert f([2.0, 2.0, 2.0, 2.4], [2.0, 2.0, 2.0, 2.0]) == pytest.approx(0.2, rel=1e-15)
    # over all elements of a 2-D output
    assert f([[1.0, 1.0], [0.0, -8.0]], [[1.0, 0.0], [0.0, -8.0]]) == 0.125
    # a negated output is off by twice the reference
    assert f([-3.0, 1.0], [3.0, -1.0]) == 2.0
    # all-zero reference: the absolute error
    assert f([0.0, 3e-4], [0.0, 0.0]) == 3e-4
    # NaN or inf anywhere in y fails any tolerance
    for bad in (np.nan, np.inf, -np.inf):
        assert not (f([1.0, bad], [1.0, 2.0]) <= 2e-3)


# ----------------------------------------------------------------------------
# activation quantizer at exact ties, and codes for given scales and zeros
# ----------------------------------------------------------------------------
def _round_half_even(fr: Fraction) -> int:
    """Python's round() of a Fraction is round-half-to-even (exact)."""
    return round(fr)


@pytest.mark.parametrize("group", [None, 128])
def test_act_quant_exact_ties_half_even(group):
    """x / s exactly halfway between two integers: round-half-to-even picks
    the even one, where round-half-up (2.5 -> 3, 126.5 -> 127) and
    round-half-away (-2.5 -> -3) do not.  The scale is exact: max|x| =
    127 * 2^-4 gives s = 2^-4."""
    s = Fraction(1, 16)
    ties = [0.5, 1.5, 2.5, 3.5, 4.5, 126.5, -0.5, -1.5, -2.5, -3.5, -126.5]
    K = 256
    x = np.zeros((2, K), np.float16)
    for m in range(2):
        for gi in range(K // 128):
            x[m, 128 * gi] = np.float16(127 * float(s) * (1 if m == 0 else -1))
            for j, t in enumerate(ties):
                x[m, 128 * gi + 1 + j] = np.float16(t * float(s))
    assert Fraction(float(x[0, 1 + ties.index(126.5)])) == Fraction(253, 32)   # exact in fp16
    A, sa = w48.quant_act(x, group)
    assert np.all(sa.astype(np.float64) == float(s))
    for m in range(2):
        for k in range(K):
            want = _round_half_even(Fraction(float(x[m, k])) / s)
            assert A[m, k] == max(-127, min(127, want)), (m, k, float(x[m, k]))
    # the cases that tell the rules apart
    assert A[0, 1 + ties.index(2.5)] == 2 and A[0, 1 + ties.index(-2.5)] == -2
    assert A[0, 1 + ties.index(126.5)] == 126 and A[0, 1 + ties.index(-1.5)] == -2


def test_codes_with_given_scale_zero_brute_force():
    """Codes for caller-given scales and zeros (a clipping search's, say):
    every checked code is the in-range code whose grid point (q - z) s is
    nearest to w, ties to (q - z) even -- found by trying every code.  The
    inputs include exact ties, values beyond both ends of the grid and
    zeros at both ends of the range, over every bitwidth."""
    g = np.random.default_rng(31)
    bits = np.array([[1, 2, 3], [4, 6, 8]], np.uint8)
    N, K = 128, 384
    G = K // 128
    L = (2 ** np.repeat(bits.astype(np.int64), 64, axis=0)) - 1          # [N][G]
    s16 = (g.uniform(0.002, 0.03, (N, G))).astype(np.float16)
    z = np.floor(g.random((N, G)) * (L + 1)).astype(np.int64)
    z[0] = 0
    z[1] = L[1]
    W = np.empty((N, K), np.float16)
    ties = {}
    for n in range(N):
        for gi in range(G):
            s = float(s16[n, gi])
            lo, hi = -z[n, gi] - 2.0, L[n, gi] - z[n, gi] + 2.0        # a little beyond both ends
            W[n, 128 * gi:128 * gi + 128] = (g.uniform(lo, hi, 128) * s).astype(np.float16)
            for j in range(4):                                          # exact ties, if fp16 holds them
                t = float(g.integers(int(lo), int(hi))) + 0.5
                v = np.float16(t * s)
                if Fraction(float(v)) == Fraction(t) * Fraction(s):
                    W[n, 128 * gi + 120 + j] = v
                    ties[(n, gi)] = ties.get((n, gi), 0) + 1
    assert sum(ties.values()) > 50
    q = bq.codes_with(W, bits, s16, z.astype(np.float16))
    for n in range(N):
        for gi in range(G):
            s = Fraction(float(s16[n, gi]))
            for k in list(range(0, 120, 9)) + list(range(120, 128)):
                v = Fraction(float(W[n, 128 * gi + k]))
                assert q[n, 128 * gi + k] == nearest_code(v, s, int(z[n, gi]), int(L[n, gi])), (n, gi, k)
