"""Host packer and C-ABI checks (CPU only, no kernel launches).

The library's packer (C++) must produce exactly the codes, scales and zeros of
the oracle's quantizer; the oracle reads the packed bytes with its own
unpacker, written from the format description.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
from oracle import blockquant as bq
from oracle import image as oimg
from oracle import w48 as ow48

gbb = pytest.importorskip("gemm_block_bit_amd")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ALLOWED = (1, 2, 3, 4, 6, 8)


def header_functions():
    txt = open(os.path.join(ROOT, "include", "gbb.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(gbb_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    so = ctypes.CDLL(gbb.binding.LIB_PATH)
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(so, n), n
    assert set(names) == set(gbb.binding.EXPORTS)
    assert gbb.version() == 100


def small(N, K, seed):
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((N, K))).astype(np.float16)
    W[g.random((N, K)) < 0.005] *= np.float16(10)
    return W


def assert_same_quant(img, W, bits):
    d = oimg.read_block_image(img)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    assert d["N"] == W.shape[0] and d["K"] == W.shape[1]
    assert np.array_equal(d["bits"], bits)
    assert np.array_equal(d["q"], q)
    assert np.array_equal(d["s16"].view(np.uint16), s16.view(np.uint16))
    assert np.array_equal(d["z16"].view(np.uint16), z16.view(np.uint16))
    assert d["size"] == len(img) == oimg.block_image_size(bits)


@pytest.mark.parametrize("b", ALLOWED)
def test_pack_uniform_bits_bit_exact(b):
    W = small(128, 256, b)
    bits = synth.uniform_bitmap(128, 256, b)
    img, s, z = gbb.pack_blocks(W, bits)
    assert_same_quant(img, W, bits)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    assert np.array_equal(s.view(np.uint16), s16.view(np.uint16)) and np.array_equal(z, z16)


@pytest.mark.parametrize("N,K,seed", [(64, 128, 0), (192, 384, 1), (320, 1280, 2)])
def test_pack_mixed_bits_bit_exact(N, K, seed):
    W = small(N, K, seed)
    bits = synth.random_bitmap(N, K, ALLOWED, seed)
    img, _, _ = gbb.pack_blocks(W, bits)
    assert_same_quant(img, W, bits)


def test_pack_linear_4096_workload():
    W, bits, _ = synth.linear_4096()
    img, _, _ = gbb.pack_blocks(W, bits)
    assert len(img) == 7_036_416
    assert_same_quant(img, W, bits)


def test_pack_edge_values():
    """Constant groups, zero groups, tiny ranges, subnormals, +-65504."""
    W = np.zeros((64, 768), np.float16)
    W[:, 128:256] = np.float16(-0.5)
    W[:, 256:384] = np.float16(2.0 ** -24) * np.arange(128)
    W[:3, 384:512] = np.float16(65504)
    W[3:, 384:512] = np.float16(-65504)
    W[:, 512] = np.float16(65504)
    W[:, 640:768] = np.float16(1e-3)
    W[5, 700] = np.float16(1.0009765625e-3)
    for b in ALLOWED:
        bits = synth.uniform_bitmap(64, 768, b)
        img, _, _ = gbb.pack_blocks(W, bits)
        assert_same_quant(img, W, bits)


def test_pack_is_deterministic():
    W = small(256, 512, 7)
    bits = synth.random_bitmap(256, 512, ALLOWED, 7)
    a, _, _ = gbb.pack_blocks(W, bits)
    b, _, _ = gbb.pack_blocks(W, bits)
    assert np.array_equal(a, b)


def test_pack_with_given_scale_zero():
    W = small(128, 256, 9)
    bits = synth.random_bitmap(128, 256, ALLOWED, 9)
    _, s, z = gbb.pack_blocks(W, bits)
    s_clip = (s.astype(np.float32) * np.float32(0.85)).astype(np.float16)   # e.g. a clipping search
    img, _, _ = gbb.pack_blocks(W, bits, s_clip, z)
    d = oimg.read_block_image(img)
    assert np.array_equal(d["s16"].view(np.uint16), s_clip.view(np.uint16))
    assert np.array_equal(d["z16"], z)
    assert np.array_equal(d["q"], bq.codes_with(W, bits, s_clip, z))


def expect_status(status, fn, *a):
    with pytest.raises(gbb.GbbError) as e:
        fn(*a)
    assert e.value.status == status, str(e.value)


def test_pack_errors():
    W = small(64, 256, 1)
    expect_status(-3, gbb.pack_blocks, W, np.array([[4, 5]], np.uint8))
    expect_status(-3, gbb.pack_blocks, W, np.array([[0, 4]], np.uint8))
    expect_status(-2, gbb.pack_blocks, small(96, 256, 1), np.full((1, 2), 4, np.uint8))
    expect_status(-2, gbb.pack_blocks, small(64, 200, 1), np.full((1, 1), 4, np.uint8))
    Wn = W.copy()
    Wn[3, 7] = np.float16(np.inf)
    expect_status(-1, gbb.pack_blocks, Wn, np.full((1, 2), 4, np.uint8))
    bits = np.full((1, 2), 2, np.uint8)
    _, s, z = gbb.pack_blocks(W, bits)
    zbad = z.copy()
    zbad[0, 0] = np.float16(4)            # outside [0, 3]
    expect_status(-3, gbb.pack_blocks, W, bits, s, zbad)
    sbad = s.copy()
    sbad[1, 1] = np.float16(0)
    expect_status(-1, gbb.pack_blocks, W, bits, sbad, z)
    L = gbb.lib()
    Wu = W.view(np.uint16)
    img = np.empty(gbb.packed_bytes(bits, 64, 256), np.uint8)
    assert L.gbb_pack_blocks(Wu.ctypes.data, 64, 256, bits.ctypes.data, None, None, 0, img.ctypes.data,
                             img.size - 1) == -5
    assert L.gbb_pack_blocks(None, 64, 256, bits.ctypes.data, None, None, 0, img.ctypes.data, img.size) == -1
    assert L.gbb_pack_blocks(Wu.ctypes.data, 64, 256, bits.ctypes.data, None, None, 8, img.ctypes.data,
                             img.size) == -1
    assert L.gbb_packed_bytes(bits.ctypes.data, 64, 100) == 0
    assert b"multiple" in L.gbb_last_error()


def test_device_entry_points_reject_shapes_before_any_device_work():
    """Shape checks come first, on the host: a bogus (aligned) image pointer
    is never touched, so this runs without a GPU.  N and K are each capped at
    2^20 (the decode kernels address a token's activations with a 32-bit
    byte offset of up to 32 * 2 * K)."""
    L = gbb.lib()
    fake = 1 << 20
    for N, K, st in [((1 << 20) + 64, 128, -2), (64, (1 << 20) + 128, -2), (96, 128, -2), (64, 200, -2),
                     (0, 128, -1), (64, -128, -1)]:
        assert L.gbb_gemm_mixed_w(fake, N, K, fake, fake, 1, None, 0, None) == st, (N, K)
        assert L.gbb_gemm_mixed_w_path(fake, N, K, fake, fake, 1, None, 0, 1, None) == st, (N, K)
    assert b"exceeds" in (L.gbb_gemm_mixed_w(fake, 64, 1 << 21, fake, fake, 1, None, 0, None) == -2
                          and L.gbb_last_error())
    assert L.gbb_gemm_mixed_w(None, 64, 128, fake, fake, 1, None, 0, None) == -1
    assert L.gbb_gemm_mixed_w(fake + 8, 64, 128, fake, fake, 1, None, 0, None) == -4
    # grouped products: the count and every problem are checked first
    arr = lambda t, v: (t * len(v))(*v)
    imgs, Ns, Ks = arr(ctypes.c_void_p, [fake, fake]), arr(ctypes.c_int, [64, 64]), arr(ctypes.c_int, [128, 200])
    xs, ys = arr(ctypes.c_void_p, [fake, fake]), arr(ctypes.c_void_p, [fake + 4096, fake + 8192])
    assert L.gbb_gemm_mixed_w_batched(0, imgs, Ns, Ks, xs, ys, 1, None, 0, None) == -1
    assert L.gbb_gemm_mixed_w_batched(33, imgs, Ns, Ks, xs, ys, 1, None, 0, None) == -1
    assert L.gbb_gemm_mixed_w_batched(2, None, Ns, Ks, xs, ys, 1, None, 0, None) == -1
    assert L.gbb_gemm_mixed_w_batched(2, imgs, Ns, Ks, xs, ys, 1, None, 0, None) == -2
    assert b"problem 1" in L.gbb_last_error()
    assert L.gbb_gemm_mixed_w_batched_workspace(2, Ns, Ks, 1) == 0
    Ks[1] = 128
    assert L.gbb_gemm_mixed_w_batched_workspace(0, Ns, Ks, 1) == 0


@pytest.mark.parametrize("b", ALLOWED)
def test_pack_64x64_uniform_bits_bit_exact(b):
    W = small(128, 256, 40 + b)
    bits = np.full((2, 4), b, np.uint8)
    img, s, z = gbb.pack_blocks(W, bits, block_cols=64)
    d = oimg.read_block_image(img)
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    assert d["block_cols"] == 64 and np.array_equal(d["bits"], bits)
    assert np.array_equal(d["q"], q)
    assert np.array_equal(d["s16"].view(np.uint16), s16.view(np.uint16)) and np.array_equal(s, s16)
    assert np.array_equal(d["z16"].view(np.uint16), z16.view(np.uint16)) and np.array_equal(z, z16)
    assert len(img) == gbb.packed_bytes(bits, 128, 256, block_cols=64) == oimg.block_image_size(bits, 64)


@pytest.mark.parametrize("N,K,seed", [(64, 64, 0), (192, 448, 1), (320, 1152, 2)])
def test_pack_64x64_mixed_bits_bit_exact(N, K, seed):
    W = small(N, K, seed)
    bits = synth.random_bitmap64(N, K, ALLOWED, seed)
    img, _, _ = gbb.pack_blocks(W, bits, block_cols=64)
    d = oimg.read_block_image(img)
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    assert np.array_equal(d["q"], q)
    assert np.array_equal(d["s16"].view(np.uint16), s16.view(np.uint16))
    assert np.array_equal(d["z16"].view(np.uint16), z16.view(np.uint16))
    gbb.check_image(img, N, K)


def test_pack_64x64_given_scale_zero_and_errors():
    W = small(128, 192, 9)
    bits = synth.random_bitmap64(128, 192, ALLOWED, 9)
    _, s, z = gbb.pack_blocks(W, bits, block_cols=64)
    s_clip = (s.astype(np.float32) * np.float32(0.85)).astype(np.float16)
    img, _, _ = gbb.pack_blocks(W, bits, s_clip, z, block_cols=64)
    assert np.array_equal(oimg.read_block_image(img)["q"], bq.codes_with(W, bits, s_clip, z, block_cols=64))
    expect_status(-2, gbb.pack_blocks, small(64, 96, 1), np.full((1, 1), 4, np.uint8), None, None, 64)
    expect_status(-3, gbb.pack_blocks, small(64, 128, 1), np.array([[4, 7]], np.uint8), None, None, 64)
    L = gbb.lib()
    fake = 1 << 20
    # K must be a multiple of 64; 64 but not 128 is fine for this entry point
    assert L.gbb_gemm_mixed_w_64x64(fake, 64, 96, fake, fake + 8192, 1, None, 0, None) == -2
    assert L.gbb_gemm_mixed_w(fake, 64, 192, fake, fake + 8192, 1, None, 0, None) == -2
    assert L.gbb_gemm_mixed_w_64x64_workspace(64, 96, 1) == 0


def test_check_image():
    W = small(128, 256, 3)
    bits = synth.random_bitmap(128, 256, ALLOWED, 3)
    img, _, _ = gbb.pack_blocks(W, bits)
    gbb.check_image(img, 128, 256)
    expect_status(-6, gbb.check_image, img, 64, 256)
    bad = img.copy()
    bad[0] ^= 0xFF
    expect_status(-6, gbb.check_image, bad, 128, 256)
    expect_status(-6, gbb.check_image, img[:-1], 128, 256)


# ----------------------------------------------------------------------------
# W4/W8 packer
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,frac", [(48, 256, 0.1), (200, 384, 0.1), (64, 128, 0.0), (40, 256, 1.0)])
def test_pack_w48_bit_exact(N, K, frac):
    W = small(N, K, N)
    rows8 = synth.salient_rows_by_l2(W, frac) if frac < 1 else np.arange(N, dtype=np.int32)
    img, s, z = gbb.pack_w48(W, rows8)
    assert len(img) == oimg.w48_image_size(N, K, rows8.size)
    d = oimg.read_w48_image(img)
    ref = ow48.quantize_w48(W, rows8)
    assert np.array_equal(d["rows8"], ref["rows8"]) and np.array_equal(d["rows4"], ref["rows4"])
    assert np.array_equal(d["q8"], ref["q8"]) and np.array_equal(d["q4"], ref["q4"])
    assert np.array_equal(d["s8"].view(np.uint16), ref["s8"].view(np.uint16))
    assert np.array_equal(d["s4"].view(np.uint16), ref["s4"].view(np.uint16))
    assert np.array_equal(d["z4"], ref["z4"])
    assert np.all(d["q8_pad"] == 0) and np.all(d["q4_pad"] == 0)
    assert np.all(d["s_pad8"] == 0) and np.all(d["s_pad4"] == 0)
    pad = d["rows_pad"]
    assert np.sum(pad == -1) == (len(pad) - N)
    # scale / zero outputs in original row order
    if ref["rows8"].size:
        assert np.array_equal(s[ref["rows8"]].view(np.uint16), ref["s8"].view(np.uint16))
        assert np.all(z[ref["rows8"]] == 0)
    if ref["rows4"].size:
        assert np.array_equal(s[ref["rows4"]].view(np.uint16), ref["s4"].view(np.uint16))
        assert np.array_equal(z[ref["rows4"]], ref["z4"])


def test_pack_w48_errors():
    W = small(64, 256, 1)
    expect_status(-2, gbb.pack_w48, W, np.array([3, 3], np.int32))
    expect_status(-2, gbb.pack_w48, W, np.array([5, 2], np.int32))
    expect_status(-2, gbb.pack_w48, W, np.array([64], np.int32))
    expect_status(-2, gbb.pack_w48, small(64, 200, 1), np.array([1], np.int32))


def test_graph_create_argument_errors():
    """gbb_graph_create rejects bad arguments before touching the device."""
    import ctypes
    L = gbb.lib()
    out = ctypes.c_void_p(1)
    assert L.gbb_graph_create(0, None, None, None, None, None, 1, None, 0, ctypes.byref(out)) == -1
    assert out.value is None
    assert L.gbb_graph_create(1, None, None, None, None, None, 1, None, 0, ctypes.byref(out)) == -1
    assert L.gbb_graph_create(1, None, None, None, None, None, 1, None, 0, None) == -1
    assert L.gbb_graph_launch(None, None) == -1
    assert L.gbb_graph_destroy(None) == 0


def test_graph_wrapper_rejects_mismatched_shapes():
    """gbb.Graph checks x [M][K] and y [M][N] before calling the library."""
    import pytest

    torch = pytest.importorskip("torch")
    x = torch.zeros((4, 256), dtype=torch.float16)
    y = torch.zeros((4, 64), dtype=torch.float16)
    img = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        gbb.Graph([(img, 64, 128, x, y)])            # x has K = 256, not 128
    with pytest.raises(ValueError):
        gbb.Graph([(img, 128, 256, x, y)])           # y has N = 64, not 128
    with pytest.raises(ValueError):
        gbb.Graph([])


def _prefill_split(N, K, M, bc, cus):
    """The documented K split of the prefill kernel: when the 128 x 512 tile
    grid fills at most half the CUs, up to 16 segments of at least 1024
    columns, as many as fill the CUs once.  Returns (tiles, segments,
    workspace bytes: the segments' fp32 partials)."""
    nbc = K // bc
    tiles = -(-M // 128) * -(-N // 512)
    k = min(cus // tiles, 16, max(1, nbc // (1024 // bc))) if 2 * tiles <= cus else 1
    seg = -(-nbc // k)
    kseg = -(-nbc // seg)
    return tiles, kseg, (kseg * M * N * 4 if kseg > 1 else 0)


def _chunked(N, K, M, bc, cus):
    """The documented choice of 32-token decode chunks for M > 32: the
    chunk count (a ragged last chunk counted as half) times the larger of
    CUs / 4 and the split prefill's workgroups is at most 3/4 of the CUs."""
    tiles, kseg, _ = _prefill_split(N, K, M, bc, cus)
    halves = 2 * (M // 32) + (1 if M % 32 else 0)
    return M > 32 and 2 * halves * max(cus // 4, tiles * kseg) <= 3 * cus


@pytest.mark.parametrize("N,K", [(8192, 28672), (28672, 8192), (4096, 4096), (8192, 8192), (1024, 8192),
                                 (14336, 4096), (64, 128)])
def test_workspace_follows_the_batch_route(N, K):
    """Host side of the dispatch: above 32 tokens the batch runs as 32-token
    decode chunks when few chunks would each cost less than the prefill
    kernel on its (split) grid (256 CUs when the library finds no device);
    the workspace is then the larger of the full and the ragged last
    chunk's needs, and otherwise the prefill kernel's K split.  The
    path-aware query gives the same for path 0 and the split for a forced
    prefill."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    lib = gbb.lib()
    for M in (33, 64, 65, 96, 97, 128, 200, 256, 512, 1024, 2048):
        tiles, kseg, split_ws = _prefill_split(N, K, M, 128, cus)
        chunked = _chunked(N, K, M, 128, cus)
        need = gbb.gemm_mixed_w_workspace(N, K, M)
        assert lib.gbb_gemm_mixed_w_path_workspace(N, K, M, 0) == need
        assert lib.gbb_gemm_mixed_w_path_workspace(N, K, M, 2) == split_ws
        assert lib.gbb_gemm_mixed_w_path_workspace(N, K, M, 1) == 0   # the decode kernel takes M <= 32
        if not chunked:
            assert need == split_ws, (M, need)
            continue
        want = gbb.gemm_mixed_w_workspace(N, K, 32)
        if M % 32:
            want = max(want, gbb.gemm_mixed_w_workspace(N, K, M % 32))
        assert need == want, (M, need, want)
    if K % 64 == 0:
        for M in (512, 2048):
            assert lib.gbb_gemm_mixed_w_64x64_path_workspace(N, K, M, 2) == _prefill_split(N, K, M, 64, cus)[2]


def test_two_row_decode_workspace_is_partials():
    """17 <= M <= 32 on a matrix of at least 2^26 weights runs two block rows
    per workgroup; its K split keeps fp32 partials per segment (segments x M
    x N x 4 bytes) for an ordered second launch, with the documented segment
    count: as many as fill two workgroups per CU once, at most nbc / 8 and
    K / (32 M).  Elsewhere the decode route keeps 12 bytes per output (or
    none).  Every such workspace fits the 16 MiB of the allocation-free
    entry point."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    for N, K in [(8192, 8192), (8256, 8192), (4096, 16384), (10240, 8192), (8192, 28672), (57344, 8192),
                 (1 << 17, 512), (1024, 1 << 16), (4096, 4096), (1024, 8192)]:
        nbr, nbc = N // 64, K // 128
        for M in (1, 8, 16, 17, 24, 32):
            ws = gbb.gemm_mixed_w_workspace(N, K, M)
            if M > 16 and N * K >= 1 << 26:
                units = -(-nbr // 2)
                nseg = 1
                if units < 2 * cus:
                    nseg = min(2 * cus // units, max(1, nbc // 8), max(1, K // (32 * M)), 32)
                seg_cols = -(-nbc // nseg)
                nseg = -(-nbc // seg_cols)
                assert ws == (nseg * M * N * 4 if nseg > 1 else 0), (N, K, M, ws, nseg)
            else:
                assert ws in (0, M * N * 12), (N, K, M, ws)
            assert ws <= 16 << 20, (N, K, M, ws)


def test_64x64_workspace_sizes():
    """The 64x64 plans on the host (no device work): every shape with whole
    64-column blocks, down to a single block, gets a workspace of 0 or 12
    bytes per output of the decode launch (of the largest 32-token chunk),
    or above 32 tokens the prefill kernel's K split when that is the
    route."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    for N in (64, 128, 448, 8192):
        for K in (64, 128, 192, 1216, 4096, 28672):
            for M in (1, 2, 8, 16, 17, 32, 33, 70):
                ws = gbb.gemm_mixed_w_64x64_workspace(N, K, M)
                tiles, kseg, split_ws = _prefill_split(N, K, M, 64, cus)
                if M > 32 and not _chunked(N, K, M, 64, cus):
                    assert ws == split_ws, (N, K, M, ws)
                    continue
                assert ws in (0, min(M, 32) * N * 12) or (M > 32 and ws % (N * 12) == 0 and ws <= 32 * N * 12), \
                    (N, K, M, ws)
    assert gbb.gemm_mixed_w_64x64_workspace(64, 96, 1) == 0      # not whole blocks


@pytest.mark.parametrize("N,K,frac", [(8192, 28672, 0.1), (28672, 8192, 0.1), (2048, 16384, 0.1), (4096, 4096, 0.1),
                                      (48, 256, 0.1), (300, 1024, 1.0)])
def test_w48_split_workspace(N, K, frac):
    """Host side of the W4.4A8 K split.  The streaming kernel (M <= 64 with
    per-token scales, or per-group ones over an even group count; 64-token
    passes up to 128 tokens with per-token scales where the tile kernel has
    at most one row block per CU) splits K when its 64-row blocks, an 8-bit
    one counted twice, number at most 3/4 of the CUs; it then streams
    128-row blocks (two tiles per wave), cut into segments of at least 8
    groups, at most 16, about enough for two workgroups per CU, an 8-bit
    row block taking twice the segments of a 4-bit one.  The tile kernel (M > 64 otherwise)
    splits K when its token tiles x row blocks, a 4-bit one counted twice,
    fill at most half of its resident workgroups (three per CU, two with
    group scales), a 4-bit row block taking twice the segments of an 8-bit
    one.
    The workspace is the fp32 partials over the padded rows (the larger
    segment count x the call's (pass's) tokens x 16 (T8 + T4) x 4 bytes),
    0 everywhere else."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    n8 = int(np.floor(frac * N + 0.5))
    T8, T4 = -(-n8 // 16), -(-(N - n8) // 16)
    nb8, nb4, G = -(-T8 // 4), -(-T4 // 4), K // 128
    nrb8, nrb4 = -(-T8 // 4), -(-T4 // 8)
    kcap = max(1, min(16, G // 8))
    kseg = lambda k: -(-G // -(-G // k))
    P = 16 * (T8 + T4)
    k8 = k4 = 1
    if 4 * (2 * nb8 + nb4) <= 3 * cus:
        b8, b4 = -(-T8 // 8), -(-T4 // 8)   # split: 128-row blocks (two tiles per wave)
        if b4:
            k4 = max(1, min(kcap, 2 * cus // (2 * b8 + b4)))
            k8 = min(kcap, 2 * k4) if b8 else 1
        else:
            k8 = max(1, min(kcap, 2 * cus // b8))
    stream_kmax = max(kseg(k8), kseg(k4))

    def tile_kmax(M, ga):
        ntm = -(-M // 128)
        slots = (2 if ga == 128 else 3) * cus
        u = ntm * (nrb8 + 2 * nrb4)
        t8 = t4 = 1
        if 2 * u <= slots:
            if nrb8:
                t8 = max(1, min(kcap, slots // u))
                t4 = min(kcap, 2 * t8)
            else:
                t4 = max(1, min(kcap, slots // (ntm * nrb4)))
        return max(kseg(t8), kseg(t4))

    for M in (1, 16, 32, 64, 65, 96, 128, 129, 256, 512, 2048):
        for ga in (K, 128):
            if ga == 128:
                streams = M <= 64 and G % 2 == 0
            else:
                streams = M <= 64 or (M <= 128 and nrb8 + nrb4 <= cus)
            if streams:
                want = stream_kmax * min(M, 64) * P * 4 if stream_kmax > 1 else 0
            elif M > 64:
                km = tile_kmax(M, ga)
                want = km * M * P * 4 if km > 1 else 0
            else:
                want = 0
            assert gbb.gemm_w48a8_workspace(N, K, n8, M, ga) == want, (M, ga)
    assert gbb.gemm_w48a8_workspace(N, K, n8, 0, K) == 0


def test_w48_split_argument_errors():
    """gbb_gemm_w48a8_split rejects bad arguments before touching the device
    (the pointers are never dereferenced: every call fails a check first)."""
    L = gbb.lib()
    A = 4096   # a 16-byte aligned fake device address
    N, K, n8 = 64, 256, 8
    assert L.gbb_gemm_w48a8_split(None, N, K, n8, A, A, K, A, 4, A, 256, None) == -1      # no image
    assert L.gbb_gemm_w48a8_split(A, N, 200, n8, A, A, 200, A, 4, A, 256, None) == -2     # K % 128
    assert L.gbb_gemm_w48a8_split(A, N, K, N + 1, A, A, K, A, 4, A, 256, None) == -2      # n8 > N
    assert L.gbb_gemm_w48a8_split(A, N, K, n8, A, A, K, A, -1, A, 256, None) == -1        # M < 0
    assert L.gbb_gemm_w48a8_split(A, N, K, n8, A, A, K, A, 0, A, 256, None) == 0          # M == 0: nothing
    assert L.gbb_gemm_w48a8_split(A, N, K, n8, None, A, K, A, 4, A, 256, None) == -1      # no xq
    assert L.gbb_gemm_w48a8_split(A, N, K, n8, A, A, 64, A, 4, A, 256, None) == -1        # ga neither K nor 128
    assert L.gbb_gemm_w48a8_split(A, N, K, n8, A + 2, A, K, A, 4, A, 256, None) == -4     # xq misaligned
    assert L.gbb_gemm_w48a8_split(A, N, K, n8, A, A, K, A, 4, A + 4, 256, None) == -4     # workspace misaligned
    assert L.gbb_gemm_w48a8_workspace(N, K, n8, 4, 64) == 0                               # invalid ga: 0
    assert L.gbb_gemm_w48a8_workspace(N, 200, n8, 4, 200) == 0                            # invalid K: 0
