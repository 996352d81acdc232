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


@pytest.mark.parametrize("N,K", [(8192, 28672), (28672, 8192), (4096, 4096), (64, 128)])
def test_workspace_follows_the_batch_route(N, K):
    """Host side of the dispatch: above 32 tokens a workspace is asked for
    exactly when the batch runs as 32-token decode chunks, that is when
    ceil(M/32) prefill grids of 128x512 tiles fit in one wave of the CUs
    (256 when the library finds no device), and it is then the larger of the
    full and the ragged last chunk's needs."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count if torch.cuda.is_available() else 256
    for M in (33, 64, 65, 96, 128, 200, 256, 512, 1024, 2048):
        tiles = -(-M // 128) * -(-N // 512)
        chunked = -(-M // 32) * tiles <= cus
        need = gbb.gemm_mixed_w_workspace(N, K, M)
        if not chunked:
            assert need == 0, (M, need)
            continue
        want = gbb.gemm_mixed_w_workspace(N, K, 32)
        if M % 32:
            want = max(want, gbb.gemm_mixed_w_workspace(N, K, M % 32))
        assert need == want, (M, need, want)
