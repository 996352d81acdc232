"""GPU parity: the HIP path through the C ABI against the oracle.

Bars: codes and int32 group products bit-exact; dequantized weights bit-exact
against the oracle's fp32 (q - z) * s; one-hot activations give fp16(w')
exactly on every path; fp16 outputs within ||y - y_ref||_inf / ||y_ref||_inf
<= 2e-3 of the fp64 oracle.  Full-size workloads are checked on sampled output
rows in the same launch configuration the benchmark uses.
"""
import functools

import numpy as np
import pytest

import synth
from oracle import alloc
from oracle import blockquant as bq
from oracle import w48 as ow48

torch = pytest.importorskip("torch")
gbb = pytest.importorskip("gemm_block_bit_amd")

pytestmark = pytest.mark.gpu
TOL = 2e-3
ALLOWED = (1, 2, 3, 4, 6, 8)


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def to_dev(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if t.dtype == torch.uint16:
        t = t.view(torch.float16)
    return t.to(dev())


def small(N, K, seed):
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((N, K))).astype(np.float16)
    W[g.random((N, K)) < 0.005] *= np.float16(10)
    return W


def rand_x(M, K, seed):
    return np.random.default_rng(1000 + seed).standard_normal((M, K)).astype(np.float16)


def packed(W, bits):
    img, s, z = gbb.pack_blocks(W, bits)
    return to_dev(img)


def rel_err(y_gpu, y_ref):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(y))
    return bq.rel_inf_err(y, y_ref)


# ----------------------------------------------------------------------------
# bit-exact unpack / dequant
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,seed", [(64, 128, 0), (192, 384, 1), (448, 1280, 2)])
def test_unpack_dequant_bit_exact(N, K, seed):
    W = small(N, K, seed)
    bits = synth.random_bitmap(N, K, ALLOWED, seed)
    img = packed(W, bits)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    qg = gbb.unpack_codes(img, N, K).cpu().numpy()
    assert np.array_equal(qg, q)
    w32, w16 = gbb.dequant(img, N, K)
    ref = bq.dequant_fp32(q, s16, z16)
    assert np.array_equal(w32.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(w16.cpu().numpy().view(np.uint16), bq.fp16_rne(ref).view(np.uint16))


def test_unpack_linear_4096_bit_exact():
    W, bits, _ = synth.linear_4096()
    img = packed(W, bits)
    q, s16, z16 = bq.quantize_blocks(W, bits)
    assert np.array_equal(gbb.unpack_codes(img, 4096, 4096).cpu().numpy(), q)
    w32, _ = gbb.dequant(img, 4096, 4096)
    assert np.array_equal(w32.cpu().numpy().view(np.uint32), bq.dequant_fp32(q, s16, z16).view(np.uint32))


# ----------------------------------------------------------------------------
# one-hot activations: exact on every path
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("path,M", [(1, 1), (1, 16), (1, 32), (2, 1), (2, 200)])
def test_one_hot_rows_exact(path, M):
    N, K = 192, 1280
    W = small(N, K, 3)
    bits = synth.random_bitmap(N, K, ALLOWED, 3)
    img = packed(W, bits)
    ks = np.random.default_rng(M).choice(K, size=M, replace=M > K)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1
    y = gbb.gemm_mixed_w_path(img, N, K, to_dev(x), path).cpu().numpy()
    q, s16, z16 = bq.quantize_blocks(W, bits)
    w16 = bq.dequant_fp16(q, s16, z16)
    assert np.array_equal(y.view(np.uint16), w16[:, ks].T.view(np.uint16))


# ----------------------------------------------------------------------------
# random activations: 2e-3 of the fp64 oracle
# ----------------------------------------------------------------------------
DECODE_CASES = [(64, 128, 1), (128, 256, 3), (192, 384, 5), (1024, 4096, 1), (1024, 4096, 8),
                (320, 2560, 16), (960, 1408, 17), (512, 4096, 32), (64, 28672, 2)]


@pytest.mark.parametrize("N,K,M", DECODE_CASES)
def test_decode_parity(N, K, M):
    W = small(N, K, N + K)
    bits = synth.random_bitmap(N, K, ALLOWED, N + M)
    x = rand_x(M, K, M)
    img = packed(W, bits)
    ref = bq.reference_gemm(x, W, bits)
    xd = to_dev(x)
    for _ in range(3):                      # split-K counters must reset between calls
        y = gbb.gemm_mixed_w_path(img, N, K, xd, 1)
        assert rel_err(y, ref) <= TOL


# the last two have 384 tiles of 128 tokens x 512 rows: 48 per XCD, so each
# XCD's last 16 tiles run as 64-token halves (with M = 1436 some second halves
# start past the last token)
PREFILL_CASES = [(64, 128, 33), (192, 384, 100), (128, 1280, 257), (320, 512, 129), (256, 4096, 600),
                 (16384, 256, 1536), (16384, 256, 1436)]


@pytest.mark.parametrize("b", [1, 8])
@pytest.mark.parametrize("M", [2, 5, 8, 12, 16, 17, 32])
def test_uniform_extreme_bitwidths(b, M):
    """Every block at 8 bits fills a ring with one block's records; every
    block at 1 bit puts the most records in it.  An odd block-row count and
    a matrix of 2^26 weights (two rows per workgroup for M > 16) cover every
    decode kernel's ring."""
    for N, K in [(64 * 9, 128 * 12), (8192, 8192)]:
        W = small(N, K, N + b + M)
        bits = np.full((N // 64, K // 128), b, np.uint8)
        img = packed(W, bits)
        x = rand_x(M, K, b + M)
        rows = np.unique(np.concatenate([np.arange(0, N, 97), [N - 1]]))
        y = gbb.gemm_mixed_w(img, N, K, to_dev(x)).cpu().numpy()
        ref = bq.reference_rows(x, W, bits, rows)
        assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL, (N, K)


@pytest.mark.parametrize("N,K,M", PREFILL_CASES)
def test_prefill_parity(N, K, M):
    W = small(N, K, N * 7 + K)
    bits = synth.random_bitmap(N, K, ALLOWED, N + 2 * M)
    x = rand_x(M, K, M)
    img = packed(W, bits)
    y = gbb.gemm_mixed_w_path(img, N, K, to_dev(x), 2)
    assert rel_err(y, bq.reference_gemm(x, W, bits)) <= TOL


def test_workspace_reuse_across_shapes():
    """One zero-filled workspace serves split-K calls of different shapes: a
    call with few row groups followed by one with more than 64 of them."""
    ws = torch.zeros(gbb.gemm_mixed_w_workspace(16640, 1024, 8) + (1 << 20), dtype=torch.uint8, device=dev())
    for N, K, M in ((256, 4096, 8), (16640, 1024, 1), (256, 4096, 8), (16640, 1024, 8)):
        W = small(N, K, N)
        bits = synth.random_bitmap(N, K, ALLOWED, K)
        x = rand_x(M, K, N + M)
        y = gbb.gemm_mixed_w_path(packed(W, bits), N, K, to_dev(x), 1, workspace=ws)
        assert rel_err(y, bq.reference_gemm(x, W, bits)) <= TOL


@pytest.mark.parametrize("M", [1, 8, 32])
def test_split_k_deterministic_over_many_calls(M):
    """Split-K partial sums cross workgroups (and XCDs) through device-scope
    memory; the reduction order is fixed, so 200 back-to-back calls must give
    bit-identical outputs."""
    N, K = 2048, 8192
    W = small(N, K, 77)
    bits = synth.random_bitmap(N, K, ALLOWED, 77)
    img = packed(W, bits)
    x = to_dev(rand_x(M, K, 77))
    assert gbb.gemm_mixed_w_workspace(N, K, M) > 0
    outs = [gbb.gemm_mixed_w_path(img, N, K, x, 1) for _ in range(200)]
    first = outs[0].cpu()
    for o in outs[1:]:
        assert torch.equal(o.cpu().view(torch.int16), first.view(torch.int16))
    rows = sample_rows(N, 3, 32)
    assert bq.rel_inf_err(first.float().numpy()[:, rows], bq.reference_rows(rand_x(M, K, 77), W, bits, rows)) <= TOL


@pytest.mark.parametrize("M", [1, 8])
def test_split_k_large_partials(M):
    """Segment partial sums beyond the fixed-point range of the split-K
    hand-off (|partial| >= 2^18) take the fp32 overflow accumulator: two block
    columns at opposite ends of K carry identical weights against activations
    of +-30000, so their huge partials cancel in y."""
    N, K = 1024, 4096
    g = np.random.default_rng(91)
    W = g.standard_normal((N, K)).astype(np.float16)
    W[:, K - 128:] = W[:, :128]
    bits = synth.random_bitmap(N, K, ALLOWED, 91)
    bits[:, 0] = bits[:, -1] = 8
    x = (100.0 * g.standard_normal((M, K))).astype(np.float16)
    x[:, :128] = 30000.0
    x[:, K - 128:] = -30000.0
    assert gbb.gemm_mixed_w_workspace(N, K, M) > 0
    ws = torch.zeros(gbb.gemm_mixed_w_workspace(N, K, M), dtype=torch.uint8, device=dev())
    img = packed(W, bits)
    ref = bq.reference_gemm(x, W, bits)
    for _ in range(3):   # the accumulators are clean again after each call
        y = gbb.gemm_mixed_w_path(img, N, K, to_dev(x), 1, workspace=ws)
        assert rel_err(y, ref) <= TOL
    assert not torch.any(ws)


@pytest.mark.parametrize("M", [17, 32])
def test_two_row_workgroups(M):
    """At M > 16 a matrix of at least 2^26 weights runs two block rows per
    workgroup; 129 block rows leave the last workgroup a single one.  The
    K segments' partials include huge cancelling ones (fp32 overflow
    accumulator) and outputs must repeat bit for bit over calls on one
    workspace, which is clean after each."""
    N, K = 129 * 64, 8192
    g = np.random.default_rng(94)
    W = g.standard_normal((N, K)).astype(np.float16)
    W[:, K - 128:] = W[:, :128]
    bits = synth.random_bitmap(N, K, ALLOWED, 94)
    bits[:, 0] = bits[:, -1] = 8
    x = g.standard_normal((M, K)).astype(np.float16)
    x[0, :128] = 30000.0
    x[0, K - 128:] = -30000.0
    ws = torch.zeros(gbb.gemm_mixed_w_workspace(N, K, M), dtype=torch.uint8, device=dev())
    assert ws.numel() > 0
    img = packed(W, bits)
    ref = bq.reference_gemm(x, W, bits)
    first = None
    for _ in range(3):
        y = gbb.gemm_mixed_w_path(img, N, K, to_dev(x), 1, workspace=ws)
        assert rel_err(y, ref) <= TOL
        assert not torch.any(ws)
        if first is None:
            first = y.cpu()
        else:
            assert torch.equal(y.cpu().view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("M", [1, 8])
def test_split_k_nan_then_clean(M):
    """A NaN activation reaches every output through the overflow
    accumulator; the next call on the same workspace is unaffected."""
    N, K = 1024, 4096
    W = small(N, K, 92)
    bits = synth.random_bitmap(N, K, ALLOWED, 92)
    img = packed(W, bits)
    ws = torch.zeros(gbb.gemm_mixed_w_workspace(N, K, M), dtype=torch.uint8, device=dev())
    xn = rand_x(M, K, 92)
    xn[:, 5] = np.nan
    y = gbb.gemm_mixed_w_path(img, N, K, to_dev(xn), 1, workspace=ws)
    assert torch.isnan(y.float()).all()
    x = rand_x(M, K, 93)
    y = gbb.gemm_mixed_w_path(img, N, K, to_dev(x), 1, workspace=ws)
    assert rel_err(y, bq.reference_gemm(x, W, bits)) <= TOL
    assert not torch.any(ws)


def test_graph_replay_matches_eager():
    """The decode launches (M = 1, 8, and 64 as two 32-token chunks) and a
    prefill launch (M = 1024) captured in a HIP graph: every replay, with
    eager work in between, reproduces the eager result bit for bit."""
    N, K = 1024, 4096
    W = small(N, K, 88)
    bits = synth.random_bitmap(N, K, ALLOWED, 88)
    img = packed(W, bits)
    Ms = (1, 8, 64, 1024)
    xs = [to_dev(rand_x(M, K, 88 + M)) for M in Ms]
    eager = [gbb.gemm_mixed_w(img, N, K, x) for x in xs]
    torch.cuda.synchronize()
    outs = [torch.empty_like(e) for e in eager]
    need = max(gbb.gemm_mixed_w_workspace(N, K, M) for M in Ms)
    ws = torch.zeros(need + 256, dtype=torch.uint8, device=dev())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for x, o in zip(xs, outs):
            gbb.gemm_mixed_w(img, N, K, x, out=o, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x, o in zip(xs, outs):
            gbb.gemm_mixed_w(img, N, K, x, out=o, workspace=ws)
    for rep in range(5):
        for o in outs:
            o.fill_(0)
        junk = gbb.gemm_mixed_w(img, N, K, xs[1])      # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), rep
        del junk


@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_library_graph_matches_eager(M):
    """Four calls captured into one library graph (a layer's launch groups in
    miniature, with split-K decode and, at M = 64, the prefill kernel)
    replayed several times, with eager work and synchronizations between the
    replays: every replay equals the eager calls bit for bit."""
    shapes = [(384, 1024), (256, 1024), (1792, 1024), (256, 3584)]
    calls, eager = [], []
    for i, (N, K) in enumerate(shapes):
        W = small(N, K, 40 + i)
        bits = synth.random_bitmap(N, K, ALLOWED, 40 + i)
        img = packed(W, bits)
        x = to_dev(rand_x(M, K, 50 + i))
        y = torch.empty((M, N), dtype=torch.float16, device=dev())
        calls.append((img, N, K, x, y))
        eager.append(gbb.gemm_mixed_w(img, N, K, x).clone())
    g = gbb.Graph(calls)
    try:
        for rep in range(3):
            for (_, _, _, _, y) in calls:
                y.fill_(float("nan"))
            g.launch()
            torch.cuda.synchronize()
            for (_, _, _, _, y), ref in zip(calls, eager):
                assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep
            # eager work between replays, on other buffers
            gbb.gemm_mixed_w(calls[0][0], calls[0][1], calls[0][2], calls[0][3])
            torch.cuda.synchronize()
    finally:
        g.close()
    # a call the library rejects (K not a multiple of 128) fails the capture
    with pytest.raises(gbb.GbbError):
        gbb.Graph([(calls[0][0], 384, 1000, torch.empty((M, 1000), dtype=torch.float16, device=dev()),
                    calls[0][4])])


@pytest.mark.parametrize("M", [1, 8, 64])
def test_maximum_rows(M):
    """N = 2^20 rows (the largest N the block entry points take) on a single
    block column, through each kernel family; one block row more is an
    error."""
    N, K = 1 << 20, 128
    g = np.random.default_rng(60)
    W = (0.02 * g.standard_normal((N, K), dtype=np.float32)).astype(np.float16)
    bits = synth.random_bitmap(N, K, ALLOWED, 60)
    img = packed(W, bits)
    x = rand_x(M, K, 61)
    y = gbb.gemm_mixed_w(img, N, K, to_dev(x)).cpu().numpy()
    rows = sample_rows(N, 62, 64)
    ref = bq.reference_rows(x, W, bits, rows)
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL
    with pytest.raises(gbb.GbbError):
        gbb.gemm_mixed_w(img, N + 64, K, to_dev(x))


def _random_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        N = 64 * int(g.integers(1, 41))
        K = 128 * int(g.integers(1, 41))
        M = int(g.choice([1, 2, 3, 5, 8, 13, 16, 17, 24, 31, 32, 33, 47, 64, 100, 129, 200]))
        cases.append((N, K, M, int(g.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("N,K,M,seed", _random_cases(40, 2024))
def test_random_shapes(N, K, M, seed):
    """Seeded random shapes (ragged M, odd block-row counts, short and long
    K) and random bitmaps over every width, through whichever kernel the
    library picks, against the oracle on sampled rows."""
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((N, K))).astype(np.float16)
    W[g.random((N, K)) < 0.005] *= np.float16(10)
    bits = synth.random_bitmap(N, K, ALLOWED, seed % 1000)
    img = packed(W, bits)
    x = g.standard_normal((M, K)).astype(np.float16)
    y = gbb.gemm_mixed_w(img, N, K, to_dev(x)).cpu().numpy()
    rows = np.unique(np.concatenate([[0, N - 1], g.choice(N, min(N, 48), replace=False)]))
    ref = bq.reference_rows(x, W, bits, rows)
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL


@pytest.mark.parametrize("M", [33, 64, 100])
def test_batches_as_decode_chunks(M):
    """Batches just above 32 tokens on a matrix whose prefill grid would
    leave most CUs idle run as 32-token decode chunks: a workspace is then
    required (and checked), and the result matches the oracle."""
    N, K = 4096, 4096
    W = small(N, K, 90 + M)
    bits = synth.random_bitmap(N, K, ALLOWED, 90 + M)
    img = packed(W, bits)
    need = gbb.gemm_mixed_w_workspace(N, K, M)
    assert need > 0
    x = rand_x(M, K, 91 + M)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    y = gbb.gemm_mixed_w(img, N, K, to_dev(x), workspace=ws)
    rows = sample_rows(N, 92 + M)
    ref = bq.reference_rows(x, W, bits, rows)
    assert bq.rel_inf_err(y.cpu().numpy()[:, rows].astype(np.float64), ref) <= TOL
    assert torch.count_nonzero(ws) == 0
    small_ws = torch.zeros(need - 16, dtype=torch.uint8, device=dev())
    with pytest.raises(gbb.GbbError):
        gbb.gemm_mixed_w(img, N, K, to_dev(x), workspace=small_ws)


def test_auto_path_and_empty_batch():
    N, K = 128, 256
    W = small(N, K, 5)
    bits = synth.random_bitmap(N, K, ALLOWED, 5)
    img = packed(W, bits)
    for M in (1, 32, 33):
        x = rand_x(M, K, M)
        y = gbb.gemm_mixed_w(img, N, K, to_dev(x))
        assert rel_err(y, bq.reference_gemm(x, W, bits)) <= TOL
    y0 = gbb.gemm_mixed_w(img, N, K, torch.empty((0, K), dtype=torch.float16, device=dev()))
    assert y0.shape == (0, N)


def test_device_argument_errors():
    N, K = 128, 256
    W = small(N, K, 6)
    img = packed(W, synth.uniform_bitmap(N, K, 4))
    x = torch.zeros((3, K + 8), dtype=torch.float16, device=dev())
    L = gbb.lib()
    y = torch.empty((3, N), dtype=torch.float16, device=dev())
    # x shifted by one element is not 16-byte aligned
    assert L.gbb_gemm_mixed_w(img.data_ptr(), N, K, x.data_ptr() + 2, y.data_ptr(), 3, None, 0, None) == -4
    assert L.gbb_gemm_mixed_w(img.data_ptr(), N, 200, x.data_ptr(), y.data_ptr(), 3, None, 0, None) == -2
    need = gbb.gemm_mixed_w_workspace(1024, 4096, 1)
    assert need > 0
    img2 = packed(small(1024, 4096, 1), synth.uniform_bitmap(1024, 4096, 2))
    x1 = torch.zeros((1, 4096), dtype=torch.float16, device=dev())
    y1 = torch.empty((1, 1024), dtype=torch.float16, device=dev())
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    assert L.gbb_gemm_mixed_w(img2.data_ptr(), 1024, 4096, x1.data_ptr(), y1.data_ptr(), 1, ws.data_ptr(),
                              need - 16, None) == -5
    assert L.gbb_gemm_mixed_w(img2.data_ptr(), 1024, 4096, x1.data_ptr(), y1.data_ptr(), 1, None, 0, None) == -1
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# full-size workloads, sampled rows
# ----------------------------------------------------------------------------
@functools.lru_cache(maxsize=4)
def workload(name, i):
    if name == "8b":
        p, W, bits = synth.llama3_8b_proj(i)
    elif name == "70b":
        p, W, bits = synth.llama3_70b_proj(i)
    else:
        p, W, bits = synth.prefill_70b_mlp(i)
    img, _, _ = gbb.pack_blocks(W, bits)
    return p, W, bits, to_dev(img)


def sample_rows(N, seed, n=48):
    g = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 63, 64, N - 1], g.choice(N, n, replace=False)]))


@pytest.mark.parametrize("i", range(7))
def test_llama3_8b_layer_decode(i):
    p, W, bits, img = workload("8b", i)
    assert abs(synth.mean_bits(bits) - 3.1) < 0.01
    for M in (1, 8):
        x = synth.activations(M, p.K, synth.WL_LLAMA3_8B, i)
        y = gbb.gemm_mixed_w(img, p.N, p.K, to_dev(x)).cpu().numpy()
        rows = sample_rows(p.N, i)
        ref = bq.reference_rows(x, W, bits, rows)
        assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL


@pytest.mark.parametrize("i", [1, 4, 6])
def test_llama3_70b_layer_decode(i):
    p, W, bits, img = workload("70b", i)
    assert abs(synth.mean_bits(bits) - 2.1) < 0.01
    for M in (1, 8, 32):
        x = synth.activations(M, p.K, synth.WL_LLAMA3_70B, i)
        y = gbb.gemm_mixed_w(img, p.N, p.K, to_dev(x)).cpu().numpy()
        rows = sample_rows(p.N, 10 + i, 24)
        ref = bq.reference_rows(x, W, bits, rows)
        assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL


@pytest.mark.parametrize("i", [0, 1])
def test_prefill_70b_mlp_m2048(i):
    p, W, bits, img = workload("prefill", i)
    x = synth.prefill_x(2048, p.K, i)
    y = gbb.gemm_mixed_w(img, p.N, p.K, to_dev(x)).cpu().numpy()
    rows = sample_rows(p.N, 20 + i, 12)
    ref = bq.reference_rows(x, W, bits, rows)
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL


def test_reordered_allocated_layer():
    """Offline chain: channel order, bit allocation on the reordered weight,
    packing, then the kernels on the permuted activations; the outputs,
    scattered back by the row order, approximate W x."""
    N, K = 1024, 2048
    W = synth.weight_heavy_rows(N, K, synth.WL_LLAMA3_8B, 1)
    r, c = gbb.channel_order(W)
    Wr = np.ascontiguousarray(W[r][:, c])
    bits = gbb.allocate_bits(Wr, 3.0)
    assert np.array_equal(bits, alloc.allocate(Wr, 3.0))
    assert synth.mean_bits(bits) <= 3.0 and np.unique(bits).size > 1
    img = packed(Wr, bits)
    for M in (1, 8, 64):
        x = rand_x(M, K, 77 + M)
        xr = np.ascontiguousarray(x[:, c])
        y = gbb.gemm_mixed_w(img, N, K, to_dev(xr)).cpu().numpy().astype(np.float64)
        ref = bq.reference_rows(xr, Wr, bits, np.arange(N))
        assert bq.rel_inf_err(y, ref) <= TOL
        full = np.empty_like(y)
        full[:, r] = y
        exact = x.astype(np.float64) @ W.astype(np.float64).T
        assert bq.rel_inf_err(full, exact) <= 0.25


# ----------------------------------------------------------------------------
# W4/W8 x A8
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,ga", [(1, 256, None), (5, 384, None), (7, 512, 128), (64, 8192, None), (33, 4096, 128)])
def test_act_quant_bit_exact(M, K, ga):
    x = rand_x(M, K, M + K)
    x[0, :128] = 0
    if M > 2:
        x[2] = 0
    xq, xs = gbb.quant_act_i8(to_dev(x), ga)
    A, s = ow48.quant_act(x, ga)
    assert np.array_equal(xq.cpu().numpy(), A)
    assert np.array_equal(xs.cpu().numpy().view(np.uint16), s.view(np.uint16))


@pytest.mark.parametrize("N,K,M,frac", [(48, 256, 3, 0.1), (200, 384, 40, 0.1), (64, 128, 17, 0.0),
                                        (40, 256, 70, 1.0), (300, 1024, 130, 0.2)])
def test_w48_group_acc_bit_exact(N, K, M, frac):
    W = small(N, K, N + M)
    rows8 = synth.salient_rows_by_l2(W, frac) if frac < 1 else np.arange(N, dtype=np.int32)
    img, _, _ = gbb.pack_w48(W, rows8)
    x = rand_x(M, K, N)
    xq, _ = gbb.quant_act_i8(to_dev(x))
    acc = gbb.w48_group_acc(to_dev(img), N, K, rows8.size, xq).cpu().numpy()
    qd = ow48.quantize_w48(W, rows8)
    A, _ = ow48.quant_act(x)
    ref = np.zeros((M, N, K // 128), np.int64)
    if qd["rows8"].size:
        ref[:, qd["rows8"]] = ow48.group_acc(A, qd["q8"].astype(np.int64))
    if qd["rows4"].size:
        Wz = qd["q4"].astype(np.int64) - np.repeat(qd["z4"].astype(np.int64), 128, axis=1)
        ref[:, qd["rows4"]] = ow48.group_acc(A, Wz)
    assert np.array_equal(acc.astype(np.int64), ref)


@pytest.mark.parametrize("N,K,M,ga,frac", [(48, 256, 3, None, 0.1), (200, 384, 40, None, 0.1),
                                           (300, 1024, 130, None, 0.1), (300, 1024, 77, 128, 0.1),
                                           (1000, 4096, 1, None, 0.1), (256, 1024, 64, None, 0.1),
                                           (128, 640, 17, None, 0.3),
                                           # MixLLM's 20 % and 50 % 8-bit row fractions
                                           (320, 1024, 48, None, 0.2), (192, 512, 130, 128, 0.5), (192, 512, 24, None, 0.5),
                                           # batches above 64 with no 8-bit rows / only 8-bit rows
                                           (64, 256, 100, None, 0.0), (80, 256, 200, 128, 1.0)])
def test_w48_parity(N, K, M, ga, frac):
    W = small(N, K, 3 * N + M)
    rows8 = synth.salient_rows_by_l2(W, frac)
    img, _, _ = gbb.pack_w48(W, rows8)
    x = rand_x(M, K, 2 * N)
    xq, xs = gbb.quant_act_i8(to_dev(x), ga)
    y = gbb.gemm_w48a8(to_dev(img), N, K, rows8.size, xq, xs, ga)
    ref = ow48.reference(x, W, rows8, act_group=ga)
    assert rel_err(y, ref) <= TOL


@functools.lru_cache(maxsize=1)
def w44a8_image():
    W, rows8 = synth.w44a8_28672x8192()
    img, _, _ = gbb.pack_w48(W, rows8)
    return W, rows8, to_dev(img)


def _random_w48_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        N = int(g.integers(1, 400))
        K = 128 * int(g.integers(1, 24))
        M = int(g.choice([1, 2, 7, 16, 17, 31, 32, 33, 64, 65, 130, 257]))
        frac = float(g.choice([0.0, 0.05, 0.1, 0.2, 0.5, 1.0]))
        ga = None if g.random() < 0.6 else 128
        cases.append((N, K, M, frac, ga, int(g.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("N,K,M,frac,ga,seed", _random_w48_cases(20, 77))
def test_w48_random_shapes(N, K, M, frac, ga, seed):
    """Seeded random W4.4A8 shapes (any N, ragged M, every kernel), 8-bit row
    fractions from 0 to 1 and both activation-scale granularities."""
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((N, K))).astype(np.float16)
    rows8 = synth.salient_rows_by_l2(W, frac) if frac < 1 else np.arange(N, dtype=np.int32)
    img, _, _ = gbb.pack_w48(W, rows8)
    x = g.standard_normal((M, K)).astype(np.float16)
    xq, xs = gbb.quant_act_i8(to_dev(x), ga)
    y = gbb.gemm_w48a8(to_dev(img), N, K, rows8.size, xq, xs, ga)
    ref = ow48.reference(x, W, rows8, act_group=ga)
    assert rel_err(y, ref) <= TOL


@pytest.mark.parametrize("M", [32, 96, 512, 4096])
def test_w44a8_28672x8192(M):
    W, rows8, img = w44a8_image()
    assert rows8.size == 2867
    x = synth.activations(M, 8192, synth.WL_W44A8, 0)
    xq, xs = gbb.quant_act_i8(to_dev(x))
    y = gbb.gemm_w48a8(img, 28672, 8192, rows8.size, xq, xs).cpu().numpy()
    rows = np.unique(np.concatenate([rows8[:8], sample_rows(28672, M, 16)]))
    qd = ow48.quantize_w48(W[rows], np.nonzero(np.isin(rows, rows8))[0])
    ref = ow48.reference(x, W[rows], np.nonzero(np.isin(rows, rows8))[0], quant=qd)
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL
