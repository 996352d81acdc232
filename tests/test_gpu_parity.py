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
# Large batches: one block column, 67 of them (the 64-column metadata window
# reloads), a last row tile with one block row, and ragged token counts.
PREFILL_CASES = [(64, 128, 33), (192, 384, 100), (128, 1280, 257), (320, 512, 129), (256, 4096, 600),
                 (16384, 256, 1536), (16384, 256, 1436), (576, 128, 1024), (576, 128 * 67, 1030),
                 (320, 384, 2065)]


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


# the last case has 16 segments of 65 block columns: each crosses a
# 64-column window of bitwidths and offsets
@pytest.mark.parametrize("N,K,M,bc", [(1024, 8192, 300, 128), (512, 128 * 70, 1100, 128), (1024, 8192, 200, 64),
                                      (64, 128 * 1040, 40, 128)])
def test_prefill_split_k(N, K, M, bc):
    """The prefill kernel with its K split (a tile grid that fills at most half
    of the CUs, the workspace the path-aware query asks for): three calls
    on one workspace are bit-identical (the partials are added in segment
    order, whatever finishes last), within 2e-3 of the oracle, and leave
    the workspace zero.  With half that workspace the call takes fewer
    segments, with none it runs unsplit; both stay within 2e-3."""
    lib = gbb.lib()
    need = (lib.gbb_gemm_mixed_w_path_workspace if bc == 128 else lib.gbb_gemm_mixed_w_64x64_path_workspace)(N, K, M, 2)
    assert need > 0   # the split is taken
    W = small(N, K, N + K + bc)
    x = rand_x(M, K, M + bc)
    if bc == 128:
        bits = synth.random_bitmap(N, K, ALLOWED, M)
        img, call = packed(W, bits), gbb.gemm_mixed_w_path
    else:
        bits = synth.random_bitmap64(N, K, ALLOWED, M)
        img, call = packed64(W, bits), gbb.gemm_mixed_w_64x64_path
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    first = None
    for _ in range(3):
        y = call(img, N, K, to_dev(x), 2, workspace=ws)
        torch.cuda.synchronize()
        assert not torch.any(ws)
        first = y.clone() if first is None else first
        assert torch.equal(y.view(torch.int16), first.view(torch.int16))
    ref = bq.reference_gemm(x, W, bits, block_cols=bc)
    assert rel_err(first, ref) <= TOL
    half = torch.zeros(need // 2 + 16, dtype=torch.uint8, device=dev())
    yh = call(img, N, K, to_dev(x), 2, workspace=half)
    y0 = call(img, N, K, to_dev(x), 2, workspace=torch.zeros(256, dtype=torch.uint8, device=dev()))
    torch.cuda.synchronize()
    assert not torch.any(half)
    assert rel_err(yh, ref) <= TOL
    assert rel_err(y0, ref) <= TOL


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
    replays: every replay equals the eager calls bit for bit and the oracle
    within 2e-3."""
    shapes = [(384, 1024), (256, 1024), (1792, 1024), (256, 3584)]
    calls, eager, refs = [], [], []
    for i, (N, K) in enumerate(shapes):
        W = small(N, K, 40 + i)
        bits = synth.random_bitmap(N, K, ALLOWED, 40 + i)
        img = packed(W, bits)
        xh = rand_x(M, K, 50 + i)
        x = to_dev(xh)
        y = torch.empty((M, N), dtype=torch.float16, device=dev())
        calls.append((img, N, K, x, y))
        eager.append(gbb.gemm_mixed_w(img, N, K, x).clone())
        refs.append(bq.reference_gemm(xh, W, bits))
    g = gbb.Graph(calls)
    try:
        for rep in range(3):
            for (_, _, _, _, y) in calls:
                y.fill_(float("nan"))
            g.launch()
            torch.cuda.synchronize()
            for (_, _, _, _, y), ref, oref in zip(calls, eager, refs):
                assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), rep
                assert rel_err(y, oref) <= TOL, rep
            # eager work between replays, on other buffers
            gbb.gemm_mixed_w(calls[0][0], calls[0][1], calls[0][2], calls[0][3])
            torch.cuda.synchronize()
    finally:
        g.close()
    # a call the library rejects (K not a multiple of 128) fails the capture
    with pytest.raises(gbb.GbbError):
        gbb.Graph([(calls[0][0], 384, 1000, torch.empty((M, 1000), dtype=torch.float16, device=dev()),
                    calls[0][4])])


@pytest.mark.parametrize("M", [1, 5, 16, 24])
def test_batched_independent_products(M):
    """Six independent products of different shapes (some with split K) as
    one grouped call -- one launch for M <= 16 -- twice on one workspace:
    each output equals its own gbb_gemm_mixed_w call bit for bit and the
    oracle within 2e-3, and the workspace is clean afterwards."""
    shapes = [(64, 128), (384, 1024), (1024, 4096), (256, 3584), (4096, 1024), (192, 8192)]
    calls, refs, singles = [], [], []
    for i, (N, K) in enumerate(shapes):
        W = small(N, K, 70 + i)
        bits = synth.random_bitmap(N, K, ALLOWED, 70 + i)
        img = packed(W, bits)
        xh = rand_x(M, K, 80 + i)
        x = to_dev(xh)
        y = torch.full((M, N), float("nan"), dtype=torch.float16, device=dev())
        calls.append((img, N, K, x, y))
        refs.append(bq.reference_gemm(xh, W, bits))
        singles.append(gbb.gemm_mixed_w(img, N, K, x).clone())
    b = gbb.Batched(calls)
    assert b._ws.numel() >= gbb.gemm_mixed_w_batched_workspace([(N, K) for N, K in shapes], M)
    for rep in range(2):
        for c in calls:
            c[4].fill_(float("nan"))
        b.launch()
        torch.cuda.synchronize()
        for (_, N, K, _, y), ref, one in zip(calls, refs, singles):
            assert torch.equal(y.view(torch.int16), one.view(torch.int16)), (rep, N, K)
            assert rel_err(y, ref) <= TOL, (rep, N, K)
        assert not torch.any(b._ws)


@pytest.mark.parametrize("M", [1, 8])
def test_batched_graph_replays(M):
    """A grouped launch captured in a HIP graph (as bench.py times it) and
    replayed three times with eager work and synchronizations between the
    replays: every replay equals the eager grouped call bit for bit and the
    oracle within 2e-3; the shared workspace is clean after each."""
    shapes = [(384, 1024), (1024, 4096), (256, 3584)]
    calls, refs = [], []
    for i, (N, K) in enumerate(shapes):
        W = small(N, K, 110 + i)
        bits = synth.random_bitmap(N, K, ALLOWED, 110 + i)
        xh = rand_x(M, K, 120 + i)
        y = torch.empty((M, N), dtype=torch.float16, device=dev())
        calls.append((packed(W, bits), N, K, to_dev(xh), y))
        refs.append(bq.reference_gemm(xh, W, bits))
    b = gbb.Batched(calls)
    b.launch()
    torch.cuda.synchronize()
    eager = [c[4].clone() for c in calls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        b.launch()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.launch()
    for rep in range(3):
        for c in calls:
            c[4].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (_, N, K, _, y), e, ref in zip(calls, eager, refs):
            assert torch.equal(y.view(torch.int16), e.view(torch.int16)), (rep, N, K)
            assert rel_err(y, ref) <= TOL, (rep, N, K)
        assert not torch.any(b._ws)
        gbb.gemm_mixed_w(calls[1][0], calls[1][1], calls[1][2], calls[1][3])   # eager work between replays
        torch.cuda.synchronize()
    del g


def test_split_k_graph_replays():
    """The two K-split paths captured in one HIP graph -- the prefill kernel
    with split_reduce_kernel (2048 x 16384, M = 300: 3 token tiles x 4 row
    tiles, 16 segments) and the W4.4A8 stream kernel with w48_reduce_kernel
    (2048 x 16384, M = 32) -- and replayed three times with eager work and
    synchronizations between the replays: every replay equals the eager calls
    bit for bit and the oracle within 2e-3, and the workspaces are zero after
    each."""
    N1, K1, M1 = 2048, 16384, 300
    W1 = small(N1, K1, 131)
    bits1 = synth.random_bitmap(N1, K1, ALLOWED, 131)
    img1 = packed(W1, bits1)
    x1h = rand_x(M1, K1, 132)
    x1 = to_dev(x1h)
    need1 = gbb.gemm_mixed_w_workspace(N1, K1, M1)
    assert need1 == 16 * M1 * N1 * 4
    ws1 = torch.zeros(need1, dtype=torch.uint8, device=dev())
    y1 = torch.empty((M1, N1), dtype=torch.float16, device=dev())
    N2, K2, M2 = 2048, 16384, 32
    W2 = small(N2, K2, 133)
    rows8 = synth.salient_rows_by_l2(W2, 0.1)
    img2 = to_dev(gbb.pack_w48(W2, rows8)[0])
    x2h = rand_x(M2, K2, 134)
    xq, xs = gbb.quant_act_i8(to_dev(x2h))
    need2 = gbb.gemm_w48a8_workspace(N2, K2, rows8.size, M2)
    assert need2 > 0
    ws2 = torch.zeros(need2, dtype=torch.uint8, device=dev())
    y2 = torch.empty((M2, N2), dtype=torch.float16, device=dev())

    def calls():
        gbb.gemm_mixed_w(img1, N1, K1, x1, out=y1, workspace=ws1)
        gbb.gemm_w48a8(img2, N2, K2, rows8.size, xq, xs, out=y2, workspace=ws2)

    calls()
    torch.cuda.synchronize()
    e1, e2 = y1.clone(), y2.clone()
    rows1 = sample_rows(N1, 135)
    ref1 = bq.reference_rows(x1h, W1, bits1, rows1)
    assert bq.rel_inf_err(e1.cpu().numpy()[:, rows1].astype(np.float64), ref1) <= TOL
    rows2 = one_row_per(packed_rows(N2, rows8), 16, 136)
    ref2 = ow48.reference(x2h, W2[rows2], np.nonzero(np.isin(rows2, rows8))[0])
    assert bq.rel_inf_err(e2.cpu().numpy()[:, rows2].astype(np.float64), ref2) <= TOL
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        y1.fill_(float("nan"))
        y2.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1.view(torch.int16), e1.view(torch.int16)), rep
        assert torch.equal(y2.view(torch.int16), e2.view(torch.int16)), rep
        assert not torch.any(ws1) and not torch.any(ws2), rep
        gbb.gemm_mixed_w(img1, N1, K1, x1[:64].contiguous())   # eager work between replays
        torch.cuda.synchronize()
    del g


def test_batched_llama3_8b_layer_m1():
    """The Llama-3-8B layer's four launch groups (q|k|v, o, gate|up, down)
    as one grouped launch at M = 1, one checked row per block row."""
    calls, checks = [], []
    for gname, idx in synth.LAYER_LAUNCH_GROUPS:
        N, K, W, bits = synth.stacked_group(synth.llama3_8b_proj, idx)
        img = packed(W, bits)
        xh = synth.activations(1, K, synth.WL_LLAMA3_8B, 90 + len(calls))
        y = torch.empty((1, N), dtype=torch.float16, device=dev())
        calls.append((img, N, K, to_dev(xh), y))
        rows = one_row_per_block_row(N, N)
        checks.append((rows, bq.reference_rows(xh, W, bits, rows)))
        del W
    gbb.Batched(calls).launch()
    torch.cuda.synchronize()
    for (_, N, K, _, y), (rows, ref) in zip(calls, checks):
        assert bq.rel_inf_err(y.cpu().numpy()[:, rows].astype(np.float64), ref) <= TOL, (N, K)


@pytest.mark.parametrize("M", [1, 8, 17, 32, 64])
def test_maximum_rows(M):
    """N = 2^20 rows (the largest N the block entry points take) on a single
    block column, through each kernel family (at M = 17 and 32 the two-row
    decode kernel with no K split); one block row more is an error."""
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


def _random_route_cases(n, seed):
    g = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        N = 64 * int(g.integers(1, 129))
        K = 128 * int(g.integers(1, 129))
        M = int(g.choice([1, 4, 16, 32, 33, 48, 64, 65, 96, 97, 128, 160, 200, 256, 300, 400]))
        fmt = str(g.choice(["block128", "block64", "w48", "w48ga"]))
        cases.append((fmt, N, K, M, int(g.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("fmt,N,K,M,seed", _random_route_cases(32, 4242))
def test_random_routes(fmt, N, K, M, seed):
    """Seeded random shapes up to 8192 x 16384 and 400 tokens in both
    formats, through whichever route the library picks (decode, 32-token
    chunks, the prefill and tile kernels with or without their K splits,
    stream passes, per-token or per-group activation scales), against the
    oracle on sampled rows."""
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((N, K))).astype(np.float16)
    rows = np.unique(np.concatenate([[0, N - 1], g.choice(N, min(N, 16), replace=False)]))
    x = g.standard_normal((M, K)).astype(np.float16)
    if fmt.startswith("block"):
        bc = 64 if fmt == "block64" else 128
        bits = (synth.random_bitmap64 if bc == 64 else synth.random_bitmap)(N, K, ALLOWED, seed % 1000)
        img = to_dev(gbb.pack_blocks(W, bits, block_cols=bc)[0])
        call = gbb.gemm_mixed_w_64x64 if bc == 64 else gbb.gemm_mixed_w
        y = call(img, N, K, to_dev(x))
        ref = bq.reference_rows(x, W, bits, rows, block_cols=bc)
    else:
        ga = 128 if fmt == "w48ga" else None
        rows8 = synth.salient_rows_by_l2(W, float(g.choice([0.0, 0.1, 0.3])))
        img = to_dev(gbb.pack_w48(W, rows8)[0])
        xq, xs = gbb.quant_act_i8(to_dev(x), ga)
        y = gbb.gemm_w48a8(img, N, K, rows8.size, xq, xs, ga)
        ref = ow48.reference(x, W[rows], np.nonzero(np.isin(rows, rows8))[0], act_group=ga)
    assert bq.rel_inf_err(y.cpu().numpy()[:, rows].astype(np.float64), ref) <= TOL


@pytest.mark.parametrize("M", [33, 64, 96])
def test_batches_as_decode_chunks(M):
    """Batches of up to three 32-token chunks on a matrix whose split
    prefill grid would leave most CUs idle run as 32-token decode chunks: a
    workspace is then required (and checked), and the result matches the
    oracle."""
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


def one_row_per_block_row(N, seed):
    """One row at a random offset inside every 64-row block row, so every
    decode workgroup (and each of its K segments, which all write every row
    of the block row) and every prefill wave is checked."""
    g = np.random.default_rng(seed)
    return np.arange(0, N, 64) + g.integers(0, 64, N // 64)


@pytest.mark.parametrize("i", [0, 1])
def test_prefill_70b_mlp_m2048(i):
    p, W, bits, img = workload("prefill", i)
    x = synth.prefill_x(2048, p.K, i)
    y = gbb.gemm_mixed_w(img, p.N, p.K, to_dev(x)).cpu().numpy()
    rows = one_row_per_block_row(p.N, 20 + i)
    ref = bq.reference_rows(x, W, bits, rows)
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL


@functools.lru_cache(maxsize=1)
def stacked_launch(layer, group):
    """One launch group of a decoder layer, stacked as the benchmark packs it
    (q|k|v and gate|up are one matrix each)."""
    gen = synth.llama3_8b_proj if layer == "8b" else synth.llama3_70b_proj
    idx = dict(synth.LAYER_LAUNCH_GROUPS)[group]
    N, K, W, bits = synth.stacked_group(gen, idx)
    img, _, _ = gbb.pack_blocks(W, bits)
    return N, K, W, bits, to_dev(img)


# the launches and batch sizes the benchmark times: Llama-3-8B at M = 1, 8 and
# Llama-3-70B at M = 1, 8, 32 (70B gate|up at M = 32 is the two-row kernel
# without a K split)
BENCH_LAUNCHES = [("8b", gname, (1, 8)) for gname, _ in synth.LAYER_LAUNCH_GROUPS] + \
                 [("70b", gname, (1, 8, 32)) for gname, _ in synth.LAYER_LAUNCH_GROUPS]


@pytest.mark.parametrize("layer,group,Ms", BENCH_LAUNCHES)
def test_benchmark_launches(layer, group, Ms):
    N, K, W, bits, img = stacked_launch(layer, group)
    rows = one_row_per_block_row(N, N + K)
    wl = synth.WL_LLAMA3_8B if layer == "8b" else synth.WL_LLAMA3_70B
    ws = torch.zeros(max(gbb.gemm_mixed_w_workspace(N, K, M) for M in Ms) + 256, dtype=torch.uint8,
                     device=dev())
    for M in Ms:
        x = synth.activations(M, K, wl, 50 + M)
        y = gbb.gemm_mixed_w(img, N, K, to_dev(x), workspace=ws).cpu().numpy()
        ref = bq.reference_rows(x, W, bits, rows)
        assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL, M
    assert not torch.any(ws)


def test_linear_4096_output():
    """The single 4096 x 4096 layer with bits {2,3,4} on its own x, every
    output against the oracle."""
    W, bits, x = synth.linear_4096()
    img = packed(W, bits)
    y = gbb.gemm_mixed_w(img, 4096, 4096, to_dev(x))
    assert rel_err(y, bq.reference_gemm(x, W, bits)) <= TOL


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


def w48_acc_reference(x, W, rows8, rows=None, ga=None):
    """int64 [M][n][G] exact group sums of the oracle for the original rows
    `rows` (all rows if None), activations quantized per token (ga None) or
    per group of ga columns."""
    N = W.shape[0]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    is8 = np.isin(rows, rows8)
    qd = ow48.quantize_w48(W[rows], np.nonzero(is8)[0])
    A, _ = ow48.quant_act(x, ga)
    ref = np.zeros((x.shape[0], rows.size, W.shape[1] // 128), np.int64)
    if qd["rows8"].size:
        ref[:, qd["rows8"]] = ow48.group_acc(A, qd["q8"].astype(np.int64))
    if qd["rows4"].size:
        Wz = qd["q4"].astype(np.int64) - np.repeat(qd["z4"].astype(np.int64), 128, axis=1)
        ref[:, qd["rows4"]] = ow48.group_acc(A, Wz)
    return ref


# (N, K, M, 8-bit row fraction, ga): the kernel gbb_gemm_w48a8 picks for the
# same M and ga -- stream (M <= 64, per-token scales or group scales over an
# even group count; 1, 2 and 4 token tiles), two 64-token stream passes
# (65-128 tokens with per-token scales on a short tile grid), tile (M > 64,
# both scale granularities), and the register-staged kernel (group scales
# over an odd group count at M <= 64, here K = 384) -- forms the sums, with
# the K split of a call with a full workspace; K = 8192 with N reduced
# stands in for the 28672 x 8192 layer
W48_ACC_CASES = [(48, 256, 3, 0.1, None), (200, 384, 32, 0.1, None), (200, 384, 40, 0.1, None),
                 (64, 128, 17, 0.0, None), (40, 256, 70, 1.0, None), (300, 1024, 96, 0.2, None),
                 (300, 1024, 130, 0.2, None), (300, 1024, 40, 0.2, 128), (300, 1024, 130, 0.2, 128),
                 (200, 512, 77, 0.5, 128), (200, 384, 20, 0.1, 128), (200, 384, 50, 0.1, 128),
                 (2048, 8192, 32, 0.1, None), (2048, 8192, 96, 0.1, None), (2048, 8192, 32, 0.1, 128),
                 (2048, 8192, 512, 0.1, None), (2048, 8192, 512, 0.1, 128)]


@pytest.mark.parametrize("N,K,M,frac,ga", W48_ACC_CASES)
def test_w48_group_acc_bit_exact(N, K, M, frac, ga):
    W = small(N, K, N + M)
    rows8 = synth.salient_rows_by_l2(W, frac) if frac < 1 else np.arange(N, dtype=np.int32)
    img, _, _ = gbb.pack_w48(W, rows8)
    x = rand_x(M, K, N)
    xq, _ = gbb.quant_act_i8(to_dev(x), ga)
    acc = gbb.w48_group_acc(to_dev(img), N, K, rows8.size, xq, ga).cpu().numpy()
    assert np.array_equal(acc.astype(np.int64), w48_acc_reference(x, W, rows8, ga=ga))


@pytest.mark.parametrize("N,K,M,ga,frac", [(48, 256, 3, None, 0.1), (200, 384, 40, None, 0.1),
                                           (300, 1024, 130, None, 0.1), (300, 1024, 77, 128, 0.1),
                                           (1000, 4096, 1, None, 0.1), (256, 1024, 64, None, 0.1),
                                           (128, 640, 17, None, 0.3),
                                           # MixLLM's 20 % and 50 % 8-bit row fractions
                                           (320, 1024, 48, None, 0.2), (192, 512, 130, 128, 0.5), (192, 512, 24, None, 0.5),
                                           # batches above 64 with no 8-bit rows / only 8-bit rows
                                           (64, 256, 100, None, 0.0), (80, 256, 200, 128, 1.0),
                                           # 64-token tiles, ragged: per-group scales over an odd
                                           # group count (read per output), per-token scales
                                           (200, 384, 100, 128, 0.1), (200, 384, 300, None, 0.1)])
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


def packed_rows(N, rows8):
    """Original rows in the packed order of the W4/W8 image: the 8-bit rows,
    then the 4-bit rows, each ascending and padded with -1 to 16-row tiles."""
    r8 = np.asarray(rows8, np.int64)
    r4 = np.setdiff1d(np.arange(N), r8)
    pad = lambda r: np.concatenate([r, -np.ones((-r.size) % 16, np.int64)])
    return np.concatenate([pad(r8), pad(r4)])


def one_row_per(packed, stride, seed):
    """One original row from every `stride` consecutive packed rows."""
    g = np.random.default_rng(seed)
    out = []
    for c0 in range(0, packed.size, stride):
        chunk = packed[c0:c0 + stride]
        chunk = chunk[chunk >= 0]
        if chunk.size:
            out.append(int(g.choice(chunk)))
    return np.unique(out)


@pytest.mark.parametrize("M", [32, 96, 512, 4096])
def test_w44a8_28672x8192(M):
    """The 28672 x 8192 layer in the launches the benchmark times: one
    checked row in every 16-row tile (a stream-kernel wave) at M <= 128, in
    every 128-row block of tiles (a tile-kernel workgroup) above."""
    W, rows8, img = w44a8_image()
    assert rows8.size == 2867
    x = synth.activations(M, 8192, synth.WL_W44A8, 0)
    xq, xs = gbb.quant_act_i8(to_dev(x))
    y = gbb.gemm_w48a8(img, 28672, 8192, rows8.size, xq, xs).cpu().numpy()
    rows = one_row_per(packed_rows(28672, rows8), 16 if M <= 128 else 128, M)
    ref = ow48.reference(x, W[rows], np.nonzero(np.isin(rows, rows8))[0])
    err = bq.rel_inf_err(y[:, rows].astype(np.float64), ref)
    assert err <= TOL
    # the offset group sums (one fma per output on int32 sums offset by
    # 1.5 * 2^23, the offsets removed every second group) add ~2e-4 of
    # ||y||_inf at most; with the fp16 output rounding the whole error stays
    # near 3e-4 on this layer
    assert err <= 1e-3


@pytest.mark.parametrize("M", [32, 96, 512])
def test_w44a8_28672x8192_group_acc_bit_exact(M):
    """Exact int32 group sums of the kernels that run the 28672 x 8192 layer
    (stream at 32 tokens, two stream passes at 96, tile at 512), one row per
    16-row tile."""
    W, rows8, img = w44a8_image()
    x = synth.activations(M, 8192, synth.WL_W44A8, 1)
    xq, _ = gbb.quant_act_i8(to_dev(x))
    rows = one_row_per(packed_rows(28672, rows8), 16, 100 + M)
    acc = gbb.w48_group_acc(img, 28672, 8192, rows8.size, xq)
    got = acc[:, torch.from_numpy(rows).to(acc.device)].cpu().numpy().astype(np.int64)
    del acc
    assert np.array_equal(got, w48_acc_reference(x, W, rows8, rows))


@functools.lru_cache(maxsize=1)
def w48_tall_image():
    """28672 x 1024, 10 % 8-bit rows: the 28672-row layer's row blocks with K
    reduced (the tile kernel's token tile depends on the row blocks and M,
    not on K)."""
    W = small(28672, 1024, 23)
    rows8 = synth.salient_rows_by_l2(W, 0.1)
    img, _, _ = gbb.pack_w48(W, rows8)
    return W, rows8, to_dev(img)


# (M, ga) of unsplit tile-kernel launches on 256 compute units: per-token
# scales take 64-token tiles at M = 200 (ragged) and 512 and 128-token tiles
# at M = 768; per-group scales take 64-token tiles at M = 512 and 128-token
# tiles at M = 2048 (eight rounds of them)
@pytest.mark.parametrize("M,ga", [(200, None), (512, None), (768, None), (512, 128), (2048, 128)])
def test_w48_tile_token_tiles(M, ga):
    """Both token tiles of the tile kernel: exact int32 group sums and y
    against the oracle, one checked row in every 16-row tile."""
    W, rows8, img = w48_tall_image()
    N, K = W.shape
    x = rand_x(M, K, 31 + M)
    xq, xs = gbb.quant_act_i8(to_dev(x), ga)
    rows = one_row_per(packed_rows(N, rows8), 16, M)
    sel = torch.from_numpy(rows).to(xq.device)
    acc = gbb.w48_group_acc(img, N, K, rows8.size, xq, ga)
    got = acc[:, sel].cpu().numpy().astype(np.int64)
    del acc
    assert np.array_equal(got, w48_acc_reference(x, W, rows8, rows, ga=ga))
    y = gbb.gemm_w48a8(img, N, K, rows8.size, xq, xs, ga)[:, sel].cpu().numpy()
    ref = ow48.reference(x, W[rows], np.nonzero(np.isin(rows, rows8))[0], act_group=ga)
    assert bq.rel_inf_err(y.astype(np.float64), ref) <= TOL


def w48_split_call(img, N, K, n8, xq, xs, ws, ga=None):
    """gbb_gemm_w48a8_split through the C ABI with the workspace ws (a
    uint8 device tensor, or None)."""
    M = xq.shape[0]
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device=xq.device)
    st = gbb.lib().gbb_gemm_w48a8_split(img.data_ptr(), N, K, n8, xq.data_ptr(), xs.data_ptr(),
                                        K if ga is None else ga, y.data_ptr(), M,
                                        ws.data_ptr() if ws is not None else None,
                                        ws.numel() if ws is not None else 0,
                                        torch.cuda.current_stream().cuda_stream)
    assert st == 0, gbb.lib().gbb_last_error().decode()
    return y


# (N, K, M, ga): the K splits.  2048 x 16384 (10 % 8-bit rows) has 4 8-bit
# and 29 4-bit stream row blocks: 16 segments of 8 groups for the former, 13
# of 10 groups (the last one 8) for the latter; M = 96 runs two 64-token
# passes through one workspace; 4096 x 4096 at M = 1 has 4 segments of 8
# groups for both.  M = 129 and 300 run the tile kernel (4 8-bit and 15
# 4-bit row blocks per token tile), with per-token and per-group scales;
# ga = 128 at M <= 64 runs the stream kernel with per-group scales, at
# M = 96 the tile kernel.
W48_SPLIT_CASES = [(2048, 16384, 1, None), (2048, 16384, 17, None), (2048, 16384, 64, None),
                   (2048, 16384, 96, None), (4096, 4096, 1, None), (2048, 16384, 129, None),
                   (2048, 16384, 300, None), (2048, 16384, 300, 128), (4096, 4096, 256, None),
                   # the stream kernel with per-group activation scales
                   (2048, 16384, 5, 128), (2048, 16384, 64, 128), (2048, 16384, 96, 128), (1024, 4096, 32, 128)]


@pytest.mark.parametrize("N,K,M,ga", W48_SPLIT_CASES)
def test_w48_split_k(N, K, M, ga):
    """The K-split stream and tile kernels against the oracle (one row per
    16-row tile), the same on every call, the workspace zero afterwards; a
    smaller workspace takes fewer segments and stays within the tolerance;
    without a workspace the call equals gbb_gemm_w48a8 bit for bit."""
    W = small(N, K, 7 * N + M)
    rows8 = synth.salient_rows_by_l2(W, 0.1)
    img = to_dev(gbb.pack_w48(W, rows8)[0])
    x = rand_x(M, K, 5 * N + M)
    xq, xs = gbb.quant_act_i8(to_dev(x), ga)
    need = gbb.gemm_w48a8_workspace(N, K, rows8.size, M, ga)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    ys = [w48_split_call(img, N, K, rows8.size, xq, xs, ws, ga) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws) == 0
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    rows = one_row_per(packed_rows(N, rows8), 16, N + M)
    ref = ow48.reference(x, W[rows], np.nonzero(np.isin(rows, rows8))[0], act_group=ga)
    assert bq.rel_inf_err(ys[0].cpu().numpy()[:, rows].astype(np.float64), ref) <= TOL
    half = torch.zeros(need // 2 + 16, dtype=torch.uint8, device=dev())
    yh = w48_split_call(img, N, K, rows8.size, xq, xs, half, ga)
    y0 = w48_split_call(img, N, K, rows8.size, xq, xs, None, ga)
    y1 = gbb.gemm_w48a8(img, N, K, rows8.size, xq, xs, ga, split=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(half) == 0
    assert bq.rel_inf_err(yh.cpu().numpy()[:, rows].astype(np.float64), ref) <= TOL
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))
    assert bq.rel_inf_err(y0.cpu().numpy()[:, rows].astype(np.float64), ref) <= TOL
    with pytest.raises(gbb.GbbError):
        gbb.gemm_w48a8(img, N, K, rows8.size, xq, xs, ga, workspace=ws[4:])


@functools.lru_cache(maxsize=1)
def w44a8_down_image():
    W, rows8 = synth.w44a8_8192x28672()
    img, _, _ = gbb.pack_w48(W, rows8)
    return W, rows8, to_dev(img)


@pytest.mark.parametrize("M", [1, 32, 64, 96, 256])
def test_w44a8_8192x28672(M):
    """The 8192 x 28672 (down projection) layer in the launches the benchmark
    times, with the K split: one checked row in every 16-row tile."""
    W, rows8, img = w44a8_down_image()
    assert rows8.size == 819
    x = synth.activations(M, 28672, synth.WL_W44A8, 2)
    xq, xs = gbb.quant_act_i8(to_dev(x))
    y = gbb.gemm_w48a8(img, 8192, 28672, rows8.size, xq, xs).cpu().numpy()
    rows = one_row_per(packed_rows(8192, rows8), 16, M)
    ref = ow48.reference(x, W[rows], np.nonzero(np.isin(rows, rows8))[0])
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL


def test_w44a8_8192x28672_group_acc_bit_exact():
    """Exact int32 group sums of the K-split stream kernel on the 8192 x
    28672 layer at 32 tokens (every segment's groups), one row per tile."""
    W, rows8, img = w44a8_down_image()
    x = synth.activations(32, 28672, synth.WL_W44A8, 3)
    xq, _ = gbb.quant_act_i8(to_dev(x))
    rows = one_row_per(packed_rows(8192, rows8), 16, 7)
    acc = gbb.w48_group_acc(img, 8192, 28672, rows8.size, xq)
    got = acc[:, torch.from_numpy(rows).to(acc.device)].cpu().numpy().astype(np.int64)
    del acc
    assert np.array_equal(got, w48_acc_reference(x, W, rows8, rows))


# ----------------------------------------------------------------------------
# 64x64 blocks
# ----------------------------------------------------------------------------
def packed64(W, bits):
    img, _, _ = gbb.pack_blocks(W, bits, block_cols=64)
    return to_dev(img)


@pytest.mark.parametrize("N,K,seed", [(64, 64, 0), (192, 448, 1), (448, 1280, 2)])
def test_64x64_unpack_dequant_bit_exact(N, K, seed):
    W = small(N, K, seed)
    bits = synth.random_bitmap64(N, K, ALLOWED, seed)
    img = packed64(W, bits)
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    assert np.array_equal(gbb.unpack_codes(img, N, K, block_cols=64).cpu().numpy(), q)
    w32, w16 = gbb.dequant(img, N, K, block_cols=64)
    ref = bq.dequant_fp32(q, s16, z16)
    assert np.array_equal(w32.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(w16.cpu().numpy().view(np.uint16), bq.fp16_rne(ref).view(np.uint16))


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 40])
def test_64x64_one_hot_rows_exact(M):
    """One-hot activations give fp16(w') exactly through every 64x64 decode
    kernel (and the 32-token chunks above 32)."""
    N, K = 192, 1216
    W = small(N, K, 31)
    bits = synth.random_bitmap64(N, K, ALLOWED, 31)
    img = packed64(W, bits)
    ks = np.random.default_rng(M).choice(K, size=M, replace=False)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1
    y = gbb.gemm_mixed_w_64x64(img, N, K, to_dev(x)).cpu().numpy()
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    w16 = bq.dequant_fp16(q, s16, z16)
    assert np.array_equal(y.view(np.uint16), w16[:, ks].T.view(np.uint16))


DECODE64_CASES = [(64, 64, 1), (128, 192, 3), (192, 320, 5), (1024, 4096, 1), (1024, 4096, 8), (320, 2560, 16),
                  (960, 1408, 17), (512, 4096, 32), (64, 28672, 2), (1024, 4096, 70), (8192, 8192, 24)]


@pytest.mark.parametrize("N,K,M", DECODE64_CASES)
def test_64x64_decode_parity(N, K, M):
    W = small(N, K, N + K + 1)
    bits = synth.random_bitmap64(N, K, ALLOWED, N + M)
    x = rand_x(M, K, M + 3)
    img = packed64(W, bits)
    xd = to_dev(x)
    need = gbb.gemm_mixed_w_64x64_workspace(N, K, M)
    ws = torch.zeros(need + 256, dtype=torch.uint8, device=dev())
    rows = np.unique(np.concatenate([[0, N - 1], np.arange(0, N, 64) + 37 % 64]))
    ref = bq.reference_rows(x, W, bits, rows, block_cols=64)
    first = None
    for _ in range(3):                      # split-K counters must reset between calls
        y = gbb.gemm_mixed_w_64x64(img, N, K, xd, workspace=ws).cpu().numpy()
        assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL
        first = y if first is None else first
        assert np.array_equal(y.view(np.uint16), first.view(np.uint16))
    assert not torch.any(ws)


@pytest.mark.parametrize("i", range(7))
def test_64x64_llama3_8b_layer_decode(i):
    """A mixed 64x64 bitmap (mean 3.10 bits, ranked by block max|w|) on each
    Llama-3-8B projection at M = 1 and 8, one checked row per block row."""
    p, W, bits = synth.llama3_8b_proj64(i)
    assert abs(synth.mean_bits(bits) - 3.1) < 0.01 and bits.shape == (p.N // 64, p.K // 64)
    img = packed64(W, bits)
    rows = one_row_per_block_row(p.N, 5 + i)
    for M in (1, 8):
        x = synth.activations(M, p.K, synth.WL_LLAMA3_8B, 20 + i)
        y = gbb.gemm_mixed_w_64x64(img, p.N, p.K, to_dev(x)).cpu().numpy()
        ref = bq.reference_rows(x, W, bits, rows, block_cols=64)
        assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL, M


# the 64x64 prefill kernel, forced: ragged shapes, one block column, 67 block
# columns (the 64-column metadata window reloads), and 16384 x 128 at
# M = 1436 (each XCD's last tiles run as 64-token halves, some past the end)
PREFILL64_CASES = [(64, 64, 33), (192, 320, 100), (128, 1280, 257), (320, 4096, 130), (576, 64 * 67, 600),
                   (16384, 128, 1436)]


@pytest.mark.parametrize("N,K,M", PREFILL64_CASES)
def test_64x64_prefill_parity(N, K, M):
    W = small(N, K, N * 3 + K)
    bits = synth.random_bitmap64(N, K, ALLOWED, N + 5 * M)
    x = rand_x(M, K, M + 11)
    y = gbb.gemm_mixed_w_64x64_path(packed64(W, bits), N, K, to_dev(x), 2)
    assert rel_err(y, bq.reference_gemm(x, W, bits, block_cols=64)) <= TOL


def test_64x64_prefill_one_hot_exact():
    """One-hot activations through the 64x64 prefill kernel give fp16(w')
    exactly (every bitwidth, both halves of each word)."""
    N, K, M = 192, 1216, 100
    W = small(N, K, 33)
    bits = synth.random_bitmap64(N, K, ALLOWED, 33)
    ks = np.random.default_rng(5).choice(K, size=M, replace=False)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1
    y = gbb.gemm_mixed_w_64x64_path(packed64(W, bits), N, K, to_dev(x), 2).cpu().numpy()
    q, s16, z16 = bq.quantize_blocks(W, bits, block_cols=64)
    w16 = bq.dequant_fp16(q, s16, z16)
    assert np.array_equal(y.view(np.uint16), w16[:, ks].T.view(np.uint16))


@pytest.mark.parametrize("i", [0, 4, 6])
def test_64x64_llama3_8b_prefill(i):
    """Llama-3-8B q, gate and down projections with the mixed 64x64 bitmap at
    M = 2048 (the prefill kernel by the library's own choice), one checked
    row per block row."""
    p, W, bits = synth.llama3_8b_proj64(i)
    img = packed64(W, bits)
    rows = one_row_per_block_row(p.N, 7 + i)
    x = synth.prefill_x(2048, p.K, i)
    lib = gbb.lib()   # the library's route is the prefill kernel, not decode chunks
    assert lib.gbb_gemm_mixed_w_64x64_path_workspace(p.N, p.K, 2048, 0) == \
        lib.gbb_gemm_mixed_w_64x64_path_workspace(p.N, p.K, 2048, 2)
    y = gbb.gemm_mixed_w_64x64(img, p.N, p.K, to_dev(x)).cpu().numpy()
    ref = bq.reference_rows(x, W, bits, rows, block_cols=64)
    assert bq.rel_inf_err(y[:, rows].astype(np.float64), ref) <= TOL
