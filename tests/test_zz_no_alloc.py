"""The allocation-free block GEMM (gbb_gemm_mixed_w_noalloc) through the C
ABI against gbb_gemm_mixed_w with a caller workspace: the same kernels, so
the outputs must be bit-identical, call after call, as the shared scratch
array returns to zero after each call; and both within 2e-3 of the oracle."""
import numpy as np
import pytest

import synth
from oracle import blockquant as bq

torch = pytest.importorskip("torch")
gbb = pytest.importorskip("gemm_block_bit_amd")

pytestmark = pytest.mark.gpu
ALLOWED = (1, 2, 3, 4, 6, 8)


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def case(N, K, M, seed):
    g = np.random.default_rng(seed)
    W = (0.02 * g.standard_normal((N, K))).astype(np.float16)
    bits = synth.random_bitmap(N, K, ALLOWED, seed)
    img, _, _ = gbb.pack_blocks(W, bits)
    x = g.standard_normal((M, K)).astype(np.float16)
    return W, bits, torch.from_numpy(img).to(dev()), torch.from_numpy(x).to(dev()), x


def run_noalloc(img, N, K, xd, M):
    y = torch.full((M, N), float("nan"), dtype=torch.float16, device=xd.device)
    st = gbb.lib().gbb_gemm_mixed_w_noalloc(img.data_ptr(), N, K, xd.data_ptr(), y.data_ptr(), M,
                                            torch.cuda.current_stream(xd.device).cuda_stream)
    assert st == 0, gbb.lib().gbb_last_error().decode()
    return y


def run_with_workspace(img, N, K, xd, M):
    # the size of the allocation-free array: a prefill K split then takes the
    # same number of segments on both entry points
    ws = torch.zeros(16 << 20, dtype=torch.uint8, device=xd.device)
    y = torch.empty((M, N), dtype=torch.float16, device=xd.device)
    st = gbb.lib().gbb_gemm_mixed_w(img.data_ptr(), N, K, xd.data_ptr(), y.data_ptr(), M, ws.data_ptr(),
                                    ws.numel(), torch.cuda.current_stream(xd.device).cuda_stream)
    assert st == 0, gbb.lib().gbb_last_error().decode()
    return y


# pairs of calls in a row, the second on a smaller input: split-K decode at
# M = 1 and 8, one row per workgroup at M = 32, the two-row kernel with its
# fp32 K-segment partials (8192 x 8192 at M = 32, 4096 x 16384 at M = 17),
# 32-token decode chunks (M = 64),
# the prefill kernel with no K split (2048 x 1024, M = 600) and with a K split
# whose full size (67 MB) the array does not hold (2048 x 16384, M = 512:
# 4 segments instead of 16), followed by decode chunks
PAIRS = [((2048, 8192, 8), (1024, 4096, 1)),
         ((1024, 4096, 32), (256, 1024, 3)),
         ((8192, 8192, 32), (4096, 16384, 17)),
         ((4096, 4096, 64), (1024, 2048, 33)),
         ((2048, 1024, 600), (1024, 4096, 16)),
         ((2048, 16384, 512), (512, 8192, 300))]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (N, K, M) in enumerate((first, second)):
        W, bits, img, xd, x = case(N, K, M, N + K + M + i)
        a = run_noalloc(img, N, K, xd, M)
        b = run_with_workspace(img, N, K, xd, M)
        again = run_noalloc(img, N, K, xd, M)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (N, K, M)
        assert torch.equal(again.view(torch.int16), b.view(torch.int16)), (N, K, M)
        rows = np.unique(np.concatenate([[0, N - 1], np.arange(0, N, 64) + 17]))
        ref = bq.reference_rows(x, W, bits, rows)
        assert bq.rel_inf_err(a.cpu().numpy()[:, rows].astype(np.float64), ref) <= 2e-3


def test_noalloc_argument_errors():
    N, K = 128, 256
    _, _, img, xd, _ = case(N, K, 2, 5)
    y = torch.empty((2, N), dtype=torch.float16, device=dev())
    L = gbb.lib()
    s = torch.cuda.current_stream().cuda_stream
    assert L.gbb_gemm_mixed_w_noalloc(None, N, K, xd.data_ptr(), y.data_ptr(), 2, s) == -1
    assert L.gbb_gemm_mixed_w_noalloc(img.data_ptr(), N, 200, xd.data_ptr(), y.data_ptr(), 2, s) == -2
    assert L.gbb_gemm_mixed_w_noalloc(img.data_ptr(), N, K, xd.data_ptr() + 2, y.data_ptr(), 2, s) == -4
    assert L.gbb_gemm_mixed_w_noalloc(img.data_ptr(), N, K, xd.data_ptr(), y.data_ptr(), 0, s) == 0
    torch.cuda.synchronize()
