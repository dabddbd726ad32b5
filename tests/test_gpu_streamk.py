"""GPU checks of the stream-K path of the bf16 GEMM, used when the tiles of a product
(256 x 192) do not fill whole rounds of the 256-workgroup grid and the call has a
workspace: the k-stages are split evenly over the workgroups, the runs write the
float32 partials of split tiles, and a second kernel adds them in run order. A row
linear (Z = Y W) with a workspace takes that path and without one the tile kernel,
so the two are compared: every k-range must be summed exactly once whatever the
split (only the float32 summation order differs), and repeated calls are
bit-identical."""
import pytest
import torch

from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def _row_linear(Y, W, with_ws):
    M, K = Y.shape
    N = W.shape[1]
    Z = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    ws = None
    if with_ws:
        nbytes = tp.linear_workspace(M, K, N)
        assert nbytes > 0, "this product should take the stream-K path"
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    tp.row_linear(Y, W, Z, ws)
    torch.cuda.synchronize()
    return Z


def _inputs(M, K, N, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    Y = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16)
    W = (torch.randn(K, N, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    return Y, W


# (M, K, N): 2 tiles split 48 ways (one k-stage per run); 64 tiles split 4 ways; 2 tiles
# split 128 ways (runs on two XCDs); 120 tiles over two or three runs each; 264 tiles
# (the GPT-3 cross-entropy shape's count: one whole round, then 8 tiles split 32 ways);
# 576 tiles (two whole rounds, then 64 tiles split 4 ways) and 864 (three rounds, then
# 96 tiles split over 2-3 runs). Every K has at least the 48 k-stages below which
# stream-K is not used.
@pytest.mark.parametrize("M,K,N", [(300, 1536, 136), (2048, 2048, 1536), (64, 12288, 384), (1920, 4096, 2880),
                                   (2048, 1536, 6288), (4096, 2048, 6912), (2304, 1536, 18432)])
def test_streamk_matches_tile_kernel(M, K, N):
    note(f"stream-K row linear M={M} K={K} N={N}")
    Y, W = _inputs(M, K, N, M + K + N)
    sk = _row_linear(Y, W, True)
    tile = _row_linear(Y, W, False)
    assert not torch.isnan(sk).any()
    err = float((sk.double() - tile.double()).abs().max() / tile.double().abs().max())
    assert err < 1e-5, err


# Ragged shapes drawn once from a seeded generator (M any size, N and K multiples of 8),
# kept where the last round is at most half full: 9 to 108 remainder tiles, two with a
# whole round first (286 and 265 tiles), 58 to 140 k-stages, and M = 1. Each split
# tile's pieces are summed by the fixup's single-wave row blocks.
@pytest.mark.parametrize("M,K,N", [(767, 2616, 472), (475, 1864, 6712), (731, 3680, 6728), (2816, 3640, 4808),
                                   (1, 2200, 5384), (1792, 2272, 776), (215, 1832, 6144), (202, 2080, 2696),
                                   (2303, 4480, 1624), (1279, 4456, 10168), (512, 2848, 2296),
                                   (1281, 3544, 3080)])
def test_streamk_ragged_shapes(M, K, N):
    note(f"stream-K ragged row linear M={M} K={K} N={N}")
    Y, W = _inputs(M, K, N, 7 * M + K + N)
    sk = _row_linear(Y, W, True)
    tile = _row_linear(Y, W, False)
    assert not torch.isnan(sk).any()
    err = float((sk.double() - tile.double()).abs().max() / tile.double().abs().max())
    assert err < 1e-5, err


def test_streamk_repeatable():
    note("stream-K repeatability")
    Y, W = _inputs(64, 12288, 384, 5)
    runs = [_row_linear(Y, W, True) for _ in range(3)]
    for r in runs[1:]:
        assert torch.equal(r, runs[0])
