"""GPU checks of the stream-K path of the bf16 GEMM, used when the tiles of a product
(256 x 192) do not fill whole rounds of the 256-workgroup grid and the call has a
workspace: the k-stages are split evenly over the workgroups, the runs write the
float32 partials of split tiles, and a second kernel adds them in run order. The
vocabulary-parallel logits GEMM of tp_vocab_ce_partials leaves its float32 output at
the start of the workspace, so it can be compared with the same product from the
tile kernel (tp_row_linear against E_i^T): every k-range must be summed exactly once
whatever the split, and repeated calls are bit-identical."""
import pytest
import torch

from tests.gpu_util import DEV, note

pytestmark = pytest.mark.gpu

tp = pytest.importorskip("attention_shard_math_amd")


def _logits_streamk(H, E, lo, hi):
    M = H.shape[0]
    V = hi - lo
    tgt = torch.zeros(M, dtype=torch.int32, device=DEV)
    mx = torch.empty(M, dtype=torch.float32, device=DEV)
    se = torch.empty(M, dtype=torch.float32, device=DEV)
    tl = torch.empty(M, dtype=torch.float32, device=DEV)
    ws = torch.empty(tp.vocab_ce_workspace(M, H.shape[1], lo, hi), dtype=torch.uint8, device=DEV)
    tp.vocab_ce_partials(H, E, tgt, lo, hi, mx, se, tl, ws)
    torch.cuda.synchronize()
    return ws[: M * V * 4].view(torch.float32).view(M, V).clone()


# (M, h, V): 2 tiles split 16 ways; 64 tiles split 4 ways; 2 tiles split 128 ways
# (runs on two XCDs); 120 tiles over two or three runs each; and 264 tiles (the GPT-3
# cross-entropy shape's count: one round and 8 more), most split over two runs.
@pytest.mark.parametrize("M,h,V", [(300, 512, 136), (2048, 2048, 1536), (64, 12288, 384), (1920, 4096, 2880),
                                   (2048, 1024, 6288)])
def test_streamk_matches_tile_kernel(M, h, V):
    note(f"stream-K logits M={M} h={h} V={V}")
    g = torch.Generator(device=DEV)
    g.manual_seed(M + h + V)
    H = torch.randn(M, h, generator=g, device=DEV).to(torch.bfloat16)
    E = (torch.randn(V, h, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    lo = 8 * V
    sk = _logits_streamk(H, E, lo, lo + V)
    tile = torch.empty(M, V, dtype=torch.float32, device=DEV)
    tp.row_linear(H, E.t().contiguous(), tile)    # 'N'-layout product, tile kernel (no workspace)
    torch.cuda.synchronize()
    err = float((sk.double() - tile.double()).abs().max() / tile.double().abs().max())
    assert err < 1e-5, err


def test_streamk_repeatable():
    note("stream-K repeatability")
    M, h, V = 64, 12288, 384
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    H = torch.randn(M, h, generator=g, device=DEV).to(torch.bfloat16)
    E = (torch.randn(V, h, generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    runs = [_logits_streamk(H, E, 0, V) for _ in range(3)]
    for r in runs[1:]:
        assert torch.equal(r, runs[0])
