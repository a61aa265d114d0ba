"""The load-path probe (moe_tail_probe_stream_paths) delivers the bytes it
streams: with every source byte 0x01, the direct-to-LDS rings end holding
0x01010101 in every word and the register paths' xor of everything read is 0
(an even number of equal words per load), which the probe reports through its
sink.  Private runs and one shared run, each mode, small sizes.  MI355X only
(marker ``gpu``)."""
import pytest
import torch

from latent_moe_layer_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.probes()


@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("mode,row_bytes", [(0, 128), (1, 1792), (1, 3584), (2, 128), (3, 128)])
def test_stream_paths_deliver_the_bytes(mode, row_bytes, shared):
    per = 256 * 3584 * 2  # whole 32 KB stages and whole 256-row matrices of both row widths
    grid = 8
    src = torch.full(((1 if shared else grid) * per,), 1, dtype=torch.uint8, device="cuda")
    sink = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    want = 0x01010101 if mode < 2 else 0
    B.moe_tail_probe_stream_paths(src, per, grid, shared, mode, row_bytes, sink, magic=want)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == want
    # a magic the data cannot produce leaves the sink alone
    sink.fill_(-1)
    B.moe_tail_probe_stream_paths(src, per, grid, shared, mode, row_bytes, sink, magic=0x12345)
    torch.cuda.synchronize()
    assert int(sink.item()) == -1
