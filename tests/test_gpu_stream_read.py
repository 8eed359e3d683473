"""GPU check of nvfp4_weight_stream_read, the decode kernels' HBM reference
(the packed weight read with the decode kernel's loads and launch shape, no
arithmetic): every word of the packed buffer reaches a lane's checksum.  In a
buffer of zeros with one planted word equal to the sink's trigger value,
exactly the lane that reads that word stores it; an all-zero buffer leaves the
sink alone.  Shapes: the decode weight (five super-tiles per wave), a ragged
N with K = 1280 (waves of one and two super-tiles, so the last slot of a wave
is a clamped repeat), one super-tile per slab (three waves idle), K = 6144."""
import pytest
import torch

pytestmark = pytest.mark.gpu
TRIGGER = 0x9E3779B9


def _as_i32(v):
    return v - (1 << 32) if v >= 1 << 31 else v


@pytest.mark.parametrize("n,k", [(17408, 5120), (1000, 1280), (96, 256), (200, 6144)])
def test_every_word_reaches_the_checksum(gpu_lib, n, k):
    nwords = gpu_lib.nvfp4_packed_weight_bytes(n, k) // 4
    w = torch.zeros(nwords, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    gpu_lib.nvfp4_weight_stream_read(w.view(torch.uint8), n, k, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0, "all-zero weight: the sink must stay untouched"
    for idx in (0, nwords - 1, nwords // 2 + 7, nwords // 3 + 1):
        w.zero_()
        w[idx] = _as_i32(TRIGGER)
        sink.zero_()
        gpu_lib.nvfp4_weight_stream_read(w.view(torch.uint8), n, k, sink)
        torch.cuda.synchronize()
        assert sink.item() == _as_i32(TRIGGER), "word %d of %d not folded (n=%d, k=%d)" % (idx, nwords, n, k)
