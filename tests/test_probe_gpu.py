"""The bandwidth probe of the tuning header (qg_read_probe): every launch
shape the bench sweeps runs to completion on buffers that end inside a
tile, exactly at a tile's end and beyond the grid, and the host rejects what
it documents as errors."""
import pytest

from gpu_util import qg, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("loads", [2, 4, 8, 16])
def test_probe_every_launch_shape_completes(loads):
    q = qg()
    torch = torch_cuda()
    tile = loads * 4096
    buf = torch.zeros(64 * tile + 48, dtype=torch.uint8, device="cuda")
    sink = torch.full((4096,), 7, dtype=torch.int32, device="cuda")
    for nbytes in (16, 4096 + 16, tile, tile + 16, 3 * tile - 16, 64 * tile + 48):
        for wgs in (1, 2, 7, 64, 4096):
            q.qg_read_probe(buf, sink, wgs, loads, nbytes)
    torch.cuda.synchronize()
    # all-zero data folds to 0, never the fixed value that would be stored
    assert (sink.cpu() == 7).all()


def test_probe_abi_errors():
    q = qg()
    torch = torch_cuda()
    L = q.lib()
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    assert L.qg_read_probe(buf.data_ptr(), 4096, sink.data_ptr(), 8, 3, s) == 2          # loads not 2/4/8/16
    assert L.qg_read_probe(buf.data_ptr(), 8, sink.data_ptr(), 8, 4, s) == 2             # fewer than 16 bytes
    assert L.qg_read_probe(buf.data_ptr(), 4096, sink.data_ptr(), 0, 4, s) == 2          # no workgroup
    assert L.qg_read_probe(None, 4096, sink.data_ptr(), 8, 4, s) == 1                    # NULL buffer
    assert L.qg_read_probe(buf.data_ptr() + 8, 4096, sink.data_ptr(), 8, 4, s) == 3      # misaligned
    torch.cuda.synchronize()
