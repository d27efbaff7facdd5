"""The bare streaming read (santa_stream_read), the bench's measured ceiling:
it reads every byte at every occupancy, writes nothing (the sink keeps its
value unless the folded words hit one fixed constant), and a ragged size or
an occupancy out of range is refused before any launch."""

import ctypes

import pytest
import torch

from stochastic_sparse_decode_amd import santa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wpc", [1, 2, 4, 8])
@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 << 20, 64 << 20])
def test_reads_and_writes_nothing(wpc, nbytes):
    buf = torch.full((nbytes // 2,), 1.0, dtype=torch.float16, device="cuda")
    guard = torch.full((64,), 7, dtype=torch.int32, device="cuda")
    sink = guard[8:9]
    santa.santa_stream_read(buf, wpc, sink)
    torch.cuda.synchronize()
    assert (guard == 7).all()  # neither the sink nor its neighbours changed


def test_refuses_bad_arguments():
    lib = santa.library()
    buf = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    vp = ctypes.c_void_p
    assert lib.santa_stream_read(vp(buf.data_ptr()), 1000, 1, vp(sink.data_ptr()), None) == 2  # not a multiple of 16
    assert lib.santa_stream_read(vp(buf.data_ptr()), 1024, 0, vp(sink.data_ptr()), None) == 2
    assert lib.santa_stream_read(vp(buf.data_ptr()), 1024, 9, vp(sink.data_ptr()), None) == 2
    assert lib.santa_stream_read(None, 1024, 1, vp(sink.data_ptr()), None) == 1
