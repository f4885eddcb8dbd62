"""The read-bandwidth probe reads every 16-byte piece: a buffer of zeros
with one fixed marker word makes exactly the thread that read the marker's
piece write it to the sink (the fold of a zero piece is zero)."""
import pytest
import torch

from gpu_helpers import DEV, log

pytestmark = pytest.mark.gpu

bv = pytest.importorskip("bit_verify_gemm_amd")

MARK = 0x9E3779B9 - (1 << 32)   # as int32


@pytest.mark.parametrize("pieces", [1, 7, 1024 + 3, 8192 * 256 * 8 + 17, (64 << 20) // 16])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
@pytest.mark.parametrize("shape", range(5))
def test_probe_reads_every_piece(pieces, where, shape):
    if shape >= bv.read_probe_shapes():
        pytest.skip("no such shape")
    log("probe", pieces, where, shape)
    buf = torch.zeros(pieces * 4, dtype=torch.int32, device=DEV)
    at = {"first": 0, "middle": pieces // 2, "last": pieces - 1}[where]
    buf[4 * at + 2] = MARK
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    bv.read_probe(buf, sink, shape)
    torch.cuda.synchronize()
    assert int(sink.item()) == MARK
