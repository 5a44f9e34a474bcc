"""GPU checks of the streaming-read measurement reference (pkv_stream_read):
every 16-byte unit of the buffer is read, whatever its position relative to
the workgroups' ranges."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.mark.parametrize("units", [1, 7, 2048 * 256 + 13, 5_000_003])
def test_stream_read_reaches_every_unit(lib, units):
    """A zero buffer leaves the sink alone; a planted unit (fold value in one
    32-bit word) at the first, a middle and the last position sets it."""
    data = torch.zeros(units * 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.stream_read(data, sink)
    torch.cuda.synchronize()
    assert sink.item() == 0
    magic = np.array([MAGIC], dtype=np.uint32).view(np.int32)[0]
    for pos in sorted({0, units // 2, units - 1}):
        data.zero_()
        data[4 * pos + 2] = int(magic)
        sink.zero_()
        lib.stream_read(data, sink)
        torch.cuda.synchronize()
        assert sink.item() == 1, f"unit {pos} of {units} not read"
