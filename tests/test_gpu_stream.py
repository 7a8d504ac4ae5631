"""mxs_stream_read on the GPU: every 16-byte vector of the buffer is read.

The kernel folds the words each lane reads into an XOR and ORs 1 into the sink only when that XOR
equals 0x9E3779B9. A zero buffer leaves the sink 0; one marker vector (0x9E3779B9, 0, 0, 0) anywhere
sets it, whether the vector lies in the unrolled main loop or in the tail loop.
"""
import pytest
import torch

import mx_fp4_weight_amd as mxs
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

MARK = 0x9E3779B9 - (1 << 32)  # as a signed int32 word


def read_with_marker(n16, at):
    buf = torch.zeros((n16, 4), dtype=torch.int32, device="cuda")
    if at is not None:
        buf[at, 0] = MARK
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    mxs.stream_read(buf, sink)
    torch.cuda.synchronize()
    return int(sink.item())


@pytest.mark.parametrize("n16,at", [(65536, None), (65536, 12345), (65536, 65535), (1, 0),
                                    (4 << 20, None), (4 << 20, 3_000_001), (4 << 20, (4 << 20) - 1),
                                    ((4 << 20) + 777, (4 << 20) + 700)])
def test_stream_read_reads_every_vector(n16, at):
    say(f"stream_read n16={n16} marker={at}")
    assert read_with_marker(n16, at) == (0 if at is None else 1)
