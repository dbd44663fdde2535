"""The read probe behind the bench's read ceiling reads every byte it is
given (needs an MI355X).

Each thread of q4_read_probe folds the 32-bit words it reads with XOR (thread
t of a workgroup reads 16-byte words t, t + 256, t + 512 and t + 768 of each
16 KiB chunk the workgroup takes) and stores the fold to
sink[workgroup % 256] only when it equals 0x9E3779B9. A buffer of zeros with
that constant split over two words makes exactly one thread store it, and
only if it read both: one test puts them in its first and last load of a
chunk (the chunk's last word included), the other in chunks 0 and 2048,
which the launch's 2048 workgroups reach only through their grid-stride
loop.
"""
import ctypes

import pytest

from tests.gpu_util import announce, torch_mod

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9
CHUNK = 16384


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = torch_mod()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gptq_bit_weight_amd as q4
    q4.load_library()


def _probe(words, chunks):
    """Run the probe over `chunks` 16 KiB chunks of zeros with the (index,
    value) 32-bit words set; return the sink."""
    import gptq_bit_weight_amd as q4
    torch = torch_mod()
    buf = torch.zeros(chunks * CHUNK // 4, dtype=torch.int32, device="cuda")
    for i, v in words:
        buf[i] = v - (1 << 32) if v >= (1 << 31) else v
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    lib = q4.load_library()
    st = lib.q4_read_probe(ctypes.c_void_p(buf.data_ptr()), chunks * CHUNK, ctypes.c_void_p(sink.data_ptr()),
                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == q4.OK, lib.q4_last_error()
    torch.cuda.synchronize()
    return [int(v) & 0xFFFFFFFF for v in sink.cpu().tolist()]


def test_probe_reads_a_whole_chunk():
    a = 0x12345678
    # chunk 1 (workgroup 1 of 3), thread 255: the first word of its first
    # load (16-byte word 255) and the chunk's last word (end of word 1023)
    base = CHUNK // 4
    announce("read probe: one chunk")
    s = _probe([(base + 4 * 255, a), (base + 4 * 1023 + 3, a ^ MAGIC)], chunks=3)
    assert s[1] == MAGIC
    assert all(v == 0 for i, v in enumerate(s) if i != 1)
    # the same values in two threads' words fold to nothing
    s = _probe([(base + 4 * 255, a), (base + 4 * 1022 + 3, a ^ MAGIC)], chunks=3)
    assert all(v == 0 for v in s)


def test_probe_grid_stride_covers_every_chunk():
    # 2049 chunks, 2048 workgroups: workgroup 0 reads chunks 0 and 2048
    a = 0x0BADF00D
    announce("read probe: 2049 chunks")
    s = _probe([(0, a), (2048 * CHUNK // 4 + 3, a ^ MAGIC)], chunks=2049)
    assert s[0] == MAGIC
    assert all(v == 0 for v in s[1:])
