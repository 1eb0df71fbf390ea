"""gemmepi_stream_read, the measurement helper: it must read exactly the
requested bytes.  Workgroup w covers 128 KiB; a thread writes sink word
w % 1024 only when the XOR of the 32-bit words it read equals 0x9E3779B9,
so single planted words show which bytes were read."""
import pytest

import activation_epilogue_gemm_amd as ge

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9 - (1 << 32)   # as int32
WG_WORDS = 128 * 1024 // 4
NBYTES = 23 * 128 * 1024 + 4096  # 23 full workgroups and a partial one


def _run(planted):
    import torch
    buf = torch.zeros(26 * WG_WORDS, dtype=torch.int32, device="cuda")
    for w in planted:
        buf[w] = MAGIC
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    ge.stream_read(buf, NBYTES, sink)
    torch.cuda.synchronize()
    return {i for i, v in enumerate(sink.cpu().tolist()) if v != 0}, sink


def test_stream_read_reads_every_requested_byte():
    hit, sink = _run([5 * WG_WORDS + 777, 23 * WG_WORDS + 1000])
    assert hit == {5, 23}
    assert sink[5].item() == MAGIC and sink[23].item() == MAGIC


def test_stream_read_reads_nothing_past_the_end():
    hit, _ = _run([NBYTES // 4, NBYTES // 4 + 17, 23 * WG_WORDS + 4000, 24 * WG_WORDS + 5])
    assert hit == set()


def test_stream_read_rejects_bad_arguments():
    import torch
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(ge.GemmEpiError):
        ge.stream_read(buf, 0, sink)
    with pytest.raises(ge.GemmEpiError):
        ge.stream_read(buf, 100, sink)       # not a multiple of 16
