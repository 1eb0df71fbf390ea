"""The benchmark's stream-read reference (libgemmepi_measure): it must read
exactly the requested bytes, in every launch shape the benchmark sweeps.
Workgroup w covers threads * loads * 16 bytes; a thread writes sink word
w % 1024 only when the XOR of the 32-bit words it read equals 0x9E3779B9, so
single planted words show which bytes were read."""
import pytest

import bench

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9 - (1 << 32)   # as int32
SHAPES = [(t, l) for t in (256, 512, 1024) for l in (4, 8, 16, 32)]


def _run(planted, nbytes, threads, loads, nt, total_words):
    import torch
    buf = torch.zeros(total_words, dtype=torch.int32, device="cuda")
    for w in planted:
        buf[w] = MAGIC
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    bench.stream_read(buf, nbytes, sink, threads, loads, nt)
    torch.cuda.synchronize()
    return {i for i, v in enumerate(sink.cpu().tolist()) if v != 0}


@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("threads,loads", SHAPES)
def test_stream_read_reads_exactly_the_requested_bytes(threads, loads, nt):
    wg_words = threads * loads * 4
    nbytes = 23 * wg_words * 4 + 4096          # 23 full workgroups and a partial one
    total = 26 * wg_words
    inside = [5 * wg_words + 777 % wg_words, 23 * wg_words + 1000]
    assert _run(inside, nbytes, threads, loads, nt, total) == {5, 23}
    past = [nbytes // 4, nbytes // 4 + 17, 23 * wg_words + 4000 % wg_words + 1024,
            24 * wg_words + 5]
    past = [w for w in past if w * 4 >= nbytes]
    assert _run(past, nbytes, threads, loads, nt, total) == set()


def test_stream_read_rejects_bad_arguments():
    import torch
    buf = torch.zeros(1024, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        bench.stream_read(buf, 0, sink)
    with pytest.raises(RuntimeError):
        bench.stream_read(buf, 100, sink)       # not a multiple of 16
