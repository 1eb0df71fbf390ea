"""The benchmark's MFMA loop (libgemmepi_measure), the matrix-core work of the
256 x 256 tile with no memory traffic.  With operands of known values the
accumulators of lane 0 of wave 0 sum to a number that counts the MFMAs the
loop issued and shows which fragment slots it used: every MFMA 16x16x32 adds
sum_k a_k b_k = 32 a b to each of the 4 accumulators a lane holds per block,
and a lane holds 8 x 4 blocks."""
import pytest

import bench

pytestmark = pytest.mark.gpu

N_HALVES = bench.MFMA_LOOP_WAVES * bench.MFMA_LOOP_FRAGS * 64 * 8


def _run(src, blocks, rounds, bf16):
    import torch
    sink = torch.full((1024,), -1.0, dtype=torch.float32, device="cuda")
    bench.mfma_loop(src, sink, blocks, rounds, bf16)
    torch.cuda.synchronize()
    return sink.cpu().tolist()


@pytest.mark.parametrize("bf16", [0, 1])
def test_mfma_loop_issues_the_expected_mfmas(bf16):
    import torch
    dt = torch.bfloat16 if bf16 else torch.float16
    ones = torch.ones(N_HALVES, dtype=dt, device="cuda")
    for blocks, rounds in ((3, 5), (1, 1), (2, 77)):
        out = _run(ones, blocks, rounds, bf16)
        # 32 blocks x 4 accumulators x 32 per round
        assert out[:blocks] == [4096.0 * rounds] * blocks, (blocks, rounds, out[:blocks + 1])
        assert out[blocks:] == [-1.0] * (1024 - blocks)
    assert _run(torch.zeros_like(ones), 4, 9, bf16)[:4] == [0.0] * 4


@pytest.mark.parametrize("bf16", [0, 1])
def test_mfma_loop_reads_the_documented_fragment_slots(bf16):
    """Slots 0-7 of wave w are its A fragments (one per block row), 8-11 its
    B fragments (one per block column).  B slot 8 of wave 0 set to 2 doubles
    blocks (fm, 0): 8 x 4 x 64 + 24 x 4 x 32 = 5120 per round.  A slot 3 of
    wave 0 set to 3 triples blocks (3, fn): 4 x 4 x 96 + 28 x 4 x 32 = 5120
    as well.  Wave 1's slots do not reach wave 0's lane 0."""
    import torch
    dt = torch.bfloat16 if bf16 else torch.float16
    frag = 64 * 8   # halves per fragment slot
    for slot, val in ((8, 2.0), (3, 3.0)):
        src = torch.ones(N_HALVES, dtype=dt, device="cuda")
        src[slot * frag:(slot + 1) * frag] = val
        assert _run(src, 2, 3, bf16)[:2] == [5120.0 * 3] * 2, (slot, val)
    src = torch.ones(N_HALVES, dtype=dt, device="cuda")
    src[bench.MFMA_LOOP_FRAGS * frag:2 * bench.MFMA_LOOP_FRAGS * frag] = 5.0
    assert _run(src, 1, 2, bf16)[0] == 4096.0 * 2
