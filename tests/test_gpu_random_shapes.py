"""Seeded random sweep through the C ABI: 120 cases drawn over shape
(M, N, K up to a few hundred, K a multiple of 8, N ragged when B_TRANS),
dtype, B layout, bias orientation, epilogue, tile (or the planner's
choice) and split count.  Integer inputs make every non-GELU result
bit-exact against the oracle; GELU results use the tolerance."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import oracle as O
from parity import NUM_TILES, BGRAD_EPIS, GELU_EPIS, GpuRun, check_bgrad, check_out, check_zaux

pytestmark = pytest.mark.gpu

EPIS = list(O.EPILOGUES)


def _cases(n, seed):
    rng = np.random.default_rng(seed)
    for i in range(n):
        b_trans = bool(rng.integers(2))
        M = int(rng.integers(1, 400))
        N = int(rng.integers(1, 400)) if b_trans else 8 * int(rng.integers(1, 50))
        K = 8 * int(rng.integers(1, 100))
        dtype = ("f16", "bf16")[int(rng.integers(2))]
        epi = EPIS[int(rng.integers(len(EPIS)))]
        per_col = bool(rng.integers(2)) and epi not in BGRAD_EPIS and epi != "DEFAULT"
        tile = int(rng.integers(-1, NUM_TILES))
        splits = (None, 1, 2, 3, 5)[int(rng.integers(5))]
        yield i, M, N, K, dtype, epi, b_trans, per_col, tile, splits


@pytest.mark.parametrize("chunk", range(4))
def test_random_cases_match_the_oracle(chunk):
    for i, M, N, K, dtype, epi, b_trans, per_col, tile, splits in _cases(120, 20251202):
        if i % 4 != chunk:
            continue
        c = wl.random_case(M, N, K, dtype, epi, b_trans, per_col, 50000 + i, kind="int")
        r = GpuRun(c, tile=tile, splits=splits, guard=32)
        print(f"[random] case {i}: {r.info}", file=sys.stderr, flush=True)
        r.run()
        ref = O.gemm_epilogue(c.A, c.B, c.bias, c.aux, M, N, K, dtype, epi, b_trans, per_col)
        got = r.out_bits()
        if epi in GELU_EPIS:
            check_out(c, got, ref, label=f"case {i}")
        else:
            assert np.array_equal(got, ref.out), f"case {i} [{r.info}]: " \
                f"{int((got != ref.out).sum())} elements differ"
        if epi == "RELU_AUX_BIAS":
            assert np.array_equal(r.aux_words(), ref.mask), f"case {i}: mask"
        if epi == "GELU_AUX_BIAS":
            assert np.array_equal(r.zaux_bits(), ref.zaux), f"case {i}: z aux"
        if epi == "DRELU_BGRAD":
            assert np.array_equal(r.bgrad(), ref.bgrad), f"case {i}: bgrad"
        if epi == "DGELU_BGRAD":
            check_bgrad(c, r.bgrad(), ref, label=f"case {i}")
        assert r.guards_intact(), f"case {i}: write outside the output buffers"
        r.close()
