"""Seeded random sweeps through the C ABI.

* 120 cases drawn over shape (M, N, K up to a few hundred, K a multiple of
  8, N ragged when B_TRANS), dtype, B layout, bias orientation, epilogue,
  tile (or the planner's choice) and split count.  Integer inputs make
  every non-GELU result bit-exact against the oracle; GELU results use the
  tolerance.
* 900 wider cases: log-uniform shapes up to ~3000 x 3000 x 4000, decode
  shapes (1-16 tokens), up to 64 split ranges, the unfused sequence, normal
  and integer inputs; and 200 GEMM + bias + residual + norm cases in the
  single pass, the two-kernel form and unfused."""
import sys

import numpy as np
import pytest

import workloads as wl
from oracle import oracle as O
import activation_epilogue_gemm_amd as ge
from parity import (NUM_TILES, BGRAD_EPIS, GELU_EPIS, DeviceRun, check_bgrad, check_norm, check_out,
                    check_zaux, run_norm)

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
        r = DeviceRun(c, tile=tile, splits=splits, guard=32)
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


def _logdim(rng, lo, hi):
    return int(np.exp(rng.uniform(np.log(lo), np.log(hi))))


def _wide_cases(n, seed):
    rng = np.random.default_rng(seed)
    for i in range(n):
        b_trans = bool(rng.integers(2))
        decode = b_trans and rng.random() < 0.2
        M = int(rng.integers(1, 17)) if decode else _logdim(rng, 1, 3150)
        N = _logdim(rng, 1, 3150) if b_trans else 8 * _logdim(rng, 1, 405)
        K = 8 * _logdim(rng, 1, 540)
        dtype = ("f16", "bf16")[int(rng.integers(2))]
        epi = EPIS[int(rng.integers(len(EPIS)))]
        per_col = bool(rng.integers(2)) and epi not in BGRAD_EPIS and epi != "DEFAULT"
        tile = -1 if decode else int(rng.integers(-1, NUM_TILES))
        splits = None if decode else (None, 1, 2, 3, 4, 7, 16, 33, 64)[int(rng.integers(9))]
        flags = ge.FLAG_UNFUSED if (rng.random() < 0.15 and splits in (None, 1)) else 0
        kind = "int" if rng.random() < 0.7 else "normal"
        yield i, M, N, K, dtype, epi, b_trans, per_col, tile, splits, flags, kind


@pytest.mark.parametrize("chunk", range(3))
def test_wide_random_cases_match_the_oracle(chunk):
    for i, M, N, K, dtype, epi, b_trans, per_col, tile, splits, flags, kind in \
            _wide_cases(900, 20261203):
        if i % 3 != chunk:
            continue
        c = wl.random_case(M, N, K, dtype, epi, b_trans, per_col, 700000 + i, kind=kind)
        r = DeviceRun(c, flags=flags, tile=tile, splits=splits, guard=32)
        print(f"[random-wide] case {i} ({kind}): {r.info}", file=sys.stderr, flush=True)
        r.run()
        ref = O.gemm_epilogue(c.A, c.B, c.bias, c.aux, M, N, K, dtype, epi, b_trans, per_col)
        got = r.out_bits()
        # integer inputs are exact in the fused epilogue; the unfused sequence
        # rounds the GEMM result before the bias add (a second rounding once
        # the sums leave the exactly representable integers) and is held to
        # the tolerance, as are GELU results and normal inputs
        if kind == "int" and epi not in GELU_EPIS and not flags & ge.FLAG_UNFUSED:
            assert np.array_equal(got, ref.out), f"case {i} [{r.info}]: " \
                f"{int((got != ref.out).sum())} elements differ"
        else:
            check_out(c, got, ref, label=f"wide case {i}")
        if epi == "RELU_AUX_BIAS" and kind == "int":
            assert np.array_equal(r.aux_words(), ref.mask), f"case {i}: mask"
        if epi in BGRAD_EPIS:
            check_bgrad(c, r.bgrad(), ref, label=f"wide case {i}", unfused=bool(flags & ge.FLAG_UNFUSED))
        assert r.guards_intact(), f"case {i}: write outside the output buffers"
        r.close()


def test_random_norm_cases_match_the_oracle():
    rng = np.random.default_rng(20261204)
    for i in range(200):
        M, N, K = _logdim(rng, 1, 2700), 8 * _logdim(rng, 1, 1350), 8 * _logdim(rng, 1, 270)
        dtype = ("f16", "bf16")[int(rng.integers(2))]
        norm = ("LAYERNORM", "RMSNORM")[int(rng.integers(2))]
        b_trans = bool(rng.integers(2))
        flags = (0, ge.FLAG_NORM_TWO_PASS, ge.FLAG_UNFUSED)[int(rng.integers(3))]
        tile = int(rng.integers(-1, NUM_TILES))
        c = wl.norm_case(M, N, K, dtype, norm, b_trans, 900000 + i)
        print(f"[random-norm] case {i}: {M}x{N}x{K} {dtype} {norm} bt={b_trans} flags={flags} "
              f"tile={tile}", file=sys.stderr, flush=True)
        ref = O.gemm_norm(c.A, c.B, c.bias, c.residual, c.gamma, c.beta, c.eps, c.M, c.N, c.K,
                          c.dtype, c.norm, c.b_trans)
        out, stats, status = run_norm(c, flags=flags, tile=tile)
        check_norm(c, out, stats, ref, np.arange(M), label=f"random norm {i}", status=status)
