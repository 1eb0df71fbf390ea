"""GEMM + bias + residual + LayerNorm/RMSNorm (structural fusion) through
gemmepi_execute_norm, against the oracle's gemm_norm: the single pass (y kept
in fp32, the row statistics exchanged between the workgroups of a band of
rows) and the two-kernel form (y rounded into out, then normalised)."""
import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from oracle import oracle as O
from parity import check_norm, run_norm

pytestmark = pytest.mark.gpu

TWO = ge.FLAG_NORM_TWO_PASS


def _ref(c, rows=None):
    return O.gemm_norm(c.A, c.B, c.bias, c.residual, c.gamma, c.beta, c.eps, c.M, c.N, c.K,
                       c.dtype, c.norm, c.b_trans, rows=rows)


def _run_check(c, rows, ref, label, flags=0, tile=-1, expect_status=None):
    out, stats, status = run_norm(c, flags=flags, tile=tile)
    if expect_status is not None:
        assert status == expect_status, f"{label} {c.name}: status {status}, expected {expect_status}"
    check_norm(c, out, stats, ref, rows, label=label, status=status)
    return out, stats, status


@pytest.mark.parametrize("tile", [-1, 0, 2, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
@pytest.mark.parametrize("b_trans", [False, True])
def test_norm_every_tile(tile, norm, b_trans):
    for dtype in ("f16", "bf16"):
        c = wl.norm_case(300, 264, 200, dtype, norm, b_trans, 610 + tile)
        rows = np.arange(c.M)
        ref = _ref(c)
        _run_check(c, rows, ref, f"tile{tile}", tile=tile, expect_status=1)
        _run_check(c, rows, ref, f"tile{tile} two-pass", flags=TWO, tile=tile, expect_status=0)


def test_norm_integer_inputs_every_tile_agree():
    """Integer operands make y exact (in fp32 and in fp16) on every tile; the
    statistics are then exact fp64 sums, so every tile, in both forms, must
    produce identical bits."""
    c = wl.norm_case(272, 320, 96, "f16", "LAYERNORM", True, 77, kind="int")
    first = None
    for t in range(ge.num_tiles()):
        for flags in (0, TWO):
            o, s, status = run_norm(c, flags=flags, tile=t)
            assert status == (0 if flags else 1)
            if first is None:
                first = (o, s)
                continue
            assert np.array_equal(o, first[0]), f"tile {t} flags {flags}: output differs"
            assert np.array_equal(s, first[1]), f"tile {t} flags {flags}: stats differ"
    check_norm(c, first[0], first[1], _ref(c), np.arange(c.M), label="int", status=1)


@pytest.mark.parametrize("with_bias,with_residual,with_beta", [
    (False, False, False), (True, False, True), (False, True, False)])
def test_norm_optional_operands(with_bias, with_residual, with_beta):
    for norm in ("LAYERNORM", "RMSNORM"):
        c = wl.norm_case(130, 96, 72, "f16", norm, True, 31, with_bias=with_bias,
                         with_residual=with_residual, with_beta=with_beta)
        ref = _ref(c)
        for flags in (0, TWO):
            _run_check(c, np.arange(c.M), ref, "optional", flags=flags)


@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
def test_norm_unfused_matches_oracle(norm):
    for dtype in ("f16", "bf16"):
        c = wl.norm_case(200, 264, 136, dtype, norm, False, 91)
        # (the unfused form leaves the status word as it was: the pattern
        # run_norm fills in reads 0 there)
        _run_check(c, np.arange(c.M), _ref(c), "unfused", flags=ge.FLAG_UNFUSED, expect_status=0)


def test_norm_edge_shapes():
    for (M, N, K) in ((1, 8, 8), (17, 40, 8), (65, 1000, 24), (3, 2056, 16)):
        for norm in ("LAYERNORM", "RMSNORM"):
            c = wl.norm_case(M, N, K, "f16", norm, True, M + N)
            ref = _ref(c)
            for flags in (0, TWO):
                _run_check(c, np.arange(M), ref, f"{M}x{N}x{K}", flags=flags,
                           expect_status=0 if flags else 1)


def test_norm_grid_larger_than_the_chip_takes_two_kernels():
    """The 256 x 128 ping-pong tile holds one workgroup per CU, so 2304 rows
    of 4096 columns (9 x 32 = 288 tiles) do not fit on the 256 CUs at once:
    execute_norm must fall back to the two-kernel form (status 0), and the
    2048-row shape (256 tiles) must still run in one pass."""
    for M, expect in ((2304, 0), (2048, 1)):
        c = wl.norm_case(M, 4096, 64, "f16", "LAYERNORM", True, 5 + M)
        rows = wl.sample_rows(c.M, 256, 17)
        _run_check(c, rows, _ref(c, rows), f"M{M}", tile=7, expect_status=expect)


def test_norm_wait_gives_up_when_forced(monkeypatch):
    """The single pass's row wait is bounded.  With the bound forced to zero
    polls (GEMMEPI_NORM_WAIT_POLLS=0) a workgroup that does not see its whole
    band arrived at its first poll gives up: the call still completes, bit 1
    of the status word is set and that workgroup's rows are NaN (a loud
    result, never a hang).  Without the override the next call is correct."""
    c = wl.norm_case(512, 1024, 64, "f16", "LAYERNORM", True, 41)
    monkeypatch.setenv("GEMMEPI_NORM_WAIT_POLLS", "0")
    gave_up = 0
    for _ in range(3):
        out, _, status = run_norm(c, allow_gave_up=True)
        assert status & 1, f"status {status:#x}: not the single pass"
        if status & 2:
            gave_up += 1
            assert np.isnan(O.decode(out, c.dtype)).any(), "a wait gave up but no row is NaN"
    assert gave_up > 0, "no workgroup gave up with a zero poll bound"
    monkeypatch.delenv("GEMMEPI_NORM_WAIT_POLLS")
    _run_check(c, np.arange(c.M), _ref(c), "after forced give-up", expect_status=1)


@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
def test_norm_ffn_down_full_size(norm):
    """The 2048-token FFN down-projection shape (M 2048, N 4096, K 11008):
    single pass, two kernels and unfused, on 384 seed-chosen rows (rows 0 and
    M-1 included)."""
    c = wl.config5_ffn_down_norm(norm)
    rows = wl.sample_rows(c.M, 384, wl.row_sample_seed(5))
    ref = _ref(c, rows)
    for flags, label, expect in ((0, "single pass", 1), (TWO, "two kernels", 0),
                                 (ge.FLAG_UNFUSED, "unfused", 0)):
        _run_check(c, rows, ref, label, flags=flags, expect_status=expect)
