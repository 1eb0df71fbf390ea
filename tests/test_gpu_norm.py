"""GEMM + bias + residual + LayerNorm/RMSNorm (structural fusion) through
gemmepi_execute_norm, against the oracle's gemm_norm."""
import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from oracle import oracle as O
from parity import check_norm, run_norm

pytestmark = pytest.mark.gpu


def _ref(c, rows=None):
    return O.gemm_norm(c.A, c.B, c.bias, c.residual, c.gamma, c.beta, c.eps, c.M, c.N, c.K,
                       c.dtype, c.norm, c.b_trans, rows=rows)


@pytest.mark.parametrize("tile", [-1, 0, 2, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
@pytest.mark.parametrize("b_trans", [False, True])
def test_norm_every_tile(tile, norm, b_trans):
    for dtype in ("f16", "bf16"):
        c = wl.norm_case(300, 264, 200, dtype, norm, b_trans, 610 + tile)
        out, stats = run_norm(c, tile=tile)
        rows = np.arange(c.M)
        check_norm(c, out, stats, _ref(c), rows, label=f"tile{tile}")


def test_norm_integer_inputs_every_tile_agree():
    """Integer operands make y exact on every tile; the statistics are then
    exact fp64 sums, so every tile must produce identical bits."""
    c = wl.norm_case(272, 320, 96, "f16", "LAYERNORM", True, 77, kind="int")
    outs = [run_norm(c, tile=t) for t in range(ge.num_tiles())]
    for t, (o, s) in enumerate(outs[1:], 1):
        assert np.array_equal(o, outs[0][0]), f"tile {t} output differs from tile 0"
        assert np.array_equal(s, outs[0][1]), f"tile {t} stats differ from tile 0"
    check_norm(c, outs[0][0], outs[0][1], _ref(c), np.arange(c.M), label="int")


@pytest.mark.parametrize("with_bias,with_residual,with_beta", [
    (False, False, False), (True, False, True), (False, True, False)])
def test_norm_optional_operands(with_bias, with_residual, with_beta):
    for norm in ("LAYERNORM", "RMSNORM"):
        c = wl.norm_case(130, 96, 72, "f16", norm, True, 31, with_bias=with_bias,
                         with_residual=with_residual, with_beta=with_beta)
        out, stats = run_norm(c)
        check_norm(c, out, stats, _ref(c), np.arange(c.M), label="optional")


@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
def test_norm_unfused_matches_oracle(norm):
    for dtype in ("f16", "bf16"):
        c = wl.norm_case(200, 264, 136, dtype, norm, False, 91)
        out, stats = run_norm(c, flags=ge.FLAG_UNFUSED)
        check_norm(c, out, stats, _ref(c), np.arange(c.M), label="unfused")


def test_norm_edge_shapes():
    for (M, N, K) in ((1, 8, 8), (17, 40, 8), (65, 1000, 24), (3, 2056, 16)):
        for norm in ("LAYERNORM", "RMSNORM"):
            c = wl.norm_case(M, N, K, "f16", norm, True, M + N)
            out, stats = run_norm(c)
            check_norm(c, out, stats, _ref(c), np.arange(M), label=f"{M}x{N}x{K}")


@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
def test_norm_ffn_down_full_size(norm):
    """The 2048-token FFN down-projection shape (M 2048, N 4096, K 11008),
    fused and unfused, on 384 seed-chosen rows (rows 0 and M-1 included)."""
    c = wl.config5_ffn_down_norm(norm)
    rows = wl.sample_rows(c.M, 384, wl.row_sample_seed(5))
    ref = _ref(c, rows)
    for flags, label in ((0, "fused"), (ge.FLAG_UNFUSED, "unfused")):
        out, stats = run_norm(c, flags=flags)
        check_norm(c, out, stats, ref, rows, label=label)
