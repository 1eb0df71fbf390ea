"""GEMMEPI_FLAG_STAGE_B: B stored [K,N] is copied to [N,K] in the workspace
and the GEMM reads the copy.  On integer inputs every fp32 sum is exact, so
the staged plan must equal the oracle bit for bit, for every epilogue, both
dtypes, every tile, and ragged N and K (the copy's edge tiles); the staged
and unstaged plans must then agree bit for bit as well.  Staging applies to
GEMMs of at least 8192 rows, so the shapes are 8192 (or 8200) rows deep
and narrow."""
import sys

import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from oracle import oracle as O
from parity import NUM_TILES, BGRAD_EPIS, GELU_EPIS, DeviceRun, check_bgrad, check_out

pytestmark = pytest.mark.gpu


def say(*a):
    print("[stage_b]", *a, file=sys.stderr, flush=True)


def outputs(r):
    c = r.case
    res = {"out": r.out_bits()}
    if c.epilogue == "RELU_AUX_BIAS":
        res["aux"] = r.aux_words()
    if c.epilogue == "GELU_AUX_BIAS":
        res["aux"] = r.zaux_bits()
    if c.epilogue in BGRAD_EPIS:
        res["bgrad"] = r.bgrad().copy()
    return res


def run(c, flags, tile=-1):
    r = DeviceRun(c, flags=flags, tile=tile, guard=64)
    r.run()
    res = outputs(r)
    assert r.guards_intact(), f"{c.name} [{r.info}]: write outside the output buffers"
    info = r.info
    r.close()
    return res, info


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("epi", list(O.EPILOGUES))
def test_staged_integer_exact_every_epilogue(epi, dtype):
    M, N, K = 8200, 264, 200          # ragged M, N (264 = 4 x 64 + 8) and K
    c = wl.random_case(M, N, K, dtype, epi, False, False, 8100 + list(O.EPILOGUES).index(epi),
                       kind="int")
    ref = O.gemm_epilogue(c.A, c.B, c.bias, c.aux, M, N, K, dtype, epi, False, False)
    got, info = run(c, ge.FLAG_STAGE_B)
    say(c.name, info)
    assert "stage_b" in info, info
    plain, _ = run(c, 0)
    if epi in GELU_EPIS:
        check_out(c, got["out"], ref, label="staged")
    else:
        assert np.array_equal(got["out"], ref.out), f"{c.name}: out differs from the oracle"
    for k in got:
        if k == "bgrad" and epi == "DGELU_BGRAD":
            check_bgrad(c, got[k], ref, label="staged")
            check_bgrad(c, plain[k], ref, label="unstaged")
            continue
        assert np.array_equal(got[k], plain[k]), f"{c.name}: {k} differs staged vs unstaged"
    if epi == "RELU_AUX_BIAS":
        assert np.array_equal(got["aux"], ref.mask)
    if epi == "DRELU_BGRAD":
        assert np.array_equal(got["bgrad"], ref.bgrad)


@pytest.mark.parametrize("tile", range(NUM_TILES))
def test_staged_every_tile(tile):
    M, N, K = 8192, 136, 72
    c = wl.random_case(M, N, K, "f16", "RELU_AUX_BIAS", False, False, 8200 + tile, kind="int")
    ref = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "RELU_AUX_BIAS", False, False)
    got, info = run(c, ge.FLAG_STAGE_B, tile=tile)
    assert "stage_b" in info, info
    assert np.array_equal(got["out"], ref.out), f"tile {tile}: out differs"
    assert np.array_equal(got["aux"], ref.mask), f"tile {tile}: mask differs"


def test_small_gemm_is_not_staged():
    with ge.plan(4096, 4096, 4096, "f16", "BIAS", ge.FLAG_STAGE_B) as p:
        assert "stage_b" not in p.info() and p.workspace_bytes() == 0
    with ge.plan(8192, 4096, 4096, "f16", "BIAS", ge.FLAG_STAGE_B) as p:
        assert "stage_b" in p.info() and p.workspace_bytes() == 4096 * 4096 * 2
    with ge.plan(8192, 4096, 4096, "f16", "BIAS", ge.FLAG_STAGE_B | ge.FLAG_B_TRANS) as p:
        assert "stage_b" not in p.info()
