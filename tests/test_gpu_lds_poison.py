"""The integer-exact parity checks run through the LDS race-detector build
(libgemmepi_poison.so, compiled with GEMMEPI_LDS_POISON=1): every wave fills
each 1 KiB LDS block with NaN bits before it issues the global->LDS load
that writes the block, and the whole ring is poisoned again after the main
loop, before the epilogue and the split-K arrival flag reuse it.  A read of
a block whose load has not landed, a refill that overtakes a reader of the
previous contents, or an epilogue read of a staging slot it never wrote then
yields NaN, and integer inputs (exact fp32 sums) turn any of them into a
bit mismatch.  Covers every tile (all three schedules), both B layouts,
both dtypes, ragged edges, fewer slabs than stages, and split-K."""
import importlib.util
import os
import sys

import numpy as np
import pytest

import parity
import workloads as wl
from oracle import oracle as O

pytestmark = pytest.mark.gpu

PKG = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "activation_epilogue_gemm_amd")
EXACT_EPIS = ["DEFAULT", "BIAS", "RELU_AUX_BIAS", "DRELU_BGRAD"]


def say(*a):
    print("[lds-poison]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def poisoned():
    """A second instance of the binding, bound to the race-detector build;
    the parity helpers use it while this module's tests run."""
    lib = os.path.join(PKG, "libgemmepi_poison.so")
    if not os.path.exists(lib):
        pytest.fail(f"{lib} is not built (__graft_entry__.build())")
    spec = importlib.util.spec_from_file_location("gemmepi_poisoned_binding",
                                                  os.path.join(PKG, "__init__.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.LIB_PATH = lib
    mod.library()
    real = parity.ge
    parity.ge = mod
    yield mod
    parity.ge = real


def exact(c, flags=0, tile=-1, splits=None):
    r = parity.DeviceRun(c, flags=flags, tile=tile, guard=64, splits=splits)
    r.run()
    ref = O.gemm_epilogue(c.A, c.B, c.bias, c.aux, c.M, c.N, c.K, c.dtype, c.epilogue, c.b_trans,
                          c.bias_per_col)
    got = r.out_bits()
    assert np.array_equal(got, ref.out), \
        f"{c.name} [{r.info}]: {int((got != ref.out).sum())} elements differ"
    if c.epilogue == "RELU_AUX_BIAS":
        assert np.array_equal(r.aux_words(), ref.mask), f"{c.name} [{r.info}]: mask differs"
    if c.epilogue == "DRELU_BGRAD":
        assert np.array_equal(r.bgrad(), ref.bgrad), f"{c.name} [{r.info}]: bgrad differs"
    assert r.guards_intact(), f"{c.name} [{r.info}]: write outside the output buffers"
    info = r.info
    r.close()
    return info


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("b_trans", [False, True])
@pytest.mark.parametrize("tile", range(parity.NUM_TILES))
def test_poisoned_every_tile(poisoned, tile, b_trans, dtype):
    for ei, epi in enumerate(EXACT_EPIS):
        c = wl.random_case(300, 264, 200, dtype, epi, b_trans, b_trans, 9100 + 7 * tile + ei,
                           kind="int")
        info = exact(c, tile=tile)
    say(f"tile {tile} b_trans {b_trans} {dtype} ok ({info})")
    for K in (8, 72):  # fewer k slabs than ring stages; one partial slab
        c = wl.random_case(130, 72, K, dtype, "RELU_AUX_BIAS", b_trans, b_trans, 9300 + K + tile,
                           kind="int")
        exact(c, tile=tile)


@pytest.mark.parametrize("b_trans", [False, True])
@pytest.mark.parametrize("tile", range(parity.NUM_TILES))
def test_poisoned_split_k(poisoned, tile, b_trans):
    for epi in ("RELU_AUX_BIAS", "DRELU_BGRAD"):
        c = wl.random_case(300, 264, 600, "f16", epi, b_trans, b_trans, 9500 + tile, kind="int")
        exact(c, tile=tile, splits=3)


def test_poisoned_staged_b(poisoned):
    c = wl.random_case(8200, 264, 200, "f16", "RELU_AUX_BIAS", False, False, 9600, kind="int")
    info = exact(c, flags=poisoned.FLAG_STAGE_B)
    assert "stage_b" in info


@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
@pytest.mark.parametrize("tile", range(parity.NUM_TILES))
def test_poisoned_norm_every_tile(poisoned, tile, norm):
    """The norm operator through the race-detector build, on every tile:
    the single pass (residual staged in LDS and read again after the row
    wait, statistics slices in LDS) and the two-kernel form.  Integer inputs
    make y and the row sums exact, so both forms must give the same bits; a
    read of a poisoned or stale LDS slot would give NaN instead."""
    c = wl.norm_case(272, 320, 96, "f16", norm, True, 9500 + tile, kind="int")
    o1, s1, st1 = parity.run_norm(c, tile=tile)
    o2, s2, st2 = parity.run_norm(c, flags=poisoned.FLAG_NORM_TWO_PASS, tile=tile)
    assert (st1, st2) == (1, 0), f"tile {tile}: status {st1}, {st2}"
    assert not np.isnan(O.decode(o1, c.dtype)).any(), f"tile {tile}: NaN in the single pass"
    assert np.array_equal(o1, o2), f"tile {tile}: single pass and two kernels differ"
    assert np.array_equal(s1, s2), f"tile {tile}: statistics differ"
    ref = O.gemm_norm(c.A, c.B, c.bias, c.residual, c.gamma, c.beta, c.eps, c.M, c.N, c.K,
                      c.dtype, c.norm, c.b_trans)
    parity.check_norm(c, o1, s1, ref, np.arange(c.M), label=f"poison tile {tile}", status=1)
    say(f"norm {norm} tile {tile} ok")
