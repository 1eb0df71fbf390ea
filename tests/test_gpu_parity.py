"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small ragged shapes cover every tile configuration, both B layouts, both
dtypes, every epilogue and both bias orientations; exact-integer inputs make
those comparisons bit-exact (fp32 sums of small integers are exact, so one
rounding of the same value must agree).  Full-size workloads are compared
with the tolerance of the parity helper module, on every output for the small
and FFN workloads and on 4096 seed-chosen rows (plus all of bgrad) for the
large ones.
"""
import os
import sys

import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from oracle import oracle as O
from parity import NUM_TILES, BGRAD_EPIS, GELU_EPIS, DeviceRun, check_bgrad, check_mask, check_out, check_zaux

pytestmark = pytest.mark.gpu

EPIS = list(O.EPILOGUES)


def say(*a):
    print("[parity]", *a, file=sys.stderr, flush=True)


def oracle_of(c, rows=None, A_bits=None):
    return O.gemm_epilogue(c.A if A_bits is None else A_bits, c.B, c.bias, c.aux, c.M, c.N, c.K,
                           c.dtype, c.epilogue, c.b_trans, c.bias_per_col, rows=rows)


def run_and_check(c, flags=0, tile=-1, exact=False, guard=0, label=""):
    """exact: integer inputs, so every result that is a rounding of an exact
    sum is compared bit for bit; results that go through GELU or its
    derivative (out of the GELU epilogues, DGELU's bgrad) use the tolerance."""
    r = DeviceRun(c, flags=flags, tile=tile, guard=guard)
    say(label, c.name, r.info)
    r.run()
    ref = oracle_of(c)
    got = r.out_bits()
    if exact and c.epilogue not in GELU_EPIS:
        if not np.array_equal(got, ref.out):
            bad = np.argwhere(got != ref.out)[:5]
            raise AssertionError(f"{label} {c.name} [{r.info}]: {int((got != ref.out).sum())} "
                                 f"elements differ, first {bad.tolist()} got "
                                 f"{[O.decode(got[i, j], c.dtype) for i, j in bad]} want "
                                 f"{[O.decode(ref.out[i, j], c.dtype) for i, j in bad]}")
    else:
        check_out(c, got, ref, label=label)
    if c.epilogue == "RELU_AUX_BIAS":
        words = r.aux_words()
        if exact:
            assert np.array_equal(words, ref.mask), f"{label} {c.name}: mask differs"
        else:
            check_mask(c, words, ref, label=label)
    if c.epilogue == "GELU_AUX_BIAS":
        zb = r.zaux_bits()
        if exact:
            assert np.array_equal(zb, ref.zaux), f"{label} {c.name}: z aux differs " \
                f"{np.argwhere(zb != ref.zaux)[:5].tolist()}"
        else:
            check_zaux(c, zb, ref, label=label)
    if c.epilogue in BGRAD_EPIS:
        bg = r.bgrad()
        if exact and c.epilogue == "DRELU_BGRAD":
            assert np.array_equal(bg, ref.bgrad), f"{label} {c.name}: bgrad differs " \
                f"{np.argwhere(bg != ref.bgrad)[:5].ravel().tolist()}"
        else:
            check_bgrad(c, bg, ref, label=label, unfused=bool(flags & ge.FLAG_UNFUSED))
    assert r.guards_intact(), f"{label} {c.name}: write outside the output buffers"
    r.close()


# ---------------------------------------------------------------- every tile, exact


def test_tile_count():
    assert ge.num_tiles() == NUM_TILES


@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("b_trans", [False, True])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_exact_every_tile(tile, b_trans, dtype):
    M, N, K = 300, 264, 200   # ragged in M, N and K for every tile shape
    for ei, epi in enumerate(EPIS):
        if epi == "GELU_BIAS":
            continue  # not exact by nature; covered with tolerance below
        for per_col in (False, True):
            if (epi == "DEFAULT" or epi in BGRAD_EPIS) and per_col:
                continue
            c = wl.random_case(M, N, K, dtype, epi, b_trans, per_col, 100 + 7 * ei + per_col,
                               kind="int")
            run_and_check(c, tile=tile, exact=True, guard=64, label=f"tile{tile}")
    # fewer k slabs than pipeline stages, and a single partial slab
    for K in (8, 72):
        c = wl.random_case(70, 40, K, dtype, "RELU_AUX_BIAS", b_trans, b_trans, 900 + K,
                           kind="int")
        run_and_check(c, tile=tile, exact=True, guard=64, label=f"tile{tile} K={K}")


@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("b_trans", [False, True])
def test_tolerance_every_tile_gelu_and_normal_inputs(tile, b_trans):
    M, N, K = 260, 200, 328
    for dtype in ("f16", "bf16"):
        for epi in ("GELU_BIAS", "RELU_AUX_BIAS", "DRELU_BGRAD", "GELU_AUX_BIAS", "DGELU_BGRAD"):
            c = wl.random_case(M, N, K, dtype, epi, b_trans, b_trans, 555 + tile)
            run_and_check(c, tile=tile, label=f"tile{tile}")


# ---------------------------------------------------------------- unfused path
@pytest.mark.parametrize("epi", EPIS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_unfused_matches_oracle(epi, dtype):
    for b_trans in (False, True):
        c = wl.random_case(333, 272, 264, dtype, epi, b_trans, b_trans, 900 + EPIS.index(epi))
        run_and_check(c, flags=ge.FLAG_UNFUSED, label="unfused")
    if dtype == "f16" and epi != "GELU_BIAS":
        # small integers stay exact through the unfused fp16 intermediates
        # (GELU results themselves are held to the tolerance)
        c = wl.random_case(300, 264, 200, dtype, epi, False, False, 950, kind="int")
        run_and_check(c, flags=ge.FLAG_UNFUSED, exact=True, guard=64, label="unfused-int")


# ---------------------------------------------------------------- decode path
@pytest.mark.parametrize("T", [1, 2, 3, 4, 7, 16])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_path(T, dtype):
    for epi in ("DEFAULT", "BIAS", "RELU_BIAS", "GELU_BIAS"):
        # (4104, 520): N past 4096 rows, where four tokens take the
        # row-streaming kernel as they do with K past 4096 (203, 4104)
        for (N, K) in ((200, 520), (4096, 4096), (24, 8), (203, 4104), (203, 1000), (4104, 520)):
            c = wl.random_case(T, N, K, dtype, epi, True, True, 300 + T + N)
            r = DeviceRun(c)
            assert "path=decode" in r.info, r.info
            r.close()
            run_and_check(c, guard=32, label="decode")
            run_and_check(c, flags=ge.FLAG_UNFUSED, label="decode-unfused")
        c = wl.random_case(T, 136, 264, dtype, epi, True, False, 400 + T, kind="int")
        run_and_check(c, exact=(epi != "GELU_BIAS"), label="decode-int-rowbias")


def test_thin_m_through_tiled_kernel():
    for M in (1, 5, 16, 17, 31, 33):
        c = wl.random_case(M, 128, 96, "f16", "GELU_BIAS", True, True, 70 + M)
        run_and_check(c, flags=ge.FLAG_NO_DECODE, label="thin-tiled")


# ---------------------------------------------------------------- edge shapes
@pytest.mark.parametrize("shape", [(1, 8, 8), (1, 1, 8), (3, 5, 16), (64, 64, 64), (65, 72, 72),
                                   (257, 264, 8), (511, 520, 1032)])
def test_edge_shapes(shape):
    M, N, K = shape
    for epi in EPIS:
        b_trans = (N % 8 != 0) or (M % 2 == 1)
        c = wl.random_case(M, N, K, "f16", epi, b_trans, False, 11 + M + N + K, kind="int")
        run_and_check(c, exact=True, guard=16, label="edge")


def test_repeatable_and_stable():
    c = wl.random_case(512, 512, 512, "f16", "RELU_AUX_BIAS", False, False, 42)
    r = DeviceRun(c).run()
    o1, a1 = r.out_bits(), r.aux_words()
    r.run(times=3)
    assert np.array_equal(o1, r.out_bits()) and np.array_equal(a1, r.aux_words())
    r.close()


# ---------------------------------------------------------------- workloads at full size
def test_config0_bias_full():
    c = wl.config0_bias()
    run_and_check(c, label="config0")
    run_and_check(c, flags=ge.FLAG_UNFUSED, label="config0-unfused")


@pytest.mark.parametrize("T", [1, 4, 16])
def test_config1_decode_full(T):
    c = wl.config1_decode(T)
    run_and_check(c, label="config1")
    run_and_check(c, flags=ge.FLAG_UNFUSED, label="config1-unfused")


@pytest.mark.parametrize("variant", list(wl.FFN_TOKENS))
def test_config2_ffn_full(variant):
    """Both GEMMs compared in full: the down projection stage-isolated (fed
    the GPU's h) and chained (fed the oracle's own rounded h)."""
    up, down = wl.config2_ffn(variant)
    ref_up = oracle_of(up)
    down.A = ref_up.out
    ref_chain = oracle_of(down)
    for flags in (0, ge.FLAG_UNFUSED):
        ru = DeviceRun(up, flags=flags).run()
        say("config2", variant, ru.info)
        h_gpu = ru.out_bits()
        check_out(up, h_gpu, ref_up, label=f"config2-up-{flags}")
        rd = DeviceRun(down, flags=flags, A_dev=ru.out).run()
        say("config2", variant, rd.info)
        y_gpu = rd.out_bits()
        check_out(down, y_gpu, oracle_of(down, A_bits=h_gpu), A_bits=h_gpu,
                  label=f"config2-down-{flags}")
        check_out(down, y_gpu, ref_chain, A_bits=ref_up.out, label=f"config2-chain-{flags}")
        ru.close()
        rd.close()


def _large(c, rows_count=4096, flag_sets=(0, ge.FLAG_UNFUSED)):
    """4096 seed-chosen rows (always 0 and M-1) of out / mask, all of bgrad,
    for each of the plan flag sets (one oracle result serves them all)."""
    import torch
    cfg = 4 if c.epilogue in BGRAD_EPIS else 3
    rows = wl.sample_rows(c.M, rows_count, wl.row_sample_seed(cfg))
    B = c.host_B()
    if c.epilogue in BGRAD_EPIS:
        ref = O.gemm_epilogue(c.host_A(), B, None, c.aux, c.M, c.N, c.K, c.dtype, c.epilogue,
                              c.b_trans, c.bias_per_col, rows=rows)
    else:
        ref = O.gemm_epilogue(c.host_A(rows), B, c.bias[rows], None, len(rows), c.N, c.K,
                              c.dtype, c.epilogue, c.b_trans, c.bias_per_col)
    for flags in flag_sets:
        r = DeviceRun(c, flags=flags)
        say("large", c.name, r.info)
        if flags & ge.FLAG_STAGE_B:
            assert "stage_b" in r.info, r.info
        r.run()
        check_out(c, r.out_bits(rows), ref, label=f"large-{flags}")
        if c.epilogue == "RELU_AUX_BIAS":
            n = check_mask(c, r.aux_words(rows), ref, label=f"large-{flags}")
            say("mask bits excused", n, "of", ref.z.size)
        if c.epilogue == "GELU_AUX_BIAS":
            check_zaux(c, r.zaux_bits(rows), ref, label=f"large-{flags}")
        if c.epilogue in BGRAD_EPIS:
            check_bgrad(c, r.bgrad(), ref, label=f"large-{flags}",
                        unfused=bool(flags & ge.FLAG_UNFUSED))
        r.close()
        del r
        torch.cuda.empty_cache()


# the benchmark runs the two large workloads with B staged ([K,N] copied to
# [N,K] in the workspace, GEMMEPI_FLAG_STAGE_B): both forms, fused and unfused
STAGED = (0, ge.FLAG_UNFUSED, ge.FLAG_STAGE_B, ge.FLAG_STAGE_B | ge.FLAG_UNFUSED)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_config3_relu_aux_full(dtype):
    _large(wl.config3_relu_aux(dtype), flag_sets=STAGED)


def test_config3_relu_aux_full_b_stored_nk():
    """C3's fp16 operands with B stored [N,K] (both operands K-contiguous,
    so the 256 x 256 ping-pong tile also fetches B in double-wide slabs)."""
    c = wl.config3_relu_aux("f16")
    c.B_dev = c.B_dev.t().contiguous()
    c.b_trans = True
    c.name += "_bnk"
    _large(c)


def test_config4_drelu_bgrad_full():
    _large(wl.config4_drelu_bgrad(), flag_sets=STAGED)


def test_dgelu_bgrad_full():
    """The GELU backward at the DRELU backward's shape (dY[8192,16384],
    W[16384,4096]) with a saved z of the same size."""
    _large(wl.config4_dgelu_bgrad())


def test_gelu_aux_full():
    """The GELU forward that saves z, at the ReLU-aux forward's shape."""
    _large(wl.config3_gelu_aux())
