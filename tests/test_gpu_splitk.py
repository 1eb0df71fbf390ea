"""Split-K (gemmepi_plan_split, GEMMEPI_FLAG_SPLIT_K, gemmepi_execute_ws):
every tile with several split counts, including ranges of unequal length
and more splits than k slabs, every epilogue, fused and unfused, against
the oracle; bit-exact on integer inputs (sums of small integers are exact
in fp32 in any order).  Partial tiles are summed in split order, so
repeated executions are bitwise identical, and the arrival counters are
left at zero, so one workspace serves later executions of other plans."""
import ctypes
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
    print("[splitk]", *a, file=sys.stderr, flush=True)


def oracle_of(c):
    return O.gemm_epilogue(c.A, c.B, c.bias, c.aux, c.M, c.N, c.K, c.dtype, c.epilogue,
                           c.b_trans, c.bias_per_col)


def run_and_check(c, splits, flags=0, tile=-1, exact=False, guard=0, label=""):
    r = DeviceRun(c, flags=flags, tile=tile, guard=guard, splits=splits)
    say(label, c.name, r.info)
    r.run()
    ref = oracle_of(c)
    got = r.out_bits()
    if exact and c.epilogue not in GELU_EPIS:
        assert np.array_equal(got, ref.out), \
            f"{label} {c.name} [{r.info}]: {int((got != ref.out).sum())} elements differ"
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
            assert np.array_equal(zb, ref.zaux), f"{label} {c.name}: z aux differs"
        else:
            check_zaux(c, zb, ref, label=label)
    if c.epilogue in BGRAD_EPIS:
        bg = r.bgrad()
        if exact and c.epilogue == "DRELU_BGRAD":
            assert np.array_equal(bg, ref.bgrad), f"{label} {c.name}: bgrad differs"
        else:
            check_bgrad(c, bg, ref, label=label, unfused=bool(flags & ge.FLAG_UNFUSED))
    assert r.guards_intact(), f"{label} {c.name}: write outside the output buffers"
    info = r.info
    r.close()
    return info


@pytest.mark.parametrize("tile", range(NUM_TILES))
@pytest.mark.parametrize("b_trans", [False, True])
def test_integer_exact_every_tile_and_split(tile, b_trans):
    """K = 600: 10 slabs of 64 or 19 of 32; 3 splits give unequal ranges,
    7 leaves the last range short, 64 is capped at one slab per range."""
    M, N, K = 300, 264, 600
    for si, splits in enumerate((2, 3, 7, 64)):
        for ei, epi in enumerate(EPIS):
            c = wl.random_case(M, N, K, "f16", epi, b_trans, b_trans, 3000 + 17 * ei + si,
                               kind="int")
            info = run_and_check(c, splits, tile=tile, exact=True, guard=64,
                                 label=f"tile{tile} s{splits}")
            assert " splits=" in info, info


@pytest.mark.parametrize("tile", [0, 2, 4, 6, 7, 8])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_normal_inputs_every_epilogue(tile, dtype):
    for ei, epi in enumerate(EPIS):
        c = wl.random_case(260, 200, 1352, dtype, epi, True, True, 3500 + ei)
        run_and_check(c, 4, tile=tile, label=f"tile{tile}")


@pytest.mark.parametrize("epi", EPIS)
def test_unfused_split(epi):
    c = wl.random_case(333, 272, 1048, "f16", epi, False, False, 3600 + EPIS.index(epi))
    run_and_check(c, 3, flags=ge.FLAG_UNFUSED, label="unfused")


def test_repeatable_and_workspace_reuse():
    """Same workspace: three executions of one plan give identical bits, and
    a plan with another tile count reuses it right after."""
    import torch
    c = wl.random_case(512, 640, 2048, "f16", "RELU_AUX_BIAS", False, False, 3700)
    r = DeviceRun(c, splits=4, tile=3)
    need = r.plan.workspace_bytes()
    assert need > 0
    ws = torch.zeros(need + 4096, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        r.plan.execute(r.A, r.B, r.bias, r.aux, r.out, workspace=ws)
        torch.cuda.synchronize()
        outs.append((r.out_bits(), r.aux_words()))
    for o, a in outs[1:]:
        assert np.array_equal(o, outs[0][0]) and np.array_equal(a, outs[0][1])
    ref = oracle_of(c)
    check_out(c, outs[0][0], ref, label="reuse")
    # the arrival counters are back at zero
    ntiles = int(r.info.split("tiles=")[1].split()[0].split("x")[0]) * \
        int(r.info.split("tiles=")[1].split()[0].split("x")[1])
    assert int(ws[:4 * ntiles].view(torch.int32).abs().sum()) == 0
    r.close()
    c2 = wl.random_case(300, 264, 1000, "f16", "GELU_BIAS", True, True, 3701)
    r2 = DeviceRun(c2, splits=5, tile=5)
    assert r2.plan.workspace_bytes() <= ws.numel()
    r2.plan.execute(r2.A, r2.B, r2.bias, None, r2.out, workspace=ws)
    torch.cuda.synchronize()
    check_out(c2, r2.out_bits(), oracle_of(c2), label="reuse-2")
    r2.close()


def test_split_plan_needs_a_workspace():
    import torch
    c = wl.random_case(256, 256, 512, "f16", "BIAS", False, False, 3800)
    r = DeviceRun(c, splits=2, tile=3)
    lib = ge.library()
    st = lib.gemmepi_execute(r.plan._h, r.A.data_ptr(), r.B.data_ptr(), r.bias.data_ptr(), None,
                             r.out.data_ptr(), None)
    assert st == ge.ERR_INVALID_VALUE and "workspace" in ge.last_error()
    ws = torch.zeros(r.plan.workspace_bytes(), dtype=torch.uint8, device="cuda")
    st = lib.gemmepi_execute_ws(r.plan._h, r.A.data_ptr(), r.B.data_ptr(), r.bias.data_ptr(),
                                None, r.out.data_ptr(), ws.data_ptr(), ws.numel() - 256, None)
    assert st == ge.ERR_INVALID_VALUE
    st = lib.gemmepi_execute_ws(r.plan._h, r.A.data_ptr(), r.B.data_ptr(), r.bias.data_ptr(),
                                None, r.out.data_ptr(), ws.data_ptr(), ws.numel(), None)
    assert st == ge.OK
    torch.cuda.synchronize()
    check_out(c, r.out_bits(), oracle_of(c), label="ws")
    r.close()


@pytest.mark.parametrize("case", ["c0", "c2_512_up", "c2_512_down"])
def test_flag_chosen_split_on_the_small_workloads(case):
    """The wave-quantised workloads planned with GEMMEPI_FLAG_SPLIT_K, in full."""
    if case == "c0":
        c = wl.config0_bias()
    else:
        up, down = wl.config2_ffn("b1s512")
        if case == "c2_512_up":
            c = up
        else:
            c = down
            c.A = oracle_of(up).out
    for flags in (ge.FLAG_SPLIT_K, ge.FLAG_SPLIT_K | ge.FLAG_UNFUSED):
        run_and_check(c, None, flags=flags, label=case)


def test_first_execution_enqueued_on_another_stream():
    """The binding allocates a split plan's workspace at its first execution
    and zeroes it on torch's current stream; an execution enqueued on a
    different stream (passed explicitly, not made current) must still find
    the arrival counters at zero, or no range would run the epilogue and the
    output would be left as it was."""
    import torch
    c = wl.random_case(300, 264, 600, "f16", "RELU_BIAS", False, False, 3950, kind="int")
    r = DeviceRun(c, tile=5, splits=3)
    s = torch.cuda.Stream()
    r.out.view(torch.int16).fill_(0x7E00)
    torch.cuda.synchronize()
    r.plan.execute(r.A, r.B, r.bias, r.aux, r.out, stream=s)
    s.synchronize()
    ref = oracle_of(c)
    assert np.array_equal(r.out_bits(), ref.out)
    r.close()


def test_split_k_arrivals_over_many_rounds():
    """The arrival protocol (partials written with agent-scope stores, a
    relaxed counter increment after a barrier, the last arriver's
    agent-scope loads) rests on the hardware making a workgroup's completed
    agent-scope stores visible to a workgroup on another XCD that observes
    its counter increment.  Here it is exercised on a grid far larger than
    one round of the chip: 4096 output tiles of 64 x 64, each split 8 ways
    (32768 workgroups, 128 rounds of 256 CUs), integer inputs, every result
    bit-exact, three executions in a row on one workspace."""
    import torch
    M, N, K = 4096, 4096, 1024
    c = wl.random_case(M, N, K, "f16", "BIAS", False, False, 3900, kind="int")
    r = DeviceRun(c, tile=5, splits=8)
    say("many rounds", r.info)
    assert "splits=8" in r.info
    ref = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "BIAS", False, False)
    for rep in range(3):
        r.out.view(torch.int16).fill_(0x7E00)
        r.run()
        got = r.out_bits()
        assert np.array_equal(got, ref.out), \
            f"execution {rep}: {int((got != ref.out).sum())} elements differ"
    r.close()


@pytest.mark.parametrize("tile,splits", [(7, 2), (7, 4), (8, 2), (8, 3), (9, 2), (9, 3)])
def test_float_result_does_not_depend_on_arrival(tile, splits):
    """Normal inputs, five executions of one split plan on one workspace.
    Which split arrives last differs from tile to tile and from run to run;
    that split takes its own partial from its registers and reads the
    others' from their slots, but every element sums the partials in split
    order, so each execution gives the same bits (on the one-ahead path of
    the 256 x 128 tile, the general path of the 256 x 256 tile, and the
    two-split and general paths of the 64 x 64 x 128 tile)."""
    import torch
    c = wl.random_case(520, 392, 2200, "f16", "GELU_BIAS", True, True, 3950 + 10 * tile + splits)
    r = DeviceRun(c, splits=splits, tile=tile)
    say("arrival", tile, splits, r.info)
    assert f"splits={splits}" in r.info, r.info
    first = None
    for rep in range(5):
        r.out.view(torch.int16).fill_(0x7E00)
        r.run()
        got = r.out_bits()
        if first is None:
            first = got
            check_out(c, got, oracle_of(c), label=f"tile{tile} s{splits}")
        else:
            assert np.array_equal(got, first), \
                f"execution {rep}: {int((got != first).sum())} elements differ"
    r.close()
