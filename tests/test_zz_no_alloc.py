"""gemmepi_execute_noalloc, the entry point for callers that cannot allocate:
a split-K plan takes its workspace from the library's static device scratch
instead of a caller's buffer.  Its results must equal those of
gemmepi_execute_ws, the entry point it is a variant of (same kernels, same
split order), bit for bit: on two calls in a row, the second with a smaller
input, and for every epilogue on integer inputs (whose fp32 sums are exact
in any order, bgrad included, except DGELU's, whose terms acc * gelu'(z)
are not integers: there both runs are held to the parity tolerance)."""
import sys

import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from oracle import oracle as O
from parity import DeviceRun, check_bgrad

pytestmark = pytest.mark.gpu


def say(*a):
    print("[noalloc]", *a, file=sys.stderr, flush=True)


def results(r):
    """Copies of every output of the run's buffers."""
    c = r.case
    res = {"out": r.out_bits()}
    if c.epilogue == "RELU_AUX_BIAS":
        res["aux"] = r.aux_words()
    if c.epilogue == "GELU_AUX_BIAS":
        res["aux"] = r.zaux_bits()
    if c.epilogue in ("DRELU_BGRAD", "DGELU_BGRAD"):
        res["bgrad"] = r.bgrad().copy()
    return res


def poison(r):
    import torch
    r.out.view(torch.int16).fill_(0x7E00)
    c = r.case
    if c.epilogue in ("RELU_AUX_BIAS",):
        r.aux.fill_(-0x2A2A2A2B)
    if c.epilogue == "GELU_AUX_BIAS":
        r.aux.view(torch.int16).fill_(0x7E00)
    if c.epilogue in ("DRELU_BGRAD", "DGELU_BGRAD"):
        r.bias.fill_(1234.5)


def compare_noalloc_with_ws(c, splits=None, tile=-1, flags=0, label=""):
    """Run the case through gemmepi_execute_ws (the plan's own zeroed
    workspace), then through gemmepi_execute_noalloc into the same, poisoned,
    buffers; every output must be bitwise identical."""
    import torch
    r = DeviceRun(c, flags=flags, tile=tile, guard=64, splits=splits)
    need = r.plan.workspace_bytes()
    say(label, c.name, r.info, f"workspace {need} bytes")
    assert 0 < need <= ge.noalloc_scratch_bytes(), (need, r.info)
    r.run()
    want = results(r)
    poison(r)
    r.plan.execute_noalloc(r.A, r.B, r.bias, r.aux, r.out)
    torch.cuda.synchronize()
    got = results(r)
    for k in want:
        if k == "bgrad" and c.epilogue == "DGELU_BGRAD":
            # acc * gelu'(z) is not an integer: the fp32 atomics that sum
            # the workgroups' column partials may round differently in
            # another arrival order, so both runs are held to the parity
            # bar against the oracle instead
            ref = O.gemm_epilogue(c.A, c.B, c.bias, c.aux, c.M, c.N, c.K, c.dtype, c.epilogue,
                                  c.b_trans, c.bias_per_col)
            check_bgrad(c, want[k], ref, label=label + " execute_ws")
            check_bgrad(c, got[k], ref, label=label + " execute_noalloc")
            continue
        assert np.array_equal(got[k], want[k]), \
            f"{label} {c.name} [{r.info}]: {k}: {int((got[k] != want[k]).sum())} values differ"
    assert r.guards_intact(), f"{label} {c.name}: write outside the output buffers"
    r.close()


def test_noalloc_two_calls_second_smaller():
    """The split plans of the suite as planned, each call smaller than the
    one before and reusing the scratch it left behind: the 2048-token FFN
    down-projection (256 x 256 tiles, 2 K ranges, 64 MiB of partial tiles),
    the 512-token one (4 K ranges, 32 MiB), then the BIAS workload
    W[1024,2048].X[2048,512] (2 K ranges, 4 MiB)."""
    for i, v in enumerate(("b1s2048", "b1s512")):
        _, down = wl.config2_ffn(v)
        # the down-projection's input is the up-projection's output; any
        # [tokens, 11008] input serves this comparison
        down.A = wl.normal((down.M, down.K), 7300 + i, 1.0, down.dtype)
        compare_noalloc_with_ws(down, flags=ge.FLAG_SPLIT_K, label=f"call {i + 1}")
    compare_noalloc_with_ws(wl.config0_bias(), flags=ge.FLAG_SPLIT_K, label="call 3")


@pytest.mark.parametrize("epi", list(O.EPILOGUES))
def test_noalloc_every_epilogue_integer(epi):
    """Integer inputs, explicit tiles and split counts (unequal K ranges),
    ragged edges; a larger case, then a smaller one."""
    for i, (M, N, K, tile, splits, bt) in enumerate(((300, 264, 600, 8, 3, False),
                                                      (130, 72, 200, 5, 2, True))):
        c = wl.random_case(M, N, K, "f16", epi, bt, bt, 7100 + 13 * i, kind="int")
        compare_noalloc_with_ws(c, splits=splits, tile=tile, label=f"{epi} #{i}")


def test_noalloc_unsplit_plan_equals_execute():
    import torch
    c = wl.random_case(200, 136, 96, "bf16", "RELU_AUX_BIAS", False, False, 7200)
    r = DeviceRun(c, guard=64)
    assert r.plan.workspace_bytes() == 0
    r.run()
    want = results(r)
    poison(r)
    r.plan.execute_noalloc(r.A, r.B, r.bias, r.aux, r.out)
    torch.cuda.synchronize()
    got = results(r)
    for k in want:
        assert np.array_equal(got[k], want[k]), k
    r.close()


def test_noalloc_rejects_workspace_beyond_scratch():
    """4096 x 4096 x 8192 on the 256 x 256 tile in 8 K ranges needs 512 MiB of
    partial tiles: refused before anything is launched."""
    with ge.plan(4096, 4096, 8192, "f16", "BIAS", 0, 0, 8) as p:
        assert p.workspace_bytes() > ge.noalloc_scratch_bytes()
        with pytest.raises(ge.GemmEpiError) as ei:
            p.execute_noalloc(1 << 20, 1 << 20, 1 << 20, None, 1 << 20, check=False)
        assert ei.value.status == ge.ERR_UNSUPPORTED
        assert "static scratch" in ge.last_error()
