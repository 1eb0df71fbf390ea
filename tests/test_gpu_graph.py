"""Graph capture of execute(): a captured execution, replayed several times
with new inputs copied into the captured buffers and eager work and
synchronisations in between, must match an eager execution of the same
plan bit for bit.  Integer inputs make every fp32 sum exact, so this holds
for the bias gradient too, whatever the order of its atomic additions.
DRELU_BGRAD exercises the zero-fill kernel that precedes the GEMM (a fill
kernel, not a memset node, so that replays re-zero the gradient).  Split-K
plans capture the workspace their Plan allocated at the warm-up."""
import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from parity import download_bits, flags_of, torch_dtype, upload_bits, upload_words

pytestmark = pytest.mark.gpu


def _buffers(c):
    import torch
    d = {"A": upload_bits(c.A, c.dtype), "B": upload_bits(c.B, c.dtype),
         "out": torch.empty(c.M, c.N, dtype=torch_dtype(c.dtype), device="cuda")}
    if c.epilogue == "DRELU_BGRAD":
        d["bias"] = torch.empty(c.N, dtype=torch.float32, device="cuda")
        d["aux"] = upload_words(c.aux)
    else:
        d["bias"] = upload_bits(c.bias, c.dtype)
        d["aux"] = torch.zeros(c.M, ge.aux_ld_words(c.N), dtype=torch.int32, device="cuda")
    return d


@pytest.mark.parametrize("epi,b_trans,tile,splits", [
    ("RELU_AUX_BIAS", False, -1, None),
    ("DRELU_BGRAD", False, -1, None),
    ("GELU_BIAS", True, 6, None),
    ("BIAS", True, 7, None),
    # split-K: the arrival counters must be back at zero for every replay
    ("RELU_AUX_BIAS", False, 3, 3),
    ("DRELU_BGRAD", True, 5, 2),
])
def test_graph_replays_match_eager(epi, b_trans, tile, splits):
    import torch
    M, N, K = 520, 392, 264
    cases = [wl.random_case(M, N, K, "f16", epi, b_trans, b_trans, 4000 + 17 * r, kind="int")
             for r in range(4)]
    flags = flags_of(cases[0])
    with ge.plan(M, N, K, "f16", epi, flags, tile=tile, splits=splits) as p:
        assert (p.workspace_bytes() > 0) == (splits is not None)
        cap = _buffers(cases[0])
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            p.execute(cap["A"], cap["B"], cap["bias"], cap["aux"], cap["out"])  # warm-up
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            p.execute(cap["A"], cap["B"], cap["bias"], cap["aux"], cap["out"])
        for r, c in enumerate(cases):
            new = _buffers(c)
            for k in ("A", "B"):
                cap[k].copy_(new[k])
            if epi == "DRELU_BGRAD":
                cap["aux"].copy_(new["aux"])
                cap["bias"].fill_(777.0)          # replay must overwrite, not accumulate
            else:
                cap["bias"].copy_(new["bias"])
            cap["out"].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            # eager execution of the same plan on separate buffers
            p.execute(new["A"], new["B"], new["bias"], new["aux"], new["out"])
            torch.cuda.synchronize()
            assert np.array_equal(download_bits(cap["out"]), download_bits(new["out"])), f"replay {r}: out"
            if epi == "RELU_AUX_BIAS":
                assert torch.equal(cap["aux"], new["aux"]), f"replay {r}: mask"
            if epi == "DRELU_BGRAD":
                assert torch.equal(cap["bias"], new["bias"]), f"replay {r}: bgrad"
        del g


@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("norm", ["LAYERNORM", "RMSNORM"])
def test_graph_replays_norm_match_eager(norm, two_pass):
    """The norm operator is two launches in its single pass (workspace fill,
    GEMM with the row wait) and three in the two-kernel form (fill, GEMM, row
    norm); captured and replayed with new inputs it must match eager
    execution, workspace included."""
    import torch
    M, N, K = 264, 320, 136
    cases = [wl.norm_case(M, N, K, "f16", norm, True, 300 + 11 * r, kind="int") for r in range(3)]

    def bufs(c):
        up = lambda x: upload_bits(x, "f16")  # noqa: E731
        return {"A": up(c.A), "B": up(c.B), "bias": up(c.bias), "res": up(c.residual),
                "gamma": up(c.gamma), "beta": up(c.beta),
                "stats": ge.norm_stats_buffer(M),
                "out": torch.empty(M, N, dtype=torch.float16, device="cuda")}

    def run(p, b):
        p.execute_norm(b["A"], b["B"], b["bias"], b["res"], b["gamma"], b["beta"], 0.25,
                       b["stats"], b["out"])

    flags = ge.FLAG_B_TRANS | (ge.FLAG_NORM_TWO_PASS if two_pass else 0)
    with ge.plan(M, N, K, "f16", "BIAS_RES_" + norm, flags) as p:
        cap = bufs(cases[0])
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run(p, cap)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(p, cap)
        for r, c in enumerate(cases):
            new = bufs(c)
            for k in ("A", "B", "bias", "res", "gamma", "beta"):
                cap[k].copy_(new[k])
            cap["stats"].fill_(99.0)              # the replay must re-zero the sums
            cap["out"].fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            run(p, new)
            torch.cuda.synchronize()
            assert np.array_equal(download_bits(cap["out"]), download_bits(new["out"])), f"replay {r}: out"
            assert torch.equal(cap["stats"], new["stats"]), f"replay {r}: stats"
            assert ge.norm_pass_status(cap["stats"], M) == (0 if two_pass else 1)
        del g
