"""Parity at the edges of the accepted shapes, on seed-chosen rows against the
oracle: a very long K (262144 products per output in fp32, split-K ranges of
many slabs), and a very wide B stored [K,N] whose deepest slab (the 128 k
rows of the 64 x 64 x 128 tile) spans ~1 GiB from its buffer descriptor, half
the 32-bit offset range that plan() guards."""
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from oracle import oracle as O
from parity import DeviceRun, check_out

pytestmark = pytest.mark.gpu


def say(*a):
    print("[extreme]", *a, flush=True)


def _case(name, M, N, K, epi, b_trans, seed, a_std, b_std):
    c = wl.DeviceCase(name, M, N, K, "f16", epi, b_trans, False)
    c.A_dev = wl.device_normal((M, K), seed, a_std, "f16")
    c.B_dev = wl.device_normal((N, K) if b_trans else (K, N), seed + 1, b_std, "f16")
    c.bias = wl.normal((M,), seed + 2, 1.0, "f16")
    return c


def _ref(c, rows):
    return O.gemm_epilogue(c.host_A(rows), c.host_B(), c.bias[rows], None, len(rows), c.N, c.K,
                           c.dtype, c.epilogue, c.b_trans, c.bias_per_col)


@pytest.mark.parametrize("b_trans", [False, True])
def test_long_k(b_trans):
    """M 256, N 512, K 2^18: the planner's plan and split-K plans of 8 and 64
    ranges (4096 and 128 k per range on the 32-wide slabs)."""
    import torch
    c = _case(f"longk_{'nk' if b_trans else 'kn'}", 256, 512, 1 << 18, "BIAS", b_trans, 9100,
              1.0 / 128.0, 1.0)
    rows = wl.sample_rows(c.M, 16, 9199)
    ref = _ref(c, rows)
    for splits in (None, 8, 64):
        r = DeviceRun(c, splits=splits)
        say(c.name, splits, r.info)
        r.run()
        check_out(c, r.out_bits(rows), ref, label=f"{c.name}-splits{splits}")
        r.close()
        del r
        torch.cuda.empty_cache()


def test_wide_n_deepest_slab():
    """M 64, N 2^22, K 128, B stored [K,N]: the 64 x 64 x 128 tile (one slab
    of 128 k rows, each 8 MiB apart) and the planner's choice, RELU_BIAS."""
    import torch
    c = _case("widen_kn", 64, 1 << 22, 128, "RELU_BIAS", False, 9300, 1.0 / 16.0, 1.0)
    rows = wl.sample_rows(c.M, 4, 9399)
    ref = _ref(c, rows)
    deep = [t for t in range(ge.num_tiles()) if ge.tile_name(t).startswith("64x64x128")]
    assert deep, "no 64x64x128 tile"
    for tile in (-1, deep[0]):
        r = DeviceRun(c, tile=tile)
        say(c.name, tile, r.info)
        r.run()
        got = r.out_bits(rows)
        check_out(c, got, ref, label=f"{c.name}-tile{tile}")
        r.close()
        del r
        torch.cuda.empty_cache()
