"""gemmepi_autotune: times every tile on the caller's operands, switches the
plan to the fastest, remembers the choice for later plans of the same key
and writes it to GEMMEPI_TUNE_CACHE; results stay correct."""
import os

import numpy as np
import pytest

import activation_epilogue_gemm_amd as ge
import workloads as wl
from parity import DeviceRun, check_mask, check_out
from oracle import oracle as O

pytestmark = pytest.mark.gpu


def test_autotune_picks_the_fastest_tile_and_persists(tmp_path):
    import torch
    path = tmp_path / "tune.txt"
    os.environ["GEMMEPI_TUNE_CACHE"] = str(path)
    try:
        c = wl.random_case(1040, 1552, 520, "f16", "RELU_AUX_BIAS", False, False, 4242)
        r = DeviceRun(c)
        p = ge.plan(c.M, c.N, c.K, "f16", "RELU_AUX_BIAS", 0)
        before = p.info()
        times = p.autotune(r.A, r.B, r.bias, r.aux, r.out, reps=3)
        assert len(times) == ge.num_tiles() and all(t > 0 for t in times.values())
        best = min(times, key=times.get)
        assert f"tile={best}" in p.info() and "tuned" in p.info(), (before, p.info(), times)
        # the tuned plan still computes the operator
        p.execute(r.A, r.B, r.bias, r.aux, r.out)
        torch.cuda.synchronize()
        ref = O.gemm_epilogue(c.A, c.B, c.bias, None, c.M, c.N, c.K, "f16", "RELU_AUX_BIAS",
                              False, False)
        check_out(c, r.out_bits(), ref, label="tuned")
        check_mask(c, r.aux_words(), ref, label="tuned")
        p.destroy()
        r.close()  # last reference: the plan object is freed
        # a new plan of the same key takes the tuned tile
        with ge.plan(c.M, c.N, c.K, "f16", "RELU_AUX_BIAS", 0) as q:
            assert f"tile={best}" in q.info() and "tuned" in q.info()
        line = path.read_text().strip().splitlines()
        assert f"gemmepi-tune-v1 {c.M} {c.N} {c.K} 0 3 0 {list(times).index(best)}" in line
    finally:
        del os.environ["GEMMEPI_TUNE_CACHE"]
