"""CPU tests of the C-ABI boundary: the library loads, exports every symbol
that include/gemmepi.h declares, and validates arguments before any HIP call
(gemmepi_plan makes none; execute rejects bad pointers first)."""
import ctypes
import os
import re

import pytest

import activation_epilogue_gemm_amd as ge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemmepi.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemmepi_[a-z_]+)\s*\(", text)))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("gemmepi_plan", "gemmepi_plan_tiled", "gemmepi_execute", "gemmepi_plan_destroy",
              "gemmepi_plan_info", "gemmepi_aux_ld_words", "gemmepi_aux_bytes",
              "gemmepi_status_string", "gemmepi_last_error", "gemmepi_num_tiles",
              "gemmepi_tile_name", "gemmepi_version", "gemmepi_execute_noalloc",
              "gemmepi_execute_norm", "gemmepi_norm_stats_bytes", "gemmepi_autotune"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ge.library()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert ge.version() == 110


def _plan_status(M, N, K, dtype=0, epi=1, flags=0, tile=-1):
    lib = ge.library()
    h = ctypes.c_void_p()
    st = lib.gemmepi_plan_tiled(ctypes.byref(h), M, N, K, dtype, epi, flags, tile)
    if st == 0:
        assert lib.gemmepi_plan_destroy(h) == 0
    return st


def test_plan_validation():
    assert _plan_status(64, 64, 64) == ge.OK
    assert _plan_status(0, 64, 64) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, -1, 64) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, 64, 1 << 31) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, 64, 64, dtype=2) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, 64, 64, epi=10) == ge.ERR_INVALID_VALUE
    for epi in range(10):
        assert _plan_status(64, 64, 64, epi=epi) == ge.OK, epi
    assert _plan_status(64, 64, 64, epi=-1) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, 64, 64, flags=1 << 9) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, 64, 64, tile=ge.num_tiles()) == ge.ERR_INVALID_VALUE
    assert _plan_status(64, 64, 60) == ge.ERR_MISALIGNED          # K % 8
    assert "K=60" in ge.last_error()
    assert _plan_status(64, 60, 64) == ge.ERR_MISALIGNED          # N % 8 without B_TRANS
    assert "N=60" in ge.last_error()
    assert _plan_status(64, 60, 64, flags=ge.FLAG_B_TRANS) == ge.OK
    # 32-bit buffer offsets: 256 rows of K-contiguous operand, or 128 k rows
    # (the deepest slab, tile 9) of B stored [K,N], must span less than 2 GiB
    assert _plan_status(64, 64, 1 << 22) == ge.ERR_UNSUPPORTED
    assert _plan_status(64, 64, (1 << 22) - 8) == ge.OK
    assert _plan_status(64, 1 << 23, 64) == ge.ERR_UNSUPPORTED
    assert "leading dimension" in ge.last_error()
    assert _plan_status(64, (1 << 23) - 8, 64) == ge.OK
    assert _plan_status(64, 1 << 23, 64, flags=ge.FLAG_B_TRANS) == ge.OK
    lib = ge.library()
    assert lib.gemmepi_plan(None, 1, 1, 8, 0, 0, 0) == ge.ERR_INVALID_VALUE


def test_plan_errors_raise_with_detail():
    with pytest.raises(ge.GemmEpiError) as e:
        ge.plan(64, 64, 60)
    assert e.value.status == ge.ERR_MISALIGNED
    assert "multiple of 8" in str(e.value)


def test_plan_cache_and_refcount():
    p1 = ge.plan(128, 256, 64, "f16", "RELU_AUX_BIAS", 0)
    p2 = ge.plan(128, 256, 64, "f16", "RELU_AUX_BIAS", 0)
    assert p1._h.value == p2._h.value          # same cache entry
    p3 = ge.plan(128, 256, 64, "bf16", "RELU_AUX_BIAS", 0)
    assert p3._h.value != p1._h.value
    p1.destroy()
    assert "path=gemm" in p2.info()            # still alive through p2's reference
    p2.destroy()
    lib = ge.library()
    assert lib.gemmepi_plan_destroy(ctypes.c_void_p(p3._h.value)) == ge.OK
    p3._h = None
    assert lib.gemmepi_plan_destroy(None) == ge.ERR_INVALID_VALUE


def test_plan_paths_and_tiles():
    with ge.plan(4, 4096, 4096, "f16", "GELU_BIAS", ge.FLAG_B_TRANS | ge.FLAG_BIAS_PER_COL) as p:
        assert "path=decode" in p.info()
    # the decode kernel by token count and weight shape
    for (M, N, K, kind) in ((1, 4096, 4096, "rowwave"), (1, 4096, 11008, "rowstream"),
                            (3, 4096, 4096, "rowstream"), (4, 4096, 4096, "mfma"),
                            (4, 11008, 4096, "rowstream"), (4, 4096, 11008, "rowstream"),
                            (5, 11008, 4096, "mfma"), (16, 4096, 4096, "mfma")):
        with ge.plan(M, N, K, "f16", "GELU_BIAS", ge.FLAG_B_TRANS | ge.FLAG_BIAS_PER_COL) as p:
            assert f"kernel={kind} " in p.info(), (M, N, K, p.info())
    with ge.plan(4, 4096, 4096, "f16", "GELU_BIAS", ge.FLAG_B_TRANS | ge.FLAG_NO_DECODE) as p:
        assert "path=gemm" in p.info()
    with ge.plan(4, 4096, 4096, "f16", "GELU_BIAS", 0) as p:   # B not transposed: no decode
        assert "path=gemm" in p.info()
    with ge.plan(65536, 8192, 16384, "f16", "RELU_AUX_BIAS", 0) as p:
        assert "tile=256x256" in p.info() and "raster=chip16x16" in p.info()
    for t in range(ge.num_tiles()):
        name = ge.tile_name(t)
        assert re.match(r"\d+x\d+x\d+_w\dx\d", name)
        with ge.plan(1000, 1000, 1000, "bf16", "BIAS", 0, tile=t) as p:
            assert name in p.info()
    assert ge.tile_name(ge.num_tiles()) is None
    assert ge.tile_name(-1) is None


def test_aux_sizes():
    assert ge.aux_ld_words(1) == 4
    assert ge.aux_ld_words(128) == 4
    assert ge.aux_ld_words(129) == 8
    assert ge.aux_ld_words(8192) == 256
    assert ge.aux_bytes(65536, 8192) == 64 << 20
    assert ge.aux_bytes(8192, 4096) == 4 << 20
    assert ge.aux_ld_words(0) == 0 and ge.aux_bytes(0, 5) == 0


def test_status_strings():
    assert ge.status_string(ge.OK) == "GEMMEPI_OK"
    assert ge.status_string(ge.ERR_HIP) == "GEMMEPI_ERR_HIP"
    assert ge.status_string(99) == "unknown status"


def test_execute_rejects_bad_pointers_before_any_hip_call():
    lib = ge.library()
    with ge.plan(64, 64, 64, "f16", "RELU_AUX_BIAS", 0) as p:
        h = p._h
        # null A
        assert lib.gemmepi_execute(h, None, 4096, 4096, 4096, 4096, None) == ge.ERR_INVALID_VALUE
        # missing bias for a BIAS epilogue
        assert lib.gemmepi_execute(h, 4096, 4096, None, 4096, 4096, None) == ge.ERR_INVALID_VALUE
        # missing aux for RELU_AUX_BIAS
        assert lib.gemmepi_execute(h, 4096, 4096, 4096, None, 4096, None) == ge.ERR_INVALID_VALUE
        # misaligned A
        assert lib.gemmepi_execute(h, 4098, 4096, 4096, 4096, 4096, None) == ge.ERR_MISALIGNED
        # misaligned aux
        assert lib.gemmepi_execute(h, 4096, 4096, 4096, 4100, 4096, None) == ge.ERR_MISALIGNED
    for epi in ("DRELU_BGRAD", "DGELU_BGRAD"):
        with ge.plan(64, 64, 64, "f16", epi, 0) as p:
            # bgrad must be 4-byte aligned
            assert lib.gemmepi_execute(p._h, 4096, 4096, 4098, 4096, 4096, None) == ge.ERR_MISALIGNED
            # the saved mask or z is required
            assert lib.gemmepi_execute(p._h, 4096, 4096, 4096, None, 4096, None) == \
                ge.ERR_INVALID_VALUE
    with ge.plan(64, 64, 64, "f16", "GELU_AUX_BIAS", 0) as p:
        # z output: required, 16-byte aligned
        assert lib.gemmepi_execute(p._h, 4096, 4096, 4096, None, 4096, None) == ge.ERR_INVALID_VALUE
        assert lib.gemmepi_execute(p._h, 4096, 4096, 4096, 4104, 4096, None) == ge.ERR_MISALIGNED
    assert lib.gemmepi_execute(None, 4096, 4096, 4096, 4096, 4096, None) == ge.ERR_INVALID_VALUE
    assert lib.gemmepi_execute_noalloc(None, 4096, 4096, 4096, 4096, 4096, None) == \
        ge.ERR_INVALID_VALUE


def test_measurement_helper_is_outside_the_gemm_library():
    """The stream-read reference and the MFMA loop of the benchmark live in
    their own library; they validate their arguments before any HIP call."""
    import bench
    assert not hasattr(ge.library(), "gemmepi_stream_read")
    m = bench.measure_library()
    assert m.gemmepi_measure_stream_read(None, 4096, 4096, 512, 16, 0, None) == 1
    assert m.gemmepi_measure_stream_read(4096, 0, 4096, 512, 16, 0, None) == 1
    assert m.gemmepi_measure_stream_read(4100, 4096, 4096, 512, 16, 0, None) == 1
    assert m.gemmepi_measure_stream_read(4096, 4096, 4096, 384, 16, 0, None) == 1
    assert m.gemmepi_measure_stream_read(4096, 4096, 4096, 512, 12, 0, None) == 1
    # the MFMA loop: operands of the 8 waves (96 KiB), grid and round limits
    assert m.gemmepi_measure_mfma_loop(None, 98304, 4096, 1, 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98303, 4096, 1, 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4104, 98304, 4096, 1, 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98304, None, 1, 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98304, 4096, 0, 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98304, 4096, 65536, 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98304, 4096, 1, 0, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98304, 4096, 1, (1 << 24) + 1, 0, None) == 1
    assert m.gemmepi_measure_mfma_loop(4096, 98304, 4096, 1, 1, 2, None) == 1


def test_binding_checks_tensor_arguments():
    torch = pytest.importorskip("torch")
    with ge.plan(8, 16, 8, "f16", "BIAS", 0) as p:
        A = torch.zeros(8, 8, dtype=torch.float16)
        B = torch.zeros(8, 16, dtype=torch.float16)
        out = torch.zeros(8, 16, dtype=torch.float16)
        bias = torch.zeros(8, dtype=torch.float16)
        with pytest.raises(ValueError, match="needs GPU"):
            p.execute(A, B, bias, None, out)
        with pytest.raises(TypeError):
            p.execute(A.float(), B, bias, None, out)
        with pytest.raises(ValueError, match="elements"):
            p.execute(A, B, torch.zeros(16, dtype=torch.float16), None, out)


def test_no_oracle_in_the_product_path():
    """The package (binding and sources) never imports or names the oracle."""
    pkg = os.path.join(ROOT, "activation_epilogue_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f


def test_norm_entry_point_validation():
    """execute and execute_norm reject each other's plans, and execute_norm
    checks its pointers and eps before any HIP call."""
    lib = ge.library()
    # (mean, rstd) and the row sums (32 M bytes), a status word and one
    # counter per 64 rows, rounded up to 16 bytes
    assert ge.norm_stats_bytes(1000) == 32000 + 4 * (1 + 16) + 12
    assert ge.norm_stats_bytes(64) == 2048 + 16 and ge.norm_stats_bytes(0) == 0
    assert all(ge.norm_stats_bytes(m) % 16 == 0 for m in range(1, 300))
    with ge.plan(64, 64, 64, "f16", "BIAS_RES_LAYERNORM", ge.FLAG_B_TRANS) as p:
        assert "path=gemm" in p.info()          # never the decode kernel
        h = p._h
        assert lib.gemmepi_execute(h, 4096, 4096, 4096, 4096, 4096, None) == ge.ERR_INVALID_VALUE
        ok = dict(A=4096, B=4096, bias=4096, res=4096, gamma=4096, beta=4096, stats=4096, out=4096)

        def run(eps=1e-5, **kw):
            a = dict(ok, **kw)
            return lib.gemmepi_execute_norm(h, a["A"], a["B"], a["bias"], a["res"], a["gamma"],
                                            a["beta"], eps, a["stats"], a["out"], None)
        assert run(gamma=None) == ge.ERR_INVALID_VALUE
        assert run(stats=None) == ge.ERR_INVALID_VALUE
        assert run(eps=0.0) == ge.ERR_INVALID_VALUE
        assert run(eps=-1.0) == ge.ERR_INVALID_VALUE
        assert run(eps=float("inf")) == ge.ERR_INVALID_VALUE
        assert run(eps=float("nan")) == ge.ERR_INVALID_VALUE
        assert run(res=4104) == ge.ERR_MISALIGNED
        assert run(stats=4100) == ge.ERR_MISALIGNED
        assert run(gamma=4097) == ge.ERR_MISALIGNED
    with ge.plan(4, 64, 64, "f16", "BIAS_RES_RMSNORM", ge.FLAG_B_TRANS) as p:
        assert "path=gemm" in p.info()          # M <= 16 still takes the tiled GEMM
    with ge.plan(64, 64, 64, "f16", "BIAS", 0) as p:
        assert lib.gemmepi_execute_norm(p._h, 4096, 4096, 4096, 4096, 4096, 4096, 1e-5, 4096, 4096,
                                        None) == ge.ERR_INVALID_VALUE


def test_autotune_validation_before_any_hip_call():
    lib = ge.library()
    assert lib.gemmepi_autotune(None, 4096, 4096, 4096, 4096, 4096, 3, None, None) == ge.ERR_INVALID_VALUE
    with ge.plan(512, 512, 512, "f16", "BIAS", 0) as p:
        assert lib.gemmepi_autotune(p._h, 4096, 4096, 4096, 4096, 4096, 0, None, None) == ge.ERR_INVALID_VALUE
    with ge.plan(4, 4096, 4096, "f16", "GELU_BIAS", ge.FLAG_B_TRANS | ge.FLAG_BIAS_PER_COL) as p:
        assert "path=decode" in p.info()
        assert lib.gemmepi_autotune(p._h, 4096, 4096, 4096, 4096, 4096, 3, None, None) == ge.ERR_UNSUPPORTED
    with ge.plan(512, 512, 512, "f16", "BIAS_RES_LAYERNORM", 0) as p:
        assert lib.gemmepi_autotune(p._h, 4096, 4096, 4096, 4096, 4096, 3, None, None) == ge.ERR_UNSUPPORTED
    with ge.plan(512, 512, 512, "f16", "BIAS", 0, tile=2) as p:
        assert lib.gemmepi_autotune(p._h, 4096, 4096, 4096, 4096, 4096, 3, None, None) == ge.ERR_INVALID_VALUE


def test_tune_cache_file_is_read_by_a_new_process(tmp_path):
    """The first plan() of a process reads GEMMEPI_TUNE_CACHE: a valid line
    sets the tile of its key; malformed lines and unknown tiles are ignored."""
    import subprocess
    import sys
    f = tmp_path / "tune.txt"
    f.write_text("gemmepi-tune-v1 1000 1000 1000 0 1 0 4\n"      # f16 BIAS, no flags -> tile 4
                 "garbage line\n"
                 "gemmepi-tune-v1 2000 2000 2000 0 1 0 99\n"     # tile out of range
                 "gemmepi-tune-v2 3000 3000 3000 0 1 0 4\n")     # unknown version
    code = ("import activation_epilogue_gemm_amd as ge\n"
            "for m in (1000, 2000, 3000):\n"
            "    with ge.plan(m, m, m, 'f16', 'BIAS', 0) as p: print(p.info())\n")
    env = dict(os.environ, GEMMEPI_TUNE_CACHE=str(f), PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    lines = r.stdout.strip().splitlines()
    assert ge.tile_name(4) in lines[0] and "tuned" in lines[0]
    assert "tuned" not in lines[1] and "tuned" not in lines[2]


def _plan_split(M, N, K, epi=1, flags=0, tile=-1, splits=2):
    lib = ge.library()
    h = ctypes.c_void_p()
    st = lib.gemmepi_plan_split(ctypes.byref(h), M, N, K, 0, epi, flags, tile, splits)
    return st, h


def test_split_plan_validation_and_workspace_size():
    lib = ge.library()
    for bad in (-1, 65):
        st, _ = _plan_split(512, 512, 4096, splits=bad)
        assert st == ge.ERR_INVALID_VALUE
    st, _ = _plan_split(512, 512, 4096, epi=6, splits=2)        # norm epilogue
    assert st == ge.ERR_UNSUPPORTED
    # splits = 1 and unsplit plans need no workspace
    with ge.plan(512, 512, 4096, "f16", "BIAS", 0, tile=3, splits=1) as p:
        assert p.workspace_bytes() == 0 and "splits=" not in p.info()
    with ge.plan(512, 512, 4096, "f16", "BIAS", 0) as p:
        assert p.workspace_bytes() == 0
    assert lib.gemmepi_workspace_bytes(None) == 0
    # 128x128 tiles: 4 x 4 tiles, K = 4096 -> 64 slabs; 3 splits of 22, 22, 20
    with ge.plan(512, 512, 4096, "f16", "BIAS", 0, tile=3, splits=3) as p:
        assert "splits=3 kt_split=22" in p.info(), p.info()
        assert p.workspace_bytes() == 256 + 16 * 3 * 128 * 128 * 4
    # more splits than k slabs: one slab per range
    with ge.plan(64, 64, 72, "f16", "BIAS", 0, tile=5, splits=64) as p:
        assert "splits=2 kt_split=1" in p.info(), p.info()
    # a split request disables the decode kernel; the norms ignore the flag
    with ge.plan(4, 4096, 4096, "f16", "GELU_BIAS", ge.FLAG_B_TRANS | ge.FLAG_BIAS_PER_COL,
                 splits=2) as p:
        assert "path=gemm" in p.info()
    with ge.plan(512, 512, 4096, "f16", "BIAS_RES_RMSNORM", ge.FLAG_SPLIT_K) as p:
        assert "splits=" not in p.info()


def test_planner_prefers_64_wide_slabs_when_b_is_transposed():
    """With B stored [N,K] a 32-wide k slab fetches 64-byte row segments of
    both operands (measured 0.83x on the 65536 x 8192 x 16384 shape), so the
    planner takes the tile that fetches A in 64-wide slabs there."""
    with ge.plan(65536, 8192, 16384, "f16", "RELU_AUX_BIAS", ge.FLAG_B_TRANS) as p:
        assert f"tile={ge.tile_name(8)}" in p.info(), p.info()   # A in 64-wide slabs
    # without schedule 2 (explicit tiles only), B [N,K] prefers 64-wide slabs
    assert "_p2_" in ge.tile_name(8)


def test_split_flag_chooses_only_for_wave_quantised_shapes():
    def info(M, N, K, bt):
        f = ge.FLAG_SPLIT_K | (ge.FLAG_B_TRANS if bt else 0)
        with ge.plan(M, N, K, "f16", "BIAS", f) as p:
            return p.info(), p.workspace_bytes()
    i, ws = info(512, 4096, 11008, True)       # 512-token FFN down-projection
    assert "splits=" in i and ws > 0, i
    # 2048-token FFN down-projection: 128 tiles of 256 x 256, split twice
    i, ws = info(2048, 4096, 11008, True)
    assert f"tile={ge.tile_name(8)}" in i and "splits=2" in i and ws > 0, i
    for M, N, K, bt in ((65536, 8192, 16384, False), (4096, 4096, 4096, True)):
        i, ws = info(M, N, K, bt)
        assert "splits=" not in i and ws == 0, i


def test_split_execute_validation():
    lib = ge.library()
    with ge.plan(512, 512, 4096, "f16", "BIAS", 0, tile=3, splits=2) as p:
        need = p.workspace_bytes()
        # gemmepi_execute refuses a plan that needs a workspace
        assert lib.gemmepi_execute(p._h, 4096, 4096, 4096, None, 4096, None) == ge.ERR_INVALID_VALUE
        assert "workspace" in ge.last_error()
        ex = lib.gemmepi_execute_ws
        assert ex(p._h, 4096, 4096, 4096, None, 4096, None, need, None) == ge.ERR_INVALID_VALUE
        assert ex(p._h, 4096, 4096, 4096, None, 4096, 1 << 20, need - 1, None) == \
            ge.ERR_INVALID_VALUE
        assert ex(p._h, 4096, 4096, 4096, None, 4096, (1 << 20) + 16, need, None) == \
            ge.ERR_MISALIGNED
    with ge.plan(512, 512, 4096, "f16", "BIAS", 0, splits=2) as p:
        assert "splits=2" in p.info()
        assert lib.gemmepi_autotune(p._h, 4096, 4096, 4096, None, 4096, 3, None, None) == \
            ge.ERR_UNSUPPORTED


def test_plan_cache_is_thread_safe():
    """Eight threads plan and destroy overlapping keys at once (ctypes drops
    the GIL during each call); every call succeeds and the cache is left
    usable, with each key's entry freed or shared consistently."""
    import random
    import threading
    lib = ge.library()
    shapes = [(64, 64, 64), (128, 256, 512), (1000, 1000, 1000), (1, 4096, 4096), (2048, 11008, 4096)]
    failures = []

    def worker(seed):
        rng = random.Random(seed)
        held = []
        for _ in range(400):
            M, N, K = rng.choice(shapes)
            h = ctypes.c_void_p()
            st = lib.gemmepi_plan(ctypes.byref(h), M, N, K, 0, 1, rng.choice([0, 1]))
            if st != ge.OK:
                failures.append(("plan", st))
                continue
            held.append(h)
            if len(held) > 4:
                st = lib.gemmepi_plan_destroy(held.pop(rng.randrange(len(held))))
                if st != ge.OK:
                    failures.append(("destroy", st))
        for h in held:
            if lib.gemmepi_plan_destroy(h) != ge.OK:
                failures.append(("destroy", -1))

    threads = [threading.Thread(target=worker, args=(s,)) for s in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert failures == []
    for M, N, K in shapes:
        p = ge.plan(M, N, K, "f16", "BIAS", 0)
        assert "M=%d" % M in p.info()
        p.destroy()


def test_last_error_is_per_thread():
    """A failing call's detail stays with its own thread."""
    import threading
    lib = ge.library()
    seen = {}

    def bad():
        h = ctypes.c_void_p()
        seen["bad_status"] = lib.gemmepi_plan(ctypes.byref(h), 64, 64, 7, 0, 1, 0)
        seen["bad"] = ge.last_error()

    def good():
        h = ctypes.c_void_p()
        seen["good_status"] = lib.gemmepi_plan(ctypes.byref(h), 64, 64, 64, 0, 1, 0)
        seen["good"] = ge.last_error()
        lib.gemmepi_plan_destroy(h)

    for fn in (bad, good):
        t = threading.Thread(target=fn)
        t.start()
        t.join()
    assert seen["bad_status"] == ge.ERR_MISALIGNED and "K=7" in seen["bad"]
    assert seen["good_status"] == ge.OK and "K=7" not in seen["good"]
