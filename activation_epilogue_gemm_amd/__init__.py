"""Python binding of libgemmepi (fused-epilogue GEMM for MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgemmepi.so``.  Tensors are passed as device pointers
(torch tensors, or raw integer addresses) together with the HIP stream;
PyTorch supplies device memory and streams, nothing else.

The names follow the C ABI in ``include/gemmepi.h``:

    p = plan(M, N, K, "f16", "RELU_AUX_BIAS", flags)     # gemmepi_plan
    p.execute(A, B, bias, aux, out)                       # gemmepi_execute
                                      # (gemmepi_execute_ws for split-K plans)
    p.info()                                              # gemmepi_plan_info
    p.destroy()  /  with plan(...) as p: ...              # gemmepi_plan_destroy

The library is loaded from this package directory; importing works without
it, but any call raises :class:`GemmEpiLibraryMissing` if it was not built
(``python -c "import __graft_entry__ as g; g.build()"``).  There is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Union

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemmepi.so")

# ---- enums (include/gemmepi.h) ---------------------------------------------
OK = 0
ERR_INVALID_VALUE = 1
ERR_MISALIGNED = 2
ERR_UNSUPPORTED = 3
ERR_DEVICE = 4
ERR_HIP = 5
ERR_NO_MEMORY = 6

DTYPES = {"f16": 0, "bf16": 1}
EPILOGUES = {"DEFAULT": 0, "BIAS": 1, "RELU_BIAS": 2, "RELU_AUX_BIAS": 3, "GELU_BIAS": 4,
             "DRELU_BGRAD": 5, "BIAS_RES_RMSNORM": 6, "BIAS_RES_LAYERNORM": 7,
             "GELU_AUX_BIAS": 8, "DGELU_BGRAD": 9}
BGRAD_EPILOGUES = ("DRELU_BGRAD", "DGELU_BGRAD")
NORM_EPILOGUES = ("BIAS_RES_RMSNORM", "BIAS_RES_LAYERNORM")

FLAG_B_TRANS = 1 << 0
FLAG_BIAS_PER_COL = 1 << 1
FLAG_UNFUSED = 1 << 2
FLAG_VALIDATE = 1 << 3
FLAG_NO_DECODE = 1 << 4
FLAG_SPLIT_K = 1 << 5
FLAG_STAGE_B = 1 << 6
FLAG_NORM_TWO_PASS = 1 << 7


class GemmEpiError(RuntimeError):
    """A libgemmepi call returned a non-OK status."""

    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {detail}")


class GemmEpiLibraryMissing(ImportError):
    pass


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise GemmEpiLibraryMissing(
            f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, u32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32
    lib.gemmepi_plan.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ctypes.c_int, ctypes.c_int, u32]
    lib.gemmepi_plan.restype = ctypes.c_int
    lib.gemmepi_plan_tiled.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ctypes.c_int,
                                       ctypes.c_int, u32, i32]
    lib.gemmepi_plan_tiled.restype = ctypes.c_int
    lib.gemmepi_execute.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.gemmepi_execute.restype = ctypes.c_int
    lib.gemmepi_plan_split.argtypes = [ctypes.POINTER(vp), i64, i64, i64, ctypes.c_int,
                                       ctypes.c_int, u32, i32, i32]
    lib.gemmepi_plan_split.restype = ctypes.c_int
    lib.gemmepi_workspace_bytes.argtypes = [vp]
    lib.gemmepi_workspace_bytes.restype = ctypes.c_size_t
    lib.gemmepi_execute_ws.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.gemmepi_execute_ws.restype = ctypes.c_int
    lib.gemmepi_plan_destroy.argtypes = [vp]
    lib.gemmepi_plan_destroy.restype = ctypes.c_int
    lib.gemmepi_plan_info.argtypes = [vp, ctypes.c_char_p, ctypes.c_size_t]
    lib.gemmepi_plan_info.restype = ctypes.c_int
    lib.gemmepi_num_tiles.argtypes = []
    lib.gemmepi_num_tiles.restype = i32
    lib.gemmepi_tile_name.argtypes = [i32]
    lib.gemmepi_tile_name.restype = ctypes.c_char_p
    lib.gemmepi_aux_ld_words.argtypes = [i64]
    lib.gemmepi_aux_ld_words.restype = i64
    lib.gemmepi_aux_bytes.argtypes = [i64, i64]
    lib.gemmepi_aux_bytes.restype = ctypes.c_size_t
    lib.gemmepi_status_string.argtypes = [ctypes.c_int]
    lib.gemmepi_status_string.restype = ctypes.c_char_p
    lib.gemmepi_last_error.argtypes = []
    lib.gemmepi_last_error.restype = ctypes.c_char_p
    lib.gemmepi_version.argtypes = []
    lib.gemmepi_version.restype = i32
    lib.gemmepi_execute_norm.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.gemmepi_execute_norm.restype = ctypes.c_int
    lib.gemmepi_autotune.argtypes = [vp, vp, vp, vp, vp, vp, i32, ctypes.POINTER(ctypes.c_float), vp]
    lib.gemmepi_autotune.restype = ctypes.c_int
    lib.gemmepi_execute_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.gemmepi_execute_noalloc.restype = ctypes.c_int
    lib.gemmepi_noalloc_scratch_bytes.argtypes = []
    lib.gemmepi_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.gemmepi_norm_stats_bytes.argtypes = [i64]
    lib.gemmepi_norm_stats_bytes.restype = ctypes.c_size_t
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (raises GemmEpiLibraryMissing if not built)."""
    return _load()


def status_string(status: int) -> str:
    return _load().gemmepi_status_string(int(status)).decode()


def last_error() -> str:
    return _load().gemmepi_last_error().decode()


def version() -> int:
    return int(_load().gemmepi_version())


def num_tiles() -> int:
    return int(_load().gemmepi_num_tiles())


def tile_name(tile_id: int) -> Optional[str]:
    r = _load().gemmepi_tile_name(int(tile_id))
    return None if r is None else r.decode()


def aux_ld_words(N: int) -> int:
    return int(_load().gemmepi_aux_ld_words(int(N)))


def aux_bytes(M: int, N: int) -> int:
    return int(_load().gemmepi_aux_bytes(int(M), int(N)))


def _check(status: int, where: str):
    if status != OK:
        raise GemmEpiError(status, where, last_error())


Pointer = Union[int, None, "torch.Tensor"]  # noqa: F821


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream_handle(stream, *tensors) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else int(stream.cuda_stream)
    for t in tensors:
        if t is not None and not isinstance(t, int) and getattr(t, "is_cuda", False):
            import torch
            return int(torch.cuda.current_stream(t.device).cuda_stream)
    return None


class Plan:
    """A cached plan (gemmepi_plan_t).  Use as a context manager or call
    :meth:`destroy`; plans for the same arguments share one cache entry."""

    def __init__(self, M: int, N: int, K: int, dtype: str = "f16", epilogue: str = "BIAS",
                 flags: int = 0, tile: int = -1, splits: Optional[int] = None):
        lib = _load()
        self.M, self.N, self.K = int(M), int(N), int(K)
        self.dtype, self.epilogue, self.flags, self.tile = dtype, epilogue, int(flags), int(tile)
        self._ws = None  # workspace allocated here when execute() is given none
        if dtype not in DTYPES:
            raise ValueError(f"dtype must be one of {list(DTYPES)}")
        if epilogue not in EPILOGUES:
            raise ValueError(f"epilogue must be one of {list(EPILOGUES)}")
        h = ctypes.c_void_p()
        if splits is not None:
            st = lib.gemmepi_plan_split(ctypes.byref(h), self.M, self.N, self.K, DTYPES[dtype],
                                        EPILOGUES[epilogue], self.flags, self.tile, int(splits))
        elif tile < 0:
            st = lib.gemmepi_plan(ctypes.byref(h), self.M, self.N, self.K, DTYPES[dtype],
                                  EPILOGUES[epilogue], self.flags)
        else:
            st = lib.gemmepi_plan_tiled(ctypes.byref(h), self.M, self.N, self.K, DTYPES[dtype],
                                        EPILOGUES[epilogue], self.flags, self.tile)
        _check(st, "gemmepi_plan")
        self._h = h

    # ---- the C calls ----------------------------------------------------
    def execute(self, A: Pointer, B: Pointer, bias: Pointer = None, aux: Pointer = None,
                out: Pointer = None, stream=None, check: bool = True, workspace: Pointer = None,
                workspace_nbytes: Optional[int] = None) -> None:
        """Enqueue one execution (gemmepi_execute, or gemmepi_execute_ws when
        the plan splits K or a workspace is given).  Tensor arguments are
        checked for dtype, shape, contiguity and device first (``check``);
        raw integer pointers are passed through unchecked.  A split-K plan
        given no workspace uses a zeroed one that the Plan allocates once."""
        if self._h is None:
            raise ValueError("plan destroyed")
        if check:
            self._check_tensors(A, B, bias, aux, out)
        need = self.workspace_bytes()
        if need == 0 and workspace is None:
            st = _load().gemmepi_execute(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(aux),
                                         _ptr(out), _stream_handle(stream, A, B, out))
            _check(st, "gemmepi_execute")
            return
        if workspace is None:
            workspace = self._own_workspace(need, out)
        nbytes = workspace_nbytes if workspace_nbytes is not None else (
            need if isinstance(workspace, int) else workspace.numel() * workspace.element_size())
        st = _load().gemmepi_execute_ws(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(aux),
                                        _ptr(out), _ptr(workspace), int(nbytes),
                                        _stream_handle(stream, A, B, out))
        _check(st, "gemmepi_execute_ws")

    def execute_noalloc(self, A: Pointer, B: Pointer, bias: Pointer = None, aux: Pointer = None,
                        out: Pointer = None, stream=None, check: bool = True) -> None:
        """Enqueue one execution through gemmepi_execute_noalloc: a split-K
        plan uses the library's static device scratch instead of a
        workspace, so nothing is allocated.  Calls that overlap on one device
        race on that scratch."""
        if self._h is None:
            raise ValueError("plan destroyed")
        if check:
            self._check_tensors(A, B, bias, aux, out)
        st = _load().gemmepi_execute_noalloc(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(aux),
                                             _ptr(out), _stream_handle(stream, A, B, out))
        _check(st, "gemmepi_execute_noalloc")

    def workspace_bytes(self) -> int:
        """gemmepi_workspace_bytes: device workspace this plan needs (0 unless
        it splits K)."""
        return int(_load().gemmepi_workspace_bytes(self._h))

    def _own_workspace(self, need: int, like):
        """A zeroed workspace kept with the plan (memory plumbing only).  The
        zero fill runs on torch's current stream, which need not be the
        stream the execution is enqueued on, so the fill is waited for here
        (once per allocation): the arrival counters are zero before any
        kernel on any stream can read them."""
        if self._ws is None or self._ws.numel() < need:
            import torch
            dev = like.device if hasattr(like, "device") else torch.device("cuda")
            ws = torch.zeros(need, dtype=torch.uint8, device=dev)
            torch.cuda.current_stream(dev).synchronize()
            self._ws = ws
        return self._ws

    def execute_norm(self, A: Pointer, B: Pointer, bias: Pointer, residual: Pointer,
                     gamma: Pointer, beta: Pointer, eps: float, stats: Pointer, out: Pointer,
                     stream=None, check: bool = True) -> None:
        """Enqueue one GEMM + bias + residual + row-norm execution
        (gemmepi_execute_norm).  stats is an fp64 tensor of
        norm_stats_bytes(M) / 8 elements (norm_stats_buffer); on return its
        first 2 M elements are (mean, rstd) per row."""
        if self._h is None:
            raise ValueError("plan destroyed")
        if check:
            self._check_norm_tensors(A, B, bias, residual, gamma, beta, stats, out)
        st = _load().gemmepi_execute_norm(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(residual),
                                          _ptr(gamma), _ptr(beta), float(eps), _ptr(stats),
                                          _ptr(out), _stream_handle(stream, A, B, out))
        _check(st, "gemmepi_execute_norm")

    def autotune(self, A: Pointer, B: Pointer, bias: Pointer = None, aux: Pointer = None,
                 out: Pointer = None, reps: int = 5, stream=None, check: bool = True) -> dict:
        """gemmepi_autotune: time every tile on these operands, switch the plan
        to the fastest; returns {tile name: ms per execution}."""
        if self._h is None:
            raise ValueError("plan destroyed")
        if check:
            self._check_tensors(A, B, bias, aux, out)
        n = num_tiles()
        times = (ctypes.c_float * n)()
        st = _load().gemmepi_autotune(self._h, _ptr(A), _ptr(B), _ptr(bias), _ptr(aux), _ptr(out),
                                      int(reps), times, _stream_handle(stream, A, B, out))
        _check(st, "gemmepi_autotune")
        return {tile_name(t): float(times[t]) for t in range(n)}

    def info(self) -> str:
        buf = ctypes.create_string_buffer(512)
        _check(_load().gemmepi_plan_info(self._h, buf, len(buf)), "gemmepi_plan_info")
        return buf.value.decode()

    def destroy(self) -> None:
        if self._h is not None:
            _check(_load().gemmepi_plan_destroy(self._h), "gemmepi_plan_destroy")
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()

    def __del__(self):
        try:
            if self._h is not None and _lib is not None:
                _lib.gemmepi_plan_destroy(self._h)
                self._h = None
        except Exception:
            pass

    # ---- torch argument checks (host side, before the C call) ------------
    def _check_tensors(self, A, B, bias, aux, out):
        try:
            import torch
        except ImportError:  # pragma: no cover
            return
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[self.dtype]
        M, N, K = self.M, self.N, self.K
        epi = self.epilogue
        dev = None

        def chk(t, name, dtype, numel):
            nonlocal dev
            if t is None or isinstance(t, int):
                return
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name}: expected a torch.Tensor or an int pointer")
            if t.dtype != dtype:
                raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
            if not t.is_contiguous():
                raise ValueError(f"{name}: must be contiguous")
            if t.numel() != numel:
                raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name}: on {t.device}, other operands on {dev}")

        chk(A, "A", tdt, M * K)
        chk(B, "B", tdt, N * K)
        chk(out, "out", tdt, M * N)
        if epi in BGRAD_EPILOGUES:
            chk(bias, "bias (bgrad)", torch.float32, N)
        elif epi != "DEFAULT":
            chk(bias, "bias", tdt, N if self.flags & FLAG_BIAS_PER_COL else M)
        if epi in ("RELU_AUX_BIAS", "DRELU_BGRAD") and aux is not None and not isinstance(aux, int):
            word_types = {torch.int32} | ({torch.uint32} if hasattr(torch, "uint32") else set())
            if aux.dtype not in word_types:
                raise TypeError("aux: expected int32/uint32 words")
            if aux.numel() != M * aux_ld_words(N):
                raise ValueError(f"aux: {aux.numel()} words, expected {M * aux_ld_words(N)}")
            if not aux.is_contiguous():
                raise ValueError("aux: must be contiguous")
        if epi in ("GELU_AUX_BIAS", "DGELU_BGRAD"):
            chk(aux, "aux (pre-activation z)", tdt, M * N)
        if dev is not None and dev.type != "cuda":
            raise ValueError(f"operands are on {dev}; libgemmepi needs GPU (HIP) memory")


    def _check_norm_tensors(self, A, B, bias, residual, gamma, beta, stats, out):
        try:
            import torch
        except ImportError:  # pragma: no cover
            return
        tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[self.dtype]
        M, N, K = self.M, self.N, self.K
        devs = set()
        for t, name, dtype, numel in ((A, "A", tdt, M * K), (B, "B", tdt, N * K),
                                      (out, "out", tdt, M * N), (bias, "bias", tdt, N),
                                      (residual, "residual", tdt, M * N), (gamma, "gamma", tdt, N),
                                      (beta, "beta", tdt, N),
                                      (stats, "stats", torch.float64, norm_stats_bytes(M) // 8)):
            if t is None or isinstance(t, int):
                continue
            if not isinstance(t, torch.Tensor):
                raise TypeError(f"{name}: expected a torch.Tensor or an int pointer")
            if t.dtype != dtype:
                raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
            if not t.is_contiguous():
                raise ValueError(f"{name}: must be contiguous")
            if t.numel() != numel:
                raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
            devs.add(t.device)
        if len(devs) > 1:
            raise ValueError(f"operands on several devices: {devs}")
        if devs and next(iter(devs)).type != "cuda":
            raise ValueError("operands are not on the GPU; libgemmepi needs GPU (HIP) memory")


def noalloc_scratch_bytes() -> int:
    """gemmepi_noalloc_scratch_bytes: the per-device static scratch size."""
    return int(_load().gemmepi_noalloc_scratch_bytes())


def norm_stats_bytes(M: int) -> int:
    """gemmepi_norm_stats_bytes: bytes of execute_norm's stats buffer."""
    return int(_load().gemmepi_norm_stats_bytes(M))


def norm_stats_buffer(M: int, device="cuda"):
    """A stats buffer for execute_norm on M rows: an fp64 tensor of
    norm_stats_bytes(M) / 8 elements.  After an execution, mean and rstd of
    row m are elements 2 m and 2 m + 1 (norm_mean_rstd); the 32-bit word
    after them is 1 after a single-pass execution, 0 after two kernels
    (norm_pass_status)."""
    import torch
    return torch.zeros(norm_stats_bytes(M) // 8, dtype=torch.float64, device=device)


def norm_mean_rstd(stats, M: int):
    """The [M, 2] (mean, rstd) view of an execute_norm stats buffer."""
    return stats[: 2 * M].view(M, 2)


def norm_pass_status(stats, M: int) -> int:
    """The status word of an execute_norm stats buffer (copied to the
    host): bit 0 set after a single pass, bit 1 set if a workgroup of it
    stopped waiting for its band of rows."""
    import torch
    return int(stats[4 * M: 4 * M + 1].view(torch.int32)[0].item())


def plan(M: int, N: int, K: int, dtype: str = "f16", epilogue: str = "BIAS", flags: int = 0,
         tile: int = -1, splits: Optional[int] = None) -> Plan:
    """gemmepi_plan / gemmepi_plan_tiled / gemmepi_plan_split (splits given)."""
    return Plan(M, N, K, dtype, epilogue, flags, tile, splits)


def execute(p: Plan, A, B, bias=None, aux=None, out=None, stream=None) -> None:
    """gemmepi_execute."""
    p.execute(A, B, bias, aux, out, stream)


def plan_info(p: Plan) -> str:
    return p.info()


def plan_destroy(p: Plan) -> None:
    p.destroy()
