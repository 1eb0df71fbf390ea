"""Helpers shared by the GPU parity tests: upload seeded cases, run them
through the C ABI (via the Python binding), and compare with the oracle.

Tolerance (per element, y_ref the oracle's unrounded fp64 value):
    |y - y_ref| <= 1e-2 |y_ref| + 2e-3 sqrt(K) max|A| max|B|
with the maxima over the operand tensors actually used.  The ReLU mask is
compared bit-exactly except where |z_ref| < abs_term / 0.99 (there a result
within the tolerance may have the other sign).  bgrad uses the same formula.
The saved GELU pre-activation z is held to the same formula against the
oracle's z.  For DGELU_BGRAD the accumulator's error reaches dZ = acc gelu'(z)
scaled by |gelu'(z)| <= 1.129 (its maximum, at z = sqrt 2), so the absolute
term of dZ and of bgrad is multiplied by that bound.  The unfused sequence
sums dZ values that were rounded to the dtype (once for DRELU, twice for
DGELU: the GEMM's output and the product with gelu').  In fp16 its bgrad is
held to the same formula; in bf16, whose unit roundoff u = 2^-8 is 8 times
fp16's, the formula also gets 2 u sum_m |dZ[m, n]|, the worst-case bound of
that rounding.  The test log reports each bgrad's error against the
tolerance used and, unfused, against that rounding bound.
"""
from __future__ import annotations

import numpy as np

import activation_epilogue_gemm_amd as ge
from oracle import oracle as O


def tile_table():
    """The tiled GEMM's tile configurations, read from the table the kernels
    and the planner are built from (csrc/gemm_tiles.h): one dict per tile."""
    import os
    import re
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "activation_epilogue_gemm_amd", "csrc", "gemm_tiles.h")
    keys = ("id", "bm", "bn", "bk", "wm", "wn", "ns", "sched", "mfma")
    rows = [dict(zip(keys, map(int, m.groups())))
            for m in re.finditer(r"X\(" + r",\s*".join([r"(\d+)"] * 9) + r"\)", open(path).read())]
    assert [r["id"] for r in rows] == list(range(len(rows))), "tile ids must be 0..n-1"
    return rows


NUM_TILES = len(tile_table())


def torch_dtype(dtype: str):
    import torch
    return torch.float16 if dtype == "f16" else torch.bfloat16


def upload_bits(bits: np.ndarray, dtype: str, device="cuda"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device)
    return t.view(torch_dtype(dtype))


def upload_words(words: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(device)


def download_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


BGRAD_EPIS = ("DRELU_BGRAD", "DGELU_BGRAD")
# GELU epilogues: the activation (or its derivative) is a transcendental
# function, so out is compared with the tolerance even for integer inputs
GELU_EPIS = ("GELU_BIAS", "GELU_AUX_BIAS", "DGELU_BGRAD")
GELU_GRAD_MAX = 1.129  # max over z of |Phi(z) + z phi(z)|, attained at z = sqrt 2
GUARD_BITS = 0x7E5A
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


def flags_of(case, extra: int = 0) -> int:
    f = extra
    if case.b_trans:
        f |= ge.FLAG_B_TRANS
    if case.bias_per_col:
        f |= ge.FLAG_BIAS_PER_COL
    return f


class DeviceRun:
    """Device buffers and results of one execution of a GemmCase."""

    def __init__(self, case, flags: int = 0, tile: int = -1, A_dev=None, guard: int = 0,
                 device="cuda", splits=None):
        import torch
        c = case
        self.case = c
        tdt = torch_dtype(c.dtype)
        M, N, K = c.M, c.N, c.K
        if A_dev is not None:
            self.A = A_dev
        elif getattr(c, "A_dev", None) is not None:
            self.A = c.A_dev
        else:
            self.A = upload_bits(c.A, c.dtype, device)
        self.B = c.B_dev if getattr(c, "B_dev", None) is not None else upload_bits(c.B, c.dtype, device)
        self.guard = guard
        # guard bands: poison values around out / aux / bgrad
        self._out_full = torch.full((M * N + 2 * guard,), float("nan"), dtype=tdt, device=device)
        if guard:
            self._out_full.view(torch.int16)[:guard] = GUARD_BITS
            self._out_full.view(torch.int16)[-guard:] = GUARD_BITS
        self.out = self._out_full[guard:guard + M * N].view(M, N)
        self.bias = None
        self.aux = None
        self._aux_full = None
        self._zaux_full = None
        ld = ge.aux_ld_words(N)
        if c.epilogue in BGRAD_EPIS:
            self._bias_full = torch.full((N + 2 * guard,), 1234.5, dtype=torch.float32, device=device)
            self.bias = self._bias_full[guard:guard + N]
            if c.epilogue == "DRELU_BGRAD":
                self.aux = upload_words(c.aux, device)
            else:
                self.aux = upload_bits(c.aux, c.dtype, device).view(M, N)
        else:
            if c.bias is not None:
                self.bias = upload_bits(c.bias, c.dtype, device)
            if c.epilogue == "RELU_AUX_BIAS":
                self._aux_full = torch.full((M * ld + 2 * guard,), -0x2A2A2A2B, dtype=torch.int32,
                                            device=device)
                self.aux = self._aux_full[guard:guard + M * ld].view(M, ld)
            if c.epilogue == "GELU_AUX_BIAS":
                self._zaux_full = torch.full((M * N + 2 * guard,), float("nan"), dtype=tdt,
                                             device=device)
                if guard:
                    self._zaux_full.view(torch.int16)[:guard] = GUARD_BITS
                    self._zaux_full.view(torch.int16)[-guard:] = GUARD_BITS
                self.aux = self._zaux_full[guard:guard + M * N].view(M, N)
        self.plan = ge.plan(M, N, K, c.dtype, c.epilogue, flags_of(c, flags), tile, splits)
        self.info = self.plan.info()

    def run(self, times: int = 1):
        import torch
        for _ in range(times):
            self.plan.execute(self.A, self.B, self.bias, self.aux, self.out)
        torch.cuda.synchronize()
        return self

    def out_bits(self, rows=None) -> np.ndarray:
        if rows is None:
            return download_bits(self.out)
        import torch
        idx = torch.as_tensor(np.asarray(rows), device=self.out.device)
        return download_bits(self.out.index_select(0, idx))

    def aux_words(self, rows=None) -> np.ndarray:
        import torch
        a = self.aux
        if rows is not None:
            a = a.index_select(0, torch.as_tensor(np.asarray(rows), device=a.device))
        return a.cpu().numpy().view(np.uint32)

    def zaux_bits(self, rows=None) -> np.ndarray:
        """GELU_AUX_BIAS: storage bits of the saved pre-activation [M, N]."""
        if rows is None:
            return download_bits(self.aux)
        import torch
        idx = torch.as_tensor(np.asarray(rows), device=self.aux.device)
        return download_bits(self.aux.index_select(0, idx))

    def bgrad(self) -> np.ndarray:
        return self.bias.cpu().numpy()

    def guards_intact(self) -> bool:
        import torch
        g = self.guard
        if not g:
            return True
        ok = bool((self._out_full.view(torch.int16)[:g] == GUARD_BITS).all()) and \
            bool((self._out_full.view(torch.int16)[-g:] == GUARD_BITS).all())
        if self._zaux_full is not None:
            ok &= bool((self._zaux_full.view(torch.int16)[:g] == GUARD_BITS).all())
            ok &= bool((self._zaux_full.view(torch.int16)[-g:] == GUARD_BITS).all())
        if self._aux_full is not None:
            ok &= bool((self._aux_full[:g] == -0x2A2A2A2B).all())
            ok &= bool((self._aux_full[-g:] == -0x2A2A2A2B).all())
        if self.case.epilogue in BGRAD_EPIS:
            ok &= bool((self._bias_full[:g] == 1234.5).all()) and bool((self._bias_full[-g:] == 1234.5).all())
        return ok

    def close(self):
        self.plan.destroy()


def _absmax(host_bits, dev, dtype) -> float:
    if host_bits is not None:
        return float(np.abs(O.decode(host_bits, dtype)).max())
    return float(dev.float().abs().max())


def abs_term(case, A_bits=None) -> float:
    """2e-3 sqrt(K) max|A| max|B| over the operand tensors actually used."""
    amax = _absmax(case.A if A_bits is None else A_bits,
                   getattr(case, "A_dev", None) if A_bits is None else None, case.dtype)
    bmax = _absmax(case.B, getattr(case, "B_dev", None), case.dtype)
    return 2e-3 * np.sqrt(case.K) * amax * bmax


def grad_scale(case) -> float:
    return GELU_GRAD_MAX if case.epilogue == "DGELU_BGRAD" else 1.0


def check_out(case, got_bits: np.ndarray, ref, A_bits=None, label: str = ""):
    """Element-wise tolerance check; returns the max |error| / tolerance."""
    got = O.decode(got_bits, case.dtype)
    want_y = ref.y
    tol = 1e-2 * np.abs(want_y) + grad_scale(case) * abs_term(case, A_bits)
    err = np.abs(got - want_y)
    finite = np.isfinite(got)
    bad = (~finite) | (err > tol)
    if bad.any():
        i = np.argwhere(bad)[:5]
        detail = "; ".join(f"[{r},{c}] got {got[r, c]!r} want {want_y[r, c]!r} tol {tol[r, c]:.3g}"
                           for r, c in i)
        raise AssertionError(f"{label} {case.name}: {int(bad.sum())}/{bad.size} out of tolerance: "
                             f"{detail}")
    return float((err / tol).max())


def check_mask(case, got_words: np.ndarray, ref, A_bits=None, label: str = "") -> int:
    """Bit-exact mask check outside the excusal band; padding bits must be 0.
    Returns the number of excused differing bits."""
    N = case.N
    ld = O.aux_ld_words(N)
    assert got_words.shape[1] == ld
    got = O.unpack_mask(got_words, N)
    want = O.unpack_mask(ref.mask, N)
    excused = np.abs(ref.z) < abs_term(case, A_bits) / 0.99
    diff = got != want
    hard = diff & ~excused
    if hard.any():
        i = np.argwhere(hard)[:5]
        raise AssertionError(f"{label} {case.name}: {int(hard.sum())} mask bits differ "
                             f"(first {i.tolist()})")
    pad = O.unpack_mask(got_words, ld * 32)[:, N:]
    assert not pad.any(), f"{label} {case.name}: nonzero mask padding bits"
    return int((diff & excused).sum())


def check_zaux(case, got_bits: np.ndarray, ref, A_bits=None, label: str = ""):
    """GELU_AUX_BIAS: the saved z against the oracle's fp64 z."""
    got = O.decode(got_bits, case.dtype)
    tol = 1e-2 * np.abs(ref.z) + abs_term(case, A_bits)
    err = np.abs(got - ref.z)
    bad = (~np.isfinite(got)) | (err > tol)
    if bad.any():
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{label} {case.name}: z aux {int(bad.sum())}/{bad.size} out of "
                             f"tolerance, first {i.tolist()}")
    return float((err / tol).max())


def check_bgrad(case, got: np.ndarray, ref, label: str = "", unfused: bool = False):
    """bgrad against the oracle's, to the parity formula.  The unfused path
    sums dZ values already rounded to the dtype; in fp16 (u = 2^-11) the
    formula covers that rounding as it stands, in bf16 (u = 2^-8) it does not
    (a 333-row DGELU case measured 1.77 times the formula), so bf16 adds the
    worst-case bound of that rounding, 2 u sum_m |dZ[m, n]|.  Returns (and
    logs) the largest err / tol, and for the unfused path the largest err
    over that rounding bound."""
    import sys
    tol = 1e-2 * np.abs(ref.bgrad.astype(np.float64)) + grad_scale(case) * abs_term(case)
    err = np.abs(got.astype(np.float64) - ref.bgrad.astype(np.float64))
    extra = ""
    if unfused:
        worst = 2.0 * UNIT_ROUNDOFF[case.dtype] * ref.bgrad_abs
        extra = f"; err / (2u sum|dZ|) max {float((err / np.maximum(worst, 1e-300)).max()):.3g}"
        if case.dtype == "bf16":
            tol = tol + worst
    ratio = float((err / tol).max())
    print(f"[bgrad] {label} {case.name}: max err/tol {ratio:.3g}{extra}", file=sys.stderr,
          flush=True)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[:5].ravel()
        raise AssertionError(f"{label} {case.name}: bgrad {int(bad.sum())} out of tolerance; "
                             f"{[(int(j), float(got[j]), float(ref.bgrad[j])) for j in i]}")
    return ratio


# ---------------------------------------------------------------- GEMM + residual + norm


def run_norm(c, flags: int = 0, tile: int = -1, eps=None, allow_gave_up: bool = False):
    """Upload a NormCase, execute it through gemmepi_execute_norm and return
    (out bits [M, N], (mean, rstd) fp64 [M, 2], status word: 1 single pass,
    0 two kernels)."""
    import torch
    f = flags | (ge.FLAG_B_TRANS if c.b_trans else 0)
    up = lambda x: None if x is None else upload_bits(x, c.dtype)  # noqa: E731
    A, B, bias, res, gamma, beta = (up(c.A), up(c.B), up(c.bias), up(c.residual), up(c.gamma),
                                    up(c.beta))
    out = torch.full((c.M, c.N), float("nan"), dtype=torch_dtype(c.dtype), device="cuda")
    # a pattern the call must overwrite (it clears the workspace part, and
    # writes (mean, rstd) of every row)
    stats = ge.norm_stats_buffer(c.M).fill_(1234.5)
    epi = "BIAS_RES_" + c.norm
    with ge.plan(c.M, c.N, c.K, c.dtype, epi, f, tile=tile) as p:
        p.execute_norm(A, B, bias, res, gamma, beta, c.eps if eps is None else eps, stats, out)
        torch.cuda.synchronize()
    status = ge.norm_pass_status(stats, c.M)
    assert status in (0, 1) or allow_gave_up, f"{c.name}: norm status word {status:#x} (a row wait gave up)"
    return download_bits(out), ge.norm_mean_rstd(stats, c.M).cpu().numpy(), status


def norm_tolerance(c, ref, rows, y_rounded: bool = True):
    """Per-element bound derived from the arithmetic of
    out = (y - mean) rstd gamma + beta: y carries the GEMM's accumulation
    error tau = 2e-3 sqrt(K) max|A| max|B| (the bound used for every GEMM
    here) plus, in the two-kernel form (y_rounded), two storage roundings:
    Delta_m = tau + 2 u max_n |y_mn|.  The single pass keeps y in fp32, so
    only the two fp32 additions of bias and residual remain:
    Delta_m = tau + 2^-22 max_n |y_mn|.  Delta_m moves the mean by at most
    Delta_m and rstd by a relative Delta_m rstd, so
    |d out_mn| <= |gamma_n| rstd_m Delta_m (2 + rstd_m |y_mn - mean_m|), plus
    1e-2 |out| for the final rounding and fp32 arithmetic and 2^-7 |beta|."""
    u = UNIT_ROUNDOFF[c.dtype] if y_rounded else 2.0 ** -23
    A = O.decode(c.A, c.dtype)
    B = O.decode(c.B, c.dtype)
    tau = 2e-3 * np.sqrt(c.K) * np.abs(A).max() * np.abs(B).max()
    y = ref.y
    delta = tau + 2 * u * np.abs(y).max(axis=1)                     # [R]
    g = np.abs(O.decode(c.gamma, c.dtype))[None, :]
    r = ref.rstd[:, None]
    tol = 1e-2 * np.abs(ref.out64) + g * r * delta[:, None] * (2 + r * np.abs(y - ref.mean[:, None]))
    if c.beta is not None and c.norm == "LAYERNORM":
        tol = tol + 2.0 ** -7 * np.abs(O.decode(c.beta, c.dtype))[None, :]
    return tol, delta


def check_norm(c, out_bits, stats, ref, rows, label="", status: int = 0):
    """out and (mean, rstd) of the given rows against the oracle's, to
    norm_tolerance for the form that ran (status 1: single pass)."""
    got = O.decode(out_bits[rows], c.dtype)
    tol, delta = norm_tolerance(c, ref, rows, y_rounded=status != 1)
    err = np.abs(got - ref.out64)
    bad = err > tol
    assert not np.isnan(got).any(), f"{label} {c.name}: NaN in output"
    assert not bad.any(), (f"{label} {c.name}: {int(bad.sum())} elements out of tolerance, worst "
                           f"{float((err - tol).max()):.3g} at {np.argwhere(bad)[0].tolist()}")
    st = stats[rows]
    if c.norm == "LAYERNORM":
        assert np.all(np.abs(st[:, 0] - ref.mean) <= delta + 1e-9 * np.abs(ref.mean)), \
            f"{label} {c.name}: row means"
    else:
        assert np.all(st[:, 0] == 0.0), f"{label} {c.name}: RMSNorm mean slot"
    assert np.all(np.abs(st[:, 1] - ref.rstd) <= ref.rstd * (2 * delta * ref.rstd + 1e-9)), \
        f"{label} {c.name}: rstd"
