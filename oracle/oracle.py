"""CPU oracle for the fused-epilogue GEMM.  TEST INFRASTRUCTURE ONLY.

Only the tests, the package's smoke check and the bench's CPU-baseline leg
may import this module.  The product path (the HIP library and its Python
binding) never calls it and shares no code with it.

What it computes is the plain definition of the method.  Fusing the epilogue
into the GEMM only moves work from separate kernels into registers ("Fusing
bias addition with matrix multiplication using nvmath-python", paragraph 2;
ops-nn MatMul fusion article, section "Level 1: basic fusion"), so the
fused result is the unfused one up to rounding order:

    acc[i,j] = sum_k A[i,k] * B[k,j]                  fp64, exact inputs
    z[i,j]   = acc[i,j] + bias[i]  (or bias[j])       fp64
    y        = epilogue(z)                            fp64
    out      = round_to_nearest_even(y -> fp16/bf16)  one rounding

with these epilogues (the MatmulEpilog members the pages name):
  DEFAULT        y = acc
  BIAS           y = acc + bias; the bias is an (m,1) column broadcast over
                 the columns of the (m,n) result ("nvmath-python cuBLASLt bias
                 fusion guide", section "Core API and parameter configuration")
  RELU_BIAS      y = max(z, 0)  (Y = ReLU(WX + B): "Fusing bias addition ...",
                 paragraph 1)
  RELU_AUX_BIAS  as RELU_BIAS plus the ReLU mask (z > 0) kept as an auxiliary
                 output ("Fusing bias addition ...", paragraph 4)
  GELU_BIAS      y = z Phi(z) = 0.5 z erfc(-z / sqrt 2), the exact (erf) GELU
                 that the unfused code of the ops-nn article calls by default
  DRELU_BGRAD    backward of ReLU+bias: dZ = mask ? acc : 0 and
                 bgrad[j] = sum_i dZ[i,j] ("nvmath-python cuBLASLt bias fusion
                 guide", section "Advanced techniques and engineering practice")
  GELU_AUX_BIAS  as GELU_BIAS, plus the pre-activation z (rounded once to the
                 storage dtype) kept as the auxiliary output, the GELU
                 counterpart of RELU_AUX_BIAS's mask
  DGELU_BGRAD    backward of GELU+bias, the GELU counterpart of DRELU_BGRAD:
                 dZ = acc * gelu'(z) with z the stored pre-activation and
                 gelu'(z) = Phi(z) + z phi(z); bgrad[j] = sum_i dZ[i,j]

Readings where the pages are silent:
  * accumulate in fp32 on the device, fp64 here; alpha = 1, beta = 0;
  * ReLU keeps z only when z > 0; the mask bit is (z > 0) on the unrounded z;
  * the bias is converted to the accumulator type and added before one
    rounding; bgrad is taken from the unrounded masked accumulator and
    rounded once to fp32;
  * mask layout: uint32 words, row-major with a pitch of ceil(N/32) words
    rounded up to a multiple of 4; column j of row i is bit (j & 31) of word
    (i, j >> 5); padding bits are 0.

Structural fusion (ops-nn MatMul fusion article, section "Level 2:
structural fusion": MatMul + bias + residual + LayerNorm/RMSNorm as one
operator) is in gemm_norm():

    y[i,:]   = acc[i,:] + bias[:] + residual[i,:]     fp64
    LAYERNORM  out = (y - mean(y)) / sqrt(var(y) + eps) * gamma + beta
    RMSNORM    out = y / sqrt(mean(y^2) + eps) * gamma
    mean/var over the N columns of a row; var is the biased (1/N) variance

with the readings: the residual is added to the GEMM result before the
normalisation (post-norm order); eps sits inside the square root; gamma,
beta and bias are per column.  The page names the operator but prints no
formula; these are the standard definitions of the two norms.

Pins: tests/test_oracle_pins.py checks this module against brute-force
exact sums (math.fsum over exactly-represented products, Fraction-based
rounding), exact integer arithmetic, closed-form GELU values, invariants of
the epilogues and an independent fp16 rounding (Python's struct 'e').
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

EPILOGUES = ("DEFAULT", "BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "DRELU_BGRAD",
             "GELU_AUX_BIAS", "DGELU_BGRAD")
NORMS = ("RMSNORM", "LAYERNORM")


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def decode_f16(bits: np.ndarray) -> np.ndarray:
    """fp16 storage bits -> exact fp64 values."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 storage bits -> exact fp64 values (bf16 is the top half of an
    fp32 word)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return decode_f16(bits)
    if dtype == "bf16":
        return decode_bf16(bits)
    raise ValueError(dtype)


def round_to_format(x: np.ndarray, sig_bits: int, emin: int, emax: int) -> np.ndarray:
    """Round fp64 values to a binary floating-point format with ``sig_bits``
    significant bits (hidden bit included), smallest normal exponent ``emin``
    and largest exponent ``emax``, ties to even, subnormals kept, overflow to
    +-inf.  The result is returned as fp64 (exactly representable in the
    format).

    Method: for |x| = f * 2^e with 0.5 <= f < 1 the format's spacing around
    x is 2^(max(e-1, emin) - sig_bits + 1); dividing by that power of two is
    exact, np.rint rounds half to even, and multiplying back is exact.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)
    exp = np.maximum(e - 1, emin)
    q = np.ldexp(1.0, exp - (sig_bits - 1))
    y = np.rint(xf / q) * q
    max_finite = (2.0 - 2.0 ** (1 - sig_bits)) * 2.0 ** emax
    y = np.where(np.abs(y) > max_finite, np.copysign(np.inf, y), y)
    out[finite] = y
    return out


def encode_f16(y: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 bits, one round-to-nearest-even (numpy converts double to
    half directly, without an fp32 step)."""
    with np.errstate(over="ignore"):
        return np.asarray(y, dtype=np.float64).astype(np.float16).view(np.uint16)


def encode_bf16(y: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits with a single round-to-nearest-even on the fp64
    value (8 significant bits, fp32 exponent range).  The rounded value is
    exact in fp32, so its top 16 bits are the bf16 encoding."""
    r = round_to_format(y, 8, -126, 127)
    r32 = r.astype(np.float32)
    return (r32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def encode(y: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return encode_f16(y)
    if dtype == "bf16":
        return encode_bf16(y)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# epilogue pieces
# --------------------------------------------------------------------------
_erfc = np.frompyfunc(math.erfc, 1, 1)


def gelu(z: np.ndarray) -> np.ndarray:
    """Exact GELU, z * Phi(z), with the standard normal CDF written through
    libm's complementary error function, Phi(z) = erfc(-z / sqrt 2) / 2.
    This equals 0.5 z (1 + erf(z / sqrt 2)) but does not cancel to zero in
    the negative tail (1 + erf(x) rounds to 0 in fp64 below x ~ -5.9)."""
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * _erfc(-z / math.sqrt(2.0)).astype(np.float64)


def gelu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz of z Phi(z): Phi(z) + z phi(z), phi the standard normal density
    exp(-z^2 / 2) / sqrt(2 pi)."""
    z = np.asarray(z, dtype=np.float64)
    Phi = 0.5 * _erfc(-z / math.sqrt(2.0)).astype(np.float64)
    phi = np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)
    return Phi + z * phi


def aux_ld_words(n: int) -> int:
    """Mask row pitch in uint32 words."""
    return ((n + 31) // 32 + 3) // 4 * 4


def pack_mask(bits: np.ndarray) -> np.ndarray:
    """bool [R, N] -> uint32 [R, aux_ld_words(N)]; column j is bit (j & 31)
    of word j >> 5; padding bits are 0."""
    bits = np.asarray(bits, dtype=bool)
    r, n = bits.shape
    ld = aux_ld_words(n)
    padded = np.zeros((r, ld * 32), dtype=np.uint64)
    padded[:, :n] = bits
    padded = padded.reshape(r, ld, 32)
    weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
    return (padded * weights).sum(axis=2).astype(np.uint32)


def unpack_mask(words: np.ndarray, n: int) -> np.ndarray:
    """uint32 [R, ld] -> bool [R, n] (inverse of pack_mask on valid columns)."""
    words = np.asarray(words, dtype=np.uint32)
    shifts = np.arange(32, dtype=np.uint32)
    bits = (words[:, :, None] >> shifts) & np.uint32(1)
    return bits.reshape(words.shape[0], -1)[:, :n].astype(bool)


# --------------------------------------------------------------------------
# the reference
# --------------------------------------------------------------------------
@dataclass
class OracleResult:
    rows: np.ndarray                 # which output rows were computed
    out: np.ndarray                  # storage bits [R, N] (uint16)
    z: np.ndarray                    # fp64 pre-activation (acc + bias, or acc) [R, N]
    y: np.ndarray                    # fp64 epilogue value before rounding [R, N]
    mask: Optional[np.ndarray] = None    # RELU_AUX_BIAS: uint32 [R, ld]
    zaux: Optional[np.ndarray] = None    # GELU_AUX_BIAS: storage bits of z [R, N]
    bgrad: Optional[np.ndarray] = None   # *_BGRAD: float32 [N]
    bgrad_abs: Optional[np.ndarray] = None  # *_BGRAD: fp64 sum over rows of |dZ| [N]
                                            # (the weight of a rounding-error bound)


def gemm_epilogue(A: np.ndarray, B: np.ndarray, bias: Optional[np.ndarray],
                  aux: Optional[np.ndarray], M: int, N: int, K: int, dtype: str,
                  epilogue: str, b_trans: bool, bias_per_col: bool,
                  rows: Optional[np.ndarray] = None) -> OracleResult:
    """Reference result of one fused GEMM call.

    A: storage bits [M, K];  B: [K, N], or [N, K] when ``b_trans``;
    bias: [M] (or [N] with ``bias_per_col``) storage bits, for the *_BIAS
    epilogues; aux: packed input mask for DRELU_BGRAD, storage bits of the
    saved pre-activation [M, N] for DGELU_BGRAD.  ``rows`` restricts the
    returned rows (the BGRAD epilogues still reduce bgrad over every row).
    """
    if epilogue not in EPILOGUES:
        raise ValueError(epilogue)
    A64 = decode(np.asarray(A).reshape(M, K), dtype)
    B64 = decode(np.asarray(B).reshape((N, K) if b_trans else (K, N)), dtype)
    if b_trans:
        B64 = B64.T
    all_rows = np.arange(M)
    rows = all_rows if rows is None else np.asarray(rows)
    need_all = epilogue in ("DRELU_BGRAD", "DGELU_BGRAD")
    comp_rows = all_rows if need_all else rows

    acc = A64[comp_rows] @ B64                         # [R, N] fp64

    if epilogue in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "GELU_AUX_BIAS"):
        b64 = decode(np.asarray(bias), dtype)
        if bias_per_col:
            z = acc + b64[None, :N]
        else:
            z = acc + b64[comp_rows][:, None]
    else:
        z = acc

    mask_words = None
    zaux = None
    bgrad = None
    if epilogue in ("DEFAULT", "BIAS"):
        y = z
    elif epilogue in ("RELU_BIAS", "RELU_AUX_BIAS"):
        y = np.where(z > 0, z, 0.0)
        if epilogue == "RELU_AUX_BIAS":
            mask_words = pack_mask(z > 0)
    elif epilogue in ("GELU_BIAS", "GELU_AUX_BIAS"):
        y = gelu(z)
        if epilogue == "GELU_AUX_BIAS":
            zaux = encode(z, dtype)
    elif epilogue == "DGELU_BGRAD":
        zs = decode(np.asarray(aux).reshape(M, N), dtype)
        y = z * gelu_grad(zs)
        bgrad = y.sum(axis=0).astype(np.float32)
    else:  # DRELU_BGRAD
        m = unpack_mask(np.asarray(aux).reshape(M, -1), N)
        y = np.where(m, z, 0.0)
        bgrad = y.sum(axis=0).astype(np.float32)
    bgrad_abs = np.abs(y).sum(axis=0) if need_all else None

    out = encode(y, dtype)
    if need_all and rows is not comp_rows:
        sel = rows
        out, z, y = out[sel], z[sel], y[sel]
    return OracleResult(rows=rows, out=out, z=z, y=y, mask=mask_words, bgrad=bgrad, zaux=zaux,
                        bgrad_abs=bgrad_abs)


def ffn_block(x, W1, b1, W2, b2, tokens: int, hidden: int, inter: int, dtype: str):
    """FFN block of two fused GEMMs with an activation between them (ops-nn
    MatMul fusion article, section "Level 1: basic fusion"):
    h = GELU_BIAS(x W1^T + b1) rounded to the storage dtype, then
    y = BIAS(h W2^T + b2).  Returns (h_result, y_result)."""
    h = gemm_epilogue(x, W1, b1, None, tokens, inter, hidden, dtype, "GELU_BIAS", True, True)
    y = gemm_epilogue(h.out, W2, b2, None, tokens, hidden, inter, dtype, "BIAS", True, True)
    return h, y


@dataclass
class NormResult:
    rows: np.ndarray                 # which output rows were computed
    out: np.ndarray                  # storage bits [R, N] (uint16)
    y: np.ndarray                    # fp64 acc + bias + residual [R, N]
    mean: np.ndarray                 # fp64 row mean of y [R] (RMSNORM: 0)
    rstd: np.ndarray                 # fp64 1 / sqrt(var + eps) (RMSNORM: of mean(y^2))
    out64: np.ndarray                # fp64 normalised value before rounding [R, N]


def gemm_norm(A: np.ndarray, B: np.ndarray, bias: Optional[np.ndarray],
              residual: Optional[np.ndarray], gamma: np.ndarray, beta: Optional[np.ndarray],
              eps: float, M: int, N: int, K: int, dtype: str, norm: str, b_trans: bool,
              rows: Optional[np.ndarray] = None) -> NormResult:
    """Reference of the GEMM + bias + residual + row-norm operator (ops-nn
    MatMul fusion article, section "Level 2: structural fusion").

    A: storage bits [M, K]; B: [K, N], or [N, K] with ``b_trans``; bias,
    gamma, beta: [N] storage bits (bias and beta may be None: zero);
    residual: [M, N] storage bits or None.  Every row is normalised over all
    N of its columns; ``rows`` selects the rows computed and returned.
    """
    if norm not in NORMS:
        raise ValueError(norm)
    A64 = decode(np.asarray(A).reshape(M, K), dtype)
    B64 = decode(np.asarray(B).reshape((N, K) if b_trans else (K, N)), dtype)
    if b_trans:
        B64 = B64.T
    rows = np.arange(M) if rows is None else np.asarray(rows)
    y = A64[rows] @ B64                                # [R, N]
    if bias is not None:
        y = y + decode(np.asarray(bias), dtype)[None, :N]
    if residual is not None:
        y = y + decode(np.asarray(residual).reshape(M, N), dtype)[rows]
    g = decode(np.asarray(gamma), dtype)[None, :N]
    if norm == "LAYERNORM":
        mean = y.mean(axis=1)
        d = y - mean[:, None]
        var = (d * d).mean(axis=1)                     # two-pass, biased
        rstd = 1.0 / np.sqrt(var + eps)
        out64 = d * rstd[:, None] * g
        if beta is not None:
            out64 = out64 + decode(np.asarray(beta), dtype)[None, :N]
    else:
        mean = np.zeros(len(rows))
        ms = (y * y).mean(axis=1)
        rstd = 1.0 / np.sqrt(ms + eps)
        out64 = y * rstd[:, None] * g
    return NormResult(rows=rows, out=encode(out64, dtype), y=y, mean=mean, rstd=rstd,
                      out64=out64)
