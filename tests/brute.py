"""Brute-force fused GEMM for tiny shapes, independent of oracle/.

Pure Python: storage bits are decoded with ``struct`` ('e' for fp16, the top
half of an 'f' word for bf16), every product of two 16-bit floats is exact in
a Python float (at most 22 significant bits), ``math.fsum`` returns the
correctly rounded exact sum, and the final rounding is done by ``struct``
('e', round half to even) for fp16 and by exact ``Fraction`` arithmetic for
bf16 and fp32.  It shares nothing with the numpy oracle beyond the definition
of the method, so a dropped term, a wrong index, a transposed operand or a
wrong rounding in either shows up as a mismatch.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction
from typing import List, Optional, Sequence


def f16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def value(bits: int, dtype: str) -> float:
    return f16_value(bits) if dtype == "f16" else bf16_value(bits)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); fix up to 2^e <= a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    return e


def round_fraction(x: float, sig_bits: int, emin: int, emax: int) -> float:
    """Exact round-half-even of x to the given binary format using Fractions
    (Python's round() on a Fraction is round-half-even)."""
    if x == 0 or math.isinf(x) or math.isnan(x):
        return x
    a = abs(Fraction(x))
    e = max(_floor_log2(a), emin)
    q = Fraction(2) ** (e - (sig_bits - 1))
    v = round(a / q) * q
    max_finite = (2 - Fraction(2) ** (1 - sig_bits)) * Fraction(2) ** emax
    if v > max_finite:
        return math.copysign(math.inf, x)
    return math.copysign(float(v), x)


def f16_bits(x: float) -> int:
    """struct's 'e' packer rounds half to even; it refuses values that round
    past the largest half (65504), which are +-inf."""
    try:
        return struct.unpack("<H", struct.pack("<e", x))[0]
    except OverflowError:
        return 0x7C00 if x > 0 else 0xFC00


def bf16_bits(x: float) -> int:
    r = round_fraction(x, 8, -126, 127)
    return struct.unpack("<I", struct.pack("<f", r))[0] >> 16


def out_bits(x: float, dtype: str) -> int:
    return f16_bits(x) if dtype == "f16" else bf16_bits(x)


def f32_round(x: float) -> float:
    return round_fraction(x, 24, -126, 127)


def fused(A: Sequence[int], B: Sequence[int], bias: Optional[Sequence[int]],
          mask_words: Optional[Sequence[Sequence[int]]], M: int, N: int, K: int,
          dtype: str, epilogue: str, b_trans: bool, bias_per_col: bool,
          col_abs: Optional[List[float]] = None):
    """Returns (out_bits[M][N], mask bits or z bits [M][N] or None, bgrad[N]
    or None).

    A, B, bias are flat sequences of storage bits (row-major); mask_words is
    the packed mask [M][words] for DRELU_BGRAD and the flat z storage bits
    [M*N] for DGELU_BGRAD.  For the BGRAD epilogues a list passed as
    ``col_abs`` receives sum over rows of |dZ| per column."""
    a = [[value(A[i * K + k], dtype) for k in range(K)] for i in range(M)]
    if b_trans:
        b = [[value(B[j * K + k], dtype) for j in range(N)] for k in range(K)]
    else:
        b = [[value(B[k * N + j], dtype) for j in range(N)] for k in range(K)]
    has_bias = epilogue in ("BIAS", "RELU_BIAS", "RELU_AUX_BIAS", "GELU_BIAS", "GELU_AUX_BIAS")
    out: List[List[int]] = []
    mask: List[List[bool]] = []
    colsum_terms: List[List[float]] = [[] for _ in range(N)]
    abs_terms: List[List[float]] = [[] for _ in range(N)]
    for i in range(M):
        orow, mrow = [], []
        for j in range(N):
            terms = [a[i][k] * b[k][j] for k in range(K)]
            if has_bias:
                terms.append(value(bias[j] if bias_per_col else bias[i], dtype))
            z = math.fsum(terms)
            if epilogue in ("DEFAULT", "BIAS"):
                y = z
            elif epilogue in ("RELU_BIAS", "RELU_AUX_BIAS"):
                y = z if z > 0 else 0.0
                mrow.append(z > 0)
            elif epilogue in ("GELU_BIAS", "GELU_AUX_BIAS"):
                y = 0.5 * z * math.erfc(-z / math.sqrt(2.0))
                mrow.append(out_bits(z, dtype))
            elif epilogue == "DGELU_BGRAD":
                zs = value(mask_words[i * N + j], dtype)       # saved pre-activation bits
                g = 0.5 * math.erfc(-zs / math.sqrt(2.0)) + zs * math.exp(-0.5 * zs * zs) / math.sqrt(2.0 * math.pi)
                y = z * g
                colsum_terms[j].append(y)
            elif epilogue == "DRELU_BGRAD":
                bit = (mask_words[i][j >> 5] >> (j & 31)) & 1
                y = z if bit else 0.0
                if bit:
                    colsum_terms[j].extend(terms)
            else:
                raise ValueError(epilogue)
            abs_terms[j].append(abs(y))
            orow.append(out_bits(y, dtype))
        out.append(orow)
        mask.append(mrow)
    bgrad = None
    if epilogue in ("DRELU_BGRAD", "DGELU_BGRAD"):
        bgrad = [f32_round(math.fsum(t)) for t in colsum_terms]
        if col_abs is not None:
            col_abs[:] = [math.fsum(t) for t in abs_terms]
    # RELU_AUX_BIAS: mask bits; GELU_AUX_BIAS: storage bits of z
    return out, (mask if epilogue in ("RELU_AUX_BIAS", "GELU_AUX_BIAS") else None), bgrad


def norm(A: Sequence[int], B: Sequence[int], bias: Optional[Sequence[int]],
         residual: Optional[Sequence[int]], gamma: Sequence[int], beta: Optional[Sequence[int]],
         eps: float, M: int, N: int, K: int, dtype: str, kind: str, b_trans: bool):
    """GEMM + bias + residual + row norm on tiny shapes; returns
    (out_bits[M][N], out_values[M][N]).  y is the correctly rounded exact sum
    of the products, the bias and the residual; the row statistics use
    math.fsum as well."""
    a = [[value(A[i * K + k], dtype) for k in range(K)] for i in range(M)]
    if b_trans:
        b = [[value(B[j * K + k], dtype) for j in range(N)] for k in range(K)]
    else:
        b = [[value(B[k * N + j], dtype) for j in range(N)] for k in range(K)]
    g = [value(gamma[j], dtype) for j in range(N)]
    bt = [value(beta[j], dtype) if beta is not None else 0.0 for j in range(N)]
    bits, vals = [], []
    for i in range(M):
        y = []
        for j in range(N):
            terms = [a[i][k] * b[k][j] for k in range(K)]
            if bias is not None:
                terms.append(value(bias[j], dtype))
            if residual is not None:
                terms.append(value(residual[i * N + j], dtype))
            y.append(math.fsum(terms))
        if kind == "LAYERNORM":
            mean = math.fsum(y) / N
            var = math.fsum((v - mean) ** 2 for v in y) / N
            rstd = 1.0 / math.sqrt(var + eps)
            row = [(y[j] - mean) * rstd * g[j] + bt[j] for j in range(N)]
        else:
            ms = math.fsum(v * v for v in y) / N
            rstd = 1.0 / math.sqrt(ms + eps)
            row = [y[j] * rstd * g[j] for j in range(N)]
        vals.append(row)
        bits.append([out_bits(v, dtype) for v in row])
    return bits, vals
