"""Seeded synthetic inputs for the fused-epilogue GEMM workloads.

This module only draws random numbers and stores them in fp16 / bf16 / uint32
form.  It contains none of the GEMM or epilogue arithmetic, so both the CPU
oracle side (tests) and the GPU side (tests, bench) can take their inputs from
it without sharing any of the method's code.

Every tensor is returned as host numpy arrays of raw storage bits
(``uint16`` for fp16/bf16, ``uint32`` for packed masks) so that the exact
same bytes reach the oracle and the device.

Shapes and distributions follow the workloads of the pages:
  * small BIAS case: W[1024,2048] @ X[2048,512] + b[1024] (uniform [0,1), fp16)
    -- "nvmath-python cuBLASLt bias fusion guide", section "Core API and
    parameter configuration", the minimal code example;
  * decode shape x[T,4096] @ W[4096,4096]^T -- ops-nn MatMul fusion article,
    section "Why MatMul is the core bottleneck of LLM inference";
  * FFN block hidden 4096, token counts 512/2048/4x512/16x128 -- same article,
    section "Performance before and after fusion" (its test table); the
    intermediate width 11008 is the LLaMA-style FFN size those rows name;
  * (65536x16384)·(16384x8192) RELU_AUX_BIAS -- "Fusing bias addition with
    matrix multiplication using nvmath-python", paragraph 4 (the H200 figure);
  * DRELU_BGRAD backward -- "nvmath-python cuBLASLt bias fusion guide",
    section "Advanced techniques and engineering practice".
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence

import numpy as np

# storage dtypes
F16 = "f16"
BF16 = "bf16"

_CHUNK = 1 << 24  # elements drawn per RNG call (bounds host memory)


# --------------------------------------------------------------------------
# fp32 -> storage bits.  These are *input preparation* only (turning a float32
# draw into the 16-bit value that is then the exact input of both sides).
# --------------------------------------------------------------------------
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> fp16, returned as uint16 bits."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 (upper 16 bits), as uint16 bits.

    Finite inputs only (generated inputs never hold NaN): adding 0x7FFF plus
    the lowest kept bit to the fp32 word and truncating rounds the low 16 bits
    to nearest, ties to even.  Works in chunks with uint32 arithmetic.
    """
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    for s in range(0, flat.size, _CHUNK):
        u = flat[s:s + _CHUNK].view(np.uint32)
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        out[s:s + _CHUNK] = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    return out.reshape(x.shape)


def to_bits(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return f32_to_f16_bits(x32)
    if dtype == BF16:
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# draws
# --------------------------------------------------------------------------
def _draw(shape: Sequence[int], seed: int, kind: str, scale: float) -> np.ndarray:
    """fp32 draw of ``shape`` in row-major chunks from one PCG64 stream."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        if kind == "uniform":
            out[s:e] = rng.random(e - s, dtype=np.float32)
        elif kind == "normal":
            out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
        elif kind == "int":
            out[s:e] = rng.integers(-3, 4, e - s).astype(np.float32)
        else:
            raise ValueError(kind)
        if scale != 1.0:
            out[s:e] *= np.float32(scale)
    return out.reshape(shape)


def uniform01(shape, seed: int, dtype: str = F16) -> np.ndarray:
    """U[0,1) fp32 draw rounded to the storage dtype (values that round up to
    1.0 are kept, as an fp16 ``rand`` would produce)."""
    return to_bits(_draw(shape, seed, "uniform", 1.0), dtype)


def normal(shape, seed: int, std: float = 1.0, dtype: str = F16) -> np.ndarray:
    """N(0, std^2) fp32 draw rounded to the storage dtype."""
    return to_bits(_draw(shape, seed, "normal", std), dtype)


def small_ints(shape, seed: int, dtype: str = F16) -> np.ndarray:
    """Integers in {-3..3}: every product and partial sum is exact in fp32
    while |sum| < 2^24, which makes bit-exact comparisons possible."""
    return to_bits(_draw(shape, seed, "int", 1.0), dtype)


def aux_ld_words(n: int) -> int:
    """Row pitch of a packed bit mask in uint32 words: ceil(n/32) rounded up
    to a multiple of 4 words (16 bytes)."""
    w = (n + 31) // 32
    return (w + 3) // 4 * 4


def random_mask(m: int, n: int, seed: int, p_one: float = 0.5) -> np.ndarray:
    """Packed [m, aux_ld_words(n)] uint32 mask with Bernoulli(p) bits for the
    n valid columns and zero padding bits.  Column j of row i is bit (j & 31)
    of word (i, j >> 5)."""
    rng = np.random.default_rng(seed)
    ld = aux_ld_words(n)
    if p_one == 0.5:
        words = rng.integers(0, 1 << 32, size=(m, ld), dtype=np.uint64).astype(np.uint32)
    else:
        bits = (rng.random((m, ld, 32)) < p_one).astype(np.uint64)
        weights = np.uint64(1) << np.arange(32, dtype=np.uint64)
        words = (bits * weights).sum(axis=-1).astype(np.uint32)
    # zero the padding bits
    full = n // 32
    rem = n % 32
    if rem:
        words[:, full] &= np.uint32((1 << rem) - 1)
        words[:, full + 1:] = 0
    else:
        words[:, full:] = 0
    return np.ascontiguousarray(words)


def const_mask(m: int, n: int, value: bool) -> np.ndarray:
    ld = aux_ld_words(n)
    words = np.zeros((m, ld), dtype=np.uint32)
    if value:
        full = n // 32
        words[:, :full] = np.uint32(0xFFFFFFFF)
        if n % 32:
            words[:, full] = np.uint32((1 << (n % 32)) - 1)
    return words


# --------------------------------------------------------------------------
# the workloads
# --------------------------------------------------------------------------
@dataclasses.dataclass
class GemmCase:
    """One GEMM call: out[M,N] = A[M,K] @ B (+ epilogue)."""
    name: str
    M: int
    N: int
    K: int
    dtype: str
    epilogue: str            # a key of the binding's EPILOGUES (not the norms)
    b_trans: bool            # B stored [N,K] (K contiguous) instead of [K,N]
    bias_per_col: bool       # bias indexed by n instead of m
    A: np.ndarray = None     # uint16 bits [M,K]
    B: np.ndarray = None     # uint16 bits [K,N] or [N,K]
    bias: Optional[np.ndarray] = None   # uint16 bits [M] or [N]
    aux: Optional[np.ndarray] = None    # DRELU: uint32 mask [M, aux_ld_words(N)];
                                        # DGELU: uint16 bits of the saved z [M, N]

    @property
    def flops(self) -> float:
        return 2.0 * self.M * self.N * self.K


def seed_of(config: int, tensor: int) -> int:
    return 1000 + 10 * config + tensor


def row_sample_seed(config: int) -> int:
    return 9000 + config


def config0_bias(dtype: str = F16) -> GemmCase:
    """Y[1024,512] = W[1024,2048] X[2048,512] + b[1024] (per row), U[0,1)."""
    M, N, K = 1024, 512, 2048
    c = GemmCase("c0_bias", M, N, K, dtype, "BIAS", False, False)
    c.A = uniform01((M, K), seed_of(0, 0), dtype)
    c.B = uniform01((K, N), seed_of(0, 1), dtype)
    c.bias = uniform01((M,), seed_of(0, 2), dtype)
    return c


def config1_decode(T: int, dtype: str = F16, copy: int = 0) -> GemmCase:
    """y[T,4096] = gelu(x[T,4096] W[4096,4096]^T + b[4096]).  ``copy`` selects
    an independent replica (used to rotate weights past the caches)."""
    N = K = 4096
    c = GemmCase(f"c1_decode_T{T}", T, N, K, dtype, "GELU_BIAS", True, True)
    s = 100 * copy
    c.A = normal((T, K), seed_of(1, 0) + s + T, 1.0, dtype)
    c.B = normal((N, K), seed_of(1, 1) + s, 1.0 / 64.0, dtype)
    c.bias = normal((N,), seed_of(1, 2) + s, 0.1, dtype)
    return c


FFN_TOKENS = {"b1s512": 512, "b1s2048": 2048, "b4s512": 2048, "b16s128": 2048}
FFN_HIDDEN = 4096
FFN_INTER = 11008


def config2_ffn(variant: str, dtype: str = F16):
    """Two GEMM cases of one FFN block: up (GELU_BIAS) then down (BIAS).
    The down case's A is the up case's output and is left None here."""
    tok = FFN_TOKENS[variant]
    vi = list(FFN_TOKENS).index(variant)
    H, I = FFN_HIDDEN, FFN_INTER
    up = GemmCase(f"c2_{variant}_up", tok, I, H, dtype, "GELU_BIAS", True, True)
    up.A = normal((tok, H), seed_of(2, 0) + 100 * vi, 1.0, dtype)
    up.B = normal((I, H), seed_of(2, 1), 1.0 / np.sqrt(H), dtype)
    up.bias = normal((I,), seed_of(2, 2), 0.1, dtype)
    down = GemmCase(f"c2_{variant}_down", tok, H, I, dtype, "BIAS", True, True)
    down.B = normal((H, I), seed_of(2, 3), 1.0 / np.sqrt(I), dtype)
    down.bias = normal((H,), seed_of(2, 4), 0.1, dtype)
    return up, down


def device_normal(shape, seed: int, std: float, dtype: str, device="cuda"):
    """N(0, std^2) drawn on the GPU with torch's seeded Philox generator in
    fp32, scaled, then rounded to the storage dtype (round to nearest even).
    Used for the two large workloads, whose operands (up to 2^30 elements)
    would take minutes to draw on the host.  The oracle reads the exact same
    bits back from device memory (these are inputs; no kernel of the library
    touches them before that)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(float(std))
    y = x.to(torch.float16 if dtype == F16 else torch.bfloat16)
    del x
    return y


@dataclasses.dataclass
class DeviceCase(GemmCase):
    """A GemmCase whose A and B live in device memory (torch tensors);
    ``host_A(rows)`` / ``host_B()`` return their storage bits for the oracle."""
    A_dev: object = None
    B_dev: object = None

    def host_A(self, rows=None) -> np.ndarray:
        import torch
        a = self.A_dev
        if rows is not None:
            a = a.index_select(0, torch.as_tensor(np.asarray(rows), device=a.device))
        return a.view(torch.int16).cpu().numpy().view(np.uint16)

    def host_B(self) -> np.ndarray:
        import torch
        return self.B_dev.view(torch.int16).cpu().numpy().view(np.uint16)


def config3_relu_aux(dtype: str = F16, device="cuda", M: int = 65536, N: int = 8192,
                     K: int = 16384) -> DeviceCase:
    """out = relu(A[M,K] B[K,N] + bias[M]) plus the packed ReLU mask.
    A ~ N(0,1)/128, B ~ N(0,1), bias ~ N(0,1) (per row)."""
    c = DeviceCase(f"c3_relu_aux_{dtype}", M, N, K, dtype, "RELU_AUX_BIAS", False, False)
    c.A_dev = device_normal((M, K), seed_of(3, 0), 1.0 / 128.0, dtype, device)
    c.B_dev = device_normal((K, N), seed_of(3, 1), 1.0, dtype, device)
    c.bias = normal((M,), seed_of(3, 2), 1.0, dtype)
    return c


def config4_drelu_bgrad(dtype: str = F16, device="cuda", M: int = 8192, N: int = 4096,
                        K: int = 16384) -> DeviceCase:
    """dZ = mask ? dY[M,K] W[K,N] : 0 and bgrad[N] = column sums of dZ;
    dY, W ~ N(0,1)/128, mask bits Bernoulli(0.5)."""
    c = DeviceCase(f"c4_drelu_bgrad_{dtype}", M, N, K, dtype, "DRELU_BGRAD", False, False)
    c.A_dev = device_normal((M, K), seed_of(4, 0), 1.0 / 128.0, dtype, device)
    c.B_dev = device_normal((K, N), seed_of(4, 1), 1.0 / 128.0, dtype, device)
    c.aux = random_mask(M, N, seed_of(4, 2))
    return c


def config3_gelu_aux(dtype: str = F16, device="cuda", M: int = 65536, N: int = 8192,
                     K: int = 16384) -> DeviceCase:
    """C3's operands with the GELU epilogue that also saves z = A B + bias."""
    c = config3_relu_aux(dtype, device, M, N, K)
    c.name = f"c3_gelu_aux_{dtype}"
    c.epilogue = "GELU_AUX_BIAS"
    return c


def config4_dgelu_bgrad(dtype: str = F16, device="cuda", M: int = 8192, N: int = 4096,
                        K: int = 16384) -> DeviceCase:
    """dZ = (dY[M,K] W[K,N]) * gelu'(z) and bgrad[N] = column sums of dZ;
    dY, W ~ N(0,1)/128 as in the ReLU backward, the saved pre-activation
    z ~ N(0, 1.5^2) in the storage dtype, [M, N]."""
    c = DeviceCase(f"c4_dgelu_bgrad_{dtype}", M, N, K, dtype, "DGELU_BGRAD", False, False)
    c.A_dev = device_normal((M, K), seed_of(4, 0), 1.0 / 128.0, dtype, device)
    c.B_dev = device_normal((K, N), seed_of(4, 1), 1.0 / 128.0, dtype, device)
    c.aux = normal((M, N), seed_of(4, 3), 1.5, dtype)
    return c


def sample_rows(M: int, count: int, seed: int) -> np.ndarray:
    """``count`` distinct rows chosen by seed, always including 0 and M-1."""
    if count >= M:
        return np.arange(M)
    rng = np.random.default_rng(seed)
    rows = rng.choice(np.arange(1, M - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, M - 1], rows]))


def random_case(M: int, N: int, K: int, dtype: str, epilogue: str, b_trans: bool,
                bias_per_col: bool, seed: int, kind: str = "normal") -> GemmCase:
    """Generic seeded case for parity sweeps (shapes of any size)."""
    c = GemmCase(f"rand_{M}x{N}x{K}_{dtype}_{epilogue}_{int(b_trans)}{int(bias_per_col)}",
                 M, N, K, dtype, epilogue, b_trans, bias_per_col)
    if kind == "int":
        c.A = small_ints((M, K), seed, dtype)
        c.B = small_ints((N, K) if b_trans else (K, N), seed + 1, dtype)
        c.bias = small_ints((N if bias_per_col else M,), seed + 2, dtype)
    else:
        c.A = normal((M, K), seed, 1.0, dtype)
        c.B = normal((N, K) if b_trans else (K, N), seed + 1, 1.0 / np.sqrt(K), dtype)
        c.bias = normal((N if bias_per_col else M,), seed + 2, 0.5, dtype)
    if epilogue == "DRELU_BGRAD":
        c.bias = None
        c.aux = random_mask(M, N, seed + 3)
    if epilogue == "DGELU_BGRAD":
        # the saved pre-activation z of a GELU forward, [M, N] storage bits
        c.bias = None
        c.aux = normal((M, N), seed + 3, 1.5, dtype)
    return c


@dataclasses.dataclass
class NormCase:
    """Operands of one GEMM + bias + residual + norm call (storage bits)."""
    name: str
    M: int
    N: int
    K: int
    dtype: str
    norm: str                        # "RMSNORM" or "LAYERNORM"
    b_trans: bool
    A: Optional[np.ndarray] = None
    B: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None
    residual: Optional[np.ndarray] = None
    gamma: Optional[np.ndarray] = None
    beta: Optional[np.ndarray] = None
    eps: float = 1e-5


def norm_case(M: int, N: int, K: int, dtype: str, norm: str, b_trans: bool, seed: int,
              kind: str = "normal", with_bias: bool = True, with_residual: bool = True,
              with_beta: bool = True) -> NormCase:
    """Seeded operands for the structural-fusion operator.  The residual has
    a per-row offset (residual streams are not zero-mean), so the LayerNorm
    mean matters.  kind="int": integer operands in {-3..3} (exact sums)."""
    c = NormCase(f"norm_{M}x{N}x{K}_{dtype}_{norm}_{int(b_trans)}_{kind}", M, N, K, dtype, norm,
                 b_trans)
    if kind == "int":
        c.A = small_ints((M, K), seed, dtype)
        c.B = small_ints((N, K) if b_trans else (K, N), seed + 1, dtype)
        c.bias = small_ints((N,), seed + 2, dtype) if with_bias else None
        c.residual = small_ints((M, N), seed + 3, dtype) if with_residual else None
        c.gamma = small_ints((N,), seed + 4, dtype)
        c.beta = small_ints((N,), seed + 5, dtype) if with_beta else None
        c.eps = 0.25
        return c
    c.A = normal((M, K), seed, 1.0, dtype)
    c.B = normal((N, K) if b_trans else (K, N), seed + 1, 1.0 / np.sqrt(K), dtype)
    c.bias = normal((N,), seed + 2, 0.5, dtype) if with_bias else None
    if with_residual:
        offs = _draw((M, 1), seed + 6, "normal", 2.0)
        c.residual = to_bits(_draw((M, N), seed + 3, "normal", 1.0) + offs, dtype)
    c.gamma = to_bits(1.0 + _draw((N,), seed + 4, "normal", 0.2), dtype)
    c.beta = normal((N,), seed + 5, 0.2, dtype) if with_beta else None
    return c


def config5_ffn_down_norm(norm: str, dtype: str = F16) -> NormCase:
    """The FFN down-projection of the 2048-token FFN (W2 [4096, 11008], x.W^T)
    followed by bias + residual + norm over the 4096-wide hidden dimension:
    the 'MatMul + residual + LayerNorm/RMSNorm' operator of the ops-nn
    article's structural fusion, at the same shape as the FFN workloads."""
    return norm_case(2048, 4096, 11008, dtype, norm, True, 5000 + (norm == "LAYERNORM"))
