"""Pins of the CPU oracle against facts that do not come from the oracle.

* hand-worked example of the pages' bias broadcast / ReLU / mask / DRELU_BGRAD
  definitions (tests/golden/worked_example.json);
* brute force on tiny inputs: math.fsum exact sums and Fraction rounding
  (tests/brute.py) for every epilogue, both dtypes, both B layouts, both bias
  orientations, ragged sizes;
* exact integer arithmetic at large K;
* GELU against standard-normal-table values (tests/golden/normal_cdf.json) and
  its symmetry gelu(z) - gelu(-z) = z;
* rounding against hand-derived bit patterns (tests/golden/rounding_cases.json)
  and against numpy's own double->half conversion;
* invariants that relate the epilogues to each other.
"""
import json
import math
import os

import numpy as np
import pytest

import brute
import workloads as wl
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f16(vals):
    return np.asarray(vals, dtype=np.float64).astype(np.float16).view(np.uint16)


# ---------------------------------------------------------------- worked example
def test_worked_example_all_epilogues():
    g = _golden("worked_example.json")
    W = _f16(g["W"]); X = _f16(g["X"])
    bcol = _f16(g["bias_col"]); brow = _f16(g["bias_row"])
    ex = g["expected"]
    M, K, N = 2, 3, 2

    def run(epi, bias=None, per_col=False, aux=None):
        return O.gemm_epilogue(W, X, bias, aux, M, N, K, "f16", epi, False, per_col)

    def vals(r):
        return O.decode_f16(r.out).tolist()

    assert vals(run("DEFAULT")) == ex["DEFAULT"]
    assert vals(run("BIAS", bcol)) == ex["BIAS"]
    assert vals(run("RELU_BIAS", bcol)) == ex["RELU_BIAS"]
    r = run("RELU_AUX_BIAS", bcol)
    assert vals(r) == ex["RELU_BIAS"]
    assert r.mask[:, 0].tolist() == ex["RELU_AUX_BIAS_mask_words"]
    assert np.all(r.mask[:, 1:] == 0)
    assert vals(run("BIAS", brow, per_col=True)) == ex["BIAS_PER_COL"]
    aux = np.zeros((M, O.aux_ld_words(N)), dtype=np.uint32)
    aux[:, 0] = ex["DRELU_BGRAD_mask_words"]
    r = run("DRELU_BGRAD", aux=aux)
    assert vals(r) == ex["DRELU_BGRAD_dZ"]
    assert r.bgrad.tolist() == ex["DRELU_BGRAD_bgrad"]


def test_relu_and_mask_at_exact_zero():
    """ReLU passes z only where z > 0 (Y = ReLU(WX + B)), and the aux mask
    records where it passed, so an exactly zero pre-activation gives output 0
    and mask bit 0.  Hand-worked, M = 1, K = 2, N = 4:
      A = [1, 2];  B columns (1, -0.5), (-1, 0.5), (3, -1), (2, -1)
      acc = [1 - 1, -1 + 1, 3 - 2, 2 - 2] = [0, 0, 1, 0]
    bias 0:  out = [0, 0, 1, 0], mask word = bit 2 = 4;
    bias -1: z = [-1, -1, 0, -1], out = 0, mask word = 0."""
    A = _f16([1.0, 2.0])
    B = _f16([[1.0, -1.0, 3.0, 2.0], [-0.5, 0.5, -1.0, -1.0]])
    for b, want_out, want_word in ((0.0, [0.0, 0.0, 1.0, 0.0], 4), (-1.0, [0.0] * 4, 0)):
        for epi in ("RELU_BIAS", "RELU_AUX_BIAS"):
            r = O.gemm_epilogue(A, B, _f16([b]), None, 1, 4, 2, "f16", epi, False, False)
            assert O.decode_f16(r.out).tolist() == [want_out]
            if epi == "RELU_AUX_BIAS":
                assert r.mask[0].tolist() == [want_word, 0, 0, 0]


# ---------------------------------------------------------------- brute force
BRUTE_SHAPES = [(1, 1, 1), (3, 5, 8), (7, 6, 5), (8, 8, 8), (5, 33, 4), (2, 65, 3)]


@pytest.mark.parametrize("epi", O.EPILOGUES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_brute_force_tiny(epi, dtype):
    for si, (M, N, K) in enumerate(BRUTE_SHAPES):
        for b_trans in (False, True):
            for per_col in (False, True):
                seed = 77 + 13 * si + 2 * b_trans + per_col
                c = wl.random_case(M, N, K, dtype, epi, b_trans, per_col, seed)
                r = O.gemm_epilogue(c.A, c.B, c.bias, c.aux, M, N, K, dtype, epi,
                                    b_trans, per_col)
                if c.aux is None:
                    mask_in = None
                elif epi == "DGELU_BGRAD":
                    mask_in = c.aux.ravel().tolist()
                else:
                    mask_in = c.aux.tolist()
                babs = []
                bout, bmask, bbgrad = brute.fused(
                    c.A.ravel().tolist(), c.B.ravel().tolist(),
                    None if c.bias is None else c.bias.tolist(), mask_in,
                    M, N, K, dtype, epi, b_trans, per_col, col_abs=babs)
                assert r.out.tolist() == bout, (M, N, K, b_trans, per_col)
                if epi == "RELU_AUX_BIAS":
                    assert np.array_equal(O.unpack_mask(r.mask, N), np.array(bmask, bool))
                if epi == "GELU_AUX_BIAS":
                    assert r.zaux.tolist() == bmask
                if epi in ("DRELU_BGRAD", "DGELU_BGRAD"):
                    assert r.bgrad.tolist() == bbgrad
                    np.testing.assert_allclose(r.bgrad_abs, babs, rtol=1e-12, atol=1e-300)


def test_brute_force_row_subset():
    M, N, K = 9, 7, 6
    c = wl.random_case(M, N, K, "f16", "RELU_AUX_BIAS", False, False, 5)
    full = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "RELU_AUX_BIAS", False, False)
    rows = np.array([0, 4, 8])
    sub = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "RELU_AUX_BIAS", False,
                          False, rows=rows)
    assert np.array_equal(sub.out, full.out[rows])
    assert np.array_equal(sub.mask, full.mask[rows])
    c = wl.random_case(M, N, K, "f16", "DRELU_BGRAD", False, False, 6)
    full = O.gemm_epilogue(c.A, c.B, None, c.aux, M, N, K, "f16", "DRELU_BGRAD", False, False)
    sub = O.gemm_epilogue(c.A, c.B, None, c.aux, M, N, K, "f16", "DRELU_BGRAD", False, False,
                          rows=rows)
    assert np.array_equal(sub.out, full.out[rows])
    assert np.array_equal(sub.bgrad, full.bgrad)


# ---------------------------------------------------------------- exact integers
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_integer_exact_large_k(dtype):
    """A, B in {-3..3}: the exact result is an integer computed in Python ints."""
    M, N, K = 4, 40, 4096
    c = wl.random_case(M, N, K, dtype, "BIAS", False, True, 11, kind="int")
    Ai = np.rint(O.decode(c.A, dtype)).astype(np.int64)
    Bi = np.rint(O.decode(c.B, dtype)).astype(np.int64)
    bi = np.rint(O.decode(c.bias, dtype)).astype(np.int64)
    exact = [[sum(int(Ai[i, k]) * int(Bi[k, j]) for k in range(K)) + int(bi[j])
              for j in range(N)] for i in range(M)]
    r = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, dtype, "BIAS", False, True)
    got = O.decode(r.out, dtype)
    # the exact integers are within +-K*9+3, so they are exactly representable
    # in fp16 only below 2048; compare against the exactly rounded integer
    for i in range(M):
        for j in range(N):
            want = brute.f16_value(brute.f16_bits(float(exact[i][j]))) if dtype == "f16" \
                else brute.bf16_value(brute.bf16_bits(float(exact[i][j])))
            assert got[i, j] == want


# ---------------------------------------------------------------- GELU
def test_gelu_against_normal_table():
    g = _golden("normal_cdf.json")
    for z, phi in g["phi"]:
        for zz, pp in ((z, phi), (-z, 1.0 - phi)):
            want = zz * pp
            got = float(O.gelu(np.array([zz]))[0])
            assert abs(got - want) <= 1e-15 * max(1.0, abs(want)), (zz, got, want)


def test_gelu_negative_tail():
    """gelu(-z) = -z Q(z) keeps its relative accuracy far into the tail
    (bf16 outputs can represent values down to ~1e-40)."""
    g = _golden("normal_cdf.json")
    for z, q in g["tail"]:
        got = float(O.gelu(np.array([-z]))[0])
        assert abs(got - (-z * q)) <= 1e-11 * abs(z * q), (z, got, -z * q)


def test_gelu_identities():
    z = np.linspace(-12, 12, 2001)
    g = O.gelu(z)
    # gelu(z) - gelu(-z) = z * (Phi(z) + Phi(-z)) = z
    assert np.max(np.abs(g - O.gelu(-z) - z)) < 1e-13
    assert O.gelu(np.array([0.0]))[0] == 0.0
    # large |z|: gelu -> z, gelu -> 0 from below
    assert abs(O.gelu(np.array([12.0]))[0] - 12.0) < 1e-15
    assert -1e-30 < O.gelu(np.array([-12.0]))[0] <= 0.0
    # strictly below the identity and above the ReLU-minus-bound
    assert np.all(g <= np.maximum(z, 0) + 1e-15)


# ---------------------------------------------------------------- rounding
def test_rounding_golden_cases():
    g = _golden("rounding_cases.json")
    for label, s, hexbits in g["f16"]:
        x = float(s)
        assert int(O.encode_f16(np.array([x]))[0]) == int(hexbits, 16), label
        assert brute.f16_bits(x) == int(hexbits, 16), label
    for label, s, hexbits in g["bf16"]:
        x = float(s)
        assert int(O.encode_bf16(np.array([x]))[0]) == int(hexbits, 16), label
        assert brute.bf16_bits(x) == int(hexbits, 16), label


def test_round_to_format_matches_numpy_half():
    """The generic rounding used for bf16, instantiated for fp16, agrees with
    numpy's independent double->half conversion on many values, including
    subnormals, ties and overflow."""
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200000) * np.exp2(rng.integers(-30, 17, 200000)),
        (np.arange(-5000, 5000) + 0.5) * 2.0 ** -24,          # subnormal ties
        1.0 + (np.arange(0, 4096) + 0.5) * 2.0 ** -10,         # normal ties
        np.array([65504.0, 65519.99, 65520.0, 70000.0, -65520.0]),
    ])
    mine = O.round_to_format(x, 11, -14, 15)
    ref = x.astype(np.float16).astype(np.float64)
    assert np.array_equal(mine, ref, equal_nan=True)


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_bf16_decode_encode_roundtrip():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.decode_bf16(bits)
    fin = np.isfinite(v)
    back = O.encode_bf16(v[fin])
    # -0 and +0 both decode to a zero; compare values for zeros
    assert np.array_equal(O.decode_bf16(back), v[fin])


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_invariants(dtype):
    M, N, K = 37, 70, 48
    c = wl.random_case(M, N, K, dtype, "BIAS", False, False, 21)
    zero = np.zeros_like(c.bias)
    d = O.gemm_epilogue(c.A, c.B, None, None, M, N, K, dtype, "DEFAULT", False, False)
    b0 = O.gemm_epilogue(c.A, c.B, zero, None, M, N, K, dtype, "BIAS", False, False)
    assert np.array_equal(d.out, b0.out)                      # zero bias == DEFAULT
    b = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, dtype, "BIAS", False, False)
    r = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, dtype, "RELU_AUX_BIAS", False, False)
    rv = O.decode(r.out, dtype)
    bv = O.decode(b.out, dtype)
    assert np.all(rv >= 0)                                    # ReLU output >= 0
    assert np.array_equal(rv, np.maximum(bv, 0))              # relu == max(bias_out, 0)
    m = O.unpack_mask(r.mask, N)
    assert np.array_equal(rv, np.where(m, bv, 0.0))           # relu == mask * z
    assert np.array_equal(m, r.z > 0)
    # B_TRANS with the transposed storage gives the same result
    Bt = np.ascontiguousarray(c.B.reshape(K, N).T)
    bt = O.gemm_epilogue(c.A, Bt, c.bias, None, M, N, K, dtype, "BIAS", True, False)
    assert np.array_equal(bt.out, b.out)
    # DRELU_BGRAD: all-ones mask == DEFAULT and bgrad = column sums of acc
    ones = wl.const_mask(M, N, True)
    g1 = O.gemm_epilogue(c.A, c.B, None, ones, M, N, K, dtype, "DRELU_BGRAD", False, False)
    assert np.array_equal(g1.out, d.out)
    colsum = (O.decode(c.A, dtype).reshape(M, K) @ O.decode(c.B, dtype).reshape(K, N)).sum(0)
    assert np.allclose(g1.bgrad, colsum.astype(np.float32), rtol=1e-6, atol=1e-6)
    # all-zeros mask -> dZ = 0 and bgrad = 0 exactly
    z0 = O.gemm_epilogue(c.A, c.B, None, wl.const_mask(M, N, False), M, N, K, dtype,
                         "DRELU_BGRAD", False, False)
    assert np.all(O.decode(z0.out, dtype) == 0) and np.all(z0.bgrad == 0)
    # bgrad equals the column sum of the masked gradient
    rm = wl.random_mask(M, N, 5)
    g = O.gemm_epilogue(c.A, c.B, None, rm, M, N, K, dtype, "DRELU_BGRAD", False, False)
    mm = O.unpack_mask(rm, N)
    acc = O.decode(c.A, dtype).reshape(M, K) @ O.decode(c.B, dtype).reshape(K, N)
    assert np.allclose(g.bgrad, np.where(mm, acc, 0).sum(0), rtol=1e-6, atol=1e-6)


def test_identity_b():
    """B = I: y = round(A + bias)."""
    M, K = 10, 24
    A = wl.normal((M, K), 4, 1.0)
    bias = wl.normal((M,), 5, 1.0)
    eye = np.eye(K).astype(np.float16).view(np.uint16)
    r = O.gemm_epilogue(A, eye, bias, None, M, K, K, "f16", "BIAS", False, False)
    want = (O.decode_f16(A) + O.decode_f16(bias)[:, None]).astype(np.float16).view(np.uint16)
    assert np.array_equal(r.out, want)


def test_mask_pack_roundtrip_and_padding():
    rng = np.random.default_rng(0)
    for n in (1, 31, 32, 33, 100, 128, 129):
        bits = rng.random((5, n)) < 0.5
        w = O.pack_mask(bits)
        assert w.shape == (5, O.aux_ld_words(n))
        assert O.aux_ld_words(n) % 4 == 0
        assert np.array_equal(O.unpack_mask(w, n), bits)
        allbits = O.unpack_mask(w, w.shape[1] * 32)
        assert not allbits[:, n:].any()
    # bit order: column j is bit (j & 31) of word j >> 5
    b = np.zeros((1, 64), bool); b[0, 33] = True
    assert O.pack_mask(b)[0, 1] == 2 and O.pack_mask(b)[0, 0] == 0


def test_ffn_chain_composes():
    tok, H, I = 3, 16, 24
    x = wl.normal((tok, H), 1)
    W1 = wl.normal((I, H), 2, 0.25); b1 = wl.normal((I,), 3, 0.1)
    W2 = wl.normal((H, I), 4, 0.2); b2 = wl.normal((H,), 5, 0.1)
    h, y = O.ffn_block(x, W1, b1, W2, b2, tok, H, I, "f16")
    hb, _, _ = brute.fused(x.ravel().tolist(), W1.ravel().tolist(), b1.tolist(), None,
                           tok, I, H, "f16", "GELU_BIAS", True, True)
    assert h.out.tolist() == hb
    yb, _, _ = brute.fused(np.array(hb, np.uint16).ravel().tolist(), W2.ravel().tolist(),
                           b2.tolist(), None, tok, H, I, "f16", "BIAS", True, True)
    assert y.out.tolist() == yb


# ---------------------------------------------------------------- GEMM + residual + norm
def test_norm_worked_example():
    g = _golden("norm_example.json")
    M, N, K = g["M"], g["N"], g["K"]
    A = _f16(g["A"]).ravel()
    B = _f16(g["B_KxN"]).ravel()
    args = dict(bias=_f16(g["bias"]), residual=_f16(g["residual"]).ravel(),
                gamma=_f16(g["gamma"]), beta=_f16(g["beta"]))
    for kind, key in (("LAYERNORM", "layernorm"), ("RMSNORM", "rmsnorm")):
        r = O.gemm_norm(A, B, args["bias"], args["residual"], args["gamma"],
                        args["beta"] if kind == "LAYERNORM" else None, g[key]["eps"],
                        M, N, K, "f16", kind, False)
        assert np.array_equal(r.out64, np.asarray(g[key]["out"], dtype=np.float64)), kind
        assert np.array_equal(r.out, _f16(g[key]["out"])), kind
        assert np.array_equal(r.rstd, np.asarray(g[key]["rstd"])), kind
        if kind == "LAYERNORM":
            assert np.array_equal(r.mean, np.asarray(g[key]["mean"], dtype=np.float64))


@pytest.mark.parametrize("kind", ["LAYERNORM", "RMSNORM"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_norm_brute_force_tiny(kind, dtype):
    rng = np.random.default_rng(77)
    for M, N, K, bt, with_bias, with_res in ((3, 5, 7, False, True, True), (2, 8, 4, True, True, False),
                                             (4, 6, 9, True, False, True), (1, 3, 2, False, False, False)):
        def draw(*shape, scale=1.0):
            v = (rng.standard_normal(shape) * scale).astype(np.float32)
            return wl.to_bits(v, dtype).ravel()
        A = draw(M, K)
        B = draw(N, K) if bt else draw(K, N)
        bias = draw(N, scale=0.5) if with_bias else None
        res = draw(M, N) if with_res else None
        gamma = draw(N)
        beta = draw(N, scale=0.3) if kind == "LAYERNORM" else None
        eps = 1e-5
        bits, vals = brute.norm(A, B, bias, res, gamma, beta, eps, M, N, K, dtype, kind, bt)
        r = O.gemm_norm(A, B, bias, res, gamma, beta, eps, M, N, K, dtype, kind, bt)
        assert np.allclose(r.out64, np.asarray(vals), rtol=1e-12, atol=1e-12)
        assert np.array_equal(r.out, np.asarray(bits, dtype=np.uint16))


def test_norm_closed_forms():
    """Constant rows: LayerNorm gives beta exactly; RMSNorm gives
    c / sqrt(c^2 + eps) * gamma."""
    M, N, K = 3, 16, 4
    A = _f16(np.zeros((M, K))).ravel()
    B = _f16(np.ones((K, N))).ravel()
    consts = np.array([1.5, -2.0, 0.0])
    res = _f16(np.repeat(consts[:, None], N, axis=1)).ravel()
    gamma = _f16(np.linspace(-1, 1, N))
    beta = _f16(np.linspace(0.25, 2.0, N))
    eps = 0.0625
    ln = O.gemm_norm(A, B, None, res, gamma, beta, eps, M, N, K, "f16", "LAYERNORM", False)
    assert np.array_equal(ln.out, np.tile(beta, (M, 1)))
    rms = O.gemm_norm(A, B, None, res, gamma, None, eps, M, N, K, "f16", "RMSNORM", False)
    g = O.decode(gamma, "f16")
    want = consts[:, None] / np.sqrt(consts[:, None] ** 2 + eps) * g[None, :]
    assert np.allclose(rms.out64, want, rtol=1e-15, atol=1e-15)


def test_norm_invariants():
    rng = np.random.default_rng(5)
    M, N, K = 6, 40, 24
    A = wl.to_bits(rng.standard_normal((M, K)).astype(np.float32), "f16").ravel()
    B = wl.to_bits(rng.standard_normal((K, N)).astype(np.float32), "f16").ravel()
    ones = _f16(np.ones(N))
    zeros = _f16(np.zeros(N))
    ln = O.gemm_norm(A, B, None, None, ones, zeros, 1e-3, M, N, K, "f16", "LAYERNORM", False)
    y = ln.y
    var = y.var(axis=1)
    # normalised rows: mean 0, mean square var / (var + eps)
    assert np.allclose(ln.out64.mean(axis=1), 0.0, atol=1e-12)
    assert np.allclose((ln.out64 ** 2).mean(axis=1), var / (var + 1e-3), rtol=1e-12)
    # shift invariance: a per-row constant in the residual changes nothing
    shift = _f16(np.repeat(np.array([0.5, -4, 8, 0, 2, -1])[:, None], N, axis=1)).ravel()
    ln2 = O.gemm_norm(A, B, None, shift, ones, zeros, 1e-3, M, N, K, "f16", "LAYERNORM", False)
    assert np.allclose(ln2.out64, ln.out64, rtol=1e-9, atol=1e-9)
    # RMSNorm: mean square of the output is ms / (ms + eps)
    rms = O.gemm_norm(A, B, None, None, ones, None, 1e-3, M, N, K, "f16", "RMSNORM", False)
    ms = (y * y).mean(axis=1)
    assert np.allclose((rms.out64 ** 2).mean(axis=1), ms / (ms + 1e-3), rtol=1e-12)
    # the GEMM part is the plain product: y equals the DEFAULT epilogue's value
    d = O.gemm_epilogue(A, B, None, None, M, N, K, "f16", "DEFAULT", False, False)
    assert np.array_equal(ln.y, d.y)
    # bias and residual enter y additively, per column and per element
    bias = _f16(np.linspace(-1, 1, N))
    res = wl.to_bits(rng.standard_normal((M, N)).astype(np.float32), "f16").ravel()
    both = O.gemm_norm(A, B, bias, res, ones, zeros, 1e-3, M, N, K, "f16", "LAYERNORM", False)
    want = d.y + O.decode(bias, "f16")[None, :] + O.decode(res, "f16").reshape(M, N)
    assert np.array_equal(both.y, want)
    # rows select rows
    sub = O.gemm_norm(A, B, bias, res, ones, zeros, 1e-3, M, N, K, "f16", "LAYERNORM", False,
                      rows=np.array([4, 1]))
    assert np.array_equal(sub.out, both.out[[4, 1]])



# ---------------------------------------------------------------- GELU backward
def test_gelu_grad_closed_forms():
    """gelu'(z) = Phi(z) + z phi(z): gelu'(0) = 1/2; gelu'(1) and gelu'(-1)
    from the standard-normal table values Phi(1) (tests/golden/normal_cdf.json)
    and phi(1) = exp(-1/2) / sqrt(2 pi); gelu'(z) + gelu'(-z) = 1 (the
    derivative of gelu(z) - gelu(-z) = z); the far tails tend to 1 and 0."""
    Phi1 = dict((float(k), v) for k, v in _golden("normal_cdf.json")["phi"])[1.0]
    phi1 = 0.24197072451914337   # exp(-1/2) / sqrt(2 pi), the standard normal density at 1
    assert O.gelu_grad(np.array([0.0]))[0] == 0.5
    assert abs(O.gelu_grad(np.array([1.0]))[0] - (Phi1 + phi1)) < 1e-12
    assert abs(O.gelu_grad(np.array([-1.0]))[0] - (1.0 - Phi1 - phi1)) < 1e-12
    z = np.linspace(-9, 9, 721)
    assert np.allclose(O.gelu_grad(z) + O.gelu_grad(-z), 1.0, rtol=0, atol=1e-15)
    assert abs(O.gelu_grad(np.array([12.0]))[0] - 1.0) < 1e-15
    assert 0.0 > O.gelu_grad(np.array([-6.0]))[0] > -1e-7


def test_gelu_grad_is_the_derivative_of_gelu():
    """Central differences of the oracle's own gelu agree with gelu_grad."""
    z = np.linspace(-7, 7, 281)
    h = 1e-5
    fd = (O.gelu(z + h) - O.gelu(z - h)) / (2 * h)
    assert np.allclose(fd, O.gelu_grad(z), rtol=0, atol=2e-9)


def test_gelu_aux_and_dgelu_compose():
    """GELU_AUX_BIAS keeps z = the BIAS epilogue's output bits and the same
    out as GELU_BIAS; DGELU_BGRAD with z = 0 everywhere halves the DEFAULT
    product (gelu'(0) = 1/2) and its bgrad is the column sum."""
    M, N, K = 6, 20, 9
    c = wl.random_case(M, N, K, "f16", "GELU_AUX_BIAS", True, True, 12)
    aux = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "GELU_AUX_BIAS", True, True)
    gl = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "GELU_BIAS", True, True)
    bs = O.gemm_epilogue(c.A, c.B, c.bias, None, M, N, K, "f16", "BIAS", True, True)
    assert np.array_equal(aux.out, gl.out) and np.array_equal(aux.zaux, bs.out)
    zeros = np.zeros((M, N), dtype=np.uint16)
    d = O.gemm_epilogue(c.A, c.B, None, zeros, M, N, K, "f16", "DGELU_BGRAD", True, False)
    base = O.gemm_epilogue(c.A, c.B, None, None, M, N, K, "f16", "DEFAULT", True, False)
    assert np.array_equal(d.y, 0.5 * base.y)
    assert np.array_equal(d.bgrad, (0.5 * base.y).sum(axis=0).astype(np.float32))
