"""Mutation check of the oracle's pins: each plausible mistake below is
planted in a copy of oracle/oracle.py (on the CPU, never on a device), the
pin tests of tests/test_oracle_pins.py are run against that copy, and at
least one of them must fail.  A mutant that every pin accepts would be a
mistake the pins cannot see."""
import importlib.util
import inspect
import itertools
import os
import sys
import types
import warnings

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.py")

# (name, text in oracle.py, replacement); the text must occur exactly once
MUTANTS = [
    ("bf16 decode shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("rounding truncates", "y = np.rint(xf / q) * q", "y = np.floor(xf / q) * q"),
    ("rounding keeps one bit too many", "q = np.ldexp(1.0, exp - (sig_bits - 1))",
     "q = np.ldexp(1.0, exp - sig_bits)"),
    ("subnormals not kept", "exp = np.maximum(e - 1, emin)", "exp = e - 1"),
    ("fp16 through fp32 (double rounding)",
     "return np.asarray(y, dtype=np.float64).astype(np.float16).view(np.uint16)",
     "return np.asarray(y, dtype=np.float64).astype(np.float32).astype(np.float16).view(np.uint16)"),
    ("bf16 through fp32 (double rounding)", "r = round_to_format(y, 8, -126, 127)",
     "r = round_to_format(np.asarray(y, dtype=np.float32).astype(np.float64), 8, -126, 127)"),
    ("GELU sign of the erfc argument", "return 0.5 * z * _erfc(-z / math.sqrt(2.0))",
     "return 0.5 * z * _erfc(z / math.sqrt(2.0))"),
    ("GELU without the half", "return 0.5 * z * _erfc(-z / math.sqrt(2.0))",
     "return z * _erfc(-z / math.sqrt(2.0))"),
    ("GELU gradient drops z", "return Phi + z * phi", "return Phi + phi"),
    ("GELU gradient density scale", "np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)",
     "np.exp(-0.5 * z * z) / math.sqrt(math.pi)"),
    ("mask pitch", "return ((n + 31) // 32 + 3) // 4 * 4", "return ((n + 31) // 32 + 1) // 2 * 2"),
    ("mask bit order (pack)", "weights = np.uint64(1) << np.arange(32, dtype=np.uint64)",
     "weights = np.uint64(1) << np.arange(31, -1, -1, dtype=np.uint64)"),
    ("mask bit order (unpack)", "bits = (words[:, :, None] >> shifts) & np.uint32(1)",
     "bits = (words[:, :, None] >> (np.uint32(31) - shifts)) & np.uint32(1)"),
    ("B_TRANS ignored", "    if b_trans:\n        B64 = B64.T\n    all_rows",
     "    if b_trans:\n        B64 = B64.reshape(K, N)\n    all_rows"),
    ("last k term dropped", "acc = A64[comp_rows] @ B64 ", "acc = A64[comp_rows, :-1] @ B64[:-1] "),
    ("per-column bias dropped", "z = acc + b64[None, :N]", "z = acc"),
    ("per-row bias indexed by column", "z = acc + b64[comp_rows][:, None]",
     "z = acc + np.resize(b64, N)[None, :]"),
    ("ReLU leaks", "y = np.where(z > 0, z, 0.0)\n", "y = np.where(z > 0, z, 0.01 * z)\n"),
    ("mask tie at zero", "mask_words = pack_mask(z > 0)", "mask_words = pack_mask(z >= 0)"),
    ("mask from the activation", "mask_words = pack_mask(z > 0)", "mask_words = pack_mask(y > 1e-3)"),
    ("DRELU mask inverted", "y = np.where(m, z, 0.0)", "y = np.where(m, 0.0, z)"),
    ("DRELU bgrad unmasked", "y = np.where(m, z, 0.0)\n        bgrad = y.sum(axis=0)",
     "y = np.where(m, z, 0.0)\n        bgrad = z.sum(axis=0)"),
    ("DGELU gradient of the accumulator", "y = z * gelu_grad(zs)", "y = z * gelu_grad(z)"),
    ("GELU_AUX saves the activation", "zaux = encode(z, dtype)", "zaux = encode(y, dtype)"),
    ("norm: unbiased variance", "var = (d * d).mean(axis=1)",
     "var = (d * d).sum(axis=1) / (d.shape[1] - 1)"),
    ("norm: eps outside the root", "rstd = 1.0 / np.sqrt(var + eps)", "rstd = 1.0 / (np.sqrt(var) + eps)"),
    ("norm: residual dropped", "y = y + decode(np.asarray(residual).reshape(M, N), dtype)[rows]", "y = y"),
    ("norm: beta subtracted", "out64 = out64 + decode(np.asarray(beta), dtype)[None, :N]",
     "out64 = out64 - decode(np.asarray(beta), dtype)[None, :N]"),
    ("norm: gamma dropped", "out64 = d * rstd[:, None] * g", "out64 = d * rstd[:, None]"),
    ("RMSNorm subtracts the mean", "out64 = y * rstd[:, None] * g",
     "out64 = (y - y.mean(axis=1)[:, None]) * rstd[:, None] * g"),
    ("norm: bias dropped", "y = y + decode(np.asarray(bias), dtype)[None, :N]", "y = y"),
]


def _pins_module():
    spec = importlib.util.spec_from_file_location("_pins_under_mutation",
                                                  os.path.join(HERE, "test_oracle_pins.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _mutant_module(src: str) -> types.ModuleType:
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = ORACLE_SRC
    sys.modules["oracle_mutant"] = mod  # dataclasses resolve their module by name
    try:
        exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    finally:
        sys.modules.pop("oracle_mutant", None)
    return mod


def _calls(fn):
    """Every (kwargs) combination of a test function's parametrize marks."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    axes = []
    for m in marks:
        names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
        vals = m.args[1]
        axes.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in vals])
    for combo in itertools.product(*axes) if axes else [()]:
        kw = {}
        for d in combo:
            kw.update(d)
        yield kw


def _pin_tests(pins):
    tests = [(n, f) for n, f in inspect.getmembers(pins, inspect.isfunction)
             if n.startswith("test_") and f.__module__ == pins.__name__]
    # cheap pins first, the large-K integer pin last
    tests.sort(key=lambda t: ("large_k" in t[0], t[0]))
    return tests


def _caught_by(pins, mutant):
    """Name of the first pin test that fails against the mutant, or None."""
    real = pins.O
    pins.O = mutant
    try:
        for name, fn in _pin_tests(pins):
            for kw in _calls(fn):
                try:
                    with warnings.catch_warnings(), np.errstate(all="ignore"):
                        warnings.simplefilter("ignore")
                        fn(**kw)
                except Exception:  # an assertion, or the mutant breaking outright
                    return f"{name}{kw if kw else ''}"
        return None
    finally:
        pins.O = real


def test_pins_pass_on_the_oracle_itself():
    """The harness itself: the unmodified source passes every pin."""
    pins = _pins_module()
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert _caught_by(pins, _mutant_module(src)) is None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_every_mutant_is_caught(name, old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site of '{name}' not unique in oracle.py"
    pins = _pins_module()
    caught = _caught_by(pins, _mutant_module(src.replace(old, new)))
    assert caught is not None, f"no pin catches the mutant '{name}'"
