"""The oracle against its own stored results (tests/golden/oracle_regression.json,
written by tests/golden/make_oracle_regression.py from the oracle alone).

A drift guard, not a pin: any change to the oracle's arithmetic -- a
quantization rule, the exponent's rounding, a mask, the W8A8 block rule --
fails here and must come with a regenerated fixture and a commit message
that names the passage or reading behind it.  Integer codes, scales and
E8M0 bytes must match exactly; float64 outputs to 1e-12 relative (BLAS may
sum in another order on another machine)."""
import json
import os
import sys

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
sys.path.insert(0, GOLDEN)
import make_oracle_regression as M  # noqa: E402


@pytest.fixture(scope="module")
def stored():
    with open(os.path.join(GOLDEN, "oracle_regression.json")) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def fresh():
    return {"attention": M.attention_record(), "linear": M.linear_record()}


def _floats(h):
    return np.array([float.fromhex(x) for x in h])


def _close(a, b):
    a, b = _floats(a), _floats(b)
    assert a.shape == b.shape
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)


def test_cases_unchanged(stored):
    assert stored["attention"]["case"] == M.ATTN and stored["attention"]["rows"] == M.ROWS
    assert stored["linear"]["case"] == M.LIN and stored["linear"]["rows"] == M.LIN_ROWS


@pytest.mark.parametrize("key", ["k_mean", "chan_shift", "q_codes_sha256", "q_scale", "k_codes_sha256", "k_scale",
                                 "v_e4m3_sha256", "v_e8m0_sha256"])
def test_quantized_operands_exact(stored, fresh, key):
    assert fresh["attention"][key] == stored["attention"][key]


@pytest.mark.parametrize("key", ["emulated_pv16", "emulated_pvfp8", "fp64_attention"])
def test_attention_outputs(stored, fresh, key):
    _close(fresh["attention"][key], stored["attention"][key])


def test_linear_layer(stored, fresh):
    for key in ("x_codes_sha256", "x_scale_sha256", "w_codes_sha256", "w_scale"):
        assert fresh["linear"][key] == stored["linear"][key], key
    _close(fresh["linear"]["y_rows"], stored["linear"]["y_rows"])


def test_emulation_close_to_exact_attention(stored):
    """The stored results are sane: the emulated outputs sit near exact
    attention (16-bit P.V closer than FP8), the rows see some keys."""
    ref = _floats(stored["attention"]["fp64_attention"])
    assert np.abs(ref).max() > 0.05
    e16 = _floats(stored["attention"]["emulated_pv16"])
    e8 = _floats(stored["attention"]["emulated_pvfp8"])
    cos = lambda a, b: a @ b / np.sqrt((a @ a) * (b @ b))
    assert cos(e16, ref) > 0.999 and cos(e8, ref) > 0.99
    assert np.abs(e16 - ref).max() < np.abs(e8 - ref).max()
