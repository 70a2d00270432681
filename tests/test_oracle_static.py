"""Pins for the oracle's fused epilogue with a static per-tensor FP8 scale
(the scale_factor argument on the tokenspeed trtllm.py page, section
"AllReduce fusion"; read as the dequantisation multiplier, codes =
e4m3(clamp(y / s))).

Independent facts checked:
  * a row with RMS exactly 1, unit weight and eps = 0 has y = x, so its codes
    are the e4m3 codes of x / s, known by hand;
  * brute force: each code is a nearest of all 253 finite e4m3 values to y / s;
  * tiny s saturates every nonzero value to +-448;
  * with s equal to a token's own dynamic scale, the codes equal the dynamic
    per-token variant's (a separately written oracle function), near-ties aside;
  * everything but the codes is identical to the plain fused epilogue.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_norm import enc, rand_bf16
from tests.test_oracle_quant import ALL_FINITE, _inputs


def test_hand_row_unit_rms():
    # x = +-1 everywhere: mean of squares 1, so y = x (unit weight, eps 0)
    x = np.array([[1, -1, 1, 1, -1, -1, 1, -1]], np.float64)
    for s, want in ((1.0, (0x38, 0xB8)), (0.5, (0x40, 0xC0)), (2.0, (0x30, 0xB0)),
                    (1.0 / 448.0, (0x7E, 0xFE))):
        out = oracle.fused_add_rmsnorm_static([enc(x)], enc(np.zeros_like(x)), enc(np.ones(8)),
                                              0.0, s)
        got = out["codes"][0]
        assert list(got) == [want[0] if v > 0 else want[1] for v in x[0]], s


@pytest.mark.parametrize("s", [1e-3, 0.01, 0.05, 0.3])
def test_brute_force_nearest_code(s):
    rng = np.random.default_rng(int(s * 1e4))
    parts, res, w = _inputs(rng, 2, 16, 256, outliers=True)
    out = oracle.fused_add_rmsnorm_static(parts, res, w, 1e-6, s, want_pre=True)
    r = np.clip(out["y"] / np.float64(np.float32(s)), -448, 448)
    table = oracle.e4m3_decode(ALL_FINITE)
    best = np.abs(r[..., None] - table).min(-1)
    got = oracle.e4m3_decode(out["codes"])
    assert np.all(np.abs(np.abs(r - got) - best) <= 1e-9 * np.maximum(np.abs(r), 1.0))


def test_tiny_scale_saturates():
    rng = np.random.default_rng(41)
    parts, res, w = _inputs(rng, 1, 4, 64)
    out = oracle.fused_add_rmsnorm_static(parts, res, w, 1e-6, 1e-30, want_pre=True)
    nz = out["y"] != 0
    assert np.all((out["codes"][nz] & 0x7F) == 0x7E)


def test_token_scale_reproduces_the_dynamic_variant():
    rng = np.random.default_rng(42)
    parts, res, w = _inputs(rng, 3, 1, 512, outliers=True)
    dyn = oracle.fused_add_rmsnorm(parts, res, w, 1e-6, quant="token")
    st = oracle.fused_add_rmsnorm_static(parts, res, w, 1e-6, float(dyn["scales"][0]))
    ok = ~(dyn["near_tie"] | st["near_tie"])
    # the fp32 rounding of the scale moves y / s by at most 2^-24 relative
    assert np.mean(dyn["codes"][ok] == st["codes"][ok]) > 0.999


def test_other_outputs_equal_the_plain_epilogue():
    rng = np.random.default_rng(43)
    parts, res, w = _inputs(rng, 4, 6, 384)
    a = oracle.fused_add_rmsnorm(parts, res, w, 1e-6)
    b = oracle.fused_add_rmsnorm_static(parts, res, w, 1e-6, 0.02)
    assert np.array_equal(a["residual"], b["residual"]) and np.array_equal(a["norm"], b["norm"])
