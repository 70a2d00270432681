"""Pins for the oracle's fused add + RMSNorm (no quantisation).

What fixes the answer here, independent of the oracle's own code:
  * hand-derived fp32 partial-sum cases and closed-form rows (tests/golden),
  * exact integer sums, permutation invariance when the sum is exact,
  * the fp32 summation error bound against an fp64 sum of the same terms,
  * RMS(y) = 1 with unit weight and eps = 0, scale invariance,
  * torch's own RMSNorm (``torch.nn.functional.rms_norm``) in fp64 on the CPU,
    the textbook special case P = 1 with a zero partial.
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def enc(v):
    """fp64 values that must be exact bf16 -> uint16 bits."""
    v = np.asarray(v, np.float64)
    b = oracle.bf16_encode(v)
    assert np.array_equal(oracle.bf16_decode(b), v), "value not representable in bf16"
    return b


def rand_bf16(rng, shape, scale=1.0):
    return oracle.bf16_encode(rng.standard_normal(shape) * scale)


def test_golden_fp32_partial_sum_order():
    with open(os.path.join(GOLDEN, "fp32_partial_sum_order.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        P = len(case["partials"])
        H = 8
        parts = [enc(np.full((1, H), v)) for v in case["partials"]]
        res = enc(np.full((1, H), case["residual"]))
        out = oracle.fused_add_rmsnorm(parts, res, enc(np.ones(H)), 1e-6, want_pre=True)
        x = out["x"].astype(np.float64)
        assert np.all(x == case["x_fp32"]), case["name"]
        if case["x_fp32"] == 0.0:
            assert not np.signbit(x).any(), case["name"]
        assert P == len(parts)


def test_golden_closed_form_rows():
    with open(os.path.join(GOLDEN, "rmsnorm_closed_forms.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        row = enc(np.array([case["row"]], np.float64))
        zero = enc(np.zeros_like(np.array([case["row"]], np.float64)))
        w = enc(np.array(case["weight"], np.float64))
        out = oracle.fused_add_rmsnorm([row], zero, w, case["eps"])
        want = np.array([int(h, 16) for h in case["norm_bf16_hex"]], np.uint16)
        assert np.array_equal(out["norm"][0], want), case["name"]
        assert np.array_equal(out["residual"], row)


@pytest.mark.parametrize("P", [1, 2, 3, 8, 16])
def test_integer_sums_are_exact_and_order_free(P):
    rng = np.random.default_rng(P)
    T, H = 5, 64
    ints = rng.integers(-16, 17, size=(P, T, H))
    resid = rng.integers(-16, 17, size=(T, H))
    parts = [enc(ints[p].astype(np.float64)) for p in range(P)]
    w = rand_bf16(rng, H)
    out = oracle.fused_add_rmsnorm(parts, enc(resid.astype(np.float64)), w, 1e-6, want_pre=True)
    exact = ints.sum(0) + resid                      # integers, exact in fp32
    assert np.array_equal(out["x"].astype(np.float64), exact.astype(np.float64))
    assert np.array_equal(out["residual"], oracle.bf16_encode(exact.astype(np.float64)))
    perm = rng.permutation(P)
    out2 = oracle.fused_add_rmsnorm([parts[i] for i in perm], enc(resid.astype(np.float64)), w,
                                    1e-6, want_pre=True)
    assert np.array_equal(out2["norm"], out["norm"])
    assert np.array_equal(out2["residual"], out["residual"])


def test_partial_sum_within_fp32_error_bound():
    # |fl32(sum) - sum| <= gamma_n * sum|terms| with gamma_n = n*u/(1-n*u), u = 2^-24,
    # n = P additions (P - 1 between partials, one for the residual; 0 + p0 is exact).
    rng = np.random.default_rng(7)
    P, T, H = 8, 16, 512
    parts = [rand_bf16(rng, (T, H), 0.35) for _ in range(P)]
    res = rand_bf16(rng, (T, H))
    out = oracle.fused_add_rmsnorm(parts, res, enc(np.ones(H)), 1e-6, want_pre=True)
    terms = np.stack([oracle.bf16_decode(p) for p in parts] + [oracle.bf16_decode(res)])
    exact = terms.sum(0)                             # exact for these inputs in fp64
    u = 2.0**-24
    gamma = P * u / (1 - P * u)
    err = np.abs(out["x"].astype(np.float64) - exact)
    assert np.all(err <= gamma * np.abs(terms).sum(0))
    # and dropping any single term would break the bound somewhere
    for k in range(P + 1):
        wrong = exact - terms[k]
        assert np.any(np.abs(out["x"] - wrong) > gamma * np.abs(terms).sum(0))


def test_unit_rms_with_unit_weight_and_zero_eps():
    rng = np.random.default_rng(3)
    P, T, H = 3, 20, 1000
    parts = [rand_bf16(rng, (T, H), 0.5) for _ in range(P)]
    out = oracle.fused_add_rmsnorm(parts, rand_bf16(rng, (T, H)), enc(np.ones(H)), 0.0,
                                   want_pre=True)
    ms = (out["y"] ** 2).mean(axis=1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-12)


def test_scale_invariance_power_of_two_exact():
    rng = np.random.default_rng(4)
    T, H = 6, 256
    base = rand_bf16(rng, (T, H))
    zero = enc(np.zeros((T, H)))
    w = rand_bf16(rng, H)
    ref = oracle.fused_add_rmsnorm([base], zero, w, 0.0, want_pre=True)
    for k in (-20, -3, 5, 40):
        scaled = oracle.bf16_encode(oracle.bf16_decode(base) * 2.0**k)
        got = oracle.fused_add_rmsnorm([scaled], zero, w, 0.0, want_pre=True)
        assert np.array_equal(got["y"], ref["y"])
        assert np.array_equal(got["norm"], ref["norm"])


def test_scale_invariance_integer_rows():
    # c*x stays exact in bf16 for small integer rows and c = 3
    rng = np.random.default_rng(5)
    T, H = 4, 64
    ints = rng.integers(-20, 21, size=(T, H)).astype(np.float64)
    zero = enc(np.zeros((T, H)))
    w = rand_bf16(rng, H)
    a = oracle.fused_add_rmsnorm([enc(ints)], zero, w, 0.0, want_pre=True)
    b = oracle.fused_add_rmsnorm([enc(3 * ints)], zero, w, 0.0, want_pre=True)
    np.testing.assert_allclose(b["y"], a["y"], rtol=1e-12, atol=0)


def test_constant_and_spike_rows_closed_form():
    H = 96
    eps = np.float32(1e-6)
    for c in (0.5, 3.0, -7.0, 1e-3):
        cb = float(oracle.bf16_decode(oracle.bf16_encode(np.array([c])))[0])
        out = oracle.fused_add_rmsnorm([enc(np.full((1, H), cb))], enc(np.zeros((1, H))),
                                       enc(np.ones(H)), float(eps), want_pre=True)
        np.testing.assert_allclose(out["y"], cb / np.sqrt(cb * cb + float(eps)), rtol=1e-14)
    a = 6.0
    row = np.zeros((1, H)); row[0, 17] = a
    out = oracle.fused_add_rmsnorm([enc(row)], enc(np.zeros((1, H))), enc(np.ones(H)),
                                   float(eps), want_pre=True)
    want = np.zeros((1, H)); want[0, 17] = a / np.sqrt(a * a / H + float(eps))
    np.testing.assert_allclose(out["y"], want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("H", [8, 1024, 7168])
def test_textbook_rmsnorm_matches_torch(H):
    # P = 1 with an all-zero partial: x is the residual itself, and the result is
    # the textbook RMSNorm that torch implements as F.rms_norm.
    rng = np.random.default_rng(H)
    T = 9
    res = rand_bf16(rng, (T, H))
    w = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(H))
    eps = float(np.float32(1e-6))
    out = oracle.fused_add_rmsnorm([enc(np.zeros((T, H)))], res, w, eps, want_pre=True)
    xt = torch.from_numpy(oracle.bf16_decode(res))
    wt = torch.from_numpy(oracle.bf16_decode(w))
    ref = F.rms_norm(xt, (H,), wt, eps).numpy()
    np.testing.assert_allclose(out["y"], ref, rtol=1e-12, atol=1e-300)
    assert np.array_equal(out["norm"], oracle.bf16_encode(ref))


def test_eps_is_the_fp32_value_inside_the_rsqrt():
    # eps = 0.1 is not exact in fp32; the oracle uses the fp32 value (what the
    # C interface receives), added to the mean of squares.
    H = 16
    out = oracle.fused_add_rmsnorm([enc(np.ones((1, H)))], enc(np.zeros((1, H))),
                                   enc(np.ones(H)), 0.1, want_pre=True)
    e32 = float(np.float32(0.1))
    np.testing.assert_array_equal(out["y"][0], 1.0 / np.sqrt(1.0 + e32))


def test_norm_is_taken_from_unrounded_x():
    # x = 1 + 2^-23 (fp32) rounds to 1.0 in bf16; the normalised value must see
    # the fp32 x. Put x in column 0 and a large constant elsewhere so the
    # difference is visible in the pre-rounding y.
    H = 8
    tiny = 2.0**-24
    parts = [enc(np.array([[tiny] + [0.0] * 7])), enc(np.array([[tiny] + [0.0] * 7]))]
    res = enc(np.array([[1.0] + [2.0] * 7]))
    out = oracle.fused_add_rmsnorm(parts, res, enc(np.ones(H)), 0.0, want_pre=True)
    x0 = 1.0 + 2.0**-23
    ms = (x0 * x0 + 7 * 4.0) / H
    assert out["x"][0, 0] == np.float32(x0)
    assert out["residual"][0, 0] == 0x3F80
    np.testing.assert_allclose(out["y"][0, 0], x0 / np.sqrt(ms), rtol=1e-15)
