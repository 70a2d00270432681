"""Pins for the oracle's FP8 epilogues (per-token and 1x128 block scales).

Independent facts checked:
  * the amax element of every token / group gets the largest code (0x7E / 0xFE);
  * codes do not depend on eps or the row's RMS (the rsqrt cancels in
    y / (amax / 448)), so they are pinned apart from the statistics, and the
    scales are pinned by the RMSNorm values;
  * codes are invariant to scaling the row by 2^k; block codes of a group depend
    only on that group's values;
  * brute force on tiny rows: each code is a nearest e4m3 value to y / scale,
    searched over all 253 finite codes (not the oracle's own search), and the
    dequantised value is within half a code spacing of y;
  * a zero token gets scale 0 and codes 0x00.
"""
import numpy as np
import pytest

import oracle
from tests.test_oracle_norm import enc, rand_bf16

ALL_FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)


def _quant(parts, res, w, eps, quant, **kw):
    return oracle.fused_add_rmsnorm(parts, res, w, eps, quant=quant, want_pre=True, **kw)


def _inputs(rng, P, T, H, sigma=0.5, outliers=False):
    parts = []
    for _ in range(P):
        v = rng.standard_normal((T, H)) * sigma
        if outliers:
            v[rng.random((T, H)) < 0.01] *= 64
        parts.append(oracle.bf16_encode(v))
    return parts, rand_bf16(rng, (T, H)), oracle.bf16_encode(1 + 0.1 * rng.standard_normal(H))


@pytest.mark.parametrize("quant", ["token", "block"])
def test_amax_element_gets_the_top_code(quant):
    rng = np.random.default_rng(11)
    T, H = 12, 512
    parts, res, w = _inputs(rng, 2, T, H, outliers=True)
    out = _quant(parts, res, w, 1e-6, quant)
    y = out["y"]
    G = 1 if quant == "token" else H // 128
    yg = y.reshape(T, G, -1)
    cg = out["codes"].reshape(T, G, -1)
    idx = np.abs(yg).argmax(-1)
    top = np.take_along_axis(cg, idx[..., None], -1)[..., 0]
    sign = np.take_along_axis(yg, idx[..., None], -1)[..., 0] < 0
    assert np.all(top == np.where(sign, 0xFE, 0x7E))
    # scale = amax / 448 as the dequantisation multiplier
    amax = np.abs(yg).max(-1)
    np.testing.assert_array_equal(out["scales"].reshape(T, G), (amax / 448.0).astype(np.float32))


@pytest.mark.parametrize("quant", ["token", "block"])
def test_codes_independent_of_eps_and_rms(quant):
    rng = np.random.default_rng(12)
    T, H = 10, 384
    parts, res, w = _inputs(rng, 3, T, H)
    a = _quant(parts, res, w, 1e-6, quant)
    b = _quant(parts, res, w, 25.0, quant)             # very different rsqrt
    ok = ~(a["near_tie"] | b["near_tie"])
    assert np.array_equal(a["codes"][ok], b["codes"][ok])
    assert ok.mean() > 0.999
    assert not np.allclose(a["scales"], b["scales"])   # the statistics do move


@pytest.mark.parametrize("quant", ["token", "block"])
def test_codes_invariant_to_power_of_two_scaling(quant):
    rng = np.random.default_rng(13)
    T, H = 8, 256
    base = rand_bf16(rng, (T, H))
    zero = enc(np.zeros((T, H)))
    w = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(H))
    ref = _quant([base], zero, w, 0.0, quant)
    for k in (-9, 7):
        s = oracle.bf16_encode(oracle.bf16_decode(base) * 2.0**k)
        got = _quant([s], zero, w, 0.0, quant)
        assert np.array_equal(got["codes"], ref["codes"])
        np.testing.assert_array_equal(got["scales"], ref["scales"])  # eps = 0: y unchanged


def test_block_codes_depend_only_on_their_group():
    rng = np.random.default_rng(14)
    T, H = 4, 1024
    parts, res, w = _inputs(rng, 2, T, H)
    a = _quant(parts, res, w, 1e-6, "block")
    bumped = [p.copy() for p in parts]
    bumped[0][:, 256:384] = oracle.bf16_encode(oracle.bf16_decode(parts[0][:, 256:384]) * 3 + 1)
    b = _quant(bumped, res, w, 1e-6, "block")
    other = np.ones(H, bool); other[256:384] = False
    ok = ~(a["near_tie"] | b["near_tie"])[:, other]
    assert np.array_equal(a["codes"][:, other][ok], b["codes"][:, other][ok])
    assert not np.array_equal(a["codes"][:, 256:384], b["codes"][:, 256:384])
    # other groups' scales change only through the token's rsqrt: by one common ratio
    g_other = [g for g in range(H // 128) if g != 2]
    ratio = (b["scales"][:, g_other].astype(np.float64)
             / a["scales"][:, g_other].astype(np.float64))
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[:, :1], ratio.shape), rtol=3e-7)


@pytest.mark.parametrize("quant,H", [("token", 8), ("token", 16), ("token", 128),
                                     ("block", 128), ("block", 256)])
def test_brute_force_nearest_code_on_tiny_rows(quant, H):
    rng = np.random.default_rng(H + (0 if quant == "token" else 1000))
    T = 64
    parts, res, w = _inputs(rng, 2, T, H, outliers=True)
    out = _quant(parts, res, w, 1e-6, quant)
    y, codes = out["y"], out["codes"]
    scales = out["scales"].reshape(T, -1).astype(np.float64)
    glen = H if quant == "token" else 128
    s = np.repeat(scales, glen, axis=1)
    table = oracle.e4m3_decode(ALL_FINITE)
    r = y / s
    dist = np.abs(r[..., None] - table)               # all 253 finite codes
    best = dist.min(-1)
    got = oracle.e4m3_decode(codes)
    # the chosen code is at the minimum distance (up to the fp32 rounding of the
    # scale, far below a code spacing)
    assert np.all(np.abs(np.abs(r - got) - best) <= 1e-6 * np.maximum(np.abs(r), 1e-3))
    # dequantisation error is at most half the local code spacing
    spacing = np.where(np.abs(got) < 2.0**-6, 2.0**-9,
                       2.0 ** (np.floor(np.log2(np.maximum(np.abs(got), 2.0**-6))) - 3))
    assert np.all(np.abs(got * s - y) <= 0.5 * spacing * s * (1 + 1e-6))


def test_zero_token_and_zero_group():
    T, H = 3, 256
    zero = enc(np.zeros((T, H)))
    w = enc(np.ones(H))
    res = zero.copy()
    res[1, :128] = enc(np.ones((1, 128)))           # token 1: only group 0 nonzero
    for quant in ("token", "block"):
        out = _quant([zero], res, w, 1e-6, quant)
        sc = out["scales"].reshape(T, -1)
        assert np.all(sc[0] == 0) and np.all(out["codes"][0] == 0)
        assert np.all(out["codes"][2] == 0) and np.all(sc[2] == 0)
        if quant == "block":
            assert sc[1, 1] == 0 and np.all(out["codes"][1, 128:] == 0)
            assert np.all(out["codes"][1, :128] == 0x7E)
        else:
            # equal values all sit at amax -> top code; zeros -> 0x00
            assert np.all(out["codes"][1, :128] == 0x7E) and np.all(out["codes"][1, 128:] == 0)


def test_hand_row_per_token():
    # x = [448, 224, -112, 1, 0.5, 0, -0.25, 8] with unit weights, eps 0:
    # y = x * inv, amax = 448 * inv, y / scale = x exactly, so codes are the
    # e4m3 codes of x itself: 0x7E, 0x76, 0xEE, 0x38, 0x30, 0x00, 0xA8, 0x50.
    x = np.array([[448, 224, -112, 1, 0.5, 0, -0.25, 8]], np.float64)
    out = _quant([enc(x)], enc(np.zeros_like(x)), enc(np.ones(8)), 0.0, "token")
    assert list(out["codes"][0]) == [0x7E, 0x76, 0xEE, 0x38, 0x30, 0x00, 0xA8, 0x50]
    ms = (x ** 2).mean()
    np.testing.assert_allclose(out["scales"][0], 448 / np.sqrt(ms) / 448, rtol=1e-7)
