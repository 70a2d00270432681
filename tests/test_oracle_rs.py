"""Pins for the oracle's reduce-scatter epilogue (tokenspeed trtllm.py page,
sections "ReduceScatter fusion" and "Pattern enums").

Independent facts checked:
  * the addition order (partials, then add_in, then residual) on hand-derived
    fp32 cases (tests/golden/rs_add_in_order.json);
  * slice invariance: the epilogue of a token slice equals the whole-batch
    epilogue restricted to those rows;
  * integer inputs give exact sums including add_in;
  * an all-zero add_in leaves every output of the non-add pattern unchanged;
  * the static-scale patterns on a row of RMS 1 give hand-known codes for the
    scale passed in, and pattern 4 also writes the bf16 norm.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.test_oracle_norm import enc, rand_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_add_in_order():
    with open(os.path.join(GOLDEN, "rs_add_in_order.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        H = 8
        parts = [enc(np.full((1, H), v)) for v in case["partials"]]
        out = oracle.rs_epilogue(oracle.RS_ADD_RESIDUAL_RMSNORM, parts, 0,
                                 enc(np.full((1, H), case["add_in"])),
                                 enc(np.full((1, H), case["residual"])), enc(np.ones(H)), 1e-6)
        x = oracle.bf16_decode(out["residual"])
        assert np.all(x == oracle.bf16_decode(oracle.bf16_encode(np.array([case["x_fp32"]])))), \
            case["name"]
        full = oracle.fused_add_rmsnorm(parts + [enc(np.full((1, H), case["add_in"]))],
                                        enc(np.full((1, H), case["residual"])), enc(np.ones(H)),
                                        1e-6, want_pre=True)
        assert np.all(full["x"] == np.float32(case["x_fp32"])), case["name"]


@pytest.mark.parametrize("pattern", [1, 6, 8, 7])
def test_slice_equals_whole_batch_rows(pattern):
    rng = np.random.default_rng(pattern)
    N, T, H, P = 40, 9, 256, 4
    parts = [rand_bf16(rng, (N, H), 0.5) for _ in range(P)]
    add = rand_bf16(rng, (N, H)) if pattern in (7, 8) else None
    res = rand_bf16(rng, (N, H))
    w = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(H))
    whole = oracle.rs_epilogue(pattern, parts, 0, add, res, w, 1e-6)
    for off in (0, 13, N - T):
        sl = oracle.rs_epilogue(pattern, parts, off,
                                None if add is None else np.ascontiguousarray(add[off:off + T]),
                                np.ascontiguousarray(res[off:off + T]), w, 1e-6)
        for k in ("residual", "norm", "codes", "scales"):
            if whole.get(k) is not None:
                assert np.array_equal(sl[k], whole[k][off:off + T]), (k, off)


def test_integer_sums_with_add_in():
    rng = np.random.default_rng(3)
    T, H, P = 5, 64, 3
    ints = rng.integers(-20, 21, size=(P + 2, T, H)).astype(np.float64)
    out = oracle.rs_epilogue(oracle.RS_ADD_RESIDUAL_RMSNORM, [enc(ints[p]) for p in range(P)], 0,
                             enc(ints[P]), enc(ints[P + 1]), enc(np.ones(H)), 1e-6)
    assert np.array_equal(oracle.bf16_decode(out["residual"]), ints.sum(0))


def test_zero_add_in_changes_nothing():
    rng = np.random.default_rng(4)
    T, H = 6, 384
    parts = [rand_bf16(rng, (T, H)) for _ in range(2)]
    res, w = rand_bf16(rng, (T, H)), oracle.bf16_encode(1 + 0.1 * rng.standard_normal(H))
    a = oracle.rs_epilogue(6, parts, 0, None, res, w, 1e-6)
    b = oracle.rs_epilogue(7, parts, 0, enc(np.zeros((T, H))), res, w, 1e-6)
    for k in ("residual", "codes", "scales"):
        assert np.array_equal(a[k], b[k])


def test_static_patterns_and_rejections():
    rng = np.random.default_rng(5)
    T, H = 4, 128
    parts = [rand_bf16(rng, (T, H))]
    res, w = rand_bf16(rng, (T, H)), enc(np.ones(H))
    two = oracle.rs_epilogue(2, parts, 0, None, res, w, 1e-6, scale_factor=0.01)
    four = oracle.rs_epilogue(4, parts, 0, None, res, w, 1e-6, scale_factor=0.01)
    assert two["norm"] is None and four["norm"] is not None
    assert np.array_equal(two["codes"], four["codes"])
    with pytest.raises(ValueError):
        oracle.rs_epilogue(8, parts, 0, None, res, w, 1e-6)
    with pytest.raises(ValueError):
        oracle.rs_epilogue(3, parts, 0, None, res, w, 1e-6)


@pytest.mark.parametrize("pattern", [2, 4])
def test_static_patterns_hand_row(pattern):
    # one partial of +-1, zero residual, unit weight, eps 0: y = x, codes = e4m3(x / s)
    x = np.array([[1, -1, 1, 1, -1, -1, 1, -1]], np.float64)
    for s_, want in ((0.5, (0x40, 0xC0)), (1.0 / 448.0, (0x7E, 0xFE))):
        out = oracle.rs_epilogue(pattern, [enc(x)], 0, None, enc(np.zeros_like(x)),
                                 enc(np.ones(8)), 0.0, scale_factor=s_)
        assert np.array_equal(out["codes"][0], np.where(x[0] > 0, want[0], want[1]))
        if pattern == 4:
            assert np.array_equal(oracle.bf16_decode(out["norm"]), x)
