"""Pins for the oracle's all-gather epilogue for MLA (tokenspeed trtllm.py
page, section "AllGather fusion": two RMSNorms over the q_lora_rank and
kv_lora_rank segments with their own weights and eps; 1x128 e4m3 of the q part).

Independent facts checked:
  * each segment is torch's F.rms_norm (fp64, CPU) with its own weight and eps;
  * the eps of one segment does not touch the other segment's output;
  * with equal eps it agrees with the separately written QK oracle;
  * the rope part is never read (NaN-poisoned);
  * q-part codes: the group's amax element gets 0x7E/0xFE, brute-force nearest
    codes, and scale = amax / 448 of the group.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from tests.test_oracle_norm import rand_bf16
from tests.test_oracle_quant import ALL_FINITE

Q, KV, ROPE = 256, 64, 16


def _rows(rng, T):
    r = rand_bf16(rng, (T, Q + KV + ROPE))
    r[:, Q + KV:] = 0x7FC0                    # rope part: NaN, must never be read
    return r


def test_segments_are_torch_rms_norm_with_their_own_eps():
    rng = np.random.default_rng(51)
    T = 7
    rows = _rows(rng, T)
    gx = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(Q))
    gy = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(KV))
    ex, ey = float(np.float32(1e-6)), float(np.float32(0.5))
    out = oracle.ag_dual_rmsnorm(rows, Q, KV, gx, gy, ex, ey, want_pre=True)
    v = torch.from_numpy(oracle.bf16_decode(rows[:, :Q + KV]))
    rx = F.rms_norm(v[:, :Q], (Q,), torch.from_numpy(oracle.bf16_decode(gx)), ex).numpy()
    ry = F.rms_norm(v[:, Q:Q + KV], (KV,), torch.from_numpy(oracle.bf16_decode(gy)), ey).numpy()
    np.testing.assert_allclose(out["yx"], rx, rtol=1e-12)
    np.testing.assert_allclose(out["yy"], ry, rtol=1e-12)
    other = oracle.ag_dual_rmsnorm(rows, Q, KV, gx, gy, ex, 1e-6, want_pre=True)
    assert np.array_equal(other["x"], out["x"]) and not np.array_equal(other["yy"], out["yy"])


def test_equal_eps_agrees_with_the_qk_oracle():
    rng = np.random.default_rng(52)
    rows = _rows(rng, 5)
    gx, gy = rand_bf16(rng, Q), rand_bf16(rng, KV)
    a = oracle.ag_dual_rmsnorm(rows, Q, KV, gx, gy, 1e-6, 1e-6)
    b = oracle.qk_rmsnorm(rows, Q, KV, gx, gy, 1e-6)
    assert np.array_equal(a["x"], b["q"]) and np.array_equal(a["y"], b["k"])


def test_q_part_block_codes():
    rng = np.random.default_rng(53)
    T = 9
    rows = _rows(rng, T)
    gx = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(Q))
    gy = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(KV))
    out = oracle.ag_dual_rmsnorm(rows, Q, KV, gx, gy, 1e-6, 1e-6, quant=True, want_pre=True)
    yx = out["yx"].reshape(T, Q // 128, 128)
    codes = out["codes"].reshape(T, Q // 128, 128)
    amax = np.abs(yx).max(-1)
    np.testing.assert_array_equal(out["scales"], (amax / 448).astype(np.float32))
    idx = np.abs(yx).argmax(-1)
    top = np.take_along_axis(codes, idx[..., None], -1)[..., 0]
    assert np.all((top & 0x7F) == 0x7E)
    r = yx / np.repeat(out["scales"][..., None].astype(np.float64), 128, -1)
    table = oracle.e4m3_decode(ALL_FINITE)
    best = np.abs(r[..., None] - table).min(-1)
    got = oracle.e4m3_decode(codes)
    assert np.all(np.abs(np.abs(r - got) - best) <= 1e-6 * np.maximum(np.abs(r), 1e-3))


def test_hand_rows():
    # x = y = +-1 everywhere, unit gammas: mean of squares 1 in both segments, so
    # x_norm = x / sqrt(1 + x_eps) and y_norm = y / sqrt(1 + y_eps); with x_eps = 0
    # every x group's amax is 1, its scale 1/448 and its codes +-448 = 0x7E / 0xFE.
    T = 3
    sign = np.where(np.arange(Q + KV + ROPE) % 3 == 0, -1.0, 1.0)
    rows = np.tile(oracle.bf16_encode(sign), (T, 1))
    rows[:, Q + KV:] = 0x7FC0
    out = oracle.ag_dual_rmsnorm(rows, Q, KV, oracle.bf16_encode(np.ones(Q)),
                                 oracle.bf16_encode(np.ones(KV)), 0.0, 0.25, quant=True,
                                 want_pre=True)
    np.testing.assert_array_equal(out["yx"], np.tile(sign[:Q], (T, 1)))
    np.testing.assert_allclose(out["yy"], np.tile(sign[Q:Q + KV], (T, 1)) / np.sqrt(1.25),
                               rtol=1e-15)
    np.testing.assert_array_equal(out["scales"], np.float32(1 / 448))
    np.testing.assert_array_equal(out["codes"], np.where(np.tile(sign[:Q], (T, 1)) > 0, 0x7E, 0xFE))
    assert not out["near_tie"].any()
