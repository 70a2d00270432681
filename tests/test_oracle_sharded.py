"""Pins for the oracle's sharded-hidden RMSNorm (the single-matrix form of the
MiniMax norm on the tokenspeed trtllm.py page, section "MiniMax QK fused AR +
RMSNorm"; its two stages around the all-reduce as on the vLLM
minimax_rms_norm/rms_norm_tp page).

Independent facts checked:
  * shard identity: the row's mean of squares is the sum of its tp_world equal
    shards' means over tp_world, and the post stage on one shard, given that
    sum, equals torch's RMSNorm of the whole row restricted to the shard;
  * with local statistics it is torch's F.rms_norm (fp64, CPU) on the rows;
  * it agrees with the separately written QK oracle's q segment;
  * tp_world only divides the supplied sum.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
from tests.test_oracle_norm import rand_bf16


def test_shard_identity_against_torch_rms_norm():
    rng = np.random.default_rng(31)
    T, tp, Hl = 9, 4, 40
    full = rand_bf16(rng, (T, tp * Hl))
    w = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(tp * Hl))
    shards = [np.ascontiguousarray(full[:, r * Hl:(r + 1) * Hl]) for r in range(tp)]
    var = sum(oracle.sharded_means(s, Hl) for s in shards)
    np.testing.assert_allclose(var / tp, oracle.sharded_means(full, tp * Hl), rtol=1e-14)
    eps = float(np.float32(1e-6))
    ref = F.rms_norm(torch.from_numpy(oracle.bf16_decode(full)), (tp * Hl,),
                     torch.from_numpy(oracle.bf16_decode(w)), eps).numpy()
    for r in range(tp):
        got = oracle.sharded_rmsnorm(shards[r], Hl, np.ascontiguousarray(w[r * Hl:(r + 1) * Hl]),
                                     eps, tp, var.astype(np.float32), want_pre=True)
        np.testing.assert_allclose(got["y"], ref[:, r * Hl:(r + 1) * Hl], rtol=2e-7)


def test_local_statistics_are_torch_rms_norm_and_strided_rows():
    rng = np.random.default_rng(32)
    T, H, stride = 7, 96, 130
    x = rand_bf16(rng, (T, stride))
    w = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(H))
    eps = float(np.float32(1e-6))
    got = oracle.sharded_rmsnorm(x, H, w, eps, want_pre=True)
    ref = F.rms_norm(torch.from_numpy(oracle.bf16_decode(x[:, :H])), (H,),
                     torch.from_numpy(oracle.bf16_decode(w)), eps).numpy()
    np.testing.assert_allclose(got["y"], ref, rtol=1e-12)
    assert np.array_equal(got["out"], oracle.bf16_encode(ref))


def test_matches_the_qk_oracle_q_segment():
    rng = np.random.default_rng(33)
    T, q, k = 6, 64, 16
    qkv = rand_bf16(rng, (T, q + 2 * k))
    wq, wk = rand_bf16(rng, q), rand_bf16(rng, k)
    a = oracle.qk_rmsnorm(qkv, q, k, wq, wk, 1e-6, want_pre=True)
    b = oracle.sharded_rmsnorm(qkv, q, wq, 1e-6, want_pre=True)
    np.testing.assert_allclose(b["y"], a["yq"], rtol=1e-15)
    np.testing.assert_allclose(oracle.sharded_means(qkv, q), oracle.qk_means(qkv, q, k)[:, 0],
                               rtol=1e-15)


def test_tp_world_divides_the_supplied_sum():
    rng = np.random.default_rng(34)
    x = rand_bf16(rng, (5, 32))
    w = rand_bf16(rng, 32)
    m = oracle.sharded_means(x, 32)
    a = oracle.sharded_rmsnorm(x, 32, w, 1e-6, 1, m.astype(np.float32), want_pre=True)
    b = oracle.sharded_rmsnorm(x, 32, w, 1e-6, 8, (8 * m).astype(np.float32), want_pre=True)
    assert np.array_equal(a["y"], b["y"])
