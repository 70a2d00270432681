"""Pins for the oracle's MiniMax QK RMSNorm (vLLM minimax_rms_norm/rms_norm_tp
page) and its tensor-parallel "pre" stage (local means of squares).

Independent facts checked:
  * the equal-shard identity: the mean of squares of a row equals the sum of
    its tp_world equal shards' means divided by tp_world; and mode B on one
    shard, given that sum, equals mode A on the whole row restricted to it;
  * mode A on a segment equals torch's own RMSNorm (fp64, CPU) of that segment,
    and equals the separately written fused-epilogue oracle with P = 1;
  * RMS(y) = 1 with unit weights and eps = 0;
  * the v segment is never read (NaN-poisoned v leaves outputs unchanged);
  * tp_world is a pure divisor of the supplied sum.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from residual_add_rmsnorm_amd import workloads
from tests.test_oracle_norm import enc, rand_bf16

Q, K = 48, 16


def _row(rng, T, stride, q=Q, k=K, outliers=True):
    v = rng.standard_normal((T, stride))
    if outliers:
        v[rng.random((T, stride)) < 0.01] *= 50
    return oracle.bf16_encode(v)


def test_shard_means_sum_over_world_is_the_full_mean():
    rng = np.random.default_rng(21)
    T, tp = 7, 4
    shards = [_row(rng, T, 2 * (Q + K)) for _ in range(tp)]
    full_q = np.concatenate([s[:, :Q] for s in shards], axis=1)
    full_k = np.concatenate([s[:, Q:Q + K] for s in shards], axis=1)
    full = np.ascontiguousarray(np.concatenate([full_q, full_k], axis=1))
    m_full = oracle.qk_means(full, tp * Q, tp * K)
    m_sum = sum(oracle.qk_means(s, Q, K) for s in shards)
    np.testing.assert_allclose(m_sum / tp, m_full, rtol=1e-14)


def test_mode_b_on_a_shard_equals_mode_a_on_the_full_row():
    rng = np.random.default_rng(22)
    T, tp, stride = 9, 4, 2 * (Q + K)
    shards = [_row(rng, T, stride) for _ in range(tp)]
    wq = [oracle.bf16_encode(1 + 0.1 * rng.standard_normal(Q)) for _ in range(tp)]
    wk = [oracle.bf16_encode(1 + 0.1 * rng.standard_normal(K)) for _ in range(tp)]
    var_in = sum(oracle.qk_means(s, Q, K) for s in shards).astype(np.float32)
    full = np.ascontiguousarray(np.concatenate(
        [np.concatenate([s[:, :Q] for s in shards], 1),
         np.concatenate([s[:, Q:Q + K] for s in shards], 1)], 1))
    full_out = oracle.qk_rmsnorm(full, tp * Q, tp * K, np.concatenate(wq), np.concatenate(wk),
                                 1e-6, want_pre=True)
    for r in range(tp):
        got = oracle.qk_rmsnorm(shards[r], Q, K, wq[r], wk[r], 1e-6, tp_world=tp,
                                var_in=var_in, want_pre=True)
        # var_in is fp32: relative 2^-24 on the variance, half that on the rsqrt
        np.testing.assert_allclose(got["yq"], full_out["yq"][:, r * Q:(r + 1) * Q], rtol=1e-7)
        np.testing.assert_allclose(got["yk"], full_out["yk"][:, r * K:(r + 1) * K], rtol=1e-7)


def test_tp_world_is_a_divisor_of_the_supplied_sum():
    rng = np.random.default_rng(23)
    T, stride = 5, 80
    qkv = _row(rng, T, stride)
    wq, wk = rand_bf16(rng, Q), rand_bf16(rng, K)
    m = oracle.qk_means(qkv, Q, K)
    a = oracle.qk_rmsnorm(qkv, Q, K, wq, wk, 1e-6, tp_world=1, var_in=m.astype(np.float32),
                          want_pre=True)
    b = oracle.qk_rmsnorm(qkv, Q, K, wq, wk, 1e-6, tp_world=4,
                          var_in=(4 * m).astype(np.float32), want_pre=True)
    assert np.array_equal(a["yq"], b["yq"]) and np.array_equal(a["yk"], b["yk"])
    # and mode A equals mode B fed its own local means (up to fp32 var_in)
    c = oracle.qk_rmsnorm(qkv, Q, K, wq, wk, 1e-6, want_pre=True)
    np.testing.assert_allclose(a["yq"], c["yq"], rtol=1e-7)


@pytest.mark.parametrize("q,k", [(48, 16), (6144, 1024)])
def test_mode_a_matches_torch_rms_norm(q, k):
    rng = np.random.default_rng(q)
    T = 6
    qkv = _row(rng, T, q + 2 * k)
    wq = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(q))
    wk = oracle.bf16_encode(1 + 0.1 * rng.standard_normal(k))
    eps = float(np.float32(1e-6))
    out = oracle.qk_rmsnorm(qkv, q, k, wq, wk, eps, want_pre=True)
    xv = torch.from_numpy(oracle.bf16_decode(qkv))
    ref_q = F.rms_norm(xv[:, :q], (q,), torch.from_numpy(oracle.bf16_decode(wq)), eps).numpy()
    ref_k = F.rms_norm(xv[:, q:q + k], (k,), torch.from_numpy(oracle.bf16_decode(wk)), eps).numpy()
    np.testing.assert_allclose(out["yq"], ref_q, rtol=1e-12)
    np.testing.assert_allclose(out["yk"], ref_k, rtol=1e-12)


def test_mode_a_matches_the_fused_epilogue_oracle():
    rng = np.random.default_rng(24)
    T, stride = 8, 96
    qkv = _row(rng, T, stride)
    wq, wk = rand_bf16(rng, Q), rand_bf16(rng, K)
    out = oracle.qk_rmsnorm(qkv, Q, K, wq, wk, 1e-6, want_pre=True)
    zq = enc(np.zeros((T, Q)))
    fq = oracle.fused_add_rmsnorm([np.ascontiguousarray(qkv[:, :Q])], zq, wq, 1e-6,
                                  want_pre=True)
    np.testing.assert_allclose(out["yq"], fq["y"], rtol=1e-15)
    assert np.array_equal(out["q"], fq["norm"])


def test_unit_rms_and_strided_rows():
    rng = np.random.default_rng(25)
    T, stride = 11, 136                                # row stride > q + 2k
    qkv = _row(rng, T, stride)
    out = oracle.qk_rmsnorm(qkv, Q, K, enc(np.ones(Q)), enc(np.ones(K)), 0.0, want_pre=True)
    np.testing.assert_allclose((out["yq"] ** 2).mean(1), 1.0, rtol=1e-12)
    np.testing.assert_allclose((out["yk"] ** 2).mean(1), 1.0, rtol=1e-12)


def test_v_segment_never_read():
    rng = np.random.default_rng(26)
    T, stride = 6, Q + 2 * K
    qkv = _row(rng, T, stride)
    wq, wk = rand_bf16(rng, Q), rand_bf16(rng, K)
    a = oracle.qk_rmsnorm(qkv, Q, K, wq, wk, 1e-6)
    poisoned = qkv.copy()
    poisoned[:, Q + K:] = 0x7FC0                     # NaN
    b = oracle.qk_rmsnorm(poisoned, Q, K, wq, wk, 1e-6)
    assert np.array_equal(a["q"], b["q"]) and np.array_equal(a["k"], b["k"])


def test_workload_generator_shapes_and_determinism():
    w = workloads.WORKLOADS["qk_sharded"]
    a = workloads.make_inputs(w, T=16)
    b = workloads.make_inputs(w, T=16)
    assert a.qkv.shape == (16, 8192) and len(a.shards) == 3
    assert torch.equal(a.qkv, b.qkv) and torch.equal(a.shards[2], b.shards[2])
    n = workloads.make_inputs(workloads.WORKLOADS["prefill_fp8_token"], T=4)
    assert len(n.partials) == 8 and n.partials[0].shape == (4, 8192)
    # outliers are exact powers-of-two multiples (x64) of bf16 draws
    big = np.abs(workloads.bits(n.partials[0]).view(np.int16).astype(np.int32) & 0x7FFF)
    assert big.max() > 0
