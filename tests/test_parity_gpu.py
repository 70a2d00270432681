"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Bar (the tolerances stated for this path):
  * residual_out: bit-exact (both sides perform the same fp32 additions in the
    same order, so the stated 1-ulp allowance is not needed);
  * norm_out, q_out, k_out: within 1 bf16 ulp;
  * fp32 scales: relative 1e-6;
  * e4m3 codes: bit-exact except off-by-one codes at near-ties and signed
    zeros, which are counted and printed.
Inputs come from the seeded generator in residual_add_rmsnorm_amd.workloads.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.compare import compare_bf16, compare_e4m3, compare_scales
from residual_add_rmsnorm_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-6


@pytest.fixture(scope="module")
def fn():
    from residual_add_rmsnorm_amd import fusednorm
    return fusednorm


def u16(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def u8(t):
    return t.detach().cpu().contiguous().view(torch.uint8).numpy()


def say(*a):
    print(*a, flush=True)


# ----------------------------------------------------------------------------- helpers

MODES = {"norm": None, "quant_token": "token", "quant_block": "block"}


def run_gpu(fn, inp, mode, want_norm=True, inplace=False):
    parts = [p.to(DEV) for p in inp.partials]
    res = inp.residual.to(DEV)
    w = inp.weight.to(DEV)
    eps = inp.workload.eps
    rout = res if inplace else None
    if mode == "norm":
        norm, rout = fn.fused_add_rmsnorm(parts, res, w, eps, residual_out=rout)
        torch.cuda.synchronize()
        return dict(norm=norm, residual=rout)
    norm = torch.empty_like(res) if want_norm else None
    f = fn.fused_add_rmsnorm_quant_fp8 if mode == "quant_token" else \
        fn.fused_add_rmsnorm_quant_fp8_block
    q, s, rout, norm = f(parts, res, w, eps, norm_out=norm, residual_out=rout)
    torch.cuda.synchronize()
    return dict(norm=norm, residual=rout, codes=q, scales=s)


def run_oracle(inp, mode, want_norm=True, rows=None, want_pre=None):
    """The oracle on the same inputs; with the unrounded normalised values
    whenever norm_out is compared (want_pre None)."""
    if want_pre is None:
        want_pre = mode == "norm" or want_norm
    parts = [wl.bits(p) for p in inp.partials]
    res = wl.bits(inp.residual)
    if rows is not None:
        parts = [np.ascontiguousarray(p[rows]) for p in parts]
        res = np.ascontiguousarray(res[rows])
    return oracle.fused_add_rmsnorm(parts, res, wl.bits(inp.weight), inp.workload.eps,
                                    quant=MODES[mode], want_norm=want_norm, want_pre=want_pre)


def check(gpu, ref, mode, want_norm=True, rows=None, label=""):
    def g(name, conv):
        a = conv(gpu[name])
        return a if rows is None else a[rows]
    rep = [label]
    compare_bf16(g("residual", u16), ref["residual"], max_ulp=0, what="residual_out")
    if mode == "norm" or want_norm:
        # with the oracle's unrounded y, a value one unit off must bracket it
        rep.append(str(compare_bf16(g("norm", u16), ref["norm"], what="norm_out",
                                    exact=ref.get("y") if rows is None else None)))
    if mode != "norm":
        rep.append(str(compare_e4m3(g("codes", u8), ref["codes"], ref["near_tie"])))
        sc = gpu["scales"].cpu().numpy()
        sc = sc if rows is None else sc[rows]
        rel = compare_scales(sc, ref["scales"])
        rep.append(f"scale max rel {rel:.3g}")
    say(" | ".join(rep))


def norm_case(T, H, P, kind="norm", sigma=0.5, outliers=0.0, seed=0):
    w = wl.Workload(f"case", kind, T=T, H=H, P=P, sigma=sigma, outlier_frac=outliers,
                    outlier_mult=64.0, seed=seed)
    return wl.make_inputs(w)


# ----------------------------------------------------------------------------- workloads

@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_workload_norm_full(fn, name):
    inp = wl.make_inputs(wl.WORKLOADS[name])
    check(run_gpu(fn, inp, "norm"), run_oracle(inp, "norm"), "norm", label=name)


@pytest.mark.parametrize("name", ["prefill_fp8_token", "fp8_block"])
@pytest.mark.parametrize("want_norm", [False, True])
def test_workload_quant_reduced(fn, name, want_norm):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w, T=384)
    mode = w.kind
    check(run_gpu(fn, inp, mode, want_norm), run_oracle(inp, mode, want_norm), mode, want_norm,
          label=f"{name} T=384 norm_out={want_norm}")


@pytest.mark.parametrize("name", ["prefill_fp8_token", "fp8_block"])
def test_workload_quant_full_size(fn, name):
    """Full size, in the launch configuration the benchmark times; every token
    against the oracle: residual_out bit-exact, every code and every scale."""
    w = wl.WORKLOADS[name]
    say(f"[{name}] drawing T={w.T} H={w.H} P={w.P}")
    inp = wl.make_inputs(w)
    gpu = run_gpu(fn, inp, w.kind, want_norm=False)
    ref = run_oracle(inp, w.kind, want_norm=False)
    check(gpu, ref, w.kind, want_norm=False, label=f"{name} full size, all {w.T} tokens")
    # a property that holds at any size: every token / group reaches the top code
    codes = u8(gpu["codes"]).reshape(w.T, -1, 128 if w.kind == "quant_block" else w.H)
    assert np.all((codes & 0x7F).max(axis=-1) == 0x7E)


@pytest.mark.parametrize("name", ["qk_local", "qk_sharded"])
def test_workload_qk_full(fn, name):
    w = wl.WORKLOADS[name]
    inp = wl.make_inputs(w)
    qkv = inp.qkv.to(DEV)
    wq, wk = inp.q_weight.to(DEV), inp.k_weight.to(DEV)
    qkv_b = wl.bits(inp.qkv)
    var_in = None
    if w.tp_world > 1:
        rows = [qkv_b] + [wl.bits(s) for s in inp.shards]
        var_in = sum(oracle.qk_means(r, w.q_size, w.kv_size) for r in rows).astype(np.float32)
    q, k = fn.qk_rmsnorm(qkv, w.q_size, w.kv_size, wq, wk, w.eps, w.tp_world,
                         None if var_in is None else torch.from_numpy(var_in).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.qk_rmsnorm(qkv_b, w.q_size, w.kv_size, wl.bits(inp.q_weight),
                            wl.bits(inp.k_weight), w.eps, w.tp_world, var_in, want_pre=True)
    say(name, compare_bf16(u16(q), ref["q"], what="q_out", exact=ref["yq"]),
        compare_bf16(u16(k), ref["k"], what="k_out", exact=ref["yk"]))


# ----------------------------------------------------------------------------- sweeps

SWEEP_NORM = [(H, P) for H in (8, 24, 64, 1000, 1024, 2048, 4096, 4104, 7168, 8192, 16384)
              for P in (1, 3, 8, 16)] + [(7168, P) for P in (2, 4, 5, 6, 7, 9, 12)]


@pytest.mark.parametrize("H,P", SWEEP_NORM)
def test_sweep_norm(fn, H, P):
    inp = norm_case(7, H, P, seed=H * 31 + P)
    check(run_gpu(fn, inp, "norm"), run_oracle(inp, "norm"), "norm", label=f"norm H={H} P={P}")


@pytest.mark.parametrize("H,P", [(H, P) for H in (8, 64, 1000, 4104, 7168, 8192, 16384)
                                 for P in (1, 2, 8, 16)])
def test_sweep_quant_token(fn, H, P):
    inp = norm_case(7, H, P, "quant_token", outliers=0.01, seed=H * 17 + P)
    check(run_gpu(fn, inp, "quant_token"), run_oracle(inp, "quant_token"), "quant_token",
          label=f"token H={H} P={P}")


@pytest.mark.parametrize("H,P", [(H, P) for H in (128, 384, 1152, 7168, 16384)
                                 for P in (1, 2, 5, 16)])
def test_sweep_quant_block(fn, H, P):
    inp = norm_case(7, H, P, "quant_block", outliers=0.01, seed=H * 13 + P)
    check(run_gpu(fn, inp, "quant_block"), run_oracle(inp, "quant_block"), "quant_block",
          label=f"block H={H} P={P}")


@pytest.mark.parametrize("H,T", [(128, 300), (256, 1000), (512, 1000), (512, 4099)])
def test_block_one_wave_workgroups(fn, H, T):
    """Block FP8 on rows of at most 64 vectors with more tokens than CUs: one
    workgroup of a single wave per token, where the token's reduction crosses
    no barrier and the group maxima reach the scale-row store through the
    kernel's own one-wave barrier; every row compared."""
    inp = norm_case(T, H, 3, "quant_block", outliers=0.01, seed=H + T)
    check(run_gpu(fn, inp, "quant_block"), run_oracle(inp, "quant_block"), "quant_block",
          label=f"block one wave H={H} T={T}")


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("T", [1, 255, 4096])
def test_token_counts(fn, mode, T):
    inp = norm_case(T, 7168, 4, mode, seed=T)
    check(run_gpu(fn, inp, mode), run_oracle(inp, mode), mode, label=f"{mode} T={T}")


# ----------------------------------------------------------------------------- edge cases

@pytest.mark.parametrize("mode", list(MODES))
def test_in_place_residual(fn, mode):
    inp = norm_case(33, 4096, 3, mode, seed=77)
    ref = run_oracle(inp, mode)
    gpu = run_gpu(fn, inp, mode, inplace=True)
    check(gpu, ref, mode, label=f"{mode} in-place")


@pytest.mark.parametrize("mode", list(MODES))
def test_zero_and_tiny_tokens(fn, mode):
    inp = norm_case(6, 1024, 2, mode, seed=3)
    for p in inp.partials:
        p[0].zero_()
        p[1].zero_()
    inp.residual[0].zero_()
    inp.residual[1].zero_()
    inp.residual[1, 5] = 1.0                                   # one nonzero channel
    for p in inp.partials:                                     # a row of tiny magnitudes
        p[2] = (p[2].float() * 1e-35).to(torch.bfloat16)
    inp.residual[2] = (inp.residual[2].float() * 1e-35).to(torch.bfloat16)
    check(run_gpu(fn, inp, mode), run_oracle(inp, mode), mode, label=f"{mode} zero/tiny rows")


def test_empty_batch_launches_nothing(fn):
    res = torch.zeros(0, 64, dtype=torch.bfloat16, device=DEV)
    norm, rout = fn.fused_add_rmsnorm([res.clone()], res, torch.ones(64, dtype=torch.bfloat16,
                                                                    device=DEV))
    q, s, r2, _ = fn.fused_add_rmsnorm_quant_fp8([res.clone()], res,
                                                 torch.ones(64, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert norm.shape == (0, 64) and q.shape == (0, 64) and s.shape == (0,)


def test_invalid_arguments_write_nothing(fn):
    T, H = 4, 256
    parts = [torch.randn(T, H, device=DEV).to(torch.bfloat16)]
    res = torch.randn(T, H, device=DEV).to(torch.bfloat16)
    w = torch.ones(H, dtype=torch.bfloat16, device=DEV)
    norm = torch.full((T, H), 7.0, dtype=torch.bfloat16, device=DEV)
    rout = norm.clone()
    with pytest.raises(fn.FusedNormError) as e:
        fn.fused_add_rmsnorm(parts, res, w, -1.0, norm_out=norm, residual_out=rout)
    assert e.value.status == 1
    with pytest.raises(fn.FusedNormUnsupported):
        fn.fused_add_rmsnorm_quant_fp8_block(parts, res, w, group_size=64)
    with pytest.raises(fn.FusedNormUnsupported):   # norm_out aliasing a partial
        fn.fused_add_rmsnorm(parts, res, w, norm_out=parts[0], residual_out=rout)
    with pytest.raises(ValueError):                # binding refuses a short output
        fn.fused_add_rmsnorm(parts, res, w, norm_out=norm[:2], residual_out=rout)
    with pytest.raises(ValueError, match=r"\[T, H\]"):  # a residual that is not [T, H]
        fn.fused_add_rmsnorm_quant_fp8(parts, res.reshape(-1), w)
    torch.cuda.synchronize()
    assert torch.all(norm == 7.0) and torch.all(rout == 7.0)


def test_non_default_stream_and_determinism(fn):
    inp = norm_case(300, 8192, 8, "quant_token", outliers=0.001, seed=9)
    a = run_gpu(fn, inp, "quant_token")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        b = run_gpu(fn, inp, "quant_token")
    s.synchronize()
    for k in ("residual", "codes", "scales", "norm"):
        assert torch.equal(a[k].view(torch.uint8) if k == "codes" else a[k],
                           b[k].view(torch.uint8) if k == "codes" else b[k]), k


# ----------------------------------------------------------------------------- e4m3 conversion

def test_e4m3_encode_midpoints_and_neighbours(fn):
    codes = np.arange(127, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    mid = 0.5 * (vals[:-1] + vals[1:])
    m32 = mid.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mid)           # midpoints are exact in fp32
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(-np.inf))
    extra = np.array([0.0, 448.0, 448.5, 464.0, 480.0, 1e30, 2.0**-10, 2.0**-12, 1e-30,
                      np.float32(2.0**-149)], np.float32)
    x = np.concatenate([m32, up, dn, vals.astype(np.float32), extra])
    x = np.concatenate([x, -x]).astype(np.float32)
    rng = np.random.default_rng(0)
    rnd = (rng.standard_normal(100003) * np.exp2(rng.integers(-12, 9, 100003))).astype(np.float32)
    x = np.concatenate([x, np.clip(rnd, -1e4, 1e4)]).astype(np.float32)
    got = u8(fn.e4m3_encode(torch.from_numpy(x).to(DEV)))
    want = oracle.e4m3_encode(x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4099])
def test_e4m3_encode_ragged_lengths(fn, n):
    x = np.linspace(-500, 500, n).astype(np.float32)
    buf = torch.full((n + 64,), 0xAB, dtype=torch.uint8, device=DEV)
    out = buf[:n]
    fn.e4m3_encode(torch.from_numpy(x).to(DEV), out=out)
    torch.cuda.synchronize()
    assert np.array_equal(u8(out), oracle.e4m3_encode(x.astype(np.float64)))
    assert torch.all(buf[n:] == 0xAB)                            # nothing past the end


# ----------------------------------------------------------------------------- QK edge cases

@pytest.mark.parametrize("q,k,stride", [(8, 8, 24), (48, 16, 96), (48, 16, 200),
                                        (1024, 128, 1280), (6144, 1024, 8192),
                                        (12288, 2048, 16384)])
@pytest.mark.parametrize("supplied", [False, True])
def test_qk_shapes_strides_and_poisoned_v(fn, q, k, stride, supplied):
    T = 37
    g = torch.Generator().manual_seed(q + k + stride)
    base = torch.randn(T, stride, generator=g).to(torch.bfloat16)
    base[:, q + k:] = float("nan")                                 # v and padding: never read
    wq = (1 + 0.1 * torch.randn(q, generator=g)).to(torch.bfloat16)
    wk = (1 + 0.1 * torch.randn(k, generator=g)).to(torch.bfloat16)
    b = wl.bits(base)
    var_in, tp = None, 1
    if supplied:
        var_in = (oracle.qk_means(b, q, k) * 3).astype(np.float32)   # as if 3 equal shards
        tp = 3
    qo, ko = fn.qk_rmsnorm(base.to(DEV), q, k, wq.to(DEV), wk.to(DEV), EPS, tp,
                           None if var_in is None else torch.from_numpy(var_in).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.qk_rmsnorm(b, q, k, wl.bits(wq), wl.bits(wk), EPS, tp, var_in)
    compare_bf16(u16(qo), ref["q"], what="q_out")
    compare_bf16(u16(ko), ref["k"], what="k_out")


def test_qk_strided_view_of_a_wider_tensor(fn):
    T, q, k = 64, 6144, 1024
    big = torch.randn(T, 8192 + 512, dtype=torch.float32).to(torch.bfloat16)
    view = big[:, 256:256 + 8192]                                  # offset 512 B: aligned
    wq = torch.ones(q, dtype=torch.bfloat16)
    wk = torch.ones(k, dtype=torch.bfloat16)
    qo, ko = fn.qk_rmsnorm(big.to(DEV)[:, 256:256 + 8192], q, k, wq.to(DEV), wk.to(DEV))
    torch.cuda.synchronize()
    vb = np.ascontiguousarray(wl.bits(big)[:, 256:256 + 8192])
    ref = oracle.qk_rmsnorm(vb, q, k, wl.bits(wq), wl.bits(wk), EPS)
    compare_bf16(u16(qo), ref["q"], what="q_out")
    compare_bf16(u16(ko), ref["k"], what="k_out")
    assert qo.is_contiguous() and ko.is_contiguous() and view.shape == (T, 8192)


def test_qk_local_means_stage(fn):
    w = wl.WORKLOADS["qk_local"]
    inp = wl.make_inputs(w, T=512)
    var = fn.qk_rmsnorm_var(inp.qkv.to(DEV), w.q_size, w.kv_size)
    torch.cuda.synchronize()
    ref = oracle.qk_means(wl.bits(inp.qkv), w.q_size, w.kv_size)
    rel = compare_scales(var.cpu().numpy(), ref, rtol=1e-6, what="local means")
    say(f"qk local means: max rel {rel:.3g}")


def test_qk_empty_and_invalid(fn):
    qkv = torch.zeros(0, 96, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(48, dtype=torch.bfloat16, device=DEV)
    qo, ko = fn.qk_rmsnorm(qkv, 48, 16, w, w[:16])
    assert qo.shape == (0, 48)
    qkv = torch.zeros(4, 96, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(fn.FusedNormError):
        fn.qk_rmsnorm(qkv, 48, 16, w, w[:16].contiguous(), tp_world=4)


# ----------------------------------------------------------------------------- persistent loop

@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("H,P", [(8, 1), (1024, 3), (4104, 8), (7168, 2), (8192, 8), (16384, 16),
                                 (1152, 5), (2048, 12)])
def test_many_tokens_per_workgroup(fn, mode, H, P):
    """T well above the number of CUs (700 or 1100 tokens, at most 8 per CU):
    rows of at least 14 KiB (7168, 8192, 16384 wide) run on two resident
    workgroups per CU that loop over tokens and prefetch across them; the
    narrower rows run one workgroup per token."""
    if mode == "quant_block" and H % 128:
        pytest.skip("block FP8 needs H % 128 == 0")
    T = 1100 if H <= 8192 else 700
    inp = norm_case(T, H, P, mode, outliers=0.002, seed=H + P)
    check(run_gpu(fn, inp, mode), run_oracle(inp, mode), mode, label=f"{mode} T={T} H={H} P={P}")


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("H,P", [(7168, 2), (8192, 9), (4096, 3)])
@pytest.mark.parametrize("where", ["cus", "cus+1", "8cus", "8cus+1"])
def test_launch_policy_boundaries(fn, mode, H, P, where):
    """Token counts on both sides of the launch rule's boundaries (as many
    tokens as CUs; 8 tokens per CU, up to which wide rows take the persistent
    grid): the grid decides only speed, every shape computes the same result."""
    n = _cus()
    T = {"cus": n, "cus+1": n + 1, "8cus": 8 * n, "8cus+1": 8 * n + 1}[where]
    inp = norm_case(T, H, P, mode, outliers=0.002, seed=T + H + P)
    check(run_gpu(fn, inp, mode), run_oracle(inp, mode), mode, label=f"{mode} T={T} H={H} P={P}")


@pytest.mark.parametrize("mode", ["norm", "quant_token"])
def test_grid_stride_past_the_grid_limit(fn, mode):
    """More tokens than the largest grid (2^20 workgroups): the first 37
    workgroups also take a second token."""
    T, H, P = (1 << 20) + 37, 8, 1
    inp = norm_case(T, H, P, mode, seed=5)
    check(run_gpu(fn, inp, mode), run_oracle(inp, mode), mode, label=f"{mode} T={T} H={H} P={P}")


def test_sharded_grid_stride_past_the_grid_limit(fn):
    T, H = (1 << 20) + 37, 16
    g = torch.Generator().manual_seed(11)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    out = fn.sharded_rmsnorm(x.to(DEV), w.to(DEV), EPS)
    torch.cuda.synchronize()
    ref = oracle.sharded_rmsnorm(wl.bits(x), H, wl.bits(w), EPS)
    compare_bf16(u16(out), ref["out"], what="sharded out")


@pytest.mark.parametrize("q,k,stride,supplied", [(6144, 1024, 8192, False), (6144, 1024, 8192, True),
                                                 (48, 16, 96, False), (1024, 128, 1280, True)])
def test_qk_many_tokens_per_workgroup(fn, q, k, stride, supplied):
    T = 1500
    g = torch.Generator().manual_seed(q + stride)
    base = torch.randn(T, stride, generator=g).to(torch.bfloat16)
    base[:, q + k:] = float("nan")
    wq = (1 + 0.1 * torch.randn(q, generator=g)).to(torch.bfloat16)
    wk = (1 + 0.1 * torch.randn(k, generator=g)).to(torch.bfloat16)
    b = wl.bits(base)
    var_in, tp = (None, 1) if not supplied else ((oracle.qk_means(b, q, k) * 2).astype(np.float32), 2)
    qo, ko = fn.qk_rmsnorm(base.to(DEV), q, k, wq.to(DEV), wk.to(DEV), EPS, tp,
                           None if var_in is None else torch.from_numpy(var_in).to(DEV))
    var = fn.qk_rmsnorm_var(base.to(DEV), q, k)
    torch.cuda.synchronize()
    ref = oracle.qk_rmsnorm(b, q, k, wl.bits(wq), wl.bits(wk), EPS, tp, var_in)
    compare_bf16(u16(qo), ref["q"], what="q_out")
    compare_bf16(u16(ko), ref["k"], what="k_out")
    compare_scales(var.cpu().numpy(), oracle.qk_means(b, q, k), what="local means")


def test_concurrent_calls_from_two_threads(fn):
    import threading
    inps = [norm_case(700, 7168, 2, "quant_block", seed=s) for s in (1, 2)]
    refs = [run_oracle(i, "quant_block") for i in inps]
    errors = []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(10):
                    out = run_gpu(fn, inps[k], "quant_block")
            s.synchronize()
            check(out, refs[k], "quant_block", label=f"thread {k}")
        except Exception as e:  # surfaced below
            errors.append(e)

    ts = [threading.Thread(target=worker, args=(k,)) for k in (0, 1)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors


def test_graph_capture_replays_match_eager(fn):
    """The four launches of a benchmark step captured in a HIP graph: every replay,
    interleaved with eager work and synchronisation, equals the eager result."""
    c = norm_case(1100, 8192, 8, "quant_token", outliers=0.001, seed=5)
    b = norm_case(1100, 7168, 2, "quant_block", seed=6)
    wq = wl.WORKLOADS["qk_local"]
    qk = wl.make_inputs(wq, T=1100)
    dev_c = ([p.to(DEV) for p in c.partials], c.residual.to(DEV), c.weight.to(DEV))
    dev_b = ([p.to(DEV) for p in b.partials], b.residual.to(DEV), b.weight.to(DEV))
    qkv, wqq, wkk = qk.qkv.to(DEV), qk.q_weight.to(DEV), qk.k_weight.to(DEV)
    outs = dict(
        c=(torch.empty_like(dev_c[1]), torch.empty(1100, 8192, dtype=torch.uint8, device=DEV),
           torch.empty(1100, device=DEV)),
        b=(torch.empty_like(dev_b[1]), torch.empty(1100, 7168, dtype=torch.uint8, device=DEV),
           torch.empty(1100, 56, device=DEV)),
        qk=(torch.empty(1100, 6144, dtype=torch.bfloat16, device=DEV),
            torch.empty(1100, 1024, dtype=torch.bfloat16, device=DEV)))

    def step():
        fn.fused_add_rmsnorm_quant_fp8(*dev_c, 1e-6, residual_out=outs["c"][0],
                                       quant_out=outs["c"][1], scale_out=outs["c"][2])
        fn.qk_rmsnorm(qkv, wq.q_size, wq.kv_size, wqq, wkk, 1e-6, q_out=outs["qk"][0],
                      k_out=outs["qk"][1])
        fn.fused_add_rmsnorm_quant_fp8_block(*dev_b, 1e-6, residual_out=outs["b"][0],
                                             quant_out=outs["b"][1], scale_out=outs["b"][2])

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for v in outs.values() for t in v]

    def clear():
        for v in outs.values():
            for t in v:
                t.zero_()

    step()
    eager = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                                     # warm the launch-shape cache off-capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for k in range(4):
        clear()
        torch.cuda.synchronize()
        g.replay()
        got = snapshot()
        for a, e in zip(got, eager):
            assert torch.equal(a, e), f"replay {k} differs from the eager result"
        step()                                     # eager work between replays
        torch.cuda.synchronize()




def test_graph_capture_further_entry_points(fn):
    """The sharded stages, static-scale FP8 and the reduce-scatter epilogue
    (both on the persistent grid of wide rows) and the MLA epilogue captured in one HIP
    graph: every replay, between eager runs, equals the eager result."""
    g_ = torch.Generator().manual_seed(21)
    x = torch.randn(700, 2048, generator=g_).to(torch.bfloat16).to(DEV)
    wx = torch.ones(2048, dtype=torch.bfloat16, device=DEV)
    st = norm_case(600, 8192, 4, "quant_token", seed=22)
    st_dev = ([p.to(DEV) for p in st.partials], st.residual.to(DEV), st.weight.to(DEV))
    scale = torch.tensor([0.02], dtype=torch.float32, device=DEV)
    rs_parts = [(torch.randn(1500, 7168, generator=g_) * 0.5).to(torch.bfloat16).to(DEV)
                for _ in range(3)]
    rs_add = torch.randn(900, 7168, generator=g_).to(torch.bfloat16).to(DEV)
    rs_res = torch.randn(900, 7168, generator=g_).to(torch.bfloat16).to(DEV)
    rs_w = torch.ones(7168, dtype=torch.bfloat16, device=DEV)
    mla_rows = torch.randn(800, 2112, generator=g_).to(torch.bfloat16).to(DEV)
    gx = torch.ones(1536, dtype=torch.bfloat16, device=DEV)
    gy = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    outs = dict(
        var=torch.empty(700, device=DEV), sh=torch.empty(700, 2048, dtype=torch.bfloat16, device=DEV),
        st_q=torch.empty(600, 8192, dtype=torch.uint8, device=DEV), st_r=torch.empty_like(st_dev[1]),
        rs_r=torch.empty_like(rs_res), rs_q=torch.empty(900, 7168, dtype=torch.uint8, device=DEV),
        rs_s=torch.empty(900, 56, device=DEV),
        y=torch.empty(800, 512, dtype=torch.bfloat16, device=DEV),
        c=torch.empty(800, 1536, dtype=torch.uint8, device=DEV), cs=torch.empty(800, 12, device=DEV))

    def step():
        fn.sharded_rmsnorm_var(x, var_out=outs["var"])
        fn.sharded_rmsnorm(x, wx, EPS, 1, outs["var"], out=outs["sh"])
        fn.fused_add_rmsnorm_quant_fp8_static(*st_dev, scale, EPS, residual_out=outs["st_r"],
                                              quant_out=outs["st_q"])
        fn.fused_rs_epilogue(7, rs_parts, 550, rs_res, rs_w, EPS, add_in=rs_add,
                             residual_out=outs["rs_r"], quant_out=outs["rs_q"],
                             scale_out=outs["rs_s"])
        fn.ag_dual_rmsnorm(mla_rows, 1536, 512, gx, gy, EPS, EPS, quant=True, want_x=False,
                           y_norm_out=outs["y"], quant_out=outs["c"], scale_out=outs["cs"])

    def snapshot():
        torch.cuda.synchronize()
        return [t.clone() for t in outs.values()]

    step()
    eager = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for k in range(4):
        for t in outs.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        for name, a, e in zip(outs, snapshot(), eager):
            assert torch.equal(a, e), f"replay {k}: {name} differs from the eager result"
        step()
        torch.cuda.synchronize()

# ----------------------------------------------------------------------------- sharded-hidden RMSNorm

@pytest.mark.parametrize("T", [1, 37, 1500])
@pytest.mark.parametrize("H,stride", [(8, 8), (1536, 1536), (1536, 6144), (2048, 2112),
                                      (6144, 8192), (16384, 16384)])
def test_sharded_rmsnorm(fn, T, H, stride):
    tp = 4
    g = torch.Generator().manual_seed(H + T + stride)
    shards = [torch.randn(T, stride, generator=g).to(torch.bfloat16) for _ in range(tp)]
    for s_ in shards:
        s_[:, H:] = float("nan")                            # past the shard's width: never read
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    bits = [wl.bits(s_) for s_ in shards]
    # pre stage on every rank, then the all-reduce (a sum) and the post stage on rank 0
    dev_shards = [s_.to(DEV) for s_ in shards]
    var = [fn.sharded_rmsnorm_var(d, H=H) for d in dev_shards]
    torch.cuda.synchronize()
    for b, v in zip(bits, var):
        compare_scales(v.cpu().numpy(), oracle.sharded_means(b, H), what="local means")
    var_in = sum(oracle.sharded_means(b, H) for b in bits).astype(np.float32)
    out = fn.sharded_rmsnorm(dev_shards[0], w.to(DEV), EPS, tp, torch.from_numpy(var_in).to(DEV),
                             H=H)
    local = fn.sharded_rmsnorm(dev_shards[0], w.to(DEV), EPS, H=H)
    torch.cuda.synchronize()
    ref = oracle.sharded_rmsnorm(bits[0], H, wl.bits(w), EPS, tp, var_in)
    ref_local = oracle.sharded_rmsnorm(bits[0], H, wl.bits(w), EPS)
    compare_bf16(u16(out), ref["out"], what="sharded out")
    compare_bf16(u16(local), ref_local["out"], what="local out")



# ----------------------------------------------------------------------------- static FP8 scale

@pytest.mark.parametrize("T,H,P", [(7, 1024, 1), (37, 7168, 2), (1100, 8192, 8), (300, 16384, 16),
                                   (600, 4104, 3)])
@pytest.mark.parametrize("scale", [0.004, 0.02, 1.0])
@pytest.mark.parametrize("want_norm", [False, True])
def test_static_scale_quant(fn, T, H, P, scale, want_norm):
    inp = norm_case(T, H, P, "quant_token", outliers=0.002, seed=H + P + T)
    parts = [p.to(DEV) for p in inp.partials]
    res, w = inp.residual.to(DEV), inp.weight.to(DEV)
    norm = torch.empty_like(res) if want_norm else None
    q, rout, norm = fn.fused_add_rmsnorm_quant_fp8_static(parts, res, w, scale, EPS,
                                                          norm_out=norm)
    torch.cuda.synchronize()
    ref = oracle.fused_add_rmsnorm_static([wl.bits(p) for p in inp.partials],
                                          wl.bits(inp.residual), wl.bits(inp.weight), EPS, scale,
                                          want_norm=want_norm)
    compare_bf16(u16(rout), ref["residual"], max_ulp=0, what="residual_out")
    if want_norm:
        compare_bf16(u16(norm), ref["norm"], what="norm_out")
    say(f"static s={scale} T={T} H={H} P={P}:",
        compare_e4m3(u8(q), ref["codes"], ref["near_tie"]))



# ----------------------------------------------------------------------------- reduce-scatter epilogue

@pytest.mark.parametrize("pattern", [1, 2, 4, 6, 7, 8])
@pytest.mark.parametrize("N,T,off,H,P", [(64, 16, 0, 1024, 2), (64, 16, 48, 7168, 8),
                                         (3000, 1100, 1900, 8192, 4), (40, 7, 13, 384, 15)])
def test_rs_epilogue(fn, pattern, N, T, off, H, P):
    if pattern in (7, 8) and P > 15:
        pytest.skip("add_in needs P <= 15")
    g = torch.Generator().manual_seed(pattern * 1000 + N + H)
    parts = [(torch.randn(N, H, generator=g) * 0.5).to(torch.bfloat16) for _ in range(P)]
    add = (torch.randn(T, H, generator=g) * 0.5).to(torch.bfloat16) if pattern in (7, 8) else None
    res = torch.randn(T, H, generator=g).to(torch.bfloat16)
    w = (1 + 0.1 * torch.randn(H, generator=g)).to(torch.bfloat16)
    scale = 0.02 if pattern in (2, 4) else None
    out = fn.fused_rs_epilogue(pattern, [p.to(DEV) for p in parts], off, res.to(DEV), w.to(DEV),
                               EPS, add_in=None if add is None else add.to(DEV),
                               scale_factor=scale)
    torch.cuda.synchronize()
    ref = oracle.rs_epilogue(pattern, [wl.bits(p) for p in parts], off,
                             None if add is None else wl.bits(add), wl.bits(res), wl.bits(w), EPS,
                             scale_factor=scale)
    compare_bf16(u16(out["residual"]), ref["residual"], max_ulp=0, what="residual_out")
    if ref.get("norm") is not None:
        compare_bf16(u16(out["norm"]), ref["norm"], what="norm_out")
    if ref.get("codes") is not None:
        rep = compare_e4m3(u8(out["codes"]), ref["codes"], ref["near_tie"])
        if ref.get("scales") is not None:
            compare_scales(out["scales"].cpu().numpy(), ref["scales"])
        say(f"rs pattern {pattern} N={N} T={T} off={off} H={H} P={P}:", rep)


# ----------------------------------------------------------------------------- MLA all-gather epilogue

@pytest.mark.parametrize("T", [1, 37, 2500])
@pytest.mark.parametrize("q,kv,stride", [(128, 8, 144), (256, 64, 336), (1536, 512, 2112),
                                         (1536, 512, 2176), (3072, 1024, 4160)])
@pytest.mark.parametrize("quant", [False, True])
def test_ag_dual_rmsnorm(fn, T, q, kv, stride, quant):
    g = torch.Generator().manual_seed(q + kv + stride + T)
    rows = torch.randn(T, stride, generator=g).to(torch.bfloat16)
    rows[:, q + kv:] = float("nan")                       # rope part and padding: never read
    if T > 1:
        rows[T // 2, :q + kv] = 0                         # an all-zero token: codes 0, scales 0
        rows[T // 3, :128] = 0                            # an all-zero q group
        rows[T // 4, 5] = 60.0                            # an outlier in one group
    gx = (1 + 0.1 * torch.randn(q, generator=g)).to(torch.bfloat16)
    gy = (1 + 0.1 * torch.randn(kv, generator=g)).to(torch.bfloat16)
    xe, ye = 1e-6, 0.25                                  # the second eps is visible in y
    out = fn.ag_dual_rmsnorm(rows.to(DEV), q, kv, gx.to(DEV), gy.to(DEV), xe, ye, quant=quant,
                             want_x=not quant or T != 37)
    torch.cuda.synchronize()
    ref = oracle.ag_dual_rmsnorm(wl.bits(rows), q, kv, wl.bits(gx), wl.bits(gy), xe, ye,
                                 quant=quant)
    compare_bf16(u16(out["y"]), ref["y"], what="y_norm_out")
    if out["x"] is not None:
        compare_bf16(u16(out["x"]), ref["x"], what="x_norm_out")
    if quant:
        compare_scales(out["scales"].cpu().numpy(), ref["scales"])
        say(f"ag q={q} kv={kv} stride={stride} T={T}:",
            compare_e4m3(u8(out["codes"]), ref["codes"], ref["near_tie"]))



def test_stream_aids(fn):
    # the measurement aids: the copy reproduces its input, the read runs cleanly
    src = torch.arange(3 * 8192, dtype=torch.int32, device=DEV)       # 96 KiB
    dst = torch.empty_like(src)
    fn.stream_copy(src, dst)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    fn.stream_read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


# ----------------------------------------------------------------------------- further entry points, full size

def test_next_sharded_post_full_size(fn):
    """The sharded post stage as the benchmark launches it (16384 rows of 2048,
    supplied sum of 4 ranks' local means); every row against the oracle."""
    w = wl.WORKLOADS["sharded_post"]
    inp = wl.make_inputs(w)
    H = w.q_size
    bits = [wl.bits(inp.qkv)] + [wl.bits(s) for s in inp.shards]
    var_in = sum(oracle.sharded_means(b, H) for b in bits).astype(np.float32)
    out = fn.sharded_rmsnorm(inp.qkv.to(DEV), inp.q_weight.to(DEV), w.eps, w.tp_world,
                             torch.from_numpy(var_in).to(DEV), H=H)
    torch.cuda.synchronize()
    ref = oracle.sharded_rmsnorm(bits[0], H, wl.bits(inp.q_weight), w.eps, w.tp_world, var_in)
    say("sharded_post full size:", compare_bf16(u16(out), ref["out"], what="out"))


def test_next_static_fp8_full_size(fn):
    """Static-scale FP8 as the benchmark launches it; every token against the
    oracle."""
    w = wl.WORKLOADS["static_fp8"]
    say(f"[static_fp8] drawing T={w.T} H={w.H} P={w.P}")
    inp = wl.make_inputs(w)
    q, rout, _ = fn.fused_add_rmsnorm_quant_fp8_static(
        [p.to(DEV) for p in inp.partials], inp.residual.to(DEV), inp.weight.to(DEV),
        torch.tensor([w.static_scale], dtype=torch.float32, device=DEV), w.eps)
    torch.cuda.synchronize()
    ref = oracle.fused_add_rmsnorm_static([wl.bits(p) for p in inp.partials],
                                          wl.bits(inp.residual), wl.bits(inp.weight), w.eps,
                                          w.static_scale)
    compare_bf16(u16(rout), ref["residual"], max_ulp=0, what="residual_out")
    say(f"static_fp8 full size, all {w.T} tokens:",
        compare_e4m3(u8(q), ref["codes"], ref["near_tie"]))


def test_next_rs_fp8_block_full_size(fn):
    """Pattern 7 on the benchmark's slice (2048 of 16384 tokens, 8 partials +
    add_in); every row of the slice against the oracle."""
    w = wl.WORKLOADS["rs_fp8_block"]
    inp = wl.make_inputs(w)
    out = fn.fused_rs_epilogue(w.pattern, [p.to(DEV) for p in inp.partials], w.token_offset,
                               inp.residual.to(DEV), inp.weight.to(DEV), w.eps,
                               add_in=inp.add_in.to(DEV))
    torch.cuda.synchronize()
    ref = oracle.rs_epilogue(w.pattern, [wl.bits(p) for p in inp.partials], w.token_offset,
                             wl.bits(inp.add_in), wl.bits(inp.residual), wl.bits(inp.weight), w.eps)
    compare_bf16(u16(out["residual"]), ref["residual"], max_ulp=0, what="residual_out")
    compare_scales(out["scales"].cpu().numpy(), ref["scales"])
    say("rs_fp8_block full size:", compare_e4m3(u8(out["codes"]), ref["codes"], ref["near_tie"]))


def test_next_mla_full_size(fn):
    """The MLA epilogue as the benchmark launches it (8192 rows, pattern 2,
    no x_norm_out), then pattern 1; every row against the oracle."""
    w = wl.WORKLOADS["mla_ag_fp8"]
    inp = wl.make_inputs(w)
    rows = inp.qkv.to(DEV)
    gx, gy = inp.q_weight.to(DEV), inp.k_weight.to(DEV)
    two = fn.ag_dual_rmsnorm(rows, w.q_size, w.kv_size, gx, gy, w.eps, w.eps, quant=True,
                             want_x=False)
    one = fn.ag_dual_rmsnorm(rows, w.q_size, w.kv_size, gx, gy, w.eps, w.eps)
    torch.cuda.synchronize()
    b = wl.bits(inp.qkv)
    ref = oracle.ag_dual_rmsnorm(b, w.q_size, w.kv_size, wl.bits(inp.q_weight),
                                 wl.bits(inp.k_weight), w.eps, w.eps, quant=True)
    compare_bf16(u16(two["y"]), ref["y"], what="y_norm_out")
    compare_bf16(u16(one["y"]), ref["y"], what="y_norm_out (pattern 1)")
    compare_bf16(u16(one["x"]), ref["x"], what="x_norm_out (pattern 1)")
    compare_scales(two["scales"].cpu().numpy(), ref["scales"])
    say("mla full size:", compare_e4m3(u8(two["codes"]), ref["codes"], ref["near_tie"]))


_FIRST_CALL_UNDER_CAPTURE = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from residual_add_rmsnorm_amd import fusednorm as fn
dev = "cuda:0"
g = torch.Generator().manual_seed(3)
parts = [torch.randn(600, 7168, generator=g).to(torch.bfloat16).to(dev) for _ in range(2)]
res = torch.randn(600, 7168, generator=g).to(torch.bfloat16).to(dev)
w = torch.ones(7168, dtype=torch.bfloat16, device=dev)
q = torch.empty(600, 7168, dtype=torch.uint8, device=dev)
s = torch.empty(600, 56, device=dev)
r = torch.empty_like(res)
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph):   # the library's first call in this process
    fn.fused_add_rmsnorm_quant_fp8_block(parts, res, w, 1e-6, residual_out=r, quant_out=q, scale_out=s)
graph.replay()
torch.cuda.synchronize()
got = (r.clone(), q.clone(), s.clone())
fn.fused_add_rmsnorm_quant_fp8_block(parts, res, w, 1e-6, residual_out=r, quant_out=q, scale_out=s)
torch.cuda.synchronize()
assert all(torch.equal(a, b) for a, b in zip(got, (r, q, s))), "graph replay differs from eager"
print("ok", flush=True)
"""


def test_first_call_inside_a_graph_capture():
    """A process whose first library call is captured (the persistent grid,
    here 600 tokens of 7168, queries the kernel's occupancy on first use)
    replays correctly."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _FIRST_CALL_UNDER_CAPTURE, root], capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout[-2000:] + r.stderr[-2000:]


# ----------------------------------------------------------------------------- seeded random shapes

def _random_epilogue_case(seed):
    """Seeded random valid shape: mode, H (a multiple of 8, of 128 for block
    FP8), P in 1..16, T up to 3000, optional norm_out; at most ~2^25 elements
    over all buffers so the oracle stays quick."""
    rng = np.random.default_rng(1000 + seed)
    mode = ["norm", "quant_token", "quant_block"][seed % 3]
    P = int(rng.integers(1, 17))
    H = int(rng.integers(1, 129)) * 128 if mode == "quant_block" else int(rng.integers(1, 2049)) * 8
    tmax = max(1, min(3000, (1 << 25) // (H * (P + 3))))
    T = int(rng.integers(1, tmax + 1))
    return mode, T, H, P, bool(rng.integers(0, 2))


@pytest.mark.parametrize("seed", range(18))
def test_random_shapes_epilogue(fn, seed):
    mode, T, H, P, want_norm = _random_epilogue_case(seed)
    inp = norm_case(T, H, P, mode, sigma=0.5, outliers=0.001, seed=seed)
    want_norm = want_norm or mode == "norm"
    check(run_gpu(fn, inp, mode, want_norm), run_oracle(inp, mode, want_norm), mode, want_norm,
          label=f"seed {seed}: {mode} T={T} H={H} P={P} norm_out={want_norm}")


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_qk_family(fn, seed):
    """Seeded random QK, sharded and MLA shapes, strides and token counts."""
    rng = np.random.default_rng(2000 + seed)
    kind = ["qk", "sharded", "mla"][seed % 3]
    q = int(rng.integers(1, 97)) * 128 if kind == "mla" else int(rng.integers(1, 1025)) * 8
    k = 0 if kind == "sharded" else int(rng.integers(1, 257)) * 8
    if q + k > 16384:
        q = 16384 - k - (16384 - k) % (128 if kind == "mla" else 8)
    stride = q + k + int(rng.integers(0, 33)) * 8
    T = int(rng.integers(1, max(2, min(3000, (1 << 24) // stride)) + 1))
    g = torch.Generator().manual_seed(3000 + seed)
    rows = torch.randn(T, stride, generator=g).to(torch.bfloat16)
    rows[:, q + k:] = float("nan")                       # past the segments: never read
    wq = (1 + 0.1 * torch.randn(q, generator=g)).to(torch.bfloat16)
    wk = (1 + 0.1 * torch.randn(max(k, 1), generator=g)).to(torch.bfloat16)[:k]
    b = wl.bits(rows)
    label = f"seed {seed}: {kind} T={T} q={q} k={k} stride={stride}"
    if kind == "qk":
        tp = int(rng.integers(1, 5))
        var = None if tp == 1 else (oracle.qk_means(b, q, k) * tp).astype(np.float32)
        qo, ko = fn.qk_rmsnorm(rows.to(DEV), q, k, wq.to(DEV), wk.to(DEV), EPS, tp,
                               None if var is None else torch.from_numpy(var).to(DEV))
        torch.cuda.synchronize()
        ref = oracle.qk_rmsnorm(b, q, k, wl.bits(wq), wl.bits(wk), EPS, tp, var)
        compare_bf16(u16(qo), ref["q"], what="q_out")
        say(label, compare_bf16(u16(ko), ref["k"], what="k_out"))
    elif kind == "sharded":
        tp = int(rng.integers(1, 9))
        var = None if tp == 1 else (oracle.sharded_means(b, q) * tp).astype(np.float32)
        out = fn.sharded_rmsnorm(rows.to(DEV), wq.to(DEV), EPS, tp,
                                 None if var is None else torch.from_numpy(var).to(DEV), H=q)
        torch.cuda.synchronize()
        ref = oracle.sharded_rmsnorm(b, q, wl.bits(wq), EPS, tp, var)
        say(label, compare_bf16(u16(out), ref["out"], what="out"))
    else:
        quant = bool(rng.integers(0, 2))
        out = fn.ag_dual_rmsnorm(rows.to(DEV), q, k, wq.to(DEV), wk.to(DEV), 1e-6, 0.01,
                                 quant=quant)
        torch.cuda.synchronize()
        ref = oracle.ag_dual_rmsnorm(b, q, k, wl.bits(wq), wl.bits(wk), 1e-6, 0.01, quant=quant)
        compare_bf16(u16(out["x"]), ref["x"], what="x_norm_out")
        rep = compare_bf16(u16(out["y"]), ref["y"], what="y_norm_out")
        if quant:
            compare_scales(out["scales"].cpu().numpy(), ref["scales"])
            rep = compare_e4m3(u8(out["codes"]), ref["codes"], ref["near_tie"])
        say(label, rep)


# ----------------------------------------------------------------------------- nothing written past the outputs

GUARD = 4096   # elements of sentinel after each output


def _guarded(shape, dtype, fill):
    n = int(np.prod(shape))
    buf = torch.full((n + GUARD,), fill, dtype=dtype, device=DEV)
    return buf, buf[:n].view(*shape)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("T,H,P", [(37, 7168, 3), (300, 7168, 2), (300, 1000, 5), (37, 4104, 8),
                                   (600, 16384, 2)])
def test_no_write_past_the_outputs(fn, mode, T, H, P):
    """Lanes past a row's end (e.g. 7168-wide rows on 256-thread workgroups) and
    the last token write nothing beyond the outputs: guard bands keep their
    sentinels."""
    if mode == "quant_block" and H % 128:
        pytest.skip("block FP8 needs H % 128 == 0")
    inp = norm_case(T, H, P, mode, seed=T + H)
    parts = [p.to(DEV) for p in inp.partials]
    res, w = inp.residual.to(DEV), inp.weight.to(DEV)
    rb, rout = _guarded((T, H), torch.bfloat16, 3.0)
    nb, norm = _guarded((T, H), torch.bfloat16, 3.0)
    if mode == "norm":
        fn.fused_add_rmsnorm(parts, res, w, EPS, norm_out=norm, residual_out=rout)
        guards = [rb, nb]
    else:
        qb, q = _guarded((T, H), torch.uint8, 0x5A)
        groups = H // 128 if mode == "quant_block" else 0
        sb, sc = _guarded((T, groups) if groups else (T,), torch.float32, -7.0)
        f = fn.fused_add_rmsnorm_quant_fp8 if mode == "quant_token" else \
            fn.fused_add_rmsnorm_quant_fp8_block
        f(parts, res, w, EPS, norm_out=norm, residual_out=rout, quant_out=q, scale_out=sc)
        guards = [rb, nb, qb, sb]
    torch.cuda.synchronize()
    for g in guards:
        tail = g[-GUARD:]
        assert torch.all(tail == tail[0]) and float(tail[0]) in (3.0, 0x5A, -7.0), \
            "an output's guard band was written"
    check(dict(residual=rout, norm=norm, **({} if mode == "norm" else dict(codes=q, scales=sc))),
          run_oracle(inp, mode), mode, label=f"{mode} T={T} H={H} P={P} guarded")


@pytest.mark.parametrize("kind", ["qk", "sharded", "mla"])
def test_no_write_past_the_qk_family_outputs(fn, kind):
    T, q, k = 300, 1536, (0 if kind == "sharded" else 520 if kind == "qk" else 512)
    g = torch.Generator().manual_seed(5)
    rows = torch.randn(T, q + k + 64, generator=g).to(torch.bfloat16).to(DEV)
    wq = torch.ones(q, dtype=torch.bfloat16, device=DEV)
    wk = torch.ones(max(k, 8), dtype=torch.bfloat16, device=DEV)[:k]
    qb, qo = _guarded((T, q), torch.bfloat16, 3.0)
    bufs = [qb]
    if kind == "qk":
        kb, ko = _guarded((T, k), torch.bfloat16, 3.0)
        fn.qk_rmsnorm(rows, q, k, wq, wk, EPS, q_out=qo, k_out=ko)
        bufs.append(kb)
    elif kind == "sharded":
        fn.sharded_rmsnorm(rows, wq, EPS, out=qo, H=q)
    else:
        yb, yo = _guarded((T, k), torch.bfloat16, 3.0)
        cb, co = _guarded((T, q), torch.uint8, 0x5A)
        sb, so = _guarded((T, q // 128), torch.float32, -7.0)
        fn.ag_dual_rmsnorm(rows, q, k, wq, wk, quant=True, x_norm_out=qo, y_norm_out=yo,
                           quant_out=co, scale_out=so)
        bufs += [yb, cb, sb]
    torch.cuda.synchronize()
    for b in bufs:
        tail = b[-GUARD:]
        assert torch.all(tail == tail[0]) and float(tail[0]) in (3.0, 0x5A, -7.0), \
            f"{kind}: an output's guard band was written"


# ----------------------------------------------------------------------------- measurement aid

@pytest.mark.parametrize("n_src,row,stride,widths", [
    (9, 16384, 16384, (16384, 8192)),      # the prefill epilogue's mix
    (3, 14336, 14336, (14336, 7168, 224)),  # the block FP8 epilogue's mix
    (1, 14336, 16384, (12288, 2048)),       # the QK norm's mix (strided rows)
    (2, 1040, 1040, (16,)),                 # a ragged row: lanes past its end
])
def test_stream_mix_writes_the_xor_of_its_sources(fn, n_src, row, stride, widths):
    """The mixed-stream ceiling moves the bytes it claims: destination k holds,
    per row, the XOR of the first widths[k] bytes of every source row."""
    rows = 300
    g = torch.Generator(device="cpu").manual_seed(3)
    srcs = [torch.randint(-2**31, 2**31 - 1, ((rows - 1) * stride // 4 + row // 4,),
                          dtype=torch.int32, generator=g).to(DEV) for _ in range(n_src)]
    dsts = [torch.full((rows * w // 4,), -1, dtype=torch.int32, device=DEV) for w in widths]
    fn.stream_mix(srcs, dsts, rows, row, stride)
    torch.cuda.synchronize()
    for d, w in zip(dsts, widths):
        want = torch.zeros(rows, w // 4, dtype=torch.int32)
        for sbuf in srcs:
            sc = sbuf.cpu()
            view = torch.stack([sc[r * stride // 4: r * stride // 4 + w // 4] for r in range(rows)])
            want ^= view
        assert torch.equal(d.cpu().view(rows, w // 4), want)
