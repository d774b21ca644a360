"""GPU parity of attn_prefill_fwd against the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_close, note, ref_f64, to_f64, to_gpu
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


def run(ga, q, k, v, dtype, causal, scale=None):
    import torch
    qt, kt, vt = to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype)
    o = ga.attn_prefill_fwd(qt, kt, vt, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o


def inputs(seed, B, Hq, Hkv, Sq, Sk, d, dtype, qmul=1.0):
    q = W.normal([seed, 0], (B, Hq, Sq, d), "f32") * np.float32(qmul)
    k = W.normal([seed, 1], (B, Hkv, Sk, d), "f32")
    v = W.normal([seed, 2], (B, Hkv, Sk, d), "f32")
    if dtype == "bf16":
        q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    return q, k, v


def check_vs_oracle(ga, q, k, v, dtype, causal, scale=None, what="", beyond_unit=False):
    note(f"prefill {what} q{q.shape} k{k.shape} {dtype} causal={causal}")
    o = run(ga, q, k, v, dtype, causal, scale)
    ref = oracle.attention(ref_f64(q, dtype), ref_f64(k, dtype), ref_f64(v, dtype), scale=scale, causal=causal)
    return assert_close(to_f64(o), ref, dtype, what, beyond_unit)


# ----------------------------------------------------------------------------
# the tiny fp32 workload, and fp32 variants
# ----------------------------------------------------------------------------
def test_tiny_fp32_gqa_workload(ga):
    w = W.CFG1
    q, k, v = W.prefill_inputs(w)
    worst, _ = check_vs_oracle(ga, q, k, v, "f32", False, w.scale_value, w.name)
    assert worst <= 1e-4


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d,causal", [
    (2, 4, 1, 70, 133, 128, True), (1, 3, 3, 65, 65, 64, True), (2, 6, 2, 1, 17, 64, False),
    (1, 2, 1, 200, 200, 128, False),
])
def test_fp32_variants(ga, B, Hq, Hkv, Sq, Sk, d, causal):
    q, k, v = inputs(11, B, Hq, Hkv, Sq, Sk, d, "f32")
    check_vs_oracle(ga, q, k, v, "f32", causal, None, "fp32")


# ----------------------------------------------------------------------------
# bf16 MFMA path: several tiles, ragged tails, every supported group size
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1), (16, 4)])
@pytest.mark.parametrize("Sq,Sk,causal", [(200, 200, True), (200, 200, False), (77, 300, True), (1, 1, False),
                                          (130, 129, False), (64, 64, True), (1, 190, True)])
def test_bf16_small(ga, d, Hq, Hkv, Sq, Sk, causal):
    q, k, v = inputs(12, 2, Hq, Hkv, Sq, Sk, d, "bf16")
    check_vs_oracle(ga, q, k, v, "bf16", causal, None, "bf16 small")


@pytest.mark.parametrize("Hq,Hkv,S", [(32, 1, 100), (64, 2, 70), (128, 1, 40), (64, 1, 129)])
def test_bf16_large_groups(ga, Hq, Hkv, S):
    q, k, v = inputs(13, 1, Hq, Hkv, S, S, 128, "bf16")
    check_vs_oracle(ga, q, k, v, "bf16", True, None, "bf16 g>=32")


@pytest.mark.parametrize("qmul", [8.0, 64.0])
def test_bf16_peaked_softmax(ga, qmul):
    q, k, v = inputs(14, 1, 8, 2, 257, 257, 128, "bf16", qmul=qmul)
    # near one-hot softmax: outputs approach single V rows (|O| up to ~4)
    check_vs_oracle(ga, q, k, v, "bf16", True, None, f"peaked x{qmul}", beyond_unit=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_rising_scores_force_rescales(ga, d, causal):
    # Key norms grow along the sequence and one late key dominates from inside a
    # tile, so every row's running max rises tile after tile: the kernel has to
    # recompute tiles against a new maximum and rescale the partial output and
    # sum many times per row.
    B, Hq, Hkv, S = 1, 8, 2, 700
    q = W.normal([23, 0], (B, Hq, S, d), "f32")
    k = W.normal([23, 1], (B, Hkv, S, d), "f32") * (1 + np.arange(S, dtype=np.float32) / 50)[:, None]
    k[:, :, 451] *= 4
    v = W.normal([23, 2], (B, Hkv, S, d), "f32")
    q, k, v = (W.f32_to_bf16_bits(x) for x in (q, k, v))
    check_vs_oracle(ga, q, k, v, "bf16", causal, None, "rising scores", beyond_unit=True)


def test_bf16_explicit_scale(ga):
    q, k, v = inputs(15, 1, 4, 2, 96, 160, 128, "bf16")
    check_vs_oracle(ga, q, k, v, "bf16", True, 0.37, "scale 0.37")


# ----------------------------------------------------------------------------
# GPU-side pins that need no oracle
# ----------------------------------------------------------------------------
def test_single_key_returns_value_row_exactly(ga):
    import torch
    q, k, v = inputs(16, 2, 8, 2, 33, 1, 128, "bf16")
    o = run(ga, q, k, v, "bf16", False)
    vt = to_gpu(v, "bf16")
    for h in range(8):
        assert torch.equal(o[:, h], vt[:, h // 4].expand(-1, 33, -1))


def test_causal_row0_is_v0_exactly(ga):
    import torch
    q, k, v = inputs(17, 2, 8, 2, 150, 150, 128, "bf16")
    o = run(ga, q, k, v, "bf16", True)
    vt = to_gpu(v, "bf16")
    for h in range(8):
        assert torch.equal(o[:, h, 0], vt[:, h // 4, 0])


def test_all_ones_values_give_ones(ga):
    q, k, v = inputs(18, 1, 8, 2, 300, 300, 128, "bf16")
    v = np.full_like(v, 0x3F80)     # bf16 1.0
    o = to_f64(run(ga, q, k, v, "bf16", True))
    assert np.abs(o - 1.0).max() <= 1e-2


def test_zero_query_gives_running_mean(ga):
    q, k, v = inputs(19, 1, 4, 4, 160, 160, 64, "bf16")
    q[:] = 0
    o = to_f64(run(ga, q, k, v, "bf16", True))
    vf = ref_f64(v, "bf16")
    ref = np.cumsum(vf, axis=2) / np.arange(1, 161)[None, None, :, None]
    assert np.abs(o - ref).max() <= 1.5e-2


def test_identity_values_expose_probabilities(ga):
    # V = I (Sk = d = 64): output row i is softmax row i
    q, k, _ = inputs(20, 1, 2, 1, 64, 64, 64, "bf16")
    eye = W.f32_to_bf16_bits(np.eye(64, dtype=np.float32))[None, None]
    o = to_f64(run(ga, q, k, eye, "bf16", False))
    _, _, p = oracle.attention_head(ref_f64(q, "bf16")[0, 0], ref_f64(k, "bf16")[0, 0], np.eye(64), 1 / 8)
    assert np.abs(o[0, 0] - p).max() <= 1e-2
    assert np.abs(o[0, 0].sum(axis=1) - 1).max() <= 2e-2


def test_gqa_equals_mha_on_repeated_kv_bitwise(ga):
    import torch
    q, k, v = inputs(21, 2, 8, 2, 190, 190, 128, "bf16")
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    for causal in (False, True):
        a = run(ga, q, k, v, "bf16", causal)
        b = run(ga, q, kr, vr, "bf16", causal)
        assert torch.equal(a, b)


def test_run_to_run_bitwise(ga):
    import torch
    q, k, v = inputs(22, 2, 32, 8, 512, 512, 128, "bf16")
    a = run(ga, q, k, v, "bf16", True)
    b = run(ga, q, k, v, "bf16", True)
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------
# full-size workloads, sampled rows (the launch configuration the benchmark times)
# ----------------------------------------------------------------------------
def sample_rows(S, rng, extra=6):
    fixed = {0, 1, 63, 64, 127, 128, S // 2, S - 65, S - 64, S - 2, S - 1}
    rand = set(rng.integers(0, S, extra).tolist())
    return np.array(sorted(r for r in fixed | rand if 0 <= r < S))


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_prefill_sampled(ga, cfg):
    import torch
    w = W.PREFILL_WORKLOADS[cfg]
    note(f"full-size prefill {w.name}: generating inputs")
    q, k, v = W.prefill_inputs(w)
    o = run(ga, q, k, v, w.dtype, w.causal, w.scale_value)
    of = o.view(torch.int16).cpu().numpy()
    rng = np.random.default_rng(100 + cfg)
    worst = 0.0
    for b in range(w.B):
        for hq in range(w.Hq):
            rows = sample_rows(w.Sq, rng)
            hk = oracle.kv_head_index(hq, w.Hq, w.Hkv)
            ref, _ = oracle.attention_rows(ref_f64(q[b:b + 1, hq:hq + 1], "bf16"), ref_f64(k[b:b + 1, hk:hk + 1], "bf16"),
                                           ref_f64(v[b:b + 1, hk:hk + 1], "bf16"), 0, 0, rows, w.scale_value, w.causal)
            got = ref_f64(of[b, hq, rows].view(np.uint16), "bf16")
            w_, _ = assert_close(got, ref, "bf16", f"{w.name} b{b} h{hq}")
            worst = max(worst, w_)
    note(f"{w.name}: worst sampled abs err {worst:.3e}")


@pytest.mark.slow
@pytest.mark.parametrize("window", [None, 4096])
def test_long_context_32k_sampled(ga, window):
    # LLaMA-3-8B-shaped attention (32 query heads, 8 K/V heads, d 128) at the
    # 32K context the pages discuss for it [Attention variants deep-dive, §8
    # Q4], causal and with a 4096-key sliding window: 512 key tiles per row
    # block, planes far longer than an XCD's share of the grid.
    import torch
    B, Hq, Hkv, S, d = 1, 32, 8, 32768, 128
    q = W.normal([7400, 0], (B, Hq, S, d), "bf16")
    k = W.normal([7400, 1], (B, Hkv, S, d), "bf16")
    v = W.normal([7400, 2], (B, Hkv, S, d), "bf16")
    note(f"prefill 32K context window={window}")
    qt, kt, vt = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    o = torch.full_like(qt, float("nan"))
    ga.attn_prefill_fwd(qt, kt, vt, o, causal=True, window=window)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    of = o.view(torch.int16).cpu().numpy()
    rng = np.random.default_rng(7400 + (window or 0))
    for hq in range(0, Hq, 3):
        rows = sample_rows(S, rng)
        hk = oracle.kv_head_index(hq, Hq, Hkv)
        ref, _ = oracle.attention_rows(ref_f64(q[:, hq:hq + 1], "bf16"), ref_f64(k[:, hk:hk + 1], "bf16"),
                                       ref_f64(v[:, hk:hk + 1], "bf16"), 0, 0, rows, None, True, window)
        got = ref_f64(of[0, hq, rows].view(np.uint16), "bf16")
        assert_close(got, ref, "bf16", f"32K window={window} h{hq}")
