"""GPU parity of the forward's log-sum-exp output (attn_prefill_lse_fwd) and
of the backward by recomputation (attn_prefill_bwd) against the fp64 oracle
[Attention variants deep-dive, §6.2 technique 2 (recomputation); §5 GQA code
for the gradients of shared K/V heads].

The HIP side runs end to end (its own forward's o and lse feed its
backward); the oracle computes the gradients from q, k, v and dO alone.

Gradient bound.  A gradient entry is a long sum with cancellation (dk of a
key sums g * Sq terms), so its error scales with the sum of its terms'
absolute values M (oracle.gradient_magnitudes), not with its value.  Each
term is perturbed by at most about 3 * 2^-9 relative: the bf16 rounding of
its P or dS operand, P recomputed from a log-sum-exp that is itself off by
up to 2^-9 (see LSE_TOL), and D formed from the bf16-rounded o.  The
entrywise bound is 2^-7 * M + 2^-8 * |ref| (the second part for the bf16
rounding of the result), and the relative Frobenius error must stay within
the bf16 bar of 1e-2 (relative to 2^-7 ||M|| where the gradient cancels).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_close, note, ref_f64, to_f64, to_gpu
from tests.test_gpu_prefill import inputs, sample_rows
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

# |lse_gpu - lse_ref|.  The bf16 kernel sums fp32 probabilities on its common
# path and bf16-rounded ones (the values it multiplies V with) on its
# recomputing path, which every row takes for its first tile and for any tile
# whose sum passes 2^8; a rounded term carries a relative error of at most
# 2^-9, which does not average out on rows with few keys, so ln(l) is off by
# up to about 2^-9.  The fp32 kernel sums unrounded probabilities.
LSE_TOL = {"bf16": 2.0 ** -8, "f32": 1e-4}


@pytest.fixture(scope="module")
def ga():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


@pytest.mark.parametrize("dtype,d,Hq,Hkv,Sq,Sk,causal,Wn", [
    ("bf16", 128, 32, 8, 512, 512, True, 0),
    ("bf16", 128, 4, 4, 300, 700, False, 0),
    ("bf16", 64, 8, 1, 130, 257, True, 0),
    ("bf16", 128, 8, 2, 400, 400, True, 100),
    ("f32", 64, 4, 2, 100, 130, True, 0),
    ("f32", 128, 4, 4, 70, 70, False, 0),
    ("f32", 64, 4, 2, 128, 128, True, 17),
])
def test_lse_forward_matches_oracle(ga, dtype, d, Hq, Hkv, Sq, Sk, causal, Wn):
    import torch
    note(f"lse forward {dtype} d{d} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal={causal} W{Wn}")
    q, k, v = inputs(80 + Sq, 2, Hq, Hkv, Sq, Sk, d, dtype)
    qg, kg, vg = (to_gpu(x, dtype) for x in (q, k, v))
    o, lse = ga.attn_prefill_lse_fwd(qg, kg, vg, causal=causal, window=Wn)
    if Wn:
        o_plain = ga.attn_prefill_window_fwd(qg, kg, vg, window=Wn)
    else:
        o_plain = ga.attn_prefill_fwd(qg, kg, vg, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain)                 # the LSE output changes nothing else
    ref_o, ref_lse = oracle.attention(ref_f64(q, dtype), ref_f64(k, dtype), ref_f64(v, dtype), causal=causal,
                                      return_lse=True, window=Wn or None)
    assert_close(to_f64(o), ref_o, dtype, "o")
    err = np.abs(to_f64(lse) - ref_lse).max()
    assert err <= LSE_TOL[dtype], f"lse max abs err {err:.3e}"


GRAD_TERM_TOL = 2.0 ** -7
GRAD_OUT_TOL = 2.0 ** -8


def assert_grad_close(got, ref, mag, what):
    assert got.shape == ref.shape == mag.shape
    assert np.all(np.isfinite(got)), f"{what}: non-finite gradient"
    err = np.abs(got - ref)
    bound = GRAD_TERM_TOL * mag + GRAD_OUT_TOL * np.abs(ref) + 1e-30
    worst = float((err / bound).max())
    # normwise check; a gradient that cancels to ~0 (one key: dS = 0) is
    # measured against its terms' scale instead
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), GRAD_TERM_TOL * np.linalg.norm(mag), 1e-300))
    assert worst <= 1.0, f"{what}: error reaches {worst:.2f} x its bound (max abs err {err.max():.3e})"
    assert rel <= 1e-2, f"{what}: relative Frobenius error {rel:.3e}"


def run_fwd_bwd(ga, q, k, v, do, causal, Wn, scale=None):
    import torch
    qg, kg, vg, dog = (to_gpu(x, "bf16") for x in (q, k, v, do))
    o, lse = ga.attn_prefill_lse_fwd(qg, kg, vg, causal=causal, window=Wn, scale=scale)
    dq, dk, dv = ga.attn_prefill_bwd(qg, kg, vg, o, lse, dog, causal=causal, window=Wn, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


CASES = [
    # d, B, Hq, Hkv, Sq, Sk, causal, window
    (128, 1, 8, 2, 300, 300, True, 0),       # GQA, ragged, several tiles
    (64, 2, 4, 4, 200, 333, False, 0),       # MHA, Sq < Sk, non-causal
    (128, 1, 8, 1, 130, 260, True, 0),       # MQA, causal with offset
    (128, 2, 4, 2, 400, 400, True, 100),     # sliding window
    (64, 1, 16, 1, 128, 128, True, 0),       # g = 16
    (128, 1, 2, 1, 1, 1, False, 0),          # one query, one key
    (64, 1, 4, 2, 5, 70, True, 0),           # fewer queries than a tile
    (128, 1, 4, 4, 64, 64, True, 1),         # one-key window: dq = dk = 0, dv = dO
    (64, 2, 4, 2, 300, 100, False, 0),       # non-causal with more queries than keys
    (128, 1, 128, 1, 40, 300, True, 0),      # g = 128 (every query head reads one K/V head)
    (128, 1, 8, 2, 513, 700, True, 300),     # window with Sq < Sk, several 256-row blocks
]


@pytest.mark.parametrize("d,B,Hq,Hkv,Sq,Sk,causal,Wn", CASES)
def test_backward_matches_oracle(ga, d, B, Hq, Hkv, Sq, Sk, causal, Wn):
    note(f"backward d{d} B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal={causal} W{Wn}")
    q, k, v = inputs(90 + Sq + Sk, B, Hq, Hkv, Sq, Sk, d, "bf16")
    do = W.normal([91 + Sq, 3], (B, Hq, Sq, d), "bf16")
    dq, dk, dv = run_fwd_bwd(ga, q, k, v, do, causal, Wn)
    args = (ref_f64(q, "bf16"), ref_f64(k, "bf16"), ref_f64(v, "bf16"), ref_f64(do, "bf16"))
    rq, rk, rv = oracle.attention_backward(*args, causal=causal, window=Wn or None)
    mq, mk, mv = oracle.gradient_magnitudes(*args, causal=causal, window=Wn or None)
    assert_grad_close(to_f64(dq), rq, mq, "dq")
    assert_grad_close(to_f64(dk), rk, mk, "dk")
    assert_grad_close(to_f64(dv), rv, mv, "dv")
    if Wn == 1:
        # each row attends only its diagonal key with probability 1: dS is 0
        # up to fp32 rounding of dP - D, and dv is dO exactly
        assert np.abs(to_f64(dq)).max() <= 1e-3 and np.abs(to_f64(dk)).max() <= 1e-3
        assert np.array_equal(to_f64(dv), ref_f64(do, "bf16"))


# fp32: each term carries a relative error of a few fp32 units (the lse of
# the fp32 forward is exact to about 1e-6); 2^-14 of the term magnitudes
# leaves a wide margin over sums of a few thousand terms.
F32_TERM_TOL = 2.0 ** -14


@pytest.mark.parametrize("d,B,Hq,Hkv,Sq,Sk,causal,Wn", [
    (64, 1, 4, 2, 128, 128, True, 0),        # the tiny fp32 workload's shape, causal
    (128, 2, 4, 4, 70, 150, False, 0),       # MHA, non-causal, Sq < Sk
    (64, 1, 8, 1, 100, 100, True, 17),       # MQA with a window
])
def test_backward_f32_matches_oracle(ga, d, B, Hq, Hkv, Sq, Sk, causal, Wn):
    import torch
    note(f"backward f32 d{d} B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} causal={causal} W{Wn}")
    q, k, v = inputs(120 + Sq, B, Hq, Hkv, Sq, Sk, d, "f32")
    do = W.normal([121 + Sq, 3], (B, Hq, Sq, d), "f32")
    qg, kg, vg, dog = (to_gpu(x, "f32") for x in (q, k, v, do))
    o, lse = ga.attn_prefill_lse_fwd(qg, kg, vg, causal=causal, window=Wn)
    grads = ga.attn_prefill_bwd(qg, kg, vg, o, lse, dog, causal=causal, window=Wn)
    torch.cuda.synchronize()
    args = tuple(np.asarray(x, np.float64) for x in (q, k, v, do))
    refs = oracle.attention_backward(*args, causal=causal, window=Wn or None)
    mags = oracle.gradient_magnitudes(*args, causal=causal, window=Wn or None)
    for got, ref, mag, name in zip(grads, refs, mags, ("dq", "dk", "dv")):
        got = to_f64(got)
        assert np.all(np.isfinite(got)), name
        err = np.abs(got - ref)
        worst = float((err / (F32_TERM_TOL * mag + 1e-30)).max())
        assert worst <= 1.0, f"{name}: error reaches {worst:.2f} x its bound (max abs err {err.max():.3e})"


def test_backward_scale_and_outputs_overwritten(ga):
    """A non-default scale, and dq/dk/dv buffers holding garbage on entry."""
    import torch
    q, k, v = inputs(95, 1, 4, 2, 96, 160, 128, "bf16")
    do = W.normal([95, 3], (1, 4, 96, 128), "bf16")
    qg, kg, vg, dog = (to_gpu(x, "bf16") for x in (q, k, v, do))
    o, lse = ga.attn_prefill_lse_fwd(qg, kg, vg, causal=True, scale=0.05)
    bufs = [torch.full_like(t, float("nan")) for t in (qg, kg, vg)]
    dq, dk, dv = ga.attn_prefill_bwd(qg, kg, vg, o, lse, dog, *bufs, causal=True, scale=0.05)
    torch.cuda.synchronize()
    args = (ref_f64(q, "bf16"), ref_f64(k, "bf16"), ref_f64(v, "bf16"), ref_f64(do, "bf16"))
    refs = oracle.attention_backward(*args, scale=0.05, causal=True)
    mags = oracle.gradient_magnitudes(*args, scale=0.05, causal=True)
    for got, ref, mag, name in zip((dq, dk, dv), refs, mags, ("dq", "dk", "dv")):
        assert_grad_close(to_f64(got), ref, mag, name)


def test_backward_is_deterministic(ga):
    """No atomics: two runs give the same bits."""
    import torch
    q, k, v = inputs(96, 1, 8, 2, 256, 256, 128, "bf16")
    do = W.normal([96, 3], (1, 8, 256, 128), "bf16")
    a = run_fwd_bwd(ga, q, k, v, do, True, 0)
    b = run_fwd_bwd(ga, q, k, v, do, True, 0)
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.slow
def test_full_size_backward_sampled(ga):
    """The GQA S = 8192 causal workload: dq at sampled rows of a group's query
    heads, dk and dv at sampled keys, for one K/V head of each batch entry."""
    w = W.PREFILL_WORKLOADS[3]
    note(f"full-size backward {w.name}: generating inputs")
    q, k, v = W.prefill_inputs(w)
    do = W.normal([w.seed, 9], (w.B, w.Hq, w.Sq, w.d), "bf16")
    dq, dk, dv = run_fwd_bwd(ga, q, k, v, do, True, 0, scale=w.scale_value)
    dq, dk, dv = (t.view(__import__("torch").int16).cpu().numpy().view(np.uint16) for t in (dq, dk, dv))
    rng = np.random.default_rng(97)
    g = w.Hq // w.Hkv

    class Bf16:
        def __init__(self, bits):
            self.bits, self.shape = bits, bits.shape

        def __getitem__(self, idx):
            return oracle.bf16_bits_to_f64(self.bits[idx])
    for b, hk in ((0, 0), (w.B - 1, w.Hkv - 1)):
        rows = sample_rows(w.Sq, rng)
        keys = sample_rows(w.Sk, rng)
        note(f"full-size backward b{b} hk{hk}: oracle")
        rq, rk, rv, (mq, mk, mv) = oracle.attention_backward_sampled(
            Bf16(q), Bf16(k), Bf16(v), Bf16(do), b, hk, rows, keys, scale=w.scale_value, causal=True,
            magnitudes=True)
        for h in range(hk * g, hk * g + g):
            assert_grad_close(ref_f64(dq[b, h, rows], "bf16"), rq[h], mq[h], f"dq b{b} h{h}")
        assert_grad_close(ref_f64(dk[b, hk, keys], "bf16"), rk, mk, f"dk b{b} hk{hk}")
        assert_grad_close(ref_f64(dv[b, hk, keys], "bf16"), rv, mv, f"dv b{b} hk{hk}")
