"""GPU parity of prefill on seeded random configurations against the fp64 oracle.

Each case draws the dtype (bf16 or fp32), group size, K/V heads, head
dimension, batch, query and key lengths (ragged, Sq <= Sk when causal),
causal or not and a sliding window, and compares the output element by
element with the oracle's definition (bf16: 1.5e-2 plus the output's bf16
rounding, 2^-8 |ref|; fp32: 1e-4).  The query block of a bf16 workgroup
holds 256/g positions, so the draws put the causal diagonal, the window's
first key and the ragged key tail at varied places inside the tiles.
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import note, ref_f64, to_f64, to_gpu
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def draw(case: int):
    rng = np.random.default_rng([8200, case])
    dtype = "bf16" if rng.random() < 0.75 else "f32"
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2]))
    B = int(rng.choice([1, 2]))
    causal = bool(rng.random() < 0.7)
    Sk = int(rng.integers(1, 700))
    Sq = int(rng.integers(1, Sk + 1)) if causal else int(rng.integers(1, 500))
    window = int(rng.choice([0, 0, 1, 33, 200])) if causal else 0
    return dtype, d, g * Hkv, Hkv, B, Sq, Sk, causal, window


@pytest.mark.parametrize("case", range(24))
def test_prefill_random_configuration(case):
    import torch
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    dtype, d, Hq, Hkv, B, Sq, Sk, causal, window = draw(case)
    note(f"prefill random {case}: {dtype} B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} d{d} causal={causal} window={window}")
    seed = [8201, case]
    q = W.normal(seed + [0], (B, Hq, Sq, d), dtype)
    k = W.normal(seed + [1], (B, Hkv, Sk, d), dtype)
    v = W.normal(seed + [2], (B, Hkv, Sk, d), dtype)
    win = window or None
    o = gqa_attn.attn_prefill_fwd(to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype), causal=causal, window=win)
    torch.cuda.synchronize()
    ref = oracle.attention(ref_f64(q, dtype), ref_f64(k, dtype), ref_f64(v, dtype), causal=causal, window=win)
    got = to_f64(o)
    assert np.all(np.isfinite(got))
    if dtype == "bf16":
        excess = np.abs(got - ref) - 2.0 ** -8 * np.abs(ref)
        assert float(excess.max()) <= 1.5e-2, f"case {case}: max excess {float(excess.max()):.3e}"
    else:
        assert float(np.abs(got - ref).max()) <= 1e-4, f"case {case}: max error {float(np.abs(got - ref).max()):.3e}"
