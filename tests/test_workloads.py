"""The seeded input generators: bfloat16 rounding, determinism, block placement."""
import numpy as np
import pytest

from transformer_exact_attention_amd import workloads as W


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),      # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38,
                  1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32),
    ])
    # exact ties: low 16 bits = 0x8000 with either parity of bit 16
    ties = (rng.integers(0, 0x7F00, 500, dtype=np.uint32) << 16 | 0x8000).astype(np.uint32)  # finite
    x = np.concatenate([x, ties.view(np.float32)])
    got = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    nan = W.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert (nan[0] & 0x7FFF) == 0x7FC0


def test_generators_are_deterministic_and_normal():
    a = W.normal_f32([9, 0], (1000, 7))
    b = W.normal_f32([9, 0], (1000, 7))
    assert np.array_equal(a, b)
    assert abs(a.mean()) < 0.05 and abs(a.std() - 1) < 0.05
    bits = W.normal_bf16([9, 0], (1000, 7))
    assert np.array_equal(bits, W.f32_to_bf16_bits(a))
    assert not np.array_equal(W.normal_f32([9, 1], (10,)), W.normal_f32([9, 0], (10,)))


def test_block_placement_is_a_permutation():
    lens = np.array([17, 1, 32, 48, 5], np.int32)
    table, nb = W.block_placement(5, lens, 4)
    nblk = -(-lens // 16)
    assert nb == nblk.sum()
    used = np.concatenate([table[b, :nblk[b]] for b in range(len(lens))])
    assert np.array_equal(np.sort(used), np.arange(nb))
    for b in range(len(lens)):
        assert np.all(table[b, nblk[b]:] == -1)
    with pytest.raises(ValueError):
        W.block_placement(5, np.array([65]), 4)


def test_workload_flop_counts():
    assert W.CFG1.flops() == 4 * 64 * 4 * 128 * 128
    assert W.CFG2.flops() == 4 * 128 * 32 * 4 * (2048 * 2049 // 2)
    assert abs(W.CFG2.flops() - 1.375e11) / 1.375e11 < 2e-3
    assert abs(W.CFG3.flops() - 1.0997e12) / 1.0997e12 < 1e-4
    lens = W.seq_lengths(4, 64, 512, 4096)
    assert lens.min() >= 512 and lens.max() <= 4096
    assert np.array_equal(lens, W.seq_lengths(4, 64, 512, 4096))


def test_decode_inputs_small_paged():
    w = W.DecodeWorkload("t", 7, 3, 4, 2, 8, 1, 40, True)
    di = W.decode_inputs(w)
    assert di.k_cache.shape == (di.num_blocks, 2, 16, 8)
    assert di.block_table.shape == (3, 3)
    assert di.q.dtype == np.uint16
