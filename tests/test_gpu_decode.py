"""GPU parity of attn_decode_fwd (contiguous and paged) against the fp64 oracle."""
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


def run_contig(ga, q, kc, vc, lens):
    import torch
    o = ga.attn_decode_fwd(to_gpu(q, "bf16"), to_gpu(kc, "bf16"), to_gpu(vc, "bf16"), to_gpu(lens, "i32"))
    torch.cuda.synchronize()
    return o


def run_paged(ga, q, kp, vp, lens, table, max_seq_len=None):
    import torch
    o = ga.attn_decode_fwd(to_gpu(q, "bf16"), to_gpu(kp, "bf16"), to_gpu(vp, "bf16"), to_gpu(lens, "i32"),
                           block_table=to_gpu(table, "i32"), max_seq_len=max_seq_len)
    torch.cuda.synchronize()
    return o


def small_case(seed, B, Hq, Hkv, lens, S_max, paged, d=128):
    lens = np.asarray(lens, np.int32)
    q = W.normal_bf16([seed, 0], (B, Hq, d))
    if paged:
        max_blocks = -(-S_max // 16)
        table, nb = W.block_placement(seed, lens, max_blocks, spare_blocks=3)
        kp = W.normal_bf16([seed, 1], (nb, Hkv, 16, d))
        vp = W.normal_bf16([seed, 2], (nb, Hkv, 16, d))
        return q, kp, vp, lens, table
    kc = W.normal_bf16([seed, 1], (B, Hkv, S_max, d))
    vc = W.normal_bf16([seed, 2], (B, Hkv, S_max, d))
    return q, kc, vc, lens, None


LENS = [0, 1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 700, 1024]


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (8, 1), (32, 8), (32, 1), (32, 2), (16, 1)])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("d", [128, 64])
def test_decode_small(ga, Hq, Hkv, paged, d):
    q, kc, vc, lens, table = small_case(30 + Hq + Hkv + d, len(LENS), Hq, Hkv, LENS, 1024, paged, d)
    note(f"decode small Hq{Hq} Hkv{Hkv} d{d} paged={paged}")
    if paged:
        o = run_paged(ga, q, kc, vc, lens, table)
        ref = oracle.decode_paged(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), table, lens)
    else:
        o = run_contig(ga, q, kc, vc, lens)
        ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), lens)
    got = to_f64(o)
    assert np.all(got[0] == 0)                       # empty sequence -> zero output
    assert_close(got, ref, "bf16", "decode small")


@pytest.mark.parametrize("paged", [False, True])
def test_decode_many_short_sequences(ga, paged):
    # The largest supported batch (4096 sequences, the prefix sums live in LDS)
    # with short and empty sequences: every wavefront's share crosses dozens
    # of (sequence, K/V head) segments, so the pipeline runs across many
    # piece boundaries and the combine meets segments of one or two pieces.
    B, Hq, Hkv = 4096, 8, 2
    lens = np.random.default_rng(44).integers(0, 41, B).astype(np.int32)
    lens[::97] = 0
    note(f"decode many short sequences B{B} paged={paged}")
    q, kc, vc, lens, table = small_case(44, B, Hq, Hkv, lens, 48, paged)
    if paged:
        o = run_paged(ga, q, kc, vc, lens, table, max_seq_len=48)
        ref = oracle.decode_paged(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), table, lens)
    else:
        o = run_contig(ga, q, kc, vc, lens)
        ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), lens)
    got = to_f64(o)
    assert np.all(got[lens == 0] == 0)
    # (short sequences: outputs are close to single V rows, |O| up to ~4)
    assert_close(got, ref, "bf16", "decode many short sequences", beyond_unit=True)


def test_decode_single_token_returns_value_row(ga):
    import torch
    q, kc, vc, lens, _ = small_case(40, 3, 8, 2, [1, 1, 1], 32, False)
    o = run_contig(ga, q, kc, vc, lens)
    v = to_gpu(vc, "bf16")
    for h in range(8):
        assert torch.equal(o[:, h], v[:, h // 4, 0])


def test_decode_peaked(ga):
    q, kc, vc, lens, _ = small_case(41, 4, 32, 8, [300, 1000, 2047, 5], 2048, False)
    q = W.f32_to_bf16_bits(ref_f64(q, "bf16").astype(np.float32) * 8)
    o = run_contig(ga, q, kc, vc, lens)
    ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), lens)
    assert_close(to_f64(o), ref, "bf16", "decode peaked", beyond_unit=True)


@pytest.mark.parametrize("Hq,Hkv,d", [(32, 8, 128), (32, 1, 128), (32, 1, 64), (16, 8, 64)])
def test_decode_rising_scores_force_rescales(ga, Hq, Hkv, d):
    # key norms grow with the token index, so the running max of every piece
    # keeps rising and the lazily rescaled accumulators are redone many times
    lens = np.array([1500, 2048, 5, 600], np.int32)
    q = W.normal([43, 0], (4, Hq, d), "f32")
    kc = W.normal([43, 1], (4, Hkv, 2048, d), "f32") * (1 + np.arange(2048, dtype=np.float32) / 100)[:, None]
    kc[:, :, 1333] *= 3
    vc = W.normal([43, 2], (4, Hkv, 2048, d), "f32")
    q, kc, vc = (W.f32_to_bf16_bits(x) for x in (q, kc, vc))
    note(f"decode rising scores Hq{Hq} Hkv{Hkv} d{d}")
    o = run_contig(ga, q, kc, vc, lens)
    ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), lens)
    assert_close(to_f64(o), ref, "bf16", "decode rising scores", beyond_unit=True)


@pytest.mark.parametrize("Hkv,d", [(8, 128), (8, 64), (1, 128), (1, 64)])
def test_paged_equals_contiguous_bitwise_and_permutation_invariant(ga, Hkv, d):
    import torch
    B, Hq = 6, 32
    lens = np.array([1, 16, 300, 513, 1000, 2048], np.int32)
    q, kp, vp, lens, table = small_case(42, B, Hq, Hkv, lens, 2048, True, d)
    note(f"paged == contiguous Hkv{Hkv} d{d}")
    o_paged = run_paged(ga, q, kp, vp, lens, table)
    # contiguous cache with the same logical contents
    kc = np.zeros((B, Hkv, 2048, d), np.uint16)
    vc = np.zeros_like(kc)
    for b in range(B):
        t = np.arange(lens[b])
        kc[b, :, t] = kp[table[b, t // 16], :, t % 16]
        vc[b, :, t] = vp[table[b, t // 16], :, t % 16]
    o_contig = run_contig(ga, q, kc, vc, lens)
    assert torch.equal(o_paged, o_contig)
    # another physical placement of the same logical blocks
    nb = kp.shape[0]
    perm = np.random.default_rng(7).permutation(nb)          # new physical id of old block i
    kp2 = np.empty_like(kp)
    vp2 = np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1).astype(np.int32)
    o_perm = run_paged(ga, q, kp2, vp2, lens, table2)
    assert torch.equal(o_paged, o_perm)
    o_again = run_paged(ga, q, kp, vp, lens, table)
    assert torch.equal(o_paged, o_again)


def test_validate_device_data(ga):
    import torch
    lens = to_gpu(np.array([3, 40], np.int32), "i32")
    table = to_gpu(np.array([[0, -1, -1], [1, 2, 3]], np.int32), "i32")
    assert ga.attn_decode_validate(lens, table, 48, 4) == 0
    assert ga.attn_decode_validate(lens, table, 48, 3) == 1          # entry 3 out of range
    assert ga.attn_decode_validate(lens, None, 39) == 1              # length 40 > max
    bad = to_gpu(np.array([[0, -1, -1], [1, -1, 3]], np.int32), "i32")
    assert ga.attn_decode_validate(lens, bad, 48, 4) == 1            # -1 inside the used range
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# full-size workloads (the launch configuration the benchmark times)
# ----------------------------------------------------------------------------
@pytest.mark.slow
def test_full_size_contiguous_decode(ga):
    w = W.CFG4
    note(f"full-size decode {w.name}: generating inputs")
    di = W.decode_inputs(w)
    o = run_contig(ga, di.q, di.k_cache, di.v_cache, di.seq_lens)
    got = to_f64(o)
    ref = oracle.decode_contiguous(ref_f64(di.q, "bf16"), _Bf16Pages(di.k_cache), _Bf16Pages(di.v_cache),
                                   di.seq_lens, scale=w.scale_value)
    assert_close(got, ref, "bf16", w.name)


@pytest.mark.slow
@pytest.mark.parametrize("Hkv", [32, 8, 1])
def test_full_size_paged_decode(ga, Hkv):
    import torch
    w = W.cfg5(Hkv)
    note(f"full-size paged decode {w.name}: generating inputs")
    di = W.decode_inputs(w)
    o = run_paged(ga, di.q, di.k_cache, di.v_cache, di.seq_lens, di.block_table, di.max_seq_len)
    got = to_f64(o)
    rng = np.random.default_rng(50 + Hkv)
    heads = sorted({(b, int(h)) for b in range(w.B) for h in rng.choice(w.Hq, 3, replace=False)} |
                   {(b, 0) for b in range(w.B)} | {(b, w.Hq - 1) for b in range(w.B)})
    ref = oracle.decode_paged(ref_f64(di.q, "bf16"), _Bf16Pages(di.k_cache), _Bf16Pages(di.v_cache),
                              di.block_table, di.seq_lens, scale=w.scale_value, heads=heads)
    idx = tuple(np.array(heads).T)
    assert_close(got[idx], ref[idx], "bf16", w.name)
    # block-table gather bit-exact: the same logical contents through a contiguous cache with the same
    # (B, Hkv, max_seq_len), hence the same split plan; the contiguous copy is gathered on the device.
    kp_t, vp_t = to_gpu(di.k_cache, "bf16"), to_gpu(di.v_cache, "bf16")
    S = di.max_seq_len
    kc = torch.zeros((w.B, Hkv, S, 128), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    for b in range(w.B):
        L = int(di.seq_lens[b])
        t = torch.arange(L, device="cuda")
        phys = torch.from_numpy(di.block_table[b]).to("cuda").long()[t // 16]
        kc[b, :, :L] = kp_t[phys, :, t % 16].transpose(0, 1)
        vc[b, :, :L] = vp_t[phys, :, t % 16].transpose(0, 1)
    del kp_t, vp_t
    qd, ld = to_gpu(di.q, "bf16"), to_gpu(di.seq_lens, "i32")
    oc = ga.attn_decode_fwd(qd, kc, vc, ld, max_seq_len=S)
    torch.cuda.synchronize()
    assert torch.equal(oc, o), "paged != contiguous"


class _Bf16Pages:
    """Lazy exact upcast of bf16 pages: the oracle indexes it like an array."""

    def __init__(self, bits):
        self.bits = bits
        self.shape = bits.shape

    def __getitem__(self, idx):
        return oracle.bf16_bits_to_f64(self.bits[idx])
