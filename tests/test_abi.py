"""The C ABI without a GPU: the library loads, exports what the header declares,
and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa_attn.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+|void\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text,
                                re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from transformer_exact_attention_amd import gqa_attn
    return gqa_attn.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["gqa_attn_abi_version", "gqa_attn_status_string", "attn_prefill_fwd",
                            "attn_decode_workspace_bytes", "attn_decode_fwd", "attn_decode_validate",
                            "gqa_kv_pool_create", "gqa_kv_pool_destroy", "gqa_kv_pool_free_blocks",
                            "gqa_kv_seq_new", "gqa_kv_seq_fork", "gqa_kv_seq_release", "gqa_kv_seq_len",
                            "gqa_kv_reserve", "gqa_kv_block_table", "attn_kv_append", "attn_kv_copy_blocks",
                            "attn_decode_fp8_fwd", "attn_kv_append_fp8", "attn_kv_copy_blocks_fp8",
                            "attn_prefill_window_fwd", "attn_decode_window_fwd", "attn_prefill_lse_fwd",
                            "attn_prefill_bwd_workspace_bytes", "attn_prefill_bwd", "attn_decode_fwd_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    from transformer_exact_attention_amd import gqa_attn
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(gqa_attn.EXPORTS) == set(declared_functions())


def test_abi_version_and_status_strings(lib):
    ver = int(re.search(r"#define GQA_ATTN_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.gqa_attn_abi_version() == ver
    for s in range(6):
        assert lib.gqa_attn_status_string(s)
    assert lib.gqa_attn_status_string(99) == b"unknown status"


FAKE = 0x100000   # never dereferenced: every call below fails validation first


def prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=4, Hkv=2, Sq=16, Sk=16, d=64, scale=0.125, causal=0,
             dtype=1, stream=None)
    a.update(kw)
    return lib.attn_prefill_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                a["d"], a["scale"], a["causal"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(B=0), 1), (dict(Hq=-1), 1), (dict(Sk=0), 1),
    (dict(Hq=6, Hkv=4), 1),                  # query heads not a multiple of K/V heads
    (dict(causal=1, Sq=17, Sk=16), 1),       # causal needs Sq <= Sk
    (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1), (dict(scale=-1.0), 1),
    (dict(dtype=7), 1),
    (dict(d=96), 2), (dict(d=32), 2),
    (dict(Hq=6, Hkv=2), 2),                  # bf16 group size 3 not supported
    (dict(Sq=1 << 25, d=64), 1),             # plane element count overflow
])
def test_prefill_rejects_on_host(lib, kw, status):
    assert prefill(lib, **kw) == status


def decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, table=None, B=2, Hq=8, Hkv=2, d=128, max_seq_len=64,
             block_size=0, max_blocks=0, scale=0.1, dtype=1, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.attn_decode_fwd(a["q"], a["k"], a["v"], a["o"], a["lens"], a["table"], a["B"], a["Hq"], a["Hkv"],
                               a["d"], a["max_seq_len"], a["block_size"], a["max_blocks"], a["scale"], a["dtype"],
                               a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(lens=None), 1), (dict(B=0), 1), (dict(Hq=6, Hkv=4), 1), (dict(max_seq_len=0), 1),
    (dict(scale=0.0), 1),
    (dict(table=FAKE, block_size=8, max_blocks=8), 1),       # pages hold 16 tokens
    (dict(table=FAKE, block_size=16, max_blocks=3), 1),      # 3 * 16 < max_seq_len
    (dict(table=FAKE, block_size=16, max_blocks=0), 1),
    (dict(d=96), 2), (dict(d=32), 2), (dict(dtype=0), 2), (dict(Hq=128, Hkv=2), 2),   # g = 64 not supported
    (dict(B=4097), 2),
    (dict(ws=None), 3), (dict(ws=FAKE + 8), 3), (dict(ws_bytes=16), 3),
])
def test_decode_rejects_on_host(lib, kw, status):
    assert decode(lib, **kw) == status


def test_decode_workspace_formula(lib):
    # fp32 partial outputs [B, Hq, P, d] + fp32 LSE [B, Hq, P] + int64 prefix sums [B + 1],
    # each 256-byte aligned; P = ceil(L / 256) + 1 partials per (sequence, query head)
    def expect(B, Hq, d, L, share=256):
        P = -(-L // share) + 1
        al = lambda x: (x + 255) // 256 * 256
        return al(B * Hq * P * d * 4) + al(B * Hq * P * 4) + al((B + 1) * 8)
    for args in [(64, 32, 128, 4096), (16, 32, 128, 32768), (1, 1, 128, 1), (3, 5, 128, 257)]:
        assert lib.attn_decode_workspace_bytes(*args) == expect(*args)
    assert lib.attn_decode_workspace_bytes(0, 32, 128, 10) == 0
    assert lib.attn_decode_workspace_bytes(1, 32, 128, 0) == 0


def test_validate_rejects_null(lib):
    assert lib.attn_decode_validate(None, None, 1, 1, 0, 0, 0, None) == 1
    assert lib.attn_decode_validate(FAKE, FAKE, 1, 16, 16, 0, 4, None) == 1


def test_binding_raises_typed_errors_without_touching_the_gpu():
    from transformer_exact_attention_amd import gqa_attn
    with pytest.raises(ValueError):
        gqa_attn._raise(1, "x")
    with pytest.raises(NotImplementedError):
        gqa_attn._raise(2, "x")
    with pytest.raises(gqa_attn.GqaAttnError):
        gqa_attn._raise(4, "x")
    gqa_attn._raise(0, "x")


def decode_fp8(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, o=FAKE, lens=FAKE, table=None, B=2, Hq=8, Hkv=2, d=128,
             max_seq_len=64, block_size=0, max_blocks=0, scale=0.1, ws=FAKE, ws_bytes=1 << 30, stream=None)
    a.update(kw)
    return lib.attn_decode_fp8_fwd(a["q"], a["k"], a["v"], a["ks"], a["vs"], a["o"], a["lens"], a["table"], a["B"],
                                   a["Hq"], a["Hkv"], a["d"], a["max_seq_len"], a["block_size"], a["max_blocks"],
                                   a["scale"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), 1), (dict(vs=None), 1), (dict(q=None), 1), (dict(Hq=6, Hkv=4), 1), (dict(scale=-1.0), 1),
    (dict(d=64), 2), (dict(Hq=96, Hkv=1), 2),
    (dict(max_seq_len=100), 2),                       # contiguous fp8 caches need max_seq_len % 16 == 0
    (dict(table=FAKE, block_size=16, max_blocks=2, max_seq_len=64), 1),   # table narrower than max_seq_len
    (dict(ws=None), 3), (dict(ws_bytes=16), 3),
])
def test_decode_fp8_rejects_on_host(lib, kw, status):
    assert decode_fp8(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [(dict(window=0), 1), (dict(window=-3), 1), (dict(Sq=17, Sk=16), 1),
                                       (dict(q=None), 1), (dict(d=96), 2)])
def test_prefill_window_rejects_on_host(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, B=1, Hq=4, Hkv=2, Sq=16, Sk=16, d=64, scale=0.125, window=8, dtype=1)
    a.update(kw)
    assert lib.attn_prefill_window_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"],
                                       a["d"], a["scale"], a["window"], a["dtype"], None) == status


@pytest.mark.parametrize("kw,status", [(dict(window=0), 1), (dict(lens=None), 1), (dict(dtype=0), 2),
                                       (dict(ws=None), 3)])
def test_decode_window_rejects_on_host(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, table=None, B=2, Hq=8, Hkv=2, d=128, max_seq_len=64,
             block_size=0, max_blocks=0, scale=0.1, window=16, dtype=1, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    assert lib.attn_decode_window_fwd(a["q"], a["k"], a["v"], a["o"], a["lens"], a["table"], a["B"], a["Hq"],
                                      a["Hkv"], a["d"], a["max_seq_len"], a["block_size"], a["max_blocks"],
                                      a["scale"], a["window"], a["dtype"], a["ws"], a["ws_bytes"], None) == status


@pytest.mark.parametrize("kw,status", [(dict(lse=None), 1), (dict(window=-1), 1), (dict(Sq=17, Sk=16, window=4), 1),
                                       (dict(q=None), 1), (dict(d=96), 2), (dict(dtype=5), 1)])
def test_prefill_lse_rejects_on_host(lib, kw, status):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, Hq=4, Hkv=2, Sq=16, Sk=16, d=64, scale=0.125, causal=0,
             window=0, dtype=1)
    a.update(kw)
    assert lib.attn_prefill_lse_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                                    a["Sk"], a["d"], a["scale"], a["causal"], a["window"], a["dtype"], None) == status


def bwd(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=4, Hkv=2, Sq=16,
             Sk=16, d=64, scale=0.125, causal=1, window=0, dtype=1, ws=0x100000 * 256, ws_bytes=1 << 20)
    a.update(kw)
    return lib.attn_prefill_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"], a["B"],
                                a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["d"], a["scale"], a["causal"], a["window"],
                                a["dtype"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(o=None), 1), (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(k=None), 1), (dict(window=-2), 1), (dict(Sq=32, Sk=16), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(scale=0.0), 1), (dict(dtype=5), 1), (dict(d=96), 2), (dict(B=2048, Hq=128, Hkv=128, Sq=1024, Sk=1024), 2),
    (dict(ws=None), 3), (dict(ws=0x100000 * 256 + 64), 3), (dict(ws_bytes=16 * 4 * 4 - 4), 3),
])
def test_prefill_bwd_rejects_on_host(lib, kw, status):
    assert bwd(lib, **kw) == status


def test_prefill_bwd_workspace_formula(lib):
    assert lib.attn_prefill_bwd_workspace_bytes(1, 4, 16) == 256
    assert lib.attn_prefill_bwd_workspace_bytes(2, 32, 8192) == 2 * 32 * 8192 * 4
    assert lib.attn_prefill_bwd_workspace_bytes(1, 1, 65) == 512
    assert lib.attn_prefill_bwd_workspace_bytes(0, 4, 16) == 0


def decode_noalloc(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lens=FAKE, table=None, B=2, Hq=8, Hkv=2, d=128, max_seq_len=64,
             block_size=0, max_blocks=0, scale=0.1, dtype=1)
    a.update(kw)
    return lib.attn_decode_fwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lens"], a["table"], a["B"], a["Hq"],
                                       a["Hkv"], a["d"], a["max_seq_len"], a["block_size"], a["max_blocks"],
                                       a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1), (dict(lens=None), 1), (dict(B=0), 1), (dict(Hq=6, Hkv=4), 1),
    (dict(scale=float("nan")), 1), (dict(table=FAKE, block_size=8, max_blocks=8), 1),
    (dict(table=FAKE, block_size=16, max_blocks=3), 1),
    (dict(dtype=0), 2), (dict(Hq=128, Hkv=2), 2), (dict(B=4097), 2),
    # the workspace these sizes need exceeds the static scratch (64 MiB)
    (dict(B=64, Hq=32, Hkv=8, max_seq_len=65536), 3),
    (dict(B=4096, Hq=32, Hkv=8, max_seq_len=1024), 3),
])
def test_decode_noalloc_rejects_on_host(lib, kw, status):
    assert decode_noalloc(lib, **kw) == status


def test_decode_noalloc_limit_matches_the_header(lib):
    from transformer_exact_attention_amd import gqa_attn
    text = open(HEADER).read()
    assert "#define GQA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)" in text
    assert gqa_attn.DECODE_NOALLOC_MAX_BYTES == 64 << 20
    # the benchmark's decode workloads fit
    assert lib.attn_decode_workspace_bytes(16, 32, 128, 32768) <= gqa_attn.DECODE_NOALLOC_MAX_BYTES
    assert lib.attn_decode_workspace_bytes(64, 32, 128, 4096) <= gqa_attn.DECODE_NOALLOC_MAX_BYTES
