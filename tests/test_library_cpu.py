"""The C-ABI library: it loads, exports every declared symbol, and validates on the host.

No kernel is launched here (no GPU in this container): every call below fails
validation before any HIP call, or is a pure host query.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

klib = pytest.importorskip("kv_cache_flashattention_attn_amd")


def _lib_or_skip():
    if not os.path.exists(klib.lib_path):
        pytest.skip("libattn.so not built")
    return klib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for f in ("attn_prefill", "kv_append", "attn_decode", "attn_decode_paged"):
        assert f in names
    assert set(names) == set(klib.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    L = _lib_or_skip()
    for name in declared_functions():
        assert hasattr(L, name), name
    # dynamic symbol table check, independent of ctypes lookups
    out = os.popen(f"nm -D --defined-only {klib.lib_path}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_version_and_last_error():
    L = _lib_or_skip()
    assert b"gfx950" in L.attn_version()
    assert isinstance(L.attn_last_error(), bytes)


def test_workspace_bytes_host_logic():
    L = _lib_or_skip()
    # S = ceil(len / 256) + 1 partials per (b, h): fp32 outputs, then fp32 lse
    # (each region 256-byte aligned), then one int32 piece count per (b, h)
    def layout(B, H, cap, d):
        S = -(-cap // 256) + 1
        up = lambda x: -(-x // 256) * 256
        lse_off = up(B * H * S * d * 4)
        cnt_off = up(lse_off + B * H * S * 4)
        return cnt_off + B * H * 4
    assert L.attn_decode_workspace_bytes(1, 1, 256, 128) == layout(1, 1, 256, 128) == 1024 + 256 + 4
    assert L.attn_decode_workspace_bytes(32, 64, 32784, 128) == layout(32, 64, 32784, 128)
    assert L.attn_decode_workspace_bytes(3, 5, 1000, 64) == layout(3, 5, 1000, 64)
    assert L.attn_decode_workspace_bytes(0, 1, 1, 1) == 0


FAKE = 1 << 20  # an aligned, non-null address never dereferenced: validation fails first


@pytest.mark.parametrize("args,code", [
    # (q, k, v, o, lse, B, H_q, H_kv, N, d, causal, scale, dtype, out_fp32)
    ((0, FAKE, FAKE, FAKE, 0, 1, 1, 1, 8, 64, 0, 0.1, 2, 0), 1),          # null q
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 6, 4, 8, 64, 0, 0.1, 2, 0), 1),       # H_q % H_kv
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 1, 0, 64, 0, 0.1, 2, 0), 1),       # N = 0
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 1, 8, 48, 0, 0.1, 2, 0), 2),       # d = 48
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 1, 8, 64, 0, 0.1, 7, 0), 2),       # dtype
    ((FAKE + 2, FAKE, FAKE, FAKE, 0, 1, 1, 1, 8, 64, 0, 0.1, 2, 0), 1),   # misaligned
    ((FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 1, 8, 64, 0, float("nan"), 2, 0), 1),  # scale
])
def test_prefill_rejects_bad_arguments(args, code):
    L = _lib_or_skip()
    assert L.attn_prefill(*args, None) == code
    assert L.attn_last_error()


def test_decode_rejects_bad_arguments():
    L = _lib_or_skip()
    ws = L.attn_decode_workspace_bytes(2, 8, 64, 128)
    # workspace too small
    assert L.attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 64, 128, 0.1, 2, 0, FAKE, ws - 1, None) == 3
    # missing workspace
    assert L.attn_decode(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 64, 128, 0.1, 2, 0, 0, ws, None) == 3
    # null seq_lens
    assert L.attn_decode(FAKE, FAKE, FAKE, 0, FAKE, 0, 2, 8, 2, 64, 128, 0.1, 2, 0, FAKE, ws, None) == 1
    # paged: block size 32
    assert L.attn_decode_paged(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 128, 32, 4, 8, 0.1, 2, 0,
                               FAKE, ws, None) == 2
    # paged: null table
    assert L.attn_decode_paged(FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, 2, 8, 2, 128, 16, 4, 8, 0.1, 2, 0,
                               FAKE, ws, None) == 1


def test_append_rejects_bad_arguments():
    L = _lib_or_skip()
    # block size 8
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 128, 0, 8, 4, 4, 2, None) == 2
    # n_new = 0
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 0, 128, 64, 16, 0, 0, 2, None) == 1
    # contiguous with max_len 0
    assert L.kv_append(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1, 1, 1, 128, 0, 16, 0, 0, 2, None) == 1
    # int4: V pairs channel groups, so d must be a multiple of 32 (16 is refused, 32 gets past the check)
    assert L.kv_append_int4(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 16, 16, 4, 4, 2, FAKE, FAKE, None) == 2
    assert L.kv_append_int4(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 1, 32, 16, 0, 4, 2, FAKE, FAKE, None) == 1


@pytest.mark.parametrize("args,code", [
    # (q, k_pool, v_pool, table, cache_lens, o, lse, B, H_q, H_kv, n_new, d, block_size,
    #  max_blocks_per_seq, num_blocks, causal, scale, dtype)
    ((0, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 32, 128, 16, 8, 16, 1, 0.1, 2), 1),     # null q
    ((FAKE, FAKE, FAKE, 0, FAKE, FAKE, 0, 2, 8, 2, 32, 128, 16, 8, 16, 1, 0.1, 2), 1),     # null table
    ((FAKE, FAKE, FAKE, FAKE, 0, FAKE, 0, 2, 8, 2, 32, 128, 16, 8, 16, 1, 0.1, 2), 1),     # null lengths
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 6, 4, 32, 128, 16, 8, 16, 1, 0.1, 2), 1),  # H_q % H_kv
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 0, 128, 16, 8, 16, 1, 0.1, 2), 1),   # n_new = 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 200, 128, 16, 8, 16, 1, 0.1, 2), 1),  # n_new > 8 * 16
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 32, 128, 32, 8, 16, 1, 0.1, 2), 2),  # block size 32
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 32, 128, 16, 8, 16, 1, 0.1, 0), 2),  # f32
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 32, 32, 16, 8, 16, 1, 0.1, 2), 2),   # d = 32
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 2, 8, 2, 32, 128, 16, 8, 16, 1, 0.0, 2), 2),  # scale 0
    ((FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 0, 2, 8, 2, 32, 128, 16, 8, 16, 1, 0.1, 2), 1),  # misaligned o
])
def test_prefill_paged_rejects_bad_arguments(args, code):
    L = _lib_or_skip()
    assert L.attn_prefill_paged(*args, None) == code
    assert L.attn_last_error()


def test_noalloc_decode_refuses_a_workspace_beyond_its_static_array():
    """The allocation-free paged decode checks its workspace need against the
    library's static array before anything else: nothing is launched."""
    L = _lib_or_skip()
    # B = 32, H_q = 64, 32,784 tokens of capacity at d = 128: about 136 MB > 64 MiB
    rc = L.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 32, 64, 8, 128, 16, 2049, 40000,
                                     0.088, 2, 0, None)
    assert rc == 3
    msg = L.attn_last_error().decode()
    assert "static scratch" in msg and str(64 << 20) in msg
