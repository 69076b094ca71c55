"""Python binding of libattn: exact tiled softmax attention for MI355X (gfx950).

Thin ctypes wrappers with the C ABI's names (``include/attn.h``): they check
tensor properties, pass device pointers and the current HIP stream, and raise
on a nonzero status.  Every step of the computation runs in the HIP kernels of
``libattn.so``; there is no fallback.  PyTorch provides device memory and
streams only.

    attn_prefill(q, k, v, causal=False, scale=None, return_lse=False, out_fp32=False)
    kv_append(k_cache, v_cache, k_new, v_new, cache_lens, block_table=None, num_blocks=None)
    attn_decode(q, k_cache, v_cache, seq_lens, scale=None, return_lse=False, workspace=None)
    attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale=None, ...)
    kv_copy_blocks(k_pool, v_pool, pairs)
    BlockPool (block_pool.py): the host block pool's calls
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "AttnError", "lib", "lib_path", "attn_prefill", "attn_prefill_paged", "kv_append", "attn_decode",
    "attn_decode_paged", "kv_append_fp8", "attn_decode_paged_fp8", "kv_append_int8", "attn_decode_paged_int8",
    "kv_copy_blocks", "attn_prefill_fp8", "attn_prefill_fp8_workspace_bytes", "kv_append_int4",
    "attn_decode_paged_int4", "attn_decode_paged_noalloc",
    "attn_decode_workspace_bytes", "attn_device_error_flags", "attn_version", "DTYPE_CODES",
    "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_PKG, "libattn.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
DTYPE_CODES = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
STATUS = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID_ARG", 2: "ATTN_ERR_UNSUPPORTED", 3: "ATTN_ERR_WORKSPACE",
          4: "ATTN_ERR_HIP", 5: "ATTN_ERR_NO_BLOCKS"}
EXPORTED_SYMBOLS = ("attn_prefill", "attn_prefill_paged", "kv_append", "attn_decode", "attn_decode_paged",
                    "kv_append_fp8", "attn_decode_paged_fp8", "kv_append_int8", "attn_decode_paged_int8",
                    "kv_copy_blocks", "attn_prefill_fp8", "attn_prefill_fp8_workspace_bytes", "kv_append_int4",
                    "attn_decode_paged_int4", "attn_decode_paged_noalloc",
                    "attn_decode_workspace_bytes", "attn_last_error", "attn_version",
                    "attn_device_error_flags",
                    "attn_block_pool_create", "attn_block_pool_destroy", "attn_block_pool_free_blocks",
                    "attn_block_pool_holders", "attn_block_pool_reserve", "attn_block_pool_reserve_batch",
                    "attn_block_pool_release", "attn_block_pool_fork")


class AttnError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """Load libattn.so (built in-tree by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is missing: build it with "
                          "`python -m kv_cache_flashattention_attn_amd.build`")
    L = ctypes.CDLL(lib_path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.attn_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, i32, i32, vp]
    L.attn_prefill_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, f32,
                                     i32, vp]
    L.kv_append.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32, vp]
    L.kv_append_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f32, f32, vp]
    L.attn_decode_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, f32,
                                        f32, i32, i32, vp, sz, vp]
    L.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, sz, vp]
    L.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                    i32, vp, sz, vp]
    L.attn_decode_paged_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, i32,
                                            i32, vp]
    L.attn_decode_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.attn_decode_workspace_bytes.restype = sz
    L.attn_last_error.restype = ctypes.c_char_p
    L.attn_version.restype = ctypes.c_char_p
    L.attn_device_error_flags.argtypes = [vp]
    L.kv_copy_blocks.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.attn_prefill_fp8.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, f32, f32, f32, i32, i32, vp,
                                   sz, vp]
    L.attn_prefill_fp8_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.attn_prefill_fp8_workspace_bytes.restype = sz
    L.kv_append_int8.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    L.attn_decode_paged_int8.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, f32, vp,
                                         vp, i32, i32, vp, sz, vp]
    L.kv_append_int4.argtypes = L.kv_append_int8.argtypes
    L.attn_decode_paged_int4.argtypes = L.attn_decode_paged_int8.argtypes
    L.attn_block_pool_create.argtypes = [i32]
    L.attn_block_pool_create.restype = vp
    L.attn_block_pool_destroy.argtypes = [vp]
    L.attn_block_pool_destroy.restype = None
    L.attn_block_pool_free_blocks.argtypes = [vp]
    L.attn_block_pool_holders.argtypes = [vp, i32]
    L.attn_block_pool_reserve.argtypes = [vp, vp, i32, i32, i32, vp]
    L.attn_block_pool_reserve_batch.argtypes = [vp, vp, i32, i32, vp, vp, vp, vp, vp]
    L.attn_block_pool_release.argtypes = [vp, vp, i32, i32]
    L.attn_block_pool_fork.argtypes = [vp, vp, vp, i32, i32]
    for name in ("attn_prefill", "attn_prefill_paged", "kv_append", "attn_decode", "attn_decode_paged",
                 "kv_append_fp8", "attn_decode_paged_fp8", "attn_device_error_flags", "kv_copy_blocks",
                 "kv_append_int8", "attn_decode_paged_int8", "attn_prefill_fp8", "kv_append_int4",
                 "attn_decode_paged_int4", "attn_decode_paged_noalloc",
                 "attn_block_pool_free_blocks", "attn_block_pool_holders", "attn_block_pool_reserve",
                 "attn_block_pool_reserve_batch", "attn_block_pool_release", "attn_block_pool_fork"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise AttnError(fn, rc, lib().attn_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _code(t: torch.Tensor) -> int:
    if t.dtype not in DTYPE_CODES:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return DTYPE_CODES[t.dtype]


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                 scale: Optional[float] = None, return_lse: bool = False, out_fp32: bool = False,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
    """softmax(scale * Q K^T) V for q [B, H_q, N, d] and k, v [B, H_kv, N, d]."""
    B, H_q, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_kv, N, d] matching q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if out_fp32 else q.dtype, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, N), dtype=torch.float32, device=q.device)
    rc = lib().attn_prefill(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"),
                            _dev(lse, "lse", torch.float32) if return_lse else 0,
                            B, H_q, H_kv, N, d, int(bool(causal)), scale, _code(q), int(bool(out_fp32)),
                            _stream())
    _check("attn_prefill", rc)
    return (out, lse) if return_lse else out


def attn_prefill_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                       cache_lens: torch.Tensor, causal: bool = True, scale: Optional[float] = None,
                       return_lse: bool = False, out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None):
    """Chunk of n_new queries per sequence, q [B, H_q, n_new, d], against paged pools
    [num_blocks, H_kv, 16, d] that already hold the chunk's keys (query t of sequence b
    is token cache_lens[b] + t)."""
    B, H_q, n_new, d = q.shape
    nb, H_kv, bs, _ = k_pool.shape
    if v_pool.shape != k_pool.shape or k_pool.dtype != q.dtype or v_pool.dtype != q.dtype:
        raise ValueError("k_pool and v_pool must match each other and q's dtype")
    mbps = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = torch.empty_like(q) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, n_new), dtype=torch.float32, device=q.device)
    rc = lib().attn_prefill_paged(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                  _dev(block_table, "block_table", torch.int32),
                                  _dev(cache_lens, "cache_lens", torch.int32), _dev(out, "out"),
                                  _dev(lse, "lse", torch.float32) if return_lse else 0,
                                  B, H_q, H_kv, n_new, d, bs, mbps, nb, int(bool(causal)), scale, _code(q),
                                  _stream())
    _check("attn_prefill_paged", rc)
    return (out, lse) if return_lse else out


def kv_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
              cache_lens: torch.Tensor, block_table: Optional[torch.Tensor] = None) -> None:
    """Write k_new/v_new [B, H_kv, n_new, d] at positions cache_lens[b] + t.

    Contiguous caches are [B, H_kv, max_len, d]; with a block table the caches are
    pools [num_blocks, H_kv, 16, d] and block_table is int32 [B, max_blocks_per_seq].
    """
    B, H_kv, n_new, d = k_new.shape
    if v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must match")
    if k_cache.shape != v_cache.shape or k_cache.dtype != k_new.dtype or v_cache.dtype != k_new.dtype:
        raise ValueError("caches must match each other and the new rows' dtype")
    if block_table is None:
        max_len, bs, mbps, nb = k_cache.shape[2], 16, 0, 0
    else:
        max_len, bs, mbps, nb = 0, k_cache.shape[2], block_table.shape[1], k_cache.shape[0]
    rc = lib().kv_append(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_new, "k_new"),
                         _dev(v_new, "v_new"), _dev(cache_lens, "cache_lens", torch.int32),
                         _dev(block_table, "block_table", torch.int32), B, H_kv, n_new, d, max_len, bs,
                         mbps, nb, _code(k_new), _stream())
    _check("kv_append", rc)


def attn_decode_workspace_bytes(B: int, H_q: int, max_seq_len: int, d: int) -> int:
    return int(lib().attn_decode_workspace_bytes(B, H_q, max_seq_len, d))


def _workspace(ws: Optional[torch.Tensor], nbytes: int, device) -> torch.Tensor:
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws


def _out(q: torch.Tensor, shape, out_fp32: bool, dtype=None) -> torch.Tensor:
    return torch.empty(shape, dtype=torch.float32 if out_fp32 else (dtype or q.dtype), device=q.device)


def attn_decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, seq_lens: torch.Tensor,
                scale: Optional[float] = None, return_lse: bool = False,
                workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """One query per head, q [B, H_q, d], against a contiguous cache [B, H_kv, max_len, d].
    ``out_fp32``: the output in fp32 (the result before its rounding to q's dtype)."""
    B, H_q, d = q.shape
    _, H_kv, max_len, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = attn_decode_workspace_bytes(B, H_q, max_len, d)
    workspace = _workspace(workspace, nbytes, q.device)
    out = _out(q, q.shape, out_fp32) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = lib().attn_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(seq_lens, "seq_lens", torch.int32), _dev(out, "out"),
                           _dev(lse, "lse", torch.float32) if return_lse else 0,
                           B, H_q, H_kv, max_len, d, scale, _code(q), int(bool(out_fp32)),
                           _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream())
    _check("attn_decode", rc)
    return (out, lse) if return_lse else out


def attn_decode_paged(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                      seq_lens: torch.Tensor, scale: Optional[float] = None, return_lse: bool = False,
                      workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                      lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """attn_decode over pools [num_blocks, H_kv, 16, d] and an int32 block table [B, max_blocks]."""
    B, H_q, d = q.shape
    nb, H_kv, bs, _ = k_pool.shape
    mbps = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = attn_decode_workspace_bytes(B, H_q, mbps * bs, d)
    workspace = _workspace(workspace, nbytes, q.device)
    out = _out(q, q.shape, out_fp32) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = lib().attn_decode_paged(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                 _dev(block_table, "block_table", torch.int32),
                                 _dev(seq_lens, "seq_lens", torch.int32), _dev(out, "out"),
                                 _dev(lse, "lse", torch.float32) if return_lse else 0,
                                 B, H_q, H_kv, d, bs, mbps, nb, scale, _code(q), int(bool(out_fp32)),
                                 _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
                                 _stream())
    _check("attn_decode_paged", rc)
    return (out, lse) if return_lse else out


def attn_decode_paged_noalloc(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                              block_table: torch.Tensor, seq_lens: torch.Tensor, scale: Optional[float] = None,
                              return_lse: bool = False, out: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """attn_decode_paged with the library's static workspace (no workspace argument,
    no allocation in the library; pass ``out`` and ``lse`` to allocate nothing here either)."""
    B, H_q, d = q.shape
    nb, H_kv, bs, _ = k_pool.shape
    mbps = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out = _out(q, q.shape, out_fp32) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = lib().attn_decode_paged_noalloc(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                         _dev(block_table, "block_table", torch.int32),
                                         _dev(seq_lens, "seq_lens", torch.int32), _dev(out, "out"),
                                         _dev(lse, "lse", torch.float32) if return_lse else 0,
                                         B, H_q, H_kv, d, bs, mbps, nb, scale, _code(q), int(bool(out_fp32)),
                                         _stream())
    _check("attn_decode_paged_noalloc", rc)
    return (out, lse) if return_lse else out


def kv_append_fp8(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                  cache_lens: torch.Tensor, block_table: torch.Tensor, k_scale: float = 1.0,
                  v_scale: float = 1.0) -> None:
    """Quantize and append k_new, v_new [B, H_kv, n_new, d] into FP8 E4M3 pools (uint8
    tensors [num_blocks, H_kv, 16, d])."""
    B, H_kv, n_new, d = k_new.shape
    nb, _, bs, _ = k_pool.shape
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise ValueError("FP8 pools are uint8 tensors of E4M3 codes")
    rc = lib().kv_append_fp8(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                             _dev(v_new, "v_new"), _dev(cache_lens, "cache_lens", torch.int32),
                             _dev(block_table, "block_table", torch.int32), B, H_kv, n_new, d, bs,
                             block_table.shape[1], nb, _code(k_new), float(k_scale), float(v_scale), _stream())
    _check("kv_append_fp8", rc)


def attn_decode_paged_fp8(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                          seq_lens: torch.Tensor, k_scale: float = 1.0, v_scale: float = 1.0,
                          scale: Optional[float] = None, return_lse: bool = False,
                          workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """attn_decode_paged over FP8 E4M3 pools (uint8 [num_blocks, H_kv, 16, d])."""
    B, H_q, d = q.shape
    nb, H_kv, bs, _ = k_pool.shape
    mbps = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = attn_decode_workspace_bytes(B, H_q, mbps * bs, d)
    workspace = _workspace(workspace, nbytes, q.device)
    out = _out(q, q.shape, out_fp32) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = lib().attn_decode_paged_fp8(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                                     _dev(block_table, "block_table", torch.int32),
                                     _dev(seq_lens, "seq_lens", torch.int32), _dev(out, "out"),
                                     _dev(lse, "lse", torch.float32) if return_lse else 0,
                                     B, H_q, H_kv, d, bs, mbps, nb, scale, float(k_scale), float(v_scale), _code(q),
                                     int(bool(out_fp32)), _dev(workspace, "workspace"),
                                     workspace.numel() * workspace.element_size(), _stream())
    _check("attn_decode_paged_fp8", rc)
    return (out, lse) if return_lse else out


def attn_device_error_flags() -> int:
    """Synchronise the current stream, then read and clear the kernels' error flags."""
    v = lib().attn_device_error_flags(_stream())
    if v < 0:
        raise AttnError("attn_device_error_flags", 4, "HIP call failed")
    return v


def attn_version() -> str:
    return lib().attn_version().decode()


def kv_copy_blocks(k_pool: torch.Tensor, v_pool: torch.Tensor, pairs: torch.Tensor) -> None:
    """Copy whole blocks of both pools ([num_blocks, H_kv, 16, d], any element
    size) for each (src, dst) row of the device int32 tensor ``pairs`` [n, 2]."""
    nb, H_kv, bs, d = k_pool.shape
    if v_pool.shape != k_pool.shape or v_pool.dtype != k_pool.dtype:
        raise ValueError("k_pool and v_pool must match")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be [n, 2]")
    rc = lib().kv_copy_blocks(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(pairs, "pairs", torch.int32),
                              pairs.shape[0], H_kv, d, bs, nb, k_pool.element_size(), _stream())
    _check("kv_copy_blocks", rc)


def _append_int(fn: str, nib: int, k_pool, v_pool, k_new, v_new, cache_lens, block_table, k_scales, v_scales):
    B, H_kv, n_new, d = k_new.shape
    nb, _, bs, _ = k_pool.shape
    if k_pool.shape[-1] * nib != d or v_pool.shape != k_pool.shape:
        raise ValueError(f"{fn}: pools must be [num_blocks, H_kv, 16, d{'/2' if nib == 2 else ''}]")
    if k_scales.shape != (H_kv, d) or v_scales.shape != (H_kv, d):
        raise ValueError("k_scales and v_scales must be [H_kv, d]")
    rc = getattr(lib(), fn)(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"), _dev(k_new, "k_new"),
                            _dev(v_new, "v_new"), _dev(cache_lens, "cache_lens", torch.int32),
                            _dev(block_table, "block_table", torch.int32), B, H_kv, n_new, d, bs,
                            block_table.shape[1], nb, _code(k_new), _dev(k_scales, "k_scales", torch.float32),
                            _dev(v_scales, "v_scales", torch.float32), _stream())
    _check(fn, rc)


def kv_append_int8(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   cache_lens: torch.Tensor, block_table: torch.Tensor, k_scales: torch.Tensor,
                   v_scales: torch.Tensor) -> None:
    """Quantize and append k_new, v_new [B, H_kv, n_new, d] into int8 pools
    [num_blocks, H_kv, 16, d] with per-channel scales (device fp32 [H_kv, d])."""
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8:
        raise ValueError("int8 pools are torch.int8 tensors")
    _append_int("kv_append_int8", 1, k_pool, v_pool, k_new, v_new, cache_lens, block_table, k_scales, v_scales)


def kv_append_int4(k_pool: torch.Tensor, v_pool: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                   cache_lens: torch.Tensor, block_table: torch.Tensor, k_scales: torch.Tensor,
                   v_scales: torch.Tensor) -> None:
    """Quantize and append into int4 pools (torch.uint8 [num_blocks, H_kv, 16, d / 2],
    two codes per byte) with per-channel scales (device fp32 [H_kv, d])."""
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise ValueError("int4 pools are torch.uint8 tensors of packed codes")
    _append_int("kv_append_int4", 2, k_pool, v_pool, k_new, v_new, cache_lens, block_table, k_scales, v_scales)


def _decode_int(fn: str, nib: int, q, k_pool, v_pool, block_table, seq_lens, k_scales, v_scales, scale, return_lse,
                workspace, out, lse, out_fp32=False):
    B, H_q, d = q.shape
    nb, H_kv, bs, _ = k_pool.shape
    if k_pool.shape[-1] * nib != d or v_pool.shape != k_pool.shape:
        raise ValueError(f"{fn}: pools must be [num_blocks, H_kv, 16, d{'/2' if nib == 2 else ''}]")
    if k_scales.shape != (H_kv, d) or v_scales.shape != (H_kv, d):
        raise ValueError("k_scales and v_scales must be [H_kv, d]")
    mbps = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = attn_decode_workspace_bytes(B, H_q, mbps * bs, d)
    workspace = _workspace(workspace, nbytes, q.device)
    out = _out(q, q.shape, out_fp32) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    rc = getattr(lib(), fn)(_dev(q, "q"), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool"),
                            _dev(block_table, "block_table", torch.int32),
                            _dev(seq_lens, "seq_lens", torch.int32), _dev(out, "out"),
                            _dev(lse, "lse", torch.float32) if return_lse else 0,
                            B, H_q, H_kv, d, bs, mbps, nb, scale,
                            _dev(k_scales, "k_scales", torch.float32),
                            _dev(v_scales, "v_scales", torch.float32), _code(q), int(bool(out_fp32)),
                            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream())
    _check(fn, rc)
    return (out, lse) if return_lse else out


def attn_decode_paged_int8(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, k_scales: torch.Tensor, v_scales: torch.Tensor,
                           scale: Optional[float] = None, return_lse: bool = False,
                           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """attn_decode_paged over int8 pools (torch.int8 [num_blocks, H_kv, 16, d])
    with per-channel scales (device fp32 [H_kv, d])."""
    if k_pool.dtype != torch.int8 or v_pool.dtype != torch.int8:
        raise ValueError("int8 pools are torch.int8 tensors")
    return _decode_int("attn_decode_paged_int8", 1, q, k_pool, v_pool, block_table, seq_lens, k_scales, v_scales,
                       scale, return_lse, workspace, out, lse, out_fp32)


def attn_decode_paged_int4(q: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor, block_table: torch.Tensor,
                           seq_lens: torch.Tensor, k_scales: torch.Tensor, v_scales: torch.Tensor,
                           scale: Optional[float] = None, return_lse: bool = False,
                           workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """attn_decode_paged over int4 pools (torch.uint8 [num_blocks, H_kv, 16, d / 2])
    with per-channel scales (device fp32 [H_kv, d])."""
    if k_pool.dtype != torch.uint8 or v_pool.dtype != torch.uint8:
        raise ValueError("int4 pools are torch.uint8 tensors of packed codes")
    return _decode_int("attn_decode_paged_int4", 2, q, k_pool, v_pool, block_table, seq_lens, k_scales, v_scales,
                       scale, return_lse, workspace, out, lse, out_fp32)


def attn_prefill_fp8_workspace_bytes(B: int, H_kv: int, N: int, d: int) -> int:
    return int(lib().attn_prefill_fp8_workspace_bytes(B, H_kv, N, d))


def attn_prefill_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                     scale: Optional[float] = None, q_scale: float = 1.0, k_scale: float = 1.0, v_scale: float = 1.0,
                     out_dtype=torch.bfloat16, return_lse: bool = False, workspace: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None, out_fp32: bool = False):
    """Attention over FP8 E4M3 codes (uint8) q [B, H_q, N, d], k, v [B, H_kv, N, d],
    each times its scale; the output in out_dtype (torch.bfloat16 or torch.float16),
    or in fp32 with ``out_fp32`` (the result before its rounding to out_dtype)."""
    B, H_q, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d) or v.shape != k.shape:
        raise ValueError("k and v must be [B, H_kv, N, d] matching q")
    if q.dtype != torch.uint8 or k.dtype != torch.uint8 or v.dtype != torch.uint8:
        raise ValueError("FP8 inputs are uint8 tensors of E4M3 codes")
    if out_dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float16")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    del workspace  # accepted for compatibility; the kernel widens V on chip and needs none
    out = _out(q, (B, H_q, N, d), out_fp32, out_dtype) if out is None else out
    if return_lse and lse is None:
        lse = torch.empty((B, H_q, N), dtype=torch.float32, device=q.device)
    rc = lib().attn_prefill_fp8(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
                                _dev(out, "out", torch.float32 if out_fp32 else out_dtype),
                                _dev(lse, "lse", torch.float32) if return_lse else 0, B, H_q, H_kv, N, d,
                                int(bool(causal)), scale, float(q_scale), float(k_scale), float(v_scale),
                                DTYPE_CODES[out_dtype], int(bool(out_fp32)), None, 0, _stream())
    _check("attn_prefill_fp8", rc)
    return (out, lse) if return_lse else out
