"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module only *draws and lays out* inputs: it holds none of the attention
arithmetic.  Every tensor is returned as a numpy array of its storage bits:

* ``f32``  -> ``np.float32`` (the value is its own bit pattern),
* ``f16``  -> ``np.uint16`` holding IEEE binary16 bits,
* ``bf16`` -> ``np.uint16`` holding bfloat16 bits (upper half of a binary32).

Values are drawn as float32 standard normals from ``numpy.random.SFC64(seed)``
and rounded to the storage type with round-to-nearest-even, so the GPU path and
the CPU oracle always see the very same bytes.

Workload shapes follow the pages: the ``[B, H, T, d]`` layout of the KV-cache
tables ("KV Cache:推理慢的真正原因", section 缓存的是什么), the fp16
``[1, 8, 1024, 64]`` example of "推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理"
(section 三、实际落地), the 7B / 70B layer shapes of "KV缓存与Flash注意力"
(section KV缓存数学) and 16-token physical blocks with a block table
("KV Cache:推理慢的真正原因", section 工程优化手段 / PagedAttention).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16}
BLOCK_SIZE = 16

# Filler for cache slots that hold no token: K = 0 and V = 8192.  A kernel that
# gives any weight to such a slot picks up an error of order 8192 * weight.
SENTINEL_K = 0.0
SENTINEL_V = 8192.0


# --------------------------------------------------------------------------
# rounding float32 -> storage bits (input preparation, pinned by unit tests)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE binary16 (numpy's cast is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_fill(shape, value: float, dtype: str) -> np.ndarray:
    one = to_storage(np.array([value], dtype=np.float32), dtype)[0]
    return np.full(shape, one, dtype=STORAGE[dtype])


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = rng.standard_normal(int(np.prod(shape)), dtype=np.float32).reshape(shape)
    return to_storage(x, dtype)


def make_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.SFC64(seed))


# --------------------------------------------------------------------------
# workload definitions
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillCase:
    name: str
    B: int
    H_q: int
    H_kv: int
    N: int
    d: int
    dtype: str
    causal: bool
    want_lse: bool
    seed: int
    scale: Optional[float] = None  # None -> 1/sqrt(d)

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*d per visible (query, key) pair (QK^T and PV)."""
        pairs = self.N * (self.N + 1) // 2 if self.causal else self.N * self.N
        return 4.0 * self.d * self.B * self.H_q * pairs


@dataclasses.dataclass(frozen=True)
class DecodeCase:
    name: str
    B: int
    H_q: int
    H_kv: int
    d: int
    dtype: str
    len_lo: int          # cached tokens before the append, inclusive bounds
    len_hi: int
    paged: bool
    seed: int
    n_new: int = 1
    scale: Optional[float] = None

    @property
    def sm_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def max_len(self) -> int:
        """Contiguous capacity: room for len_hi + n_new tokens, a multiple of 16."""
        need = self.len_hi + self.n_new
        return -(-need // BLOCK_SIZE) * BLOCK_SIZE

    @property
    def max_blocks(self) -> int:
        return -(-(self.len_hi + self.n_new) // BLOCK_SIZE)


# The five workloads: one tiny fp32 exactness case, two prefill shapes and two
# decode shapes.  Seeds are the workload's index.
TINY_PREFILL = PrefillCase("tiny_f32_prefill", 1, 2, 2, 64, 16, "f32", False, True, 0)
TINY_DECODE_STEPS = 16
PREFILL_F16 = PrefillCase("prefill_f16_1x8x1024x64", 1, 8, 8, 1024, 64, "f16", False, False, 1)
PREFILL_BF16_CAUSAL = PrefillCase("prefill_bf16_causal_4x32x4096x128", 4, 32, 32, 4096, 128,
                                  "bf16", True, True, 2)
DECODE_CONTIG = DecodeCase("decode_bf16_gqa_contig_b32_hq64_hkv8", 32, 64, 8, 128, "bf16",
                           1024, 32768, False, 3)
DECODE_PAGED = DecodeCase("decode_bf16_gqa_paged_b64_hq32_hkv8", 64, 32, 8, 128, "bf16",
                          128, 8192, True, 4)

WORKLOADS = {c.name: c for c in (TINY_PREFILL, PREFILL_F16, PREFILL_BF16_CAUSAL,
                                 DECODE_CONTIG, DECODE_PAGED)}

# Beyond the five: a chunked prefill against the paged cache, 512 new tokens per
# sequence after a cached prefix of 0 .. 4096 tokens (shaped like the paged
# decode layer: GQA 32 / 8 heads, d = 128).
CHUNK_PAGED = DecodeCase("chunk_prefill_bf16_paged_b16_hq32_hkv8_n512", 16, 32, 8, 128, "bf16",
                         0, 4096, True, 5, n_new=512)


# --------------------------------------------------------------------------
# prefill inputs
# --------------------------------------------------------------------------
def prefill_inputs(case: PrefillCase) -> Dict[str, np.ndarray]:
    """Draw order: Q, then K, then V (each the full tensor, C order)."""
    rng = make_rng(case.seed)
    q = _normal(rng, (case.B, case.H_q, case.N, case.d), case.dtype)
    k = _normal(rng, (case.B, case.H_kv, case.N, case.d), case.dtype)
    v = _normal(rng, (case.B, case.H_kv, case.N, case.d), case.dtype)
    return {"q": q, "k": k, "v": v}


def random_prefill(seed: int, B: int, H_q: int, H_kv: int, N: int, d: int, dtype: str,
                   scale_by: float = 1.0) -> Dict[str, np.ndarray]:
    """Small ad-hoc prefill inputs for the edge-case sweeps."""
    rng = make_rng(seed)
    out = {}
    for name, H in (("q", H_q), ("k", H_kv), ("v", H_kv)):
        x = rng.standard_normal(B * H * N * d, dtype=np.float32).reshape(B, H, N, d)
        out[name] = to_storage(x * np.float32(scale_by), dtype)
    return out


# --------------------------------------------------------------------------
# decode inputs
# --------------------------------------------------------------------------
def draw_lengths(rng: np.random.Generator, B: int, lo: int, hi: int) -> np.ndarray:
    """Integer lengths uniform on [lo, hi], both ends inclusive."""
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


def block_table_from_perm(lens_after: np.ndarray, perm: np.ndarray, max_blocks: int) -> np.ndarray:
    """Sequence b takes the next ceil(len_b/16) ids of ``perm`` in order; -1 elsewhere."""
    B = lens_after.shape[0]
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    cur = 0
    for b in range(B):
        nb = -(-int(lens_after[b]) // BLOCK_SIZE)
        table[b, :nb] = perm[cur:cur + nb]
        cur += nb
    return table


def decode_inputs(case: DecodeCase, lens: Optional[np.ndarray] = None,
                  rng: Optional[np.random.Generator] = None) -> Dict[str, np.ndarray]:
    """Inputs of one decode step: cache (before the append), q, k_new, v_new.

    Draw order from ``SFC64(case.seed)``: lengths (unless given); then for each
    sequence b in order its cached K rows ``[H_kv, L_b, d]`` followed by its V
    rows; then q ``[B, H_q, d]``; k_new; v_new ``[B, H_kv, n_new, d]``; then (paged
    only) a permutation of the pool's block ids.

    ``lens`` holds the tokens cached *before* the append; attention after the
    append covers ``lens + n_new`` tokens.  Contiguous caches are
    ``[B, H_kv, max_len, d]``; paged pools are ``[num_blocks, H_kv, 16, d]`` with
    exactly the blocks the sequences need after the append (the append's slots
    are already owned) and an int32 block table ``[B, max_blocks]``.  Slots that
    hold no token carry the K/V sentinels.
    """
    rng = rng if rng is not None else make_rng(case.seed)
    if lens is None:
        lens = draw_lengths(rng, case.B, case.len_lo, case.len_hi)
    lens = np.asarray(lens, dtype=np.int32)
    B, Hk, d, dt = case.B, case.H_kv, case.d, case.dtype
    lens_after = lens + case.n_new
    per_seq_k: List[np.ndarray] = []
    per_seq_v: List[np.ndarray] = []
    for b in range(B):
        L = int(lens[b])
        per_seq_k.append(_normal(rng, (Hk, L, d), dt))
        per_seq_v.append(_normal(rng, (Hk, L, d), dt))
    q = _normal(rng, (B, case.H_q, d), dt)
    k_new = _normal(rng, (B, Hk, case.n_new, d), dt)
    v_new = _normal(rng, (B, Hk, case.n_new, d), dt)
    out = {"lens": lens, "q": q, "k_new": k_new, "v_new": v_new}
    if not case.paged:
        kc = storage_fill((B, Hk, case.max_len, d), SENTINEL_K, dt)
        vc = storage_fill((B, Hk, case.max_len, d), SENTINEL_V, dt)
        for b in range(B):
            L = int(lens[b])
            kc[b, :, :L] = per_seq_k[b]
            vc[b, :, :L] = per_seq_v[b]
        out.update(k_cache=kc, v_cache=vc)
    else:
        nblk = int(sum(-(-int(x) // BLOCK_SIZE) for x in lens_after))
        perm = rng.permutation(nblk).astype(np.int32)
        table = block_table_from_perm(lens_after, perm, case.max_blocks)
        kp = storage_fill((nblk, Hk, BLOCK_SIZE, d), SENTINEL_K, dt)
        vp = storage_fill((nblk, Hk, BLOCK_SIZE, d), SENTINEL_V, dt)
        for b in range(B):
            L = int(lens[b])
            for j in range(-(-L // BLOCK_SIZE)):
                lo, hi = j * BLOCK_SIZE, min(L, (j + 1) * BLOCK_SIZE)
                blk = table[b, j]
                kp[blk, :, :hi - lo] = per_seq_k[b][:, lo:hi]
                vp[blk, :, :hi - lo] = per_seq_v[b][:, lo:hi]
        out.update(k_pool=kp, v_pool=vp, block_table=table)
    del per_seq_k, per_seq_v
    return out


def chunk_inputs(case: DecodeCase, lens: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Inputs of one chunked-prefill step: a chunk of ``case.n_new`` new tokens per
    sequence, each with a query.

    Everything of ``decode_inputs(case, lens)`` (cache before the chunk, lengths,
    the chunk's K/V rows ``[B, H_kv, n_new, d]``); its single-token q is replaced
    by the chunk's queries ``[B, H_q, n_new, d]`` drawn from ``SFC64(case.seed + 5000)``.
    """
    out = decode_inputs(case, lens=lens)
    rng = make_rng(case.seed + 5000)
    out["q"] = _normal(rng, (case.B, case.H_q, case.n_new, case.d), case.dtype)
    return out


def chunk_flops(lens: np.ndarray, n_new: int, H_q: int, d: int, causal: bool = True) -> float:
    """Algorithmic FLOPs of a chunk step: 4*d per visible (query, key) pair."""
    L = lens.astype(np.int64)
    if causal:  # query t sees L + t + 1 keys
        pairs = int(np.sum(L * n_new + n_new * (n_new + 1) // 2))
    else:
        pairs = int(np.sum((L + n_new) * n_new))
    return 4.0 * d * H_q * pairs


def fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    """Uniform over the 254 finite OCP FP8 E4M3 codes: every byte but 0x7F and
    0xFF (the two NaNs), i.e. both signs, all sixteen exponent fields (field 0
    holds the subnormals) and every mantissa, up to +-448."""
    c = rng.integers(0, 254, size=shape, dtype=np.uint8)
    return (c + (c >= 0x7F).astype(np.uint8)).astype(np.uint8)


# E4M3 scales that keep the full code range usable at the decode and prefill
# tolerances: K values up to 448 / 64 = 7 (logits of order one against N(0,1)
# queries at d = 128) and V values up to 448 / 256 = 1.75 (outputs of order
# one, where a 16-bit output's storage rounding is below 1e-2).
FP8_K_SCALE = 1.0 / 64
FP8_V_SCALE = 1.0 / 256
FP8_Q_SCALE = 1.0 / 64


def fp8_decode_inputs(case: DecodeCase, lens: Optional[np.ndarray] = None,
                      base: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """Inputs of one decode step over an 8-bit (OCP FP8 E4M3) paged cache.

    Lengths, block table, q and the new token's K/V rows (in ``case.dtype``) are
    those of ``decode_inputs(case, lens)`` (or of ``base``, a result of that
    call, passed to skip drawing it again).  The pools hold E4M3 codes (uint8)
    drawn from ``SFC64(case.seed + 7000)``, uniform over every finite code
    (``fp8_codes``), K's pool then V's; slots that hold no token carry code 0x7F
    (NaN) in both, which a decode must never weigh.
    """
    out = dict(base) if base is not None else decode_inputs(case, lens=lens)
    lens = out["lens"]
    table = out["block_table"]
    nblk, Hk, bs, d = out["k_pool"].shape
    rng = make_rng(case.seed + 7000)

    # which (block, slot) pairs hold a cached token
    held = np.zeros((nblk, bs), dtype=bool)
    for b in range(case.B):
        L = int(lens[b])
        nb = -(-L // BLOCK_SIZE)
        fill = np.clip(L - BLOCK_SIZE * np.arange(nb), 0, BLOCK_SIZE)
        held[table[b, :nb]] = np.arange(bs)[None, :] < fill[:, None]
    mask = held[:, None, :, None]
    kp = np.where(mask, fp8_codes(rng, (nblk, Hk, bs, d)), np.uint8(0x7F)).astype(np.uint8)
    vp = np.where(mask, fp8_codes(rng, (nblk, Hk, bs, d)), np.uint8(0x7F)).astype(np.uint8)
    out.update(k_pool=kp, v_pool=vp)
    return out


def int8_decode_inputs(case: DecodeCase, lens: Optional[np.ndarray] = None,
                       base: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """Inputs of one decode step over an int8 paged cache with per-channel scales.

    Lengths, block table, q and the new token's K/V rows (in ``case.dtype``) are
    those of ``decode_inputs(case, lens)`` (or of ``base``).  From
    ``SFC64(case.seed + 8000)``, in this order:

    * ``k_scales``, ``v_scales`` [H_kv, d] float32: 2^u with u uniform in
      [-9, -6) (values up to 2), and in every KV head 4 random channels of K
      multiplied by 8 (outlier key channels, values up to 16);
    * the pools' codes: K's whole pool then V's, uniform integers in
      [-127, 127] where a slot holds a cached token; slots holding none carry
      K = 0 and V = 127 (the largest code).
    """
    out = dict(base) if base is not None else decode_inputs(case, lens=lens)
    lens = out["lens"]
    table = out["block_table"]
    nblk, Hk, bs, d = out["k_pool"].shape
    rng = make_rng(case.seed + 8000)
    ks = np.exp2(rng.uniform(-9.0, -6.0, size=(Hk, d))).astype(np.float32)
    for h in range(Hk):
        ks[h, rng.choice(d, size=4, replace=False)] *= np.float32(8.0)
    vs = np.exp2(rng.uniform(-9.0, -6.0, size=(Hk, d))).astype(np.float32)
    held = np.zeros((nblk, bs), dtype=bool)
    for b in range(case.B):
        L = int(lens[b])
        nb = -(-L // BLOCK_SIZE)
        fill = np.clip(L - BLOCK_SIZE * np.arange(nb), 0, BLOCK_SIZE)
        held[table[b, :nb]] = np.arange(bs)[None, :] < fill[:, None]
    mask = held[:, None, :, None]
    kp = np.where(mask, rng.integers(-127, 128, size=(nblk, Hk, bs, d), dtype=np.int8), np.int8(0))
    vp = np.where(mask, rng.integers(-127, 128, size=(nblk, Hk, bs, d), dtype=np.int8), np.int8(127))
    out.update(k_pool=kp.astype(np.int8), v_pool=vp.astype(np.int8), k_scales=ks, v_scales=vs)
    return out


def int4_decode_inputs(case: DecodeCase, lens: Optional[np.ndarray] = None,
                       base: Optional[Dict[str, np.ndarray]] = None) -> Dict[str, np.ndarray]:
    """Inputs of one decode step over an int4 paged cache with per-channel scales.

    Lengths, block table, q and the new rows as in ``decode_inputs``; from
    ``SFC64(case.seed + 8500)``: ``k_scales``, ``v_scales`` [H_kv, d] float32,
    2^u with u uniform in [-5, -2) and, in every KV head, 4 random key channels
    8x larger; then the pools' packed bytes [num_blocks, H_kv, 16, d / 2], K's
    then V's: uniform random bytes where a byte holds a token (two uniform codes
    in [-8, 7] each; -8 never comes out of quantization but decodes like any
    code); bytes of slots holding none carry 0x00 in K and 0x77 (codes 7, 7) in
    V.  A K byte belongs to the token of its row; V's bytes of a (block, KV
    head) are in the pool's order, where byte o belongs to token
    4 ((o // (d / 8)) // 16) + (0, 2, 1, 3)[(o % (d / 8)) % 4].
    """
    out = dict(base) if base is not None else decode_inputs(case, lens=lens)
    lens = out["lens"]
    table = out["block_table"]
    nblk, Hk, bs, d = out["k_pool"].shape
    rng = make_rng(case.seed + 8500)
    ks = np.exp2(rng.uniform(-5.0, -2.0, size=(Hk, d))).astype(np.float32)
    for h in range(Hk):
        ks[h, rng.choice(d, size=4, replace=False)] *= np.float32(8.0)
    vs = np.exp2(rng.uniform(-5.0, -2.0, size=(Hk, d))).astype(np.float32)
    held = np.zeros((nblk, bs), dtype=bool)
    for b in range(case.B):
        L = int(lens[b])
        nb = -(-L // BLOCK_SIZE)
        fill = np.clip(L - BLOCK_SIZE * np.arange(nb), 0, BLOCK_SIZE)
        held[table[b, :nb]] = np.arange(bs)[None, :] < fill[:, None]
    mask = held[:, None, :, None]
    shape = (nblk, Hk, bs, d // 2)
    o = np.arange(8 * d)
    vtok = (4 * ((o // (d // 8)) // 16) + np.array([0, 2, 1, 3])[(o % (d // 8)) % 4]).reshape(bs, d // 2)
    vmask = held[:, None, vtok]
    kp = np.where(mask, rng.integers(0, 256, size=shape, dtype=np.uint8), np.uint8(0x00))
    vp = np.where(vmask, rng.integers(0, 256, size=shape, dtype=np.uint8), np.uint8(0x77))
    out.update(k_pool=kp.astype(np.uint8), v_pool=vp.astype(np.uint8), k_scales=ks, v_scales=vs)
    return out


def fp8_prefill_inputs(case: PrefillCase) -> Dict[str, np.ndarray]:
    """Q, K, V of ``case``'s shapes as OCP FP8 E4M3 codes (uint8), drawn from
    ``SFC64(case.seed + 9000)`` in the order Q, K, V, each uniform over every
    finite code (``fp8_codes``: subnormals, all exponent fields, +-448)."""
    rng = make_rng(case.seed + 9000)
    return {"q": fp8_codes(rng, (case.B, case.H_q, case.N, case.d)),
            "k": fp8_codes(rng, (case.B, case.H_kv, case.N, case.d)),
            "v": fp8_codes(rng, (case.B, case.H_kv, case.N, case.d))}


def tiny_decode_steps(case: PrefillCase = TINY_PREFILL, steps: int = TINY_DECODE_STEPS):
    """The tiny case's decode phase: per step a query [B,H,d] and one new K/V row.

    Drawn from ``SFC64(case.seed + 1000)`` in order q, k_new, v_new per step.
    """
    rng = make_rng(case.seed + 1000)
    out = []
    for _ in range(steps):
        q = _normal(rng, (case.B, case.H_q, case.d), case.dtype)
        kn = _normal(rng, (case.B, case.H_kv, 1, case.d), case.dtype)
        vn = _normal(rng, (case.B, case.H_kv, 1, case.d), case.dtype)
        out.append({"q": q, "k_new": kn, "v_new": vn})
    return out


def kv_bytes_read(lens_after: np.ndarray, H_kv: int, d: int, dtype: str) -> int:
    """Bytes of K and V one decode step must read: every valid token, both tensors."""
    return int(np.sum(lens_after.astype(np.int64))) * H_kv * d * 2 * ELEM_BYTES[dtype]


# --------------------------------------------------------------------------
# chat-completion lengths for the block-pool serving simulation
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class ChatCase:
    name: str
    n_requests: int
    prompt_lo: int
    prompt_hi: int
    output_lo: int
    output_hi: int
    max_len: int
    memory_tokens: int
    seed: int


# 1,000 chat completions of different lengths ("KV缓存与Flash注意力", 练习); memory
# for 64 contiguous max_len reservations of 2,048 tokens.
CHAT_SIM = ChatCase("chat_sim_1000_prompt16-1024_out16-1024_max2048_mem131072",
                    1000, 16, 1024, 16, 1024, 2048, 64 * 2048, 11)


def chat_requests(case: ChatCase = CHAT_SIM):
    """Prompt and output lengths (int64 arrays), each uniform over its inclusive
    range, drawn from ``SFC64(case.seed)``: all prompts, then all outputs."""
    rng = make_rng(case.seed)
    prompts = rng.integers(case.prompt_lo, case.prompt_hi + 1, size=case.n_requests)
    outputs = rng.integers(case.output_lo, case.output_hi + 1, size=case.n_requests)
    return prompts.astype(np.int64), outputs.astype(np.int64)
