/*
 * attn.h -- C ABI of libattn: exact softmax attention for MI355X (gfx950).
 *
 * The library computes softmax(scale * Q K^T) V tile by tile with an online
 * softmax (a running maximum and normaliser per query row), so the N x N score
 * matrix never reaches device memory.  This is the tiled method of
 * "推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理" (section 二) and of
 * "KV缓存与Flash注意力" (Flash Attention — 分块技巧, 步骤2), applied to prefill and
 * to incremental decoding against a KV cache ("推理速度慢怎么办？..." section 一;
 * "KV Cache:推理慢的真正原因", 缓存的是什么 and 工程优化手段).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller (the block
 *    pool calls at the end are the exception: they work on host memory only).  Tensors are
 *    dense, row-major (C order) and 16-byte aligned.  The library never
 *    allocates, frees or keeps a pointer after a call returns.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream).
 *    Calls are asynchronous and never synchronise, except
 *    attn_device_error_flags().  The compute calls launch kernels only (no
 *    allocation, no memset, no copy), so a stream under HIP graph capture may
 *    record them; a replay repeats exactly what the call did.  Make one eager
 *    call of each kind before capturing (the first decode call also sizes its
 *    persistent grid from an occupancy query).
 *  - dtype is one of ATTN_F32, ATTN_F16, ATTN_BF16; Q, K, V, caches and the
 *    output share it (unless out_fp32 asks for an fp32 output).  lse outputs
 *    are always fp32, natural log.
 *  - Query head h reads KV head h / (H_q / H_kv): contiguous groups of query
 *    heads share one K/V head (grouped-query attention, "KV Cache:推理慢的真正原因",
 *    工程优化手段 / 2).  H_q must be a multiple of H_kv.
 *  - Return value: ATTN_OK (0) or an error code.  On error nothing is
 *    launched; attn_last_error() returns a message for the calling thread.
 *  - Lengths and block ids that live in device memory cannot be checked on the
 *    host.  Kernels never read or write outside the buffers the sizes describe:
 *    a length beyond the capacity is clamped, an invalid block id is skipped,
 *    and a device error flag is raised (see attn_device_error_flags()).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_dtype { ATTN_F32 = 0, ATTN_F16 = 1, ATTN_BF16 = 2 };

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, H_q % H_kv != 0, misalignment */
  ATTN_ERR_UNSUPPORTED = 2, /* dtype, head dimension or block size not built      */
  ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required          */
  ATTN_ERR_HIP = 4,         /* the HIP runtime refused a launch                    */
  ATTN_ERR_NO_BLOCKS = 5    /* a block pool cannot meet a reservation              */
};

/* Device error flags raised by kernels (bitwise OR), see attn_device_error_flags. */
enum attn_device_error {
  ATTN_DEVERR_LEN_OVERFLOW = 1, /* a length exceeded the cache capacity (clamped)   */
  ATTN_DEVERR_BAD_BLOCK = 2,    /* a block-table entry was < 0 or >= num_blocks      */
  ATTN_DEVERR_BAD_LEN = 4       /* a length was negative (treated as 0)              */
};

/* Head dimensions accepted (any dtype): 16, 32, 64, 128, 256 for the plain
 * kernels; the MFMA prefill and decode kernels serve f16/bf16 at d = 64, 128. */

/*
 * attn_prefill -- attention of N queries over N keys per (batch, head).
 *
 *   q, o : [B, H_q, N, d]      (o is fp32 when out_fp32 != 0)
 *   k, v : [B, H_kv, N, d]
 *   lse  : [B, H_q, N] fp32 or NULL; lse = ln sum_j exp(scale * q_i . k_j)
 *   causal != 0: query i sees keys j <= i only.
 *   scale: multiplies q . k before the softmax (usually 1/sqrt(d), as in the
 *          pages' code, "推理速度慢怎么办？..." sections 一 and 二).
 *
 * The result equals one-shot softmax attention up to rounding: the tiles carry
 * a running (max, sum) pair so the final normalisation is exact
 * ("KV缓存与Flash注意力", 数值技巧 under Flash Attention — 分块技巧).
 * Causal runs skip key tiles wholly above the diagonal and start the longest
 * query tiles first (the causal ordering named for FlashAttention-2 in the
 * 版本演进 table of "KV缓存与Flash注意力").
 * Errors: INVALID_ARG (null q/k/v/o, B/H/N < 1, H_q % H_kv, misaligned),
 *         UNSUPPORTED (dtype, d), HIP.
 */
int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H_q, int H_kv, int N, int d, int causal, float scale,
                 int dtype, int out_fp32, void* stream);

/*
 * kv_append -- write n_new new tokens' K and V rows into a KV cache.
 *
 * Appending only the new token's K/V (instead of recomputing the history) is
 * the whole point of the cache ("推理速度慢怎么办？..." section 一; the append
 * method of the cache class in "KV Cache:推理慢的真正原因", 缓存的是什么, which
 * writes k_new.shape[2] tokens at once).
 *
 *   k_new, v_new : [B, H_kv, n_new, d]
 *   cache_lens   : device int32 [B], tokens already cached for each sequence.
 *                  Token t of sequence b goes to position cache_lens[b] + t.
 *                  cache_lens is read, never advanced: the caller owns lengths.
 *   block_table == NULL: contiguous caches k_cache, v_cache [B, H_kv, max_len, d].
 *   block_table != NULL: paged pools k_cache, v_cache [num_blocks, H_kv, block_size, d]
 *                  and block_table: device int32 [B, max_blocks_per_seq]; token p
 *                  of sequence b lives in block block_table[b][p / block_size] at
 *                  row p % block_size ("KV Cache:推理慢的真正原因", 工程优化手段 / 1).
 *                  block_size must be 16.  max_len is ignored.
 *   contiguous: num_blocks, block_size and max_blocks_per_seq are ignored.
 *
 * A pure bit copy.  Positions past the capacity, or blocks outside [0, num_blocks),
 * are skipped and raise a device error flag.
 * Errors: INVALID_ARG, UNSUPPORTED (dtype, d, block_size != 16), HIP.
 */
int kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
              const int32_t* cache_lens, const int32_t* block_table,
              int B, int H_kv, int n_new, int d, int max_len,
              int block_size, int max_blocks_per_seq, int num_blocks,
              int dtype, void* stream);

/*
 * attn_decode -- one query per head against a contiguous KV cache.
 *
 *   q, o      : [B, H_q, d]   (the single new query of each head; o in dtype,
 *               or fp32 when out_fp32 != 0: the same result before its rounding
 *               to dtype, for telling arithmetic error from storage rounding)
 *   k_cache, v_cache : [B, H_kv, max_len, d]
 *   seq_lens  : device int32 [B]; sequence b attends to keys 0 .. seq_lens[b]-1,
 *               i.e. after the append (the decode step concatenates the new
 *               token's K/V before attending, "推理速度慢怎么办？..." section 一).
 *               A length of 0 yields o = 0 and lse = -inf.  Slots at or past
 *               a sequence's length are never weighted and may hold anything,
 *               NaN and infinities included: they do not reach o or lse.
 *   lse       : [B, H_q] fp32 or NULL.
 *   workspace : device buffer of at least
 *               attn_decode_workspace_bytes(B, H_q, max_len, d) bytes; it holds the
 *               split partials (the cache length is split over workgroups and the
 *               partial results merged through their log-sum-exp).
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
int attn_decode(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* seq_lens, void* o, float* lse,
                int B, int H_q, int H_kv, int max_len, int d, float scale, int dtype,
                int out_fp32, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_paged -- attn_decode over a paged KV cache.
 *
 *   k_pool, v_pool : [num_blocks, H_kv, block_size, d], block_size == 16
 *   block_table    : device int32 [B, max_blocks_per_seq]; token p of sequence b
 *                    is row p % 16 of block block_table[b][p / 16]
 *                    ("KV Cache:推理慢的真正原因", 工程优化手段 / 1. PagedAttention).
 *   seq_lens       : device int32 [B], at most max_blocks_per_seq * 16.
 *   workspace      : at least attn_decode_workspace_bytes(B, H_q,
 *                    max_blocks_per_seq * block_size, d) bytes.
 * Other arguments as attn_decode.
 */
int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const int32_t* seq_lens,
                      void* o, float* lse,
                      int B, int H_q, int H_kv, int d, int block_size,
                      int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                      int out_fp32, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_prefill_paged -- a chunk of n_new queries per sequence against a paged
 * KV cache that already holds the chunk's own keys (chunked prefill, prefix
 * reuse).
 *
 * The KV cache exists so that the keys and values of tokens already processed
 * are never recomputed ("推理速度慢怎么办？..." section 一; "KV Cache:推理慢的真正原因",
 * 为什么需要 KV Cache); here a block of new tokens attends to that cached
 * prefix plus itself, using the same block table as decode
 * ("KV Cache:推理慢的真正原因", 工程优化手段 / 1. PagedAttention).  Call
 * kv_append with the chunk's K/V first.
 *
 *   q, o        : [B, H_q, n_new, d]; query t of sequence b is token
 *                 cache_lens[b] + t.
 *   k_pool, v_pool : [num_blocks, H_kv, block_size, d], block_size == 16.
 *   block_table : device int32 [B, max_blocks_per_seq], as for attn_decode_paged.
 *   cache_lens  : device int32 [B], tokens cached BEFORE the chunk; sequence b
 *                 has cache_lens[b] + n_new keys.
 *   causal != 0 : query t sees keys 0 .. cache_lens[b] + t; otherwise all
 *                 cache_lens[b] + n_new keys.
 *   lse         : [B, H_q, n_new] fp32 or NULL.
 * f16/bf16 at d = 64 or 128, scale > 0 (the MFMA path).  A length outside
 * [0, max_blocks_per_seq * 16 - n_new] is clamped and raises
 * ATTN_DEVERR_LEN_OVERFLOW / ATTN_DEVERR_BAD_LEN; a block id outside
 * [0, num_blocks) reads block 0 (its keys' contribution is then unspecified)
 * and raises ATTN_DEVERR_BAD_BLOCK.
 * Errors: INVALID_ARG, UNSUPPORTED (dtype, d, block_size, scale <= 0), HIP.
 */
int attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* cache_lens,
                       void* o, float* lse,
                       int B, int H_q, int H_kv, int n_new, int d, int block_size,
                       int max_blocks_per_seq, int num_blocks, int causal, float scale,
                       int dtype, void* stream);

/*
 * attn_decode_paged_noalloc -- attn_decode_paged with no workspace argument and
 * no allocation of any kind.
 *
 * For callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The workspace is a
 * 64 MiB static device array inside the library (one per GPU, held until the
 * process ends); its address is looked up once per device, on the first call
 * there.  Arguments, layouts, results and errors are those of
 * attn_decode_paged; the workspace it would need,
 * attn_decode_workspace_bytes(B, H_q, max_blocks_per_seq * 16, d), must fit in
 * the 64 MiB (e.g. B = 64, H_q = 32, d = 128 and 8,208 tokens of capacity need
 * about 37 MB), else ATTN_ERR_WORKSPACE and nothing is launched.
 * Every call on a GPU uses the same array: calls that overlap in time on one
 * GPU (different streams, or other host threads) race and must not be issued;
 * calls in one stream are ordered and safe.  Nothing in the array has to start
 * at zero: every part a call reads was written earlier in the same call.
 */
int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* o, float* lse,
                              int B, int H_q, int H_kv, int d, int block_size,
                              int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                              int out_fp32, void* stream);

/*
 * kv_append_int4 / attn_decode_paged_int4 -- the int8 cache's scheme at 4 bits.
 *
 * Same per-channel scales and rounding as kv_append_int8 with codes clamped to
 * [-7, 7] (int4 caches: "KV Cache:推理慢的真正原因", 工程优化手段, the
 * quantization item), two codes per byte, each 4-bit two's complement.  The
 * pools are bytes [num_blocks, H_kv, 16, d / 2].
 *  - K: row t of a block is token t, element 2i in the low nibble and element
 *    2i + 1 in the high nibble.
 *  - V: the 8 d bytes of a (block, KV head) are in the order the decode's
 *    P V matrix product reads them: 64 runs of d / 8 bytes; run 16 g + i holds
 *    tokens 4 g .. 4 g + 3 of channels i, i + 16, i + 32, ...; byte 4 w + j of
 *    a run holds token 4 g + (0, 2, 1, 3)[j] of channel 32 w + i (low nibble)
 *    and of channel 32 w + 16 + i (high nibble).  A byte holds one token.
 * A nibble holding -8 (never written by kv_append_int4) decodes to -8.  d must
 * be a multiple of 32 (UNSUPPORTED otherwise).  Arguments, errors and
 * workspace as for the int8 calls; attn_decode_paged_int4 takes f16 / bf16
 * queries at d = 64 or 128.
 */
int kv_append_int4(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                   const int32_t* cache_lens, const int32_t* block_table,
                   int B, int H_kv, int n_new, int d, int block_size,
                   int max_blocks_per_seq, int num_blocks, int dtype,
                   const float* k_scales, const float* v_scales, void* stream);

int attn_decode_paged_int4(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           void* o, float* lse,
                           int B, int H_q, int H_kv, int d, int block_size,
                           int max_blocks_per_seq, int num_blocks, float scale,
                           const float* k_scales, const float* v_scales, int dtype,
                           int out_fp32, void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_prefill_fp8 -- attn_prefill over FP8 E4M3 inputs.
 *
 * The FP8 attention of FlashAttention-3 ("KV缓存与Flash注意力", the 版本演进
 * table and the Flash Attention section): q [B, H_q, N, d] and k, v
 * [B, H_kv, N, d] are E4M3 codes (one byte each, the format of kv_append_fp8),
 * with one fp32 scale per tensor; the result is attention over the
 * dequantized values:
 *   O = softmax(scale * (q_scale Q)(k_scale K)^T) (v_scale V)
 * o [B, H_q, N, d] in out_dtype (F16 or BF16), or fp32 when out_fp32 != 0 (the
 * same result before its rounding to out_dtype); lse as for attn_prefill.
 * Q K^T runs on the FP8 matrix cores (exact products, fp32 sums).  V's codes
 * are widened (exactly) to out_dtype inside the kernel, on their way into
 * on-chip memory, and P V runs as in the 16-bit kernel, P rounded to out_dtype.
 * workspace, workspace_bytes: not used (no workspace is needed; NULL and 0 are
 * fine), kept so that callers written for a workspace stay valid.
 * Errors: INVALID_ARG (pointers, sizes, scales, alignment), UNSUPPORTED
 *         (out_dtype, d not 64 / 128, scale <= 0), HIP.
 */
int attn_prefill_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H_q, int H_kv, int N, int d, int causal, float scale,
                     float q_scale, float k_scale, float v_scale, int out_dtype,
                     int out_fp32, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of attn_prefill_fp8: always 0 (V is widened inside the kernel). */
size_t attn_prefill_fp8_workspace_bytes(int B, int H_kv, int N, int d);

/*
 * kv_append_fp8 / attn_decode_paged_fp8 -- a paged KV cache stored in 8 bits.
 *
 * Storing the cache in 8 bits halves the bytes decode must read ("KV Cache:
 * 推理慢的真正原因", 工程优化手段 / quantization; the fp8 KV-cache option listed
 * in "KV缓存与Flash注意力", 实际应用).  Format: OCP FP8 E4M3 (1 sign, 4 exponent
 * bits with bias 7, 3 mantissa bits, no infinities, largest finite 448), one
 * per-tensor scale for K and one for V:
 *   stored = E4M3(x * (1 / k_scale))   -- x converted exactly to fp32, the product
 *            rounded to the nearest E4M3 value, ties to even, saturating at
 *            +-448; NaN stays NaN.  1 / k_scale is computed in fp32.
 *   value  = E4M3 value * k_scale      (likewise for V with v_scale)
 * The pools are [num_blocks, H_kv, 16, d] bytes; block table and lengths as for
 * kv_append / attn_decode_paged.
 */
/* Append n_new tokens' K/V ([B, H_kv, n_new, d] in `dtype`: F32, F16 or BF16),
 * quantized, at positions cache_lens[b] ..; cache_lens is not advanced.
 * Errors: INVALID_ARG (pointers, sizes, scales <= 0 or not finite),
 *         UNSUPPORTED (dtype, d, block_size != 16), HIP. */
int kv_append_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                  const int32_t* cache_lens, const int32_t* block_table,
                  int B, int H_kv, int n_new, int d, int block_size,
                  int max_blocks_per_seq, int num_blocks, int dtype,
                  float k_scale, float v_scale, void* stream);

/* attn_decode_paged over the FP8 pools: q, o [B, H_q, d] in `dtype` (F16 or
 * BF16), d = 64 or 128, scale > 0.  Same workspace as attn_decode_paged.
 * Errors: as attn_decode_paged; UNSUPPORTED for other dtypes / d. */
int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* seq_lens,
                          void* o, float* lse,
                          int B, int H_q, int H_kv, int d, int block_size,
                          int max_blocks_per_seq, int num_blocks, float scale,
                          float k_scale, float v_scale, int dtype,
                          int out_fp32, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_append_int8 / attn_decode_paged_int8 -- a paged KV cache stored as int8
 * with one scale per (KV head, channel).
 *
 * Quantizing to int8 quarters the bytes of an fp32 cache and halves those of a
 * 16-bit one; a few key channels hold very large values, and one scale for a
 * whole tensor would magnify their error, so the scales are per channel ("KV
 * Cache:推理慢的真正原因", 工程优化手段, the quantization item; int8 and int4
 * caches are also named in "推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理",
 * section 三).  k_scales and v_scales are device fp32 [H_kv, d], > 0, fixed by
 * the caller and shared by every token (equal entries give group scales):
 *   stored = clamp(rint(x / s[h][c]), -127, 127)  -- x converted exactly to fp32,
 *            the quotient rounded to fp32, rint ties to even; NaN -> 0
 *   value  = stored * s[h][c]
 * The pools are int8 [num_blocks, H_kv, 16, d]; block table and lengths as for
 * kv_append / attn_decode_paged.
 */
/* Append n_new tokens' K/V ([B, H_kv, n_new, d] in `dtype`: F32, F16 or BF16),
 * quantized, at positions cache_lens[b] ..; cache_lens is not advanced.
 * Errors: INVALID_ARG (pointers, sizes, misaligned scale arrays),
 *         UNSUPPORTED (dtype, d, block_size != 16), HIP. */
int kv_append_int8(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                   const int32_t* cache_lens, const int32_t* block_table,
                   int B, int H_kv, int n_new, int d, int block_size,
                   int max_blocks_per_seq, int num_blocks, int dtype,
                   const float* k_scales, const float* v_scales, void* stream);

/* attn_decode_paged over the int8 pools: q, o [B, H_q, d] in `dtype` (F16 or
 * BF16), d = 64 or 128, scale > 0.  Same workspace as attn_decode_paged.
 * The scores are computed on the int8 matrix cores: the query times the key
 * scales, rescaled per head so that its largest element is 2^22 - 1, is
 * rounded to an integer held as three int8 digits (23 bits with the sign),
 * each multiplied with the codes in exact int32 sums.
 * Errors: as attn_decode_paged; INVALID_ARG for null or misaligned scale arrays;
 *         UNSUPPORTED for other dtypes / d. */
int attn_decode_paged_int8(const void* q, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, const int32_t* seq_lens,
                           void* o, float* lse,
                           int B, int H_q, int H_kv, int d, int block_size,
                           int max_blocks_per_seq, int num_blocks, float scale,
                           const float* k_scales, const float* v_scales, int dtype,
                           int out_fp32, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_copy_blocks -- copy whole physical blocks of the K and V pools.
 *
 * The device half of copy on write: when a sequence forked from a shared
 * prompt (attn_block_pool_fork) first writes into the prompt's partly filled
 * last block, attn_block_pool_reserve hands it a fresh block and reports the
 * (old, new) pair; this call copies the old block's K and V into the new one
 * ("KV缓存与Flash注意力", 练习: one pass over the prompt fills the cache, and
 * every completion branches from it).
 *
 *   pairs : device int32 [n_pairs][2] = (src, dst); n_pairs in [0, 65535].
 *           The dst blocks must be distinct and must not be a src of the same
 *           call (fresh blocks from the pool always are).
 *   pools : [num_blocks, H_kv, 16, d] elements of elem_bytes bytes (1 for the
 *           FP8 pools, 2 for f16/bf16, 4 for f32); every KV head of a block is
 *           copied.
 * An id outside [0, num_blocks) skips its pair and raises ATTN_DEVERR_BAD_BLOCK.
 * Errors: INVALID_ARG, UNSUPPORTED (d, elem_bytes, block_size != 16), HIP.
 */
int kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int n_pairs, int H_kv, int d,
                   int block_size, int num_blocks, int elem_bytes, void* stream);

/* Workspace bytes every decode call (attn_decode, attn_decode_paged and its
 * 8- and 4-bit forms) needs for a cache capacity of max_seq_len tokens per
 * sequence.  Layout, each region 256-byte aligned: split partial outputs fp32
 * [B][H_q][S][d], their lse fp32 [B][H_q][S], then piece counts int32
 * [B][H_q]; S = ceil(max_seq_len / 256) + 1.  0 on invalid sizes. */
size_t attn_decode_workspace_bytes(int B, int H_q, int max_seq_len, int d);

/* Message describing the last error returned on the calling thread ("" if none). */
const char* attn_last_error(void);

/* Library version string. */
const char* attn_version(void);

/* Reads and clears the device error flags (enum attn_device_error) of the current
 * device after synchronising `stream`.  Returns the flags, or -1 if HIP failed. */
int attn_device_error_flags(void* stream);

/*
 * Block pool -- host bookkeeping of the paged pools' physical blocks.
 *
 * The cache is cut into 16-token blocks, a block table maps each sequence's
 * logical blocks to physical ones, and a finished sequence's blocks are reused
 * at once ("KV Cache:推理慢的真正原因", 工程优化手段 / 1).  Blocks come from a
 * free list and go back to it when a sequence finishes ("KV缓存与Flash注意力",
 * 练习).  Forked sequences share blocks; each block counts its holders and
 * returns to the free list when the count reaches zero.
 *
 * Free-list order: a stack.  Initially block 0 is on top, then 1, 2, ...; a
 * freed block goes on top, so the most recently freed block is reused first.
 *
 * All pointers here are HOST pointers; a row is one sequence's block-table row
 * (int32, max_blocks entries, -1 = unassigned), the layout attn_decode_paged
 * reads once copied to the device.  Row entry j holds tokens 16j .. 16j+15.
 * Every call checks all its arguments before it changes anything, so a failed
 * call leaves the pool and the rows as they were.  A pool is not thread-safe:
 * calls on one pool must not overlap.
 */
typedef struct attn_block_pool attn_block_pool;

/* A pool of num_blocks free blocks; NULL (and attn_last_error) if num_blocks < 1. */
attn_block_pool* attn_block_pool_create(int num_blocks);

/* Frees the pool's host memory; NULL is a no-op. */
void attn_block_pool_destroy(attn_block_pool* pool);

/* Number of free blocks; -1 for a NULL pool. */
int attn_block_pool_free_blocks(const attn_block_pool* pool);

/* Number of sequences holding `block`; -1 for a NULL pool or an id out of range. */
int attn_block_pool_holders(const attn_block_pool* pool, int block);

/* Grow a sequence holding cur_len tokens so its row covers new_len tokens:
 * entries ceil(cur_len/16) .. ceil(new_len/16)-1 receive blocks from the free
 * list.  Copy on write: if new_len > cur_len, cur_len is not a multiple of 16
 * and the block holding token cur_len is shared, the row gets a fresh block in
 * its place and copy_pair[0..1] = (old, new) (the caller copies the contents
 * with kv_copy_blocks before appending); otherwise copy_pair = (-1, -1).
 * Errors: INVALID_ARG (null pointers, 0 <= cur_len <= new_len <= 16*max_blocks
 *         violated, or the row's first ceil(cur_len/16) entries not held blocks),
 *         NO_BLOCKS (too few free blocks: nothing changes). */
int attn_block_pool_reserve(attn_block_pool* pool, int32_t* row, int max_blocks, int cur_len, int new_len,
                            int32_t* copy_pair);

/* attn_block_pool_reserve for sequences b = 0 .. B-1 in order, rows of
 * `table` [B][max_blocks].  Copy pairs are written densely to copy_pairs
 * [B][2] and counted in *n_copies.  *n_done = the number of sequences reserved;
 * on an error the sequences from *n_done on are unchanged (the caller can free
 * blocks, e.g. by preempting a sequence, and continue from there). */
int attn_block_pool_reserve_batch(attn_block_pool* pool, int32_t* table, int B, int max_blocks,
                                  const int32_t* cur_lens, const int32_t* new_lens, int32_t* copy_pairs,
                                  int* n_copies, int* n_done);

/* Drop a sequence of len tokens: each of its first ceil(len/16) blocks loses a
 * holder (in row order; a block left with none goes on top of the free list)
 * and the entries become -1.  Errors: INVALID_ARG. */
int attn_block_pool_release(attn_block_pool* pool, int32_t* row, int max_blocks, int len);

/* Fork: dst's first ceil(len/16) entries become src's blocks, each gaining a
 * holder.  dst should hold no blocks in those entries (they are overwritten).
 * Errors: INVALID_ARG. */
int attn_block_pool_fork(attn_block_pool* pool, const int32_t* src, int32_t* dst, int max_blocks, int len);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
