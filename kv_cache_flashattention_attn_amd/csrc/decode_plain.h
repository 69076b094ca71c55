// Plain split decode on the vector ALUs (any dtype, d <= 256), and the split merge.
//
// A decode step attends one new query per head to every cached key
// ("推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理", section 一).  The
// cache length is cut into chunks of kPlainChunk tokens, one workgroup per
// (chunk, query head, sequence).  Each workgroup returns a normalised partial
// output and its log-sum-exp; decode_merge_kernel combines the chunks with
// the same running-(max, sum) identity the tiles use ("KV缓存与Flash注意力",
// 数值技巧): weights exp(lse_c - max_c lse_c).
//
// Workspace layout (fp32): partial outputs [B][H_q][S_max][d] followed by the
// partial lse [B][H_q][S_max].
#pragma once
#include "common.h"

namespace attn {

constexpr int kPlainChunk = 256;

struct DecodeArgs {
  const void* q;        // [B, H_q, d]
  const void* k;        // contiguous [B, H_kv, max_len, d] or pool [NB, H_kv, 16, d]
  const void* v;
  const int32_t* table; // paged only: [B, max_blocks_per_seq]
  const int32_t* seq_lens;
  float* part_o;        // [B, H_q, S_max, d]
  float* part_lse;      // [B, H_q, S_max]
  int B, H_q, H_kv;
  int capacity;         // max_len, or max_blocks_per_seq * 16
  int max_blocks_per_seq;
  int num_blocks;
  int s_max;            // splits per (b, h_q) the workspace holds
  float scale_log2;
  int out_fp32;         // the output o is fp32 instead of T
};

// Length of sequence b, clamped to [0, capacity]; raises a flag when clamped.
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b, bool report) {
  int len = a.seq_lens[b];
  if (len < 0) {
    if (report) raise_device_error(4);
    len = 0;
  }
  if (len > a.capacity) {
    if (report) raise_device_error(1);
    len = a.capacity;
  }
  return len;
}

// Row index (in units of d elements) of token t of sequence b, KV head g.
// Returns -1 for an invalid block id (after raising the flag once per call site).
template <bool PAGED>
__device__ __forceinline__ int64_t token_row(const DecodeArgs& a, int b, int g, int t) {
  if (!PAGED) return ((int64_t)b * a.H_kv + g) * a.capacity + t;
  const int blk = a.table[(int64_t)b * a.max_blocks_per_seq + (t >> 4)];
  if (blk < 0 || blk >= a.num_blocks) return -1;
  return ((int64_t)blk * a.H_kv + g) * 16 + (t & 15);
}

template <typename T, int D, bool PAGED>
__global__ void __launch_bounds__(256) decode_plain_kernel(DecodeArgs a) {
  __shared__ float qs[D];
  __shared__ float sc[kPlainChunk];
  __shared__ int64_t rows[kPlainChunk];
  __shared__ float red[8];

  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int len = clamp_len(a, b, s == 0 && h == 0 && tid == 0);
  const int start = s * kPlainChunk;
  if (start >= len) return;
  const int n = min(kPlainChunk, len - start);
  const int g = h / (a.H_q / a.H_kv);

  for (int c = tid; c < D; c += 256) qs[c] = load_elem<T>(a.q, ((size_t)b * a.H_q + h) * D + c);
  for (int t = tid; t < n; t += 256) {
    const int64_t row = token_row<PAGED>(a, b, g, start + t);
    if (row < 0) raise_device_error(2);
    rows[t] = row;
  }
  __syncthreads();

  // scores: one wave per token, lanes across d
  for (int t = wave; t < n; t += 4) {
    const int64_t row = rows[t];
    float part = 0.f;
    if (row >= 0)
      for (int c = lane; c < D; c += 64) part = fmaf(qs[c], load_elem<T>(a.k, row * D + c), part);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += xor_shfl(part, off);
    if (lane == 0) sc[t] = row >= 0 ? part * a.scale_log2 : kNegInf;
  }
  __syncthreads();

  // maximum over the chunk
  float mx = kNegInf;
  for (int t = tid; t < n; t += 256) mx = fmaxf(mx, sc[t]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, xor_shfl(mx, off));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float base = mx == kNegInf ? 0.f : mx;
  __syncthreads();

  // weights and their sum
  float sum = 0.f;
  for (int t = tid; t < n; t += 256) {
    const float p = fast_exp2(sc[t] - base);
    sc[t] = p;
    sum += p;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += xor_shfl(sum, off);
  if (lane == 0) red[4 + wave] = sum;
  __syncthreads();
  sum = red[4] + red[5] + red[6] + red[7];

  // weighted sum of value rows: one lane per output component
  const size_t pidx = ((size_t)b * a.H_q + h) * a.s_max + s;
  for (int c = tid; c < D; c += 256) {
    float o = 0.f;
    for (int t = 0; t < n; ++t) {
      const int64_t row = rows[t];
      if (row >= 0) o = fmaf(sc[t], load_elem<T>(a.v, row * D + c), o);
    }
    a.part_o[pidx * D + c] = sum > 0.f ? o / sum : 0.f;
  }
  if (tid == 0) a.part_lse[pidx] = sum > 0.f ? (mx + __log2f(sum)) * kLn2 : kNegInf;
}

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* seq_lens;
  const int32_t* piece_cnt;  // [B][H_q] pieces per segment, or nullptr: ceil(len / chunk) splits
  void* o;          // [B, H_q, d]
  float* lse;       // [B, H_q] or nullptr
  int H_q;
  int capacity;
  int s_max;
  int chunk;        // tokens per split (piece_cnt == nullptr)
  int G, n_hg;      // query heads per KV head, groups of 16 of them (piece_cnt != nullptr)
  int out_fp32;     // o is fp32 (the result before its rounding to T)
};

// Combine the split partials of one (sequence, query head): one wave, lanes
// across d (PER consecutive channels each).  A chunk of up to 64 splits is
// weighted at once (lane s holds split s; the weights are broadcast with
// v_readlane), and the partial rows of BATCH splits are loaded before any is
// used.  The merge is latency-bound, so the loads are ordered for the fewest
// round trips: the length and the piece count together, then a chunk's lse
// values together with the rows of its first batch.  A chunk whose largest lse
// exceeds the running maximum rescales what was summed before it (the tiles'
// identity again), so the common case of at most 64 splits reads every lse once.
template <typename T, int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(MergeArgs a) {
  constexpr int PER = D >= 64 ? D / 64 : 1;  // consecutive output channels per lane
  constexpr int BATCH = 16;                  // splits whose rows are in flight together
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x;
  const int gh = a.piece_cnt == nullptr ? 0 : (h / a.G) * a.n_hg + (h % a.G) / 16;  // segment of this head
  int len = a.seq_lens[b];
  const int pc = a.piece_cnt == nullptr ? 0 : a.piece_cnt[(size_t)b * a.H_q + gh];
  len = len < 0 ? 0 : (len > a.capacity ? a.capacity : len);
  int ns;
  if (a.piece_cnt == nullptr)
    ns = (len + a.chunk - 1) / a.chunk;
  else
    ns = len == 0 ? 0 : (pc < 0 ? 0 : (pc > a.s_max ? a.s_max : pc));
  const size_t base = ((size_t)b * a.H_q + h) * a.s_max;
  const int c0 = lane * PER;  // first channel of this lane
  const bool has_c = c0 < D;
  float M = kNegInf, wsum = 0.f, acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 64) {
    const int cnt = min(64, ns - s0);
    const float lse_l = lane < cnt ? a.part_lse[base + s0 + lane] : kNegInf;
    const float* rows = a.part_o + (base + s0) * D + c0;
    float w_l = 0.f;
    for (int s1 = 0; s1 < cnt; s1 += BATCH) {
      float v[BATCH][PER];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const bool in = s1 + u < cnt && has_c;
        const float* src = rows + (size_t)(in ? s1 + u : 0) * D;
        if constexpr (PER == 4) {
          const float4 x = in ? *reinterpret_cast<const float4*>(src) : float4{0.f, 0.f, 0.f, 0.f};
          v[u][0] = x.x, v[u][1] = x.y, v[u][2] = x.z, v[u][3] = x.w;
        } else if constexpr (PER == 2) {
          const float2 x = in ? *reinterpret_cast<const float2*>(src) : float2{0.f, 0.f};
          v[u][0] = x.x, v[u][1] = x.y;
        } else {
          v[u][0] = in ? src[0] : 0.f;
        }
      }
      if (s1 == 0) {
        // this chunk's weights, while its first rows are in flight
        float cm = lse_l;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, xor_shfl(cm, off));
        if (cm > M) {
          const float alpha = M == kNegInf ? 0.f : fast_exp2((M - cm) * kLog2e);
          wsum *= alpha;
#pragma unroll
          for (int j = 0; j < PER; ++j) acc[j] *= alpha;
          M = cm;
        }
        w_l = lane < cnt && M != kNegInf ? fast_exp2((lse_l - M) * kLog2e) : 0.f;
        float ws = w_l;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) ws += xor_shfl(ws, off);
        wsum += ws;
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        // weight of split s0 + s1 + u (lanes at or past cnt hold 0)
        const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_l), (s1 + u) & 63));
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] = fmaf(wu, v[u][j], acc[j]);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  if (has_c) {
    const size_t i = ((size_t)b * a.H_q + h) * D + c0;
    if (a.out_fp32) {
#pragma unroll
      for (int j = 0; j < PER; ++j) static_cast<float*>(a.o)[i + j] = acc[j] * inv;
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) store_elem<T>(a.o, i + j, acc[j] * inv);
    }
  }
  if (a.lse != nullptr && lane == 0)
    a.lse[(size_t)b * a.H_q + h] = wsum > 0.f ? M + __logf(wsum) : kNegInf;
}

}  // namespace attn
