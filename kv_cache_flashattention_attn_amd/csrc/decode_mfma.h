// MFMA split decode for f16 / bf16 at d in {64, 128}, contiguous or paged cache.
//
// A decode step is one new query per head against every cached key
// ("推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理", section 一); with a
// cache the cost is reading K and V from memory ("KV Cache:推理慢的真正原因",
// 缓存的是什么: the bottleneck moves to bandwidth).  Grouped-query attention lets
// the query heads of a group share one K/V head (same page, 工程优化手段 / 2), so
// a workgroup reads each K/V row ONCE for all G = H_q / H_kv query heads.
//
// Work split: one workgroup per (chunk of kChunk tokens, KV head [x head group
// of 16], sequence); its 4 waves each take a contiguous quarter of the chunk in
// steps of 32 tokens.  Per step a wave
//   * loads 32 K rows straight into MFMA A-operand registers (lane -> token,
//     16 contiguous bytes of the row per k-step),
//   * loads 32 V rows with 16-byte loads and writes them transposed into a
//     wave-private LDS area, V^T[d][token],
//   * computes S^T = K Q^T with v_mfma_f32_16x16x32 (16 query heads as columns,
//     zero-padded beyond G), updates the running (max, sum) of each head,
//   * accumulates O^T += V^T P^T, with P^T taken straight from the S^T
//     registers (rounded to 16 bits).
// The four waves' states are merged in LDS and the chunk's normalised partial
// output and lse go to the workspace; decode_merge_kernel combines chunks.
//
// Paged caches ("KV Cache:推理慢的真正原因", 工程优化手段 / 1. PagedAttention): each
// 32-token step covers exactly two 16-token blocks, whose ids are read from the
// block table once per step; one (block, KV head) is 16 contiguous rows.
#pragma once
#include "common.h"
#include "decode_plain.h"

namespace attn {

constexpr int kMfmaChunk = 512;

template <typename T>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <typename T, int D, bool PAGED>
__global__ void __launch_bounds__(256) decode_mfma_kernel(DecodeArgs a, int n_hg) {
  constexpr int WT = kMfmaChunk / 4;   // tokens per wave
  constexpr int KS = D / 32;           // 32-deep k-steps of Q K^T
  constexpr int DB = D / 16;           // 16-wide blocks of d
  constexpr int VSTR = 32 + 4;         // V^T row stride (elements): 72 B
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int PPP = 64 / CPR;        // V token pairs per pass (per wave)
  constexpr int VPASS = 16 / PPP;
  constexpr int WAVE_LDS = D * VSTR;   // uint16 elements per wave
  static_assert(4 * WAVE_LDS * 2 >= 4 * 16 * D * 4, "LDS reuse for the merge");

  __shared__ __attribute__((aligned(16))) uint16_t lds[4 * WAVE_LDS];
  __shared__ float mrg_m[4][16], mrg_l[4][16];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int col = l & 15, grp = l >> 4;   // MFMA column (head / token row) and k-group
  const int s = blockIdx.x;
  const int g = blockIdx.y / n_hg, hg = blockIdx.y % n_hg;
  const int b = blockIdx.z;
  const int G = a.H_q / a.H_kv;

  const int len = clamp_len(a, b, s == 0 && blockIdx.y == 0 && tid == 0);
  const int start = s * kMfmaChunk;
  if (start >= len) return;
  const int cend = min(start + kMfmaChunk, len);
  const int wbeg = start + w * WT;
  const int wend = min(wbeg + WT, cend);

  const uint16_t* kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v);
  const int gi = 16 * hg + col;          // head within the group served by this column
  const bool head_ok = gi < G;
  const int hq = g * G + gi;

  float c = a.scale_log2;                // > 0 on this path
  u32x4 qf[KS];
  {
    const uint16_t* src = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.H_q + (head_ok ? hq : 0)) * D +
                          8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = head_ok ? *reinterpret_cast<const u32x4*>(src + 32 * ks) : u32x4{0, 0, 0, 0};
  }

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;
  uint16_t* vt = lds + w * WAVE_LDS;
  const int64_t contig_base = ((int64_t)b * a.H_kv + g) * a.capacity;
  const int vc = l % CPR, vpair = l / CPR;

  for (int t0 = wbeg; t0 < wend; t0 += 32) {
    // physical row of token t0 + r (r in [0, 32)); -1 when invalid
    int64_t row0, row1;  // rows of the first token of each 16-token half
    bool ok0 = true, ok1 = true;
    if (PAGED) {
      const int64_t tb = (int64_t)b * a.max_blocks_per_seq + (t0 >> 4);
      const int blk0 = a.table[tb];
      const int blk1 = (t0 + 16 < wend) ? a.table[tb + 1] : 0;
      ok0 = blk0 >= 0 && blk0 < a.num_blocks;
      ok1 = blk1 >= 0 && blk1 < a.num_blocks;
      if ((!ok0 || !ok1) && l == 0) raise_device_error(2);
      row0 = ((int64_t)(ok0 ? blk0 : 0) * a.H_kv + g) * 16;
      row1 = ((int64_t)(ok1 ? blk1 : 0) * a.H_kv + g) * 16;
    } else {
      row0 = contig_base + t0;
      row1 = contig_base + t0 + 16;
    }
    auto token_ok = [&](int r) { return t0 + r < wend && (r < 16 ? ok0 : ok1); };
    auto row_of = [&](int r) { return (r < 16 ? row0 + r : row1 + (r - 16)); };

    // K fragments: lane -> token row (col), 16 bytes at d = 32 ks + 8 grp
    u32x4 kf[2][KS];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 16 * rb + col;
      const bool ok = token_ok(r);
      const uint16_t* src = kp + row_of(r) * D + 8 * grp;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[rb][ks] = ok ? *reinterpret_cast<const u32x4*>(src + 32 * ks) : u32x4{0, 0, 0, 0};
    }
    // V rows, two tokens per item, for the transposed LDS copy
    u32x4 vr[VPASS][2];
#pragma unroll
    for (int i = 0; i < VPASS; ++i) {
      const int r = 2 * (vpair + PPP * i);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        vr[i][u] = token_ok(r + u) ? *reinterpret_cast<const u32x4*>(vp + row_of(r + u) * D + 8 * vc)
                                   : u32x4{0, 0, 0, 0};
    }

    // S^T = K Q^T
    f32x4 sacc[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) sacc[rb] = mfma16<T>(kf[rb][ks], qf[ks], sacc[rb]);
    }

    // V^T into this wave's LDS area
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < VPASS; ++i) {
      const int pair = vpair + PPP * i;
      const u32x4 x0 = vr[i][0], x1 = vr[i][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = x0[e >> 1], hi = x1[e >> 1];
        const uint32_t word = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        *reinterpret_cast<uint32_t*>(&vt[(8 * vc + e) * VSTR + 2 * pair]) = word;
      }
    }

    // online softmax: lane holds head `col`, tokens 16 rb + 4 grp + i
    float sv[8];
    float tmax = kNegInf;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = token_ok(16 * rb + 4 * grp + i) ? sacc[rb][i] : kNegInf;
        sv[4 * rb + i] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, xor_shfl(tmax, 16));
    tmax = fmaxf(tmax, xor_shfl(tmax, 32));
    const float m_new = fmaxf(m, tmax * c);
    const float base = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m - base);
    m = m_new;
    float p[8], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(sv[e], c, -base));
      psum += p[e];
    }
    lsum = fmaf(alpha, lsum, psum);
    const u32x4 pf = u32x4{pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                           pack2<T>(p[6], p[7])};
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] *= alpha;

    // O^T += V^T P^T
    wave_lds_sync();
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint16_t* vrow = &vt[(16 * db + col) * VSTR + 4 * grp];
      const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
      const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
      oacc[db] = mfma16<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf, oacc[db]);
    }
  }

  // merge the four waves of this workgroup
  float l_tot = lsum + xor_shfl(lsum, 16);
  l_tot += xor_shfl(l_tot, 32);
  __syncthreads();
  float* mo = reinterpret_cast<float*>(lds);  // [4][16][D]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) mo[(w * 16 + col) * D + 16 * db + 4 * grp + i] = oacc[db][i];
  if (grp == 0) {
    mrg_m[w][col] = m;
    mrg_l[w][col] = l_tot;
  }
  __syncthreads();
  const int head = tid >> 4, part = tid & 15;
  if (16 * hg + head < G) {
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mrg_m[ww][head]);
    const float Mb = M == kNegInf ? 0.f : M;
    float sc[4], L = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      sc[ww] = fast_exp2(mrg_m[ww][head] - Mb);
      L = fmaf(sc[ww], mrg_l[ww][head], L);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const int hq_out = g * G + 16 * hg + head;
    const size_t pidx = ((size_t)b * a.H_q + hq_out) * a.s_max + s;
    for (int cc = part; cc < D; cc += 16) {
      float o = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) o = fmaf(sc[ww], mo[(ww * 16 + head) * D + cc], o);
      a.part_o[pidx * D + cc] = o * inv;
    }
    if (part == 0) a.part_lse[pidx] = L > 0.f ? (M + __log2f(L)) * kLn2 : kNegInf;
  }
}

}  // namespace attn
