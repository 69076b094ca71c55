// Plain tiled prefill on the vector ALUs: any dtype, d in {16, 32, 64, 128, 256}.
//
// This is the exactness path (fp32 inputs, small or unusual head dims).  It is
// the tile loop of "KV缓存与Flash注意力" (Flash Attention — 分块技巧): a workgroup
// owns a block of query rows, streams key/value tiles through LDS, and keeps a
// running maximum m, normaliser l and unnormalised output per row, so the
// final division is exact (same page, 数值技巧; 步骤2 gives the per-tile update).
//
// Scores are kept in the base-2 domain: t = (q.k) * scale * log2(e), so that
// softmax weights are exp2(t - m) and the natural-log lse is (m + log2 l) ln 2.
//
// Layout: each query row is served by TPR = d/16 adjacent lanes, each owning
// 16 of the d components of q and of the output accumulator; dot products are
// finished with lane exchanges.
#pragma once
#include "common.h"

namespace attn {

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, H_q, H_kv, N;
  float scale_log2;  // scale * log2(e)
  int out_fp32;
  float v_scale = 1.f;  // FP8 inputs: V's scale, applied to O in the epilogue
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) prefill_plain_kernel(PrefillArgs a) {
  constexpr int DPT = 16;                // components per lane
  constexpr int TPR = D / DPT;           // lanes per query row
  constexpr int ROWS = 256 / TPR;        // query rows per workgroup
  constexpr int KT = 32;                 // keys per tile
  __shared__ float Ks[KT][D];
  __shared__ float Vs[KT][D];

  const int tid = threadIdx.x;
  const int r = tid / TPR;
  const int part = tid % TPR;
  const int n_qt = (a.N + ROWS - 1) / ROWS;
  const int qt = CAUSAL ? (n_qt - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int g = h / (a.H_q / a.H_kv);
  const int q0 = qt * ROWS;
  const int qi = q0 + r;
  const bool row_ok = qi < a.N;

  const size_t qbase = (((size_t)b * a.H_q + h) * a.N + (row_ok ? qi : 0)) * D + part * DPT;
  const size_t kvbase = ((size_t)b * a.H_kv + g) * a.N * D;

  float qv[DPT], acc[DPT];
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    qv[e] = row_ok ? load_elem<T>(a.q, qbase + e) : 0.f;
    acc[e] = 0.f;
  }
  float m = kNegInf, l = 0.f;

  const int key_end = CAUSAL ? min(a.N, q0 + ROWS) : a.N;
  for (int k0 = 0; k0 < key_end; k0 += KT) {
    for (int i = tid; i < KT * D; i += 256) {
      const int j = i / D, c = i % D;
      const bool ok = k0 + j < a.N;
      Ks[j][c] = ok ? load_elem<T>(a.k, kvbase + (size_t)(k0 + j) * D + c) : 0.f;
      Vs[j][c] = ok ? load_elem<T>(a.v, kvbase + (size_t)(k0 + j) * D + c) : 0.f;
    }
    __syncthreads();
    float s[KT];
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < KT; ++j) {
      float part_sum = 0.f;
#pragma unroll
      for (int e = 0; e < DPT; ++e) part_sum = fmaf(qv[e], Ks[j][part * DPT + e], part_sum);
#pragma unroll
      for (int off = 1; off < TPR; off <<= 1) part_sum += xor_shfl(part_sum, off);
      const int kj = k0 + j;
      const bool vis = kj < a.N && (!CAUSAL || kj <= qi);
      s[j] = vis ? part_sum * a.scale_log2 : kNegInf;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new != kNegInf) {
      const float alpha = fast_exp2(m - m_new);
      float psum = 0.f;
      float pv[DPT];
#pragma unroll
      for (int e = 0; e < DPT; ++e) pv[e] = 0.f;
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        const float p = fast_exp2(s[j] - m_new);
        psum += p;
#pragma unroll
        for (int e = 0; e < DPT; ++e) pv[e] = fmaf(p, Vs[j][part * DPT + e], pv[e]);
      }
      l = fmaf(alpha, l, psum);
#pragma unroll
      for (int e = 0; e < DPT; ++e) acc[e] = fmaf(alpha, acc[e], pv[e]);
      m = m_new;
    }
    __syncthreads();
  }

  if (!row_ok) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  const size_t obase = (((size_t)b * a.H_q + h) * a.N + qi) * D + part * DPT;
#pragma unroll
  for (int e = 0; e < DPT; ++e) {
    if (a.out_fp32)
      store_elem<F32>(a.o, obase + e, acc[e] * inv);
    else
      store_elem<T>(a.o, obase + e, acc[e] * inv);
  }
  if (a.lse != nullptr && part == 0) {
    a.lse[((size_t)b * a.H_q + h) * a.N + qi] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
  }
}

}  // namespace attn
