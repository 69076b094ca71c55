// MFMA prefill for f16 / bf16 at d in {64, 128} (gfx950 matrix cores).
//
// The method is the tile loop of "KV缓存与Flash注意力" (Flash Attention — 分块技巧)
// and "推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理" (section 二): a
// workgroup keeps one block of BM = 128 query rows on chip, streams key/value
// tiles of BN = 64 tokens through LDS, and carries a running maximum and sum
// per row so only the final output (and lse) is written to memory.  Causal runs
// stop at the diagonal and start with the longest query tiles (the causal
// ordering listed for FlashAttention-2 in the 版本演进 table of the same page).
//
// Mapping onto CDNA4:
//  * 4 waves, 32 query rows each.  A wave computes S^T = K Q^T for its rows
//    with v_mfma_f32_32x32x16 (A = K rows from LDS, B = Q^T kept in registers),
//    so each lane ends up holding 32 scores of ONE query row: row max and row
//    sum are mostly lane-local (one exchange with lane l^32 for the max; the
//    sum is exchanged once, at the end).
//  * The S^T accumulator, rounded to 16 bits, is already laid out as the B
//    operand of O^T = V^T P^T (same lane -> query, k-slot -> token mapping), so
//    P never leaves registers.  V is written to LDS transposed (V^T[d][token])
//    once per tile so the A operand is two 8-byte LDS reads.
//  * K/V tiles are double-buffered in LDS; the next tile's global loads are in
//    flight while the current tile is computed.  One barrier per tile.
//  * Scores are in the base-2 domain: t = s * scale * log2(e), weights
//    exp2(t - m) (v_exp_f32), lse = (m + log2 l) ln 2.
//  * Workgroup order: consecutive workgroup ids walk the (batch, head) pairs, so
//    all query tiles of one head land on the same XCD (ids are dealt round-robin
//    to the 8 XCDs) and share its L2; for causal runs the longest tiles go first.
#pragma once
#include "common.h"
#include "prefill_plain.h"

namespace attn {

template <typename T>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c);
template <>
__device__ __forceinline__ f32x16 mfma32<BF16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x16 mfma32<F16>(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(256) prefill_mfma_kernel(PrefillArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;          // 16-deep k-steps of Q K^T
  constexpr int DB = D / 32;          // 32-wide blocks of the output's d
  constexpr int KSTR = D + 8;         // K tile row stride (elements); +16 B staggers banks
  constexpr int VSTR = BN + 4;        // V^T row stride (elements): 136 B, 8-byte aligned
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int KROWS = 256 / CPR;    // K rows loaded per pass
  constexpr int KPASS = BN / KROWS;
  constexpr int VPAIRS = 256 / CPR;   // V token pairs per pass
  constexpr int VPASS = (BN / 2) / VPAIRS;
  static_assert(KPASS >= 1 && VPASS >= 1, "tile shape");

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2][D * VSTR];

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 31, hh = l >> 5;
  const int BH = a.B * a.H_q;
  const int n_qt = (a.N + BM - 1) / BM;
  const int bid = blockIdx.x;
  const int bh = bid % BH;
  const int qt = CAUSAL ? (n_qt - 1 - bid / BH) : (bid / BH);
  const int b = bh / a.H_q, h = bh % a.H_q;
  const int g = h / (a.H_q / a.H_kv);
  const int q0 = qt * BM;
  const int qw0 = q0 + 32 * w;        // first query row of this wave
  const int qi = qw0 + lr;            // this lane's query row
  const float c = a.scale_log2;       // > 0 on this path

  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v);
  const size_t kv_base = ((size_t)b * a.H_kv + g) * (size_t)a.N * D;

  // Q^T fragments (B operand): lane -> query qi, k-slots -> d = 16 ks + 8 hh + j
  u32x4 qf[KS];
  {
    const bool ok = qi < a.N;
    const uint16_t* src = qp + (((size_t)b * a.H_q + h) * a.N + (ok ? qi : 0)) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = ok ? *reinterpret_cast<const u32x4*>(src + 16 * ks) : u32x4{0, 0, 0, 0};
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = kNegInf, lsum = 0.f;

  const int key_end = CAUSAL ? min(a.N, q0 + BM) : a.N;
  const int n_kt = (key_end + BN - 1) / BN;

  // register staging for one K tile and one V tile
  u32x4 kreg[KPASS];
  u32x4 vreg[VPASS][2];
  const int kc = tid % CPR, kr = tid / CPR;

  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i) {
      const int key = k0 + kr + KROWS * i;
      kreg[i] = key < a.N ? *reinterpret_cast<const u32x4*>(kp + kv_base + (size_t)key * D + 8 * kc)
                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < VPASS; ++i) {
      const int key = k0 + 2 * (kr + VPAIRS * i);
      vreg[i][0] = key < a.N ? *reinterpret_cast<const u32x4*>(vp + kv_base + (size_t)key * D + 8 * kc)
                             : u32x4{0, 0, 0, 0};
      vreg[i][1] = key + 1 < a.N
                       ? *reinterpret_cast<const u32x4*>(vp + kv_base + (size_t)(key + 1) * D + 8 * kc)
                       : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KPASS; ++i)
      *reinterpret_cast<u32x4*>(&Ks[buf][(kr + KROWS * i) * KSTR + 8 * kc]) = kreg[i];
#pragma unroll
    for (int i = 0; i < VPASS; ++i) {
      const int pair = kr + VPAIRS * i;
      const u32x4 x0 = vreg[i][0], x1 = vreg[i][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t lo = x0[e >> 1], hi = x1[e >> 1];
        const uint32_t word = (e & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        *reinterpret_cast<uint32_t*>(&Vt[buf][(8 * kc + e) * VSTR + 2 * pair]) = word;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < n_kt; ++j) {
    const int buf = j & 1;
    const int k0 = j * BN;
    if (j + 1 < n_kt) load_tile(k0 + BN);

    const bool active = !CAUSAL || k0 <= qw0 + 31;
    if (active) {
      // S^T = K Q^T : two 32-token row blocks
      f32x16 sacc[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        sacc[rb] = f32x16{};
        const uint16_t* krow = &Ks[buf][(32 * rb + lr) * KSTR + 8 * hh];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(krow + 16 * ks);
          sacc[rb] = mfma32<T>(kf, qf[ks], sacc[rb]);
        }
      }
      // masking (diagonal tiles and the ragged end only)
      const bool need_mask = (k0 + BN > a.N) || (CAUSAL && k0 + BN - 1 > qw0);
      if (need_mask) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * rb + 8 * (i >> 2) + 4 * hh + (i & 3);
            const bool vis = key < a.N && (!CAUSAL || key <= qi);
            if (!vis) sacc[rb][i] = kNegInf;
          }
      }
      // online softmax update for this lane's query row
      float tmax = kNegInf;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[rb][i]);
      tmax = fmaxf(tmax, xor_shfl(tmax, 32));
      const float m_new = fmaxf(m, tmax * c);
      const float base = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m - base);
      m = m_new;
      float psum = 0.f;
      u32x4 pf[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sacc[kk >> 1][8 * (kk & 1) + e], c, -base));
          psum += p[e];
        }
        pf[kk] = u32x4{pack2<T>(p[0], p[1]), pack2<T>(p[2], p[3]), pack2<T>(p[4], p[5]),
                       pack2<T>(p[6], p[7])};
      }
      lsum = fmaf(alpha, lsum, psum);
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint16_t* vrow = &Vt[buf][(32 * db + lr) * VSTR + 4 * hh];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow + 16 * kk);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16 * kk + 8);
          oacc[db] = mfma32<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kk], oacc[db]);
        }
      }
    }
    if (j + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // epilogue: O = O_acc / l ; lse = (m + log2 l) ln 2
  const float l_tot = lsum + xor_shfl(lsum, 32);
  if (qi >= a.N) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const size_t orow = (((size_t)b * a.H_q + h) * a.N + qi) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * db + 8 * g4 + 4 * hh;
      const float o0 = oacc[db][4 * g4 + 0] * inv, o1 = oacc[db][4 * g4 + 1] * inv;
      const float o2 = oacc[db][4 * g4 + 2] * inv, o3 = oacc[db][4 * g4 + 3] * inv;
      if (a.out_fp32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + orow + d0) = f32x4{o0, o1, o2, o3};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.o) + orow + d0) =
            u32x2{pack2<T>(o0, o1), pack2<T>(o2, o3)};
      }
    }
  if (a.lse != nullptr && hh == 0)
    a.lse[((size_t)b * a.H_q + h) * a.N + qi] = l_tot > 0.f ? (m + __log2f(l_tot)) * kLn2 : kNegInf;
}

}  // namespace attn
