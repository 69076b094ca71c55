// MFMA split decode for f16 / bf16 at d in {64, 128}, contiguous or paged cache.
//
// A decode step is one new query per head against every cached key
// ("推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理", section 一); with a
// cache the cost is reading K and V from memory ("KV Cache:推理慢的真正原因",
// 缓存的是什么: the bottleneck moves to bandwidth).  Grouped-query attention lets
// the query heads of a group share one K/V head (same page, 工程优化手段 / 2), so
// a workgroup reads each K/V row ONCE for all G = H_q / H_kv query heads.
//
// Work split: one workgroup per (chunk of kMfmaChunk tokens, KV head [x head
// group of 16], sequence); each of its 4 waves streams a contiguous quarter
// of the chunk on its own, with no barrier until the end:
//  * tokens move in stages of 16 (one 16-token block of a paged cache, or 16
//    consecutive rows of a contiguous one: 4 KB of K and 4 KB of V at
//    d = 128), straight from global memory into a wave-private LDS ring of
//    kDecSlots stages with global_load_lds_dwordx4; the next stage is in
//    flight while the current one is computed;
//  * S^T = K Q^T with v_mfma_f32_16x16x32 (16 tokens x 16 query heads, heads
//    beyond G are zero columns), K rows read with ds_read_b128;
//  * running (max, sum) per head; the reference maximum only moves when a
//    stage exceeds it by 2^8, so the O accumulator is rarely rescaled;
//  * O^T += V^T P^T with v_mfma_f32_16x16x16: P^T comes straight from the S^T
//    registers (rounded to 16 bits), V^T from ds_read_b64_tr_b16 on the
//    row-major V stage.
// The four waves' states are merged in LDS and the chunk's normalised partial
// output and lse go to the workspace; decode_merge_kernel combines chunks.
//
// Paged caches ("KV Cache:推理慢的真正原因", 工程优化手段 / 1. PagedAttention): a
// stage is exactly one block; a wave reads the ids of its blocks from the
// block table once, up front; one (block, KV head) is 16 contiguous rows.
#pragma once
#include "decode_plain.h"
#include "mfma_common.h"

namespace attn {

constexpr int kDecStage = 16;                    // tokens per stage (one cache block)
constexpr int kDecSlots = 2;                     // ring stages per wave
constexpr int kDecWaveTokens = 128;              // tokens per wave per chunk
constexpr int kMfmaChunk = 4 * kDecWaveTokens;   // tokens per workgroup

template <typename T>
__device__ __forceinline__ f32x4 mfma16k32(u32x4 a, u32x4 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16k32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16k32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ f32x4 mfma16k16(i16x4 a, u32x2 b, f32x4 c);
template <>
__device__ __forceinline__ f32x4 mfma16k16<BF16>(i16x4 a, u32x2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16k16<F16>(i16x4 a, u32x2 b, f32x4 c) {
  typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b), c,
                                               0, 0, 0);
}

// Geometry of one stage (16 rows of K or V, 16-bit elements) in LDS.
template <int D>
struct DecGeom {
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int RPL = 256 / ROWB;             // rows per 256-byte bank line (1 or 2)
  static constexpr int SLOT = kDecStage * ROWB;      // bytes of K (or V) per stage
  static constexpr int COPIES = SLOT / 1024;         // wave-wide 1 KB copies per tensor per stage
  static constexpr int ROWS_PER_COPY = 1024 / ROWB;
  static constexpr int WAVE_LDS = kDecSlots * 2 * SLOT;  // bytes of ring per wave
  // K operand read: 16 lanes read 16 consecutive rows at one logical chunk.
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPL) % CH; }
  // V transposing read: a half-wave reads 8 consecutive rows at chunks {2m, 2m+1}.
  static __device__ __forceinline__ int swz_v(int r) { return 2 * ((r / RPL) % (CH / 2)); }
};

template <typename T, int D, bool PAGED>
__global__ void __launch_bounds__(256) decode_mfma_kernel(DecodeArgs a, int n_hg) {
  using Gm = DecGeom<D>;
  constexpr int KS = D / 32;   // 32-deep k-steps of Q K^T
  constexpr int DB = D / 16;   // 16-wide blocks of d
  constexpr int ROWB = Gm::ROWB, CH = Gm::CH;
  static_assert(4 * Gm::WAVE_LDS >= 4 * 16 * D * 4, "LDS reuse for the merge");

  __shared__ __attribute__((aligned(1024))) uint8_t ring[4 * Gm::WAVE_LDS];
  __shared__ float mrg_m[4][16], mrg_l[4][16], mrg_e[4][16];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int col = l & 15, grp = l >> 4;   // MFMA column (head) and k-group
  const int s = blockIdx.x;
  const int g = blockIdx.y / n_hg, hg = blockIdx.y % n_hg;
  const int b = blockIdx.z;
  const int G = a.H_q / a.H_kv;

  // lengths and block ids are wave-uniform: keep them in scalar registers so
  // the block-table reads are scalar loads (which do not count in vmcnt)
  const int len = __builtin_amdgcn_readfirstlane(clamp_len(a, b, s == 0 && blockIdx.y == 0 && tid == 0));
  const int start = s * kMfmaChunk;
  if (start >= len) return;
  const int wbeg = start + w * kDecWaveTokens;
  const int wend = min(wbeg + kDecWaveTokens, len);
  const int n_st = wend > wbeg ? (wend - wbeg + kDecStage - 1) / kDecStage : 0;

  const uint8_t* kp = static_cast<const uint8_t*>(a.k);
  const uint8_t* vp = static_cast<const uint8_t*>(a.v);
  const int gi = 16 * hg + col;          // head within the group served by this column
  const bool head_ok = gi < G;
  const float c = a.scale_log2;          // > 0 on this path

  // Q^T fragments (B operand): lane -> head col, k-slots -> d = 32 ks + 8 grp + j
  u32x4 qf[KS];
  {
    const uint16_t* src = static_cast<const uint16_t*>(a.q) +
                          ((size_t)b * a.H_q + g * G + (head_ok ? gi : 0)) * D + 8 * grp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = head_ok ? *reinterpret_cast<const u32x4*>(src + 32 * ks) : u32x4{0, 0, 0, 0};
  }
  // paged: lane i holds the block id of this wave's stage i (one 16-token
  // block per stage), read once here instead of once per stage
  int blk_ids = 0;
  if (PAGED && l < n_st) blk_ids = a.table[(int64_t)b * a.max_blocks_per_seq + (wbeg >> 4) + l];
  // Q and the block ids have landed before any stage copy is issued: the
  // loop's only vector memory operations are then the copies, whose counts
  // the waits below use.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // lane offsets of the wave-wide copies: copy i fills rows i * ROWS_PER_COPY + l / CH
  uint32_t koff[Gm::COPIES], voff[Gm::COPIES];
#pragma unroll
  for (int i = 0; i < Gm::COPIES; ++i) {
    const int r = i * Gm::ROWS_PER_COPY + l / CH;
    koff[i] = r * ROWB + 16 * ((l % CH) ^ Gm::swz_k(r));
    voff[i] = r * ROWB + 16 * ((l % CH) ^ Gm::swz_v(r));
  }
  const uint32_t wave_lds = lds_addr(ring) + w * Gm::WAVE_LDS;
  const uint8_t* wave_ring = ring + w * Gm::WAVE_LDS;

  // Copy stage st of this wave into ring slot st % kDecSlots.  Returns false
  // for an invalid block id: the stage then copies block 0 (so that every
  // stage issues the same number of copies) and is masked.
  auto issue = [&](int st) -> bool {
    const int t0 = wbeg + st * kDecStage;
    const uint32_t kdst = wave_lds + (st % kDecSlots) * 2 * Gm::SLOT;
    const uint32_t vdst = kdst + Gm::SLOT;
    if (PAGED) {
      const int blk = __builtin_amdgcn_readlane(blk_ids, st);
      const bool valid = blk >= 0 && blk < a.num_blocks;
      const size_t row0 = ((size_t)(valid ? blk : 0) * a.H_kv + g) * kDecStage;
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) {
        lds_copy16(kp + row0 * ROWB, koff[i], kdst + i * 1024);
        lds_copy16(vp + row0 * ROWB, voff[i], vdst + i * 1024);
      }
      return valid;
    } else {
      const size_t row0 = ((size_t)b * a.H_kv + g) * a.capacity + t0;
      if (t0 + kDecStage <= a.capacity) {
#pragma unroll
        for (int i = 0; i < Gm::COPIES; ++i) {
          lds_copy16(kp + row0 * ROWB, koff[i], kdst + i * 1024);
          lds_copy16(vp + row0 * ROWB, voff[i], vdst + i * 1024);
        }
      } else {  // rows past the capacity are clamped to the last row (and masked)
#pragma unroll
        for (int i = 0; i < Gm::COPIES; ++i) {
          const int r = i * Gm::ROWS_PER_COPY + l / CH;
          const ptrdiff_t shift = (ptrdiff_t)(min(t0 + r, a.capacity - 1) - (t0 + r)) * ROWB;
          lds_copy16(kp + row0 * ROWB + koff[i] + shift, kdst + i * 1024);
          lds_copy16(vp + row0 * ROWB + voff[i] + shift, vdst + i * 1024);
        }
      }
    }
    return true;
  };

  f32x4 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f, lexact = 0.f;

  // bit `slot` of ok_bits: the stage in that ring slot has a valid block
  static_assert(kDecSlots == 2, "prologue issues two stages");
  unsigned ok_bits = 0;
  if (n_st > 0) ok_bits |= issue(0) ? 1u : 0u;
  if (n_st > 1) ok_bits |= issue(1) ? 2u : 0u;
  // V operand (transposing read): group grp reads rows 4 grp + (l % 16) / 4 at
  // columns 16 db + 4 (l % 4).
  const int vrow = 4 * grp + ((l & 15) >> 2), vq = l & 3;

  for (int st = 0; st < n_st; ++st) {
    const int slot = st % kDecSlots;
    if (st + 1 < n_st) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * Gm::COPIES));  // only the next stage's copies outstanding
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    const bool ok = (ok_bits >> slot) & 1u;
    if (!ok && l == 0) raise_device_error(2);
    const uint8_t* Ks = wave_ring + slot * 2 * Gm::SLOT;
    const uint8_t* Vs = Ks + Gm::SLOT;
    const int t0 = wbeg + st * kDecStage;

    // S^T = K Q^T: lane holds head col, tokens t0 + 4 grp + i
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r = col;
      const int cc = (4 * ks + grp) ^ Gm::swz_k(r);
      const u32x4 kf = *reinterpret_cast<const u32x4*>(Ks + r * ROWB + 16 * cc);
      sacc = mfma16k32<T>(kf, qf[ks], sacc);
    }
    if (!ok || t0 + kDecStage > wend) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!ok || t0 + 4 * grp + i >= wend) sacc[i] = kNegInf;
    }
    float tmax = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    tmax = fmaxf(tmax, xor_shfl(tmax, 16));
    tmax = max_pair32(tmax);
    const float mt = tmax * c;
    const bool raise = mt > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
      const float m_new = raise ? mt : m;
      const float alpha = raise ? fast_exp2(m - m_new) : 1.f;
      m = m_new;
      lsum *= alpha;
      lexact *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
    const float base = m == kNegInf ? 0.f : m;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sacc[i], c, -base));
    const u32x2 pf = u32x2{cvt_pk<T>(p[0], p[1]), cvt_pk<T>(p[2], p[3])};
    lsum = add_pair<T>(pf[1], add_pair<T>(pf[0], lsum));
    lexact += (p[0] + p[1]) + (p[2] + p[3]);

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int cc = ((16 * db + 4 * vq) >> 3) ^ Gm::swz_v(vrow);
      const i16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(Vs + vrow * ROWB + 16 * cc + 2 * ((4 * vq) & 7)));
      oacc[db] = mfma16k16<T>(vf, pf, oacc[db]);
    }
    if (st + kDecSlots < n_st) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);  // this slot's reads are done
      const bool nok = issue(st + kDecSlots);
      ok_bits = (ok_bits & ~(1u << slot)) | (nok ? 1u << slot : 0u);
    }
  }
  (void)CH;

  // merge the four waves of this workgroup
  float l_tot = lsum + xor_shfl(lsum, 16);
  l_tot = sum_pair32(l_tot);
  float e_tot = lexact + xor_shfl(lexact, 16);
  e_tot = sum_pair32(e_tot);
  __syncthreads();
  float* mo = reinterpret_cast<float*>(ring);  // [4][16][D]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) mo[(w * 16 + col) * D + 16 * db + 4 * grp + i] = oacc[db][i];
  if (grp == 0) {
    mrg_m[w][col] = m;
    mrg_l[w][col] = l_tot;
    mrg_e[w][col] = e_tot;
  }
  __syncthreads();
  const int head = tid >> 4, part = tid & 15;
  if (16 * hg + head < G) {
    float M = kNegInf;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, mrg_m[ww][head]);
    const float Mb = M == kNegInf ? 0.f : M;
    float sc[4], L = 0.f, E = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      sc[ww] = fast_exp2(mrg_m[ww][head] - Mb);
      L = fmaf(sc[ww], mrg_l[ww][head], L);
      E = fmaf(sc[ww], mrg_e[ww][head], E);
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
    if (part == 0) a.part_lse[pidx] = E > 0.f ? (M + __log2f(E)) * kLn2 : kNegInf;
  }
}

}  // namespace attn
