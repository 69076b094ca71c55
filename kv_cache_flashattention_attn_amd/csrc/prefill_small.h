// MFMA prefill for small non-causal problems (d = 64): the key tiles of a
// query block are split over the waves of its workgroup.
//
// The tile loop and online softmax are those of "KV缓存与Flash注意力" (Flash
// Attention — 分块技巧, 步骤2) and "推理速度慢怎么办？KV Cache与Flash Attention如何加速
// 大模型推理" (section 二), as in prefill_mfma.h.  What changes is who walks the
// keys.  When a problem has fewer query blocks of 128 rows than the GPU has CUs
// (a short prompt, few heads), prefill_mfma_kernel leaves most CUs idle and
// each workgroup walks all N / 64 key tiles in sequence.  Here a workgroup owns
// only 32 query rows, and its 4 waves take every 4th key tile each: every wave
// computes S^T = K Q^T, the running (max, sum) and O^T += V^T P^T for the same
// rows over its own keys, in its own LDS tiles (copied global -> LDS, double
// buffered, one workgroup barrier per round).  At the end the waves combine
// their states through LDS with the same identity the tiles use: with
// M = max_w m_w, O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w.  There are
// four times as many workgroups, each with a quarter of the sequential work.
// Causal problems keep prefill_mfma_kernel: their blocks already differ in
// length, and splitting them measured slower on small causal shapes.
#pragma once
#include "prefill_mfma.h"

namespace attn {

constexpr int kSmallWaves = 4;  // waves per workgroup, each with a quarter of the key tiles

template <typename T, bool LSE>
__global__ void __launch_bounds__(64 * kSmallWaves) prefill_small_kernel(PrefillArgs a) {
  constexpr int D = 64, NWK = kSmallWaves;
  using Gm = PrefillGeom<D, 4>;  // BN = 64 key tiles, their row size and XOR swizzles
  constexpr int BN = Gm::BN, ROWB = Gm::ROWB, CH = Gm::CH, TILE = Gm::TILE;
  constexpr int KS = D / 16, DB = D / 32;
  constexpr int ROWS_PER_COPY = 1024 / ROWB;  // rows one wave-wide 16 B/lane copy fills

  // [wave][buffer][K, V] tiles (128 KB); after the loop, the waves' partial
  // outputs [wave][row][d] in fp32 (32 KB) reuse it
  __shared__ __attribute__((aligned(1024))) uint8_t smem[NWK][2][2][TILE];
  __shared__ float st_m[NWK][32], st_l[NWK][32], st_e[NWK][32];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, lr = l & 31, hh = l >> 5;
  const int n_qt = (a.N + 31) / 32;
  const int bh = blockIdx.x / n_qt, qt = blockIdx.x % n_qt;
  const int b = bh / a.H_q, h = bh % a.H_q;
  const int g = h / (a.H_q / a.H_kv);
  const int q0 = qt * 32, qi = q0 + lr;
  const float c = a.scale_log2;  // > 0 on this path

  // every row sees keys 0 .. N - 1 (non-causal)
  const int n_kt = (a.N + BN - 1) / BN;
  const int n_rounds = (n_kt + NWK - 1) / NWK;

  const size_t kv_base = ((size_t)b * a.H_kv + g) * (size_t)a.N * D;
  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.k) + kv_base);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(static_cast<const uint16_t*>(a.v) + kv_base);

  // this wave's copy of tile j into buffer buf: copy i fills rows
  // ROWS_PER_COPY i .. of the tile; lane l the stored chunk l % CH of row
  // l / CH, taken from the logical chunk the swizzle puts there; rows past the
  // last key read the last key (masked)
  auto issue = [&](int j, int buf) {
    const int k0 = j * BN;
    const uint32_t kdst = lds_addr(&smem[w][buf][0][0]), vdst = lds_addr(&smem[w][buf][1][0]);
#pragma unroll
    for (int i = 0; i < TILE / 1024; ++i) {
      const int r = i * ROWS_PER_COPY + l / CH;
      const size_t row = (size_t)min(k0 + r, a.N - 1) * ROWB;
      lds_copy16(kbase + row + 16 * ((l % CH) ^ Gm::swz_k(r)), kdst + i * 1024);
      lds_copy16(vbase + row + 16 * ((l % CH) ^ Gm::swz_v(r)), vdst + i * 1024);
    }
  };

  // Q^T fragments (B operand): lane -> query qi, k-slots -> d = 16 ks + 8 hh + j
  u32x4 qf[KS];
  {
    const bool ok = qi < a.N;
    const uint16_t* src = static_cast<const uint16_t*>(a.q) + (((size_t)b * a.H_q + h) * a.N + (ok ? qi : 0)) * D +
                          8 * hh;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = ok ? *reinterpret_cast<const u32x4*>(src + 16 * ks) : u32x4{0, 0, 0, 0};
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = kNegInf, lsum = 0.f, lexact = 0.f;
  const int vg = l >> 4, vrow = (l & 15) >> 2, vq = l & 3;

  // one key tile: S^T = K Q^T (two 32-key row blocks), mask, running max and
  // the rare rescale, weights, O^T += V^T P^T
  auto tile = [&](const int j, const int buf) {
    const uint8_t* Kt = &smem[w][buf][0][0];
    const uint8_t* Vt = &smem[w][buf][1][0];
    const int k0 = j * BN;
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * rb + lr;
        const int cc = (2 * ks + hh) ^ Gm::swz_k(r);
        sacc[rb] = mfma32<T>(*reinterpret_cast<const u32x4*>(Kt + r * ROWB + 16 * cc), qf[ks], sacc[rb]);
      }
    if (k0 + BN > a.N) {  // ragged last tile
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + 32 * rb + 8 * (i >> 2) + 4 * hh + (i & 3) >= a.N) sacc[rb][i] = kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[rb][i]);
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
    float psum = 0.f, esum = 0.f;
    u32x4 pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(sacc[kk >> 1][8 * (kk & 1) + e], c, -base));
        esum += p[e];
      }
      pf[kk] = u32x4{cvt_pk<T>(p[0], p[1]), cvt_pk<T>(p[2], p[3]), cvt_pk<T>(p[4], p[5]), cvt_pk<T>(p[6], p[7])};
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = add_pair<T>(pf[kk][e], psum);
    }
    lsum += psum;
    lexact += esum;
    // k-step kk covers keys 16 kk + {0..3, 8..11} + 4 hh of the tile (as the
    // S^T accumulator holds them)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i16x4 half[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 16 * kk + 8 * u + 4 * (vg >> 1) + vrow;
          const int col = 32 * db + 16 * (vg & 1) + 4 * vq;
          const int cc = (col >> 3) ^ Gm::swz_v(row);
          half[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(Vt + row * ROWB + 16 * cc + 2 * (col & 7)));
        }
        const u32x2 lo = __builtin_bit_cast(u32x2, half[0]), hi = __builtin_bit_cast(u32x2, half[1]);
        oacc[db] = mfma32<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kk], oacc[db]);
      }
  };

  // rounds: wave w computes tile NWK r + w of round r while the tiles of round
  // r + 1 are in flight; every wave runs every round (the barrier count is uniform)
  if (w < n_kt) issue(w, 0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  for (int r = 0; r < n_rounds; ++r) {
    const int j = NWK * r + w;
    if (j + NWK < n_kt) issue(j + NWK, (r + 1) & 1);
    if (j < n_kt) tile(j, r & 1);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // own copies of the next round done
    __syncthreads();
  }

  // combine the waves: per row M = max_w m_w, weights f_w = 2^(m_w - M)
  const float l_w = sum_pair32(lsum), e_w = sum_pair32(lexact);
  if (hh == 0) {
    st_m[w][lr] = m;
    st_l[w][lr] = l_w;
    st_e[w][lr] = e_w;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int u = 0; u < NWK; ++u) M = fmaxf(M, st_m[u][lr]);
  const float Mb = M == kNegInf ? 0.f : M;
  float L = 0.f, E = 0.f;
#pragma unroll
  for (int u = 0; u < NWK; ++u) {
    const float f = fast_exp2(st_m[u][lr] - Mb);  // 0 for a wave without keys
    L += f * st_l[u][lr];
    E += f * st_e[u][lr];
  }
  const float sc = L > 0.f ? fast_exp2(m - Mb) / L : 0.f;
  // this wave's scaled partial: lane (lr, hh) holds d = 32 db + 8 g4 + 4 hh + {0..3}
  float* part = reinterpret_cast<float*>(&smem[0][0][0][0]);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const f32x4 o = f32x4{oacc[db][4 * g4], oacc[db][4 * g4 + 1], oacc[db][4 * g4 + 2], oacc[db][4 * g4 + 3]} * sc;
      *reinterpret_cast<f32x4*>(part + (w * 32 + lr) * D + 32 * db + 8 * g4 + 4 * hh) = o;
    }
  __syncthreads();
  // wave w writes d = CPW w + CPL hh + {0 .. CPL - 1} of row qi: the sum of the partials
  constexpr int CPW = D / NWK, CPL = CPW / 2;  // columns per wave (16), per lane (8)
  if (qi >= a.N) return;
  float o[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) o[e] = 0.f;
#pragma unroll
  for (int u = 0; u < NWK; ++u) {
    const float* src = part + (u * 32 + lr) * D + CPW * w + CPL * hh;
#pragma unroll
    for (int e4 = 0; e4 < CPL; e4 += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + e4);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e4 + e] += x[e];
    }
  }
  const size_t orow = (((size_t)b * a.H_q + h) * a.N + qi) * D + CPW * w + CPL * hh;
  if (a.out_fp32) {
    float* dst = static_cast<float*>(a.o) + orow;
#pragma unroll
    for (int e4 = 0; e4 < CPL; e4 += 4) *reinterpret_cast<f32x4*>(dst + e4) = f32x4{o[e4], o[e4 + 1], o[e4 + 2], o[e4 + 3]};
  } else {
    uint16_t* dst = static_cast<uint16_t*>(a.o) + orow;
#pragma unroll
    for (int e4 = 0; e4 < CPL; e4 += 4)
      *reinterpret_cast<u32x2*>(dst + e4) = u32x2{cvt_pk<T>(o[e4], o[e4 + 1]), cvt_pk<T>(o[e4 + 2], o[e4 + 3])};
  }
  if (LSE && w == 0 && hh == 0)
    a.lse[((size_t)b * a.H_q + h) * a.N + qi] = E > 0.f ? (Mb + __log2f(E)) * kLn2 : kNegInf;
}

}  // namespace attn
