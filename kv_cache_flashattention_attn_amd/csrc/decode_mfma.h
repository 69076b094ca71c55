// MFMA decode for f16 / bf16 at d in {64, 128}, contiguous or paged cache.
//
// A decode step is one new query per head against every cached key
// ("推理速度慢怎么办？KV Cache与Flash Attention如何加速大模型推理", section 一); with a
// cache the cost is reading K and V from memory ("KV Cache:推理慢的真正原因",
// 缓存的是什么: the bottleneck moves to bandwidth).  Grouped-query attention lets
// the query heads of a group share one K/V head (same page, 工程优化手段 / 2), so
// each K/V row is read ONCE for all G = H_q / H_kv query heads.
//
// Work split (persistent, balanced by bytes): the cache is cut into stages of
// 16 tokens of one segment = (sequence, KV head [x group of 16 query heads]);
// a stage is exactly one block of a paged cache ("KV Cache:推理慢的真正原因",
// 工程优化手段 / 1. PagedAttention).  The stages of all segments, laid end to
// end, form one stream; the grid is a fixed number of waves (as many as fit
// on the GPU at once) and wave k takes an equal contiguous share of the
// stream.  A wave never waits for another:
//  * stage copies go straight from global memory into a wave-private LDS ring
//    of kDecSlots stages (global_load_lds_dwordx4), the next one in flight
//    while the current one is computed, across segment boundaries; the query
//    rows of a segment ride along with its first stage;
//  * S^T = K Q^T with v_mfma_f32_16x16x32 (16 tokens x 16 query heads, heads
//    beyond G are don't-care columns), K rows read with ds_read_b128;
//  * running (max, sum) per head; the reference maximum only moves when a
//    stage exceeds it by 2^8, so the O accumulator is rarely rescaled;
//  * O^T += V^T P^T with v_mfma_f32_16x16x16: P^T comes straight from the S^T
//    registers (rounded to 16 bits), V^T from ds_read_b64_tr_b16 on the
//    row-major V stage.
// Where a wave's share starts or ends inside a segment, or a segment ends, the
// wave writes that piece's normalised partial output and lse (piece p of a
// segment belongs to the p-th wave whose share overlaps it);
// decode_merge_kernel combines the pieces with their log-sum-exp weights.
#pragma once
#include "decode_plain.h"
#include "mfma_common.h"

namespace attn {

constexpr int kDecStage = 16;     // tokens per stage (one cache block)
constexpr int kDecSlots = 2;      // ring stages per wave
constexpr int kDecWaves = 2;      // waves per workgroup
constexpr int kDecMinShare = 16;  // stages per wave at least (bounds the pieces per segment)

// Pieces a segment of at most `capacity` tokens can be cut into.
inline constexpr int dec_max_pieces(int capacity) {
  return (capacity + kDecStage * kDecMinShare - 1) / (kDecStage * kDecMinShare) + 1;
}

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

// Geometry of 16 rows (of K, V or Q; 16-bit elements) in LDS.
template <int D>
struct DecGeom {
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int RPL = 256 / ROWB;             // rows per 256-byte bank line (1 or 2)
  static constexpr int SLOT = kDecStage * ROWB;      // bytes of 16 rows
  static constexpr int COPIES = SLOT / 1024;         // wave-wide 1 KB copies per 16 rows
  static constexpr int ROWS_PER_COPY = 1024 / ROWB;
  // per wave: kDecSlots x (K, V) stages, then kDecSlots query slots
  static constexpr int WAVE_LDS = kDecSlots * 3 * SLOT;
  // K and Q operand reads: 16 lanes read 16 consecutive rows at one logical chunk.
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPL) % CH; }
  // V transposing read: a half-wave reads 8 consecutive rows at chunks {2m, 2m+1}.
  static __device__ __forceinline__ int swz_v(int r) { return 2 * ((r / RPL) % (CH / 2)); }
};

struct DecodeStreamArgs {
  DecodeArgs a;
  int32_t* piece_cnt;  // [B][H_q]: pieces of segment (b, gh), written by the wave holding piece 0
  int n_hg;            // groups of 16 query heads per KV head
};

// Sum over the wave (uniform result).
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// lens and table repeat sa.a.seq_lens and sa.a.table as restrict parameters:
// nothing the kernel writes aliases them, so the compiler can read them with
// scalar loads inside the stage loop (vector loads there would count against
// the vmcnt waits of the stage copies).
template <typename T, int D, bool PAGED>
__global__ void __launch_bounds__(64 * kDecWaves)
decode_mfma_kernel(DecodeStreamArgs sa, const int32_t* __restrict__ lens, const int32_t* __restrict__ table) {
  using Gm = DecGeom<D>;
  constexpr int KS = D / 32;   // 32-deep k-steps of Q K^T
  constexpr int DB = D / 16;   // 16-wide blocks of d
  constexpr int ROWB = Gm::ROWB, CH = Gm::CH;
  constexpr int NCP = 2 * Gm::COPIES;  // copies per stage (K and V)
  constexpr int kQBase = kDecSlots * 2 * Gm::SLOT;  // query slots follow the K/V stages

  __shared__ __attribute__((aligned(1024))) uint8_t ring[kDecWaves * Gm::WAVE_LDS];

  const DecodeArgs& a = sa.a;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int col = l & 15, grp = l >> 4;   // MFMA column (head) and k-group
  const int G = a.H_q / a.H_kv;
  const int GH = a.H_kv * sa.n_hg;        // segments per sequence
  const int worker = blockIdx.x * kDecWaves + w;
  const int n_workers = gridDim.x * kDecWaves;

  auto clamp = [&](int n) { return n < 0 ? 0 : (n > a.capacity ? a.capacity : n); };
  auto stages_of = [&](int len) { return (len + kDecStage - 1) / kDecStage; };

  // total stages (lanes read 64 lengths at a time) and this wave's share
  int total = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    int n = 0;
    if (b0 + l < a.B) {
      const int len = lens[b0 + l];
      if (blockIdx.x == 0 && w == 0) {
        if (len < 0) raise_device_error(4);
        if (len > a.capacity) raise_device_error(1);
      }
      n = GH * stages_of(clamp(len));
    }
    total += wave_sum(n);
  }
  total = __builtin_amdgcn_readfirstlane(total);
  const int share = max(kDecMinShare, (total + n_workers - 1) / n_workers);
  const int beg = worker * share;
  if (beg >= total) return;
  const int end = min(total, beg + share);

  // A cursor walks the stream: stage `st` of segment (b, gh); the segment has
  // n stages and starts at stream position pos - st.
  struct Cursor {
    int pos, b, gh, st, n, len;
  };
  Cursor ic;
  {
    // first segment overlapping beg: inclusive scan of the stage counts
    int pre = 0;
    for (int b0 = 0;; b0 += 64) {
      int n = 0;
      if (b0 + l < a.B) n = GH * stages_of(clamp(lens[b0 + l]));
      int incl = n;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (l >= off) incl += y;
      }
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(pre + incl > beg);
      if (hit != 0) {
        const int lane = __builtin_ctzll(hit);
        const int b = b0 + lane;
        const int before = pre + __builtin_amdgcn_readlane(incl - n, lane);
        ic.len = clamp(lens[b]);
        ic.n = stages_of(ic.len);
        ic.b = b;
        ic.gh = (beg - before) / ic.n;
        ic.st = (beg - before) % ic.n;
        ic.pos = beg;
        break;
      }
      pre += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // the lengths above have landed before any stage copy

  auto advance = [&](Cursor& c) {
    ++c.pos;
    if (++c.st < c.n) return;
    c.st = 0;
    if (++c.gh < GH) return;
    c.gh = 0;
    do {
      ++c.b;
      c.len = c.b < a.B ? clamp(lens[c.b]) : kDecStage;
      c.n = stages_of(c.len);
    } while (c.n == 0);
  };
  // a segment's first stage in this wave's share: the query rows come with it
  auto seg_start = [&](const Cursor& c) { return c.st == 0 || c.pos == beg; };

  const uint8_t* kp = static_cast<const uint8_t*>(a.k);
  const uint8_t* vp = static_cast<const uint8_t*>(a.v);
  const uint8_t* qp = static_cast<const uint8_t*>(a.q);
  const float c_log2 = a.scale_log2;  // > 0 on this path

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

  // Block id of the stage under cursor c (paged).  Read one stage ahead of its
  // copies, so that the scalar load's latency hides behind the wait for the
  // stage being computed.
  auto block_of = [&](const Cursor& c) {
    return (PAGED && c.pos < end) ? table[(int64_t)c.b * a.max_blocks_per_seq + c.st] : 0;
  };

  // Issue the copies of the stage under cursor c (paged: in block blk) into
  // ring slot `slot` (query rows first when it starts a segment, into query
  // slot `qslot`).  Returns false for an invalid block id: block 0 is copied
  // instead (so every stage issues the same copies) and the stage is masked.
  auto issue = [&](const Cursor& c, int blk, int slot, int qslot) -> bool {
    const int g = c.gh / sa.n_hg, hg = c.gh % sa.n_hg;
    if (seg_start(c)) {
      // rows of query heads g*G + 16 hg + r (rows past the group repeat head g*G)
      const uint32_t qdst = wave_lds + kQBase + qslot * Gm::SLOT;
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) {
        const int r = i * Gm::ROWS_PER_COPY + l / CH;
        const int gi = 16 * hg + r;
        const size_t row = (size_t)c.b * a.H_q + g * G + (gi < G ? gi : 0);
        lds_copy16(qp + row * ROWB + 16 * ((l % CH) ^ Gm::swz_k(r)), qdst + i * 1024);
      }
    }
    const uint32_t kdst = wave_lds + slot * 2 * Gm::SLOT;
    const uint32_t vdst = kdst + Gm::SLOT;
    bool valid = true;
    size_t row0;
    if (PAGED) {
      valid = blk >= 0 && blk < a.num_blocks;
      row0 = ((size_t)(valid ? blk : 0) * a.H_kv + g) * kDecStage;
    } else {
      row0 = ((size_t)c.b * a.H_kv + g) * a.capacity + (size_t)c.st * kDecStage;
    }
    if (PAGED || (c.st + 1) * kDecStage <= a.capacity) {
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) {
        lds_copy16(kp + row0 * ROWB, koff[i], kdst + i * 1024);
        lds_copy16(vp + row0 * ROWB, voff[i], vdst + i * 1024);
      }
    } else {  // rows past the capacity are clamped to the last row (and masked)
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) {
        const int r = i * Gm::ROWS_PER_COPY + l / CH;
        const int t = c.st * kDecStage + r;
        const ptrdiff_t shift = (ptrdiff_t)(min(t, a.capacity - 1) - t) * ROWB;
        lds_copy16(kp + row0 * ROWB + koff[i] + shift, kdst + i * 1024);
        lds_copy16(vp + row0 * ROWB + voff[i] + shift, vdst + i * 1024);
      }
    }
    return valid;
  };

  // per-segment state
  u32x4 qf[KS];
  f32x4 oacc[DB];
  float m = kNegInf, lsum = 0.f, lexact = 0.f;
  int piece = 0;
  // V operand (transposing read): group grp reads rows 4 grp + (l % 16) / 4 at
  // columns 16 db + 4 (l % 4).
  const int vrow = 4 * grp + ((l & 15) >> 2), vq = l & 3;

  // write the piece of segment (c.b, c.gh) computed so far
  auto finish = [&](const Cursor& c) {
    float l_tot = lsum + xor_shfl(lsum, 16);
    l_tot = sum_pair32(l_tot);
    float e_tot = lexact + xor_shfl(lexact, 16);
    e_tot = sum_pair32(e_tot);
    const int g = c.gh / sa.n_hg, hg = c.gh % sa.n_hg;
    const int gi = 16 * hg + col;
    if (gi < G) {
      const size_t pidx = ((size_t)c.b * a.H_q + g * G + gi) * a.s_max + piece;
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(a.part_o + pidx * D + 16 * db + 4 * grp) = oacc[db] * inv;
      if (grp == 0) a.part_lse[pidx] = e_tot > 0.f ? (m + __log2f(e_tot)) * kLn2 : kNegInf;
    }
  };

  Cursor cc = ic;                // stage to compute; ic = next stage to issue
  int q_issued = 0, q_used = 0;  // query slots issued / consumed (ring of kDecSlots)
  unsigned ok_bits = 0;          // bit `slot`: that ring slot holds a valid block
  unsigned qs_bits = 0;          // bit `slot`: the stage in that slot also brought query rows
  static_assert(kDecSlots == 2, "the wait counts below assume two slots");
  int ic_blk = block_of(ic);
  for (int s = 0; s < kDecSlots && ic.pos < end; ++s) {
    const bool q = seg_start(ic);
    if (issue(ic, ic_blk, s, q_issued % kDecSlots)) ok_bits |= 1u << s;
    if (q) {
      qs_bits |= 1u << s;
      ++q_issued;
    }
    advance(ic);
    ic_blk = block_of(ic);
  }

  for (int pos = beg; pos < end; ++pos) {
    const int slot = (pos - beg) % kDecSlots;
    // wait until only the next stage's copies are outstanding
    if (pos + 1 < end) {
      if ((qs_bits >> (slot ^ 1)) & 1u)
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NCP + Gm::COPIES));
      else
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(NCP));
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    }
    const bool ok = (ok_bits >> slot) & 1u;
    if (!ok && l == 0) raise_device_error(2);
    if (seg_start(cc)) {
      const uint8_t* Qs = wave_ring + kQBase + (q_used % kDecSlots) * Gm::SLOT;
      ++q_used;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int ch = (4 * ks + grp) ^ Gm::swz_k(col);
        qf[ks] = *reinterpret_cast<const u32x4*>(Qs + col * ROWB + 16 * ch);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      m = kNegInf;
      lsum = 0.f;
      lexact = 0.f;
      // piece p of a segment belongs to the p-th wave whose share overlaps it
      const int seg0 = cc.pos - cc.st;
      piece = worker - seg0 / share;
      if (piece == 0 && l == 0)
        sa.piece_cnt[(size_t)cc.b * a.H_q + cc.gh] = (seg0 + cc.n - 1) / share - seg0 / share + 1;
    }
    const uint8_t* Ks = wave_ring + slot * 2 * Gm::SLOT;
    const uint8_t* Vs = Ks + Gm::SLOT;
    const int t0 = cc.st * kDecStage;

    // S^T = K Q^T: lane holds head col, tokens t0 + 4 grp + i
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int ch = (4 * ks + grp) ^ Gm::swz_k(col);
      const u32x4 kf = *reinterpret_cast<const u32x4*>(Ks + col * ROWB + 16 * ch);
      sacc = mfma16k32<T>(kf, qf[ks], sacc);
    }
    if (!ok || t0 + kDecStage > cc.len) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!ok || t0 + 4 * grp + i >= cc.len) sacc[i] = kNegInf;
    }
    float tmax = fmaxf(fmaxf(sacc[0], sacc[1]), fmaxf(sacc[2], sacc[3]));
    tmax = fmaxf(tmax, xor_shfl(tmax, 16));
    tmax = max_pair32(tmax);
    const float mt = tmax * c_log2;
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
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sacc[i], c_log2, -base));
    const u32x2 pf = u32x2{cvt_pk<T>(p[0], p[1]), cvt_pk<T>(p[2], p[3])};
    lsum = add_pair<T>(pf[1], add_pair<T>(pf[0], lsum));
    lexact += (p[0] + p[1]) + (p[2] + p[3]);

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int ch = ((16 * db + 4 * vq) >> 3) ^ Gm::swz_v(vrow);
      const i16x4 vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(Vs + vrow * ROWB + 16 * ch + 2 * ((4 * vq) & 7)));
      oacc[db] = mfma16k16<T>(vf, pf, oacc[db]);
    }

    if (cc.st + 1 == cc.n || pos + 1 == end) finish(cc);
    // refill this slot with the stage kDecSlots ahead
    if (ic.pos < end) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkmcnt0);  // this slot's reads are done
      const bool q = seg_start(ic);
      const bool valid = issue(ic, ic_blk, slot, q_issued % kDecSlots);
      ok_bits = valid ? (ok_bits | 1u << slot) : (ok_bits & ~(1u << slot));
      if (q) {
        qs_bits |= 1u << slot;
        ++q_issued;
      } else {
        qs_bits &= ~(1u << slot);
      }
      advance(ic);
      ic_blk = block_of(ic);
    }
    advance(cc);
  }
  (void)CH;
}

}  // namespace attn
