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
//  * 4 waves, 32 query rows each; two workgroups share a CU (<= 256 registers
//    per lane, 64 KB of LDS each), so while one wave runs its softmax on the
//    vector ALU the other workgroup's wave on the same SIMD keeps the matrix
//    core busy.  The two workgroups synchronise independently.
//  * K and V tiles go straight from global memory into LDS with
//    global_load_lds_dwordx4 (no register staging), double-buffered: tile j+1
//    is in flight while tile j is computed; one barrier per tile.  Rows are
//    stored with an XOR swizzle of their 16-byte chunks so that the MFMA
//    operand reads below hit distinct banks.
//  * A wave computes S^T = K Q^T with v_mfma_f32_32x32x16 (A = K rows read
//    with ds_read_b128, B = Q^T kept in registers), so each lane holds 32
//    scores of ONE query row: the row max and sum are lane-local apart from
//    one exchange with lane l^32.
//  * The S^T accumulator, rounded to 16 bits, is already laid out as the B
//    operand of O^T = V^T P^T, so P never leaves registers.  The V^T operand is
//    read from the row-major V tile with ds_read_b64_tr_b16 (gfx950's
//    transposing LDS read: each lane of a 16-lane group receives one column of
//    the 4 x 16 block the group addresses).
//  * Scores are in the base-2 domain: t = s * scale * log2(e), weights
//    exp2(t - m) (v_exp_f32), lse = (m + log2 l) ln 2.  The reference maximum m
//    of a row is only raised when a tile's maximum exceeds it by more than
//    kRescaleSlack (weights stay <= 2^8, exact in fp32 accumulation), so the
//    O accumulator is rescaled on a few tiles only, not on every tile.
//  * Workgroup order: the hardware deals workgroup ids round-robin to the 8
//    XCDs, each with its own L2.  Ids are remapped so that XCD x runs a
//    contiguous range of (batch, head) pairs a few heads at a time, so their
//    K/V (2 MB per head at N = 4096, d = 128) is mostly served from L2.
//    Causal query blocks run longest first across each group of heads (see
//    prefill_block_order).
#pragma once
#include "mfma_common.h"
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

// FP8 E4M3 x E4M3 -> fp32, 32 x 32 output, 64-deep (gfx950); 32 bytes of A
// (one row of K) and of B (one column of Q^T) per lane.  Unit block scales
// (E8M0 127 = 2^0): the tensor scales are applied outside.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma32_fp8(u32x4 a0, u32x4 a1, i32x8 b, f32x16 c) {
  const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each
constexpr int kPrefillWaves = 4;  // waves (of 32 query rows) per prefill workgroup

// Geometry of the K / V tiles in LDS for head dimension D (16-bit elements)
// and NW waves of 32 query rows per workgroup.
template <int D, int NW>
struct PrefillGeom {
  static constexpr int BM = 32 * NW, BN = 64;
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int RPL = 256 / ROWB;             // rows per 256-byte bank line (1 or 2)
  static constexpr int TILE = BN * ROWB;             // bytes per K or V tile
  static constexpr int ROWS_PER_COPY = 1024 / ROWB;  // rows one wave-wide 16 B/lane copy fills
  static constexpr int COPIES = TILE / 1024 / NW;    // copies per wave per tile
  // Copy i of wave w fills the 1 KB slice i * NW + w; consecutive copies of a
  // wave are NW * ROWS_PER_COPY rows apart, a multiple of both swizzle periods
  // below, so one lane offset serves all of them.
  static_assert((NW * ROWS_PER_COPY) % 16 == 0, "copy stride vs swizzle period");
  // Stored chunk position of logical chunk c of row r (K): rows that the K
  // operand read touches together (16 consecutive rows) use distinct positions.
  static __device__ __forceinline__ int swz_k(int r) { return (r / RPL) % CH; }
  // V: one half-wave of the transposing read touches 4 consecutive rows at
  // 4 consecutive chunks {4m .. 4m+3}; XOR with 4 (r mod 4) spreads them over
  // all 64 banks.
  static __device__ __forceinline__ int swz_v(int r) { return 4 * ((r / RPL) % (CH / 4)); }
};

// Workgroup order: (batch x head, query block) of workgroup `bid`.
// The hardware deals ids round-robin to the 8 XCDs (XCD x runs x, x + 8, ...),
// and each XCD is given a contiguous range of (b, h) pairs, so that their K/V
// stay in its own L2.  Causal query blocks differ in length (the last block of
// a head does n_qt times the work of the first), so within each group of
// kHeadGroup heads of that range the blocks run longest first across the
// group: the last blocks the GPU starts are the shortest ones and the CUs
// finish together.  Two heads per group: their K and V (2 MB per head at
// N = 4096, d = 128, 16-bit) still fit an XCD's 4 MB L2 together, so each K/V
// byte is fetched from memory about once; with four heads per group the
// prefill fetched 1.7 times its algorithmic bytes, at about the same speed.
constexpr int kHeadGroup = 2;
__device__ __forceinline__ void prefill_block_order(int bid, int n_qt, int total, bool causal, int& bh, int& qt) {
  if (total % kNumXcd == 0) {
    const int per_xcd = total / kNumXcd;  // workgroups per XCD
    const int k = bid / kNumXcd;          // position within this XCD
    const int base = (bid % kNumXcd) * per_xcd;
    if (causal && per_xcd % n_qt == 0) {
      const int heads = per_xcd / n_qt;
      const int hg = heads % kHeadGroup == 0 ? kHeadGroup : (heads % 2 == 0 ? 2 : 1);
      const int gi = k / (hg * n_qt), j = k % (hg * n_qt);
      bh = base / n_qt + gi * hg + j % hg;
      qt = n_qt - 1 - j / hg;
      return;
    }
    const int t = base + k;
    bh = t / n_qt;
    qt = causal ? n_qt - 1 - t % n_qt : t % n_qt;
    return;
  }
  bh = bid / n_qt;
  qt = causal ? n_qt - 1 - bid % n_qt : bid % n_qt;
}

// Workgroup order for chunked prefill.  The work of a sequence grows with its
// cached prefix, so sequences run longest prefix first: KV heads are listed
// sequence by sequence in that order and dealt to the XCDs round-robin, which
// also spreads every sequence over all XCDs.  The G query heads and the query
// blocks of one KV head run next to each other, so they find its K/V in the
// XCD's L2.  rank_to_seq(r) returns the sequence of rank r.
template <typename RankToSeq>
__device__ __forceinline__ void chunk_block_order(int bid, int n_qt, int H_q, int H_kv, int KV, bool causal,
                                                  RankToSeq rank_to_seq, int& bh, int& qt) {
  const int G = H_q / H_kv, per_kv = G * n_qt;
  int pos, rr;
  if (KV % kNumXcd == 0) {
    const int x = bid % kNumXcd, k = bid / kNumXcd;
    pos = (k / per_kv) * kNumXcd + x;
    rr = k % per_kv;
  } else {
    pos = bid / per_kv;
    rr = bid % per_kv;
  }
  const int b = rank_to_seq(pos / H_kv), g = pos % H_kv;
  const int hq = rr / n_qt, qi = rr % n_qt;
  bh = b * H_q + g * G + hq;
  qt = causal ? n_qt - 1 - qi : qi;
}

// Keys and values of a paged cache (chunked prefill): pools
// [num_blocks, H_kv, 16, d], token p of sequence b in block
// table[b * max_blocks_per_seq + p / 16], row p % 16; the N queries of
// sequence b sit at positions cache_lens[b] .. cache_lens[b] + N - 1 (their
// keys already appended), so it has cache_lens[b] + N keys.
struct PagedKV {
  int max_blocks_per_seq;
  int num_blocks;
};
// Block ids a workgroup keeps in LDS (32K tokens); ids past them are read
// from the table directly.
constexpr int kLdsBlocks = 2048;

// F8: Q, K and V are FP8 E4M3 codes (one byte per element) and Q K^T runs on
// the FP8 matrix cores.  V tiles are read as codes into registers (8 bytes per
// lane: the 8 channels of the chunk the 16-bit copy would move), widened
// exactly to T and stored in the 16-bit tile layout, so P V runs in T as in the
// 16-bit kernel; the codes never pass through memory widened.
template <typename T, int D, int NW, bool CAUSAL, bool LSE, bool PAGED, bool F8 = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
prefill_mfma_kernel(PrefillArgs a, PagedKV pk, const int32_t* __restrict__ table,
                    const int32_t* __restrict__ cache_lens) {
  using Gm = PrefillGeom<D, NW>;
  constexpr int BM = Gm::BM, BN = Gm::BN, ROWB = Gm::ROWB, CH = Gm::CH, TILE = Gm::TILE;
  constexpr int KS = D / 16;  // 16-deep k-steps of Q K^T
  constexpr int DB = D / 32;  // 32-wide blocks of the output's d
  static_assert(Gm::COPIES >= 1, "tile shape");
  static_assert(!(F8 && PAGED), "FP8 inputs are contiguous");
  // K tile geometry: an FP8 row of D bytes has the size of D / 2 16-bit elements
  using GK = PrefillGeom<F8 ? D / 2 : D, NW>;
  constexpr int KROWB = GK::ROWB;
  constexpr int K8S = D / 64;  // 64-deep k-steps of the FP8 Q K^T

  // [buffer][K, V] tiles
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2][2][TILE];
  // paged: the sequence's (validated) block ids
  __shared__ __attribute__((aligned(16))) int32_t blk_lds[PAGED ? kLdsBlocks : 1];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l = tid & 63, lr = l & 31, hh = l >> 5;
  const int BH = a.B * a.H_q;
  const int n_qt = (a.N + BM - 1) / BM;
  const int total = n_qt * BH;
  int bh, qt;
  if (PAGED) {
    // rank of sequence i = sequences with a longer prefix, or an equal one and
    // a smaller index; lane i of each 64-sequence slice ranks sequence i
    auto rank_to_seq = [&](int r) {
      const int lane = tid & 63;
      for (int s0 = 0; s0 < a.B; s0 += 64) {
        const int i = s0 + lane;
        const int li = i < a.B ? cache_lens[i] : 0;
        int rank = 0;
        for (int t0 = 0; t0 < a.B; t0 += 64) {  // other lengths, 64 per vector load, shared by readlane
          const int lt = t0 + lane < a.B ? cache_lens[t0 + lane] : 0;
          const int nt = min(64, a.B - t0);
          for (int u = 0; u < nt; ++u) {
            const int lj = __builtin_amdgcn_readlane(lt, u);
            rank += (lj > li || (lj == li && t0 + u < i)) ? 1 : 0;
          }
        }
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(i < a.B && rank == r);
        if (hit != 0) return s0 + (int)__builtin_ctzll(hit);
      }
      return 0;  // not reached: ranks are a permutation of 0 .. B-1
    };
    chunk_block_order(blockIdx.x, n_qt, a.H_q, a.H_kv, a.B * a.H_kv, CAUSAL, rank_to_seq, bh, qt);
  } else {
    prefill_block_order(blockIdx.x, n_qt, total, CAUSAL, bh, qt);
  }
  const int b = bh / a.H_q, h = bh % a.H_q;
  const int g = h / (a.H_q / a.H_kv);
  const int q0 = qt * BM;
  const int qw0 = q0 + 32 * w;  // first query row of this wave
  const int qi = qw0 + lr;      // this lane's query row
  const float c = a.scale_log2; // > 0 on this path

  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* vp = static_cast<const uint16_t*>(a.v);
  const size_t kv_base = PAGED ? 0 : ((size_t)b * a.H_kv + g) * (size_t)a.N * D;

  // Nk keys; query row i sits at key position off + i
  int off = 0;
  if (PAGED) {
    off = cache_lens[b];
    const int room = pk.max_blocks_per_seq * 16 - a.N;  // >= 0 (checked on the host)
    if (off < 0 || off > room) {
      if (tid == 0) raise_device_error(off < 0 ? 4 : 1);
      off = off < 0 ? 0 : room;
    }
  }
  const int Nk = off + a.N;
  const int key_end = CAUSAL ? min(Nk, off + q0 + BM) : Nk;
  const int n_kt = (key_end + BN - 1) / BN;
  // tiles every row of the workgroup sees in full (no mask, no skip)
  const int n_full = CAUSAL ? min((off + q0 + 1) / BN, Nk / BN) : Nk / BN;
  const uint32_t smem_base = lds_addr(&smem[0][0][0]);

  // global -> LDS copy of one K and one V tile: copy i of this wave fills the
  // 1 KB slice i * NW + w of each; lane l fills stored chunk l % CH of row r.
  // Tiles that lie wholly inside the sequence use a scalar tile base plus one
  // lane offset; the ragged last tile clamps each row to the last key.
  const int r0 = w * Gm::ROWS_PER_COPY + l / CH;  // row of copy 0
  const uint32_t koff = r0 * ROWB + 16 * ((l % CH) ^ Gm::swz_k(r0));
  const int r0k = w * GK::ROWS_PER_COPY + l / GK::CH;  // FP8 K: row of copy 0
  const uint32_t koff8 = r0k * KROWB + 16 * ((l % GK::CH) ^ GK::swz_k(r0k));
  const uint32_t voff = r0 * ROWB + 16 * ((l % CH) ^ Gm::swz_v(r0));
  constexpr int kCopyStride = NW * 1024;  // bytes between consecutive copies of a wave
  // one tensor's tile: src = K or V, off = its lane offset, which = 0 (K) / 1 (V)
  // paged: the chunk offset of this lane's 16 bytes within its row
  const uint32_t kch = 16 * ((l % CH) ^ Gm::swz_k(r0)), vch = 16 * ((l % CH) ^ Gm::swz_v(r0));
  // block id of the table slot j (an id outside the pool reads block 0 and raises a flag)
  auto checked_block = [&](int j) {
    int blk = table[(size_t)b * pk.max_blocks_per_seq + j];
    if (blk < 0 || blk >= pk.num_blocks) {
      raise_device_error(2);
      blk = 0;
    }
    return blk;
  };
  // block id of key position p: from LDS (filled below, before the first copy)
  auto block_at = [&](int p) {
    const int j = p >> 4;
    const int blk = j < kLdsBlocks ? __builtin_amdgcn_readfirstlane(blk_lds[j]) : checked_block(j);
    return min(max(blk, 0), pk.num_blocks - 1);  // already valid; kept inside the pool regardless
  };
  // paged full tiles: copy i of wave w covers rows w * RPC + i * NW * RPC of the
  // tile, i.e. block slot pw_slot + i * kSlotStep, rows starting at row
  // (w * RPC) % 16 of that block (NW * RPC is a multiple of 16)
  const int pw = w & (NW - 1);
  const int pw_slot = (pw * Gm::ROWS_PER_COPY) >> 4;
  constexpr int kSlotStep = NW * Gm::ROWS_PER_COPY / 16;
  const uint64_t pw_off = ((uint64_t)g * 16 + ((pw * Gm::ROWS_PER_COPY) & 15)) * ROWB;
  const uint32_t blk_bytes = (uint32_t)a.H_kv * 16 * ROWB;  // one block, all KV heads (< 2^28)
  auto issue_paged = [&](const uint16_t* src, const uint32_t ch, int which, int k0, int buf) {
    const uint32_t dst = smem_base + (2 * buf + which) * TILE + w * 1024;
    const uint8_t* base = reinterpret_cast<const uint8_t*>(src);
    const int last = Nk - 1;
    // the tile's 4 block ids with one LDS read (slot k0 / 16 is a multiple of 4)
    const int j0 = k0 >> 4;
    int ids[4];
    if (j0 + 3 < kLdsBlocks) {
      const int4 v4 = *reinterpret_cast<const int4*>(&blk_lds[j0]);
      ids[0] = __builtin_amdgcn_readfirstlane(v4.x);
      ids[1] = __builtin_amdgcn_readfirstlane(v4.y);
      ids[2] = __builtin_amdgcn_readfirstlane(v4.z);
      ids[3] = __builtin_amdgcn_readfirstlane(v4.w);
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) ids[u] = (j0 + u) * 16 <= last ? checked_block(j0 + u) : 0;
    }
    const uint32_t lane_off = (l / CH) * ROWB + ch;  // this lane's bytes within the copy's rows
    if (k0 + BN <= Nk) {
#pragma unroll
      for (int u = 0; u < 4; ++u) ids[u] = min(max(ids[u], 0), pk.num_blocks - 1);  // valid already; kept in the pool
      // full tile: copy i fills rows of block slot pw_slot + i * kSlotStep, at the
      // wave's fixed row offset within the block; the scalar base is the block's
      // offset (one 32 x 32 -> 64-bit product) plus a per-wave constant
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) {
        const int slot = pw_slot + i * kSlotStep;  // 0 .. 3, wave-uniform
        const int blk = slot == 0 ? ids[0] : slot == 1 ? ids[1] : slot == 2 ? ids[2] : ids[3];
        const uint8_t* cb = base + pw_off + (uint64_t)(uint32_t)blk * blk_bytes;
        lds_copy16(cb, lane_off, dst + i * kCopyStride);
      }
      return;
    }
    // ragged last tile: rows past the last key read the last key instead
    const int blk_last = min(max(block_at(last), 0), pk.num_blocks - 1);
#pragma unroll
    for (int i = 0; i < Gm::COPIES; ++i) {
      // the copy's ROWS_PER_COPY rows lie in one 16-row block of the tile
      const int fr = k0 + w * Gm::ROWS_PER_COPY + i * NW * Gm::ROWS_PER_COPY;
      const int slot = (fr >> 4) - j0;  // 0 .. 3, wave-uniform
      int blk = slot == 0 ? ids[0] : slot == 1 ? ids[1] : slot == 2 ? ids[2] : ids[3];
      blk = min(max(blk, 0), pk.num_blocks - 1);  // valid already; kept inside the pool regardless
      const int r = fr + l / CH;
      const bool in = r <= last;
      const size_t row = ((size_t)(in ? blk : blk_last) * a.H_kv + g) * 16 + ((in ? r : last) & 15);
      lds_copy16(base + row * ROWB + ch, dst + i * kCopyStride);
    }
  };
  auto issue = [&](const uint16_t* src, const uint32_t off, int which, int k0, int buf) {
    if (PAGED) {
      issue_paged(src, which ? vch : kch, which, k0, buf);
      return;
    }
    const uint32_t dst = smem_base + (2 * buf + which) * TILE + w * 1024;
    const uint8_t* tile_base = reinterpret_cast<const uint8_t*>(src + kv_base + (size_t)k0 * D);
    if (k0 + BN <= a.N) {
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) lds_copy16(tile_base + i * kCopyStride, off, dst + i * kCopyStride);
    } else {
#pragma unroll
      for (int i = 0; i < Gm::COPIES; ++i) {
        const int r = r0 + i * NW * Gm::ROWS_PER_COPY;
        const ptrdiff_t shift = (ptrdiff_t)(min(k0 + r, a.N - 1) - (k0 + r)) * ROWB;  // <= 0: clamp to the last key
        lds_copy16(tile_base + i * kCopyStride + off + shift, dst + i * kCopyStride);
      }
    }
  };
  auto issue_k = [&](int k0, int buf) {
    if constexpr (F8) {
      const uint32_t dst = smem_base + 2 * buf * TILE + w * 1024;
      const uint8_t* tile_base = static_cast<const uint8_t*>(a.k) + kv_base + (size_t)k0 * D;
      if (k0 + BN <= a.N) {
#pragma unroll
        for (int i = 0; i < GK::COPIES; ++i) lds_copy16(tile_base + i * kCopyStride, koff8, dst + i * kCopyStride);
      } else {
#pragma unroll
        for (int i = 0; i < GK::COPIES; ++i) {
          const int r = r0k + i * NW * GK::ROWS_PER_COPY;
          const ptrdiff_t shift = (ptrdiff_t)(min(k0 + r, a.N - 1) - (k0 + r)) * KROWB;  // <= 0
          lds_copy16(tile_base + i * kCopyStride + koff8 + shift, dst + i * kCopyStride);
        }
      }
    } else {
      issue(kp, koff, 0, k0, buf);
    }
  };
  auto issue_v = [&](int k0, int buf) { issue(vp, voff, 1, k0, buf); };
  // F8 V: copy i of this lane = row r0 + i NW ROWS_PER_COPY of the tile, logical
  // chunk l % CH (channels 8 (l % CH) .. + 7), as in the 16-bit copy
  u32x2 v8[F8 ? Gm::COPIES : 1];
  auto load_v8 = [&](int k0) {
    const uint8_t* vb = static_cast<const uint8_t*>(a.v) + kv_base + 8 * (l % CH);
#pragma unroll
    for (int i = 0; i < Gm::COPIES; ++i) {
      const int key = min(k0 + r0 + i * NW * Gm::ROWS_PER_COPY, a.N - 1);  // past the end: the last key
      v8[i] = *reinterpret_cast<const u32x2*>(vb + (size_t)key * D);
    }
  };
  auto store_v8 = [&](int buf) {
#pragma unroll
    for (int i = 0; i < Gm::COPIES; ++i) {
      const int r = r0 + i * NW * Gm::ROWS_PER_COPY;
      *reinterpret_cast<u32x4*>(&smem[buf][1][r * ROWB + 16 * ((l % CH) ^ Gm::swz_v(r))]) = fp8x8_to<T>(v8[i]);
    }
  };
  auto issue_v_full = [&](int k0, int buf) {  // a tile known to lie inside the sequence
    if (PAGED) {
      issue_paged(vp, vch, 1, k0, buf);
      return;
    }
    const uint32_t dst = smem_base + (2 * buf + 1) * TILE + w * 1024;
    const uint8_t* tile_base = reinterpret_cast<const uint8_t*>(vp + kv_base + (size_t)k0 * D);
#pragma unroll
    for (int i = 0; i < Gm::COPIES; ++i) lds_copy16(tile_base + i * kCopyStride, voff, dst + i * kCopyStride);
  };

  // Q^T fragments (B operand): lane -> query qi, k-slots -> d = 16 ks + 8 hh + j
  // (F8: 32 bytes per 64-deep step, d = 64 ks + 32 hh + j; K rows use the same
  // assignment, so the products pair the same d whatever order the matrix
  // core gives the 32 bytes)
  u32x4 qf[F8 ? 1 : KS];
  i32x8 qf8[F8 ? K8S : 1];
  {
    const bool ok = qi < a.N;
    const size_t qrow = (((size_t)b * a.H_q + h) * a.N + (ok ? qi : 0)) * D;
    if constexpr (F8) {
      const uint8_t* src = static_cast<const uint8_t*>(a.q) + qrow + 32 * hh;
#pragma unroll
      for (int ks = 0; ks < K8S; ++ks) {
        const u32x4 x0 = ok ? *reinterpret_cast<const u32x4*>(src + 64 * ks) : u32x4{0, 0, 0, 0};
        const u32x4 x1 = ok ? *reinterpret_cast<const u32x4*>(src + 64 * ks + 16) : u32x4{0, 0, 0, 0};
        qf8[ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2],
                        (int)x1[3]};
      }
    } else {
      const uint16_t* src = qp + qrow + 8 * hh;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = ok ? *reinterpret_cast<const u32x4*>(src + 16 * ks) : u32x4{0, 0, 0, 0};
      }
    }
  }

  f32x16 oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
  float m = kNegInf, lsum = 0.f, lexact = 0.f;

  // V operand (transposing read): 16-lane group G = l / 16 addresses rows
  // key0 + (l % 16) / 4 at columns 32 db + 16 (G & 1) + 4 (l % 4).
  const int vg = l >> 4, vrow = (l & 15) >> 2, vq = l & 3;

  // S^T = K_j Q^T for the 64 keys of tile j (two 32-key row blocks).
  auto qk = [&](const int j, f32x16* sacc) {
    const uint8_t* Kt = &smem[j & 1][0][0];
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
    if constexpr (F8) {
#pragma unroll
      for (int ks = 0; ks < K8S; ++ks) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int r = 32 * rb + lr;
          const int c0 = (4 * ks + 2 * hh) ^ GK::swz_k(r), c1 = (4 * ks + 2 * hh + 1) ^ GK::swz_k(r);
          const u32x4 k0 = *reinterpret_cast<const u32x4*>(Kt + r * KROWB + 16 * c0);
          const u32x4 k1 = *reinterpret_cast<const u32x4*>(Kt + r * KROWB + 16 * c1);
          sacc[rb] = mfma32_fp8(k0, k1, qf8[ks], sacc[rb]);
        }
      }
      return;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * rb + lr;
        const int cc = (2 * ks + hh) ^ Gm::swz_k(r);
        const u32x4 kf = *reinterpret_cast<const u32x4*>(Kt + r * ROWB + 16 * cc);
        sacc[rb] = mfma32<T>(kf, qf[ks], sacc[rb]);
      }
    }
  };

  // Mask (diagonal / ragged tiles), row maximum and the rare rescale of the
  // running state.  Kept apart from softmax_pv so that the latter is one
  // straight block the scheduler can interleave with the next tile's Q K^T.
  auto row_max = [&](const int j, f32x16* sacc, const bool masked) {
    const int k0 = j * BN;
    if (masked) {
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + 32 * rb + 8 * (i >> 2) + 4 * hh + (i & 3);
          const bool vis = key < Nk && (!CAUSAL || key <= off + qi);
          if (!vis) sacc[rb][i] = kNegInf;
        }
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
      if (LSE) lexact *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
    }
  };

  // Weights of tile j and O^T += V_j^T P^T.
  auto softmax_pv = [&](const int j, const f32x16* sacc) {
    const uint8_t* Vt = &smem[j & 1][1][0];
    const float base = m == kNegInf ? 0.f : m;
    float psum = 0.f, esum = 0.f;
    u32x4 pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(fmaf(sacc[kk >> 1][8 * (kk & 1) + e], c, -base));
        if (LSE) esum += p[e];
      }
      pf[kk] = u32x4{cvt_pk<T>(p[0], p[1]), cvt_pk<T>(p[2], p[3]), cvt_pk<T>(p[4], p[5]),
                     cvt_pk<T>(p[6], p[7])};
#pragma unroll
      for (int e = 0; e < 4; ++e) psum = add_pair<T>(pf[kk][e], psum);
    }
    lsum += psum;
    if (LSE) lexact += esum;
    // k-step kk = 2 rb + jj covers keys 32 rb + 16 jj + {0..3, 8..11} + 4 hh
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i16x4 half[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int row = 16 * kk + 8 * u + 4 * (vg >> 1) + vrow;
          const int col = 32 * db + 16 * (vg & 1) + 4 * vq;
          const int cc = (col >> 3) ^ Gm::swz_v(row);
          half[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_i16x4*)(Vt + row * ROWB + 16 * cc + 2 * (col & 7)));
        }
        const u32x2 lo = __builtin_bit_cast(u32x2, half[0]), hi = __builtin_bit_cast(u32x2, half[1]);
        oacc[db] = mfma32<T>(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kk], oacc[db]);
      }
    }
  };

  // Software pipeline over key tiles.  Iteration j computes the weights and
  // P V of tile j while the matrix core already runs Q K^T of tile j+1; the
  // copies in flight during iteration j are K_{j+2} and V_{j+1}, so K_j and
  // V_j buffers alternate independently.
  auto active = [&](int j) { return !CAUSAL || j * BN <= off + qw0 + 31; };
  if (PAGED) {
    // every block the copies can touch: the tiles reach past key_end, and
    // rows past the last key read the last key (block of Nk - 1)
    const int nb = min((Nk + 15) >> 4, kLdsBlocks);
    for (int j = tid; j < nb; j += 64 * NW) blk_lds[j] = checked_block(j);
    __syncthreads();
  }
  issue_k(0, 0);
  if constexpr (F8)
    load_v8(0);
  else
    issue_v(0, 0);
  if (n_kt > 1) issue_k(BN, 1);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // own copies done
  if constexpr (F8) store_v8(0);
  __syncthreads();

  f32x16 s_cur[2], s_nxt[2];
  if (active(0)) qk(0, s_cur);

  int j = 0;
  // steady state: tiles j and j+1 both unmasked and active for every wave.
  // One straight block per tile: the 16 MFMAs of Q K_{j+1}^T (each with the
  // next K read) and the vector work of tile j's weights are independent, so
  // the scheduler interleaves them; P V_j follows with its transposing reads.
  auto steady = [&](const int jj, f32x16* sc, f32x16* sn) {
    if (jj + 2 < n_kt) issue_k((jj + 2) * BN, jj & 1);
    if constexpr (F8)
      load_v8((jj + 1) * BN);
    else
      issue_v_full((jj + 1) * BN, (jj + 1) & 1);
    row_max(jj, sc, false);
    qk(jj + 1, sn);
    softmax_pv(jj, sc);
    constexpr int kQkMfma = F8 ? 2 * K8S : 2 * KS, kKReads = F8 ? 2 : 1;  // per MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * kKReads, 0);  // K reads ahead
#pragma unroll
    for (int i = 0; i < kQkMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // 1 MFMA of Q K^T
      __builtin_amdgcn_sched_group_barrier(0x100, kKReads, 0);  // its K reads
    }
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // 2 V^T reads
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA of P V
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // own copies of K_{j+2}, V_{j+1} done
    if constexpr (F8) store_v8((jj + 1) & 1);
    __syncthreads();
  };
  for (; j + 2 < n_full; j += 2) {
    steady(j, s_cur, s_nxt);
    steady(j + 1, s_nxt, s_cur);
  }
  if (j + 1 < n_full) {
    steady(j, s_cur, s_nxt);
    s_cur[0] = s_nxt[0];
    s_cur[1] = s_nxt[1];
    ++j;
  }
  // diagonal / ragged tiles
  for (; j < n_kt; ++j) {
    const bool act = active(j);
    if (act) row_max(j, s_cur, j >= n_full);
    if (j + 2 < n_kt) issue_k((j + 2) * BN, j & 1);
    if (j + 1 < n_kt) {
      if constexpr (F8)
        load_v8((j + 1) * BN);
      else
        issue_v((j + 1) * BN, (j + 1) & 1);
    }
    if (j + 1 < n_kt && active(j + 1)) qk(j + 1, s_nxt);
    if (act) softmax_pv(j, s_cur);
    s_cur[0] = s_nxt[0];
    s_cur[1] = s_nxt[1];
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if constexpr (F8) {
      if (j + 1 < n_kt) store_v8((j + 1) & 1);
    }
    __syncthreads();
  }
  (void)CH;

  // epilogue: O = O_acc / l ; lse = (m + log2 l) ln 2
  const float l_tot = sum_pair32(lsum);
  if (qi >= a.N) return;
  const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * (F8 ? a.v_scale : 1.f);
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
            u32x2{cvt_pk<T>(o0, o1), cvt_pk<T>(o2, o3)};
      }
    }
  if (LSE) {
    const float e_tot = sum_pair32(lexact);
    if (hh == 0)
      a.lse[((size_t)b * a.H_q + h) * a.N + qi] = e_tot > 0.f ? (m + __log2f(e_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace attn
