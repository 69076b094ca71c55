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
// one segment = (sequence, KV head [x group of 16 query heads]); a stage is
// one block of 16 tokens of a paged cache ("KV Cache:推理慢的真正原因",
// 工程优化手段 / 1. PagedAttention), or several blocks of an int8 or int4
// cache (SB below).  The stages of all segments, laid end to end, form one
// stream; the grid is a fixed number of waves (as many as fit
// on the GPU at once) and wave k takes an equal contiguous share of the
// stream.  A wave never waits for another:
//  * each stage's K rows are loaded straight into MFMA operand registers and
//    its V rows into registers, the next stage's loads in flight while the
//    current one is computed, across segment boundaries (loads with the
//    non-temporal hint: they stream faster than global-to-LDS copies or
//    ordinary loads on this part); the query rows of a segment are loaded
//    with its first stage;
//  * V goes through a wave-private LDS tile (16-bit values, 16 rows per
//    block) to be read transposed, 8-bit values widened on the way; the int4
//    cache stores V in the P V operand's order, so its V is loaded straight
//    into registers and widened there (no LDS tile);
//  * S^T = K Q^T (16 tokens x 16 query heads, heads beyond G are don't-care
//    columns) with v_mfma_f32_16x16x32 on 16-bit and FP8 keys (FP8 widened in
//    registers), or v_mfma_i32_16x16x64_i8 on int8 and int4 codes against the
//    query's three int8 digits (made at each segment's start, query_digits);
//  * running (max, sum) per head; the reference maximum only moves when a
//    stage exceeds it by 2^8, so the O accumulator is rarely rescaled;
//  * O^T += V^T P^T with v_mfma_f32_16x16x16 (16x16x32 over two blocks when a
//    stage has several): P^T comes straight from the S^T registers (rounded
//    to 16 bits), V^T from ds_read_b64_tr_b16 on the row-major V stage (int4:
//    widened from the loaded runs).
// Where a wave's share starts or ends inside a segment, or a segment ends, the
// wave writes that piece's normalised partial output and lse (piece p of a
// segment belongs to the p-th wave whose share overlaps it);
// decode_merge_kernel combines the pieces with their log-sum-exp weights.
#pragma once
#include <type_traits>
#include "decode_plain.h"
#include "mfma_common.h"

namespace attn {

constexpr int kDecStage = 16;     // tokens per stage (one cache block)
constexpr int kDecWaves = 4;      // waves per workgroup
constexpr int kDecMinShare = 16;  // 16-token blocks per wave at least: a share covers 256 tokens or more,
                                  // which bounds the pieces per segment

// Pieces a segment of at most `capacity` tokens can be cut into.
inline constexpr int dec_max_pieces(int capacity) {
  return (capacity + kDecStage * kDecMinShare - 1) / (kDecStage * kDecMinShare) + 1;
}

typedef int i32x4 __attribute__((ext_vector_type(4)));
// int8 x int8 -> int32, 16 x 16 output, 64-deep (gfx950): 16 bytes of A and of
// B per lane; any assignment of the 64 k to lanes that A and B share gives the
// same sums.
__device__ __forceinline__ i32x4 mfma16k64_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
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

// Geometry of one V stage (16 rows, 16-bit elements) in LDS.
template <int D>
struct DecGeom {
  static constexpr int ROWB = D * 2;                 // bytes per row
  static constexpr int CH = D / 8;                   // 16-byte chunks per row
  static constexpr int RPL = 256 / ROWB;             // rows per 256-byte bank line (1 or 2)
  static constexpr int SLOT = kDecStage * ROWB;      // bytes of 16 rows
  static constexpr int VCH = SLOT / 16 / 64;         // 16-byte chunks of V per lane per stage
  // V transposing read: a half-wave reads 8 consecutive rows at chunks {2m, 2m+1}.
  static __device__ __forceinline__ int swz_v(int r) { return 2 * ((r / RPL) % (CH / 2)); }
  // V stage store: instruction i of lane l writes row crow(l) + i * 1024 / ROWB
  // at chunk l % CH (16 lanes fill a 256-byte line in order).  Measured on this
  // part with the LDS bank-conflict counter, this is conflict-free, while
  // stores in which neighbouring lanes write chunks that are not neighbours
  // (every second or fourth chunk of a row) are not, whatever the XOR.  So the
  // 8-bit stages rotate their chunks (vchunk) to the same effect.
  static __device__ __forceinline__ int crow(int l) { return l / CH; }
  static constexpr int CROW_STEP = 1024 / ROWB;
};

struct DecodeStreamArgs {
  DecodeArgs a;
  int32_t* piece_cnt;  // [B][H_q]: pieces of segment (b, gh), written by the wave holding piece 0
  int n_hg;            // groups of 16 query heads per KV head
  float v_scale;       // fp8 cache: V = stored value * v_scale (1 otherwise)
  const float* v_scales;  // int8 / int4 cache: [H_kv][d] per-channel scales of V
  const float* k_scales;  // int8 / int4 cache: [H_kv][d] per-channel scales of K
};

// Cache rows are read exactly once per step, so they are loaded with the
// non-temporal hint (global_load ... nt): measured on this part, a stream of
// random 4 KB blocks reads about 14% faster that way than with ordinary loads,
// which allocate the lines in the caches for reuse that never comes.
__device__ __forceinline__ u32x4 load_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 load_stream8(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
template <typename VT>
__device__ __forceinline__ VT load_stream_as(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const VT*>(p));
}

// Cache element formats of the decode kernel.
enum DecKV { kKV16 = 0, kKVFp8 = 1, kKVInt8 = 2, kKVInt4 = 3 };

// Sum over the wave (uniform result).
__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// int4 V in the pool's operand order (kv_append_int4_kernel): lane (i, g) of a
// block's d * 8 bytes loads its run of d / 8 bytes, tokens 4 g .. 4 g + 3 of
// channels i + 16 m; word w holds channel groups m = 2 w (low nibbles) and
// 2 w + 1 (high nibbles), its bytes tokens 0, 2, 1, 3 of the four.  The P V
// operand of channel group m is the four tokens' values in order, two f16 per
// word: tokens 0 and 1 are nibbles 0 and 4 of the word (m even; 1 and 5 for m
// odd), tokens 2 and 3 nibbles 2 and 6 (3 and 7).  With u = code + 8 (the
// nibble XOR 8), one three-input bit operation per f16 pair takes the two
// nibbles shifted to bits 0 and 16 and makes 0x6400 | u, i.e. 1024 + u exactly:
// ((y & 0x000F000F) ^ 0x64086408), truth table 0x6A = (S0 & S1) ^ S2.  V then
// carries the codes + kI4VOffset, removed once from the normalised output.
constexpr float kI4VOffset = 1032.f;
__device__ __forceinline__ u32x2 i4_v_operand(uint32_t x, int m) {
  const int sh = (m & 1) * 4;
  auto pick = [](uint32_t y) -> uint32_t { return __builtin_amdgcn_bitop3_b32(y, 0x000F000Fu, 0x64086408u, 0x6A); };
  return u32x2{pick(x >> sh), pick(x >> (sh + 8))};
}

// 8 int8 codes (words w[0..1]) -> 8 biased f16 values.  After the XOR with 0x80
// (byte u = code + 128), one byte permute per pair builds the f16 words 0x64uu,
// i.e. 1024 + u exactly (spacing 1 in [1024, 2048)): the code + kI8Offset.  The
// V path removes the offset once from the normalised output.
__device__ __forceinline__ u32x4 i8x8_to_f16_biased(const u32x2 w) {
  const u32x2 b = w ^ 0x80808080u;
  // v_perm_b32 selectors: result bytes (low to high) = b0, 0x64, b1, 0x64 and b2, 0x64, b3, 0x64
  auto pair = [](uint32_t x, uint32_t sel) { return __builtin_amdgcn_perm(0x64646464u, x, sel); };
  constexpr uint32_t kLo = 0x04010400u, kHi = 0x04030402u;
  return u32x4{pair(b[0], kLo), pair(b[0], kHi), pair(b[1], kLo), pair(b[1], kHi)};
}
constexpr float kI8Offset = 1152.f;  // widened int8 V values: code + 1152

// kI4Channel: a lane's 16 bytes of int4 keys (32 codes, channels c0 .. c0 + 31)
// unpack to 32 bytes: word w (channels c0 + 8 w .. + 7) gives the even channels
// of its 8 (low nibbles, shifted up) and then the odd ones (high nibbles), so
// byte p of each 16 enters the int8 Q K^T with channel kI4Channel(p) of its 16:
// 0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15.  The query's digits are
// placed likewise.
__device__ __forceinline__ constexpr int kI4Channel(int p) { return (p & 8) | ((p & 3) << 1) | ((p >> 2) & 1); }
constexpr float kQTop = 4194303.f;  // 2^22 - 1: the largest |x| of a query's int8 digits

// lens and table repeat sa.a.seq_lens and sa.a.table as restrict parameters:
// nothing the kernel writes aliases them, so the compiler can read them with
// scalar loads inside the stage loop (vector loads there would count against
// the vmcnt waits of the stage copies).
template <typename T, int D, bool PAGED, int KV>
__global__ void __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(2)))
decode_mfma_kernel(DecodeStreamArgs sa, const int32_t* __restrict__ lens, const int32_t* __restrict__ table) {
  using Gm = DecGeom<D>;
  constexpr bool FP8 = KV == kKVFp8, I8 = KV == kKVInt8, I4 = KV == kKVInt4, Q8 = KV != kKV16;
  constexpr bool QS = I8 || I4;  // integer codes: key scales folded into the query's int8 digits
  // P V operand type: the query's type, except over an integer cache, where the
  // widened V codes and P are f16 (codes exact, P to 11 bits)
  using TC = typename std::conditional<QS, F16, T>::type;
  constexpr int KS = D / 32;   // 32-deep k-steps of Q K^T
  constexpr int DB = D / 16;   // 16-wide blocks of d
  constexpr int ROWB = Gm::ROWB, VCH = Gm::VCH;
  // bytes per cache row, and 16-byte pieces of K and of V a lane loads per stage
  constexpr int RB = I4 ? D / 2 : (Q8 ? D : ROWB);
  constexpr int NKL = I4 ? 1 : (Q8 ? D / 64 : KS);
  // V loads of an 8- or 4-bit cache.  Wide (8-bit, WV true): the 16-bit
  // path's 16-byte loads, each widening to two chunks of one row, stored in the
  // rotated chunk order (vchunk).  4-bit: one load per lane per block of its
  // run of VB = D / 8 bytes, already in P V operand order (no LDS tile).
  constexpr bool WV = Q8 && !I4;
  constexpr int VB = I4 ? D / 8 : 16;
  constexpr int NV = WV ? D / 64 : I4 ? 1 : VCH;  // V loads per lane per block
  using VT = typename std::conditional<VB == 16, u32x4,
                                       typename std::conditional<VB == 8, u32x2, uint32_t>::type>::type;
  // Physical 16-byte chunk of logical chunk c of tile row r.  The wide 8-bit
  // stores write chunks 2m and 2m + 1 of a row from lane m, so neighbouring
  // lanes write every second chunk; measured on this part, a 16-byte store is
  // conflict-free when neighbouring lanes write neighbouring chunks, so these
  // tiles rotate the chunk index (2m -> m, 2m + 1 -> m + CH / 2) before the
  // per-line XOR, which keeps the transposing reads conflict-free as well.
  constexpr bool ROT = WV;
  auto vchunk = [](int r, int c) {
    if constexpr (ROT)
      return ((c >> 1) | ((c & 1) * (Gm::CH / 2))) ^ ((r / Gm::RPL) % (Gm::CH / 2));
    else
      return c ^ Gm::swz_v(r);
  };
  // Cache blocks per stage.  A 16-bit stage of one block is 128 bytes per lane
  // at d = 128; the int8 stage takes as many blocks as give the same bytes (two
  // at d = 128, four at d = 64), so the per-stage work (the softmax's
  // reductions, the loop, the bookkeeping) is spread over as many bytes and as
  // many bytes are in flight.  The int4 stage is four blocks at either d (at
  // d = 64, four measured 6% faster than the eight that give the same bytes).
  // The 16-bit and FP8 stages keep one block at d = 128 (two measured about 1%
  // slower for FP8, against about 2.5% faster for int8) and take two at d = 64,
  // where a block is half the bytes (1-2% faster there).
  constexpr int SB = I4 ? 4 : I8 ? 256 / RB : (D == 64 ? 2 : 1);
  constexpr int TS = kDecStage * SB;  // tokens per stage
  // vector memory instructions every stage's load issues (K, then V), before
  // any query row or key-scale copy
  constexpr int kStageLoads = SB * (NKL + NV);
  static_assert(!Q8 || PAGED, "8- and 4-bit caches are paged");

  __shared__ __attribute__((aligned(1024))) uint8_t vtile[I4 ? 16 : kDecWaves * Gm::SLOT * SB];
  // int8 / int4: two slots per wave for the key scales of a segment's KV head,
  // copied from global memory with the stage that starts the segment
  __shared__ __attribute__((aligned(16))) float sktile[QS ? kDecWaves * 2 * D : 1];

  const DecodeArgs& a = sa.a;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int col = l & 15, grp = l >> 4;   // MFMA column (head / token row) and k-group
  const int G = a.H_q / a.H_kv;
  const int GH = a.H_kv * sa.n_hg;        // segments per sequence
  const int worker = blockIdx.x * kDecWaves + w;
  const int n_workers = gridDim.x * kDecWaves;

  auto clamp = [&](int n) { return n < 0 ? 0 : (n > a.capacity ? a.capacity : n); };
  // d of the 8 values lane group grp contributes to k-step ks of the 16-bit
  // Q K^T (K and the query fragments agree on it): 16-bit rows 32 ks + 8 grp;
  // FP8 rows 64 (ks / 2) + 16 grp + 8 (ks % 2) (each K load is 64 contiguous
  // bytes of a row, widened into k-steps 2i and 2i + 1).  The int8 and int4
  // caches take their query digits as bytes (the segment start below).
  auto qd = [&](int ks) {
    if constexpr (Q8) return 64 * (ks >> 1) + 16 * grp + 8 * (ks & 1);
    else return 32 * ks + 8 * grp;
  };
  // int8 / int4: first of the 16 channels whose query digits k-step i of the
  // int8 Q K^T takes from lane group grp: the channels its keys give it (int8,
  // bytes 64 i + 16 grp of a row, as the K loads; int4, the 32 codes D / 4 grp
  // .. + 31 unpacked, k-step i taking 16 of them in kI4Channel order)
  auto qs_base = [&](int i) { return I4 ? (D / 4) * grp + 16 * i : 64 * i + 16 * grp; };
  int skslot = 0;  // next LDS slot for a segment's key scales
  // Paged loads, per-lane byte offsets from a block's first row.  K: 16-bit
  // rows, lane (col, grp) takes bytes 16 grp (+ 64 ks) of row col, so each
  // instruction covers half of every row's 128-byte lines and the next one the
  // other half, straight into MFMA operand layout; 8-bit rows, bytes 16 grp (+
  // 64 i) of row col, so one instruction covers 64 contiguous bytes of every
  // row (the query fragments use the same assignment of d to k-steps, qd);
  // 4-bit rows, D / 8 bytes at D / 8 grp (one 16-byte load at d = 128, 8 bytes
  // at d = 64).  V: 16-bit rows, 16 bytes of row crow(l) + i CROW_STEP at
  // 16 (l % CH), so each instruction covers whole rows; the wide 8-bit loads
  // take 16 bytes of row l / (RB / 16) + i 1024 / RB at 16 (l % (RB / 16)) (in
  // load); int4, lane l's run of D / 8 bytes at D / 8 l (1 KB per instruction
  // at d = 128).
  const uint32_t klane = I4 ? col * RB + (D / 8) * grp : col * RB + 16 * grp;
  const uint32_t vlane = I4 ? VB * l : Gm::crow(l) * RB + VB * (l % Gm::CH);
  constexpr int VSTEP = Gm::CROW_STEP * RB;
  auto stages_of = [&](int len) { return (len + TS - 1) / TS; };

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
  // at least 256 tokens per share whatever the stage size (SB blocks per stage),
  // so a stage of several blocks does not leave waves idle on small problems
  const int share = max(kDecMinShare / SB, (total + n_workers - 1) / n_workers);
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
  // a segment's first stage in this wave's share: its query rows are loaded with it
  auto seg_start = [&](const Cursor& c) { return c.st == 0 || c.pos == beg; };

  const uint8_t* kp = static_cast<const uint8_t*>(a.k);
  const uint8_t* vp = static_cast<const uint8_t*>(a.v);
  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const float c_log2 = a.scale_log2;  // > 0 on this path
  float cl = c_log2;                  // the segment's logit scale (int8: over the rescaled query)
  uint8_t* vt = I4 ? vtile : vtile + w * Gm::SLOT * SB;  // int4: no V tile

  // One stage in registers: K rows in MFMA operand layout (lane -> token row
  // col, 16 bytes at d = 32 ks + 8 grp), V as loaded (16-bit: bytes
  // 16 l + 1024 i of the stage; 8-bit: 16 bytes of a row per load; int4: the
  // lane's run of operand-order bytes per block), and the query rows when the
  // stage starts a segment.
  struct Stage {
    u32x4 k[SB][NKL];  // block j of the stage: tokens 16 j .. 16 j + 15
    VT v[SB][NV];
    u32x4 q[KS];
    bool ok;     // valid block ids (paged)
    bool qnew;   // q holds a new segment's query rows
    int skslot;  // int8 / int4, qnew: LDS slot holding the segment's key scales
  };
  // K and V loads come first and are unconditional (same count on every
  // path, so the compiler's vmcnt waits stay exact); query rows follow only
  // when the stage starts a segment.
  // Paged: block ids of the stage under cursor c, read one stage before its
  // loads so the scalar loads' latency hides behind the current stage.  A block
  // of the stage that lies wholly past the sequence's length is not read from
  // the table (its entry may be anything): block 0 of the stage stands in, and
  // its rows get weight 0.
  struct Blocks {
    int id[SB];
  };
  auto block_of = [&](const Cursor& c) {
    Blocks r;
    if constexpr (PAGED) {
      const int32_t* row = table + (int64_t)c.b * a.max_blocks_per_seq + c.st * SB;
      r.id[0] = row[0];
#pragma unroll
      for (int j = 1; j < SB; ++j) r.id[j] = (c.st * SB + j) * kDecStage < c.len ? row[j] : r.id[0];
    } else {
      r.id[0] = 0;
    }
    return r;
  };
  auto load = [&](const Cursor& c, const Blocks& blk, Stage& S) {
    const int g = c.gh / sa.n_hg, hg = c.gh % sa.n_hg;
    S.ok = true;
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      // block j of the stage: tokens t1 .. t1 + 15 (block 0 again if it lies past the length)
      const int t1 = c.st * TS + ((c.st * SB + j) * kDecStage < c.len ? j : 0) * kDecStage;
      size_t row0;
      if (PAGED) {
        const bool ok = blk.id[j] >= 0 && blk.id[j] < a.num_blocks;
        S.ok = S.ok && ok;
        row0 = ((size_t)(ok ? blk.id[j] : 0) * a.H_kv + g) * kDecStage;
      } else {
        row0 = ((size_t)c.b * a.H_kv + g) * a.capacity + (size_t)t1;
      }
      // K and V of block j: the block's rows start at byte row0 * RB of the
      // pool (the same offset in both pools), a wave-uniform base; each lane
      // adds a constant offset (klane, vlane) and each instruction an immediate,
      // so the loads need no per-lane address arithmetic.
      // Contiguous: K rows past the capacity (last stage only) read the last row
      // instead.  V rows past the sequence's length read its last row: their
      // weights are 0, but a slot that was never written may hold a NaN or an
      // infinity, and 0 times those is not 0 (K rows past the length are harmless:
      // their scores are replaced by -inf).  Paged: a block has all 16 rows; the
      // wide 8-bit V loads clamp their row likewise (measured faster here than
      // zeroing), the 16-bit ones read every row and zero those past the length
      // after the load (compute); every int4 code is a finite value, so its V
      // needs neither (weight 0 times a finite value is 0).
      const uint8_t* kb = kp + row0 * RB;
      const uint8_t* vb = vp + row0 * RB;
      if constexpr (PAGED) {
        if constexpr (I4 && D == 64) {
          const u32x2 k2 = load_stream8(kb + klane);
          S.k[j][0] = u32x4{k2[0], k2[1], 0u, 0u};
        } else {
#pragma unroll
          for (int i = 0; i < NKL; ++i) S.k[j][i] = load_stream(kb + klane + 64 * i);
        }
        if constexpr (WV) {
          const int lim = min(kDecStage - 1, c.len - 1 - t1);
#pragma unroll
          for (int i = 0; i < NV; ++i) {
            const int r = min(l / (RB / 16) + i * (1024 / RB), lim);
            S.v[j][i] = load_stream_as<VT>(vb + r * RB + 16 * (l % (RB / 16)));
          }
        } else {
#pragma unroll
          for (int i = 0; i < NV; ++i) S.v[j][i] = load_stream_as<VT>(vb + vlane + i * VSTEP);
        }
      } else {
        const int kr = min(col, a.capacity - 1 - t1);
        const int vlim = c.len - 1 - t1;  // >= 0: the block starts inside the sequence
        const uint8_t* ks_src = kb + kr * ROWB + 16 * grp;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) S.k[j][ks] = load_stream(ks_src + 64 * ks);
        const int lim = min(kDecStage - 1, vlim);
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int r = min(Gm::crow(l) + i * Gm::CROW_STEP, lim);
          S.v[j][i] = load_stream_as<VT>(vb + r * RB + VB * (l % Gm::CH));
        }
      }
    }
    S.qnew = seg_start(c);
    if (S.qnew) {
      // query heads g*G + 16 hg + col (columns past the group repeat head g*G)
      const int gi = 16 * hg + col;
      const size_t qhead = (size_t)c.b * a.H_q + g * G + (gi < G ? gi : 0);
      if constexpr (QS) {
        // the 16 consecutive channels qs_base(i) .. + 15 of k-step i, as loaded
        // (the digits are made in compute), and the KV head's key scales into
        // the next LDS slot (D floats, 16 bytes per lane)
        const uint16_t* src = qp + qhead * D;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
          S.q[2 * i] = *reinterpret_cast<const u32x4*>(src + qs_base(i));
          S.q[2 * i + 1] = *reinterpret_cast<const u32x4*>(src + qs_base(i) + 8);
        }
        S.skslot = skslot;
        skslot ^= 1;
        if (l < D / 4)
          lds_copy16(sa.k_scales + (size_t)g * D + 4 * l, lds_addr(sktile + (2 * w + S.skslot) * D));
      } else {
        const uint16_t* src = qp + qhead * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) S.q[ks] = *reinterpret_cast<const u32x4*>(src + qd(ks));
      }
    }
  };

  // per-segment state
  u32x4 qf[QS ? 3 * (D / 64) : KS];
  // int8 / int4 caches: the key scales fold into the query, q'[c] = q[c] sk[c]
  // in fp32.  Each head's q' is scaled so that its largest element is kQTop =
  // 2^22 - 1 and rounded to an integer x, held as three int8 digits x = 65536
  // d2 + 256 d1 + d0: Q K^T then runs on the int8 matrix cores, exactly (int32
  // sums), against the key codes.  x carries 22 bits and a sign, 2^-22 of the
  // head's largest element (two digits, 15 bits, left errors of 3e-3 in the
  // lse of heads with logits near 60).  qf[3 i .. 3 i + 2] hold d2, d1, d0 of
  // k-step i, byte p for channel qs_base(i) + p (int4: + kI4Channel(p)).  The
  // four lanes of a head (grp 0..3) hold all its channels, so its maximum
  // takes two lane exchanges.  Returns the factor that undoes the scaling in
  // the logit scale: max |q'| / kQTop, and a further 1/16 for the int4 cache,
  // whose codes enter the products as bytes holding 16 times the code.
  auto query_digits = [&](const Stage& S) {
    // the key scales' copy was issued in this stage's load, before the next
    // stage's K and V loads (kStageLoads of them, and perhaps more)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(kStageLoads));
    asm volatile("" ::: "memory");  // the LDS reads below stay after the wait
    const float* skw = sktile + (2 * w + S.skslot) * D;
    float v[D / 64][16];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      const uint16_t* qh = reinterpret_cast<const uint16_t*>(&S.q[2 * i]);
#pragma unroll
      for (int p = 0; p < 16; p += 4) {
        const f32x4 sk4 = *reinterpret_cast<const f32x4*>(skw + qs_base(i) + p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t b = qh[p + e];
          v[i][p + e] = (std::is_same<T, BF16>::value ? bf16_bits_to_f32(b) : f16_bits_to_f32(b)) * sk4[e];
          amax = fmaxf(amax, fabsf(v[i][p + e]));
        }
      }
    }
    amax = fmaxf(amax, xor_shfl(amax, 16));
    amax = max_pair32(amax);
    // A head whose largest |q'| is at most 1e-30 (an all-zero query, in
    // practice) gets zero digits: its true scores (q' times codes of at most
    // 127 in magnitude, over d channels) are below 2e-26, zero to within fp32
    // rounding of the softmax.  This also keeps kQTop / amax finite and the
    // returned factor positive, so that a masked score (-inf) times the logit
    // scale stays -inf rather than becoming -inf * 0 = NaN.
    const bool live = amax > 1e-30f;
    const float up = live ? kQTop / amax : 0.f;
    // rint(v up) = x lands in the low bits of fma(v, up, 1.5 * 2^23): the bits are
    // 0x4B400000 + x for |x| <= 2^22 (the binade [2^23, 2^24) has spacing 1).
    // x = 65536 d2 + 256 d1 + d0 with d0, d1 in [-128, 127] and d2 in [-64, 64]:
    // d0 is byte 0 of x, d1 byte 1 of x + 128, d2 byte 2 of x + 32896, each read
    // as a two's-complement byte (the constant's bytes 0 and 1 are zero).
    const auto byte = [](const uint32_t* u, uint32_t add, uint32_t sel) {
      return __builtin_amdgcn_perm(__builtin_amdgcn_perm(u[3] + add, u[2] + add, sel),
                                   __builtin_amdgcn_perm(u[1] + add, u[0] + add, sel), 0x05040100u);
    };
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {
      uint32_t t[16];
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int ch = I4 ? kI4Channel(p) : p;
        t[p] = __float_as_uint(fmaf(v[i][ch], up, 12582912.f));
      }
      uint32_t d2[4], d1[4], d0[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        d0[d] = byte(t + 4 * d, 0u, 0x0c0c0400u);
        d1[d] = byte(t + 4 * d, 128u, 0x0c0c0501u);
        d2[d] = byte(t + 4 * d, 32896u - 0x4B400000u, 0x0c0c0602u);
      }
      qf[3 * i] = u32x4{d2[0], d2[1], d2[2], d2[3]};
      qf[3 * i + 1] = u32x4{d1[0], d1[1], d1[2], d1[3]};
      qf[3 * i + 2] = u32x4{d0[0], d0[1], d0[2], d0[3]};
    }
    return live ? amax * (1.f / kQTop) * (I4 ? 0.0625f : 1.f) : 1.f;
  };
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
      const bool has_w = l_tot > 0.f;  // the piece has a key with weight > 0
      const float inv = has_w ? 1.f / l_tot : 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 o = oacc[db] * (FP8 ? inv * sa.v_scale : inv);
        if constexpr (I8) o -= has_w ? kI8Offset : 0.f;   // V carried the codes + 1152
        if constexpr (I4) o -= has_w ? kI4VOffset : 0.f;  // V carried the codes + 1032
        if constexpr (QS) o *= *reinterpret_cast<const f32x4*>(sa.v_scales + (size_t)g * D + 16 * db + 4 * grp);
        *reinterpret_cast<f32x4*>(a.part_o + pidx * D + 16 * db + 4 * grp) = o;
      }
      if (grp == 0) a.part_lse[pidx] = e_tot > 0.f ? (m + __log2f(e_tot)) * kLn2 : kNegInf;
    }
  };

  auto compute = [&](const Cursor& c, const Stage& S, const bool last) {
    if (!S.ok && l == 0) raise_device_error(2);
    if (S.qnew) {
      // New segment: clear the running state and O.
      if constexpr (QS)
        cl = c_log2 * query_digits(S);
      else
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = S.q[ks];
      m = kNegInf;
      lsum = 0.f;
      lexact = 0.f;
#pragma unroll
      for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
      // piece p of a segment belongs to the p-th wave whose share overlaps it
      const int seg0 = c.pos - c.st;
      piece = worker - seg0 / share;
      if (piece == 0 && l == 0)
        sa.piece_cnt[(size_t)c.b * a.H_q + c.gh] = (seg0 + c.n - 1) / share - seg0 / share + 1;
    }
    // V rows into the LDS tile (widened to 16 bits: one chunk per load, at tile
    // row 16 j + crow(l) + i CROW_STEP, chunk l % CH), and S^T = K Q^T per block
    // j of the stage: lane holds head col, tokens t0 + 16 j + 4 grp + i.
    const int t0 = c.st * TS;
    // paged: rows at or past the sequence's length (never written, perhaps NaN
    // or infinite, and weighted 0) become 0 before the widening; only the last
    // stage of a segment has such rows, so the others skip the selects
    VT vraw[SB][NV];
#pragma unroll
    for (int j = 0; j < SB; ++j)
#pragma unroll
      for (int i = 0; i < NV; ++i) vraw[j][i] = S.v[j][i];
    if constexpr (PAGED && !WV && !I4) {
      if (t0 + TS > c.len) {
#pragma unroll
        for (int j = 0; j < SB; ++j)
#pragma unroll
          for (int i = 0; i < NV; ++i)
            vraw[j][i] = t0 + 16 * j + Gm::crow(l) + i * Gm::CROW_STEP < c.len ? vraw[j][i] : VT{};
      }
    }
    f32x4 sacc[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      if constexpr (WV) {
        // 8-bit V: 16 values of row r at columns 16 (l % (RB / 16)): logical
        // chunks 2 (l % (RB / 16)) and the next one (int8: the codes + 1152)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const u32x2 w0 = u32x2{vraw[j][i][0], vraw[j][i][1]}, w1 = u32x2{vraw[j][i][2], vraw[j][i][3]};
          const u32x4 lo = I8 ? i8x8_to_f16_biased(w0) : fp8x8_to<T>(w0);
          const u32x4 hi = I8 ? i8x8_to_f16_biased(w1) : fp8x8_to<T>(w1);
          const int r = 16 * j + l / (RB / 16) + i * (1024 / RB), ch = 2 * (l % (RB / 16));
          *reinterpret_cast<u32x4*>(vt + r * ROWB + 16 * vchunk(r, ch)) = lo;
          *reinterpret_cast<u32x4*>(vt + r * ROWB + 16 * vchunk(r, ch + 1)) = hi;
        }
      } else if constexpr (!Q8) {
        // 16-bit V: the loaded chunks as they are (int4 V needs no tile: its
        // operands are built from the loaded runs in the P V step below)
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int r = 16 * j + Gm::crow(l) + i * Gm::CROW_STEP, ch = l % Gm::CH;
          *reinterpret_cast<u32x4*>(vt + r * ROWB + 16 * vchunk(r, ch)) = vraw[j][i];
        }
      }
      sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (QS) {
        // the key codes against the query's three int8 digits on the int8 matrix
        // cores: exact int32 sums (each below 2^22 in magnitude), 256 S1 + S0
        // exact in int32, then 65536 S2 added in fp32 (one rounding).  int8: the codes as stored (16 bytes
        // per k-step).  int4: each word of 8 codes unpacks to 8 bytes holding 16
        // times the codes, even channels then odd (kI4Channel), with one shift
        // and two ANDs; the 1/16 is in the query's factor.
        i32x4 a2 = i32x4{0, 0, 0, 0}, a1 = i32x4{0, 0, 0, 0}, a0 = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
          u32x4 kb;
          if constexpr (I4) {
            const uint32_t w0 = S.k[j][0][2 * i], w1 = S.k[j][0][2 * i + 1];
            kb = u32x4{(w0 << 4) & 0xF0F0F0F0u, w0 & 0xF0F0F0F0u, (w1 << 4) & 0xF0F0F0F0u, w1 & 0xF0F0F0F0u};
          } else {
            kb = S.k[j][i];
          }
          a2 = mfma16k64_i8(kb, qf[3 * i], a2);
          a1 = mfma16k64_i8(kb, qf[3 * i + 1], a1);
          a0 = mfma16k64_i8(kb, qf[3 * i + 2], a0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sacc[j][e] = fmaf((float)a2[e], 65536.f, (float)(a1[e] * 256 + a0[e]));
      } else if constexpr (Q8) {
        // FP8 K: 16 bytes per load, widened into two k-steps
#pragma unroll
        for (int i = 0; i < NKL; ++i) {
          const u32x2 w0 = u32x2{S.k[j][i][0], S.k[j][i][1]}, w1 = u32x2{S.k[j][i][2], S.k[j][i][3]};
          sacc[j] = mfma16k32<TC>(fp8x8_to<T>(w0), qf[2 * i], sacc[j]);
          sacc[j] = mfma16k32<TC>(fp8x8_to<T>(w1), qf[2 * i + 1], sacc[j]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc[j] = mfma16k32<T>(S.k[j][ks], qf[ks], sacc[j]);
      }
    }
    // 16-bit and FP8 keys: mask without a branch, as the S^T accumulator is read right after the MFMA
    // that writes it, and the wait states that read needs are only inserted
    // reliably within one basic block.  A branch here once let the row maximum
    // read a stale accumulator register on one path (a segment's non-final
    // stages): the reference maximum of a column then came from stale data, and
    // at a segment start the O accumulator was not cleared for that column.
    // The int8 and int4 scores are converted from the integer sums by vector
    // instructions, pinned here to the MFMAs' block (an empty asm statement
    // that takes them, so the compiler cannot sink the conversions, which read
    // the MFMA results, past the branch); the mask then sits behind a
    // wave-uniform branch that skips it on every stage the sequence fills.
    if constexpr (QS) {
#pragma unroll
      for (int j = 0; j < SB; ++j) asm volatile("" ::"v"(sacc[j][0]), "v"(sacc[j][1]), "v"(sacc[j][2]), "v"(sacc[j][3]));
    }
    if (!(QS && S.ok && t0 + TS <= c.len)) {
      const int lim = S.ok ? c.len - t0 - 4 * grp : 0;  // rows 16 j + i below lim are keys
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[j][i] = 16 * j + i < lim ? sacc[j][i] : kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < SB; ++j)
      tmax = fmaxf(tmax, fmaxf(fmaxf(sacc[j][0], sacc[j][1]), fmaxf(sacc[j][2], sacc[j][3])));
    tmax = fmaxf(tmax, xor_shfl(tmax, 16));
    tmax = max_pair32(tmax);
    const float mt = tmax * cl;
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
    u32x2 pf[SB];
#pragma unroll
    for (int j = 0; j < SB; ++j) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(sacc[j][i], cl, -base));
      pf[j] = u32x2{cvt_pk<TC>(p[0], p[1]), cvt_pk<TC>(p[2], p[3])};
      lsum = add_pair<TC>(pf[j][1], add_pair<TC>(pf[j][0], lsum));
      lexact += (p[0] + p[1]) + (p[2] + p[3]);
    }
    // O^T += V^T P^T (the wave's own LDS writes above precede these reads).
    // Lane (i, g) of a transposing read holds V^T[16 db + i][4 g .. 4 g + 3] of
    // block j, and pf[j] holds P^T[4 g .. 4 g + 3][head] of the same block, so
    // with several blocks per stage two blocks pair into one 32-deep k-step
    // (k = 8 g + e: e < 4 from block j, e >= 4 from block j + 1, the same order
    // on both operands); the channel tiles go inside, so that consecutive MFMAs
    // are independent.
    auto vread = [&](int j, int db) {
      const int ch = vchunk(vrow, (16 * db + 4 * vq) >> 3);
      return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_i16x4*)(vt + (16 * j + vrow) * ROWB + 16 * ch + 2 * ((4 * vq) & 7)));
    };
    if constexpr (I4) {
      // operands straight from the loaded runs: lane (i, g) holds channel
      // 16 db + i, tokens 4 g .. 4 g + 3 of blocks j and j + 1, as the
      // transposing reads give the other caches
#pragma unroll
      for (int j = 0; j < SB; j += 2) {
        const u32x4 pp = u32x4{pf[j][0], pf[j][1], pf[j + 1][0], pf[j + 1][1]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 v0 = i4_v_operand(vraw[j][0][db >> 1], db), v1 = i4_v_operand(vraw[j + 1][0][db >> 1], db);
          oacc[db] = mfma16k32<TC>(u32x4{v0[0], v0[1], v1[0], v1[1]}, pp, oacc[db]);
        }
      }
    } else if constexpr (SB % 2 == 0) {
#pragma unroll
      for (int j = 0; j < SB; j += 2) {
        const u32x4 pp = u32x4{pf[j][0], pf[j][1], pf[j + 1][0], pf[j + 1][1]};
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const u32x2 v0 = __builtin_bit_cast(u32x2, vread(j, db)), v1 = __builtin_bit_cast(u32x2, vread(j + 1, db));
          oacc[db] = mfma16k32<TC>(u32x4{v0[0], v0[1], v1[0], v1[1]}, pp, oacc[db]);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < SB; ++j)
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = mfma16k16<TC>(vread(j, db), pf[j], oacc[db]);
    }
    if (c.st + 1 == c.n || last) finish(c);
  };

  // two stages in registers: compute one while the next one's loads are in
  // flight.  Past the end of the share the loads repeat the current stage
  // (never used), so every iteration issues the same loads.
  Cursor cc = ic;
#pragma unroll
  for (int db = 0; db < DB; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  // nblk: block ids of stage ic (the dummy reloads past the end reuse them;
  // load checks every id it is given)
  Stage A, B;
  Blocks nblk = block_of(ic);
  load(ic, nblk, A);
  advance(ic);
  if (ic.pos < end) nblk = block_of(ic);
  // One load call per half, its cursor selected: the compiler's wait counting
  // then sees the next stage's loads issued on every path before the current
  // stage's compute (with two call sites it also weighed a path through
  // neither, and waited for every load before computing).
  for (int pos = beg; pos < end; pos += 2) {
    load(pos + 1 < end ? ic : cc, nblk, B);
    if (pos + 1 < end) {
      advance(ic);
      if (ic.pos < end) nblk = block_of(ic);
    }
    compute(cc, A, pos + 1 == end);
    advance(cc);
    if (pos + 1 >= end) break;
    load(pos + 2 < end ? ic : cc, nblk, A);
    if (pos + 2 < end) {
      advance(ic);
      if (ic.pos < end) nblk = block_of(ic);
    }
    compute(cc, B, pos + 2 == end);
    advance(cc);
  }
}

}  // namespace attn
