// libattn host side: argument validation, kernel selection and launches.
//
// The whole library is one translation unit so that every kernel shares the
// device error flag (common.h) without relocatable device code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>

#include "attn.h"
#include "block_pool.h"
#include "common.h"
#include "decode_mfma.h"
#include "decode_plain.h"
#include "kv_append.h"
#include "prefill_mfma.h"
#include "prefill_plain.h"
#include "prefill_small.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return ATTN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(int dtype) { return dtype == ATTN_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == ATTN_F32 || dtype == ATTN_F16 || dtype == ATTN_BF16; }

bool plain_head_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

bool mfma_path(int dtype, int d, float scale) {
  return (dtype == ATTN_F16 || dtype == ATTN_BF16) && (d == 64 || d == 128) && scale > 0.f;
}

int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

// Workspace: split partials [B][H_q][S][d] fp32, their lse [B][H_q][S] fp32,
// then the piece counts [B][H_q] int32 of the streaming MFMA decode.  S covers
// both the plain kernel's kPlainChunk-token splits and the MFMA kernel's pieces.
int splits_for(int capacity) {
  const int plain = (capacity + attn::kPlainChunk - 1) / attn::kPlainChunk;
  const int pieces = attn::dec_max_pieces(capacity);
  return plain > pieces ? plain : pieces;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WorkspaceLayout {
  size_t lse_off, cnt_off, bytes;
};

WorkspaceLayout workspace_layout(int B, int H_q, int capacity, int d) {
  const size_t S = (size_t)splits_for(capacity);
  WorkspaceLayout w;
  w.lse_off = align_up((size_t)B * H_q * S * d * sizeof(float), 256);
  w.cnt_off = align_up(w.lse_off + (size_t)B * H_q * S * sizeof(float), 256);
  w.bytes = w.cnt_off + (size_t)B * H_q * sizeof(int32_t);
  return w;
}

size_t workspace_bytes(int B, int H_q, int capacity, int d) { return workspace_layout(B, H_q, capacity, d).bytes; }

// Workgroups of `kernel` (block of `threads`) that fit on the current device at once.
int resident_grid(const void* kernel, int threads) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) return 0;
  return cus * (per_cu > 0 ? per_cu : 1);
}

// Compute units of the current device (0 if the query fails).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

// Small non-causal prefill (d = 64): one workgroup per 32 query rows, key tiles
// split over its waves (prefill_small.h).
template <typename T>
int launch_prefill_small(const attn::PrefillArgs& a, hipStream_t st) {
  const long long blocks = (long long)((a.N + 31) / 32) * a.B * a.H_q;
  if (blocks > 0x7FFFFFFFLL) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: problem too large");
  const dim3 grid((unsigned)blocks), block(64 * attn::kSmallWaves);
  if (a.lse != nullptr)
    hipLaunchKernelGGL((attn::prefill_small_kernel<T, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((attn::prefill_small_kernel<T, false>), grid, block, 0, st, a);
  return launch_status("attn_prefill");
}

// ---------------------------------------------------------------------------
// prefill dispatch
// ---------------------------------------------------------------------------
template <typename T, int D>
int launch_prefill_plain(const attn::PrefillArgs& a, bool causal, hipStream_t st) {
  constexpr int ROWS = 256 / (D / 16);
  dim3 grid((a.N + ROWS - 1) / ROWS, a.H_q, a.B);
  if (causal)
    hipLaunchKernelGGL((attn::prefill_plain_kernel<T, D, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn::prefill_plain_kernel<T, D, false>), grid, dim3(256), 0, st, a);
  return launch_status("attn_prefill");
}

template <typename T>
int prefill_plain_d(const attn::PrefillArgs& a, int d, bool causal, hipStream_t st) {
  switch (d) {
    case 16: return launch_prefill_plain<T, 16>(a, causal, st);
    case 32: return launch_prefill_plain<T, 32>(a, causal, st);
    case 64: return launch_prefill_plain<T, 64>(a, causal, st);
    case 128: return launch_prefill_plain<T, 128>(a, causal, st);
    case 256: return launch_prefill_plain<T, 256>(a, causal, st);
  }
  return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: head dim %d not supported", d);
}

template <typename T, int D, bool PAGED, bool F8 = false>
int launch_prefill_mfma(const attn::PrefillArgs& a, bool causal, hipStream_t st, const attn::PagedKV& pk = {0, 0},
                        const int32_t* table = nullptr, const int32_t* cache_lens = nullptr) {
  constexpr int NW = attn::kPrefillWaves;
  const long long n_qt = (a.N + 32 * NW - 1) / (32 * NW);
  const long long blocks = n_qt * a.B * a.H_q;
  if (blocks > 0x7FFFFFFFLL) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: problem too large");
  if constexpr (D == 64 && !PAGED && !F8) {
    // non-causal with fewer query blocks than CUs: split each block's keys over
    // the waves instead
    static const int cus = device_cus();  // every device here is an MI355X
    if (!causal && blocks < cus) return launch_prefill_small<T>(a, st);
  }
  const dim3 grid((unsigned)blocks), block(64 * NW);
  const bool lse = a.lse != nullptr;
  if (causal && lse)
    hipLaunchKernelGGL((attn::prefill_mfma_kernel<T, D, NW, true, true, PAGED, F8>), grid, block, 0, st, a, pk, table,
                       cache_lens);
  else if (causal)
    hipLaunchKernelGGL((attn::prefill_mfma_kernel<T, D, NW, true, false, PAGED, F8>), grid, block, 0, st, a, pk, table,
                       cache_lens);
  else if (lse)
    hipLaunchKernelGGL((attn::prefill_mfma_kernel<T, D, NW, false, true, PAGED, F8>), grid, block, 0, st, a, pk, table,
                       cache_lens);
  else
    hipLaunchKernelGGL((attn::prefill_mfma_kernel<T, D, NW, false, false, PAGED, F8>), grid, block, 0, st, a, pk, table,
                       cache_lens);
  return launch_status("attn_prefill");
}

template <typename T>
int prefill_mfma_d(const attn::PrefillArgs& a, int d, bool causal, hipStream_t st) {
  return d == 64 ? launch_prefill_mfma<T, 64, false>(a, causal, st) : launch_prefill_mfma<T, 128, false>(a, causal, st);
}

// FP8 prefill: one launch; the kernel widens V's codes on the way into LDS.
template <typename T>
int prefill_fp8_d(const attn::PrefillArgs& a, int d, bool causal, hipStream_t st) {
  return d == 64 ? launch_prefill_mfma<T, 64, false, true>(a, causal, st)
                 : launch_prefill_mfma<T, 128, false, true>(a, causal, st);
}

template <typename T>
int prefill_paged_d(const attn::PrefillArgs& a, int d, bool causal, const attn::PagedKV& pk, const int32_t* table,
                    const int32_t* cache_lens, hipStream_t st) {
  return d == 64 ? launch_prefill_mfma<T, 64, true>(a, causal, st, pk, table, cache_lens)
                 : launch_prefill_mfma<T, 128, true>(a, causal, st, pk, table, cache_lens);
}

// ---------------------------------------------------------------------------
// decode dispatch
// ---------------------------------------------------------------------------
template <typename T, int D, bool PAGED>
int launch_decode_plain(const attn::DecodeArgs& a, hipStream_t st) {
  dim3 grid((a.capacity + attn::kPlainChunk - 1) / attn::kPlainChunk, a.H_q, a.B);
  hipLaunchKernelGGL((attn::decode_plain_kernel<T, D, PAGED>), grid, dim3(256), 0, st, a);
  return launch_status("attn_decode");
}

// How the cache stores K and V: 16-bit (the query's type), FP8 E4M3 with one
// scale per tensor, or int8 / int4 with one scale per (KV head, channel).
struct CacheQuant {
  int kind = attn::kKV16;
  float k_scale = 1.f, v_scale = 1.f;              // FP8
  const float* k_scales = nullptr;                 // int8 / int4: [H_kv][d], device
  const float* v_scales = nullptr;
};

template <typename T, int D, bool PAGED, int KV>
int launch_decode_mfma(const attn::DecodeArgs& a, int32_t* piece_cnt, hipStream_t st,
                       const CacheQuant& cq = CacheQuant()) {
  const int G = a.H_q / a.H_kv;
  const attn::DecodeStreamArgs sa{a, piece_cnt, (G + 15) / 16, cq.v_scale, cq.v_scales, cq.k_scales};
  const void* kernel = reinterpret_cast<const void*>(&attn::decode_mfma_kernel<T, D, PAGED, KV>);
  static int grid = 0;  // one value per instantiation; every device here is an MI355X
  if (grid == 0) grid = resident_grid(kernel, 64 * attn::kDecWaves);
  if (grid <= 0) return fail(ATTN_ERR_HIP, "attn_decode: occupancy query failed");
  hipLaunchKernelGGL((attn::decode_mfma_kernel<T, D, PAGED, KV>), dim3(grid), dim3(64 * attn::kDecWaves), 0, st,
                     sa, a.seq_lens, a.table);
  return launch_status("attn_decode");
}

template <typename T, int D>
int launch_merge(const attn::DecodeArgs& a, void* o, float* lse, int chunk, const int32_t* piece_cnt,
                 hipStream_t st) {
  const int G = a.H_q / a.H_kv;
  attn::MergeArgs m{a.part_o, a.part_lse, a.seq_lens, piece_cnt, o, lse, a.H_q, a.capacity, a.s_max, chunk,
                    G, (G + 15) / 16, a.out_fp32};
  hipLaunchKernelGGL((attn::decode_merge_kernel<T, D>), dim3(a.H_q, a.B), dim3(64), 0, st, m);
  return launch_status("attn_decode merge");
}

template <typename T, int D, bool PAGED>
int decode_typed(const attn::DecodeArgs& a, void* o, float* lse, bool mfma, int32_t* piece_cnt, hipStream_t st) {
  if constexpr ((D == 64 || D == 128) && !std::is_same<T, attn::F32>::value) {
    if (mfma) {
      const int rc = launch_decode_mfma<T, D, PAGED, attn::kKV16>(a, piece_cnt, st);
      if (rc != ATTN_OK) return rc;
      return launch_merge<T, D>(a, o, lse, 0, piece_cnt, st);
    }
  }
  const int rc = launch_decode_plain<T, D, PAGED>(a, st);
  if (rc != ATTN_OK) return rc;
  return launch_merge<T, D>(a, o, lse, attn::kPlainChunk, nullptr, st);
}

template <typename T, bool PAGED>
int decode_d(const attn::DecodeArgs& a, void* o, float* lse, int d, bool mfma, int32_t* cnt, hipStream_t st) {
  switch (d) {
    case 16: return decode_typed<T, 16, PAGED>(a, o, lse, mfma, cnt, st);
    case 32: return decode_typed<T, 32, PAGED>(a, o, lse, mfma, cnt, st);
    case 64: return decode_typed<T, 64, PAGED>(a, o, lse, mfma, cnt, st);
    case 128: return decode_typed<T, 128, PAGED>(a, o, lse, mfma, cnt, st);
    case 256: return decode_typed<T, 256, PAGED>(a, o, lse, mfma, cnt, st);
  }
  return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: head dim %d not supported", d);
}

template <bool PAGED>
int decode_dispatch(const attn::DecodeArgs& a, void* o, float* lse, int d, int dtype, float scale, int32_t* cnt,
                    hipStream_t st) {
  const bool mfma = mfma_path(dtype, d, scale);
  switch (dtype) {
    case ATTN_F32: return decode_d<attn::F32, PAGED>(a, o, lse, d, false, cnt, st);
    case ATTN_F16: return decode_d<attn::F16, PAGED>(a, o, lse, d, mfma, cnt, st);
    case ATTN_BF16: return decode_d<attn::BF16, PAGED>(a, o, lse, d, mfma, cnt, st);
  }
  return fail(ATTN_ERR_UNSUPPORTED, "attn_decode: dtype %d not supported", dtype);
}

// 8- and 4-bit paged cache (FP8, int8, int4): the MFMA decode (the integer
// caches fold the key scales into the query's digits at each segment's start),
// then the merge.
template <typename T, int KV>
int decode_q8_typed(attn::DecodeArgs a, void* o, float* lse, int d, const CacheQuant& cq, int32_t* cnt,
                    hipStream_t st) {
  int rc = d == 64 ? launch_decode_mfma<T, 64, true, KV>(a, cnt, st, cq)
                   : launch_decode_mfma<T, 128, true, KV>(a, cnt, st, cq);
  if (rc != ATTN_OK) return rc;
  return d == 64 ? launch_merge<T, 64>(a, o, lse, 0, cnt, st) : launch_merge<T, 128>(a, o, lse, 0, cnt, st);
}

template <typename T>
int decode_q8_dispatch(const attn::DecodeArgs& a, void* o, float* lse, int d, const CacheQuant& cq, int32_t* cnt,
                       hipStream_t st) {
  if (cq.kind == attn::kKVFp8) return decode_q8_typed<T, attn::kKVFp8>(a, o, lse, d, cq, cnt, st);
  if (cq.kind == attn::kKVInt4) return decode_q8_typed<T, attn::kKVInt4>(a, o, lse, d, cq, cnt, st);
  return decode_q8_typed<T, attn::kKVInt8>(a, o, lse, d, cq, cnt, st);
}

// Workspace of attn_decode_paged_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it is a stand-in, not a device address): it
// uses the address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// The device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; nullptr if the lookup fails.
void* scratch_address() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

int check_decode_common(const char* fn, const void* q, const void* k, const void* v, const int32_t* lens,
                        const void* o, int B, int H_q, int H_kv, int d, int dtype, float scale) {
  if (!q || !k || !v || !lens || !o) return fail(ATTN_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (B < 1 || H_q < 1 || H_kv < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: B, H_q, H_kv must be >= 1", fn);
  if (H_q % H_kv != 0) return fail(ATTN_ERR_INVALID_ARG, "%s: H_q (%d) is not a multiple of H_kv (%d)", fn, H_q, H_kv);
  if (H_kv > 65535 || B > 65535 || H_q > 65535) return fail(ATTN_ERR_INVALID_ARG, "%s: B or heads too large", fn);
  if (!valid_dtype(dtype)) return fail(ATTN_ERR_UNSUPPORTED, "%s: dtype %d not supported", fn, dtype);
  if (!plain_head_dim(d)) return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d not supported", fn, d);
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "%s: scale must be finite", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(ATTN_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_prefill(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H_q, int H_kv,
                 int N, int d, int causal, float scale, int dtype, int out_fp32, void* stream) {
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: null tensor pointer");
  if (B < 1 || H_q < 1 || H_kv < 1 || N < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: B, H_q, H_kv, N must be >= 1");
  if (H_q % H_kv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: H_q (%d) is not a multiple of H_kv (%d)", H_q, H_kv);
  if (B > 65535 || H_q > 65535) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: B or H_q too large");
  if (!valid_dtype(dtype)) return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: dtype %d not supported", dtype);
  if (!plain_head_dim(d)) return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill: head dim %d not supported", d);
  if (!std::isfinite(scale)) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: scale must be finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: tensors must be 16-byte aligned");
  if ((long long)N * d > 0x7FFFFFFFLL) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill: N*d too large");

  attn::PrefillArgs a{q, k, v, o, lse, B, H_q, H_kv, N, scale * attn::kLog2e, out_fp32 != 0};
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool c = causal != 0;
  if (mfma_path(dtype, d, scale)) {
    return dtype == ATTN_BF16 ? prefill_mfma_d<attn::BF16>(a, d, c, st) : prefill_mfma_d<attn::F16>(a, d, c, st);
  }
  switch (dtype) {
    case ATTN_F32: return prefill_plain_d<attn::F32>(a, d, c, st);
    case ATTN_F16: return prefill_plain_d<attn::F16>(a, d, c, st);
    default: return prefill_plain_d<attn::BF16>(a, d, c, st);
  }
}

size_t attn_prefill_fp8_workspace_bytes(int B, int H_kv, int N, int d) {
  (void)B, (void)H_kv, (void)N, (void)d;
  return 0;  // V is widened inside the kernel
}

int attn_prefill_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H_q, int H_kv, int N,
                     int d, int causal, float scale, float q_scale, float k_scale, float v_scale, int out_dtype,
                     int out_fp32, void* workspace, size_t workspace_bytes_given, void* stream) {
  const char* fn = "attn_prefill_fp8";
  if (!q || !k || !v || !o) return fail(ATTN_ERR_INVALID_ARG, "%s: null tensor pointer", fn);
  if (B < 1 || H_q < 1 || H_kv < 1 || N < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: B, H_q, H_kv, N must be >= 1", fn);
  if (H_q % H_kv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "%s: H_q (%d) is not a multiple of H_kv (%d)", fn, H_q, H_kv);
  if (B > 65535 || H_q > 65535) return fail(ATTN_ERR_INVALID_ARG, "%s: B or H_q too large", fn);
  if (!(out_dtype == ATTN_F16 || out_dtype == ATTN_BF16) || !(d == 64 || d == 128))
    return fail(ATTN_ERR_UNSUPPORTED, "%s: f16/bf16 output with d = 64 or 128 only", fn);
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(ATTN_ERR_UNSUPPORTED, "%s: scale must be positive", fn);
  if (!std::isfinite(q_scale) || !std::isfinite(k_scale) || !std::isfinite(v_scale) || !(q_scale > 0.f) ||
      !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(ATTN_ERR_INVALID_ARG, "%s: q_scale, k_scale and v_scale must be finite and positive", fn);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ATTN_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  if ((long long)N * d > 0x7FFFFFFFLL) return fail(ATTN_ERR_INVALID_ARG, "%s: N*d too large", fn);
  (void)workspace, (void)workspace_bytes_given;  // none needed
  attn::PrefillArgs a{q, k, v, o, lse, B, H_q, H_kv, N, scale * q_scale * k_scale * attn::kLog2e, out_fp32 != 0,
                      v_scale};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return out_dtype == ATTN_BF16 ? prefill_fp8_d<attn::BF16>(a, d, causal != 0, st)
                                : prefill_fp8_d<attn::F16>(a, d, causal != 0, st);
}

int attn_prefill_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                       const int32_t* cache_lens, void* o, float* lse, int B, int H_q, int H_kv, int n_new, int d,
                       int block_size, int max_blocks_per_seq, int num_blocks, int causal, float scale, int dtype,
                       void* stream) {
  if (!q || !k_pool || !v_pool || !block_table || !cache_lens || !o)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: null pointer");
  if (B < 1 || H_q < 1 || H_kv < 1 || n_new < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: B, H_q, H_kv, n_new must be >= 1");
  if (H_q % H_kv != 0)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: H_q (%d) is not a multiple of H_kv (%d)", H_q, H_kv);
  if (B > 65535 || H_q > 65535) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: B or H_q too large");
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_paged: block_size must be 16 (got %d)", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: max_blocks_per_seq and num_blocks must be >= 1");
  if ((long long)max_blocks_per_seq * 16 > 0x7FFFFFFFLL || (long long)max_blocks_per_seq * B > 0x7FFFFFFFLL)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: block table too large");
  if (n_new > max_blocks_per_seq * 16)
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: n_new (%d) exceeds the table's capacity (%d)", n_new,
                max_blocks_per_seq * 16);
  if (!(dtype == ATTN_F16 || dtype == ATTN_BF16) || !(d == 64 || d == 128))
    return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_paged: f16/bf16 with d = 64 or 128 only");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_paged: scale must be finite and positive");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) || (lse && !aligned16(lse)))
    return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: tensors must be 16-byte aligned");
  if ((long long)n_new * d > 0x7FFFFFFFLL) return fail(ATTN_ERR_INVALID_ARG, "attn_prefill_paged: n_new*d too large");

  attn::PrefillArgs a{q, k_pool, v_pool, o, lse, B, H_q, H_kv, n_new, scale * attn::kLog2e, 0};
  const attn::PagedKV pk{max_blocks_per_seq, num_blocks};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return dtype == ATTN_BF16 ? prefill_paged_d<attn::BF16>(a, d, causal != 0, pk, block_table, cache_lens, st)
                            : prefill_paged_d<attn::F16>(a, d, causal != 0, pk, block_table, cache_lens, st);
}

int kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* cache_lens,
              const int32_t* block_table, int B, int H_kv, int n_new, int d, int max_len, int block_size,
              int max_blocks_per_seq, int num_blocks, int dtype, void* stream) {
  if (!k_cache || !v_cache || !k_new || !v_new || !cache_lens)
    return fail(ATTN_ERR_INVALID_ARG, "kv_append: null pointer");
  if (B < 1 || H_kv < 1 || n_new < 1) return fail(ATTN_ERR_INVALID_ARG, "kv_append: B, H_kv, n_new must be >= 1");
  if (!valid_dtype(dtype)) return fail(ATTN_ERR_UNSUPPORTED, "kv_append: dtype %d not supported", dtype);
  if (!plain_head_dim(d)) return fail(ATTN_ERR_UNSUPPORTED, "kv_append: head dim %d not supported", d);
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(ATTN_ERR_INVALID_ARG, "kv_append: tensors must be 16-byte aligned");
  if (block_table) {
    if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "kv_append: block_size must be 16 (got %d)", block_size);
    if (max_blocks_per_seq < 1 || num_blocks < 1)
      return fail(ATTN_ERR_INVALID_ARG, "kv_append: max_blocks_per_seq and num_blocks must be >= 1");
  } else if (max_len < 1) {
    return fail(ATTN_ERR_INVALID_ARG, "kv_append: max_len must be >= 1");
  }
  attn::AppendArgs a;
  a.k_cache = static_cast<uint4*>(k_cache);
  a.v_cache = static_cast<uint4*>(v_cache);
  a.k_new = static_cast<const uint4*>(k_new);
  a.v_new = static_cast<const uint4*>(v_new);
  a.cache_lens = cache_lens;
  a.block_table = block_table;
  a.B = B;
  a.H_kv = H_kv;
  a.n_new = n_new;
  a.chunks_per_row = d * elem_bytes(dtype) / 16;
  a.max_len = max_len;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  const long long total = (long long)B * H_kv * n_new * a.chunks_per_row;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return fail(ATTN_ERR_INVALID_ARG, "kv_append: too many rows");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (block_table)
    hipLaunchKernelGGL((attn::kv_append_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn::kv_append_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, st, a);
  return launch_status("kv_append");
}

size_t attn_decode_workspace_bytes(int B, int H_q, int max_seq_len, int d) {
  if (B < 1 || H_q < 1 || max_seq_len < 1 || d < 1) return 0;
  return workspace_bytes(B, H_q, max_seq_len, d);
}

static int decode_common(const char* fn, bool paged, const void* q, const void* k, const void* v,
                         const int32_t* table, const int32_t* seq_lens, void* o, float* lse, int B, int H_q,
                         int H_kv, int capacity, int mbps, int num_blocks, int d, float scale, int dtype,
                         int out_fp32, void* workspace, size_t workspace_bytes_given, void* stream,
                         const CacheQuant& cq = CacheQuant()) {
  int rc = check_decode_common(fn, q, k, v, seq_lens, o, B, H_q, H_kv, d, dtype, scale);
  if (rc != ATTN_OK) return rc;
  const bool q8 = cq.kind != attn::kKV16;
  if (q8) {
    if (!(dtype == ATTN_F16 || dtype == ATTN_BF16) || !(d == 64 || d == 128))
      return fail(ATTN_ERR_UNSUPPORTED, "%s: f16/bf16 queries with d = 64 or 128 only", fn);
    if (!(scale > 0.f)) return fail(ATTN_ERR_UNSUPPORTED, "%s: scale must be positive", fn);
  }
  if (cq.kind == attn::kKVFp8) {
    if (!std::isfinite(cq.k_scale) || !std::isfinite(cq.v_scale) || !(cq.k_scale > 0.f) || !(cq.v_scale > 0.f))
      return fail(ATTN_ERR_INVALID_ARG, "%s: k_scale and v_scale must be finite and positive", fn);
  }
  if (cq.kind == attn::kKVInt8 || cq.kind == attn::kKVInt4) {
    if (!cq.k_scales || !cq.v_scales) return fail(ATTN_ERR_INVALID_ARG, "%s: null scale array", fn);
    if (!aligned16(cq.k_scales) || !aligned16(cq.v_scales))
      return fail(ATTN_ERR_INVALID_ARG, "%s: scale arrays must be 16-byte aligned", fn);
  }
  if (capacity < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: cache capacity must be >= 1", fn);
  const size_t need = workspace_bytes(B, H_q, capacity, d);
  if (!workspace || workspace_bytes_given < need)
    return fail(ATTN_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need, workspace_bytes_given);
  if (!aligned16(workspace) || (lse && !aligned16(lse)))
    return fail(ATTN_ERR_INVALID_ARG, "%s: workspace and lse must be 16-byte aligned", fn);
  const int S = splits_for(capacity);
  const WorkspaceLayout lay = workspace_layout(B, H_q, capacity, d);
  attn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.table = table;
  a.seq_lens = seq_lens;
  a.part_o = static_cast<float*>(workspace);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.lse_off);
  a.B = B;
  a.H_q = H_q;
  a.H_kv = H_kv;
  a.capacity = capacity;
  a.max_blocks_per_seq = mbps;
  a.num_blocks = num_blocks;
  a.s_max = S;
  a.scale_log2 = scale * (cq.kind == attn::kKVFp8 ? cq.k_scale : 1.f) * attn::kLog2e;
  a.out_fp32 = out_fp32 != 0;
  int32_t* cnt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + lay.cnt_off);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (q8) {
    return dtype == ATTN_BF16 ? decode_q8_dispatch<attn::BF16>(a, o, lse, d, cq, cnt, st)
                              : decode_q8_dispatch<attn::F16>(a, o, lse, d, cq, cnt, st);
  }
  return paged ? decode_dispatch<true>(a, o, lse, d, dtype, scale, cnt, st)
               : decode_dispatch<false>(a, o, lse, d, dtype, scale, cnt, st);
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, const int32_t* seq_lens, void* o,
                float* lse, int B, int H_q, int H_kv, int max_len, int d, float scale, int dtype, int out_fp32,
                void* workspace, size_t workspace_bytes_given, void* stream) {
  return decode_common("attn_decode", false, q, k_cache, v_cache, nullptr, seq_lens, o, lse, B, H_q, H_kv, max_len,
                       0, 0, d, scale, dtype, out_fp32, workspace, workspace_bytes_given, stream);
}

int attn_decode_paged(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                      const int32_t* seq_lens, void* o, float* lse, int B, int H_q, int H_kv, int d, int block_size,
                      int max_blocks_per_seq, int num_blocks, float scale, int dtype, int out_fp32,
                      void* workspace, size_t workspace_bytes_given, void* stream) {
  if (!block_table) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged: null block table");
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged: block_size must be 16 (got %d)", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged: max_blocks_per_seq and num_blocks must be >= 1");
  if ((long long)max_blocks_per_seq * 16 > 0x7FFFFFFFLL)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged: max_blocks_per_seq too large");
  return decode_common("attn_decode_paged", true, q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H_q, H_kv,
                       max_blocks_per_seq * 16, max_blocks_per_seq, num_blocks, d, scale, dtype, out_fp32,
                       workspace, workspace_bytes_given, stream);
}

int attn_decode_paged_fp8(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                          const int32_t* seq_lens, void* o, float* lse, int B, int H_q, int H_kv, int d,
                          int block_size, int max_blocks_per_seq, int num_blocks, float scale, float k_scale,
                          float v_scale, int dtype, int out_fp32, void* workspace, size_t workspace_bytes_given,
                          void* stream) {
  if (!block_table) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_fp8: null block table");
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_fp8: block_size must be 16 (got %d)", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_fp8: max_blocks_per_seq and num_blocks must be >= 1");
  if ((long long)max_blocks_per_seq * 16 > 0x7FFFFFFFLL)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_fp8: max_blocks_per_seq too large");
  CacheQuant cq;
  cq.kind = attn::kKVFp8;
  cq.k_scale = k_scale;
  cq.v_scale = v_scale;
  return decode_common("attn_decode_paged_fp8", true, q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H_q,
                       H_kv, max_blocks_per_seq * 16, max_blocks_per_seq, num_blocks, d, scale, dtype, out_fp32,
                       workspace, workspace_bytes_given, stream, cq);
}

int attn_decode_paged_int8(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, void* o, float* lse, int B, int H_q, int H_kv, int d,
                           int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                           const float* k_scales, const float* v_scales, int dtype, int out_fp32,
                           void* workspace, size_t workspace_bytes_given, void* stream) {
  if (!block_table) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_int8: null block table");
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_int8: block_size must be 16 (got %d)", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_int8: max_blocks_per_seq and num_blocks must be >= 1");
  if ((long long)max_blocks_per_seq * 16 > 0x7FFFFFFFLL)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_int8: max_blocks_per_seq too large");
  CacheQuant cq;
  cq.kind = attn::kKVInt8;
  cq.k_scales = k_scales;
  cq.v_scales = v_scales;
  return decode_common("attn_decode_paged_int8", true, q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H_q,
                       H_kv, max_blocks_per_seq * 16, max_blocks_per_seq, num_blocks, d, scale, dtype, out_fp32,
                       workspace, workspace_bytes_given, stream, cq);
}

int attn_decode_paged_int4(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, void* o, float* lse, int B, int H_q, int H_kv, int d,
                           int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                           const float* k_scales, const float* v_scales, int dtype, int out_fp32,
                           void* workspace, size_t workspace_bytes_given, void* stream) {
  if (!block_table) return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_int4: null block table");
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_int4: block_size must be 16 (got %d)", block_size);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_int4: max_blocks_per_seq and num_blocks must be >= 1");
  if ((long long)max_blocks_per_seq * 16 > 0x7FFFFFFFLL)
    return fail(ATTN_ERR_INVALID_ARG, "attn_decode_paged_int4: max_blocks_per_seq too large");
  CacheQuant cq;
  cq.kind = attn::kKVInt4;
  cq.k_scales = k_scales;
  cq.v_scales = v_scales;
  return decode_common("attn_decode_paged_int4", true, q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H_q,
                       H_kv, max_blocks_per_seq * 16, max_blocks_per_seq, num_blocks, d, scale, dtype, out_fp32,
                       workspace, workspace_bytes_given, stream, cq);
}

}  // extern "C"

namespace {

// mode: 0 = FP8 E4M3 (per-tensor scales), 1 = int8, 2 = int4 (per-channel scales)
int append_8bit(const char* fn, int mode, void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                const int32_t* cache_lens, const int32_t* block_table, int B, int H_kv, int n_new, int d,
                int block_size, int max_blocks_per_seq, int num_blocks, int dtype, float k_scale, float v_scale,
                const float* k_scales, const float* v_scales, void* stream) {
  if (!k_pool || !v_pool || !k_new || !v_new || !cache_lens || !block_table)
    return fail(ATTN_ERR_INVALID_ARG, "%s: null pointer", fn);
  if (B < 1 || H_kv < 1 || n_new < 1) return fail(ATTN_ERR_INVALID_ARG, "%s: B, H_kv, n_new must be >= 1", fn);
  if (!valid_dtype(dtype)) return fail(ATTN_ERR_UNSUPPORTED, "%s: dtype %d not supported", fn, dtype);
  if (!plain_head_dim(d)) return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d not supported", fn, d);
  if (block_size != 16) return fail(ATTN_ERR_UNSUPPORTED, "%s: block_size must be 16 (got %d)", fn, block_size);
  if (mode == 2 && d % 32 != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d not supported (int4 V pairs channel groups: d % 32 == 0)", fn, d);
  if (max_blocks_per_seq < 1 || num_blocks < 1)
    return fail(ATTN_ERR_INVALID_ARG, "%s: max_blocks_per_seq and num_blocks must be >= 1", fn);
  const bool i8 = mode != 0;
  if (i8) {
    if (!k_scales || !v_scales) return fail(ATTN_ERR_INVALID_ARG, "%s: null scale array", fn);
    if (!aligned16(k_scales) || !aligned16(v_scales))
      return fail(ATTN_ERR_INVALID_ARG, "%s: scale arrays must be 16-byte aligned", fn);
  } else if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f)) {
    return fail(ATTN_ERR_INVALID_ARG, "%s: k_scale and v_scale must be finite and positive", fn);
  }
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(ATTN_ERR_INVALID_ARG, "%s: tensors must be 16-byte aligned", fn);
  attn::Append8Args a{static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), k_new, v_new, cache_lens,
                      block_table, B, H_kv, n_new, d, max_blocks_per_seq, num_blocks,
                      i8 ? 1.f : 1.0f / k_scale, i8 ? 1.f : 1.0f / v_scale, k_scales, v_scales};
  const long long threads = (long long)B * H_kv * n_new * (d / (mode == 2 ? 32 : 8));
  const dim3 grid((unsigned)((threads + 255) / 256));
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (mode == 2) {
    switch (dtype) {
      case ATTN_F32: hipLaunchKernelGGL((attn::kv_append_int4_kernel<attn::F32>), grid, dim3(256), 0, st, a); break;
      case ATTN_F16: hipLaunchKernelGGL((attn::kv_append_int4_kernel<attn::F16>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((attn::kv_append_int4_kernel<attn::BF16>), grid, dim3(256), 0, st, a); break;
    }
  } else if (i8) {
    switch (dtype) {
      case ATTN_F32: hipLaunchKernelGGL((attn::kv_append_8bit_kernel<attn::F32, true>), grid, dim3(256), 0, st, a); break;
      case ATTN_F16: hipLaunchKernelGGL((attn::kv_append_8bit_kernel<attn::F16, true>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((attn::kv_append_8bit_kernel<attn::BF16, true>), grid, dim3(256), 0, st, a); break;
    }
  } else {
    switch (dtype) {
      case ATTN_F32: hipLaunchKernelGGL((attn::kv_append_8bit_kernel<attn::F32, false>), grid, dim3(256), 0, st, a); break;
      case ATTN_F16: hipLaunchKernelGGL((attn::kv_append_8bit_kernel<attn::F16, false>), grid, dim3(256), 0, st, a); break;
      default: hipLaunchKernelGGL((attn::kv_append_8bit_kernel<attn::BF16, false>), grid, dim3(256), 0, st, a); break;
    }
  }
  return launch_status(fn);
}

}  // namespace

extern "C" {

int kv_append_fp8(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* cache_lens,
                  const int32_t* block_table, int B, int H_kv, int n_new, int d, int block_size,
                  int max_blocks_per_seq, int num_blocks, int dtype, float k_scale, float v_scale, void* stream) {
  return append_8bit("kv_append_fp8", 0, k_pool, v_pool, k_new, v_new, cache_lens, block_table, B, H_kv, n_new,
                     d, block_size, max_blocks_per_seq, num_blocks, dtype, k_scale, v_scale, nullptr, nullptr,
                     stream);
}

int kv_append_int8(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* cache_lens,
                   const int32_t* block_table, int B, int H_kv, int n_new, int d, int block_size,
                   int max_blocks_per_seq, int num_blocks, int dtype, const float* k_scales,
                   const float* v_scales, void* stream) {
  return append_8bit("kv_append_int8", 1, k_pool, v_pool, k_new, v_new, cache_lens, block_table, B, H_kv, n_new,
                     d, block_size, max_blocks_per_seq, num_blocks, dtype, 1.f, 1.f, k_scales, v_scales, stream);
}

int kv_append_int4(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* cache_lens,
                   const int32_t* block_table, int B, int H_kv, int n_new, int d, int block_size,
                   int max_blocks_per_seq, int num_blocks, int dtype, const float* k_scales,
                   const float* v_scales, void* stream) {
  return append_8bit("kv_append_int4", 2, k_pool, v_pool, k_new, v_new, cache_lens, block_table, B, H_kv, n_new,
                     d, block_size, max_blocks_per_seq, num_blocks, dtype, 1.f, 1.f, k_scales, v_scales, stream);
}

int kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int n_pairs, int H_kv, int d, int block_size,
                   int num_blocks, int elem_bytes, void* stream) {
  if (n_pairs == 0) return ok();
  if (!k_pool || !v_pool || !pairs) return fail(ATTN_ERR_INVALID_ARG, "kv_copy_blocks: null pointer");
  if (n_pairs < 0 || n_pairs > 65535)
    return fail(ATTN_ERR_INVALID_ARG, "kv_copy_blocks: n_pairs must be in [0, 65535] (got %d)", n_pairs);
  if (H_kv < 1 || num_blocks < 1) return fail(ATTN_ERR_INVALID_ARG, "kv_copy_blocks: H_kv, num_blocks must be >= 1");
  if (block_size != 16)
    return fail(ATTN_ERR_UNSUPPORTED, "kv_copy_blocks: block_size must be 16 (got %d)", block_size);
  if (!plain_head_dim(d)) return fail(ATTN_ERR_UNSUPPORTED, "kv_copy_blocks: head dim %d not supported", d);
  if (!(elem_bytes == 1 || elem_bytes == 2 || elem_bytes == 4))
    return fail(ATTN_ERR_UNSUPPORTED, "kv_copy_blocks: elem_bytes must be 1, 2 or 4 (got %d)", elem_bytes);
  if (!aligned16(k_pool) || !aligned16(v_pool) || (reinterpret_cast<uintptr_t>(pairs) & 7u))
    return fail(ATTN_ERR_INVALID_ARG, "kv_copy_blocks: pools must be 16-byte and pairs 8-byte aligned");
  const int64_t chunks = (int64_t)H_kv * 16 * d * elem_bytes / 16;
  attn::CopyBlocksArgs a{static_cast<uint4*>(k_pool), static_cast<uint4*>(v_pool), pairs, chunks, num_blocks};
  const int64_t gx = std::min<int64_t>((chunks + 255) / 256, 64);
  hipLaunchKernelGGL(attn::kv_copy_blocks_kernel, dim3((unsigned)gx, (unsigned)n_pairs), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  return launch_status("kv_copy_blocks");
}

// ---- host block pool -------------------------------------------------------

attn_block_pool* attn_block_pool_create(int num_blocks) {
  if (num_blocks < 1) {
    fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_create: num_blocks must be >= 1 (got %d)", num_blocks);
    return nullptr;
  }
  try {
    auto* p = reinterpret_cast<attn_block_pool*>(new attn::BlockPool(num_blocks));
    ok();
    return p;
  } catch (...) {
    fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_create: out of host memory");
    return nullptr;
  }
}

void attn_block_pool_destroy(attn_block_pool* pool) { delete reinterpret_cast<attn::BlockPool*>(pool); }

int attn_block_pool_free_blocks(const attn_block_pool* pool) {
  if (!pool) return -1;
  return (int)reinterpret_cast<const attn::BlockPool*>(pool)->free_stack.size();
}

int attn_block_pool_holders(const attn_block_pool* pool, int block) {
  if (!pool) return -1;
  const auto* p = reinterpret_cast<const attn::BlockPool*>(pool);
  if (block < 0 || block >= p->num_blocks()) return -1;
  return p->holders[block];
}

int attn_block_pool_reserve(attn_block_pool* pool, int32_t* row, int max_blocks, int cur_len, int new_len,
                            int32_t* copy_pair) {
  if (!pool || !row || !copy_pair) return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_reserve: null pointer");
  auto* p = reinterpret_cast<attn::BlockPool*>(pool);
  if (max_blocks < 1 || cur_len < 0 || new_len < cur_len || attn::pool_blocks_for(new_len) > max_blocks)
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_reserve: need 0 <= cur_len (%d) <= new_len (%d) <= 16 * %d",
                cur_len, new_len, max_blocks);
  if (!p->row_ok(row, cur_len))
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_reserve: the row's first %d entries are not held blocks",
                attn::pool_blocks_for(cur_len));
  const int have = attn::pool_blocks_for(cur_len), want = attn::pool_blocks_for(new_len);
  const bool cow = new_len > cur_len && cur_len % attn::kPoolBlockTokens != 0 && p->holders[row[have - 1]] > 1;
  const int need = want - have + (cow ? 1 : 0);
  if (need > (int)p->free_stack.size())
    return fail(ATTN_ERR_NO_BLOCKS, "attn_block_pool_reserve: %d blocks needed, %d free", need,
                (int)p->free_stack.size());
  copy_pair[0] = copy_pair[1] = -1;
  if (cow) {
    const int32_t old = row[have - 1];
    const int32_t fresh = p->take();
    p->drop(old);  // another sequence still holds it
    row[have - 1] = fresh;
    copy_pair[0] = old;
    copy_pair[1] = fresh;
  }
  for (int j = have; j < want; ++j) row[j] = p->take();
  return ok();
}

int attn_block_pool_reserve_batch(attn_block_pool* pool, int32_t* table, int B, int max_blocks,
                                  const int32_t* cur_lens, const int32_t* new_lens, int32_t* copy_pairs,
                                  int* n_copies, int* n_done) {
  if (!pool || !table || !cur_lens || !new_lens || !copy_pairs || !n_copies || !n_done)
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_reserve_batch: null pointer");
  if (B < 0) return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_reserve_batch: B < 0");
  *n_copies = 0;
  *n_done = 0;
  for (int b = 0; b < B; ++b) {
    int32_t pair[2];
    const int rc = attn_block_pool_reserve(pool, table + (int64_t)b * max_blocks, max_blocks, cur_lens[b],
                                           new_lens[b], pair);
    if (rc != ATTN_OK) return rc;
    if (pair[0] >= 0) {
      copy_pairs[2 * *n_copies] = pair[0];
      copy_pairs[2 * *n_copies + 1] = pair[1];
      ++*n_copies;
    }
    *n_done = b + 1;
  }
  return ok();
}

int attn_block_pool_release(attn_block_pool* pool, int32_t* row, int max_blocks, int len) {
  if (!pool || !row) return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_release: null pointer");
  auto* p = reinterpret_cast<attn::BlockPool*>(pool);
  if (max_blocks < 1 || len < 0 || attn::pool_blocks_for(len) > max_blocks)
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_release: need 0 <= len (%d) <= 16 * %d", len, max_blocks);
  if (!p->row_ok(row, len))
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_release: the row's first %d entries are not held blocks",
                attn::pool_blocks_for(len));
  const int nb = attn::pool_blocks_for(len);
  for (int j = 0; j < nb; ++j) {
    p->drop(row[j]);
    row[j] = -1;
  }
  return ok();
}

int attn_block_pool_fork(attn_block_pool* pool, const int32_t* src, int32_t* dst, int max_blocks, int len) {
  if (!pool || !src || !dst) return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_fork: null pointer");
  auto* p = reinterpret_cast<attn::BlockPool*>(pool);
  if (max_blocks < 1 || len < 0 || attn::pool_blocks_for(len) > max_blocks)
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_fork: need 0 <= len (%d) <= 16 * %d", len, max_blocks);
  if (!p->row_ok(src, len))
    return fail(ATTN_ERR_INVALID_ARG, "attn_block_pool_fork: the source row's first %d entries are not held blocks",
                attn::pool_blocks_for(len));
  const int nb = attn::pool_blocks_for(len);
  for (int j = 0; j < nb; ++j) {
    dst[j] = src[j];
    ++p->holders[src[j]];
  }
  return ok();
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

int attn_decode_paged_noalloc(const void* q, const void* k_pool, const void* v_pool, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int B, int H_q, int H_kv, int d,
                              int block_size, int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                              int out_fp32, void* stream) {
  const char* fn = "attn_decode_paged_noalloc";
  // sizes that attn_decode_paged would reject are left to its own checks
  if (B >= 1 && H_q >= 1 && d >= 1 && max_blocks_per_seq >= 1 && (long long)max_blocks_per_seq * 16 <= 0x7FFFFFFFLL) {
    const size_t need = workspace_bytes(B, H_q, max_blocks_per_seq * 16, d);
    if (need > kScratchBytes)
      return fail(ATTN_ERR_WORKSPACE,
                  "%s: B=%d, H_q=%d, max_blocks_per_seq=%d, d=%d need %zu bytes of workspace; the library's "
                  "static scratch holds %zu (use attn_decode_paged with a caller workspace instead)",
                  fn, B, H_q, max_blocks_per_seq, d, need, kScratchBytes);
  }
  void* ws = scratch_address();
  if (!ws) return fail(ATTN_ERR_HIP, "%s: the address of the static scratch could not be obtained", fn);
  return attn_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, B, H_q, H_kv, d, block_size,
                           max_blocks_per_seq, num_blocks, scale, dtype, out_fp32, ws, kScratchBytes, stream);
}

const char* attn_version(void) { return "libattn 0.1.0 (gfx950)"; }

int attn_device_error_flags(void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return -1;
  unsigned int v = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(attn::g_device_errors), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess)
    return -1;
  const unsigned int zero = 0;
  if (hipMemcpyToSymbol(HIP_SYMBOL(attn::g_device_errors), &zero, sizeof(zero), 0, hipMemcpyHostToDevice) !=
      hipSuccess)
    return -1;
  return (int)v;
}

}  // extern "C"
