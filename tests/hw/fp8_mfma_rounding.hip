// How gfx950's FP8 matrix core sums products: v_mfma_scale_f32_32x32x64_f8f6f4 with
// E4M3 x E4M3 operands and unit block scales.
//
// Products of two E4M3 values are exact in fp32, but the instruction does not add
// them exactly: within each group of 8 consecutive bytes of a lane's 32-byte operand,
// every product is cut toward zero to a multiple of 2^(E - 13), where 2^E <= the
// group's largest |product| < 2^(E + 1); the groups are then summed.  The FP8 prefill
// test derives its per-row lse bound from this rule (test_gpu_prefill_fp8.py,
// fp8_mfma_logit_shift).  This program prints the cases that establish it.
//
// Build and run on a gfx950 GPU (one wave, 64-byte operands, in bounds):
//   hipcc --offload-arch=gfx950 -O2 tests/hw/fp8_mfma_rounding.hip -o fp8_mfma_rounding
//   ./fp8_mfma_rounding
// Expected: a product below the group's granule is lost only in bytes 0..7 of lane
// half 0 (the group of the large product), for either sign; products 1.0 .. 0.5 beside
// 448^2 (granule 16) vanish; beside 32^2 (granule 1/8) 0.125 survives and 0.0625 does not.
#include <hip/hip_runtime.h>
#include <cmath>
#include <cstdio>

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void dot_kernel(const unsigned char* a, const unsigned char* b, float* out) {
  const int l = threadIdx.x;  // one wave: lane l holds bytes 32 (l / 32) .. + 31 of a and b
  i32x8 A, B;
  for (int i = 0; i < 8; ++i) {
    A[i] = *reinterpret_cast<const int*>(a + 32 * (l >> 5) + 4 * i);
    B[i] = *reinterpret_cast<const int*>(b + 32 * (l >> 5) + 4 * i);
  }
  f32x16 c;
  for (int i = 0; i < 16; ++i) c[i] = 0.f;
  c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 0, 0, 0, 127, 0, 127);
  out[l] = c[0];  // every output element is the same 64-term dot product
}

static double e4m3(unsigned c) {
  const int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
  const double v = e == 0 ? m * std::ldexp(1.0, -9) : (1 + m / 8.0) * std::ldexp(1.0, e - 7);
  return s ? -v : v;
}

static int run(unsigned char* da, unsigned char* db, float* dout, const unsigned char* a, const unsigned char* b,
               float* got) {
  if (hipMemcpy(da, a, 64, hipMemcpyHostToDevice) != hipSuccess) return 1;
  if (hipMemcpy(db, b, 64, hipMemcpyHostToDevice) != hipSuccess) return 1;
  hipLaunchKernelGGL(dot_kernel, dim3(1), dim3(64), 0, 0, da, db, dout);
  float h[64];
  if (hipMemcpy(h, dout, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return 1;
  *got = h[0];
  return 0;
}

int main() {
  unsigned char *da, *db;
  float* dout;
  if (hipMalloc(&da, 64) != hipSuccess || hipMalloc(&db, 64) != hipSuccess || hipMalloc(&dout, 256) != hipSuccess)
    return 1;
  unsigned char a[64], b[64];
  float got;
  // 1. one large product (code 0x7E = 448, or 0x60 = 32) beside 63 products of 1 * small
  const unsigned bigs[] = {0x7E, 0x60};
  const unsigned smalls[] = {0x30, 0x28, 0x20, 0x18};  // 0.5, 0.25, 0.125, 0.0625
  for (unsigned big : bigs)
    for (unsigned sm : smalls) {
      for (int i = 0; i < 64; ++i) a[i] = 0x38, b[i] = sm;  // 1.0 * small
      a[0] = big, b[0] = big;
      if (run(da, db, dout, a, b, &got)) return 2;
      const double exact = e4m3(big) * e4m3(big) + 63 * e4m3(sm);
      printf("big^2 %9.1f + 63 x %-7g: exact %.4f got %.4f (lost %g = %g products)\n", e4m3(big) * e4m3(big),
             e4m3(sm), exact, got, exact - got, (exact - got) / e4m3(sm));
    }
  // 2. which positions share the large product's group, and the direction of the cut
  for (unsigned sm : {0x30u, 0xB0u}) {  // +0.5, -0.5
    int lost_first = -1, lost_last = -1;
    for (int pos = 1; pos < 64; ++pos) {
      for (int i = 0; i < 64; ++i) a[i] = 0, b[i] = 0;
      a[0] = 0x7E, b[0] = 0x7E, a[pos] = 0x38, b[pos] = sm;
      if (run(da, db, dout, a, b, &got)) return 2;
      if (got == 200704.0f) {
        if (lost_first < 0) lost_first = pos;
        lost_last = pos;
      }
    }
    printf("a product of %+g beside 448^2 is lost at byte positions %d .. %d of 63\n", e4m3(sm), lost_first,
           lost_last);
  }
  return 0;
}
