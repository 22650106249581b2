// Sustained bf16 MFMA throughput of the device, for the roofline of the step
// kernel: every wave issues v_mfma_f32_32x32x16_bf16 back to back on register
// operands (four independent accumulators, no memory traffic in the loop),
// optionally each followed by independent v_fma_f32, or by the step
// kernel's softmax instruction mix.  The figure it prints is the dense bf16
// rate the chip sustains under load, next to the published 2516.6 TFLOP/s.
//
// Build: part of long_sequence_causal_cp_amd.build (hipcc, gfx950).
// Run:   long_sequence_causal_cp_amd/mfma_ceiling
// Every loop is bounded; the one store per lane is in bounds.
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kIters = 4000;
constexpr double kFlopPerMfma = 2.0 * 32 * 32 * 16;

#define CEIL_MFMA "v_mfma_f32_32x32x16_bf16 %0, %9, %10, %0\n"
#define CEIL_FMA(i) "v_fma_f32 %" #i ", %" #i ", %11, %12\n"
#define CEIL_OUTS(c) "+v"(c), "+v"(f0), "+v"(f1), "+v"(f2), "+v"(f3), "+v"(f4), "+v"(f5), "+v"(f6), "+v"(f7)
#define CEIL_INS "v"(a), "v"(b), "v"(m), "v"(ad)

// One MFMA and NF independent FMAs, in this order (one asm block, so the
// compiler cannot regroup them).
// NF = -1: the step kernel's softmax mix per MFMA instead of plain FMAs: one
// FMA (scale and shift), one exp2, one add (row sum) and, every second MFMA,
// one bf16 pack of two values.
#define CEIL_SOFTMAX "v_fma_f32 %1, %1, %11, %12\nv_exp_f32 %2, %1\nv_add_f32 %3, %3, %2\n"
#define CEIL_PACK "v_cvt_pk_bf16_f32 %4, %2, %3\n"

template <int NF>
__device__ __forceinline__ void mfma_step(f32x16& c, const bf16x8& a, const bf16x8& b, float& f0, float& f1, float& f2,
                                          float& f3, float& f4, float& f5, float& f6, float& f7, float m, float ad) {
  if constexpr (NF == 0) asm volatile(CEIL_MFMA : CEIL_OUTS(c) : CEIL_INS);
  if constexpr (NF == -1) {
    asm volatile(CEIL_MFMA CEIL_SOFTMAX : CEIL_OUTS(c) : CEIL_INS);
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %9, %10, %0\n"
                 "v_fma_f32 %5, %5, %11, %12\nv_exp_f32 %6, %5\nv_add_f32 %7, %7, %6\n" CEIL_PACK
                 : CEIL_OUTS(c)
                 : CEIL_INS);
  }
  if constexpr (NF == 4) asm volatile(CEIL_MFMA CEIL_FMA(1) CEIL_FMA(2) CEIL_FMA(3) CEIL_FMA(4) : CEIL_OUTS(c) : CEIL_INS);
  if constexpr (NF == 8)
    asm volatile(CEIL_MFMA CEIL_FMA(1) CEIL_FMA(2) CEIL_FMA(3) CEIL_FMA(4) CEIL_FMA(5) CEIL_FMA(6) CEIL_FMA(7)
                     CEIL_FMA(8)
                 : CEIL_OUTS(c)
                 : CEIL_INS);
}

template <int NF>
__global__ void __launch_bounds__(256) ceiling_kernel(float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.01f * (float)((lane * 7 + i * 13) % 97) - 0.48f);
    b[i] = (__bf16)(0.01f * (float)((lane * 11 + i * 5) % 89) - 0.44f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  float f0 = lane, f1 = lane + 1, f2 = lane + 2, f3 = lane + 3, f4 = lane + 4, f5 = lane + 5, f6 = lane + 6,
        f7 = lane + 7;
  const float m = 0.999f, ad = 0.5f;
  for (int it = 0; it < kIters; ++it) {
    mfma_step<NF>(c0, a, b, f0, f1, f2, f3, f4, f5, f6, f7, m, ad);
    mfma_step<NF>(c1, a, b, f0, f1, f2, f3, f4, f5, f6, f7, m, ad);
    mfma_step<NF>(c2, a, b, f0, f1, f2, f3, f4, f5, f6, f7, m, ad);
    mfma_step<NF>(c3, a, b, f0, f1, f2, f3, f4, f5, f6, f7, m, ad);
  }
  float acc = f0 + f1 + f2 + f3 + f4 + f5 + f6 + f7;
  for (int r = 0; r < 16; ++r) acc += c0[r] + c1[r] + c2[r] + c3[r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// waves_per_simd waves on every SIMD: workgroups of 4 waves, waves_per_simd per CU
template <int NF>
int run(int n_cu, int waves_per_simd, float* out) {
  const int n_wg = n_cu * waves_per_simd;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return 1;
  hipLaunchKernelGGL((ceiling_kernel<NF>), dim3(n_wg), dim3(256), 0, 0, out);  // warm-up
  if (hipEventRecord(e0, 0) != hipSuccess) return 1;
  hipLaunchKernelGGL((ceiling_kernel<NF>), dim3(n_wg), dim3(256), 0, 0, out);
  if (hipEventRecord(e1, 0) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return 1;
  float ms = 0.f;
  if (hipEventElapsedTime(&ms, e0, e1) != hipSuccess) return 1;
  const int per_call = (NF == -1) ? 2 : 1;  // MFMAs per mfma_step
  const double n_mfma = (double)n_wg * 4 * kIters * 4 * per_call;  // waves x MFMAs per wave
  const double tflops = n_mfma * kFlopPerMfma / (ms * 1e-3) / 1e12;
  const double ns_per_mfma_simd = ms * 1e6 / ((double)kIters * 4 * per_call * waves_per_simd);
  if (NF >= 0)
    std::printf("%d wave(s)/SIMD, %d FMA per MFMA: %8.3f ms  %7.1f TFLOP/s  %6.2f ns per MFMA per SIMD\n",
                waves_per_simd, NF, ms, tflops, ns_per_mfma_simd);
  else
    std::printf("%d wave(s)/SIMD, softmax mix per MFMA (fma, exp2, add, 1/2 bf16 pack): %8.3f ms  %7.1f TFLOP/s  "
                "%6.2f ns per MFMA per SIMD\n",
                waves_per_simd, ms, tflops, ns_per_mfma_simd);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return 0;
}

}  // namespace

int main() {
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0) {
    std::fprintf(stderr, "mfma_ceiling: no device\n");
    return 1;
  }
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)n_cu * 4 * 256 * sizeof(float)) != hipSuccess) {
    std::fprintf(stderr, "mfma_ceiling: hipMalloc failed\n");
    return 1;
  }
  std::printf("device compute units: %d; published dense bf16 peak: 2516.6 TFLOP/s\n", n_cu);
  int rc = 0;
  for (int w : {1, 2, 4}) rc |= run<0>(n_cu, w, out);
  for (int w : {1, 2, 4}) rc |= run<4>(n_cu, w, out);
  for (int w : {1, 2, 4}) rc |= run<8>(n_cu, w, out);
  for (int w : {1, 2, 4}) rc |= run<-1>(n_cu, w, out);
  (void)hipDeviceSynchronize();
  (void)hipFree(out);
  return rc;
}
