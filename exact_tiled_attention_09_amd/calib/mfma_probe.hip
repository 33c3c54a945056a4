// Matrix-core calibration for gfx950 (a standalone program, not part of
// libmiattn): the rates that bound the attention kernels, measured on the
// device the program runs on.  Prints one JSON object per measurement.
//
//  1. A stream of independent v_mfma_f32_32x32x16_bf16 with register
//     operands, accumulators in VGPRs (the compiler's form when a kernel
//     keeps at most 256 registers per wave) and in AGPRs: the practical
//     bf16 matrix rate.
//  2. Two waves per SIMD, one issuing only MFMAs and the other only vector
//     work (FMA and exp2): alone and together.  "Together" close to the
//     larger of the two means the SIMD overlaps them; close to the sum means
//     it serialises them.
//  3. One wave per SIMD issuing a fixed pattern of one MFMA (AGPR
//     accumulators) followed by independent vector instructions: how much
//     vector work a single wave hides under its own MFMAs.
//
// No memory is read; each thread writes one float of its results so that
// nothing is optimised away.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                            \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(1);                                                                         \
    }                                                                                       \
  } while (0)

__device__ __forceinline__ void operands(bf16x8& a, bf16x8& b) {
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
}

// 1 and 2: eight waves, waves w and w + 4 share SIMD w % 4.  mode bit 0: the
// MFMA waves (0-3) run, bit 1: the vector waves (4-7) run.
template <bool AGPR>
__global__ void __launch_bounds__(512, 1) two_wave(float* out, int iters, int mode) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float result = 0.f;
  if (wave < 4) {
    if (mode & 1) {
      bf16x8 a, b;
      operands(a, b);
      f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
      for (int it = 0; it < iters; ++it) {
        if constexpr (AGPR) {
          asm volatile(
              "v_mfma_f32_32x32x16_bf16 %0, %4, %5, %0\n\t"
              "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
              "v_mfma_f32_32x32x16_bf16 %2, %4, %5, %2\n\t"
              "v_mfma_f32_32x32x16_bf16 %3, %4, %5, %3"
              : "+a"(c0), "+a"(c1), "+a"(c2), "+a"(c3)
              : "v"(a), "v"(b));
        } else {
          c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
          c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
          c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
          c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
        }
      }
      // the asm MFMAs' last results are read only after their latency
      if constexpr (AGPR) asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::);
      for (int i = 0; i < 16; ++i) result += c0[i] + c1[i] + c2[i] + c3[i];
    }
  } else if (mode & 2) {
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = 0.01f * (lane + i);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_amdgcn_exp2f(x[i]) * 0.5f;
    }
    for (int i = 0; i < 8; ++i) result += x[i];
  }
  out[blockIdx.x * 512 + threadIdx.x] = result;
}

// 3: four waves, one per SIMD (the 96 KiB of LDS keep one workgroup per
// CU).  Per group: one MFMA, then NF independent FMAs and NE exp2, as
// written (one asm statement each, in program order).
template <int MF, int NF, int NE>
__global__ void __launch_bounds__(256, 1) one_wave(float* out, int iters) {
  __shared__ float pad[24 * 1024];
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
  operands(a, b);
  f32x16 c0 = {}, c1 = {};
  float x0 = lane, x1 = 1, x2 = 2, x3 = 3, x4 = 4, x5 = 5, x6 = 6, x7 = 7;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if constexpr (MF) {
        if (g & 1) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c1) : "v"(a), "v"(b));
        else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c0) : "v"(a), "v"(b));
      }
      if constexpr (NF >= 4)
        asm volatile("v_fma_f32 %0, %0, %4, 1.0\n\tv_fma_f32 %1, %1, %4, 1.0\n\t"
                     "v_fma_f32 %2, %2, %4, 1.0\n\tv_fma_f32 %3, %3, %4, 1.0"
                     : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3) : "v"(0.5f));
      if constexpr (NF >= 8)
        asm volatile("v_fma_f32 %0, %0, %4, 1.0\n\tv_fma_f32 %1, %1, %4, 1.0\n\t"
                     "v_fma_f32 %2, %2, %4, 1.0\n\tv_fma_f32 %3, %3, %4, 1.0"
                     : "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7) : "v"(0.5f));
      if constexpr (NE >= 2) asm volatile("v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1" : "+v"(x0), "+v"(x1));
    }
  }
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::);
  float r = x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i];
  pad[threadIdx.x] = r;
  __syncthreads();
  out[blockIdx.x * 256 + threadIdx.x] = pad[(threadIdx.x + 1) & 255];
}

template <typename F>
static float best_ms(F launch) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  float best = 1e30f;
  for (int rep = 0; rep < 4; ++rep) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    best = std::min(best, ms);
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best;
}

int main() {
  hipDeviceProp_t prop;
  CHECK(hipGetDeviceProperties(&prop, 0));
  const int cus = prop.multiProcessorCount;
  const double peak = cus * 4.0 * 1024.0 * prop.clockRate * 1e3 / 1e12;  // 1024 bf16 FLOP/clk/SIMD
  std::printf("{\"device\": \"%s\", \"cus\": %d, \"max_clock_mhz\": %.0f, \"bf16_dense_peak_tflops\": %.1f}\n",
              prop.gcnArchName, cus, prop.clockRate / 1e3, peak);
  float* out = nullptr;
  const int blocks2 = cus * 4, iters2 = 4096;
  CHECK(hipMalloc(&out, (size_t)blocks2 * 512 * sizeof(float)));
  const double flop2 = (double)blocks2 * 4 * iters2 * 4 * 32768.0;
  for (int agpr = 0; agpr < 2; ++agpr) {
    float t[4] = {};
    for (int mode = 1; mode <= 3; ++mode) {
      t[mode] = best_ms([&] {
        if (agpr) hipLaunchKernelGGL(two_wave<true>, dim3(blocks2), dim3(512), 0, 0, out, iters2, mode);
        else hipLaunchKernelGGL(two_wave<false>, dim3(blocks2), dim3(512), 0, 0, out, iters2, mode);
      });
    }
    std::printf("{\"probe\": \"two waves per SIMD\", \"accumulators\": \"%s\", \"mfma_only_ms\": %.4f, "
                "\"mfma_tflops\": %.1f, \"pct_of_peak\": %.1f, \"vector_only_ms\": %.4f, \"both_ms\": %.4f, "
                "\"sum_ms\": %.4f, \"max_ms\": %.4f}\n",
                agpr ? "AGPR" : "VGPR", t[1], flop2 / t[1] / 1e9, 100.0 * flop2 / t[1] / 1e9 / peak, t[2], t[3],
                t[1] + t[2], std::max(t[1], t[2]));
  }
  const int blocks1 = cus * 2, iters1 = 2048;
  auto one = [&](auto k) {
    return best_ms([&] { hipLaunchKernelGGL(k, dim3(blocks1), dim3(256), 0, 0, out, iters1); });
  };
  const float m = one(one_wave<1, 0, 0>);
  const double flop1 = (double)blocks1 * 4 * iters1 * 8 * 32768.0;
  struct Row { const char* name; float vec, both; };
  const Row rows[] = {
      {"4 FMA", one(one_wave<0, 4, 0>), one(one_wave<1, 4, 0>)},
      {"8 FMA", one(one_wave<0, 8, 0>), one(one_wave<1, 8, 0>)},
      {"2 exp2", one(one_wave<0, 0, 2>), one(one_wave<1, 0, 2>)},
      {"4 FMA + 2 exp2", one(one_wave<0, 4, 2>), one(one_wave<1, 4, 2>)},
  };
  for (const Row& r : rows)
    std::printf("{\"probe\": \"one wave per SIMD\", \"per_mfma\": \"%s\", \"mfma_only_ms\": %.4f, "
                "\"mfma_tflops\": %.1f, \"vector_only_ms\": %.4f, \"both_ms\": %.4f}\n",
                r.name, m, flop1 / m / 1e9, r.vec, r.both);
  CHECK(hipFree(out));
  return 0;
}
