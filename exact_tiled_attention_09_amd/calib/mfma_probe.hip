// Matrix-core and vector-issue calibration for gfx950 (a standalone program,
// not part of libmiattn): the rates that bound the attention kernels,
// measured on the device the program runs on.  Prints one JSON object per
// measurement.  Cycle counts come from the shader clock (s_memtime through
// clock64()); every kernel runs one workgroup of eight waves per CU (a 128
// KiB LDS array keeps it alone there), waves w and w + 4 sharing SIMD w % 4.
//
//  1. clock: a stream of independent v_mfma_f32_32x32x16_bf16 per SIMD,
//     cycles per MFMA and wall time, hence the shader clock under sustained
//     matrix load (the nominal peak assumes 2.4 GHz).
//  2. accumulator chains: the same stream with 1, 2, 4 or 8 independent
//     accumulators held in VGPRs (compiler builtin) or AGPRs (inline asm),
//     one or two MFMA waves per SIMD, as a fraction of the nominal peak.
//  3. vector issue: cycles per v_fma_f32 and per v_exp_f32 (independent
//     registers), one or two waves per SIMD.
//  4. split roles: one wave per SIMD issuing only MFMAs beside one issuing
//     only vector work (FMA, exp2, or a softmax-like mix: scale-and-shift,
//     exp2, row sum and bf16 packing), alone and together.
//  5. interleaving inside a wave: one MFMA followed by 4 FMA, 2 exp2, or both,
//     one or two waves per SIMD.
// No memory is read; each thread writes one float so nothing is optimised
// away.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                            \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      std::exit(1);                                                                         \
    }                                                                                       \
  } while (0)

constexpr int kPadFloats = 32 * 1024;  // 128 KiB of LDS: one workgroup per CU

__device__ __forceinline__ void operands(bf16x8& a, bf16x8& b) {
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (lane + i));
    b[i] = (__bf16)(0.002f * (lane - i));
  }
}

// Publishes a per-thread result through LDS (keeping the workgroup's LDS
// allocation live) and the wave's cycle count.
__device__ __forceinline__ void finish(float r, long long cycles, float* out, long long* cyc, float* pad) {
  pad[threadIdx.x] = r;
  __syncthreads();
  out[blockIdx.x * 512 + threadIdx.x] = pad[(threadIdx.x + 1) & 511];
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * 8 + (threadIdx.x >> 6)] = cycles;
}

// 1 and 2: NC independent accumulators, waves 0 .. 4 W - 1 issue MFMAs.
template <int NC, bool AGPR>
__global__ void __launch_bounds__(512, 1) chains(float* out, long long* cyc, int iters, int waves_per_simd) {
  __shared__ float pad[kPadFloats];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float r = 0.f;
  long long t = 0;
  if (wave < 4 * waves_per_simd) {
    bf16x8 a, b;
    operands(a, b);
    f32x16 c[NC];
    for (int j = 0; j < NC; ++j) c[j] = f32x16{};
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int rep = 0; rep < 8 / NC; ++rep)
#pragma unroll
        for (int j = 0; j < NC; ++j) {
          if constexpr (AGPR) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c[j]) : "v"(a), "v"(b));
          else c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
        }
    }
    // the asm MFMAs' last results are read only after their latency
    if constexpr (AGPR) asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::);
    t = clock64() - t0;
    for (int j = 0; j < NC; ++j)
      for (int i = 0; i < 16; ++i) r += c[j][i];
  }
  finish(r, t, out, cyc, pad);
}

// Vector work units (one asm statement each, independent registers).
// MIX 0: 8 v_fma_f32; 1: 8 v_exp_f32; 2: softmax-like, 8 scores through
// scale-and-shift, exp2, row sum and bf16 packing.
template <int MIX>
__device__ __forceinline__ void vec_unit(float (&x)[8], float& acc, uint32_t (&pk)[4]) {
  if constexpr (MIX == 0) {
    asm volatile("v_fma_f32 %0, %0, %8, 1.0\n\tv_fma_f32 %1, %1, %8, 1.0\n\tv_fma_f32 %2, %2, %8, 1.0\n\t"
                 "v_fma_f32 %3, %3, %8, 1.0\n\tv_fma_f32 %4, %4, %8, 1.0\n\tv_fma_f32 %5, %5, %8, 1.0\n\t"
                 "v_fma_f32 %6, %6, %8, 1.0\n\tv_fma_f32 %7, %7, %8, 1.0"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7])
                 : "v"(0.5f));
  } else if constexpr (MIX == 1) {
    asm volatile("v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
                 "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7"
                 : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]), "+v"(x[7]));
  } else {
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], 0.999f, -0.5f));
      acc += e[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      pk[i] ^= __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){e[2 * i], e[2 * i + 1]}, bf16x2));
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = e[i] - 0.25f;
  }
}

// 3: waves 0 .. 4 W - 1 run vec_unit<MIX>, four units per iteration.
template <int MIX>
__global__ void __launch_bounds__(512, 1) vector_rate(float* out, long long* cyc, int iters, int waves_per_simd) {
  __shared__ float pad[kPadFloats];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float r = 0.f;
  long long t = 0;
  if (wave < 4 * waves_per_simd) {
    float x[8], acc = 0.f;
    uint32_t pk[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 8; ++i) x[i] = 0.01f * (lane + i) - 1.0f;
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 4; ++u) vec_unit<MIX>(x, acc, pk);
    }
    t = clock64() - t0;
    for (int i = 0; i < 8; ++i) r += x[i];
    r += acc + (float)(pk[0] ^ pk[1] ^ pk[2] ^ pk[3]);
  }
  finish(r, t, out, cyc, pad);
}

// 4: waves 0-3 issue only MFMAs (4 VGPR accumulators per iteration), waves
// 4-7 only vec_unit<MIX> (four units per iteration); role bit 0 runs the MFMA
// waves, bit 1 the vector waves.
template <int MIX>
__global__ void __launch_bounds__(512, 1) split_roles(float* out, long long* cyc, int mfma_iters, int vec_iters,
                                                      int role) {
  __shared__ float pad[kPadFloats];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float r = 0.f;
  long long t = 0;
  if (wave < 4) {
    if (role & 1) {
      bf16x8 a, b;
      operands(a, b);
      f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
      const long long t0 = clock64();
      for (int it = 0; it < mfma_iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
      }
      t = clock64() - t0;
      for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
    }
  } else if (role & 2) {
    float x[8], acc = 0.f;
    uint32_t pk[4] = {0u, 0u, 0u, 0u};
    for (int i = 0; i < 8; ++i) x[i] = 0.01f * (lane + i) - 1.0f;
    const long long t0 = clock64();
    for (int it = 0; it < vec_iters; ++it) {
#pragma unroll
      for (int u = 0; u < 4; ++u) vec_unit<MIX>(x, acc, pk);
    }
    t = clock64() - t0;
    for (int i = 0; i < 8; ++i) r += x[i];
    r += acc + (float)(pk[0] ^ pk[1] ^ pk[2] ^ pk[3]);
  }
  finish(r, t, out, cyc, pad);
}

// 5: one MFMA (AGPR accumulator) then NF independent FMAs and NE exp2, as
// one asm statement, four times per iteration.
template <int NF, int NE>
__global__ void __launch_bounds__(512, 1) interleave(float* out, long long* cyc, int iters, int waves_per_simd) {
  __shared__ float pad[kPadFloats];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  float r = 0.f;
  long long t = 0;
  if (wave < 4 * waves_per_simd) {
    bf16x8 a, b;
    operands(a, b);
    f32x16 c = {};
    float x0 = lane, x1 = 1, x2 = 2, x3 = 3, x4 = 4, x5 = 5;
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (NF == 4 && NE == 2)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %7, %8, %0\n\tv_fma_f32 %1, %1, %9, 1.0\n\t"
                       "v_fma_f32 %2, %2, %9, 1.0\n\tv_fma_f32 %3, %3, %9, 1.0\n\tv_fma_f32 %4, %4, %9, 1.0\n\t"
                       "v_exp_f32 %5, %5\n\tv_exp_f32 %6, %6"
                       : "+a"(c), "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5)
                       : "v"(a), "v"(b), "v"(0.5f));
        else if constexpr (NF == 4)
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0\n\tv_fma_f32 %1, %1, %7, 1.0\n\t"
                       "v_fma_f32 %2, %2, %7, 1.0\n\tv_fma_f32 %3, %3, %7, 1.0\n\tv_fma_f32 %4, %4, %7, 1.0"
                       : "+a"(c), "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3) : "v"(a), "v"(b), "v"(0.5f));
        else
          asm volatile("v_mfma_f32_32x32x16_bf16 %0, %3, %4, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2"
                       : "+a"(c), "+v"(x4), "+v"(x5) : "v"(a), "v"(b));
      }
    }
    asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15" ::);
    t = clock64() - t0;
    r = x0 + x1 + x2 + x3 + x4 + x5;
    for (int i = 0; i < 16; ++i) r += c[i];
  }
  finish(r, t, out, cyc, pad);
}

struct Result {
  float ms;
  double cyc_lo, cyc_hi;  // largest cycle count among waves 0-3 and 4-7
};

template <typename F>
static Result launch_best(int blocks, float* out, long long* cyc, long long* host, F launch) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  Result best{1e30f, 0, 0};
  for (int rep = 0; rep < 3; ++rep) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    CHECK(hipMemcpy(host, cyc, (size_t)blocks * 8 * sizeof(long long), hipMemcpyDeviceToHost));
    long long lo = 0, hi = 0;
    for (int i = 0; i < blocks * 8; ++i) {
      if ((i & 7) < 4) lo = std::max(lo, host[i]);
      else hi = std::max(hi, host[i]);
    }
    if (ms < best.ms) best = {ms, (double)lo, (double)hi};
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
  const int blocks = cus;
  float* out = nullptr;
  long long* cyc = nullptr;
  CHECK(hipMalloc(&out, (size_t)blocks * 512 * sizeof(float)));
  CHECK(hipMalloc(&cyc, (size_t)blocks * 8 * sizeof(long long)));
  long long* host = (long long*)std::malloc((size_t)blocks * 8 * sizeof(long long));
  const int iters = 2048;  // 8 MFMAs per iteration

  // 1 and 2
  auto chain_line = [&](auto kern, const char* form, int nc, int w) {
    const Result r = launch_best(blocks, out, cyc, host, [&] {
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), 0, 0, out, cyc, iters, w);
    });
    const double mfmas = 8.0 * iters;  // per wave
    const double flop = (double)blocks * 4 * w * mfmas * 32768.0;
    const double c = std::max(r.cyc_lo, r.cyc_hi);  // the slowest wave: all MFMAs of its SIMD are done
    std::printf("{\"probe\": \"accumulator chains\", \"accumulators\": \"%s\", \"chains\": %d, \"mfma_waves_per_simd\": %d, "
                "\"ms\": %.4f, \"pct_of_peak\": %.1f, \"simd_cycles_per_mfma\": %.2f, \"shader_clock_mhz\": %.0f}\n",
                form, nc, w, r.ms, 100.0 * flop / r.ms / 1e9 / peak, c / (mfmas * w), c / (r.ms * 1e3));
  };
  chain_line(chains<4, true>, "AGPR", 4, 1);
  for (int w = 1; w <= 2; ++w) {
    chain_line(chains<1, false>, "VGPR", 1, w);
    chain_line(chains<2, false>, "VGPR", 2, w);
    chain_line(chains<4, false>, "VGPR", 4, w);
    chain_line(chains<8, false>, "VGPR", 8, w);
    chain_line(chains<1, true>, "AGPR", 1, w);
    chain_line(chains<2, true>, "AGPR", 2, w);
    chain_line(chains<8, true>, "AGPR", 8, w);
  }

  // 3
  auto vec_line = [&](auto kern, const char* what, int per_iter, int w) {
    const int vi = 256;
    const Result r = launch_best(blocks, out, cyc, host, [&] {
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), 0, 0, out, cyc, vi, w);
    });
    const double c = std::max(r.cyc_lo, r.cyc_hi) / vi / (4 * per_iter);
    std::printf("{\"probe\": \"vector issue\", \"instruction\": \"%s\", \"waves_per_simd\": %d, "
                "\"cycles_per_instruction_per_wave\": %.2f, \"simd_cycles_per_instruction\": %.2f}\n",
                what, w, c, c / w);
  };
  for (int w = 1; w <= 2; ++w) {
    vec_line(vector_rate<0>, "v_fma_f32", 8, w);
    vec_line(vector_rate<1>, "v_exp_f32", 8, w);
  }

  // 4
  auto split_line = [&](auto kern, const char* mix, int vec_iters) {
    const int mi = 2048;  // 4 MFMAs per iteration
    double alone_m = 0, alone_v = 0;
    for (int role = 1; role <= 3; ++role) {
      const Result r = launch_best(blocks, out, cyc, host, [&] {
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), 0, 0, out, cyc, mi, vec_iters, role);
      });
      if (role == 1) alone_m = r.cyc_lo;
      if (role == 2) alone_v = r.cyc_hi;
      if (role == 3)
        std::printf("{\"probe\": \"split roles\", \"vector_wave\": \"%s\", \"cycles_per_mfma_alone\": %.2f, "
                    "\"cycles_per_mfma_beside_vector_wave\": %.2f, \"vector_cycles_per_unit_alone\": %.2f, "
                    "\"vector_cycles_per_unit_beside_mfma_wave\": %.2f}\n",
                    mix, alone_m / (4.0 * mi), r.cyc_lo / (4.0 * mi), alone_v / (4.0 * vec_iters),
                    r.cyc_hi / (4.0 * vec_iters));
    }
  };
  split_line(split_roles<0>, "8 FMA per unit", 256);
  split_line(split_roles<1>, "8 exp2 per unit", 128);
  split_line(split_roles<2>, "softmax of 8 scores per unit", 128);

  // 5
  auto inter_line = [&](auto kern, const char* what, int w) {
    const int ii = 1024;  // 4 MFMAs per iteration
    const Result r = launch_best(blocks, out, cyc, host, [&] {
      hipLaunchKernelGGL(kern, dim3(blocks), dim3(512), 0, 0, out, cyc, ii, w);
    });
    std::printf("{\"probe\": \"interleaved in one wave\", \"per_mfma\": \"%s\", \"waves_per_simd\": %d, "
                "\"simd_cycles_per_mfma\": %.2f}\n",
                what, w, std::max(r.cyc_lo, r.cyc_hi) / (4.0 * ii) / w);
  };
  for (int w = 1; w <= 2; ++w) {
    inter_line(interleave<4, 0>, "4 FMA", w);
    inter_line(interleave<0, 2>, "2 exp2", w);
    inter_line(interleave<4, 2>, "4 FMA + 2 exp2", w);
  }

  CHECK(hipFree(out));
  CHECK(hipFree(cyc));
  std::free(host);
  return 0;
}
