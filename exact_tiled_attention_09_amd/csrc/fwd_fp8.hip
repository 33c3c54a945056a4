// FP8 (E4M3) attention forward and its quantizers ("第 18 章 FlashAttention"
// section 18.6.2: Q, K and V in FP8 E4M3 with dynamic per-block scales
// s = max|X_block| / 448 for the load blocks of Q and K, S = Q K^T and the
// softmax in fp32, O dequantized to bf16).
//
// Quantizers (HBM-bound, one pass each):
//  * rows: Q or K [B, H, N, 128] bf16 -> codes of the same shape and one fp32
//    scale per 64-row block (one workgroup per block);
//  * V: one scale per (batch, head) (per-tile maxima, their max per head,
//    then the codes; no atomics), the
//    codes stored per 64-key tile transposed, [B, H, N/64, 128, 64], with the
//    keys of a tile in the order in which a lane finds them in its score
//    accumulators, so that P needs no shuffle before the P V product.
// Conversion is the hardware's round-to-nearest-even to OCP E4M3FN.
//
// Forward: the staggered schedule of the bf16 forward (eight waves, 256
// query rows, 64-key tiles in three LDS slots filled by direct loads two
// tiles ahead) with the 32x32x64 FP8 MFMA.  The order of the 64 products
// inside one MFMA is free as long as both operands use the same one, so every
// operand is two contiguous 16-byte LDS reads: K rows (64 features per
// k-step), Q^T rows kept in registers, V^T rows of the transposed tile, and
// P^T straight from the score accumulators.  Scores are scaled by
// scale * s_q * s_k of the tile pair inside the softmax's single FMA.  P is
// rounded to E4M3 after multiplying by 2^6 with the reference max allowed to
// lag by 2 (base-2 units): P * 2^6 lies in [2^-6, 2^8] for every P >= 2^-12,
// all normal E4M3 values; the 2^6 is folded into the exponent, so l carries
// it too.  The epilogue divides by l and multiplies by the head's V scale.
#include "miattn_device.h"
#include "miattn_launch.h"

#include <type_traits>

namespace miattn {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kFp8Max = 448.0f;
constexpr float kPScaleLog2 = 6.0f;     // P is rounded to E4M3 as P * 2^6
constexpr float kLazyMaxFp8 = 2.0f;     // P <= 2^2, so P * 2^6 <= 256 < 448

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // E8M0 block scales of 127 (2^0): the plain E4M3 x E4M3 product
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Two fp32 values -> two E4M3 codes in the low (HI = false) or high half of w.
template <bool HI>
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t w) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, HI);
}

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const int addr = (int)((__lane_id() ^ (unsigned)o) << 2);
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x))));
  }
  return x;
}

// ------------------------------------------------------------------ quantizers
// x / s rounded to nearest, as the fp32 division gives it, for one scale s of
// a whole block: Markstein's correction of a reciprocal product (IBM RISC
// System/6000, 1990).  With y = RN(1/s) formed once, q = RN(x y) lies within
// an ulp of x / s, the remainder r = x - s q is exact in one fma, and
// RN(q + r y) = RN(x / s) as long as nothing underflows; so scales outside
// [2^-60, 2^60] keep the division.  A zero quotient takes x's sign, as the
// division's does.  Three instructions instead of the division's sequence.
struct DivByScale {
  float s, y;
  bool fast;
  __device__ __forceinline__ explicit DivByScale(float s_) : s(s_), y(1.f / s_), fast(s_ >= 0x1p-60f && s_ <= 0x1p60f) {}
  __device__ __forceinline__ float operator()(float x) const {
    if (!fast) return x / s;
    const float q = x * y;
    const float r = __builtin_fmaf(-q, s, x);
    return __builtin_copysignf(__builtin_fmaf(r, y, q), x);
  }
};

struct QuantArgs {
  const uint16_t* x;   // bf16 [B*H, N, D]
  uint8_t* x8;         // codes
  float* scales;
  int BH;
  int N;
};

// One workgroup (256 threads) per 64-row block of one (batch, head).
template <int D>
__global__ void __launch_bounds__(256) quant_rows_kernel(QuantArgs a, int nb) {
  constexpr int ELEMS = 64 * D;
  constexpr int PER = ELEMS / 256 / 8;   // 16-byte chunks per thread
  __shared__ float s_max[4];
  const int bh = blockIdx.x / nb;
  const int t = blockIdx.x - bh * nb;
  const int r0 = t * 64;
  const int rows = min(64, a.N - r0);
  const uint16_t* src = a.x + ((int64_t)bh * a.N + r0) * D;
  uint8_t* dst = a.x8 + ((int64_t)bh * a.N + r0) * D;
  const int tid = threadIdx.x;
  u32x4 raw[PER];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * 256 + tid;          // chunk of 8 elements
    const bool ok = c * 8 < rows * D;
    raw[i] = ok ? *(const u32x4*)(src + c * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i][w] & 0xffffu)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(raw[i][w] >> 16)));
    }
  }
  amax = wave_max64(amax);
  if ((tid & 63) == 0) s_max[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
  const float s = amax == 0.f ? 1.f : amax / kFp8Max;
  if (tid == 0) a.scales[(int64_t)bh * nb + t] = s;
  const DivByScale div(s);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * 256 + tid;
    if (c * 8 < rows * D) {
      uint32_t lo = 0u, hi = 0u;
      lo = cvt_fp8x2<false>(div(bf16_bits_to_f32(raw[i][0] & 0xffffu)), div(bf16_bits_to_f32(raw[i][0] >> 16)), lo);
      lo = cvt_fp8x2<true>(div(bf16_bits_to_f32(raw[i][1] & 0xffffu)), div(bf16_bits_to_f32(raw[i][1] >> 16)), lo);
      hi = cvt_fp8x2<false>(div(bf16_bits_to_f32(raw[i][2] & 0xffffu)), div(bf16_bits_to_f32(raw[i][2] >> 16)), hi);
      hi = cvt_fp8x2<true>(div(bf16_bits_to_f32(raw[i][3] & 0xffffu)), div(bf16_bits_to_f32(raw[i][3] >> 16)), hi);
      *(u32x2*)(dst + c * 8) = u32x2{lo, hi};
    }
  }
}

// Per-head V scale in two steps without atomics: each 64-key tile's max goes
// to the first word of that tile's region of the output codes (overwritten by
// the codes afterwards), then one wave per (batch, head) takes the max over
// its tiles and writes the scale.
template <int D>
__global__ void __launch_bounds__(256) tile_amax_kernel(QuantArgs a, int nt) {
  constexpr int PER = 64 * D / 256 / 8;
  __shared__ float s_max[4];
  const int bh = blockIdx.x / nt;
  const int t = blockIdx.x - bh * nt;
  const int rows = min(64, a.N - t * 64);
  const uint16_t* src = a.x + ((int64_t)bh * a.N + t * 64) * D;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = i * 256 + threadIdx.x;
    if (c * 8 < rows * D) {
      const u32x4 r = *(const u32x4*)(src + c * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(r[w] & 0xffffu)));
        amax = fmaxf(amax, fabsf(bf16_bits_to_f32(r[w] >> 16)));
      }
    }
  }
  amax = wave_max64(amax);
  if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = amax;
  __syncthreads();
  if (threadIdx.x == 0)
    *(float*)(a.x8 + ((int64_t)bh * nt + t) * (int64_t)D * 64) =
        fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
}

template <int D>
__global__ void __launch_bounds__(64) head_scale_kernel(QuantArgs a, int nt) {
  const int bh = blockIdx.x;  // one wave per (batch, head), lanes over tiles
  float amax = 0.f;
  for (int t = threadIdx.x; t < nt; t += 64)
    amax = fmaxf(amax, *(const float*)(a.x8 + ((int64_t)bh * nt + t) * (int64_t)D * 64));
  amax = wave_max64(amax);
  if (threadIdx.x == 0) a.scales[bh] = amax == 0.f ? 1.f : amax / kFp8Max;
}

// Codes of one 64-key tile of V, transposed: out[f * 64 + p] = code of key
// k(p) = 32 (p % 32 / 16) + 8 (p % 16 / 4) + 4 (p / 32) + p % 4, feature f.
// The tile goes through LDS (rows of D bf16 padded by 8 elements).
template <int D>
__global__ void __launch_bounds__(256) quant_vt_kernel(QuantArgs a, int nt) {
  constexpr int LD = D + 8;
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * LD];
  const int bh = blockIdx.x / nt;
  const int t = blockIdx.x - bh * nt;
  const int rows = min(64, a.N - t * 64);
  const uint16_t* src = a.x + ((int64_t)bh * a.N + t * 64) * D;
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;
  for (int c = tid; c < 64 * CPR; c += 256) {
    const int r = c / CPR, col = (c - r * CPR) * 8;
    const u32x4 v = r < rows ? *(const u32x4*)(src + r * D + col) : u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)(tile + r * LD + col) = v;
  }
  __syncthreads();
  const DivByScale div(a.scales[bh]);
  uint8_t* dst = a.x8 + ((int64_t)bh * nt + t) * (int64_t)D * 64;
  // 16 consecutive positions p0..p0+15 of one feature per thread and step,
  // one 16-byte store; each word = 4 positions p..p+3 = keys k(p)..k(p)+3
  for (int w = tid; w < D * 4; w += 256) {
    const int f = w >> 2;
    const int pb = (w & 3) * 16;
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int p0 = pb + 4 * j;
      const int k0 = 32 * ((p0 % 32) / 16) + 8 * ((p0 % 16) / 4) + 4 * (p0 / 32);
      const float x0 = div(bf16_bits_to_f32(tile[(k0 + 0) * LD + f]));
      const float x1 = div(bf16_bits_to_f32(tile[(k0 + 1) * LD + f]));
      const float x2 = div(bf16_bits_to_f32(tile[(k0 + 2) * LD + f]));
      const float x3 = div(bf16_bits_to_f32(tile[(k0 + 3) * LD + f]));
      uint32_t word = cvt_fp8x2<false>(x0, x1, 0u);
      out[j] = cvt_fp8x2<true>(x2, x3, word);
    }
    *(u32x4*)(dst + f * 64 + pb) = out;
  }
}

// -------------------------------------------------------------------- forward
template <bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_fp8_kernel(Fp8Args a, int n_qtiles) {
  constexpr int D = 128;
  constexpr int NW = 8;
  constexpr int BC = 64;
  constexpr int BR = NW * 32;
  constexpr int DB = D / 32;
  constexpr int KTILE = BC * D;          // bytes
  constexpr int VTILE = D * BC;

  __shared__ __attribute__((aligned(16))) uint8_t sK[3][KTILE];
  __shared__ __attribute__((aligned(16))) uint8_t sV[3][VTILE];
  // The per-tile K scales of the sequence, read once into LDS: read from
  // memory inside the key loop, each would make the compiler wait for every
  // load in flight there (it does not count the hand-issued tile loads).
  // Sequences of more tiles than the table holds read them from memory.
  constexpr int KSC_CAP = 2048;  // 64-key tiles (N <= 131072)
  __shared__ float s_ksc[KSC_CAP];

  int bh, tile;
  wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, CAUSAL, bh, tile);
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const int hk = h / (a.H / a.Hkv);
  const int bhk = b * a.Hkv + hk;
  const int q_tile0 = tile * BR;
  const int len = a.N;
  if (q_tile0 >= len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool late = wave >= 4;
  const int q_wave0 = q_tile0 + wave * 32;
  const int nkb = (len + 63) / 64;       // 64-row scale blocks (and V tiles)

  const uint8_t* __restrict__ qp = a.q8 + (int64_t)bh * len * D;
  const uint8_t* __restrict__ kp = a.k8 + (int64_t)bhk * len * D;
  const uint8_t* __restrict__ vp = a.v8t + (int64_t)bhk * nkb * VTILE;
  const float* __restrict__ ksc = a.k_scale + (int64_t)bhk * nkb;

  // |scale| * log2(e) * s_q of this wave's 64-row block; a negative scale
  // flips the sign of Q's codes (bit 7 of every byte).
  float c_q = fabsf(a.scale_log2) * a.q_scale[(int64_t)bh * nkb + min(q_wave0, len - 1) / 64];
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80808080u : 0u;
  i32x8 qf[2];
  {
    const int qi = min(q_wave0 + l32, len - 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint8_t* p = qp + (int64_t)qi * D + ks * 64 + hi * 32;
      const u32x4 x0 = *(const u32x4*)p;
      const u32x4 x1 = *(const u32x4*)(p + 16);
      qf[ks] = i32x8{(int)(x0[0] ^ qsign), (int)(x0[1] ^ qsign), (int)(x0[2] ^ qsign), (int)(x0[3] ^ qsign),
                     (int)(x1[0] ^ qsign), (int)(x1[1] ^ qsign), (int)(x1[2] ^ qsign), (int)(x1[3] ^ qsign)};
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int kv_end = CAUSAL ? min(len, q_tile0 + BR) : len;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int jw_last = CAUSAL ? min(ntiles - 1, (q_wave0 + 31) / BC) : ntiles - 1;
  // The K scales of the tiles this workgroup visits, before any tile load (so
  // the wait for them waits for nothing else); the prologue's barrier
  // publishes them.
  const bool ksc_lds = ntiles <= KSC_CAP;
  if (ksc_lds)
    for (int i = tid; i < ntiles; i += NW * 64) s_ksc[i] = ksc[i];

  // Direct loads: one 16-byte chunk per thread per tile and tensor.  K tile
  // rows are 128 bytes (8 chunks, chunk c of row r stored at c ^ (r/2 % 8));
  // V^T tile rows are 64 bytes (4 chunks, at c ^ (r/4 % 4)).
  // The early waves (0-3) issue every tile load: chunk p = i * 256 + tid,
  // i = 0, 1.  At this tile size the matrix phases are half as long as the
  // softmax, so loads issued after the barrier would delay the late waves'
  // softmax, the longer phase; the early waves carry them inside their
  // matrix phases instead (K_{j+3} during P_j V_j, V_{j+1} during S_j), or
  // right after the barrier when they skip a tile.
  constexpr int NTE = 256;
  int k_row[2], k_col[2], v_row[2], v_col[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int pch = i * NTE + (tid & (NTE - 1));
    k_row[i] = pch >> 3;
    k_col[i] = (((pch & 7) ^ ((k_row[i] >> 1) & 7)) << 4);
    v_row[i] = pch >> 2;
    v_col[i] = (((pch & 3) ^ ((v_row[i] >> 2) & 3)) << 4);
  }
  auto dma_k = [&](int j, int slot, int i) __attribute__((always_inline)) {
    const int key = min(j * BC + k_row[i], len - 1);
    uint32_t wb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MIATTN_LDS void*)(sK[slot] + wave * 64 * 16));
    __asm__ volatile("" : "+s"(wb));
    lds_dma16_m0(kp + (int64_t)key * D + k_col[i], wb + i * NTE * 16);
  };
  auto dma_v = [&](int j, int slot, int i) __attribute__((always_inline)) {
    uint32_t wb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MIATTN_LDS void*)(sV[slot] + wave * 64 * 16));
    __asm__ volatile("" : "+s"(wb));
    lds_dma16_m0(vp + (int64_t)j * VTILE + v_row[i] * 64 + v_col[i], wb + i * NTE * 16);
  };
  auto issue_k = [&](int j, int slot) __attribute__((always_inline)) {
    dma_k(j, slot, 0);
    dma_k(j, slot, 1);
  };
  auto issue_v = [&](int j, int slot) __attribute__((always_inline)) {
    dma_v(j, slot, 0);
    dma_v(j, slot, 1);
  };
  // operand offsets: K row kb*32 + l32, chunks 4 ks + 2 hi + {0, 1}; V^T row
  // db*32 + l32, chunks 2 hi + {0, 1}
  int koff[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r = kb * 32 + l32;
      koff[kb][ks] = r * 128 + (((4 * ks + 2 * hi) ^ ((r >> 1) & 7)) << 4);
    }
  // the second chunk: logical c + 1 sits at (c + 1) ^ x = (c ^ x) ^ 1 for even c
  int voff[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int r = db * 32 + l32;
    voff[db] = r * 64 + (((2 * hi) ^ ((r >> 2) & 3)) << 4);
  }
  auto read32 = [&](const uint8_t* base, int off) __attribute__((always_inline)) -> i32x8 {
    const u32x4 x0 = *(const u32x4*)(base + off);
    const u32x4 x1 = *(const u32x4*)(base + (off ^ 16));
    return i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };

  f32x16 s[2];
  i32x8 p8 = {};
  auto mma_s = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const uint8_t* kt = sK[SL];
    const bool ld = !late && j + 1 < ntiles;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_fp8(read32(kt, koff[kb][ks]), qf[ks], s[kb]);
      if (ld) {
        __builtin_amdgcn_sched_barrier(0);
        dma_v(j + 1, (SL + 1) % 3, ks);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto mma_pv = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const uint8_t* vt = sV[SL];
    const bool ld = !late && j + 3 < ntiles;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      o[db] = mfma_fp8(read32(vt, voff[db]), p8, o[db]);
      if (ld && (db % (DB / 2)) == DB / 2 - 1) {
        __builtin_amdgcn_sched_barrier(0);
        dma_k(j + 3, SL, db / (DB / 2));
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int kt0 = j * BC;
    // the LDS read unconditionally and the memory read volatile: otherwise
    // the compiler merges the two into one flat load of a selected address,
    // which it then waits for like a memory load on every tile
    float ks = s_ksc[min(j, KSC_CAP - 1)];
    if (!ksc_lds) ks = *(const volatile float*)(ksc + j);
    const float c = c_q * ks;
    bool need_mask = kt0 + BC > len;
    if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > q_wave0);
    float cc = c;
    if (need_mask) {
      cc = 1.f;
      const int qi = pin_in_branch(q_wave0 + l32);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt0 + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          bool vis = key < len;
          if (CAUSAL) vis = vis && key <= qi;
          s[kb][r] = vis ? s[kb][r] * c : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_max_halves(mx) * cc;
    const float m_new = (mx > m + kLazyMaxFp8) ? mx : m;
    const bool dead = m_new == kNegInf;
    const float alpha = dead ? 1.f : fast_exp2(m - m_new);
    // exp2 returns P * 2^6 directly (the scaling folded into the exponent);
    // l then carries the same factor, removed exactly in the epilogue
    const float mu = dead ? 0.f : m_new - kPScaleLog2;
    float rs = -0.f;  // -0 + x == x: the first add folds away
    uint32_t w[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[i] = fast_exp2(__builtin_fmaf(s[kb][4 * q4 + i], cc, -mu));
          rs += e[i];
        }
        // the old word's low half is replaced here and its high half by
        // the second conversion: passing the previous tile's word (dead by
        // now) saves clearing a register
        uint32_t x = cvt_fp8x2<false>(e[0], e[1], (uint32_t)p8[kb * 4 + q4]);
        w[kb * 4 + q4] = cvt_fp8x2<true>(e[2], e[3], x);
      }
    p8 = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    l = alpha * l + rs;
    m = m_new;
    if (wave_any(alpha != 1.f)) {
      const float a_ = pin_in_branch(alpha);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= a_;
    }
  };

  // Interval t loads K_{t+2} and V_{t+1}; the barrier ending interval t
  // needs interval t-1's loads (K_{t+1}, V_t) and lets interval t's stay in
  // flight.  The late waves hold no loads.
  auto live = [&](int j) __attribute__((always_inline)) -> bool { return j >= 0 && j <= jw_last; };
  auto end_interval = [&](int t) __attribute__((always_inline)) {
    if (!late) {
      const int pending = (t + 2 < ntiles ? 2 : 0) + (t + 1 < ntiles ? 2 : 0);
      if (pending == 4) barrier_vmem_n<4>();
      else if (pending == 2) barrier_vmem_n<2>();
      else barrier_vmem_n<0>();
      if (!live(t) && t + 3 < ntiles) issue_k(t + 3, (t + 3) % 3);
      if (!live(t + 1) && t + 2 < ntiles) issue_v(t + 2, (t + 2) % 3);
    } else {
      barrier_vmem_n<0>();
    }
  };

  // Prologue (early waves): K_0, K_1, V_0 and interval 0's K_2 (no P V
  // precedes S_0); K_0 must land.
  if (!late) {
    issue_k(0, 0);
    if (ntiles > 1) issue_k(1, 1);
    issue_v(0, 0);
    if (ntiles > 2) issue_k(2, 2);
    const int pending = (ntiles > 1 ? 2 : 0) + 2 + (ntiles > 2 ? 2 : 0);
    if (pending == 6) barrier_vmem_n<6>();
    else if (pending == 4) barrier_vmem_n<4>();
    else barrier_vmem_n<2>();
    if (!live(0) && ntiles > 1) issue_v(1, 1);
  } else {
    barrier_vmem_n<0>();
  }

  auto body = [&](int j, auto slot_c) __attribute__((always_inline)) {
    mma_s(slot_c, j);
    if (late) end_interval(j);
    softmax(j);
    if (!late) end_interval(j);
    mma_pv(slot_c, j);
  };
  for (int j = 0; j <= jw_last; j += 3) {
    body(j, std::integral_constant<int, 0>{});
    if (j + 1 <= jw_last) body(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 <= jw_last) body(j + 2, std::integral_constant<int, 2>{});
  }
  for (int t = jw_last + 1; t <= ntiles; ++t) end_interval(t);

  // l holds 2^6 times the row sum: O = O~ * s_v / l, LSE = ln 2 * (m + log2 l - 6).
  // In the accumulator layout a store instruction would touch 32 rows, so
  // each wave's 32 x 128 block of O goes through LDS (idle: every wave has
  // passed the last barrier after its own LDS reads) and leaves as row
  // segments, 16 bytes per lane.  The K and V buffers hold 32 x 64 per wave,
  // so the block goes in two column halves; a half is row-major with 16-byte
  // chunk c of row r at chunk c ^ (r mod 8); waves 0-5 stage in the K
  // buffers, 6 and 7 in the V buffers.
  uint16_t* __restrict__ op = (uint16_t*)a.o + (int64_t)bh * len * D;
  const float lt = wave_sum_halves(l);
  const int qi = q_wave0 + l32;
  // dead: no visible key (max -inf, sum 0); a NaN score leaves the max at
  // -inf (max ignores NaN) but the sum NaN, and the row comes out NaN
  const bool dead = (m == kNegInf) && !(lt != lt);
  const float inv = dead ? 0.f : a.v_scale[bhk] / lt;
  constexpr int HW = D / 2;  // columns per half
  static_assert(6 * 32 * HW * 2 <= 3 * KTILE && 2 * 32 * HW * 2 <= 3 * VTILE, "staging fits the tile buffers");
  uint16_t* stage = wave < 6 ? reinterpret_cast<uint16_t*>(&sK[0][0]) + wave * 32 * HW
                             : reinterpret_cast<uint16_t*>(&sV[0][0]) + (wave - 6) * 32 * HW;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int db = 2 * half; db < 2 * half + 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& x = o[db];
        u32x2 wv = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                    pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
        const int c = (db - 2 * half) * 4 + g;
        *(u32x2*)(stage + l32 * HW + ((c ^ (l32 % 8)) << 3) + hi * 4) = wv;
      }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i * 8 + lane / 8;
      const int c = lane % 8;
      const u32x4 w = *(const u32x4*)(stage + r * HW + ((c ^ (r % 8)) << 3));
      if (q_wave0 + r < len) *(u32x4*)(op + (int64_t)(q_wave0 + r) * D + half * HW + c * 8) = w;
    }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads are done before the next half's writes
  }
  if (qi < len && hi == 0) a.lse[(int64_t)bh * len + qi] = dead ? kNegInf : (m + fast_log2(lt) - kPScaleLog2) * kLn2;
}

// ------------------------------------------------------------------ launchers
hipError_t launch_quant_rows_fp8(const void* x, void* x8, float* scales, int BH, int N, int d, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  const int nb = (N + 63) / 64;
  const int64_t blocks = (int64_t)BH * nb;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  QuantArgs q = {(const uint16_t*)x, (uint8_t*)x8, scales, BH, N};
  hipLaunchKernelGGL(quant_rows_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, q, nb);
  return hipGetLastError();
}

hipError_t launch_quant_vt_fp8(const void* v, void* v8t, float* scales, int BH, int N, int d, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  const int nt = (N + 63) / 64;
  const int64_t blocks = (int64_t)BH * nt;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  QuantArgs q = {(const uint16_t*)v, (uint8_t*)v8t, scales, BH, N};
  hipLaunchKernelGGL(tile_amax_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, q, nt);
  hipLaunchKernelGGL(head_scale_kernel<128>, dim3((unsigned)BH), dim3(64), 0, stream, q, nt);
  hipLaunchKernelGGL(quant_vt_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, q, nt);
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t stream) {
  if (d != 128) return hipErrorInvalidValue;
  constexpr int BR = 256;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (causal)
    hipLaunchKernelGGL(fwd_fp8_kernel<true>, dim3((unsigned)blocks), dim3(512), 0, stream, a, n_qtiles);
  else
    hipLaunchKernelGGL(fwd_fp8_kernel<false>, dim3((unsigned)blocks), dim3(512), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

}  // namespace miattn
