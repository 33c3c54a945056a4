// Exact attention in fp32 (fp32 inputs, outputs and accumulation), gfx950.
//
// Same method as the bf16 kernels (online-softmax forward of
// "解析 FlashAttention（4）：FlashAttention-v2" section 四; LSE-recompute backward
// of its section 五 and of "分块 Attention：重建概率，累计梯度" section 04) with
// 32 x 32 tiles and one wave per workgroup.  Products use the fp32 MFMA
// v_mfma_f32_32x32x2_f32, which multiplies true fp32 values: each lane feeds a
// single element per k-step, so no operand needs a transposed read and every
// LDS access is a plain 4-byte one.  Built for accuracy on small problems
// rather than throughput.
#include "miattn_device.h"
#include "miattn_launch.h"

namespace miattn {

// ---------------------------------------------------------------- forward
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64, 1) fwd_f32_kernel(AttnArgs a, int n_qtiles) {
  constexpr int B32 = 32;
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int ROW = D + 4;
  __shared__ float sK[B32 * ROW];
  __shared__ float sV[B32 * ROW];

  const int nbh = a.B * a.H;
  const int bh = blockIdx.x % nbh;
  int tile = blockIdx.x / nbh;
  if (CAUSAL) tile = n_qtiles - 1 - tile;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const SeqView sv = seq_view<false>(a, b, h, D);
  const int q0 = tile * B32;
  if (q0 >= sv.len) return;

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hi = lane >> 5;
  const float* __restrict__ qp = (const float*)a.q + sv.base;
  const float* __restrict__ kp = (const float*)a.k + sv.kv_base;
  const float* __restrict__ vp = (const float*)a.v + sv.kv_base;
  float c = a.scale_log2;
  const float qsign = c < 0.f ? -1.f : 1.f;
  c = fabsf(c);

  const int qi = q0 + l32;
  float qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = qi < sv.len ? qsign * qp[(int64_t)qi * D + 2 * ks + hi] : 0.f;

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int kv_len = sv.len;
  const int kv_end = CAUSAL ? min(kv_len, q0 + B32) : kv_len;
  for (int kt0 = 0; kt0 < kv_end; kt0 += B32) {
    __syncthreads();
    for (int i = lane; i < B32 * D; i += 64) {
      const int row = i / D, col = i - row * D;
      const int key = kt0 + row;
      sK[row * ROW + col] = key < kv_len ? kp[(int64_t)key * D + col] : 0.f;
      sV[row * ROW + col] = key < kv_len ? vp[(int64_t)key * D + col] : 0.f;
    }
    __syncthreads();
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = mfma_f32(sK[l32 * ROW + 2 * ks + hi], qf[ks], s);
    const bool need_mask = (kt0 + B32 > kv_len) || (CAUSAL && kt0 + B32 - 1 > q0);
    float cc = c;
    if (need_mask) {
      cc = 1.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kt0 + (r >> 2) * 8 + hi * 4 + (r & 3);
        bool vis = key < kv_len;
        if (CAUSAL) vis = vis && key <= qi;
        s[r] = vis ? s[r] * c : kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = wave_max_halves(mx);
    const float mt = need_mask ? mx : mx * c;
    const float m_new = fmaxf(m, mt);
    const bool dead = m_new == kNegInf;
    const float alpha = dead ? 1.f : fast_exp2(m - m_new);
    const float mu = dead ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[r], cc, -mu));
      rs += p;
      s[r] = p;
    }
    l = alpha * l + rs;
    m = m_new;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
    // O^T += V^T P^T: k-step r pairs key ((r/4)*8 + hi*4 + r%4) on both sides.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kl = (r >> 2) * 8 + hi * 4 + (r & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] = mfma_f32(sV[kl * ROW + db * 32 + l32], s[r], o[db]);
    }
  }

  const float lt = wave_sum_halves(l);
  if (qi < sv.len) {
    // dead: no visible key (max -inf, sum 0); a NaN score leaves the max at
    // -inf (max ignores NaN) but the sum NaN, and the row comes out NaN
    const bool dead = (m == kNegInf) && !(lt != lt);
    const float inv = dead ? 0.f : 1.f / lt;
    float* __restrict__ op = (float*)a.o + sv.base + (int64_t)qi * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 w = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
        *(f32x4*)(op + db * 32 + g * 8 + hi * 4) = w;
      }
    if (hi == 0) a.lse[sv.row_base + qi] = dead ? kNegInf : (m + fast_log2(lt)) * kLn2;
  }
}

// ---------------------------------------------------------------- backward
template <int D>
__global__ void __launch_bounds__(256) bwd_prep_f32_kernel(AttnArgs a, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* o = (const float*)a.o + row * D;
  const float* g = (const float*)a.dout + row * D;
  float acc = 0.f;
  for (int i = lane; i < D; i += 64) {
    acc = __builtin_fmaf(o[i], g[i], acc);
    a.dq_acc[row * D + i] = 0.f;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (lane == 0) a.dvec[row] = acc;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64, 1) bwd_main_f32_kernel(AttnArgs a) {
  constexpr int B32 = 32;
  constexpr int KS = D / 2;
  constexpr int DB = D / 32;
  constexpr int ROW = D + 4;
  constexpr int SROW = B32 + 4;
  __shared__ float sQ[B32 * ROW];
  __shared__ float sG[B32 * ROW];
  __shared__ float sK[B32 * ROW];
  __shared__ float sDS[B32 * SROW];  // [query][key]
  __shared__ float sL[B32];
  __shared__ float sDv[B32];

  const int nbh = a.B * a.H;
  const int bh = blockIdx.x % nbh;
  const int kt = blockIdx.x / nbh;
  const int b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const SeqView sv = seq_view<false>(a, b, h, D);
  const int k0 = kt * B32;
  const int len = sv.len;
  if (k0 >= len) return;

  const int lane = threadIdx.x;
  const int l32 = lane & 31, hi = lane >> 5;
  const float c = a.scale_log2;
  const float* __restrict__ qp = (const float*)a.q + sv.base;
  const float* __restrict__ kp = (const float*)a.k + sv.kv_base;
  const float* __restrict__ vp = (const float*)a.v + sv.kv_base;
  const float* __restrict__ gp = (const float*)a.dout + sv.base;

  const int my_key = k0 + l32;
  float kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kf[ks] = my_key < len ? kp[(int64_t)my_key * D + 2 * ks + hi] : 0.f;
    vf[ks] = my_key < len ? vp[(int64_t)my_key * D + 2 * ks + hi] : 0.f;
  }
  for (int i = lane; i < B32 * D; i += 64) {
    const int row = i / D, col = i - row * D;
    sK[row * ROW + col] = k0 + row < len ? kp[(int64_t)(k0 + row) * D + col] : 0.f;
  }
  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int n_qt = (len + B32 - 1) / B32;
  for (int it = CAUSAL ? k0 / B32 : 0; it < n_qt; ++it) {
    const int q0 = it * B32;
    __syncthreads();
    for (int i = lane; i < B32 * D; i += 64) {
      const int row = i / D, col = i - row * D;
      const bool ok = q0 + row < len;
      sQ[row * ROW + col] = ok ? qp[(int64_t)(q0 + row) * D + col] : 0.f;
      sG[row * ROW + col] = ok ? gp[(int64_t)(q0 + row) * D + col] : 0.f;
    }
    if (lane < B32) {
      const int qi = q0 + lane;
      float lv = kPosInf, dvv = 0.f;
      if (qi < len) {
        const float lse = a.lse[sv.row_base + qi];
        lv = lse == kNegInf ? kPosInf : lse * kLog2e;
        dvv = a.dvec[sv.row_base + qi];
      }
      sL[lane] = lv;
      sDv[lane] = dvv;
    }
    __syncthreads();
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma_f32(sQ[l32 * ROW + 2 * ks + hi], kf[ks], s);
      dp = mfma_f32(sG[l32 * ROW + 2 * ks + hi], vf[ks], dp);
    }
    // accumulator: lane = key column, register r = query row (r/4)*8 + hi*4 + r%4
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = (r >> 2) * 8 + hi * 4 + (r & 3);
      float p = fast_exp2(__builtin_fmaf(s[r], c, -sL[ql]));
      bool vis = my_key < len;
      if (CAUSAL) vis = vis && my_key <= q0 + ql;
      p = vis ? p : 0.f;
      s[r] = p;
      dp[r] = p * (dp[r] - sDv[ql]);
      sDS[ql * SROW + l32] = dp[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ql = (r >> 2) * 8 + hi * 4 + (r & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dv[db] = mfma_f32(s[r], sG[ql * ROW + db * 32 + l32], dv[db]);
        dk[db] = mfma_f32(dp[r], sQ[ql * ROW + db * 32 + l32], dk[db]);
      }
    }
    __syncthreads();
    // dQ[q][d] += sum_key dS[q][key] K[key][d]
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f32x16 acc = f32x16{};
#pragma unroll
      for (int kk = 0; kk < B32 / 2; ++kk)
        acc = mfma_f32(sDS[l32 * SROW + 2 * kk + hi], sK[(2 * kk + hi) * ROW + db * 32 + l32], acc);
      float* dqp = a.dq_acc + sv.base + db * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + (r >> 2) * 8 + hi * 4 + (r & 3);
        if (qi < len) unsafeAtomicAdd(dqp + (int64_t)qi * D, acc[r]);
      }
    }
  }

  float* __restrict__ dkp = (float*)a.dk + sv.base;
  float* __restrict__ dvp = (float*)a.dv + sv.base;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = k0 + (r >> 2) * 8 + hi * 4 + (r & 3);
    if (key < len) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dkp[(int64_t)key * D + db * 32 + l32] = dk[db][r] * a.scale;
        dvp[(int64_t)key * D + db * 32 + l32] = dv[db][r];
      }
    }
  }
}

__global__ void __launch_bounds__(256) bwd_dq_f32_kernel(const float* __restrict__ acc, float* __restrict__ dq,
                                                         int64_t n, float scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) dq[i] = acc[i] * scale;
}

// ---------------------------------------------------------------- launchers
template <int D>
static hipError_t fwd_f32_d(const AttnArgs& a, bool causal, hipStream_t stream) {
  const int n_qtiles = (a.N + 31) / 32;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (causal) hipLaunchKernelGGL((fwd_f32_kernel<D, true>), dim3((unsigned)blocks), dim3(64), 0, stream, a, n_qtiles);
  else hipLaunchKernelGGL((fwd_f32_kernel<D, false>), dim3((unsigned)blocks), dim3(64), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const AttnArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return fwd_f32_d<64>(a, causal, stream);
  if (d == 128) return fwd_f32_d<128>(a, causal, stream);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t bwd_f32_d(const AttnArgs& a, bool causal, hipStream_t stream) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (rows <= 0) return hipSuccess;
  const int64_t pblocks = (rows + 3) / 4;
  const int64_t mblocks = (int64_t)((a.N + 31) / 32) * a.B * a.H;
  const int64_t n = rows * D;
  const int64_t cblocks = (n + 255) / 256;
  if (pblocks > 0x7fffffff || mblocks > 0x7fffffff || cblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_prep_f32_kernel<D>), dim3((unsigned)pblocks), dim3(256), 0, stream, a, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (causal) hipLaunchKernelGGL((bwd_main_f32_kernel<D, true>), dim3((unsigned)mblocks), dim3(64), 0, stream, a);
  else hipLaunchKernelGGL((bwd_main_f32_kernel<D, false>), dim3((unsigned)mblocks), dim3(64), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)cblocks), dim3(256), 0, stream, (const float*)a.dq_acc,
                     (float*)a.dq, n, a.scale);
  return hipGetLastError();
}

hipError_t launch_bwd_f32(const AttnArgs& a, int d, bool causal, hipStream_t stream) {
  if (d == 64) return bwd_f32_d<64>(a, causal, stream);
  if (d == 128) return bwd_f32_d<128>(a, causal, stream);
  return hipErrorInvalidValue;
}

}  // namespace miattn
