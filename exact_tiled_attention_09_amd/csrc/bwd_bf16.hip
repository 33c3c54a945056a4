// Exact attention backward, bf16 operands with fp32 accumulation, for gfx950.
//
// Method ("解析 FlashAttention（4）：FlashAttention-v2", section 五: the softmax
// gradient 5.1, the D identity 5.2 and the general backward 5.4; the LSE
// reconstruction of "分块 Attention：重建概率，累计梯度", section 04):
//   D = rowsum(dO o O);  P = exp(S - LSE);  dV += P^T dO;  dP = dO V^T;
//   dS = P o (dP - D);  dQ += scale dS K;  dK += scale dS^T Q.
//
// Three kernels, all on the caller's stream:
//  1. bwd_prep: D for every row (fp32) and a zeroed fp32 dQ accumulator.
//  2. bwd_main: one workgroup per (sequence, head, 128-key tile); each of the
//     4 waves owns 32 keys with their dK/dV accumulators in registers; the
//     workgroup's K and V stay in LDS as MFMA operands.  For every 64-row query tile at or after the
//     diagonal it recomputes S = Q K^T, P, dP = dO V^T and dS, accumulates
//     dV += P^T dO and dK += dS^T Q (P/dS come straight out of the accumulator
//     in A-operand layout; dO and Q are fed through the LDS transpose read),
//     parks dS^T in LDS and forms the tile's dQ contribution, which it adds
//     to the fp32 accumulator with hardware float atomics.
//  3. bwd_dq: dQ = bf16(scale * accumulator).
#include "miattn_device.h"
#include "miattn_launch.h"

namespace miattn {

// ---------------------------------------------------------------- kernel 1
// Rows are (batch, head, token) for dense tensors and (token, head) for packed
// ones; both flatten to row r with features at r*D in memory order, except
// that D is stored like LSE ([B,H,N] or [H,T]).
template <int D, bool VARLEN>
__global__ void __launch_bounds__(256) bwd_prep_kernel(AttnArgs a, int64_t rows) {
  constexpr int LPR = D / 8;        // lanes per row, 16 bytes each
  constexpr int RPB = 256 / LPR;    // rows per block
  const int tid = threadIdx.x;
  const int64_t row = (int64_t)blockIdx.x * RPB + tid / LPR;
  const int sub = tid % LPR;
  float acc = 0.f;
  const bool ok = row < rows;
  if (ok) {
    const int64_t off = row * D + sub * 8;
    const u32x4 o = *(const u32x4*)((const uint16_t*)a.o + off);
    const u32x4 g = *(const u32x4*)((const uint16_t*)a.dout + off);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = __builtin_fmaf(bf16_bits_to_f32(o[w] & 0xffffu), bf16_bits_to_f32(g[w] & 0xffffu), acc);
      acc = __builtin_fmaf(bf16_bits_to_f32(o[w] >> 16), bf16_bits_to_f32(g[w] >> 16), acc);
    }
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(a.dq_acc + off) = z;
    *(f32x4*)(a.dq_acc + off + 4) = z;
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPR);
  if (ok && sub == 0) {
    int64_t drow = row;
    if constexpr (VARLEN) {
      const int64_t t = row / a.H, h = row - t * a.H;
      drow = h * a.total_tokens + t;
    }
    a.dvec[drow] = acc;
  }
}

// ---------------------------------------------------------------- kernel 2
// LDS holds the workgroup's K and V tiles for its whole life (row-major, read
// as MFMA operands), one Q / dO tile (refilled while the dQ product runs: the
// barrier before that product is the last point any wave reads them), and the
// dS^T tile.  Per wave, registers hold only the dK/dV accumulators and the
// S/dP tiles, so everything fits the 256 architectural VGPRs.
template <int D, bool CAUSAL, bool VARLEN, bool KPAD>
__global__ void __launch_bounds__(256, 1) bwd_main_kernel(AttnArgs a, int n_ktiles) {
  constexpr int NW = 4;
  constexpr int BK = NW * 32;        // keys per workgroup
  constexpr int BQ = 64;             // query rows per step
  constexpr int KS = D / 16;         // k-steps over the head dim
  constexpr int DB = D / 32;
  constexpr int ROW = D + 16;        // padded bf16 row of Q / dO / K / V tiles
  constexpr int SROW = BQ + 16;      // padded bf16 row of the dS^T tile
  constexpr int CH_PER_ROW = D / 8;
  constexpr int QCPT = BQ * CH_PER_ROW / 256;  // 16-byte chunks per thread, Q tile
  constexpr int KCPT = BK * CH_PER_ROW / 256;
  constexpr int DQ_UNITS = 2 * DB;   // (32-row block, 32-col block) pairs of a dQ tile
  static_assert(DQ_UNITS % NW == 0, "dQ units must split evenly over the waves");

  __shared__ __attribute__((aligned(16))) uint16_t sK[BK * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sV[BK * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BQ * ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sG[BQ * ROW];    // dO
  __shared__ __attribute__((aligned(16))) uint16_t sDS[BK * SROW];  // dS^T, bf16
  __shared__ __attribute__((aligned(16))) float sL[BQ];             // LSE * log2(e), +inf if dead
  __shared__ __attribute__((aligned(16))) float sDv[BQ];            // D

  const int nbh = a.B * a.H;
  const int bh = blockIdx.x % nbh;
  const int kt = blockIdx.x / nbh;  // key tiles in order: the earliest carry the most work
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<VARLEN>(a, b, h, D);
  const int k0 = kt * BK;
  if (k0 >= sv.len) return;
  (void)n_ktiles;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int len = sv.len;
  const float c = a.scale_log2;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.base;
  const uint16_t* __restrict__ gp = (const uint16_t*)a.dout + sv.base;

  const int wk0 = k0 + wave * 32;  // this wave's 32 keys
  const int my_key = wk0 + l32;
  bool key_ok = my_key < len;
  if constexpr (KPAD) {
    if (key_ok) key_ok = a.key_valid[sv.tok0 + my_key] != 0;
  }
  const bool any_bad_key = wave_any(!key_ok);

  // The workgroup's K and V tiles, row-major (rows past the sequence are zero).
#pragma unroll
  for (int cidx = 0; cidx < KCPT; ++cidx) {
    const int chunk = tid + cidx * 256;
    const int row = chunk / CH_PER_ROW;
    const int col = (chunk - row * CH_PER_ROW) * 8;
    const int key = k0 + row;
    u32x4 xk = {0u, 0u, 0u, 0u}, xv = {0u, 0u, 0u, 0u};
    if (key < len) {
      xk = *(const u32x4*)(kp + (int64_t)key * sv.tok_stride + col);
      xv = *(const u32x4*)(vp + (int64_t)key * sv.tok_stride + col);
    }
    *(u32x4*)(sK + row * ROW + col) = xk;
    *(u32x4*)(sV + row * ROW + col) = xv;
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int n_qt = (len + BQ - 1) / BQ;
  const int qt_begin = CAUSAL ? k0 / BQ : 0;

  u32x4 rq[QCPT], rg[QCPT];
  float rl = 0.f, rd = 0.f;
  auto load_tile = [&](int it) {
    const int q0 = it * BQ;
#pragma unroll
    for (int cidx = 0; cidx < QCPT; ++cidx) {
      const int chunk = tid + cidx * 256;
      const int row = chunk / CH_PER_ROW;
      const int col = (chunk - row * CH_PER_ROW) * 8;
      const int qi = q0 + row;
      u32x4 xq = {0u, 0u, 0u, 0u}, xg = {0u, 0u, 0u, 0u};
      if (qi < len) {
        xq = *(const u32x4*)(qp + (int64_t)qi * sv.tok_stride + col);
        xg = *(const u32x4*)(gp + (int64_t)qi * sv.tok_stride + col);
      }
      rq[cidx] = xq;
      rg[cidx] = xg;
    }
    if (tid < BQ) {
      const int qi = q0 + tid;
      rl = kPosInf;
      rd = 0.f;
      if (qi < len) {
        const float lse = a.lse[sv.row_base + qi];
        rl = (lse == kNegInf) ? kPosInf : lse * kLog2e;
        rd = a.dvec[sv.row_base + qi];
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int cidx = 0; cidx < QCPT; ++cidx) {
      const int chunk = tid + cidx * 256;
      const int row = chunk / CH_PER_ROW;
      const int col = (chunk - row * CH_PER_ROW) * 8;
      *(u32x4*)(&sQ[row * ROW + col]) = rq[cidx];
      *(u32x4*)(&sG[row * ROW + col]) = rg[cidx];
    }
    if (tid < BQ) {
      sL[tid] = rl;
      sDv[tid] = rd;
    }
  };

  if (qt_begin < n_qt) {
    load_tile(qt_begin);
    store_tile();
  }
  __syncthreads();

  // Transpose-read addressing shared by every "rows of 4 x 16" operand.
  const int tr_row = hi * 4 + ((lane >> 2) & 3);
  const int tr_col = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  // B operands of S = Q K^T and dP = dO V^T: lane = this wave's key, 8 features.
  const uint16_t* kb_row = sK + (wave * 32 + l32) * ROW + hi * 8;
  const uint16_t* vb_row = sV + (wave * 32 + l32) * ROW + hi * 8;

  for (int it = qt_begin; it < n_qt; ++it) {
    const int q0 = it * BQ;
    if (it + 1 < n_qt) load_tile(it + 1);

    const bool live = !CAUSAL || (q0 + BQ - 1 >= wk0);
    if (live) {
      bool need_mask = (wk0 + 31 >= len) || any_bad_key;
      if (CAUSAL) need_mask = need_mask || (wk0 + 31 > q0);
      // One 32-row half of the query tile at a time keeps S and dP to 32
      // registers; the scheduling barriers stop the halves from interleaving.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        __builtin_amdgcn_sched_barrier(0);
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int off = (qb * 32 + l32) * ROW + ks * 16 + hi * 8;
          s = mfma_bf16(as_bf16x8(*(const u32x4*)(sQ + off)), as_bf16x8(*(const u32x4*)(kb_row + ks * 16)), s);
          dp = mfma_bf16(as_bf16x8(*(const u32x4*)(sG + off)), as_bf16x8(*(const u32x4*)(vb_row + ks * 16)), dp);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = qb * 32 + g * 8 + hi * 4;
          const f32x4 lv = *(const f32x4*)(&sL[ql]);
          const f32x4 dvv = *(const f32x4*)(&sDv[ql]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = g * 4 + e;
            float p = fast_exp2(__builtin_fmaf(s[r], c, -lv[e]));
            if (need_mask) {
              bool vis = key_ok;
              if (CAUSAL) vis = vis && (my_key <= q0 + ql + e);
              p = vis ? p : 0.f;
            }
            s[r] = p;
            dp[r] = p * (dp[r] - dvv[e]);
          }
        }
        // dV += P^T dO and dK += dS^T Q, 16 query rows per MFMA.
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const bf16x8 pa = pack_bf16x8(s[8 * t + 0], s[8 * t + 1], s[8 * t + 2], s[8 * t + 3],
                                        s[8 * t + 4], s[8 * t + 5], s[8 * t + 6], s[8 * t + 7]);
          const bf16x8 da = pack_bf16x8(dp[8 * t + 0], dp[8 * t + 1], dp[8 * t + 2], dp[8 * t + 3],
                                        dp[8 * t + 4], dp[8 * t + 5], dp[8 * t + 6], dp[8 * t + 7]);
          const int rbase = (qb * 32 + 16 * t + tr_row) * ROW + tr_col;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const uint16_t* pg = sG + rbase + db * 32;
            const uint16_t* pq = sQ + rbase + db * 32;
            const bf16x8 gb = join_u32x2(lds_read_tr16(pg), lds_read_tr16(pg + 8 * ROW));
            const bf16x8 qbv = join_u32x2(lds_read_tr16(pq), lds_read_tr16(pq + 8 * ROW));
            dv[db] = mfma_bf16(pa, gb, dv[db]);
            dk[db] = mfma_bf16(da, qbv, dk[db]);
          }
        }
        // dS^T into LDS: row = key of this wave, 4 consecutive query rows per write.
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 w = {pack_bf16x2(dp[4 * g + 0], dp[4 * g + 1]), pack_bf16x2(dp[4 * g + 2], dp[4 * g + 3])};
          *(u32x2*)(sDS + (wave * 32 + l32) * SROW + qb * 32 + g * 8 + hi * 4) = w;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
      u32x2 z = {0u, 0u};
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(u32x2*)(sDS + (wave * 32 + l32) * SROW + qb * 32 + g * 8 + hi * 4) = z;
    }
    __syncthreads();

    // Every wave is past its last read of sQ / sG / sL / sDv: refill them now.
    if (it + 1 < n_qt) store_tile();

    // dQ tile contribution: dQ[q][d] += sum over this workgroup's keys of dS[q][key] K[key][d].
    {
      int kmax = BK;
      if (CAUSAL) kmax = min(BK, q0 + BQ - k0);  // keys past the tile's last query have dS = 0
      const int nks = (kmax + 15) / 16;
      const bool full_tile = q0 + BQ <= len;
#pragma unroll
      for (int ui = 0; ui < DQ_UNITS / NW; ++ui) {
        const int unit = wave + ui * NW;
        const int qb = unit / DB;
        const int db = unit - qb * DB;
        f32x16 acc = f32x16{};
        for (int ks = 0; ks < nks; ++ks) {
          const uint16_t* pa = sDS + (ks * 16 + tr_row) * SROW + qb * 32 + tr_col;
          const uint16_t* pb = sK + (ks * 16 + tr_row) * ROW + db * 32 + tr_col;
          const bf16x8 av = join_u32x2(lds_read_tr16(pa), lds_read_tr16(pa + 8 * SROW));
          const bf16x8 bv = join_u32x2(lds_read_tr16(pb), lds_read_tr16(pb + 8 * ROW));
          acc = mfma_bf16(av, bv, acc);
        }
        float* dqp = a.dq_acc + sv.base + (int64_t)(q0 + qb * 32 + hi * 4) * sv.tok_stride + db * 32 + l32;
        if (full_tile) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            unsafeAtomicAdd(dqp + (int64_t)((r >> 2) * 8 + (r & 3)) * sv.tok_stride, acc[r]);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qi = q0 + qb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            if (qi < len) unsafeAtomicAdd(dqp + (int64_t)((r >> 2) * 8 + (r & 3)) * sv.tok_stride, acc[r]);
          }
        }
      }
    }
    __syncthreads();
  }

  // dK = scale * acc, dV = acc; accumulator rows are keys, columns features.
  uint16_t* __restrict__ dkp = (uint16_t*)a.dk + sv.base;
  uint16_t* __restrict__ dvp = (uint16_t*)a.dv + sv.base;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int key = wk0 + (r >> 2) * 8 + hi * 4 + (r & 3);
    if (key < len) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int64_t off = (int64_t)key * sv.tok_stride + db * 32 + l32;
        const uint32_t kb = pack_bf16x2(dk[db][r] * a.scale, 0.f);
        const uint32_t vb = pack_bf16x2(dv[db][r], 0.f);
        dkp[off] = (uint16_t)(kb & 0xffffu);
        dvp[off] = (uint16_t)(vb & 0xffffu);
      }
    }
  }
}

// ---------------------------------------------------------------- kernel 3
__global__ void __launch_bounds__(256) bwd_dq_kernel(const float* __restrict__ acc, uint16_t* __restrict__ dq,
                                                     int64_t n8, float scale) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = *(const f32x4*)(acc + i * 8);
  const f32x4 x1 = *(const f32x4*)(acc + i * 8 + 4);
  u32x4 w = {pack_bf16x2(x0[0] * scale, x0[1] * scale), pack_bf16x2(x0[2] * scale, x0[3] * scale),
             pack_bf16x2(x1[0] * scale, x1[1] * scale), pack_bf16x2(x1[2] * scale, x1[3] * scale)};
  *(u32x4*)(dq + i * 8) = w;
}

// ---------------------------------------------------------------- launchers
hipError_t launch_bwd_prep_bf16(const AttnArgs& a, int d, bool varlen, hipStream_t stream) {
  const int64_t rows = varlen ? (int64_t)a.total_tokens * a.H : (int64_t)a.B * a.H * a.N;
  if (rows <= 0) return hipSuccess;
  const int rpb = 256 / (d / 8);
  const int64_t blocks = (rows + rpb - 1) / rpb;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 128) {
    if (varlen) hipLaunchKernelGGL((bwd_prep_kernel<128, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rows);
    else hipLaunchKernelGGL((bwd_prep_kernel<128, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rows);
  } else if (d == 64) {
    if (varlen) hipLaunchKernelGGL((bwd_prep_kernel<64, true>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rows);
    else hipLaunchKernelGGL((bwd_prep_kernel<64, false>), dim3((unsigned)blocks), dim3(256), 0, stream, a, rows);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN, bool KPAD>
static hipError_t launch_bwd_main_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BK = 128;
  const int n_ktiles = (a.N + BK - 1) / BK;
  const int64_t blocks = (int64_t)n_ktiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, VARLEN, KPAD>), dim3((unsigned)blocks), dim3(256), 0, stream,
                     a, n_ktiles);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_bwd_main(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
  if (varlen) {
    if (causal) return kpad ? launch_bwd_main_t<D, true, true, true>(a, s) : launch_bwd_main_t<D, true, true, false>(a, s);
    return kpad ? launch_bwd_main_t<D, false, true, true>(a, s) : launch_bwd_main_t<D, false, true, false>(a, s);
  }
  return causal ? launch_bwd_main_t<D, true, false, false>(a, s) : launch_bwd_main_t<D, false, false, false>(a, s);
}

hipError_t launch_bwd_main_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream) {
  const bool kpad = varlen && a.key_valid != nullptr;
  if (d == 128) return dispatch_bwd_main<128>(a, causal, varlen, kpad, stream);
  if (d == 64) return dispatch_bwd_main<64>(a, causal, varlen, kpad, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int d, bool varlen, hipStream_t stream) {
  const int64_t elems = (varlen ? (int64_t)a.total_tokens : (int64_t)a.B * a.N) * a.H * d;
  const int64_t n8 = elems / 8;
  if (n8 <= 0) return hipSuccess;
  const int64_t blocks = (n8 + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, (const float*)a.dq_acc,
                     (uint16_t*)a.dq, n8, a.scale);
  return hipGetLastError();
}

}  // namespace miattn
