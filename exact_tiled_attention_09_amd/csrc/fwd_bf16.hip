// Fused exact attention forward, bf16 in / bf16 O / fp32 LSE, for gfx950.
//
// Method: the online-softmax forward with an unnormalised output accumulator
// and one log-sum-exp per row ("解析 FlashAttention（4）：FlashAttention-v2",
// section 四, the general forward; running state as in "分块 Attention：重建概率，
// 累计梯度", section 01).  The N x N scores never leave registers.
//
// Work decomposition (MI355X-first, not the pages' thread-block layout):
//  * one workgroup per (sequence, head, query tile of BR = NW * QB * 32 rows);
//    each wave owns QB blocks of 32 query rows ("split-Q": no cross-wave
//    softmax traffic).
//  * the wave computes S^T = K Q^T so that the 32x32 accumulator puts one query
//    per lane column: row max / row sum are in-lane over 16 registers plus one
//    exchange with the lane 32 away, and the rescale factor is a per-lane
//    scalar.
//  * P^T leaves the accumulator already in the B-operand layout of
//    O^T += V^T P^T; V^T comes from the row-major V tile through the LDS
//    transpose read, so neither P nor V is shuffled.
//  * K/V tiles of BC = 64 keys are double-buffered in LDS (one barrier per
//    tile) in the XOR-swizzled layout of swz<D>, which keeps both the b128
//    operand reads and the transpose reads free of bank conflicts; Q stays in
//    registers for the whole key loop.
//  * softmax runs in base 2 with scale * log2(e) folded into one FMA.  A row's
//    reference max is only raised when a tile's max exceeds it by more than
//    kLazyMax (base-2 units); below that the stale reference is kept, P~ stays
//    below 2^kLazyMax, and O~ and l need no rescale.  Any reference value gives
//    the same O = O~ / l and LSE = m + log2 l, so this changes only rounding.
//  * causal: key tiles above the diagonal are never loaded; only tiles that
//    cross the diagonal, the sequence end or a padded key are masked
//    element-wise; query tiles are issued heaviest first; consecutive
//    workgroups of one (sequence, head) are spread so that the 8 XCDs each
//    keep whole heads in their L2 when B*H is a multiple of 8.
#include "miattn_device.h"
#include "miattn_launch.h"

#include <cstdlib>

namespace miattn {

constexpr float kLazyMax = 8.0f;

template <int D, int QB, int NW, int MINB, bool CAUSAL, bool VARLEN, bool KPAD>
__global__ void __launch_bounds__(NW * 64, MINB) fwd_bf16_kernel(AttnArgs a, int n_qtiles) {
  constexpr int BC = 64;                 // keys per tile
  constexpr int BR = NW * QB * 32;       // query rows per workgroup
  constexpr int KS = D / 16;             // k-steps of S over the head dim
  constexpr int DB = D / 32;             // 32-wide blocks of O columns
  constexpr int TILE = BC * D;           // one K or V tile (swizzled rows, see swz)
  constexpr int NT = NW * 64;
  constexpr int CH_PER_ROW = D / 8;      // 16-byte chunks per row
  constexpr int CPT = BC * CH_PER_ROW / NT;
  static_assert(CPT * NT == BC * CH_PER_ROW, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * TILE];
  __shared__ uint8_t s_valid[2][BC];
  __shared__ uint32_t s_anypad[2];

  const int nbh = a.B * a.H;
  const int bh = blockIdx.x % nbh;
  int tile = blockIdx.x / nbh;
  if (CAUSAL) tile = n_qtiles - 1 - tile;  // heaviest query tiles first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<VARLEN>(a, b, h, D);
  const int q_tile0 = tile * BR;
  if (q_tile0 >= sv.len) return;  // uniform across the workgroup, before any barrier

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int q_wave0 = q_tile0 + wave * QB * 32;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.base;

  // A negative scale is handled by flipping the sign of Q once.
  float c = a.scale_log2;
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  c = fabsf(c);

  // Q as the B operand of S^T = K Q^T: lane (query l32, half hi) holds
  // features ks*16 + hi*8 .. +7 for every k-step ks.
  bf16x8 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = q_wave0 + qb * 32 + l32;
    const bool ok = qi < sv.len;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (ok) x = *(const u32x4*)(qp + (int64_t)qi * sv.tok_stride + ks * 16 + hi * 8);
      x ^= qsign;
      qf[qb][ks] = as_bf16x8(x);
    }
  }

  f32x16 o[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kNegInf;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
  }

  const int kv_len = sv.len;
  const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
  const int ntiles = (kv_end + BC - 1) / BC;

  u32x4 rk[CPT], rv[CPT];
  uint32_t rvalid = 1u;
  auto load_tile = [&](int j) {
#pragma unroll
    for (int cidx = 0; cidx < CPT; ++cidx) {
      const int chunk = tid + cidx * NT;
      const int row = chunk / CH_PER_ROW;
      const int col = (chunk - row * CH_PER_ROW) * 8;
      const int key = j * BC + row;
      u32x4 zk = {0u, 0u, 0u, 0u}, zv = {0u, 0u, 0u, 0u};
      if (key < kv_len) {
        zk = *(const u32x4*)(kp + (int64_t)key * sv.tok_stride + col);
        zv = *(const u32x4*)(vp + (int64_t)key * sv.tok_stride + col);
      }
      rk[cidx] = zk;
      rv[cidx] = zv;
    }
    if constexpr (KPAD) {
      if (wave == 0) {
        const int key = j * BC + lane;
        rvalid = (key < kv_len) ? (uint32_t)(a.key_valid[sv.tok0 + key] != 0) : 1u;
      }
    }
  };
  int st_off[CPT];  // swizzled LDS offset of each staged chunk
#pragma unroll
  for (int cidx = 0; cidx < CPT; ++cidx) {
    const int chunk = tid + cidx * NT;
    const int row = chunk / CH_PER_ROW;
    st_off[cidx] = swz_off<D>(row, (chunk - row * CH_PER_ROW) * 8);
  }
  auto store_tile = [&](int buf) {
    uint16_t* sk = smem + buf * 2 * TILE;
    uint16_t* sv_ = sk + TILE;
#pragma unroll
    for (int cidx = 0; cidx < CPT; ++cidx) {
      *(u32x4*)(sk + st_off[cidx]) = rk[cidx];
      *(u32x4*)(sv_ + st_off[cidx]) = rv[cidx];
    }
    if constexpr (KPAD) {
      if (wave == 0) {
        s_valid[buf][lane] = (uint8_t)rvalid;
        const bool any = wave_any(rvalid == 0u);
        if (lane == 0) s_anypad[buf] = any ? 1u : 0u;
      }
    }
  };

  // Per-lane operand offsets inside a tile (the swizzle of a row depends only
  // on the row modulo 16, so 32-row and 16-row steps reuse them).
  int koff[KS];       // K as the A operand of S^T: row kb*32 + l32, chunk 2*ks + hi
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = swz_off<D>(l32, ks * 16 + hi * 8);
  const int tr_r = hi * 4 + ((lane >> 2) & 3);
  const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int voff[2][DB];    // V through the transpose read: rows 8R + tr_r, columns db*32 + tr_c
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);

    const int kt0 = j * BC;
    const bool wave_live = !CAUSAL || kt0 <= q_wave0 + QB * 32 - 1;
    if (wave_live) {
      const uint16_t* sk = smem + buf * 2 * TILE;
      const uint16_t* svt = sk + TILE;

      // S^T = K Q^T for two 32-key blocks.
      f32x16 s[2][QB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = as_bf16x8(*(const u32x4*)(sk + kb * 32 * D + koff[ks]));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = mfma_bf16(ka, qf[qb][ks], s[kb][qb]);
        }
      }

      bool need_mask = kt0 + BC > kv_len;
      if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > q_wave0);
      if (KPAD) need_mask = need_mask || (s_anypad[buf] != 0u);
      float cc = c;
      if (need_mask) {
        // Scale first, then hide masked entries as -inf; afterwards the
        // exponent uses multiplier 1 (so scale == 0 cannot make 0 * -inf).
        cc = 1.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qi = q_wave0 + qb * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int kl = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
              const int key = kt0 + kl;
              bool vis = key < kv_len;
              if (CAUSAL) vis = vis && key <= qi;
              if (KPAD) vis = vis && s_valid[buf][kl] != 0;
              s[kb][qb][r] = vis ? s[kb][qb][r] * c : kNegInf;
            }
          }
      }

#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        mx = wave_max_halves(mx);
        const float mt = need_mask ? mx : mx * c;
        const float m_new = (mt > m[qb] + kLazyMax) ? mt : m[qb];
        const bool dead = m_new == kNegInf;  // no visible key yet for this row
        const float alpha = dead ? 1.f : fast_exp2(m[qb] - m_new);
        const float mu = dead ? 0.f : m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(__builtin_fmaf(s[kb][qb][r], cc, -mu));
            rs += p;
            s[kb][qb][r] = p;
          }
        l[qb] = alpha * l[qb] + rs;
        m[qb] = m_new;
        if (wave_any(alpha != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) o[qb][db] *= alpha;
        }
      }

      // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          bf16x8 pb[QB];
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const f32x16& x = s[kb][qb];
            pb[qb] = pack_bf16x8(x[8 * t + 0], x[8 * t + 1], x[8 * t + 2], x[8 * t + 3],
                                 x[8 * t + 4], x[8 * t + 5], x[8 * t + 6], x[8 * t + 7]);
          }
          const uint16_t* vt = svt + (kb * 32 + 16 * t) * D;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const bf16x8 va = join_u32x2(lds_read_tr16(vt + voff[0][db]), lds_read_tr16(vt + voff[1][db]));
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma_bf16(va, pb[qb], o[qb][db]);
          }
        }
    }

    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O~ / l, LSE = ln 2 * (m + log2 l); a row that saw no
  // visible key gets O = 0 and LSE = -inf.
  uint16_t* __restrict__ op = (uint16_t*)a.o + sv.base;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = wave_sum_halves(l[qb]);
    const int qi = q_wave0 + qb * 32 + l32;
    if (qi < sv.len) {
      const bool dead = (m[qb] == kNegInf) || !(lt > 0.f);
      const float inv = dead ? 0.f : 1.f / lt;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& x = o[qb][db];
          u32x2 w = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                     pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
          *(u32x2*)(op + (int64_t)qi * sv.tok_stride + db * 32 + g * 8 + hi * 4) = w;
        }
      if (hi == 0) a.lse[sv.row_base + qi] = dead ? kNegInf : (m[qb] + fast_log2(lt)) * kLn2;
    }
  }
}

template <int D, int QB, int NW, int MINB, bool CAUSAL, bool VARLEN, bool KPAD>
static hipError_t launch_fwd_bf16_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BR = NW * QB * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, QB, NW, MINB, CAUSAL, VARLEN, KPAD>), dim3((unsigned)blocks),
                     dim3(NW * 64), 0, stream, a, n_qtiles);
  return hipGetLastError();
}

template <int D, int QB, int NW, int MINB>
static hipError_t dispatch_fwd(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
  if (varlen) {
    if (causal) return kpad ? launch_fwd_bf16_t<D, QB, NW, MINB, true, true, true>(a, s)
                            : launch_fwd_bf16_t<D, QB, NW, MINB, true, true, false>(a, s);
    return kpad ? launch_fwd_bf16_t<D, QB, NW, MINB, false, true, true>(a, s)
                : launch_fwd_bf16_t<D, QB, NW, MINB, false, true, false>(a, s);
  }
  return causal ? launch_fwd_bf16_t<D, QB, NW, MINB, true, false, false>(a, s)
                : launch_fwd_bf16_t<D, QB, NW, MINB, false, false, false>(a, s);
}

// Tile shapes: (query blocks per wave, waves per workgroup, workgroups per CU).
// MIATTN_FWD_TILE=<n> picks a shape for tuning sweeps; the default is the
// measured best.
static int fwd_tile_choice() {
  static int choice = [] {
    const char* e = getenv("MIATTN_FWD_TILE");
    return e ? atoi(e) : 0;
  }();
  return choice;
}

hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream) {
  const bool kpad = varlen && a.key_valid != nullptr;
  const int t = fwd_tile_choice();
  if (d == 128) {
    if (t == 1) return dispatch_fwd<128, 2, 4, 1>(a, causal, varlen, kpad, stream);
    if (t == 2) return dispatch_fwd<128, 1, 4, 2>(a, causal, varlen, kpad, stream);
    return dispatch_fwd<128, 1, 8, 1>(a, causal, varlen, kpad, stream);
  }
  if (d == 64) {
    if (t == 1) return dispatch_fwd<64, 2, 4, 1>(a, causal, varlen, kpad, stream);
    if (t == 2) return dispatch_fwd<64, 1, 4, 2>(a, causal, varlen, kpad, stream);
    return dispatch_fwd<64, 1, 8, 1>(a, causal, varlen, kpad, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace miattn
