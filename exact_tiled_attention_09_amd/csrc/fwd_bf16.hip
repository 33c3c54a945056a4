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

  int bh, tile;
  wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, CAUSAL, bh, tile);  // causal: heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<VARLEN>(a, b, h, D);
  const int q_tile0 = tile * BR;
  if (q_tile0 >= sv.len) return;  // uniform across the workgroup, before any barrier

  const int tid = threadIdx.x;
  const int wave = wave_id();
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
        const int q_lane = pin_in_branch(q_wave0 + l32);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int qi = q_lane + qb * 32;
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
          const float a_ = pin_in_branch(alpha);
#pragma unroll
          for (int db = 0; db < DB; ++db) o[qb][db] *= a_;
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

// Software-pipelined form of the same forward (the default).  One wave owns
// 32 query rows; in iteration j it issues, as three independent streams,
//   O += V_{j-1}^T P_{j-1}   (MFMA),   S_{j+1} = K_{j+1} Q^T   (MFMA),
//   softmax of S_j -> P_j     (VALU: max, exp2, row sum, bf16 pack),
// so the matrix cores work on tile j-1 / j+1 while the vector ALU works on
// tile j.  The scheduler is asked to interleave them (one MFMA, then a few
// LDS reads and VALU operations, repeated).  K and V tiles are fetched with
// direct global->LDS loads into the swizzled layout: in iteration j, buffer
// (j+1)%2 holds K_{j+1} and V_{j-1} (being read) while K_{j+2} and V_j land in
// buffer j%2.  Rescaling O for a raised row max is applied after the block,
// when it already contains P_{j-1} V_{j-1}, so O stays consistent with m.
template <int D, int NW, bool CAUSAL, bool VARLEN, bool KPAD>
__global__ void __launch_bounds__(NW * 64, 1) fwd_pipe_kernel(AttnArgs a, int n_qtiles) {
  constexpr int BC = 64;
  constexpr int BR = NW * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int LPT = BC * CPR / NT;     // direct loads per thread per tile
  static_assert(LPT * NT == BC * CPR, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][TILE];
  __shared__ uint8_t s_valid[3][BC];
  __shared__ uint32_t s_anypad[3];

  int bh, tile;
  wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, CAUSAL, bh, tile);  // causal: heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<VARLEN>(a, b, h, D);
  const int q_tile0 = tile * BR;
  if (q_tile0 >= sv.len) return;  // uniform across the workgroup, before any barrier

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int q_wave0 = q_tile0 + wave * 32;
  const int kv_len = sv.len;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.base;

  float c = a.scale_log2;
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  c = fabsf(c);

  bf16x8 qf[KS];
  {
    const int qi = q_wave0 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < kv_len) x = *(const u32x4*)(qp + (int64_t)qi * sv.tok_stride + ks * 16 + hi * 8);
      qf[ks] = as_bf16x8(x ^ qsign);
    }
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
  const int ntiles = (kv_end + BC - 1) / BC;
  // last key tile this wave sees anything of (waves of one tile differ under causal masking)
  const int jw_last = CAUSAL ? min(ntiles - 1, (q_wave0 + 31) / BC) : ntiles - 1;

  // Direct-load sources: LDS chunk p = i*NT + tid holds logical (row, chunk ^ swz(row)).
  int src_off[LPT], src_row[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int pch = i * NT + tid;
    const int row = pch / CPR;
    src_row[i] = row;
    src_off[i] = (((pch % CPR) ^ swz<D>(row)) << 3);
  }
  auto issue_tile = [&](uint16_t* dst, const uint16_t* src, int j) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = min(j * BC + src_row[i], kv_len - 1);  // rows past the end repeat a valid row; masked
      load_lds16(src + (int64_t)key * sv.tok_stride + src_off[i], dst + (i * NT + wave * 64) * 8);
    }
  };
  uint32_t rvalid = 1u;
  auto load_flags = [&](int j) {
    if constexpr (KPAD) {
      if (wave == 0) {
        const int key = j * BC + lane;
        rvalid = (key < kv_len) ? (uint32_t)(a.key_valid[sv.tok0 + key] != 0) : 1u;
      }
    }
  };
  auto store_flags = [&](int slot) {
    if constexpr (KPAD) {
      if (wave == 0) {
        s_valid[slot][lane] = (uint8_t)rvalid;
        const bool any = wave_any(rvalid == 0u);
        if (lane == 0) s_anypad[slot] = any ? 1u : 0u;
      }
    }
  };

  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = swz_off<D>(l32, ks * 16 + hi * 8);
  const int tr_r = hi * 4 + ((lane >> 2) & 3);
  const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int voff[2][DB];
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);

  auto mma_s = [&](const uint16_t* kt, f32x16 (&s)[2]) {
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma_bf16(as_bf16x8(*(const u32x4*)(kt + kb * 32 * D + koff[ks])), qf[ks], s[kb]);
  };
  auto mma_pv = [&](const uint16_t* vt, const bf16x8 (&p)[4]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* v0 = vt + (kb * 32 + 16 * t) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 va = join_u32x2(lds_read_tr16(v0 + voff[0][db]), lds_read_tr16(v0 + voff[1][db]));
          o[db] = mfma_bf16(va, p[kb * 2 + t], o[db]);
        }
      }
  };
  // Row max, reference update, exp2, row sum and bf16 packing of one tile.
  // cc is 1 when the tile was masked (its scores are then already scaled).
  auto softmax = [&](f32x16 (&s)[2], float cc, bf16x8 (&p)[4]) -> float {
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_max_halves(mx) * cc;
    const float m_new = (mx > m + kLazyMax) ? mx : m;
    const bool dead = m_new == kNegInf;
    const float alpha = dead ? 1.f : fast_exp2(m - m_new);
    const float mu = dead ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(__builtin_fmaf(s[kb][8 * t + i], cc, -mu));
          rs += e[i];
        }
        p[kb * 2 + t] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      }
    l = alpha * l + rs;
    m = m_new;
    return alpha;
  };
  auto tile_needs_mask = [&](int j) {
    const int kt0 = j * BC;
    bool nm = kt0 + BC > kv_len;
    if (CAUSAL) nm = nm || (kt0 + BC - 1 > q_wave0);
    if (KPAD) nm = nm || (s_anypad[j % 3] != 0u);
    return nm;
  };
  auto apply_mask = [&](f32x16 (&s)[2], int j) {
    const int kt0 = j * BC;
    const int qi = pin_in_branch(q_wave0 + l32);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
        const int key = kt0 + kl;
        bool vis = key < kv_len;
        if (CAUSAL) vis = vis && key <= qi;
        if (KPAD) vis = vis && s_valid[j % 3][kl] != 0;
        s[kb][r] = vis ? s[kb][r] * c : kNegInf;
      }
  };

  // Prologue: K_0, K_1 in LDS; S_0.
  if (ntiles > 0) {
    issue_tile(sK[0], kp, 0);
    load_flags(0);
    store_flags(0);
    if (ntiles > 1) {
      issue_tile(sK[1], kp, 1);
      load_flags(1);
      store_flags(1);
    }
  }
  wait_vmem();
  __syncthreads();
  f32x16 s_cur[2], s_nxt[2];
  bf16x8 p_prev[4], p_cur[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p_prev[i] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  if (jw_last >= 0 && ntiles > 0) mma_s(sK[0], s_cur);
  __syncthreads();  // every wave is done with K_0 before buffer 0 is refilled

  for (int j = 0; j < ntiles; ++j) {
    const int rb = (j + 1) & 1;
    const int wb = j & 1;
    if (j + 2 < ntiles) {
      issue_tile(sK[wb], kp, j + 2);
      load_flags(j + 2);
    }
    issue_tile(sV[wb], vp, j);

    const bool do_soft = j <= jw_last;
    const bool do_s = j + 1 <= jw_last;
    const bool do_pv = j >= 1 && j - 1 <= jw_last;
    float cc = c;
    if (do_soft && tile_needs_mask(j)) {
      apply_mask(s_cur, j);
      cc = 1.f;
    }
    float alpha = 1.f;
    if (do_soft && do_s && do_pv) {
      // The steady state: three independent streams in one block.
      mma_pv(sV[rb], p_prev);
      mma_s(sK[rb], s_nxt);
      alpha = softmax(s_cur, cc, p_cur);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // up to two LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // a few VALU operations
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      }
    } else {
      if (do_pv) mma_pv(sV[rb], p_prev);
      if (do_s) mma_s(sK[rb], s_nxt);
      if (do_soft) alpha = softmax(s_cur, cc, p_cur);
    }
    if (wave_any(alpha != 1.f)) {
      const float a_ = pin_in_branch(alpha);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= a_;
    }

    wait_vmem();
    if (j + 2 < ntiles) store_flags((j + 2) % 3);
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
#pragma unroll
    for (int i = 0; i < 4; ++i) p_prev[i] = p_cur[i];
  }
  if (ntiles > 0 && ntiles - 1 <= jw_last) mma_pv(sV[(ntiles - 1) & 1], p_prev);

  // Epilogue: O = O~ / l, LSE = ln 2 * (m + log2 l).
  uint16_t* __restrict__ op = (uint16_t*)a.o + sv.base;
  const float lt = wave_sum_halves(l);
  const int qi = q_wave0 + l32;
  if (qi < sv.len) {
    const bool dead = (m == kNegInf) || !(lt > 0.f);
    const float inv = dead ? 0.f : 1.f / lt;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& x = o[db];
        u32x2 w = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                   pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
        *(u32x2*)(op + (int64_t)qi * sv.tok_stride + db * 32 + g * 8 + hi * 4) = w;
      }
    if (hi == 0) a.lse[sv.row_base + qi] = dead ? kNegInf : (m + fast_log2(lt)) * kLn2;
  }
}

template <int D, int NW, bool CAUSAL, bool VARLEN, bool KPAD>
static hipError_t launch_fwd_pipe_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BR = NW * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_pipe_kernel<D, NW, CAUSAL, VARLEN, KPAD>), dim3((unsigned)blocks), dim3(NW * 64), 0, stream,
                     a, n_qtiles);
  return hipGetLastError();
}

template <int D, int NW>
static hipError_t dispatch_fwd_pipe(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
  if (varlen) {
    if (causal) return kpad ? launch_fwd_pipe_t<D, NW, true, true, true>(a, s)
                            : launch_fwd_pipe_t<D, NW, true, true, false>(a, s);
    return kpad ? launch_fwd_pipe_t<D, NW, false, true, true>(a, s)
                : launch_fwd_pipe_t<D, NW, false, true, false>(a, s);
  }
  return causal ? launch_fwd_pipe_t<D, NW, true, false, false>(a, s)
                : launch_fwd_pipe_t<D, NW, false, false, false>(a, s);
}

// Ping-pong form of the forward.  Eight waves of 32 query rows, two per SIMD.
// Each key tile takes two barrier-separated halves, and the two waves that
// share a SIMD run different phases in the first half:
//   group A:  half 1 = S_j (MFMA) then softmax_j (VALU);  half 2 = O += V_j^T P_j
//   group B:  half 1 = softmax_{j-1} (VALU) then O += V_{j-1}^T P_{j-1} (MFMA);
//             half 2 = S_j (MFMA)
// so one wave's MFMAs overlap the other wave's softmax, and the second half,
// which is MFMA only, keeps the matrix unit busy.  Group B lags by half a tile,
// so V tiles are kept three deep in LDS (K two deep).  GSEL picks which waves
// form group B: 0 = waves 4-7, 1 = odd waves.
template <int D, bool CAUSAL, bool VARLEN, bool KPAD, int GSEL>
__global__ void __launch_bounds__(512, 1) fwd_pp_kernel(AttnArgs a, int n_qtiles) {
  constexpr int NW = 8;
  constexpr int BC = 64;
  constexpr int BR = NW * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NT = NW * 64;
  constexpr int CH_PER_ROW = D / 8;
  constexpr int CPT = BC * CH_PER_ROW / NT;
  static_assert(CPT * NT == BC * CH_PER_ROW, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[3][TILE];
  __shared__ uint8_t s_valid[2][BC];
  __shared__ uint32_t s_anypad[2];

  int bh, tile;
  wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, CAUSAL, bh, tile);  // causal: heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<VARLEN>(a, b, h, D);
  const int q_tile0 = tile * BR;
  if (q_tile0 >= sv.len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool grp_b = GSEL == 0 ? (wave >= 4) : ((wave & 1) != 0);
  const int q_wave0 = q_tile0 + wave * 32;
  const int kv_len = sv.len;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.base;

  float c = a.scale_log2;
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  c = fabsf(c);

  bf16x8 qf[KS];
  {
    const int qi = q_wave0 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (qi < kv_len) x = *(const u32x4*)(qp + (int64_t)qi * sv.tok_stride + ks * 16 + hi * 8);
      qf[ks] = as_bf16x8(x ^ qsign);
    }
  }
  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int jw_last = CAUSAL ? min(ntiles - 1, (q_wave0 + 31) / BC) : ntiles - 1;

  int st_off[CPT];
#pragma unroll
  for (int cidx = 0; cidx < CPT; ++cidx) {
    const int chunk = tid + cidx * NT;
    const int row = chunk / CH_PER_ROW;
    st_off[cidx] = swz_off<D>(row, (chunk - row * CH_PER_ROW) * 8);
  }
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
  auto store_tile = [&](int j) {
    uint16_t* sk = sK[j & 1];
    uint16_t* svv = sV[j % 3];
#pragma unroll
    for (int cidx = 0; cidx < CPT; ++cidx) {
      *(u32x4*)(sk + st_off[cidx]) = rk[cidx];
      *(u32x4*)(svv + st_off[cidx]) = rv[cidx];
    }
    if constexpr (KPAD) {
      if (wave == 0) {
        s_valid[j & 1][lane] = (uint8_t)rvalid;
        const bool any = wave_any(rvalid == 0u);
        if (lane == 0) s_anypad[j & 1] = any ? 1u : 0u;
      }
    }
  };

  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = swz_off<D>(l32, ks * 16 + hi * 8);
  const int tr_r = hi * 4 + ((lane >> 2) & 3);
  const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int voff[2][DB];
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);

  // Scores of one tile; after the softmax the same registers carry the packed
  // bf16 P (words 0-7 of s[0] and s[1]), so a single array crosses the
  // mid-tile barrier for either group.
  f32x16 s[2];
  auto p_operand = [&](int kb, int t) -> bf16x8 {
    u32x4 w = {__builtin_bit_cast(uint32_t, s[kb][4 * t + 0]), __builtin_bit_cast(uint32_t, s[kb][4 * t + 1]),
               __builtin_bit_cast(uint32_t, s[kb][4 * t + 2]), __builtin_bit_cast(uint32_t, s[kb][4 * t + 3])};
    return as_bf16x8(w);
  };

  auto mma_s = [&](int j) {
    const uint16_t* kt = sK[j & 1];
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma_bf16(as_bf16x8(*(const u32x4*)(kt + kb * 32 * D + koff[ks])), qf[ks], s[kb]);
  };
  auto mma_pv = [&](int j) {
    const uint16_t* vt = sV[j % 3];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint16_t* v0 = vt + (kb * 32 + 16 * t) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8 va = join_u32x2(lds_read_tr16(v0 + voff[0][db]), lds_read_tr16(v0 + voff[1][db]));
          o[db] = mfma_bf16(va, p_operand(kb, t), o[db]);
        }
      }
  };
  // Mask (if the tile needs it), row max, reference update, exp2, row sum,
  // bf16 packing into pb and, when a row's reference moved, the O rescale.
  auto softmax = [&](int j) {
    const int kt0 = j * BC;
    bool need_mask = kt0 + BC > kv_len;
    if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > q_wave0);
    if (KPAD) need_mask = need_mask || (s_anypad[j & 1] != 0u);
    float cc = c;
    if (need_mask) {
      cc = 1.f;
      const int qi = pin_in_branch(q_wave0 + l32);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const int key = kt0 + kl;
          bool vis = key < kv_len;
          if (CAUSAL) vis = vis && key <= qi;
          if (KPAD) vis = vis && s_valid[j & 1][kl] != 0;
          s[kb][r] = vis ? s[kb][r] * c : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_max_halves(mx) * cc;
    const float m_new = (mx > m + kLazyMax) ? mx : m;
    const bool dead = m_new == kNegInf;
    const float alpha = dead ? 1.f : fast_exp2(m - m_new);
    const float mu = dead ? 0.f : m_new;
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(__builtin_fmaf(s[kb][8 * t + i], cc, -mu));
          rs += e[i];
        }
        // words 4t..4t+3 are written only after elements 8t..8t+7 were read
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[kb][4 * t + i] = __builtin_bit_cast(float, pack_bf16x2(e[2 * i], e[2 * i + 1]));
      }
    l = alpha * l + rs;
    m = m_new;
    if (wave_any(alpha != 1.f)) {
      const float a_ = pin_in_branch(alpha);
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= a_;
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    if (j + 1 < ntiles) load_tile(j + 1);
    // half 1
    if (!grp_b) {
      if (j <= jw_last) {
        mma_s(j);
        softmax(j);
      }
    } else if (j >= 1 && j - 1 <= jw_last) {
      softmax(j - 1);
      mma_pv(j - 1);
    }
    __syncthreads();
    // half 2
    if (!grp_b) {
      if (j <= jw_last) mma_pv(j);
    } else if (j <= jw_last) {
      mma_s(j);
    }
    if (j + 1 < ntiles) store_tile(j + 1);
    __syncthreads();
  }
  if (grp_b && ntiles > 0 && ntiles - 1 <= jw_last) {
    softmax(ntiles - 1);
    mma_pv(ntiles - 1);
  }

  uint16_t* __restrict__ op = (uint16_t*)a.o + sv.base;
  const float lt = wave_sum_halves(l);
  const int qi = q_wave0 + l32;
  if (qi < sv.len) {
    const bool dead = (m == kNegInf) || !(lt > 0.f);
    const float inv = dead ? 0.f : 1.f / lt;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& x = o[db];
        u32x2 w = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                   pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
        *(u32x2*)(op + (int64_t)qi * sv.tok_stride + db * 32 + g * 8 + hi * 4) = w;
      }
    if (hi == 0) a.lse[sv.row_base + qi] = dead ? kNegInf : (m + fast_log2(lt)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool VARLEN, bool KPAD, int GSEL>
static hipError_t launch_fwd_pp_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BR = 8 * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, VARLEN, KPAD, GSEL>), dim3((unsigned)blocks), dim3(512), 0, stream, a,
                     n_qtiles);
  return hipGetLastError();
}

template <int D, int GSEL>
static hipError_t dispatch_fwd_pp(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
  if (varlen) {
    if (causal) return kpad ? launch_fwd_pp_t<D, true, true, true, GSEL>(a, s)
                            : launch_fwd_pp_t<D, true, true, false, GSEL>(a, s);
    return kpad ? launch_fwd_pp_t<D, false, true, true, GSEL>(a, s)
                : launch_fwd_pp_t<D, false, true, false, GSEL>(a, s);
  }
  return causal ? launch_fwd_pp_t<D, true, false, false, GSEL>(a, s)
                : launch_fwd_pp_t<D, false, false, false, GSEL>(a, s);
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

// Kernel variants.  MIATTN_FWD_TILE=<n> picks one for tuning sweeps:
//   0 (default, measured best) one 32-row block per wave, 8 waves, lockstep;
//   1, 2 the ping-pong form with either wave grouping; 3 the software-pipelined
//   form with 4 waves.
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
    if (t == 1) return dispatch_fwd_pp<128, 0>(a, causal, varlen, kpad, stream);
    if (t == 2) return dispatch_fwd_pp<128, 1>(a, causal, varlen, kpad, stream);
    if (t == 3) return dispatch_fwd_pipe<128, 4>(a, causal, varlen, kpad, stream);
    return dispatch_fwd<128, 1, 8, 1>(a, causal, varlen, kpad, stream);
  }
  if (d == 64) {
    if (t == 1) return dispatch_fwd_pp<64, 0>(a, causal, varlen, kpad, stream);
    if (t == 2) return dispatch_fwd_pp<64, 1>(a, causal, varlen, kpad, stream);
    if (t == 3) return dispatch_fwd_pipe<64, 4>(a, causal, varlen, kpad, stream);
    return dispatch_fwd<64, 1, 8, 1>(a, causal, varlen, kpad, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace miattn
