// Forward with split roles per SIMD (selected with MIATTN_FWD_TILE=7, dense
// layout): the online-softmax forward of "解析 FlashAttention（4）" section 四,
// with the work of one 64-row query block shared by two waves on one SIMD.
//
//  * The S wave (waves 0-3) holds Q^T of its 64 rows in registers and forms
//    S^T = K Q^T for a 64-key tile: every K fragment read from LDS feeds two
//    MFMAs (the two 32-row halves), half the LDS operand traffic per MFMA of
//    one 32-row wave.  It runs the softmax (lazy reference max, base 2) and
//    hands P^T, already packed as MFMA operands, to its partner through LDS
//    in register order (lane l writes and the partner's lane l reads the same
//    16 bytes), together with the rescale factors of the tile.
//  * The PV wave (waves 4-7, wave w + 4 shares a SIMD with wave w) holds O^T
//    of the 64 rows and forms O^T = alpha O^T + V^T P^T one tile behind: every
//    V^T fragment (transpose read) feeds two MFMAs as well.
// While one wave of a SIMD runs vector work (the softmax), the other keeps
// the matrix core busy.  Measured at B4 H32 N4096 d128 causal: 0.635 ms
// against 0.585 ms for the staggered form: the softmax of 64 rows in one wave
// issues in order and no longer hides under the other wave's MFMAs the way two
// 32-row waves interleave (raising the S wave's priority during its MFMAs
// made it slower still).  Kept as a variant.  K tiles are loaded one interval ahead and V tiles in
// the interval before their use; two LDS slots each, plus two P slots per
// wave pair: 128 KiB + 4 KiB of LDS.  Intervals are separated by one
// workgroup barrier; every wave passes ntiles + 2 barriers.
#include "miattn_device.h"
#include "miattn_launch.h"

#include <type_traits>

namespace miattn {

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_split_kernel(AttnArgs a, int n_qtiles) {
  constexpr int NW = 8;
  constexpr int BC = 64;                // keys per tile
  constexpr int BR = 256;               // 4 wave pairs x 64 rows
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  constexpr int LPT = BC * CPR / NT;    // direct loads per thread per tile and tensor
  constexpr int NOP = 8;                // P operands per lane: 2 halves x 4 chunks of 16 keys
  static_assert(LPT * NT == BC * CPR, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t sK[2][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][TILE];
  __shared__ __attribute__((aligned(16))) u32x4 sP[2][4][NOP][64];   // slot, pair, operand, lane
  __shared__ __attribute__((aligned(16))) f32x2 sA[2][4][64];        // slot, pair, lane: the halves' alpha
  __shared__ __attribute__((aligned(16))) f32x4 sML[4][64];          // pair, lane: m0, l0, m1, l1

  int bh, tile;
  wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, CAUSAL, bh, tile);  // causal: heaviest first
  const int b = bh / a.H;
  const int h = bh - b * a.H;
  const SeqView sv = seq_view<false>(a, b, h, D);
  const int q_tile0 = tile * BR;
  if (q_tile0 >= sv.len) return;  // uniform across the workgroup, before any barrier

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool s_role = wave < 4;
  const int pair = wave & 3;
  const int pq0 = q_tile0 + pair * 64;
  const int kv_len = sv.len;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.kv_base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.kv_base;

  float c = a.scale_log2;
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  c = fabsf(c);

  const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int jp_last = CAUSAL ? min(ntiles - 1, (pq0 + 63) / BC) : ntiles - 1;  // the pair's last tile

  int src_row[LPT], src_col[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int pch = i * NT + tid;
    const int row = pch / CPR;
    src_row[i] = row;
    src_col[i] = ((pch % CPR) ^ swz<D>(row)) << 3;
  }
  auto issue = [&](const uint16_t* src, uint16_t* dst, int j) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = min(j * BC + src_row[i], kv_len - 1);
      lds_dma16(src + (int64_t)key * sv.kv_stride + src_col[i], dst + (i * NT + wave * 64) * 8);
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

  // The interval loop, run by both roles with their own work: interval i
  // issues the loads of K(i+1) and V(i), then the role's work, then one
  // barrier (all loads of the interval landed, the hand-over written).  Both
  // roles pass the same ntiles + 2 barriers.
  auto run = [&](auto work) __attribute__((always_inline)) {
    auto interval = [&](int i, auto par_c) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_c)::value;   // i % 2
      if (i + 1 < ntiles) issue(kp, sK[PAR ^ 1], i + 1);
      if (i < ntiles) issue(vp, sV[PAR], i);
      work(i, par_c);
      barrier_vmem_n<0>();
    };
    issue(kp, sK[0], 0);
    barrier_vmem_n<0>();
    for (int i = 0; i <= ntiles; i += 2) {
      interval(i, std::integral_constant<int, 0>{});
      if (i + 1 <= ntiles) interval(i + 1, std::integral_constant<int, 1>{});
    }
  };

  if (s_role) {
    // S role: Q^T of both halves in registers, running max and sum per half.
    bf16x8 qf[2][KS];
    float m[2] = {kNegInf, kNegInf}, l[2] = {0.f, 0.f};
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = pq0 + qb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qi < kv_len) x = *(const u32x4*)(qp + (int64_t)qi * sv.tok_stride + ks * 16 + hi * 8);
        qf[qb][ks] = as_bf16x8(x ^ qsign);
      }
    }
    // S^T = K Q^T for tile j from slot P, the softmax, and the hand-over.
    auto s_work = [&](int j, auto slot_c) __attribute__((always_inline)) {
      constexpr int P = decltype(slot_c)::value;
      const uint16_t* kt = sK[P];
      f32x16 s[2][2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[qb][0] = s[qb][1] = f32x16{};
      bf16x8 ka[3][2];
      auto kread = [&](int ks, bf16x8 (&dst)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) dst[kb] = as_bf16x8(*(const u32x4*)(kt + kb * 32 * D + koff[ks]));
      };
      kread(0, ka[0]);
      kread(1, ka[1]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (ks + 2 < KS) kread(ks + 2, ka[(ks + 2) % 3]);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[qb][kb] = mfma_bf16(ka[ks % 3][kb], qf[qb][ks], s[qb][kb]);
        __builtin_amdgcn_sched_barrier(0);
      }
      const int kt0 = j * BC;
      float al[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int r0 = pq0 + qb * 32;
        bool need_mask = kt0 + BC > kv_len;
        if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > r0);
        float cc = c;
        if (need_mask) {
          cc = 1.f;
          const int qi = pin_in_branch(r0 + l32);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = kt0 + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
              bool vis = key < kv_len;
              if (CAUSAL) vis = vis && key <= qi;
              s[qb][kb][r] = vis ? s[qb][kb][r] * c : kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = wave_max_halves(mx) * cc;
        const float m_new = (mx > m[qb] + kLazyMax) ? mx : m[qb];
        const bool dead = m_new == kNegInf;
        const float alpha = dead ? 1.f : fast_exp2(m[qb] - m_new);
        const float mu = dead ? 0.f : m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              e[i] = fast_exp2(__builtin_fmaf(s[qb][kb][8 * t + i], cc, -mu));
              rs += e[i];
            }
            sP[P][pair][qb * 4 + kb * 2 + t][lane] =
                as_u32x4(pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]));
          }
        l[qb] = alpha * l[qb] + rs;
        m[qb] = m_new;
        al[qb] = alpha;
      }
      sA[P][pair][lane] = f32x2{al[0], al[1]};
    };
    run([&](int i, auto par_c) __attribute__((always_inline)) {
      if (i <= jp_last) s_work(i, par_c);
    });
    // publish (m, l) of both halves and write LSE (a row that saw no key:
    // LSE = -inf)
    const float l0 = wave_sum_halves(l[0]);
    const float l1 = wave_sum_halves(l[1]);
    sML[pair][lane] = f32x4{m[0], l0, m[1], l1};
    if (hi == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int qi = pq0 + qb * 32 + l32;
        const float lt = qb ? l1 : l0;
        const bool dead = (m[qb] == kNegInf) || !(lt > 0.f);
        if (qi < kv_len) a.lse[sv.row_base + qi] = dead ? kNegInf : (m[qb] + fast_log2(lt)) * kLn2;
      }
    }
    __syncthreads();
  } else {
    // PV role: O^T of both halves.
    f32x16 o[2][DB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
    // O^T = alpha O^T + V^T P^T for tile j from slot P.
    auto pv_work = [&](auto slot_c) __attribute__((always_inline)) {
      constexpr int P = decltype(slot_c)::value;
      const f32x2 al = sA[P][pair][lane];
      if (wave_any(al[0] != 1.f || al[1] != 1.f)) {
        const float a0 = pin_in_branch(al[0]);
        const float a1 = pin_in_branch(al[1]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          o[0][db] *= a0;
          o[1][db] *= a1;
        }
      }
      const uint16_t* vt = sV[P];
      auto vread = [&](int kc, int db) __attribute__((always_inline)) -> bf16x8 {
        const uint16_t* v0 = vt + kc * 16 * D;
        return join_u32x2(lds_read_tr16(v0 + voff[0][db]), lds_read_tr16(v0 + voff[1][db]));
      };
      constexpr int NPV = 4 * DB;
      constexpr int PF = 3;
      bf16x8 va[NPV];
#pragma unroll
      for (int i = 0; i < PF; ++i) va[i] = vread(i / DB, i % DB);
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16x8 p0 = as_bf16x8(sP[P][pair][kc][lane]);
        const bf16x8 p1 = as_bf16x8(sP[P][pair][4 + kc][lane]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int i = kc * DB + db;
          if (i + PF < NPV) va[i + PF] = vread((i + PF) / DB, (i + PF) % DB);
          o[0][db] = mfma_bf16(va[i], p0, o[0][db]);
          o[1][db] = mfma_bf16(va[i], p1, o[1][db]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    run([&](int i, auto par_c) __attribute__((always_inline)) {
      constexpr int PAR = decltype(par_c)::value;
      if (i >= 1 && i - 1 <= jp_last) pv_work(std::integral_constant<int, PAR ^ 1>{});
    });
    __syncthreads();
    // O = O~ / l (a row that saw no key: O = 0)
    const f32x4 ml = sML[pair][lane];
    uint16_t* __restrict__ op = (uint16_t*)a.o + sv.base;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qi = pq0 + qb * 32 + l32;
      const float mm = qb ? ml[2] : ml[0];
      const float lt = qb ? ml[3] : ml[1];
      const bool dead = (mm == kNegInf) || !(lt > 0.f);
      const float inv = dead ? 0.f : 1.f / lt;
      if (qi < kv_len) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x16& x = o[qb][db];
            u32x2 w = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                       pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
            *(u32x2*)(op + (int64_t)qi * sv.tok_stride + db * 32 + g * 8 + hi * 4) = w;
          }
      }
    }
  }
}

hipError_t launch_fwd_split_bf16(const AttnArgs& a, int d, bool causal, hipStream_t stream) {
  constexpr int BR = 256;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 128) {
    if (causal)
      hipLaunchKernelGGL((fwd_split_kernel<128, true>), dim3((unsigned)blocks), dim3(512), 0, stream, a, n_qtiles);
    else
      hipLaunchKernelGGL((fwd_split_kernel<128, false>), dim3((unsigned)blocks), dim3(512), 0, stream, a, n_qtiles);
  } else if (d == 64) {
    if (causal)
      hipLaunchKernelGGL((fwd_split_kernel<64, true>), dim3((unsigned)blocks), dim3(512), 0, stream, a, n_qtiles);
    else
      hipLaunchKernelGGL((fwd_split_kernel<64, false>), dim3((unsigned)blocks), dim3(512), 0, stream, a, n_qtiles);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace miattn
