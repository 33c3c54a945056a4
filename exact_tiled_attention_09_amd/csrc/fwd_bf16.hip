// Fused exact attention forward, bf16 in / bf16 O / fp32 LSE, for gfx950.
//
// Method: the online-softmax forward with an unnormalised output accumulator
// and one log-sum-exp per row ("解析 FlashAttention（4）：FlashAttention-v2",
// section 四, the general forward; running state as in "分块 Attention：重建概率，
// 累计梯度", section 01).  The N x N scores never leave registers.
//
// Work decomposition (MI355X-first, not the pages' thread-block layout):
//  * one workgroup per (sequence, head, query tile of 256 rows); each of its
//    eight waves owns 32 query rows ("split-Q": no cross-wave softmax
//    traffic).
//  * the wave computes S^T = K Q^T so that the 32x32 accumulator puts one query
//    per lane column: row max / row sum are in-lane over 16 registers plus one
//    exchange with the lane 32 away, and the rescale factor is a per-lane
//    scalar.
//  * P^T leaves the accumulator already in the B-operand layout of
//    O^T += V^T P^T; V^T comes from the row-major V tile through the LDS
//    transpose read, so neither P nor V is shuffled.
//  * K/V tiles of BC = 64 keys go through three LDS buffers each (one barrier
//    per tile) in the XOR-swizzled layout of swz<D>, which keeps both the b128
//    operand reads and the transpose reads free of bank conflicts; Q stays in
//    registers for the whole key loop.
//  * softmax runs in base 2 with scale * log2(e) folded into one FMA.  A tile
//    is first exponentiated against the row's current reference without
//    forming the row max; only when a partial row sum exceeds 2^16 (or the row
//    has no reference yet) is the max taken and the reference raised (when
//    the max exceeds it by more than kLazyMax, base-2 units), O~ and l
//    rescaled and the tile redone.  Any reference value gives the same
//    O = O~ / l and LSE = m + log2 l, so this changes only rounding.
//  * causal: key tiles above the diagonal are never loaded; only tiles that
//    cross the diagonal, the sequence end or a padded key are masked
//    element-wise; each XCD takes its heads four at a time, their query tiles heaviest first (wg_coords_grouped);
//    without a causal mask all heads' tile 0 go first, then all tile 1, ...
#include "miattn_device.h"
#include "miattn_launch.h"

#include <type_traits>

namespace miattn {

// Staggered schedule with direct loads.  Eight waves of 32 query
// rows, two per SIMD, one barrier per interval.  Every wave runs, for each key tile j,
//   S_j^T = K_j Q^T (MFMA),  softmax of S_j (VALU),  O^T += V_j^T P_j^T (MFMA),
// and interval j ends after S_j for late waves and after softmax_j for early
// waves.  So within an interval an early wave issues P_{j-1} V_{j-1}, S_j and
// then softmax_j, while its late partner on the same SIMD issues softmax_{j-1}
// and then P_{j-1} V_{j-1}, S_j: one wave's vector work overlaps the other's
// matrix work.  Interval t reads K_t and V_{t-1}; K and V tiles travel from
// global memory straight into LDS (three buffers each), K_{t+2} and V_{t+1}
// being fetched during interval t, and before the barrier that ends interval
// t each wave waits only for its own loads of K_{t+1} and V_t.  Key-validity
// flags of tile t are read as late as interval t+1 and written two intervals
// ahead, so they are kept four deep.  The late waves are 4-7 (the partner of
// wave w on its SIMD is w + 4).  The loop is unrolled by the three buffers so that every LDS address is a register
// plus an immediate.
template <int D, bool CAUSAL, bool VARLEN, bool KPAD, int MASK = kMaskPlain>
__global__ void __launch_bounds__(512, 1) fwd_stag_kernel(AttnArgs a, int n_qtiles) {
  constexpr int NW = 8;
  constexpr int BC = 64;
  constexpr int BR = NW * 32;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  // Who issues the K/V tile loads.  d = 128: every wave, right after the
  // barrier that opens an interval.  d = 64: only the early waves, spread
  // over their MFMA phases (one load per four MFMAs): at d = 64 the matrix
  // phases are half as long as the softmax, so the early waves' matrix phase
  // has room for them, while loads issued after the barrier delay the
  // late waves' softmax, the longer phase (measured 5-9% faster at d = 64;
  // 2-3% slower at d = 128, where the two phases are balanced).
  constexpr bool SPREAD = D == 64;
  constexpr int NLD = SPREAD ? NT / 2 : NT;  // threads that issue tile loads
  constexpr int LPT = BC * CPR / NLD;        // direct loads per such thread per tensor and tile
  static_assert(LPT * NLD == BC * CPR, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t sK[3][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[3][TILE];
  __shared__ uint8_t s_valid[4][BC];
  __shared__ uint32_t s_anypad[4];

  int bh, tile;
  // causal masks, windows and block lists: groups of four heads per XCD,
  // heaviest tiles first in each group under a causal mask; plain non-causal:
  // the same groups when a head has 4 or more query tiles (its K/V no longer
  // fit in L2 for many heads at once), else all heads' tile 0, then all tile
  // 1, ... (measured faster for 2 tiles a head)
  // packed sequences: each XCD takes the same heads of every sequence (equal
  // work whatever the lengths; a contiguous range of sequences per XCD would
  // give one XCD the longest ones), one (sequence, head) at a time with its
  // tiles together, heaviest first
  if (VARLEN) {
    wg_coords_unit_major(blockIdx.x, a.B, a.H, n_qtiles, bh, tile);
    if (CAUSAL) tile = n_qtiles - 1 - tile;
  }
  else if (CAUSAL || MASK != kMaskPlain) wg_coords_grouped(blockIdx.x, a.B * a.H, n_qtiles, 4, CAUSAL, bh, tile);
  else if (n_qtiles >= 4) wg_coords_grouped(blockIdx.x, a.B * a.H, n_qtiles, 4, false, bh, tile);
  else wg_coords_tile_major(blockIdx.x, a.B * a.H, n_qtiles, false, bh, tile);
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
  const bool late = wave >= 4;  // the partner of wave w on its SIMD is w + 4
  const int q_wave0 = q_tile0 + wave * 32;
  const int kv_len = sv.len;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.kv_base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.kv_base;

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

  // The key tiles the workgroup visits form a list: position r holds key
  // tile tile_of(r).  Without a window or a block list it is 0 .. ntiles-1
  // (under a causal mask it ends at the diagonal); a window visits one
  // contiguous run; a block list visits both 64-key halves of every listed
  // 128-key block.  A wave computes only the positions wave_live accepts and
  // otherwise keeps pace with the others (loads and barriers).
  __shared__ uint8_t s_bflag[2][MASK == kMaskBlocks ? kMaxSparseBlocks : 1];
  __shared__ uint16_t s_blist[MASK == kMaskBlocks ? kMaxSparseBlocks : 1];
  __shared__ int s_bcount;
  int ntiles, jw_last, jt0 = 0, jw_first = 0;
  if constexpr (MASK == kMaskPlain) {
    const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
    ntiles = (kv_end + BC - 1) / BC;
    // the last key tile holding a key this wave may see
    jw_last = CAUSAL ? min(ntiles - 1, (q_wave0 + 31) / BC) : ntiles - 1;
  } else if constexpr (MASK == kMaskWindow) {
    jt0 = max(0, q_tile0 - a.win_left) / BC;
    const int kv_end = min(kv_len, q_tile0 + BR + a.win_right);
    ntiles = (kv_end + BC - 1) / BC - jt0;
    jw_first = max(0, q_wave0 - a.win_left) / BC - jt0;
    jw_last = min(ntiles - 1, (q_wave0 + 31 + a.win_right) / BC - jt0);
  } else {
    static_assert(BR == 2 * kSparseBlock, "two query blocks per workgroup");
    ntiles = 2 * build_key_block_list<NT, CAUSAL>(a, q_tile0, s_bflag, s_blist, &s_bcount);
    jw_last = ntiles - 1;
  }
  auto tile_of = [&](int r) __attribute__((always_inline)) -> int {
    if constexpr (MASK == kMaskPlain) return r;
    else if constexpr (MASK == kMaskWindow) return jt0 + r;
    else return (s_blist[r >> 1] & 0xfff) * 2 + (r & 1);
  };
  auto wave_live = [&](int r) __attribute__((always_inline)) -> bool {
    if constexpr (MASK == kMaskWindow) {
      return r >= jw_first && r <= jw_last;
    } else if constexpr (MASK == kMaskBlocks) {
      const int e = s_blist[r >> 1];
      const int kt0 = ((e & 0xfff) * 2 + (r & 1)) * BC;
      return ((e >> (12 + (wave >> 2))) & 1) != 0 && kt0 < kv_len && (!CAUSAL || kt0 <= q_wave0 + 31);
    } else {
      return true;
    }
  };

  // Direct-load sources: LDS chunk p = i*NLD + t of a tile (t the issuing
  // thread) holds row p / CPR, logical chunk (p % CPR) ^ swz(row).  Rows past
  // the sequence repeat its last row (finite values, masked in the softmax).
  int src_row[LPT], src_col[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int pch = i * NLD + (SPREAD ? (tid & (NLD - 1)) : tid);
    const int row = pch / CPR;
    src_row[i] = row;
    src_col[i] = ((pch % CPR) ^ swz<D>(row)) << 3;
  }
  // Load i of the key tile starting at key k0 into dst.  In the spread form
  // the wave's LDS base passes through an empty asm at each call, so the
  // compiler forms every M0 value where it is used rather than keeping one
  // scalar register per slot and chunk.
  auto dma = [&](const uint16_t* src, uint16_t* dst, int k0, int i) __attribute__((always_inline)) {
    const int key = min(k0 + src_row[i], kv_len - 1);
    if constexpr (SPREAD) {
      uint32_t wb = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MIATTN_LDS void*)(dst + wave * 64 * 8));
      __asm__ volatile("" : "+s"(wb));
      lds_dma16_m0(src + (int64_t)key * sv.kv_stride + src_col[i], wb + i * NLD * 16);
    } else {
      lds_dma16(src + (int64_t)key * sv.kv_stride + src_col[i], dst + (i * NLD + wave * 64) * 8);
    }
  };
  auto issue = [&](const uint16_t* src, uint16_t* dst, int j) __attribute__((always_inline)) {
    const int k0 = tile_of(j) * BC;
#pragma unroll
    for (int i = 0; i < LPT; ++i) dma(src, dst, k0, i);
  };
  // Key-validity flags of a tile, by wave 0.  The raw byte is loaded early
  // and converted only when stored: a use right after the load would make
  // the compiler wait there for every load in flight (vmcnt(0)), the tile
  // loads issued just before it included.
  uint32_t rvalid = 1u;
  int rkey = 0;
  auto load_flags = [&](int j) __attribute__((always_inline)) {
    if constexpr (KPAD) {
      if (wave == 0) {
        rkey = j * BC + lane;
        rvalid = a.key_valid[sv.tok0 + min(rkey, kv_len - 1)];
      }
    }
  };
  auto store_flags = [&](int j) __attribute__((always_inline)) {
    if constexpr (KPAD) {
      if (wave == 0) {
        const uint32_t ok = (rkey >= kv_len || rvalid != 0u) ? 1u : 0u;  // keys past the end are masked anyway
        s_valid[j & 3][lane] = (uint8_t)ok;
        const bool any = wave_any(ok == 0u);
        if (lane == 0) s_anypad[j & 3] = any ? 1u : 0u;
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

  f32x16 s[2];   // scores of the tile formed last
  bf16x8 p[4];   // packed P of the tile softmaxed last

  // The buffer slot (j % 3) is passed as a compile-time constant so that
  // every LDS address is a register plus an immediate.
  // The MFMA phases read their LDS operands ahead of use (K two k-steps,
  // V three MFMAs), so that a wave whose partner is busy with vector work
  // does not wait a full LDS latency before every MFMA.
  // Spread form: S_j carries the early wave's loads of V_{j+1}, P_j V_j those
  // of K_{j+3} (with the key flags of tile j+3).
  constexpr int S_STEP = KS / LPT;       // k-steps of S between two loads
  constexpr int PV_STEP = 4 * DB / LPT;  // MFMAs of P V between two loads
  static_assert(!SPREAD || (S_STEP * LPT == KS && PV_STEP * LPT == 4 * DB && S_STEP >= 1 && PV_STEP >= 1),
                "load spread");
  auto mma_s = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const uint16_t* kt = sK[SL];
    const bool ld = SPREAD && !late && j + 1 < ntiles;
    const int k0n = ld ? tile_of(j + 1) * BC : 0;
    s[0] = f32x16{};
    s[1] = f32x16{};
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
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_bf16(ka[ks % 3][kb], qf[ks], s[kb]);
      if (SPREAD && ks % S_STEP == S_STEP - 1 && ld) dma(vp, sV[(SL + 1) % 3], k0n, ks / S_STEP);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto mma_pv = [&](auto slot_c, int j) __attribute__((always_inline)) {
    constexpr int NPV = 4 * DB;
    constexpr int PF = 3;
    constexpr int SL = decltype(slot_c)::value;
    const uint16_t* vt = sV[SL];
    const bool ld = SPREAD && !late && j + 3 < ntiles;
    const int k0n = ld ? tile_of(j + 3) * BC : 0;
    if (ld) load_flags(j + 3);
    auto vread = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      const uint16_t* v0 = vt + (i / DB) * 16 * D;  // keys 16 (i / DB) .. +15
      return join_u32x2(lds_read_tr16(v0 + voff[0][i % DB]), lds_read_tr16(v0 + voff[1][i % DB]));
    };
    bf16x8 va[NPV];
#pragma unroll
    for (int i = 0; i < PF; ++i) va[i] = vread(i);
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      if (i + PF < NPV) va[i + PF] = vread(i + PF);
      o[i % DB] = mfma_bf16(va[i], p[i / DB], o[i % DB]);
      if (SPREAD && i % PV_STEP == PV_STEP - 1 && ld) dma(kp, sK[SL], k0n, i / PV_STEP);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // The VALU block for tile j.
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int kt0 = tile_of(j) * BC;
    bool need_mask = kt0 + BC > kv_len;
    if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > q_wave0);
    if (KPAD) need_mask = need_mask || (s_anypad[j & 3] != 0u);
    if (MASK == kMaskWindow)
      need_mask = need_mask || (kt0 < q_wave0 + 31 - a.win_left) || (kt0 + BC - 1 > q_wave0 + a.win_right);
    float cc = c;
    if (need_mask) {
      // Scale first, then hide masked entries as -inf; afterwards the
      // exponent uses multiplier 1 (so scale == 0 cannot make 0 * -inf).
      cc = 1.f;
      if constexpr (!KPAD && MASK != kMaskWindow) {
        // sequence end and causal diagonal only: entry r of key block kb
        // holds key kt0 + kb*32 + (r/4)*8 + hi*4 + r%4, visible iff its
        // offset kb*32 + (r/4)*8 + r%4 is at most this lane's bound
        int lim = kv_len - 1 - kt0 - hi * 4;
        if (CAUSAL) lim = min(lim, q_wave0 + l32 - kt0 - hi * 4);
        lim = pin_in_branch(lim);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] = (kb * 32 + (r >> 2) * 8 + (r & 3) <= lim) ? s[kb][r] * c : kNegInf;
      } else {
        const int qi = pin_in_branch(q_wave0 + l32);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kl = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            const int key = kt0 + kl;
            bool vis = key < kv_len;
            if (CAUSAL) vis = vis && key <= qi;
            if (KPAD) vis = vis && s_valid[j & 3][kl] != 0;
            if (MASK == kMaskWindow) vis = vis && key >= qi - a.win_left && key <= qi + a.win_right;
            s[kb][r] = vis ? s[kb][r] * c : kNegInf;
          }
      }
    }
    auto expo = [&](float mu) __attribute__((always_inline)) -> float {
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
      return rs;
    };
    // P against the current reference first, without the row max.  Only
    // when a lane's partial row sum leaves (0, 2^16] -- the row's scores rose
    // well above the reference, a NaN or Inf score, or no reference yet
    // (m = -inf) -- does the wave take the row max, move the reference (when
    // the max exceeds it by more than kLazyMax), rescale and redo the tile.
    // Any reference gives the same O = O~ / l and LSE = m + log2 l; this one
    // only keeps every P below 2^16.
    float rs = expo(m == kNegInf ? 0.f : m);
    if (wave_any(!(rs <= kSumLimit) || m == kNegInf)) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx *= cc;
      if (wave_any(!(mx <= m + kLazyMax))) {
        mx = wave_max_halves(mx);
        const float m_new = (mx > m + kLazyMax) ? mx : m;
        const bool dead = m_new == kNegInf;
        const float alpha = dead ? 1.f : fast_exp2(m - m_new);
        l *= alpha;
        m = m_new;
        if (wave_any(alpha != 1.f)) {
          const float a_ = pin_in_branch(alpha);
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= a_;
        }
      }
      rs = expo(m == kNegInf ? 0.f : m);
    }
    l += rs;
  };

  // Interval t fetches K_{t+2} (with the flags of tile t+2, stored at the end
  // of the interval) and V_{t+1}: every wave right after the barrier that
  // opens the interval, or, in the spread form, an early wave inside
  // P_{t-1} V_{t-1} and S_t (right after the barrier when it skips one of
  // them).  The barrier ending interval t needs K_{t+1} and V_t (interval
  // t-1's loads) and lets interval t's own loads stay in flight.
  auto begin_interval = [&](int t) __attribute__((always_inline)) {
    if (t + 2 < ntiles) {
      load_flags(t + 2);
      issue(kp, sK[(t + 2) % 3], t + 2);
    }
    if (t + 1 < ntiles) issue(vp, sV[(t + 1) % 3], t + 1);
  };
  // Whether this wave computes key tile j (S_j, softmax_j and P_j V_j).
  auto live = [&](int j) __attribute__((always_inline)) -> bool {
    if (j < 0 || j >= ntiles) return false;
    if constexpr (MASK == kMaskPlain) return j <= jw_last;
    else return wave_live(j);
  };
  auto end_interval = [&](int t) __attribute__((always_inline)) {
    if constexpr (SPREAD) {
      if (!late) {
        if (t + 2 < ntiles) store_flags(t + 2);
        const int pending = (t + 2 < ntiles ? LPT : 0) + (t + 1 < ntiles ? LPT : 0);
        if (pending == 2 * LPT) barrier_vmem_n<2 * LPT>();
        else if (pending == LPT) barrier_vmem_n<LPT>();
        else barrier_vmem_n<0>();
        if (!live(t) && t + 3 < ntiles) {
          load_flags(t + 3);
          issue(kp, sK[(t + 3) % 3], t + 3);
        }
        if (!live(t + 1) && t + 2 < ntiles) issue(vp, sV[(t + 2) % 3], t + 2);
      } else {
        barrier_vmem_n<0>();  // the late waves hold no loads
      }
    } else {
      if (t + 2 < ntiles) store_flags(t + 2);
      const int pending = (t + 2 < ntiles ? LPT : 0) + (t + 1 < ntiles ? LPT : 0);
      if (pending == 2 * LPT) barrier_vmem_n<2 * LPT>();
      else if (pending == LPT) barrier_vmem_n<LPT>();
      else barrier_vmem_n<0>();
      begin_interval(t + 1);
    }
  };

  // An empty block list leaves every row without a key (O = 0, LSE = -inf).
  if (MASK != kMaskBlocks || ntiles > 0) {
    // Prologue: K_0, K_1, V_0 and the flags of tiles 0 and 1; in the spread
    // form (early waves only) also interval 0's K_2, since no P V precedes
    // S_0.  K_0 must land.
    if constexpr (SPREAD) {
      if (!late) {
        load_flags(0);
        store_flags(0);
        issue(kp, sK[0], 0);
        if (ntiles > 1) {
          load_flags(1);
          store_flags(1);
          issue(kp, sK[1], 1);
        }
        issue(vp, sV[0], 0);
        if (ntiles > 2) {
          load_flags(2);
          issue(kp, sK[2], 2);
        }
        const int pending = (ntiles > 1 ? LPT : 0) + LPT + (ntiles > 2 ? LPT : 0);
        if (pending == 3 * LPT) barrier_vmem_n<3 * LPT>();
        else if (pending == 2 * LPT) barrier_vmem_n<2 * LPT>();
        else barrier_vmem_n<LPT>();
        if (!live(0) && ntiles > 1) issue(vp, sV[1], 1);
      } else {
        barrier_vmem_n<0>();
      }
    } else {
      load_flags(0);
      store_flags(0);
      issue(kp, sK[0], 0);
      if (ntiles > 1) {
        load_flags(1);
        store_flags(1);
        issue(kp, sK[1], 1);
      }
      issue(vp, sV[0], 0);
      if (ntiles > 1) barrier_vmem_n<2 * LPT>();  // K_0 has landed
      else barrier_vmem_n<LPT>();
      begin_interval(0);
    }

    // Every wave passes ntiles + 1 barriers after the prologue: one per key
    // tile it works on or skips, then the remaining intervals up to ntiles.
    auto body = [&](int j, auto slot_c) __attribute__((always_inline)) {
      if constexpr (MASK != kMaskPlain) {
        if (!wave_live(j)) {
          end_interval(j);
          return;
        }
      }
      mma_s(slot_c, j);
      if (late) end_interval(j);
      softmax(j);
      if (!late) end_interval(j);
      mma_pv(slot_c, j);
    };
    const int j_end = MASK == kMaskPlain ? jw_last : ntiles - 1;
    for (int j = 0; j <= j_end; j += 3) {
      body(j, std::integral_constant<int, 0>{});
      if (j + 1 <= j_end) body(j + 1, std::integral_constant<int, 1>{});
      if (j + 2 <= j_end) body(j + 2, std::integral_constant<int, 2>{});
    }
    for (int t = j_end + 1; t <= ntiles; ++t) end_interval(t);
  }

  // Epilogue: O = O~ / l, LSE = ln 2 * (m + log2 l); a row that saw no
  // visible key gets O = 0 and LSE = -inf.  The wave's 32 x D block of O
  // goes through LDS (idle after the last barrier: every wave has waited for
  // its own LDS reads before it) so that the global stores are whole rows,
  // 16 bytes per lane: in the accumulator layout a store instruction would
  // touch 32 rows.  Staging rows are row-major with 16-byte chunk c of row r
  // at chunk c ^ (r mod CPR); waves 0-5 stage in the K buffers, 6 and 7 in
  // the V buffers.
  uint16_t* __restrict__ op = (uint16_t*)a.o + sv.base;
  const float lt = wave_sum_halves(l);
  const int qi = q_wave0 + l32;
  // dead: no visible key (max -inf, sum 0); a NaN score leaves the max at
  // -inf (max ignores NaN) but the sum NaN, and the row comes out NaN
  const bool dead = (m == kNegInf) && !(lt != lt);
  const float inv = dead ? 0.f : 1.f / lt;
  static_assert(6 * 32 * D <= 3 * TILE && 2 * 32 * D <= 3 * TILE, "staging fits the tile buffers");
  uint16_t* stage = wave < 6 ? &sK[0][0] + wave * 32 * D : &sV[0][0] + (wave - 6) * 32 * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16& x = o[db];
      u32x2 w = {pack_bf16x2(x[4 * g + 0] * inv, x[4 * g + 1] * inv),
                 pack_bf16x2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
      const int c = db * 4 + g;
      *(u32x2*)(stage + l32 * D + ((c ^ (l32 % CPR)) << 3) + hi * 4) = w;
    }
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR;
    const int c = lane % CPR;
    const u32x4 w = *(const u32x4*)(stage + r * D + ((c ^ (r % CPR)) << 3));
    if (q_wave0 + r < sv.len) *(u32x4*)(op + (int64_t)(q_wave0 + r) * sv.tok_stride + c * 8) = w;
  }
  if (qi < sv.len && hi == 0) a.lse[sv.row_base + qi] = dead ? kNegInf : (m + fast_log2(lt)) * kLn2;
}

template <int D, bool CAUSAL, bool VARLEN, bool KPAD, int MASK = kMaskPlain>
static hipError_t launch_fwd_stag_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BR = 8 * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_stag_kernel<D, CAUSAL, VARLEN, KPAD, MASK>), dim3((unsigned)blocks), dim3(512), 0,
                     stream, a, n_qtiles);
  return hipGetLastError();
}

template <int D>
static hipError_t dispatch_fwd_stag(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
  if (varlen) {
    if (causal) return kpad ? launch_fwd_stag_t<D, true, true, true>(a, s)
                            : launch_fwd_stag_t<D, true, true, false>(a, s);
    return kpad ? launch_fwd_stag_t<D, false, true, true>(a, s)
                : launch_fwd_stag_t<D, false, true, false>(a, s);
  }
  return causal ? launch_fwd_stag_t<D, true, false, false>(a, s)
                : launch_fwd_stag_t<D, false, false, false>(a, s);
}

hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream) {
  const bool kpad = varlen && a.key_valid != nullptr;
  if (d == 128) return dispatch_fwd_stag<128>(a, causal, varlen, kpad, stream);
  if (d == 64) return dispatch_fwd_stag<64>(a, causal, varlen, kpad, stream);
  return hipErrorInvalidValue;
}

// Dense layout with a sliding window (causal folded into the window) or a
// block-sparse list (with or without the causal mask): the staggered form.
hipError_t launch_fwd_masked_bf16(const AttnArgs& a, int d, int mask, bool causal, hipStream_t stream) {
  if (mask == kMaskWindow) {
    if (d == 128) return launch_fwd_stag_t<128, false, false, false, kMaskWindow>(a, stream);
    if (d == 64) return launch_fwd_stag_t<64, false, false, false, kMaskWindow>(a, stream);
  } else if (mask == kMaskBlocks) {
    if (d == 128)
      return causal ? launch_fwd_stag_t<128, true, false, false, kMaskBlocks>(a, stream)
                    : launch_fwd_stag_t<128, false, false, false, kMaskBlocks>(a, stream);
    if (d == 64)
      return causal ? launch_fwd_stag_t<64, true, false, false, kMaskBlocks>(a, stream)
                    : launch_fwd_stag_t<64, false, false, false, kMaskBlocks>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace miattn
