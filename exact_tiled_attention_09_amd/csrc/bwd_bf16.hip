// Exact attention backward, bf16 operands with fp32 accumulation, for gfx950.
//
// Method ("解析 FlashAttention（4）：FlashAttention-v2", section 五: the softmax
// gradient 5.1, the D identity 5.2 and the general backward 5.4; the LSE
// reconstruction of "分块 Attention：重建概率，累计梯度", section 04):
//   D = rowsum(dO o O);  P = exp(S - LSE);  dV = P^T dO;  dP = dO V^T;
//   dS = P o (dP - D);  dQ = scale dS K;  dK = scale dS^T Q.
//
// Three kernels, all on the caller's stream:
//  1. bwd_prep: D for every row, in fp32.
//  2. bwd_dkdv: key-tile outer loop (the pages' loop order for dK and dV):
//     one workgroup per (sequence, head, 128-key tile); each of 4 waves owns
//     32 keys and keeps their dK/dV accumulators in registers.  For every
//     64-row query tile at or after the diagonal it rebuilds S = Q K^T and
//     P = exp(S - LSE), forms dP = dO V^T and dS, and accumulates dV += P^T dO
//     and dK += dS^T Q.  S and dS leave the accumulator already in A-operand
//     layout (lane = key); dO and Q enter through the LDS transpose read.
//  3. bwd_dq: query-tile outer loop, shaped like the forward (and on its
//     staggered schedule): one workgroup per (sequence, head, 256-row query
//     tile), 8 waves of 32 rows with Q and dO resident in registers.  For
//     every key tile up to the diagonal it rebuilds S^T = K Q^T and
//     dP^T = V dO^T (lane = query, so LSE and D are per-lane scalars) and
//     accumulates dQ^T += K^T dS^T.
// The pages accumulate dQ with atomic adds from the key-tile loop.  Here dQ
// gets its own pass instead: it re-forms S and dP (two more N^2 d products),
// but on MI355X device-scope float atomics are performed past the per-XCD L2,
// and at B4 H32 N4096 d128 they moved 4.7 GB per backward through memory.
// The split also makes dQ, like dK and dV, bitwise reproducible.
//
// All K / V / Q / dO tiles in LDS use the XOR swizzle of swz<D>.
#include "miattn_device.h"
#include "miattn_launch.h"

#include <type_traits>

namespace miattn {

// ---------------------------------------------------------------- kernel 1
// Rows are (batch, head, token) for dense tensors and (token, head) for packed
// ones; both flatten to row r with features at r*D in memory order, while D is
// stored like LSE ([B,H,N] or [H,T]).
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
// NW = 4: each wave owns 32 keys and both 32-row halves of every query tile.
// NW = 8: waves w and w+4 own the same 32 keys and split the query tile by
// halves, two waves per SIMD; their partial dK/dV are summed through LDS at
// the end.
template <int D, int NW, bool CAUSAL, bool VARLEN, bool KPAD, int MASK = kMaskPlain>
__global__ void __launch_bounds__(NW * 64, 1) bwd_dkdv_kernel(AttnArgs a, int n_ktiles) {
  constexpr int NT = NW * 64;
  constexpr int BK = 128;            // keys per workgroup (4 blocks of 32)
  constexpr int BQ = 64;             // query rows per step
  constexpr int KS = D / 16;         // k-steps over the head dim
  constexpr int DB = D / 32;
  constexpr int CH_PER_ROW = D / 8;
  constexpr int QCPT = BQ * CH_PER_ROW / NT;  // 16-byte chunks per thread, Q tile
  constexpr int KCPT = BK * CH_PER_ROW / NT;
  constexpr int QHALVES = NW == 4 ? 2 : 1;     // query halves handled per wave
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");

  // One LDS arena: Q and dO (double-buffered), then K and V (resident);
  // after the loop it is reused to sum the partial accumulators of the
  // 8-wave form.  The per-step Q/dO buffers come first so that, at D = 128,
  // every one of their offsets fits the 16-bit immediate of an LDS read.
  constexpr int KV_ELEMS = BK * D;
  constexpr int QT_ELEMS = BQ * D;
  __shared__ __attribute__((aligned(16))) uint16_t arena[2 * KV_ELEMS + 4 * QT_ELEMS];
  uint16_t* const sQb = arena;                              // [2][QT_ELEMS]
  uint16_t* const sGb = arena + 2 * QT_ELEMS;               // [2][QT_ELEMS]
  uint16_t* const sK = arena + 4 * QT_ELEMS;
  uint16_t* const sV = arena + 4 * QT_ELEMS + KV_ELEMS;
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];   // LSE * log2(e), +inf if dead
  __shared__ __attribute__((aligned(16))) float sDv[2][BQ];  // -D (the starting value of dP - D)

  // One workgroup per (sequence, key/value head, key tile).  With grouped
  // heads it runs the query-tile loop once for each of the G query heads
  // that read this key/value head, so dK and dV sum over the group in
  // registers.
  int bh, kt;
  int chunk = 0;  // block list: which chunk of the key block's query list
  if constexpr (MASK == kMaskBlocks) {
    // one work item (key block, chunk) of the balanced list per workgroup
    bh = blockIdx.x / a.blk_max_work;
    const int wi = blockIdx.x - bh * a.blk_max_work;
    if (wi >= a.blk_work[0]) return;  // uniform, before any barrier
    const int item = a.blk_work[1 + wi];
    kt = item & 0xffff;
    chunk = item >> 16;
  } else {
    // the earliest key tiles carry the most work; packed sequences: each XCD
    // takes the same heads of every sequence, one (sequence, head) at a time
    if (VARLEN) wg_coords_unit_major(blockIdx.x, a.B, a.Hkv, n_ktiles, bh, kt);
    else wg_coords(blockIdx.x, a.B * a.Hkv, n_ktiles, false, bh, kt);
  }
  const int G = a.H / a.Hkv;
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const SeqView sv = seq_view<VARLEN>(a, b, hk * G, D);  // query head hk*G: the first of the group
  const int64_t qhs = q_head_stride<VARLEN>(a, D);
  const int64_t rhs = row_head_stride<VARLEN>(a);
  const int k0 = kt * BK;
  if (k0 >= sv.len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int len = sv.len;
  const float c = a.scale_log2;
  const int kblk = wave & 3;                 // which 32 keys
  const int qh0 = NW == 4 ? 0 : (wave >> 2); // first query half handled

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.kv_base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.kv_base;
  const uint16_t* __restrict__ gp = (const uint16_t*)a.dout + sv.base;

  const int wk0 = k0 + kblk * 32;  // this wave's 32 keys
  const int my_key = wk0 + l32;
  bool key_ok = my_key < len;
  if constexpr (KPAD) {
    if (key_ok) key_ok = a.key_valid[sv.tok0 + my_key] != 0;
  }
  const bool any_bad_key = wave_any(!key_ok);

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // The query tiles a key tile meets: qt_begin .. qt_begin + nsteps - 1
  // (from the diagonal on under a causal mask; the run a window allows), or
  // with a block list both 64-row halves of every 128-row query block that
  // lists this key block (tile_at(p) = 2 * s_qlist[p / 2] + p % 2).
  const int n_qt = (len + BQ - 1) / BQ;
  __shared__ uint16_t s_qlist[MASK == kMaskBlocks ? kMaxSparseBlocks : 1];
  __shared__ int s_qcount;
  int qt_begin = 0, nsteps, seg0 = 0;
  if constexpr (MASK == kMaskPlain) {
    qt_begin = CAUSAL ? k0 / BQ : 0;
    nsteps = n_qt - qt_begin;
  } else if constexpr (MASK == kMaskWindow) {
    qt_begin = max(0, k0 - a.win_right) / BQ;
    nsteps = min(n_qt - 1, (k0 + BK - 1 + a.win_left) / BQ) - qt_begin + 1;
  } else {
    static_assert(BK == kSparseBlock && 2 * BQ == kSparseBlock, "one key block per workgroup");
    const int count = build_query_block_list<CAUSAL>(a, kt, s_qlist, &s_qcount);
    seg0 = chunk * a.blk_chunk;  // this workgroup's part of the list
    nsteps = 2 * max(0, min(count - seg0, a.blk_chunk));
  }
  auto tile_at = [&](int p) __attribute__((always_inline)) -> int {
    if constexpr (MASK == kMaskBlocks) return 2 * (int)s_qlist[seg0 + (p >> 1)] + (p & 1);
    else return qt_begin + p;
  };
  // Steps v = 0 .. nv-1 run list position v % nsteps of the group's query
  // head v / nsteps.  The tile and head of the step to fetch next are kept
  // incrementally (tile nit at position npos, of the head whose Q / dO start
  // at nq / ng and whose LSE / D rows start at nrow), so the loop does no
  // division.
  const int nv = G * nsteps;
  int npos = 0;
  int nit = tile_at(0);
  const uint16_t* nq = qp;
  const uint16_t* ng = gp;
  int64_t nrow = sv.row_base;
  auto advance = [&]() __attribute__((always_inline)) {
    if constexpr (MASK == kMaskBlocks) {
      if (++npos == nsteps) {
        npos = 0;
        nq += qhs;
        ng += qhs;
        nrow += rhs;
      }
      nit = tile_at(npos);
    } else {
      if (++nit == qt_begin + nsteps) {
        nit = qt_begin;
        nq += qhs;
        ng += qhs;
        nrow += rhs;
      }
    }
  };

  // Q and dO tiles travel from global memory straight into LDS (direct
  // loads; LDS chunk p = i*NT + tid of a tile holds row p / CH_PER_ROW, logical
  // chunk (p % CH_PER_ROW) ^ swz(row)).  Rows past the sequence repeat its last
  // row; their LSE entry is +inf, so P and dS vanish there.
  int src_row[QCPT], src_col[QCPT];
#pragma unroll
  for (int i = 0; i < QCPT; ++i) {
    const int pch = i * NT + tid;
    const int row = pch / CH_PER_ROW;
    src_row[i] = row;
    src_col[i] = ((pch % CH_PER_ROW) ^ swz<D>(row)) << 3;
  }
  // Load number n (0 .. 2*QCPT-1) of this thread for the step to fetch
  // next: Q for even n, dO for odd n, chunk n / 2.
  auto issue_part = [&](int buf, int n) {
    const int i = n >> 1;
    const int64_t off = (int64_t)min(nit * BQ + src_row[i], len - 1) * sv.tok_stride + src_col[i];
    if (n & 1) lds_dma16(ng + off, sGb + buf * QT_ELEMS + (i * NT + wave * 64) * 8);
    else lds_dma16(nq + off, sQb + buf * QT_ELEMS + (i * NT + wave * 64) * 8);
  };
  auto issue_tile = [&](int buf) {
#pragma unroll
    for (int n = 0; n < 2 * QCPT; ++n) issue_part(buf, n);
  };
  // LSE (as log2, +inf when the row is dead or past the end) and -D of the
  // tile's rows, through registers of wave 0 (BQ = 64 rows, one per lane).
  // The raw values are loaded at the start of a step and converted only when
  // stored at its end, so the wave does not wait for the loads in between.
  static_assert(BQ == 64, "one row per lane of wave 0");
  float rl = 0.f, rd = 0.f;
  int rq = 0;
  auto load_rows = [&]() {
    if (wave == 0) {
      rq = nit * BQ + lane;
      const int64_t row = nrow + min(rq, len - 1);
      rl = a.lse[row];
      rd = a.dvec[row];
    }
  };
  auto store_rows = [&](int buf) {
    if (wave == 0) {
      const bool out = rq >= len;
      sL[buf][lane] = (out || rl == kNegInf) ? kPosInf : rl * kLog2e;
      sDv[buf][lane] = out ? 0.f : -rd;
    }
  };

  // A key block no query block lists gets dK = dV = 0.
  if (MASK != kMaskBlocks || nv > 0) {
    // Prologue: the first Q/dO tile in flight, then K and V (rows past the
    // sequence are zero) and the first LSE/D rows; one wait covers all.
    issue_tile(0);
#pragma unroll
    for (int cidx = 0; cidx < KCPT; ++cidx) {
      const int chunk = tid + cidx * NT;
      const int row = chunk / CH_PER_ROW;
      const int col = (chunk - row * CH_PER_ROW) * 8;
      const int key = k0 + row;
      const int kc = min(key, len - 1);
      const uint32_t keep = key < len ? 0xffffffffu : 0u;
      const u32x4 xk = *(const u32x4*)(kp + (int64_t)kc * sv.kv_stride + col) & keep;
      const u32x4 xv = *(const u32x4*)(vp + (int64_t)kc * sv.kv_stride + col) & keep;
      const int off = swz_off<D>(row, col);
      *(u32x4*)(sK + off) = xk;
      *(u32x4*)(sV + off) = xv;
    }
    load_rows();
    store_rows(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first Q/dO tile too
    barrier_vmem_n<0>();

    // Per-lane operand offsets (a row's swizzle depends only on the row mod 16).
    int aoff[KS];       // b128 operand rows (query or key) l32, chunk 2*ks + hi
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aoff[ks] = swz_off<D>(l32, ks * 16 + hi * 8);
    const int tr_r = hi * 4 + ((lane >> 2) & 3);
    const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
    int troff[2][DB];   // transpose reads: rows 8R + tr_r, columns db*32 + tr_c
#pragma unroll
    for (int R = 0; R < 2; ++R)
#pragma unroll
      for (int db = 0; db < DB; ++db) troff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);
    const uint16_t* kb_rows = sK + kblk * 32 * D;
    const uint16_t* vb_rows = sV + kblk * 32 * D;

    // Step v from buffer BUF (= v % 2, a compile-time constant so that every
    // LDS address is a register plus an immediate).
    auto step = [&](int v, auto buf_c) {
      constexpr int buf = decltype(buf_c)::value;
      const int it = nit;
      advance();
      const int q0 = it * BQ;
      const bool fetch = v + 1 < nv;
      if (fetch) load_rows();
      // The loads of tile it+1 are spread over the first live half's S / dP
      // MFMAs (all waves issuing together would queue in the CU's memory
      // pipeline); a wave with no live half issues them at once.
      bool pending = fetch;

      const uint16_t* q_s = sQb + buf * QT_ELEMS;
      const uint16_t* g_s = sGb + buf * QT_ELEMS;
#pragma unroll
      for (int qq = 0; qq < QHALVES; ++qq) {
        const int qb = qh0 + qq;
        __builtin_amdgcn_sched_barrier(0);
        if (CAUSAL && q0 + qb * 32 + 31 < wk0) continue;  // this half sees none of the wave's keys
        if (MASK == kMaskWindow &&
            (q0 + qb * 32 + 31 + a.win_right < wk0 || q0 + qb * 32 - a.win_left > wk0 + 31))
          continue;  // the window keeps none of the wave's keys for this half
        bool need_mask = (wk0 + 31 >= len) || any_bad_key;
        if (CAUSAL) need_mask = need_mask || (wk0 + 31 > q0 + qb * 32);
        if (MASK == kMaskWindow)
          need_mask = need_mask || (wk0 < q0 + qb * 32 + 31 - a.win_left) || (wk0 + 31 > q0 + qb * 32 + a.win_right);
        // S and dP - D (the dP accumulator starts at -D of its rows), their
        // four operands read one k-step ahead.
        f32x16 s = f32x16{}, dp;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 nd = *(const f32x4*)(&sDv[buf][qb * 32 + g * 8 + hi * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) dp[g * 4 + e] = nd[e];
        }
        bf16x8 opq[2], opk[2], opg[2], opv[2];
        auto sread = [&](int ks, int u) __attribute__((always_inline)) {
          const int off = qb * 32 * D + aoff[ks];
          opq[u] = as_bf16x8(*(const u32x4*)(q_s + off));
          opk[u] = as_bf16x8(*(const u32x4*)(kb_rows + aoff[ks]));
          opg[u] = as_bf16x8(*(const u32x4*)(g_s + off));
          opv[u] = as_bf16x8(*(const u32x4*)(vb_rows + aoff[ks]));
        };
        sread(0, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ks + 1 < KS) sread(ks + 1, (ks + 1) & 1);
          s = mfma_bf16(opq[ks & 1], opk[ks & 1], s);
          dp = mfma_bf16(opg[ks & 1], opv[ks & 1], dp);
          if (pending) {
#pragma unroll
            for (int n = ks * 2 * QCPT / KS; n < (ks + 1) * 2 * QCPT / KS; ++n) issue_part(buf ^ 1, n);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        pending = false;
        float cc = c;
        if (need_mask) {
          // Masked entries get an exponent argument of -inf (exp2 -> 0); the
          // scale is applied before the select and the exponent then uses
          // multiplier 1, so a zero or negative scale cannot make 0 * -inf.
          cc = 1.f;
          const int key_m = pin_in_branch(key_ok ? my_key : 0x7fffffff);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            bool vis = key_m != 0x7fffffff;
            const int qrow = q0 + qb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
            if (CAUSAL) vis = vis && (key_m <= qrow);
            if (MASK == kMaskWindow) vis = vis && key_m >= qrow - a.win_left && key_m <= qrow + a.win_right;
            s[r] = vis ? s[r] * c : kNegInf;
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int ql = qb * 32 + g * 8 + hi * 4;
          const f32x4 lv = *(const f32x4*)(&sL[buf][ql]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = g * 4 + e;
            const float p = fast_exp2(__builtin_fmaf(s[r], cc, -lv[e]));
            s[r] = p;
            dp[r] = p * dp[r];
          }
        }
        // dV += P^T dO and dK += dS^T Q, 16 query rows per MFMA; the
        // transposed dO / Q operands are read one MFMA pair ahead.
        bf16x8 pa[2], da[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          pa[t] = pack_bf16x8(s[8 * t + 0], s[8 * t + 1], s[8 * t + 2], s[8 * t + 3],
                              s[8 * t + 4], s[8 * t + 5], s[8 * t + 6], s[8 * t + 7]);
          da[t] = pack_bf16x8(dp[8 * t + 0], dp[8 * t + 1], dp[8 * t + 2], dp[8 * t + 3],
                              dp[8 * t + 4], dp[8 * t + 5], dp[8 * t + 6], dp[8 * t + 7]);
        }
        constexpr int NKK = 2 * DB;  // (t, db) pairs
        bf16x8 opgt[2], opqt[2];
        auto tread = [&](int i, int u) __attribute__((always_inline)) {
          const int rbase = (qb * 32 + 16 * (i / DB)) * D;
          const int db = i % DB;
          opgt[u] = join_u32x2(lds_read_tr16(g_s + rbase + troff[0][db]), lds_read_tr16(g_s + rbase + troff[1][db]));
          opqt[u] = join_u32x2(lds_read_tr16(q_s + rbase + troff[0][db]), lds_read_tr16(q_s + rbase + troff[1][db]));
        };
        tread(0, 0);
#pragma unroll
        for (int i = 0; i < NKK; ++i) {
          if (i + 1 < NKK) tread(i + 1, (i + 1) & 1);
          dv[i % DB] = mfma_bf16(pa[i / DB], opgt[i & 1], dv[i % DB]);
          dk[i % DB] = mfma_bf16(da[i / DB], opqt[i & 1], dk[i % DB]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      if (pending) issue_tile(buf ^ 1);
      if (fetch) store_rows(buf ^ 1);
      barrier_vmem_n<0>();  // the next tile has landed
    };
    for (int v = 0; v < nv; v += 2) {
      step(v, std::integral_constant<int, 0>{});
      if (v + 1 < nv) step(v + 1, std::integral_constant<int, 1>{});
    }
  }

  if constexpr (NW == 8) {
    // Waves 4-7 hand their partial sums to waves 0-3 (same keys) through LDS.
    float* red = reinterpret_cast<float*>(arena);  // 4 waves x 2 x DB x 16 x 64 floats = 128 KiB at D = 128
    if (wave >= 4) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          red[(((kblk * 2 + 0) * DB + db) * 16 + r) * 64 + lane] = dk[db][r];
          red[(((kblk * 2 + 1) * DB + db) * 16 + r) * 64 + lane] = dv[db][r];
        }
    }
    __syncthreads();
    if (wave >= 4) return;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dk[db][r] += red[(((kblk * 2 + 0) * DB + db) * 16 + r) * 64 + lane];
        dv[db][r] += red[(((kblk * 2 + 1) * DB + db) * 16 + r) * 64 + lane];
      }
  }

  if constexpr (MASK == kMaskBlocks) {
    // A key block cut into chunks: this chunk's fp32 sums go to its slot
    // (rows = keys of the block, unscaled); the reduce pass adds the slots.
    const int slot = a.blk_slot[kt];
    if (slot >= 0) {
      float* part = a.blk_part + ((int64_t)bh * a.blk_nslots + slot + chunk) * 2 * BK * D;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kblk * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          part[kl * D + db * 32 + l32] = dk[db][r];
          part[(BK + kl) * D + db * 32 + l32] = dv[db][r];
        }
      }
      return;
    }
  }

  // dK = scale * acc, dV = acc; accumulator rows are keys, columns features.
  // In the accumulator layout a lane holds one feature of 16 keys, so direct
  // stores would be 2 bytes wide; the wave's 32 keys x D of each go through
  // LDS instead and leave as whole rows, 16 bytes per lane.  Staging: the dK
  // rows, then the dV rows, row-major with 16-byte chunk c of row r at chunk
  // c ^ (r mod CH_PER_ROW).  The 8-wave form reuses the wave's own part of
  // the reduction buffer (read above by this wave alone: its LDS operations
  // complete in order); the 4-wave form takes a quarter of the arena (every
  // wave has passed the last barrier after its own LDS reads, and no direct
  // load is still in flight).
  uint16_t* st;
  if constexpr (NW == 8) {
    static_assert(2 * 32 * D * 2 <= 2 * DB * 16 * 64 * 4, "staging fits the wave's part of the reduction buffer");
    st = reinterpret_cast<uint16_t*>(reinterpret_cast<float*>(arena) + kblk * 2 * DB * 16 * 64);
  } else {
    static_assert(4 * 2 * 32 * D <= 2 * KV_ELEMS + 4 * QT_ELEMS, "staging fits the arena");
    st = arena + kblk * 2 * 32 * D;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int kl = (r >> 2) * 8 + hi * 4 + (r & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = db * 4 + (l32 >> 3);
      const int so = kl * D + ((c ^ (kl % CH_PER_ROW)) << 3) + (l32 & 7);
      st[so] = (uint16_t)(pack_bf16x2(dk[db][r] * a.scale, 0.f) & 0xffffu);
      st[32 * D + so] = (uint16_t)(pack_bf16x2(dv[db][r], 0.f) & 0xffffu);
    }
  }
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  constexpr int RPI = 64 / CH_PER_ROW;  // rows per store instruction
  uint16_t* __restrict__ dkp = (uint16_t*)a.dk + sv.kv_base;
  uint16_t* __restrict__ dvp = (uint16_t*)a.dv + sv.kv_base;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CH_PER_ROW;
    const int c = lane % CH_PER_ROW;
    const int so = r * D + ((c ^ (r % CH_PER_ROW)) << 3);
    const u32x4 wk = *(const u32x4*)(st + so);
    const u32x4 wv = *(const u32x4*)(st + 32 * D + so);
    const int key = wk0 + r;
    if (key < len) {
      *(u32x4*)(dkp + (int64_t)key * sv.kv_stride + c * 8) = wk;
      *(u32x4*)(dvp + (int64_t)key * sv.kv_stride + c * 8) = wv;
    }
  }
}

// ---------------------------------------------------------------- kernel 3
// The forward's staggered schedule: one barrier per 64-key tile, and waves w
// and w + 4 on one SIMD half a tile apart.  Every wave runs, for key tile j,
//   S^T_j = K_j Q^T and dP^T_j = V_j dO^T (MFMA),  dS_j (VALU),
//   dQ^T += K_j^T dS^T_j (MFMA),
// and interval j ends after S/dP_j for the late waves (4-7) and after dS_j for
// the early ones: within an interval an early wave issues dQ_{j-1}, S/dP_j and
// then dS_j, while its partner computes dS_{j-1} and then dQ_{j-1}, S/dP_j,
// so one wave's vector work overlaps the other's matrix work.  K and V tiles
// travel from global memory straight into LDS, four slots each, tile t + 2
// fetched at the start of interval t: K_j is read in interval j (S_j) and
// again in interval j + 1 (dQ_j), so its slot is refilled only in interval
// j + 2.  Before the barrier that ends interval t each wave waits only for its
// own loads of tile t + 1.  Rows past the sequence repeat its last row and
// are masked.
template <int D, int NW, bool CAUSAL, bool VARLEN, bool KPAD, int MASK = kMaskPlain>
__global__ void __launch_bounds__(NW * 64, 1) bwd_dq_kernel(AttnArgs a, int n_qtiles) {
  static_assert(NW == 8, "two waves per SIMD");
  constexpr int BC = 64;                 // keys per tile
  constexpr int BR = NW * 32;            // query rows per workgroup
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int TILE = BC * D;
  constexpr int NT = NW * 64;
  constexpr int CPR = D / 8;
  constexpr int LPT = BC * CPR / NT;     // direct loads per thread per tensor and tile
  constexpr int NS = 4;                  // tile slots per tensor
  static_assert(LPT * NT == BC * CPR, "tile chunks must divide evenly");

  __shared__ __attribute__((aligned(16))) uint16_t sK[NS][TILE];
  __shared__ __attribute__((aligned(16))) uint16_t sV[NS][TILE];
  __shared__ uint8_t s_valid[NS][BC];
  __shared__ uint32_t s_anypad[NS];

  int bh, tile;
  // causal masks, windows and block lists: groups of four heads per XCD,
  // heaviest tiles first in each group under a causal mask; plain non-causal:
  // the same groups when a head has 4 or more query tiles (its K/V no longer
  // fit in L2 for many heads at once), else all heads' tile 0, then all tile
  // 1, ... (measured faster for 2 tiles a head)
  // packed sequences: each XCD takes the same heads of every sequence, one
  // (sequence, head) at a time, heaviest tiles first (as the forward)
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
  if (q_tile0 >= sv.len) return;

  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool late = wave >= 4;  // the partner of wave w on its SIMD is w + 4
  const int q_wave0 = q_tile0 + wave * 32;
  const int qi = q_wave0 + l32;  // this lane's query row (columns of S^T)
  const float c = a.scale_log2;

  const uint16_t* __restrict__ qp = (const uint16_t*)a.q + sv.base;
  const uint16_t* __restrict__ kp = (const uint16_t*)a.k + sv.kv_base;
  const uint16_t* __restrict__ vp = (const uint16_t*)a.v + sv.kv_base;
  const uint16_t* __restrict__ gp = (const uint16_t*)a.dout + sv.base;

  const bool row_ok = qi < sv.len;
  bf16x8 qf[KS], gf[KS];  // loaded in the prologue
  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) dq[db] = f32x16{};

  const int kv_len = sv.len;
  // Key tiles visited, as a list (the forward's schedule): position r holds
  // key tile tile_of(r); a wave computes the positions wave_live accepts.
  __shared__ uint8_t s_bflag[2][MASK == kMaskBlocks ? kMaxSparseBlocks : 1];
  __shared__ uint16_t s_blist[MASK == kMaskBlocks ? kMaxSparseBlocks : 1];
  __shared__ int s_bcount;
  int ntiles, jt0 = 0, jw_first = 0, jw_last = 0;
  if constexpr (MASK == kMaskPlain) {
    const int kv_end = CAUSAL ? min(kv_len, q_tile0 + BR) : kv_len;
    ntiles = (kv_end + BC - 1) / BC;
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

  int src_row[LPT], src_col[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int pch = i * NT + tid;
    const int row = pch / CPR;
    src_row[i] = row;
    src_col[i] = ((pch % CPR) ^ swz<D>(row)) << 3;
  }
  auto issue = [&](int j) __attribute__((always_inline)) {
    const int k0 = tile_of(j) * BC;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = min(k0 + src_row[i], kv_len - 1);
      const int64_t off = (int64_t)key * sv.kv_stride + src_col[i];
      lds_dma16(kp + off, sK[j % NS] + (i * NT + wave * 64) * 8);
      lds_dma16(vp + off, sV[j % NS] + (i * NT + wave * 64) * 8);
    }
  };
  // Key-validity flags of a tile, by wave 0: the raw byte is loaded early
  // and converted only when stored, so the wave does not wait in between.
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
        s_valid[j % NS][lane] = (uint8_t)ok;
        const bool any = wave_any(ok == 0u);
        if (lane == 0) s_anypad[j % NS] = any ? 1u : 0u;
      }
    }
  };

  int koff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) koff[ks] = swz_off<D>(l32, ks * 16 + hi * 8);
  const int tr_r = hi * 4 + ((lane >> 2) & 3);
  const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int troff[2][DB];
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int db = 0; db < DB; ++db) troff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);

  float lse2 = 0.f, dd = 0.f;
  f32x16 s[2], dp[2];  // S^T and dP^T of the tile formed last (then dS^T in dp)
  bf16x8 dsb[4];       // packed dS^T of the tile whose vector part ran last

  // Whether block kb (32 keys) of the tile starting at key kt0 lies wholly
  // above the diagonal for this wave's rows (then its products are skipped
  // and its dS is zero).
  auto above = [&](int kt0, int kb) __attribute__((always_inline)) -> bool {
    return CAUSAL && kt0 + kb * 32 > q_wave0 + 31;
  };
  // S^T and dP^T of a tile from slot SL, both 32-key blocks, K and V operands
  // read one k-step ahead across the two blocks (a deeper ring measured no
  // faster and holds eight more registers).
  auto mma_sdp = [&](auto slot_c, int kt0) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const uint16_t* sk = sK[SL];
    const uint16_t* svv = sV[SL];
    const bool skip1 = above(kt0, 1);
    constexpr int NI = 2 * KS;
    bf16x8 opk[2], opv[2];
    auto sread = [&](int i, int u) __attribute__((always_inline)) {
      const int kb = i / KS;
      const int ks = i % KS;
      opk[u] = as_bf16x8(*(const u32x4*)(sk + kb * 32 * D + koff[ks]));
      opv[u] = as_bf16x8(*(const u32x4*)(svv + kb * 32 * D + koff[ks]));
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
    sread(0, 0);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int kb = i / KS;
      const int ks = i % KS;
      if (kb == 1 && skip1) break;
      if (i + 1 < NI) sread(i + 1, (i + 1) % 2);
      s[kb] = mfma_bf16(opk[i % 2], qf[ks], s[kb]);
      dp[kb] = mfma_bf16(opv[i % 2], gf[ks], dp[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // dS^T = P^T o (dP^T - D) with P^T = exp2(S^T c - LSE log2 e), packed to
  // bf16 for the dQ products; masked entries get P = 0.
  auto vpart = [&](int j) __attribute__((always_inline)) {
    const int kt0 = tile_of(j) * BC;
    const int slot = j % NS;
    bool need_mask = kt0 + BC > kv_len;
    if (CAUSAL) need_mask = need_mask || (kt0 + BC - 1 > q_wave0);
    if (KPAD) need_mask = need_mask || (s_anypad[slot] != 0u);
    if (MASK == kMaskWindow)
      need_mask = need_mask || (kt0 < q_wave0 + 31 - a.win_left) || (kt0 + BC - 1 > q_wave0 + a.win_right);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (above(kt0, kb)) {
        dsb[kb * 2] = bf16x8{};
        dsb[kb * 2 + 1] = bf16x8{};
        continue;
      }
      float cc = c;
      if (need_mask) {
        // Masked entries get an exponent argument of -inf (exp2 -> 0), with
        // the scale applied before the select (see the key-tile pass).
        cc = 1.f;
        const int q_m = pin_in_branch(qi);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kl = kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          const int key = kt0 + kl;
          bool vis = key < kv_len;
          if (CAUSAL) vis = vis && key <= q_m;
          if (KPAD) vis = vis && s_valid[slot][kl] != 0;
          if (MASK == kMaskWindow) vis = vis && key >= q_m - a.win_left && key <= q_m + a.win_right;
          s[kb][r] = vis ? s[kb][r] * c : kNegInf;
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], cc, -lse2));
        dp[kb][r] = p * (dp[kb][r] - dd);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
        dsb[kb * 2 + t] = pack_bf16x8(dp[kb][8 * t + 0], dp[kb][8 * t + 1], dp[kb][8 * t + 2], dp[kb][8 * t + 3],
                                      dp[kb][8 * t + 4], dp[kb][8 * t + 5], dp[kb][8 * t + 6], dp[kb][8 * t + 7]);
    }
  };
  // dQ^T += K^T dS^T, 16 keys per MFMA: K through the transpose read, three
  // MFMAs ahead across the two blocks.
  auto mma_dq = [&](auto slot_c, int kt0) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot_c)::value;
    const uint16_t* sk = sK[SL];
    constexpr int NKK = 2 * DB;
    constexpr int NI = 2 * NKK;
    constexpr int PF = 3;
    const bool skip1 = above(kt0, 1);
    auto tread = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      const int kb = i / NKK;
      const int ii = i % NKK;
      const uint16_t* kt = sk + (kb * 32 + 16 * (ii / DB)) * D;
      return join_u32x2(lds_read_tr16(kt + troff[0][ii % DB]), lds_read_tr16(kt + troff[1][ii % DB]));
    };
    bf16x8 ka[NI];
#pragma unroll
    for (int i = 0; i < PF; ++i) ka[i] = tread(i);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int kb = i / NKK;
      const int ii = i % NKK;
      if (kb == 1 && skip1) break;
      if (i + PF < NI) ka[i + PF] = tread(i + PF);
      dq[ii % DB] = mfma_bf16(ka[i], dsb[kb * 2 + ii / DB], dq[ii % DB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Start of interval t: fetch tile t + 2 (and its flags, stored at the end
  // of the interval).  End of interval t: tile t + 1 must have landed (the
  // interval's own loads may still be in flight), barrier, then start t + 1.
  auto begin_interval = [&](int t) __attribute__((always_inline)) {
    if (t + 2 < ntiles) {
      load_flags(t + 2);
      issue(t + 2);
    }
  };
  auto end_interval = [&](int t) __attribute__((always_inline)) {
    if (t + 2 < ntiles) {
      store_flags(t + 2);
      barrier_vmem_n<2 * LPT>();
    } else {
      barrier_vmem_n<0>();
    }
    begin_interval(t + 1);
  };

  // An empty block list leaves dQ = 0.
  if (MASK != kMaskBlocks || ntiles > 0) {
    // Prologue: tiles 0 and 1 in flight, then this wave's Q, dO, LSE and D
    // rows; one wait (which the compiler sees, so the loop waits for none of
    // these loads again) covers all of them.
    load_flags(0);
    store_flags(0);
    if (ntiles > 1) {
      load_flags(1);
      store_flags(1);
    }
    issue(0);
    if (ntiles > 1) issue(1);
    // Q and dO as B operands (lane = query, 8 features per k-step).  Rows past
    // the sequence load its last row and are zeroed (no branch).
    const int qc = min(qi, sv.len - 1);
    const uint32_t keep = row_ok ? 0xffffffffu : 0u;
    u32x4 graw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int64_t off = (int64_t)qc * sv.tok_stride + ks * 16 + hi * 8;
      qf[ks] = as_bf16x8(*(const u32x4*)(qp + off) & keep);
      graw[ks] = *(const u32x4*)(gp + off) & keep;
      gf[ks] = as_bf16x8(graw[ks]);
    }
    // a dead or out-of-range row gets P = 0
    const float lse_raw = a.lse[sv.row_base + qc];
    lse2 = (!row_ok || lse_raw == kNegInf) ? kPosInf : lse_raw * kLog2e;
    if (a.dq_writes_d) {
      // D = rowsum(dO o O) in the summation order of the D pre-pass, so both
      // give the same bits: each 8-feature chunk in order (this lane holds
      // chunks 2 ks + hi), the chunks as a tree (partners 8, 4, 2 chunks
      // apart, i.e. ks apart by KS/2, KS/4, ...), then the even half plus
      // the odd half from the lane 32 away.
      const uint16_t* __restrict__ opp = (const uint16_t*)a.o + sv.base;
      float part[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int64_t off = (int64_t)qc * sv.tok_stride + ks * 16 + hi * 8;
        const u32x4 ov = *(const u32x4*)(opp + off) & keep;
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          acc = __builtin_fmaf(bf16_bits_to_f32(ov[w] & 0xffffu), bf16_bits_to_f32(graw[ks][w] & 0xffffu), acc);
          acc = __builtin_fmaf(bf16_bits_to_f32(ov[w] >> 16), bf16_bits_to_f32(graw[ks][w] >> 16), acc);
        }
        part[ks] = acc;
      }
#pragma unroll
      for (int w = KS / 2; w >= 1; w >>= 1)
#pragma unroll
        for (int ks = 0; ks < w; ++ks) part[ks] = part[ks] + part[ks + w];
      dd = part[0] + lane_xor32(part[0]);
      if (row_ok && hi == 0) a.dvec[sv.row_base + qi] = dd;
      dd = row_ok ? dd : 0.f;
    } else {
      dd = row_ok ? a.dvec[sv.row_base + qc] : 0.f;
    }

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    barrier_vmem_n<0>();
    begin_interval(0);

    // Every wave passes ntiles + 1 barriers after the prologue: one per key
    // tile it works on or skips, then the remaining intervals up to ntiles.
    auto body = [&](int j, auto slot_c) __attribute__((always_inline)) {
      if constexpr (MASK != kMaskPlain) {
        if (!wave_live(j)) {
          end_interval(j);
          return;
        }
      }
      const int kt0 = tile_of(j) * BC;
      mma_sdp(slot_c, kt0);
      if (late) end_interval(j);
      vpart(j);
      if (!late) end_interval(j);
      mma_dq(slot_c, kt0);
    };
    const int j_end = MASK == kMaskPlain ? jw_last : ntiles - 1;
    for (int j = 0; j <= j_end; j += NS) {
      body(j, std::integral_constant<int, 0>{});
      if (j + 1 <= j_end) body(j + 1, std::integral_constant<int, 1>{});
      if (j + 2 <= j_end) body(j + 2, std::integral_constant<int, 2>{});
      if (j + 3 <= j_end) body(j + 3, std::integral_constant<int, 3>{});
    }
    for (int t = j_end + 1; t <= ntiles; ++t) end_interval(t);
  }

  // dQ = scale * acc; the accumulator holds dQ^T (lane = query, registers =
  // features).  As in the forward's epilogue, the wave's 32 x D block goes
  // through LDS (idle: every wave has passed the last barrier after waiting
  // for its own LDS reads and loads) so that the global stores are whole
  // rows, 16 bytes per lane.  Row r is row-major with 16-byte chunk c at
  // c ^ (r mod CPR); waves 0-5 stage in the K buffers, 6 and 7 in the V
  // buffers.
  {
    static_assert(6 * 32 * D <= NS * TILE && (NW - 6) * 32 * D <= NS * TILE, "staging fits");
    uint16_t* stage = wave < 6 ? &sK[0][0] + wave * 32 * D : &sV[0][0] + (wave - 6) * 32 * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& x = dq[db];
        u32x2 w = {pack_bf16x2(x[4 * g + 0] * a.scale, x[4 * g + 1] * a.scale),
                   pack_bf16x2(x[4 * g + 2] * a.scale, x[4 * g + 3] * a.scale)};
        const int cc = db * 4 + g;
        *(u32x2*)(stage + l32 * D + ((cc ^ (l32 % CPR)) << 3) + hi * 4) = w;
      }
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int RPI = 64 / CPR;  // rows per store instruction
    uint16_t* __restrict__ dqp = (uint16_t*)a.dq + sv.base;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = i * RPI + lane / CPR;
      const int cc = lane % CPR;
      const u32x4 w = *(const u32x4*)(stage + r * D + ((cc ^ (r % CPR)) << 3));
      if (q_wave0 + r < sv.len) *(u32x4*)(dqp + (int64_t)(q_wave0 + r) * sv.tok_stride + cc * 8) = w;
    }
  }
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

// Waves per dK/dV workgroup for the plain layouts.  d = 128: eight (two per
// SIMD), 10-13% faster than four.  d = 64: four (one per SIMD, handling both
// query halves of a step), 6% faster at N = 2048 and 16% at N = 512, where
// the eight-wave form's per-step overheads weigh most.  Windows and block
// lists always take eight.
constexpr int dkdv_waves(int d) { return d == 64 ? 4 : 8; }

template <int D, bool CAUSAL, bool VARLEN, bool KPAD, int MASK = kMaskPlain>
static hipError_t launch_dkdv_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int BK = 128;
  const int n_ktiles = (a.N + BK - 1) / BK;
  const int64_t blocks = (int64_t)(MASK == kMaskBlocks ? a.blk_max_work : n_ktiles) * a.B * a.Hkv;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (MASK != kMaskPlain) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 8, CAUSAL, VARLEN, KPAD, MASK>), dim3((unsigned)blocks), dim3(512), 0,
                       stream, a, n_ktiles);
    return hipGetLastError();
  }
  if (dkdv_waves(D) == 4)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 4, CAUSAL, VARLEN, KPAD>), dim3((unsigned)blocks), dim3(256), 0, stream, a,
                       n_ktiles);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, 8, CAUSAL, VARLEN, KPAD>), dim3((unsigned)blocks), dim3(512), 0, stream, a,
                       n_ktiles);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN, bool KPAD, int MASK = kMaskPlain>
static hipError_t launch_dq_t(const AttnArgs& a, hipStream_t stream) {
  constexpr int NW = 8;
  constexpr int BR = NW * 32;
  const int n_qtiles = (a.N + BR - 1) / BR;
  const int64_t blocks = (int64_t)n_qtiles * a.B * a.H;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW, CAUSAL, VARLEN, KPAD, MASK>), dim3((unsigned)blocks), dim3(NW * 64), 0,
                     stream, a, n_qtiles);
  return hipGetLastError();
}

template <int D, bool DQ>
static hipError_t dispatch_bwd(const AttnArgs& a, bool causal, bool varlen, bool kpad, hipStream_t s) {
#define MIATTN_BWD_LAUNCH(C, V, K) (DQ ? launch_dq_t<D, C, V, K>(a, s) : launch_dkdv_t<D, C, V, K>(a, s))
  if (varlen) {
    if (causal) return kpad ? MIATTN_BWD_LAUNCH(true, true, true) : MIATTN_BWD_LAUNCH(true, true, false);
    return kpad ? MIATTN_BWD_LAUNCH(false, true, true) : MIATTN_BWD_LAUNCH(false, true, false);
  }
  return causal ? MIATTN_BWD_LAUNCH(true, false, false) : MIATTN_BWD_LAUNCH(false, false, false);
#undef MIATTN_BWD_LAUNCH
}

hipError_t launch_bwd_dkdv_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream) {
  const bool kpad = varlen && a.key_valid != nullptr;
  if (d == 128) return dispatch_bwd<128, false>(a, causal, varlen, kpad, stream);
  if (d == 64) return dispatch_bwd<64, false>(a, causal, varlen, kpad, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream) {
  const bool kpad = varlen && a.key_valid != nullptr;
  if (d == 128) return dispatch_bwd<128, true>(a, causal, varlen, kpad, stream);
  if (d == 64) return dispatch_bwd<64, true>(a, causal, varlen, kpad, stream);
  return hipErrorInvalidValue;
}

// Dense layout with a sliding window (causal folded into the window) or a
// block-sparse list.
template <bool DQ>
static hipError_t dispatch_bwd_masked(const AttnArgs& a, int d, int mask, bool causal, hipStream_t s) {
#define MIATTN_BWD_MASKED(D_, C, M) (DQ ? launch_dq_t<D_, C, false, false, M>(a, s) \
                                        : launch_dkdv_t<D_, C, false, false, M>(a, s))
  if (mask == kMaskWindow) {
    if (d == 128) return MIATTN_BWD_MASKED(128, false, kMaskWindow);
    if (d == 64) return MIATTN_BWD_MASKED(64, false, kMaskWindow);
  } else if (mask == kMaskBlocks) {
    if (d == 128) return causal ? MIATTN_BWD_MASKED(128, true, kMaskBlocks) : MIATTN_BWD_MASKED(128, false, kMaskBlocks);
    if (d == 64) return causal ? MIATTN_BWD_MASKED(64, true, kMaskBlocks) : MIATTN_BWD_MASKED(64, false, kMaskBlocks);
  }
  return hipErrorInvalidValue;
#undef MIATTN_BWD_MASKED
}

hipError_t launch_bwd_dkdv_masked_bf16(const AttnArgs& a, int d, int mask, bool causal, hipStream_t stream) {
  return dispatch_bwd_masked<false>(a, d, mask, causal, stream);
}

hipError_t launch_bwd_dq_masked_bf16(const AttnArgs& a, int d, int mask, bool causal, hipStream_t stream) {
  return dispatch_bwd_masked<true>(a, d, mask, causal, stream);
}

// One workgroup per query block r: clears row r of the table, then marks the
// key blocks listed for r.  Entries past blk_nnz and out-of-range indices
// are ignored, as in the kernels that read the list directly.
__global__ void __launch_bounds__(256) block_table_kernel(AttnArgs a, uint8_t* table) {
  const int r = blockIdx.x;
  uint8_t* row = table + (int64_t)r * a.n_kblk;
  for (int c = threadIdx.x; c < a.n_kblk; c += 256) row[c] = 0;
  __syncthreads();
  const int e0 = min(max(a.blk_row_ptr[r], 0), a.blk_nnz);
  const int e1 = min(max(a.blk_row_ptr[r + 1], e0), a.blk_nnz);
  for (int e = e0 + (int)threadIdx.x; e < e1; e += 256) {
    const int c = a.blk_col_idx[e];
    if (c >= 0 && c < a.n_kblk) row[c] = 1;
  }
}

// The balanced work list of the key-tile pass (one workgroup of 1024
// threads): per key block the length of its query list (the same causal
// filter as build_query_block_list), counted in parallel over the expanded
// table with LDS integer adds (exact, so the order does not matter); then one
// wave places the work items and the partial-sum slots of the blocks that
// are cut.  The chunks of cut blocks (the longest items) come first in the
// list, so that none of them starts last.
__global__ void __launch_bounds__(1024) block_work_kernel(AttnArgs a, int causal, int* work, int* slot, int* nch) {
  __shared__ int s_count[kMaxSparseBlocks];
  const int tid = threadIdx.x;
  for (int c = tid; c < a.n_kblk; c += 1024) s_count[c] = 0;
  __syncthreads();
  const int total = a.n_qblk * a.n_kblk;
  for (int idx = tid; idx < total; idx += 1024) {
    const int r = idx / a.n_kblk;
    const int c = idx - r * a.n_kblk;
    if ((!causal || r >= c) && a.blk_table[idx] != 0) atomicAdd(&s_count[c], 1);
  }
  __syncthreads();
  if (tid >= 64) return;
  const int lane = tid;
  // pass 0 places the chunks of cut blocks, pass 1 the uncut blocks
  int carry = 0;
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    for (int base = 0; base < a.n_kblk; base += 64) {
      const int c = base + lane;
      const int count = c < a.n_kblk ? s_count[c] : 0;
      const int n = c < a.n_kblk ? max(1, (count + a.blk_chunk - 1) / a.blk_chunk) : 0;
      const int mine = (pass == 0) ? (n > 1 ? n : 0) : (n == 1 ? 1 : 0);
      int incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int t = __builtin_amdgcn_ds_bpermute((int)(((unsigned)lane - (unsigned)o) << 2), incl);
        if (lane >= o) incl += t;
      }
      const int w0 = carry + incl - mine;   // exclusive position
      for (int k = 0; k < mine; ++k) work[1 + w0 + k] = c | (k << 16);
      if (c < a.n_kblk && pass == 0) {
        nch[c] = n;
        slot[c] = n > 1 ? w0 : -1;   // the cut blocks' items and slots share positions
      }
      carry += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  if (lane == 0) work[0] = carry;
}

// Sums the slots of each cut key block in chunk order and writes bf16 dK
// (times scale) and dV.  One workgroup per (batch, key/value head, key
// block, group of 16 keys); every thread adds 16-byte vectors of the fp32
// partial sums chunk after chunk (the order of the sum per element is the
// chunk order, as before) and writes 8-byte bf16 vectors.
template <int D>
__global__ void __launch_bounds__(256) block_reduce_kernel(AttnArgs a) {
  constexpr int BK = 128;
  constexpr int RG = 16;                      // keys per workgroup
  constexpr int PER = RG * D / 4 / 256;       // 16-byte vectors per thread and tensor
  static_assert(PER >= 1 && PER * 256 * 4 == RG * D, "whole vectors per thread");
  const int g = blockIdx.x % (BK / RG);
  const int rest = blockIdx.x / (BK / RG);
  const int c = rest % a.n_kblk;
  const int bh = rest / a.n_kblk;
  const int slot = a.blk_slot[c];
  if (slot < 0) return;
  const int n = a.blk_nch[c];
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;
  const int64_t kv_base = ((int64_t)b * a.Hkv + hk) * a.N * D;
  const float* part = a.blk_part + ((int64_t)bh * a.blk_nslots + slot) * 2 * BK * D + g * RG * D;
  f32x4 sk[PER], sv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    sk[i] = f32x4{};
    sv[i] = f32x4{};
  }
  for (int t = 0; t < n; ++t) {
    const float* pt = part + (int64_t)t * 2 * BK * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = 4 * ((int)threadIdx.x + i * 256);
      const f32x4 xk = *(const f32x4*)(pt + e);
      const f32x4 xv = *(const f32x4*)(pt + BK * D + e);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sk[i][u] += xk[u];
        sv[i][u] += xv[u];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = 4 * ((int)threadIdx.x + i * 256);
    const int kl = g * RG + e / D;
    const int key = c * BK + kl;
    if (key < a.N) {
      const int64_t off = kv_base + (int64_t)key * D + (e % D);
      *(u32x2*)((uint16_t*)a.dk + off) = u32x2{pack_bf16x2(sk[i][0] * a.scale, sk[i][1] * a.scale),
                                               pack_bf16x2(sk[i][2] * a.scale, sk[i][3] * a.scale)};
      *(u32x2*)((uint16_t*)a.dv + off) = u32x2{pack_bf16x2(sv[i][0], sv[i][1]), pack_bf16x2(sv[i][2], sv[i][3])};
    }
  }
}

hipError_t launch_block_work(const AttnArgs& a, bool causal, int* work, int* slot, int* nch, hipStream_t stream) {
  if (a.n_kblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_work_kernel, dim3(1), dim3(1024), 0, stream, a, causal ? 1 : 0, work, slot, nch);
  return hipGetLastError();
}

hipError_t launch_block_reduce(const AttnArgs& a, int d, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.B * a.Hkv * a.n_kblk * (128 / 16);
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 128) hipLaunchKernelGGL(block_reduce_kernel<128>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else if (d == 64) hipLaunchKernelGGL(block_reduce_kernel<64>, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_block_table(const AttnArgs& a, uint8_t* table, hipStream_t stream) {
  if (a.n_qblk <= 0 || a.n_kblk <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_table_kernel, dim3((unsigned)a.n_qblk), dim3(256), 0, stream, a, table);
  return hipGetLastError();
}

}  // namespace miattn
