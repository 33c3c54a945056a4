// Decoding attention: one new query token per sequence against a KV cache,
// split along the cache (FlashDecoding, "第 18 章 FlashAttention" section
// 18.8.2: cut the KV cache into pieces, compute each piece's local max, sum
// and output in parallel, merge with the online-softmax rule).
//
// Split pass: one wave per (sequence, key/value head, 32 query heads of its
// group, cache piece).  With grouped heads the G query heads that share a
// key/value head are the query rows of one MFMA tile (padded to 32), so the
// cache is read once per group.  S^T = K Q^T as in the forward (one query per
// lane): K goes straight from HBM into registers as the MFMA operand, V
// through LDS (direct loads, two buffers) for the transposed read of
// O^T += V^T P^T.  The piece's running state (max m in base-2 units, sum l,
// unnormalised O) goes to the workspace.  Decoding is HBM-bound: what matters
// is how many bytes are in flight, so each wave is its own workgroup (32 KiB
// of LDS, five per CU) and loads the next tile while it computes this one.
//
// Merge pass: one wave per (sequence, query head) combines the pieces:
// m = max m_t, O = sum O_t 2^(m_t - m) / sum l_t 2^(m_t - m), LSE = ln 2 *
// (m + log2 of the denominator); pieces with no key drop out, and a sequence
// with an empty cache gets O = 0, LSE = -inf.
#include "miattn_device.h"
#include "miattn_launch.h"

namespace miattn {

template <int D>
__global__ void __launch_bounds__(64) decode_split_kernel(DecodeArgs a) {
  constexpr int BC = 64;                 // keys per tile
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int LPT = BC * CPR / 64;     // V chunks per lane and tile
  constexpr int TILE = BC * D;
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][TILE];

  const int G = a.H / a.Hkv;
  const int ngc = (G + 31) / 32;
  int w = blockIdx.x;
  const int gc = w % ngc;
  w /= ngc;
  const int split = w % a.nsplit;
  const int bh = w / a.nsplit;
  const int b = bh / a.Hkv;
  const int hk = bh - b * a.Hkv;

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  int len = a.N;
  if (a.seqlens != nullptr) len = min(max(a.seqlens[b], 0), a.N);
  const int k_begin = split * a.chunk;
  const int k_end = min(len, k_begin + a.chunk);
  const int row = gc * 32 + l32;          // query row = head within the group
  const bool row_ok = row < G;
  const int h = hk * G + min(row, G - 1);
  const int64_t pidx = ((int64_t)b * a.H + h) * a.nsplit + split;

  if (k_begin >= k_end) {  // an empty piece: no key, drops out of the merge
    if (row_ok && hi == 0) {
      a.part_ml[2 * pidx] = kNegInf;
      a.part_ml[2 * pidx + 1] = 0.f;
    }
    return;
  }

  const uint16_t* __restrict__ kbase = (const uint16_t*)a.k + ((int64_t)b * a.Hkv + hk) * a.N * D;
  const uint16_t* __restrict__ vbase = (const uint16_t*)a.v + ((int64_t)b * a.Hkv + hk) * a.N * D;

  // Q^T as the B operand: lane = query row, 8 features per k-step; rows past
  // the group are zero.  A negative scale flips the sign of Q once.
  float c = a.scale_log2;
  const uint32_t qsign = c < 0.f ? 0x80008000u : 0u;
  c = fabsf(c);
  bf16x8 qf[KS];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((int64_t)b * a.H + h) * D;
    const uint32_t keep = row_ok ? 0xffffffffu : 0u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = as_bf16x8((*(const u32x4*)(qp + ks * 16 + hi * 8) & keep) ^ qsign);
  }

  // K operands of a tile straight from memory: key block kb, k-step ks holds
  // key t0 + kb*32 + l32, features ks*16 + hi*8 .. +7 (keys past the piece
  // repeat the last key of the sequence and are masked).
  bf16x8 ka[2][KS];
  auto load_k = [&](int t0) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = min(t0 + kb * 32 + l32, len - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ka[kb][ks] = as_bf16x8(*(const u32x4*)(kbase + (int64_t)key * D + ks * 16 + hi * 8));
    }
  };
  // V tile into LDS: chunk p = i*64 + lane holds row p / CPR, logical chunk
  // (p % CPR) ^ swz(row).
  int src_row[LPT], src_col[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int pch = i * 64 + lane;
    const int r = pch / CPR;
    src_row[i] = r;
    src_col[i] = ((pch % CPR) ^ swz<D>(r)) << 3;
  }
  auto issue_v = [&](int t0, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int key = min(t0 + src_row[i], len - 1);
      lds_dma16(vbase + (int64_t)key * D + src_col[i], dst + i * 64 * 8);
    }
  };
  const int tr_r = hi * 4 + ((lane >> 2) & 3);
  const int tr_c = ((lane >> 4) & 1) * 16 + 4 * (lane & 3);
  int voff[2][DB];
#pragma unroll
  for (int R = 0; R < 2; ++R)
#pragma unroll
    for (int db = 0; db < DB; ++db) voff[R][db] = swz_off<D>(8 * R + tr_r, db * 32 + tr_c);

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;
  const int ntiles = (k_end - k_begin + BC - 1) / BC;

  load_k(k_begin);
  issue_v(k_begin, sV[0]);

  auto step = [&](int t, auto buf_c) __attribute__((always_inline)) {
    constexpr int buf = decltype(buf_c)::value;
    const int t0 = k_begin + t * BC;
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s[kb] = mfma_bf16(ka[kb][ks], qf[ks], s[kb]);
    // the next tile's K (registers, free again) and V (other buffer)
    const bool more = t + 1 < ntiles;
    if (more) {
      load_k(t0 + BC);
      issue_v(t0 + BC, sV[buf ^ 1]);
    }
    // softmax over the tile's keys (registers: rows = keys, lane = query)
    float cc = c;
    if (t0 + BC > k_end) {
      cc = 1.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = t0 + kb * 32 + (r >> 2) * 8 + hi * 4 + (r & 3);
          s[kb][r] = key < k_end ? s[kb][r] * c : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = wave_max_halves(mx) * cc;
    const float m_new = (mx > m + kLazyMax) ? mx : m;
    const float alpha = (m == kNegInf) ? 0.f : fast_exp2(m - m_new);
    bf16x8 p[4];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          e[i] = fast_exp2(__builtin_fmaf(s[kb][8 * tt + i], cc, -m_new));
          rs += e[i];
        }
        p[kb * 2 + tt] = pack_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
      }
    l = alpha * l + rs;
    m = m_new;
    if (alpha != 1.f) {
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    // V of this tile has landed once at most the next tile's loads (K: 2*KS,
    // V: LPT) are outstanding.
    if (more) barrier_vmem_n<2 * KS + LPT>();
    else barrier_vmem_n<0>();
    const uint16_t* vt = sV[buf];
#pragma unroll
    for (int i = 0; i < 4 * DB; ++i) {
      const uint16_t* v0 = vt + (i / DB) * 16 * D;
      const bf16x8 va = join_u32x2(lds_read_tr16(v0 + voff[0][i % DB]), lds_read_tr16(v0 + voff[1][i % DB]));
      o[i % DB] = mfma_bf16(va, p[i / DB], o[i % DB]);
    }
    // This buffer is refilled by the next step's direct loads: its reads
    // must be complete, and the compiler must not move them past that issue.
    __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) step(t + 1, std::integral_constant<int, 1>{});
  }

  // The piece's state: m (base 2, scaled scores), l, and O^T unnormalised.
  const float lt = wave_sum_halves(l);
  if (row_ok) {
    float* po = a.part_o + pidx * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x16& x = o[db];
        *(f32x4*)(po + db * 32 + g * 8 + hi * 4) = f32x4{x[4 * g + 0], x[4 * g + 1], x[4 * g + 2], x[4 * g + 3]};
      }
    if (hi == 0) {
      a.part_ml[2 * pidx] = m;
      a.part_ml[2 * pidx + 1] = lt;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(64) decode_merge_kernel(DecodeArgs a) {
  constexpr int PER = D / 64;  // features per lane
  const int bh = blockIdx.x;   // b * H + h
  const int lane = threadIdx.x;
  const float* ml = a.part_ml + (int64_t)bh * a.nsplit * 2;
  const float* po = a.part_o + (int64_t)bh * a.nsplit * D + lane * PER;
  float mg = kNegInf;
  for (int t = 0; t < a.nsplit; ++t) mg = fmaxf(mg, ml[2 * t]);
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float den = 0.f;
  if (mg != kNegInf) {
    for (int t = 0; t < a.nsplit; ++t) {
      const float mt = ml[2 * t];
      if (mt == kNegInf) continue;
      const float wt = fast_exp2(mt - mg);
      den += wt * ml[2 * t + 1];
#pragma unroll
      for (int j = 0; j < PER; ++j) acc[j] += wt * po[(int64_t)t * D + j];
    }
  }
  const bool dead = mg == kNegInf || !(den > 0.f);
  const float inv = dead ? 0.f : 1.f / den;
  uint16_t* op = (uint16_t*)a.o + (int64_t)bh * D + lane * PER;
  if constexpr (PER == 2) {
    *(uint32_t*)op = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  } else {
    op[0] = (uint16_t)(pack_bf16x2(acc[0] * inv, 0.f) & 0xffffu);
  }
  if (lane == 0) a.lse[bh] = dead ? kNegInf : (mg + fast_log2(den)) * kLn2;
}

hipError_t launch_decode_bf16(const DecodeArgs& a, int d, hipStream_t stream) {
  const int G = a.H / a.Hkv;
  const int64_t split_blocks = (int64_t)a.B * a.Hkv * ((G + 31) / 32) * a.nsplit;
  const int64_t merge_blocks = (int64_t)a.B * a.H;
  if (split_blocks <= 0) return hipSuccess;
  if (split_blocks > 0x7fffffff || merge_blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 128) {
    hipLaunchKernelGGL(decode_split_kernel<128>, dim3((unsigned)split_blocks), dim3(64), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<128>, dim3((unsigned)merge_blocks), dim3(64), 0, stream, a);
  } else if (d == 64) {
    hipLaunchKernelGGL(decode_split_kernel<64>, dim3((unsigned)split_blocks), dim3(64), 0, stream, a);
    hipLaunchKernelGGL(decode_merge_kernel<64>, dim3((unsigned)merge_blocks), dim3(64), 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace miattn
