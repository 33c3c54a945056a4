// Device-side building blocks shared by the libmiattn kernels (gfx950 / CDNA4).
//
// Register layouts used throughout (checked on the device by a lane probe):
//  * v_mfma_f32_32x32x16_bf16: lane l supplies row (A) or column (B) l % 32 and
//    eight k-values; lanes 0-31 and 32-63 carry two disjoint k-halves.  A and B
//    use the same lane/element -> k assignment, so any k order is fine as long
//    as both operands are packed the same way.
//  * 32x32 fp32 accumulator: lane l holds column l % 32, register r holds row
//    (r / 4) * 8 + (l / 32) * 4 + (r % 4).
//  * ds_read_b64_tr_b16: within each 16-lane group, source lane i names 4
//    consecutive 16-bit elements M[i][0..3]; result lane j receives
//    M[j/4 + 4t][j % 4] for t = 0..3.  Pointing source lane i at row (i / 4),
//    column 4 * (i % 4) of a row-major tile hands result lane j column j of
//    four consecutive rows: a transposed read of a 4 x 16 block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace miattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MIATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();
// Online softmax with a lazy reference max: a row's reference is raised only
// when a tile's max exceeds it by more than this (base-2 units), so P~ stays
// below 2^kLazyMax; any reference gives the same O and LSE up to rounding.
constexpr float kLazyMax = 8.0f;
// The forward exponentiates a tile against the running reference without the
// row max while every partial row sum stays at or below this (so every P~ does).
constexpr float kSumLimit = 65536.0f;

// Everything a kernel needs to address one problem.  Dense tensors are
// [B, H, N, d] with LSE/D as [B, H, N]; packed tensors are [T, H, d] with
// LSE/D as [H, T] and per-sequence offsets in cu_seqlens.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;     // D = rowsum(dO * O), laid out like LSE
  float* dq_acc;   // fp32 dQ accumulator, laid out like Q
  const int* cu_seqlens;
  const uint8_t* key_valid;  // per packed token, nonzero = valid key (nullable)
  int B;           // dense: batch; packed: number of sequences
  int H;           // query heads (Q, O, dO, dQ, LSE, D)
  int Hkv;         // key/value heads (K, V, dK, dV); divides H, query head h
                   // reads key/value head h / (H / Hkv); Hkv == H without grouping
  int N;           // dense: sequence length; packed: longest sequence
  int total_tokens;
  float scale;     // multiplies Q K^T
  float scale_log2;  // scale * log2(e)
  // Sliding window (kernels with the window mask): key j is visible to query
  // i iff i - win_left <= j <= i + win_right; both are in [0, N] (the host
  // maps an unbounded side to N and folds a causal mask into win_right = 0).
  int win_left;
  int win_right;
  // Block-sparse list (kernels with the block mask): query block r attends
  // the key blocks blk_col_idx[blk_row_ptr[r] .. blk_row_ptr[r+1]), blocks of
  // kSparseBlock tokens; blk_table[r * n_kblk + c] != 0 is the same list
  // expanded (built for the backward key-tile pass).
  const int* blk_row_ptr;
  const int* blk_col_idx;
  int blk_nnz;     // length of blk_col_idx: entries past it are never read
  int n_qblk;
  int n_kblk;
  const uint8_t* blk_table;
  // Backward key-tile pass over a block list, split for balance: a key block
  // listed by more than blk_chunk query blocks is cut into chunks of
  // blk_chunk query blocks, one workgroup each.  blk_work[0] = number of work
  // items, blk_work[1 + w] = key block | (chunk << 16); blk_slot[c] = first
  // partial-sum slot of key block c (-1 when it is not cut), blk_nch[c] its
  // chunk count; blk_part holds fp32 partial dK and dV per (batch, key/value
  // head, slot): [B * Hkv][blk_nslots][2][128][D].
  const int* blk_work;
  const int* blk_slot;
  const int* blk_nch;
  float* blk_part;
  int blk_chunk;
  int blk_nslots;
  int blk_max_work;
  // Nonzero: the dQ pass computes D = rowsum(dO o O) of its rows itself (from
  // o and dout), stores it in dvec for the dK/dV pass and uses it (no D
  // pre-pass); zero: it reads dvec.
  int dq_writes_d;
};

// Decoding against a KV cache (one query token per sequence), split along
// the cache: q, o [B, H, D]; k, v [B, Hkv, N, D]; lse [B, H]; piece t of a
// sequence covers keys [t * chunk, (t + 1) * chunk).  part_ml [B*H][nsplit][2]
// holds each piece's (max in base-2 units, sum), part_o [B*H][nsplit][D] its
// unnormalised output.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* seqlens;  // [B] cache lengths, or null for N
  float* part_o;
  float* part_ml;
  int B;
  int H;
  int Hkv;
  int N;
  int nsplit;
  int chunk;
  float scale;
  float scale_log2;
};

// FP8 (E4M3) forward: codes and their fp32 scales.  Q [B, H, N, D] and K
// [B, Hkv, N, D] codes with one scale per 64-row block ([.., ceil(N/64)]);
// V codes per 64-key tile transposed, [B, Hkv, ceil(N/64), D, 64], one scale
// per (batch, head).
struct Fp8Args {
  const uint8_t* q8;
  const float* q_scale;
  const uint8_t* k8;
  const float* k_scale;
  const uint8_t* v8t;
  const float* v_scale;
  void* o;
  float* lse;
  int B;
  int H;
  int Hkv;
  int N;
  float scale;
  float scale_log2;
};

// Mask modes of the kernels besides none / causal.
enum : int { kMaskPlain = 0, kMaskWindow = 1, kMaskBlocks = 2 };
constexpr int kSparseBlock = 128;       // tokens per block of a block-sparse list
constexpr int kMaxSparseBlocks = 1024;  // blocks per sequence (N <= 131072)

// Where one (sequence, query head) lives, and the key/value head it reads.
struct SeqView {
  int64_t base;        // Q/O/dO/dQ element offset of token 0, feature 0
  int64_t tok_stride;  // elements between consecutive tokens of Q/O/dO/dQ
  int64_t kv_base;     // K/V/dK/dV element offset of token 0, feature 0
  int64_t kv_stride;   // elements between consecutive tokens of K/V/dK/dV
  int64_t row_base;    // offset of token 0 in LSE / D
  int64_t tok0;        // packed index of token 0 (key_valid indexing)
  int len;
};

template <bool VARLEN>
__device__ __forceinline__ SeqView seq_view(const AttnArgs& a, int b, int h, int D) {
  SeqView s;
  const int hk = h / (a.H / a.Hkv);
  if constexpr (VARLEN) {
    // Offsets are clamped into [0, total_tokens] and the length to [0, N]
    // (the longest sequence), so malformed offsets cannot address memory
    // outside the packed tensors: rows past the clamp are simply not written.
    const int t0 = min(max(a.cu_seqlens[b], 0), a.total_tokens);
    const int t1 = min(max(a.cu_seqlens[b + 1], t0), a.total_tokens);
    s.base = ((int64_t)t0 * a.H + h) * D;
    s.tok_stride = (int64_t)a.H * D;
    s.kv_base = ((int64_t)t0 * a.Hkv + hk) * D;
    s.kv_stride = (int64_t)a.Hkv * D;
    s.row_base = (int64_t)h * a.total_tokens + t0;
    s.tok0 = t0;
    s.len = min(t1 - t0, a.N);
  } else {
    s.base = ((int64_t)b * a.H + h) * (int64_t)a.N * D;
    s.tok_stride = D;
    s.kv_base = ((int64_t)b * a.Hkv + hk) * (int64_t)a.N * D;
    s.kv_stride = D;
    s.row_base = ((int64_t)b * a.H + h) * (int64_t)a.N;
    s.tok0 = (int64_t)b * a.N;
    s.len = a.N;
  }
  return s;
}

// Offsets of query head h within a group view: Q/O/dO/dQ element offset and
// LSE/D offset move by these per head.
template <bool VARLEN>
__device__ __forceinline__ int64_t q_head_stride(const AttnArgs& a, int D) {
  return VARLEN ? (int64_t)D : (int64_t)a.N * D;
}
template <bool VARLEN>
__device__ __forceinline__ int64_t row_head_stride(const AttnArgs& a) {
  return VARLEN ? (int64_t)a.total_tokens : (int64_t)a.N;
}

// Workgroup -> (sequence*head, tile), tile-major: every head's tile t before any
// head's tile t+1 (with heavy_last_tile, the last tile first), so the
// heaviest tiles of all heads start first and the grid ends on light ones.
// Consecutive workgroups of one head land on one XCD when the head count is a
// multiple of 8.
__device__ __forceinline__ void wg_coords_tile_major(int w, int nbh, int ntile, bool heavy_last_tile, int& bh,
                                                     int& t) {
  bh = w % nbh;
  t = w / nbh;
  if (heavy_last_tile) t = ntile - 1 - t;
}

// Workgroup -> (sequence*head, tile) for packed sequences, nh heads each:
// XCD x = w % 8 takes heads x*nh/8 .. (x+1)*nh/8 - 1 of every sequence (the
// same work on every XCD, whatever the lengths; grouped query heads keep
// their K/V head on one XCD) and works through them one (sequence, head) at a
// time, all its tiles together, so that the operands its tiles share stay in
// that XCD's L2.  With nh not a multiple of 8, tile-major.
__host__ __device__ __forceinline__ void wg_coords_unit_major(int w, int nseq, int nh, int ntile, int& bh, int& t) {
  if (nh % 8 != 0) {
    bh = w % (nseq * nh);
    t = w / (nseq * nh);
    return;
  }
  const int x = w & 7, l = w >> 3, hx = nh >> 3;
  const int u = l / ntile;
  t = l - u * ntile;
  const int seq = u / hx;
  bh = seq * nh + x * hx + (u - seq * hx);
}

// Workgroup -> (sequence*head, tile).  Workgroups are dispatched to the 8 XCDs
// in turn (w -> XCD w % 8), each XCD with its own L2.  When the grid divides by
// 8, XCD x takes the contiguous logical range [x*total/8, (x+1)*total/8),
// ordered head-major, so an XCD works through one or two heads at a time with
// all of their tiles in flight and their K/V (or Q/dO) stays in its L2.
// Otherwise the plain head-major order is used.  `heavy_last_tile` reverses
// the tile order inside a head when the last tile carries the most work.
__device__ __forceinline__ void wg_coords(int w, int nbh, int ntile, bool heavy_last_tile, int& bh, int& t) {
  const int total = nbh * ntile;
  int g = w;
  if ((total & 7) == 0) g = (w & 7) * (total >> 3) + (w >> 3);
  bh = g / ntile;
  t = g - bh * ntile;
  if (heavy_last_tile) t = ntile - 1 - t;
}

// Workgroup -> (sequence*head, tile) for query-tile passes.  The XCD split is
// that of wg_coords; inside its range an XCD takes groups of `group` heads,
// and inside a group the tiles go tile-major (every head's tile 0, then every
// head's tile 1, ...), heaviest first when `heavy_last_tile`.  group = 1 is
// wg_coords (all tiles of one head in flight together: equal-cost tiles, its
// K/V read once into L2); a small group > 1 keeps only a few heads' K/V hot
// per XCD while the heavy tiles of a group still start before its light ones
// (under a causal mask one head at a time would leave the heaviest tile of
// the last head to start late: about 9% longer in a greedy-schedule model of
// 16 heads x 16 tiles on 32 CUs, against none for groups of two or more).
// With the XCD split, the group narrows until it divides an XCD's range: a
// group that straddled two ranges would give one XCD the heavy tiles of its
// heads and the next XCD the light ones (B1 H16 N16384 causal: two heads per
// range, 3:1 work between neighbouring XCDs with groups of four).
// The result is a bijection of [0, nbh*ntile).
__host__ __device__ __forceinline__ void wg_coords_grouped(int w, int nbh, int ntile, int group,
                                                           bool heavy_last_tile, int& bh, int& t) {
  const int total = nbh * ntile;
  int g = w;
  if ((total & 7) == 0) {
    g = (w & 7) * (total >> 3) + (w >> 3);
    const int range = total >> 3;
    while (group > 1 && range % (group * ntile) != 0) --group;
  }
  const int per = group * ntile;
  const int grp = g / per;
  const int r = g - grp * per;
  const int rest = nbh - grp * group;
  const int gl = rest < group ? rest : group;  // the last group may hold fewer heads
  t = r / gl;
  bh = grp * group + (r - t * gl);
  if (heavy_last_tile) t = ntile - 1 - t;
}

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 x) { return __builtin_bit_cast(u32x4, x); }

// Round-to-nearest-even fp32 -> bf16 pairs (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

__device__ __forceinline__ bf16x8 pack_bf16x8(float x0, float x1, float x2, float x3,
                                              float x4, float x5, float x6, float x7) {
  u32x4 u = {pack_bf16x2(x0, x1), pack_bf16x2(x2, x3), pack_bf16x2(x4, x5), pack_bf16x2(x6, x7)};
  return as_bf16x8(u);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// Transposed 4 x 16 read from a row-major bf16 LDS tile (see the header note).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MIATTN_LDS i16x4*)(p));
  return __builtin_bit_cast(u32x2, t);
}

__device__ __forceinline__ bf16x8 join_u32x2(u32x2 lo, u32x2 hi) {
  u32x4 u = {lo[0], lo[1], hi[0], hi[1]};
  return as_bf16x8(u);
}

// Value held by the lane 32 positions away, through the LDS crossbar
// (ds_bpermute_b32; no LDS memory is touched).  v_permlane32_swap would be
// the natural instruction, but the compiler in use folds its two results into
// one register when both operands carry the same value, so it is not used.
__device__ __forceinline__ float lane_xor32(float x) {
  const int addr = (int)((__lane_id() ^ 32u) << 2);
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float wave_max_halves(float x) { return fmaxf(x, lane_xor32(x)); }
__device__ __forceinline__ float wave_sum_halves(float x) { return x + lane_xor32(x); }

// Swizzled LDS tiles.  A tile is row-major with rows of D bf16 elements and no
// padding; the 16-byte chunk c of row r is stored at chunk c ^ swz<D>(r).
// The XOR pattern makes both access shapes of the kernels conflict-free:
//  * 16 consecutive rows reading the same logical chunk (b128 operand reads
//    with lane = row) land on 16 distinct chunk slots of the 64 banks;
//  * the transpose read (4 consecutive rows starting at a multiple of 4, four
//    consecutive chunks starting at a multiple of 4) lands on 16 distinct
//    chunk slots.
// For D = 64 two rows share one 256-byte bank line, which the pattern for
// D = 64 accounts for.
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
  static_assert(D == 64 || D == 128, "swizzle defined for rows of 64 or 128 bf16");
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of (row r, element col) in a swizzled tile with rows of D.
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r)) << 3) | (col & 7));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value: conditions derived from it then compile to scalar branches instead
// of per-lane predication.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Masking and rescaling run only on a few tiles (diagonal, sequence end,
// padded keys, a moved row max), behind wave-uniform branches.  The compiler
// otherwise hoists their side-effect-free arithmetic above the branch and
// pays for it on every tile.  Passing an input of that arithmetic through an
// empty volatile asm inside the branch pins the computation there.
template <typename T>
__device__ __forceinline__ T pin_in_branch(T x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Direct 16-byte global -> LDS load (global_load_lds_dwordx4): lane i of the
// wave writes its 16 bytes to lds_wave_base + 16 * i; lds_wave_base must be
// wave-uniform (it goes to M0).  Issued through inline asm so that the
// compiler does not track it: it inserts no conservative waits for it before
// unrelated LDS reads, and (no memory clobber) it may schedule LDS reads and
// MFMAs across it, which lets the kernels spread their loads between MFMAs.
// Contract for callers: the destination is LDS that no wave reads before the
// next barrier_vmem_n, and that barrier waits for the load.  Both are volatile
// asm, so the compiler keeps them in program order.  M0 is written without
// being declared (the compiler rejects clobbers of reserved registers); the
// kernels keep no value of their own in M0.
__device__ __forceinline__ void lds_dma16(const void* g, void* lds_wave_base) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(MIATTN_LDS void*)lds_wave_base);
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m));
}

// The same load with the M0 value (the wave's LDS destination in bytes,
// wave-uniform) given directly, for callers that form it themselves.
__device__ __forceinline__ void lds_dma16_m0(const void* g, uint32_t m0_value) {
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0_value));
}

// Workgroup barrier for kernels that keep direct-to-LDS loads in flight
// across it.  __syncthreads() fences LDS, which makes the compiler wait for
// every outstanding direct load (vmcnt(0)) first; here the wave waits until
// at most N of its vector-memory operations (the N most recent, since they
// complete in issue order) are outstanding and all of its LDS operations are
// done, then meets the other waves.  The memory clobber keeps the compiler
// from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void barrier_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt field of 6 bits");
  __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

// Block-sparse lists in LDS.  A workgroup of query tile rows
// [q_tile0, q_tile0 + 2 * kSparseBlock) gathers the key blocks listed for its
// two query blocks into list[0 .. count): entry = block | (bits << 12), bit h
// set when query block h of the two lists it.  Out-of-range indices and
// entries past blk_nnz are ignored; a block listed twice counts once; under a
// causal mask blocks wholly above a query block's diagonal are dropped.  Every
// thread of the workgroup calls it (it holds barriers); returns count.
template <int NT, bool CAUSAL>
__device__ __forceinline__ int build_key_block_list(const AttnArgs& a, int q_tile0,
                                                    uint8_t (*flag)[kMaxSparseBlocks], uint16_t* list,
                                                    int* count_slot) {
  const int tid = threadIdx.x;
  for (int i = tid; i < a.n_kblk; i += NT) {
    flag[0][i] = 0;
    flag[1][i] = 0;
  }
  __syncthreads();
  const int qb0 = q_tile0 / kSparseBlock;
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int qb = qb0 + hb;
    if (qb < a.n_qblk) {
      const int e0 = min(max(a.blk_row_ptr[qb], 0), a.blk_nnz);
      const int e1 = min(max(a.blk_row_ptr[qb + 1], e0), a.blk_nnz);
      for (int e = e0 + tid; e < e1; e += NT) {
        const int c = a.blk_col_idx[e];
        if (c >= 0 && c < a.n_kblk && (!CAUSAL || c <= qb)) flag[hb][c] = 1;
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    int count = 0;
    for (int base = 0; base < a.n_kblk; base += 64) {
      const int c = base + lane;
      const int f = c < a.n_kblk ? (flag[0][c] | (flag[1][c] << 1)) : 0;
      const uint64_t m = __builtin_amdgcn_ballot_w64(f != 0);
      const int pos = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (f != 0) list[pos] = (uint16_t)(c | (f << 12));
      count += __builtin_popcountll(m);
    }
    if (lane == 0) *count_slot = count;
  }
  __syncthreads();
  return *count_slot;
}

// The query blocks that list key block c (from the expanded table), in
// increasing order, into list[0 .. count); under a causal mask query blocks
// wholly before the key block are dropped.  Every thread calls it; returns
// count.
template <bool CAUSAL>
__device__ __forceinline__ int build_query_block_list(const AttnArgs& a, int c, uint16_t* list, int* count_slot) {
  const int tid = threadIdx.x;
  if (tid < 64) {
    const int lane = tid;
    int count = 0;
    for (int base = 0; base < a.n_qblk; base += 64) {
      const int r = base + lane;
      const bool f = r < a.n_qblk && (!CAUSAL || r >= c) && a.blk_table[(int64_t)r * a.n_kblk + c] != 0;
      const uint64_t m = __builtin_amdgcn_ballot_w64(f);
      const int pos = count + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (f) list[pos] = (uint16_t)r;
      count += __builtin_popcountll(m);
    }
    if (lane == 0) *count_slot = count;
  }
  __syncthreads();
  return *count_slot;
}

}  // namespace miattn
