// C-ABI layer of libmiattn: argument validation, workspace carving and
// dispatch to the gfx950 kernels.  Nothing here allocates, frees or
// synchronises; every launch goes to the caller's stream.
#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/miattn.h"
#include "miattn_device.h"
#include "miattn_launch.h"

using miattn::AttnArgs;

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool ptr16(const void* p) { return p != nullptr && aligned(p, 16); }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// bf16 backward workspace: fp32 D, one entry per row.
size_t workspace_bytes_for(int64_t rows) { return round_up((size_t)rows * sizeof(float), 256); }

// fp32 backward workspace: fp32 D, then an fp32 dQ accumulator (rows * d).
size_t workspace_bytes_f32(int64_t rows, int d) {
  return round_up((size_t)rows * sizeof(float), 256) + (size_t)rows * (size_t)d * sizeof(float);
}

void carve(AttnArgs& a, void* ws, int64_t rows) {
  a.dvec = static_cast<float*>(ws);
  a.dq_acc = reinterpret_cast<float*>(static_cast<char*>(ws) + round_up((size_t)rows * sizeof(float), 256));
}

int check_dense(int B, int H, int N, int d, float scale) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || !std::isfinite(scale)) return MIATTN_ERR_INVALID_ARG;
  // Largest grid: one workgroup per (32-row tile, batch, head).
  const int64_t tiles = ((int64_t)N + 31) / 32 * (int64_t)B * H;
  if (tiles > 0x7fffffffLL || (int64_t)B * H * N > (int64_t)1 << 40) return MIATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MIATTN_ERR_UNSUPPORTED;
  return MIATTN_OK;
}

int check_varlen(const int* cu, int nseq, int max_seqlen, int total_tokens, int H, int d, float scale) {
  if (cu == nullptr || !aligned(cu, 4)) return MIATTN_ERR_INVALID_ARG;
  if (nseq <= 0 || max_seqlen <= 0 || total_tokens <= 0 || H <= 0 || !std::isfinite(scale))
    return MIATTN_ERR_INVALID_ARG;
  const int64_t tiles = ((int64_t)max_seqlen + 31) / 32 * (int64_t)nseq * H;
  if (tiles > 0x7fffffffLL) return MIATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MIATTN_ERR_UNSUPPORTED;
  return MIATTN_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MIATTN_OK : MIATTN_ERR_HIP; }

bool groups_ok(int H, int H_kv) { return H_kv > 0 && H > 0 && H % H_kv == 0; }

// Sliding window arguments -> mask mode.  A side of -1 is unbounded; sides
// are clamped to [0, N]; a causal mask is the right side 0.  A window that
// restricts nothing runs the plain kernels (mode kMaskPlain, *causal set to
// whether the result is the causal mask); otherwise a.win_* are set.
int window_mode(AttnArgs& a, int N, int left, int right, bool* causal, int* mode) {
  if (left < -1 || right < -1) return MIATTN_ERR_INVALID_ARG;
  const int L = left < 0 ? N : (left < N ? left : N);
  int R = right < 0 ? N : (right < N ? right : N);
  if (*causal) R = 0;
  if (L >= N - 1 && (R == 0 || R >= N - 1)) {
    *causal = R == 0 && N > 1;
    *mode = miattn::kMaskPlain;
    return MIATTN_OK;
  }
  a.win_left = L;
  a.win_right = R;
  *causal = false;
  *mode = miattn::kMaskWindow;
  return MIATTN_OK;
}

// Block-sparse list: blocks of MIATTN_SPARSE_BLOCK tokens, one CSR row per
// query block, shared by every (batch, head).
int sparse_args(AttnArgs& a, int N, const int* row_ptr, const int* col_idx, int nnz) {
  if (N > miattn::kMaxSparseBlocks * miattn::kSparseBlock) return MIATTN_ERR_UNSUPPORTED;
  if (row_ptr == nullptr || !aligned(row_ptr, 4) || nnz < 0) return MIATTN_ERR_INVALID_ARG;
  if (nnz > 0 && (col_idx == nullptr || !aligned(col_idx, 4))) return MIATTN_ERR_INVALID_ARG;
  a.blk_row_ptr = row_ptr;
  a.blk_col_idx = col_idx;
  a.blk_nnz = nnz;
  a.n_qblk = (N + miattn::kSparseBlock - 1) / miattn::kSparseBlock;
  a.n_kblk = a.n_qblk;
  return MIATTN_OK;
}

// Split plan of decoding: about one wave per SIMD of the chip (1024 waves) in
// total, at least 256 keys per piece, pieces a multiple of 64 keys.
constexpr int64_t kDecodeWaveTarget = 1024;

void decode_plan(int B, int H, int H_kv, int N, int* nsplit, int* chunk) {
  const int64_t units = (int64_t)B * H_kv * ((H / H_kv + 31) / 32);
  const int64_t want = (kDecodeWaveTarget + units - 1) / units;
  const int64_t most = ((int64_t)N + 255) / 256;
  int64_t ns = want < most ? want : most;
  if (ns < 1) ns = 1;
  int64_t ch = ((int64_t)N + ns - 1) / ns;
  ch = (ch + 63) / 64 * 64;
  *chunk = (int)ch;
  *nsplit = (int)(((int64_t)N + ch - 1) / ch);
}

int check_decode(int B, int H, int H_kv, int N, int d, float scale) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0 || !std::isfinite(scale) || !groups_ok(H, H_kv))
    return MIATTN_ERR_INVALID_ARG;
  if ((int64_t)B * H_kv * N > (int64_t)1 << 40 || (int64_t)B * H > 0x7fffffffLL) return MIATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MIATTN_ERR_UNSUPPORTED;
  return MIATTN_OK;
}

size_t decode_workspace_bytes(int B, int H, int H_kv, int N, int d) {
  int nsplit = 0, chunk = 0;
  decode_plan(B, H, H_kv, N, &nsplit, &chunk);
  const size_t parts = (size_t)B * H * nsplit;
  return round_up(parts * 2 * sizeof(float), 256) + parts * (size_t)d * sizeof(float);
}

size_t sparse_table_bytes(int N) {
  const size_t nb = ((size_t)N + miattn::kSparseBlock - 1) / miattn::kSparseBlock;
  return round_up(nb * nb, 256);
}

// Balanced key-tile pass over a block list: a key block listed by more than
// `chunk` query blocks is cut into chunks of `chunk` (the average list
// length, at least 4).  A cut block with list length n > chunk takes
// ceil(n / chunk) < 2 n / chunk chunks, and the list lengths add up to at
// most nnz, so fewer than 2 nnz / chunk partial slots and at most
// nb + nnz / chunk work items exist.
struct SparsePlan {
  int nb, chunk, max_work, max_slots;
  size_t off_table, off_work, off_slot, off_nch, off_part, total;
};

SparsePlan sparse_plan(int B, int H, int H_kv, int N, int d, int nnz) {
  SparsePlan p;
  p.nb = (N + miattn::kSparseBlock - 1) / miattn::kSparseBlock;
  // The per-key-block lists come from the expanded table, so they hold at
  // most nb * nb entries in total whatever nnz says (repeats and
  // out-of-range entries drop out); planning with the smaller bound keeps
  // every count below 2^21.
  const int64_t cap = (int64_t)p.nb * p.nb;
  const int L = (int)((int64_t)nnz < cap ? (int64_t)nnz : cap);
  const int avg = (L + p.nb - 1) / p.nb;
  p.chunk = avg > 4 ? avg : 4;
  p.max_work = p.nb + (L + p.chunk - 1) / p.chunk;
  p.max_slots = (2 * L + p.chunk - 1) / p.chunk + 1;
  const int64_t rows = (int64_t)B * H * N;
  p.off_table = workspace_bytes_for(rows);
  p.off_work = p.off_table + sparse_table_bytes(N);
  p.off_slot = p.off_work + round_up((size_t)(1 + p.max_work) * sizeof(int), 256);
  p.off_nch = p.off_slot + round_up((size_t)p.nb * sizeof(int), 256);
  p.off_part = p.off_nch + round_up((size_t)p.nb * sizeof(int), 256);
  p.total = p.off_part + (size_t)B * H_kv * p.max_slots * 2 * miattn::kSparseBlock * d * sizeof(float);
  return p;
}

// Scratch of the allocation-free backward (attn_bwd_noalloc): D for every
// row, in a file-scope device array that each GPU holds from the library's
// load until the process ends.  In host code `scratch` only names the symbol;
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and kept in scratch_ptr.  Every call on one GPU shares
// that GPU's copy, so calls that overlap on one GPU race.
constexpr size_t kScratchBytes = (size_t)32 << 20;   // D of up to 8M rows
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];

// Device address of this device's scratch, or nullptr on a HIP error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

AttnArgs dense_args(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int H,
                    int N, float scale) {
  AttnArgs a = {};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = const_cast<void*>(o);
  a.lse = const_cast<float*>(lse);
  a.B = B;
  a.H = H;
  a.Hkv = H;
  a.N = N;
  a.total_tokens = 0;
  a.scale = scale;
  a.scale_log2 = scale * miattn::kLog2e;
  return a;
}

}  // namespace

extern "C" {

int miattn_version(void) { return kVersion; }

const char* miattn_status_string(int status) {
  switch (status) {
    case MIATTN_OK: return "ok";
    case MIATTN_ERR_INVALID_ARG: return "invalid argument";
    case MIATTN_ERR_UNSUPPORTED: return "unsupported head dimension (supported: 64, 128)";
    case MIATTN_ERR_HIP: return "HIP runtime error at launch";
    case MIATTN_ERR_TOO_LARGE: return "problem larger than the library's built-in scratch (attn_bwd_noalloc: B*H*N <= 8388608)";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             float scale, int causal, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  return hip_status(miattn::launch_fwd_bf16(a, d, causal != 0, false, stream));
}

size_t attn_bwd_workspace_bytes(int B, int H, int N, int d) {
  if (check_dense(B, H, N, d, 1.0f) != MIATTN_OK) return 0;
  return workspace_bytes_for((int64_t)B * H * N);
}

size_t attn_bwd_f32_workspace_bytes(int B, int H, int N, int d) {
  if (check_dense(B, H, N, d, 1.0f) != MIATTN_OK) return 0;
  return workspace_bytes_f32((int64_t)B * H * N, d);
}

int attn_bwd_preprocess(const void* o, const void* dO, int B, int H, int N, int d, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(o) || !ptr16(dO) || !ptr16(workspace)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, 1.0f)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(nullptr, nullptr, nullptr, o, nullptr, B, H, N, 1.0f);
  a.dout = dO;
  carve(a, workspace, rows);
  return hip_status(miattn::launch_bwd_prep_bf16(a, d, false, stream));
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO, void* dk, void* dv,
                  int B, int H, int N, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                  hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(lse) || !ptr16(dO) || !ptr16(dk) || !ptr16(dv) ||
      !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, nullptr, lse, B, H, N, scale);
  a.dout = dO;
  a.dk = dk;
  a.dv = dv;
  carve(a, workspace, rows);
  return hip_status(miattn::launch_bwd_dkdv_bf16(a, d, causal != 0, false, stream));
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO, void* dq, int B,
                int H, int N, int d, float scale, int causal, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, nullptr, lse, B, H, N, scale);
  a.dout = dO;
  a.dq = dq;
  carve(a, workspace, rows);
  return hip_status(miattn::launch_bwd_dq_bf16(a, d, causal != 0, false, stream));
}

int attn_bwd_dq_preprocess(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, void* dq, int B, int H, int N, int d, float scale, int causal,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.dout = dO;
  a.dq = dq;
  a.dq_writes_d = 1;
  carve(a, workspace, rows);
  return hip_status(miattn::launch_bwd_dq_bf16(a, d, causal != 0, false, stream));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
             void* dk, void* dv, int B, int H, int N, int d, float scale, int causal, void* workspace,
             size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  carve(a, workspace, rows);
  // the dQ pass computes and stores D (no pre-pass); the dK/dV pass reads it
  a.dq_writes_d = 1;
  if (int st = hip_status(miattn::launch_bwd_dq_bf16(a, d, causal != 0, false, stream))) return st;
  return hip_status(miattn::launch_bwd_dkdv_bf16(a, d, causal != 0, false, stream));
}

size_t attn_bwd_noalloc_max_rows(void) { return kScratchBytes / sizeof(float); }

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                     void* dq, void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                     hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if ((size_t)rows > kScratchBytes / sizeof(float)) return MIATTN_ERR_TOO_LARGE;
  void* ws = device_scratch();
  if (ws == nullptr) return MIATTN_ERR_HIP;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  carve(a, ws, rows);
  // the same two passes as attn_bwd: the dQ pass writes D of every row into
  // the scratch before the dK/dV pass reads it, so nothing needs clearing
  a.dq_writes_d = 1;
  if (int st = hip_status(miattn::launch_bwd_dq_bf16(a, d, causal != 0, false, stream))) return st;
  return hip_status(miattn::launch_bwd_dkdv_bf16(a, d, causal != 0, false, stream));
}

int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                 int d, float scale, int causal, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.Hkv = H_kv;
  return hip_status(miattn::launch_fwd_bf16(a, d, causal != 0, false, stream));
}

int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                 void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.Hkv = H_kv;
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  carve(a, workspace, rows);
  // the dQ pass computes and stores D (no pre-pass); the dK/dV pass reads it
  a.dq_writes_d = 1;
  if (int st = hip_status(miattn::launch_bwd_dq_bf16(a, d, causal != 0, false, stream))) return st;
  return hip_status(miattn::launch_bwd_dkdv_bf16(a, d, causal != 0, false, stream));
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv, int N,
                    int d, float scale, int causal, int window_left, int window_right, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.Hkv = H_kv;
  bool c = causal != 0;
  int mode = 0;
  if (int st = window_mode(a, N, window_left, window_right, &c, &mode)) return st;
  if (mode == miattn::kMaskPlain) return hip_status(miattn::launch_fwd_bf16(a, d, c, false, stream));
  return hip_status(miattn::launch_fwd_masked_bf16(a, d, mode, false, stream));
}

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                    void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d, float scale, int causal,
                    int window_left, int window_right, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.Hkv = H_kv;
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  carve(a, workspace, rows);
  bool c = causal != 0;
  int mode = 0;
  if (int st = window_mode(a, N, window_left, window_right, &c, &mode)) return st;
  a.dq_writes_d = 1;  // the dQ pass stores D for the dK/dV pass
  if (mode == miattn::kMaskPlain) {
    if (int st = hip_status(miattn::launch_bwd_dq_bf16(a, d, c, false, stream))) return st;
    return hip_status(miattn::launch_bwd_dkdv_bf16(a, d, c, false, stream));
  }
  if (int st = hip_status(miattn::launch_bwd_dq_masked_bf16(a, d, mode, false, stream))) return st;
  return hip_status(miattn::launch_bwd_dkdv_masked_bf16(a, d, mode, false, stream));
}

int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int H_kv,
                          int N, int d, float scale, int causal, const int* row_ptr, const int* col_idx, int nnz,
                          hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.Hkv = H_kv;
  if (int st = sparse_args(a, N, row_ptr, col_idx, nnz)) return st;
  return hip_status(miattn::launch_fwd_masked_bf16(a, d, miattn::kMaskBlocks, causal != 0, stream));
}

size_t attn_bwd_block_sparse_workspace_bytes(int B, int H, int H_kv, int N, int d, int nnz) {
  if (check_dense(B, H, N, d, 1.0f) != MIATTN_OK || !groups_ok(H, H_kv) || nnz < 0) return 0;
  if (N > miattn::kMaxSparseBlocks * miattn::kSparseBlock) return 0;
  return sparse_plan(B, H, H_kv, N, d, nnz).total;
}

int attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dO, void* dq, void* dk, void* dv, int B, int H, int H_kv, int N, int d,
                          float scale, int causal, const int* row_ptr, const int* col_idx, int nnz, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  if (int st = sparse_args(a, N, row_ptr, col_idx, nnz)) return st;
  const SparsePlan plan = sparse_plan(B, H, H_kv, N, d, nnz);
  if (workspace_bytes < plan.total) return MIATTN_ERR_INVALID_ARG;
  a.Hkv = H_kv;
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  carve(a, workspace, rows);
  char* ws = static_cast<char*>(workspace);
  uint8_t* table = reinterpret_cast<uint8_t*>(ws + plan.off_table);
  int* work = reinterpret_cast<int*>(ws + plan.off_work);
  int* slot = reinterpret_cast<int*>(ws + plan.off_slot);
  int* nch = reinterpret_cast<int*>(ws + plan.off_nch);
  a.blk_table = table;
  a.blk_work = work;
  a.blk_slot = slot;
  a.blk_nch = nch;
  a.blk_part = reinterpret_cast<float*>(ws + plan.off_part);
  a.blk_chunk = plan.chunk;
  a.blk_nslots = plan.max_slots;
  a.blk_max_work = plan.max_work;
  const bool c = causal != 0;
  if (int st = hip_status(miattn::launch_block_table(a, table, stream))) return st;
  if (int st = hip_status(miattn::launch_block_work(a, c, work, slot, nch, stream))) return st;
  // The dQ pass stores D for the dK/dV pass.  A query block with an empty
  // list stores none, and no key block's list holds it (both passes drop
  // the same entries), so the dK/dV pass never reads it.
  a.dq_writes_d = 1;
  if (int st = hip_status(miattn::launch_bwd_dq_masked_bf16(a, d, miattn::kMaskBlocks, c, stream))) return st;
  if (int st = hip_status(miattn::launch_bwd_dkdv_masked_bf16(a, d, miattn::kMaskBlocks, c, stream))) return st;
  return hip_status(miattn::launch_block_reduce(a, d, stream));
}

size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int N_kv, int d) {
  if (check_decode(B, H, H_kv, N_kv, d, 1.0f) != MIATTN_OK) return 0;
  return decode_workspace_bytes(B, H, H_kv, N_kv, d);
}

int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse, int B, int H,
                int H_kv, int N_kv, int d, float scale, const int* cache_seqlens, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k_cache) || !ptr16(v_cache) || !ptr16(o) || lse == nullptr || !aligned(lse, 4) ||
      !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (cache_seqlens != nullptr && !aligned(cache_seqlens, 4)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_decode(B, H, H_kv, N_kv, d, scale)) return st;
  if (workspace_bytes < decode_workspace_bytes(B, H, H_kv, N_kv, d)) return MIATTN_ERR_INVALID_ARG;
  miattn::DecodeArgs a = {};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = o;
  a.lse = lse;
  a.seqlens = cache_seqlens;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.N = N_kv;
  decode_plan(B, H, H_kv, N_kv, &a.nsplit, &a.chunk);
  const size_t parts = (size_t)B * H * a.nsplit;
  a.part_ml = static_cast<float*>(workspace);
  a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + round_up(parts * 2 * sizeof(float), 256));
  a.scale = scale;
  a.scale_log2 = scale * miattn::kLog2e;
  return hip_status(miattn::launch_decode_bf16(a, d, stream));
}

int attn_quantize_fp8_rows(const void* x, unsigned char* x8, float* scales, int B, int H, int N, int d,
                           hipStream_t stream) {
  if (!ptr16(x) || !ptr16(x8) || scales == nullptr || !aligned(scales, 4)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, 1.0f)) return st;
  if (d != 128) return MIATTN_ERR_UNSUPPORTED;
  return hip_status(miattn::launch_quant_rows_fp8(x, x8, scales, B * H, N, d, stream));
}

int attn_quantize_fp8_vt(const void* v, unsigned char* v8t, float* scales, int B, int H, int N, int d,
                         hipStream_t stream) {
  if (!ptr16(v) || !ptr16(v8t) || scales == nullptr || !aligned(scales, 4)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, 1.0f)) return st;
  if (d != 128) return MIATTN_ERR_UNSUPPORTED;
  return hip_status(miattn::launch_quant_vt_fp8(v, v8t, scales, B * H, N, d, stream));
}

int attn_fwd_fp8(const unsigned char* q8, const float* q_scale, const unsigned char* k8, const float* k_scale,
                 const unsigned char* v8t, const float* v_scale, void* o, float* lse, int B, int H, int H_kv, int N,
                 int d, float scale, int causal, hipStream_t stream) {
  if (!ptr16(q8) || !ptr16(k8) || !ptr16(v8t) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  for (const float* p : {q_scale, k_scale, v_scale})
    if (p == nullptr || !aligned(p, 4)) return MIATTN_ERR_INVALID_ARG;
  if (!groups_ok(H, H_kv)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  if (d != 128) return MIATTN_ERR_UNSUPPORTED;
  miattn::Fp8Args a = {};
  a.q8 = q8;
  a.q_scale = q_scale;
  a.k8 = k8;
  a.k_scale = k_scale;
  a.v8t = v8t;
  a.v_scale = v_scale;
  a.o = o;
  a.lse = lse;
  a.B = B;
  a.H = H;
  a.Hkv = H_kv;
  a.N = N;
  a.scale = scale;
  a.scale_log2 = scale * miattn::kLog2e;
  return hip_status(miattn::launch_fwd_fp8(a, d, causal != 0, stream));
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int d,
                 float scale, int causal, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  return hip_status(miattn::launch_fwd_f32(a, d, causal != 0, stream));
}

int attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse, const float* dO,
                 float* dq, float* dk, float* dv, int B, int H, int N, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_dense(B, H, N, d, scale)) return st;
  const int64_t rows = (int64_t)B * H * N;
  if (workspace_bytes < workspace_bytes_f32(rows, d)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, o, lse, B, H, N, scale);
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  carve(a, workspace, rows);
  return hip_status(miattn::launch_bwd_f32(a, d, causal != 0, stream));
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens,
                    int nseq, int max_seqlen, int total_tokens, int H, int d, float scale, int causal,
                    const unsigned char* key_valid, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse)) return MIATTN_ERR_INVALID_ARG;
  if (int st = check_varlen(cu_seqlens, nseq, max_seqlen, total_tokens, H, d, scale)) return st;
  AttnArgs a = dense_args(q, k, v, o, lse, nseq, H, max_seqlen, scale);
  a.cu_seqlens = cu_seqlens;
  a.key_valid = key_valid;
  a.total_tokens = total_tokens;
  return hip_status(miattn::launch_fwd_bf16(a, d, causal != 0, true, stream));
}

size_t attn_bwd_varlen_workspace_bytes(int total_tokens, int H, int d) {
  if (total_tokens <= 0 || H <= 0 || (d != 64 && d != 128)) return 0;
  return workspace_bytes_for((int64_t)total_tokens * H);
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                    void* dq, void* dk, void* dv, const int* cu_seqlens, int nseq, int max_seqlen, int total_tokens,
                    int H, int d, float scale, int causal, const unsigned char* key_valid, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (!ptr16(q) || !ptr16(k) || !ptr16(v) || !ptr16(o) || !ptr16(lse) || !ptr16(dO) || !ptr16(dq) ||
      !ptr16(dk) || !ptr16(dv) || !ptr16(workspace))
    return MIATTN_ERR_INVALID_ARG;
  if (int st = check_varlen(cu_seqlens, nseq, max_seqlen, total_tokens, H, d, scale)) return st;
  const int64_t rows = (int64_t)total_tokens * H;
  if (workspace_bytes < workspace_bytes_for(rows)) return MIATTN_ERR_INVALID_ARG;
  AttnArgs a = dense_args(q, k, v, o, lse, nseq, H, max_seqlen, scale);
  a.dout = dO;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu_seqlens = cu_seqlens;
  a.key_valid = key_valid;
  a.total_tokens = total_tokens;
  carve(a, workspace, rows);
  a.dq_writes_d = 1;  // the dQ pass stores D for the dK/dV pass
  if (int st = hip_status(miattn::launch_bwd_dq_bf16(a, d, causal != 0, true, stream))) return st;
  return hip_status(miattn::launch_bwd_dkdv_bf16(a, d, causal != 0, true, stream));
}

}  // extern "C"
