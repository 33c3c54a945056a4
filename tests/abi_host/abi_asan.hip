// Host-only exercise of the C-ABI layer (csrc/api.hip) under AddressSanitizer.
//
// The kernel launchers are replaced by stubs that only record what they were
// given, so every entry point runs its validation, workspace carving and
// planning on the host without a GPU.  "Device" buffers are host allocations
// of exactly the documented size: the layer must never dereference them, and
// ASan reports it if it does, or if it reads or writes past any buffer of
// its own.  Exit status 0 when every check holds.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "miattn.h"
#include "miattn_device.h"
#include "miattn_launch.h"

namespace miattn {
static int g_launches = 0;
static AttnArgs g_last = {};
static DecodeArgs g_dec = {};
static hipError_t rec(const AttnArgs& a) {
  ++g_launches;
  g_last = a;
  return hipSuccess;
}
hipError_t launch_fwd_bf16(const AttnArgs& a, int, bool, bool, hipStream_t) { return rec(a); }
hipError_t launch_bwd_prep_bf16(const AttnArgs& a, int, bool, hipStream_t) { return rec(a); }
hipError_t launch_bwd_dkdv_bf16(const AttnArgs& a, int, bool, bool, hipStream_t) { return rec(a); }
hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int, bool, bool, hipStream_t) { return rec(a); }
hipError_t launch_fwd_masked_bf16(const AttnArgs& a, int, int, bool, hipStream_t) { return rec(a); }
hipError_t launch_bwd_dkdv_masked_bf16(const AttnArgs& a, int, int, bool, hipStream_t) { return rec(a); }
hipError_t launch_bwd_dq_masked_bf16(const AttnArgs& a, int, int, bool, hipStream_t) { return rec(a); }
hipError_t launch_block_table(const AttnArgs& a, uint8_t*, hipStream_t) { return rec(a); }
hipError_t launch_block_work(const AttnArgs& a, bool, int*, int*, int*, hipStream_t) { return rec(a); }
hipError_t launch_block_reduce(const AttnArgs& a, int, hipStream_t) { return rec(a); }
hipError_t launch_decode_bf16(const DecodeArgs& a, int, hipStream_t) {
  ++g_launches;
  g_dec = a;
  return hipSuccess;
}
hipError_t launch_quant_rows_fp8(const void*, void*, float*, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quant_vt_fp8(const void*, void*, float*, int, int, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_fp8(const Fp8Args&, int, bool, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fwd_f32(const AttnArgs& a, int, bool, hipStream_t) { return rec(a); }
hipError_t launch_bwd_f32(const AttnArgs& a, int, bool, hipStream_t) { return rec(a); }
}  // namespace miattn

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

// A host buffer standing in for a device allocation of `bytes`, 256-aligned.
struct Buf {
  void* p;
  size_t n;
  explicit Buf(size_t bytes) : n(bytes) { p = std::aligned_alloc(256, (bytes + 255) / 256 * 256); }
  ~Buf() { std::free(p); }
  char* c() const { return static_cast<char*>(p); }
};

static bool inside(const void* p, const Buf& b, size_t len) {
  const char* c = static_cast<const char*>(p);
  return c >= b.c() && c + len <= b.c() + b.n;
}

int main() {
  using miattn::g_last;
  using miattn::g_launches;
  const int B = 2, H = 4, N = 300, d = 128;
  const size_t E = (size_t)B * H * N * d * 2, R = (size_t)B * H * N * 4;
  Buf q(E), k(E), v(E), o(E), g(E), dq(E), dk(E), dv(E), lse(R);
  const float sc = 0.088f;

  // ---- invalid arguments: refused before any launch
  const int before = g_launches;
  CHECK(attn_fwd(nullptr, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd(q.c() + 2, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 0, H, N, d, sc, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, -5, d, sc, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, 96, sc, 1, 0) == MIATTN_ERR_UNSUPPORTED);
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, NAN, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, INFINITY, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, 1 << 20, 1 << 10, 1 << 20, d, sc, 1, 0) ==
        MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd_gqa(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, 3, N, d, sc, 1, 0) == MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd_window(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, H, N, d, sc, 0, -2, 0, 0) ==
        MIATTN_ERR_INVALID_ARG);
  const size_t ws_need = attn_bwd_workspace_bytes(B, H, N, d);
  CHECK(ws_need == (R + 255) / 256 * 256);
  CHECK(attn_bwd_workspace_bytes(B, H, N, 80) == 0 && attn_bwd_workspace_bytes(-1, H, N, d) == 0);
  {
    Buf ws(ws_need);
    CHECK(attn_bwd(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, B, H, N, d, sc, 1, ws.p, ws_need - 1,
                   0) == MIATTN_ERR_INVALID_ARG);
    CHECK(attn_bwd(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, B, H, N, d, sc, 1, nullptr, ws_need,
                   0) == MIATTN_ERR_INVALID_ARG);
  }
  int cu_host[3] = {0, 100, 300};
  CHECK(attn_fwd_varlen(q.p, k.p, v.p, o.p, (float*)lse.p, cu_host, 0, 200, 300, H, d, sc, 1, nullptr, 0) ==
        MIATTN_ERR_INVALID_ARG);
  CHECK(attn_fwd_varlen(q.p, k.p, v.p, o.p, (float*)lse.p, nullptr, 2, 200, 300, H, d, sc, 1, nullptr, 0) ==
        MIATTN_ERR_INVALID_ARG);
  CHECK(attn_decode(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, 3, N, d, sc, nullptr, q.p, 1 << 20, 0) ==
        MIATTN_ERR_INVALID_ARG);
  CHECK(attn_quantize_fp8_rows(q.p, (unsigned char*)o.p, (float*)lse.p, B, H, N, 64, 0) == MIATTN_ERR_UNSUPPORTED);
  CHECK(attn_bwd_noalloc(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, 1, 1,
                         (int)attn_bwd_noalloc_max_rows() + 1, 64, sc, 1, 0) == MIATTN_ERR_TOO_LARGE);
  CHECK(attn_bwd_noalloc(q.p, k.p, v.p, o.p, nullptr, g.p, dq.p, dk.p, dv.p, B, H, N, d, sc, 1, 0) ==
        MIATTN_ERR_INVALID_ARG);
  CHECK(g_launches == before);

  // ---- valid calls: launched once per stage, workspace carved inside its buffer
  CHECK(attn_fwd(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, N, d, sc, 1, 0) == MIATTN_OK);
  CHECK(g_last.q == q.p && g_last.B == B && g_last.N == N && g_last.Hkv == H);
  CHECK(std::fabs(g_last.scale_log2 - sc * 1.4426950408889634f) < 1e-6f);
  {
    Buf ws(ws_need);
    const int n0 = g_launches;
    CHECK(attn_bwd(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, B, H, N, d, sc, 1, ws.p, ws_need,
                   0) == MIATTN_OK);
    CHECK(g_launches == n0 + 2);
    CHECK(inside(g_last.dvec, ws, R) && g_last.dq_writes_d == 1);
  }
  {
    const int nnz = 9;
    std::vector<int> rp = {0, 3, 6, 9};
    std::vector<int> ci = {0, 1, 2, 0, 1, 2, 0, 1, 2};
    const size_t wsb = attn_bwd_block_sparse_workspace_bytes(B, H, 2, N, d, nnz);
    CHECK(wsb > ws_need);
    Buf ws(wsb);
    CHECK(attn_bwd_block_sparse(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, B, H, 2, N, d, sc, 0,
                                rp.data(), ci.data(), nnz, ws.p, wsb, 0) == MIATTN_OK);
    CHECK(inside(g_last.dvec, ws, R) && inside(g_last.blk_table, ws, 9) && inside(g_last.blk_part, ws, 4));
    CHECK(attn_bwd_block_sparse(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, B, H, 2, N, d, sc, 0,
                                rp.data(), ci.data(), nnz, ws.p, wsb - 1, 0) == MIATTN_ERR_INVALID_ARG);
  }
  {
    const size_t wsb = attn_decode_workspace_bytes(B, H, 2, 40000, d);
    CHECK(wsb > 0);
    Buf ws(wsb);
    CHECK(attn_decode(q.p, k.p, v.p, o.p, (float*)lse.p, B, H, 2, 40000, d, sc, nullptr, ws.p, wsb, 0) == MIATTN_OK);
    const auto& a = miattn::g_dec;
    CHECK(a.nsplit >= 1 && (int64_t)a.nsplit * a.chunk >= 40000 && a.chunk % 64 == 0);
    CHECK(inside(a.part_ml, ws, (size_t)B * H * a.nsplit * 8) && inside(a.part_o, ws, (size_t)B * H * a.nsplit * d * 4));
  }
  {
    const size_t wsb = attn_bwd_varlen_workspace_bytes(300, H, d);
    Buf ws(wsb);
    CHECK(attn_bwd_varlen(q.p, k.p, v.p, o.p, (float*)lse.p, g.p, dq.p, dk.p, dv.p, cu_host, 2, 200, 300, H, d, sc,
                          1, nullptr, ws.p, wsb, 0) == MIATTN_OK);
    CHECK(g_last.total_tokens == 300 && g_last.B == 2 && g_last.N == 200 && inside(g_last.dvec, ws, 300 * H * 4));
  }
  {
    const size_t wsb = attn_bwd_f32_workspace_bytes(B, H, N, 64);
    Buf ws(wsb);
    CHECK(attn_bwd_f32((float*)q.p, (float*)k.p, (float*)v.p, (float*)o.p, (float*)lse.p, (float*)g.p, (float*)dq.p,
                       (float*)dk.p, (float*)dv.p, B, H, N, 64, sc, 0, ws.p, wsb, 0) == MIATTN_OK);
    CHECK(inside(g_last.dvec, ws, R) && inside(g_last.dq_acc, ws, (size_t)B * H * N * 64 * 4));
  }
  for (int st : {MIATTN_OK, MIATTN_ERR_INVALID_ARG, MIATTN_ERR_UNSUPPORTED, MIATTN_ERR_HIP, MIATTN_ERR_TOO_LARGE, 12345})
    CHECK(miattn_status_string(st) != nullptr && std::strlen(miattn_status_string(st)) > 0);

  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("abi host checks passed (%d stub launches)\n", g_launches);
  return 0;
}
