/*
 * libmiattn -- fused exact attention for AMD MI355X (gfx950), C ABI.
 *
 * What it computes, per batch b and head h (or per packed sequence and head):
 *   S = scale * Q K^T, with masked entries -inf;  P = row-softmax(S);
 *   O = P V;  LSE_i = ln sum_j exp(S_ij)
 * ("Attention(Q,K,V) = softmax(QK^T/sqrt(d)) V" in the FlashAttention-1 notes
 * of BHHXX's Blog, section 1.1, and in "第 18 章 FlashAttention" section
 * 18.2.1; the log-sum-exp of "解析 FlashAttention（4）：FlashAttention-v2" at
 * the end of section 三 and in "分块 Attention：重建概率，累计梯度" section 04).
 * The forward never writes S or P to memory: it keeps the online-softmax
 * running state (row max m, row sum l, unnormalised output) per query tile
 * ("解析 FlashAttention（4）" section 四).  The backward rebuilds P from Q, K and
 * LSE and forms, with upstream gradient dO,
 *   D = rowsum(dO o O); dP = dO V^T; dS = P o (dP - D);
 *   dV = P^T dO; dQ = scale dS K; dK = scale dS^T Q
 * ("解析 FlashAttention（4）" section 五; "分块 Attention" section 04, which
 * also carries the 1/sqrt(d) factor of dQ and dK).
 *
 * Masks: causal keeps key j for query i iff j <= i ("第 18 章" section 18.2.2,
 * the causal mask M_ij = 0 for j <= i); in the packed interface no query sees
 * another sequence's keys and positions count from each sequence's start
 * ("第 18 章" section 18.7.1, the variable-length interface with cumulative
 * offsets); an optional key-padding mask hides keys from every query
 * ("第 18 章" section 18.2.2, padding masks).  A query row that sees no key at
 * all gets O = 0, LSE = -inf and contributes no gradient ("分块 Attention"
 * section 04, the all-masked-row convention).
 *
 * Layouts (row-major, contiguous):
 *   dense   Q, K, V, O, dO, dQ, dK, dV : [B, H, N, d]     LSE : [B, H, N] fp32
 *   packed  Q, K, V, O, dO, dQ, dK, dV : [T, H, d]        LSE : [H, T]    fp32
 *           cu_seqlens : int32 [nseq + 1], cu[0] = 0, non-decreasing,
 *                        cu[nseq] = T (total_tokens)
 *           key_valid  : uint8 [T], nonzero = the key may be attended
 * "bf16" entry points take bfloat16 tensors (raw 16-bit storage); the "_f32"
 * entry points take fp32 tensors.  LSE and every accumulation are fp32.
 *
 * Ownership and streams: every pointer is a device pointer owned by the
 * caller, including the workspace.  The library allocates nothing, frees
 * nothing, never synchronises and keeps no global state; all work is queued
 * on `stream` (0 = the default stream).  Results are valid once the stream
 * has reached the enqueued work.
 *
 * Errors: entry points return MIATTN_OK (0) or a negative status, checked in
 * this order before anything is launched:
 *   MIATTN_ERR_INVALID_ARG  a required pointer is NULL or not 16-byte aligned
 *                           (cu_seqlens: 4-byte), a size is <= 0, scale is
 *                           not finite, the workspace is too small, or the
 *                           problem's grid would not fit a launch;
 *   MIATTN_ERR_UNSUPPORTED  head dim d is not 64 or 128;
 *   MIATTN_ERR_HIP          a kernel launch was rejected by the runtime.
 * The contents of cu_seqlens and key_valid live on the device and are not
 * checked on the host (the binding's check_cu_seqlens checks a host copy);
 * the kernels clamp offsets into [0, total_tokens] and lengths to
 * max_seqlen, so offsets that break the contract above give unspecified
 * results but never address memory outside the tensors.
 *
 * Non-finite inputs are ordinary inputs: a NaN or Inf in Q, K, V or dO makes
 * NaN of what depends on it and never faults.  A query row whose scores hold
 * a NaN or an Inf gets NaN in its O and LSE (other rows are unaffected).  In
 * the backward, masked pairs enter the matrix products as exact zeros and
 * 0 * Inf = NaN, so a non-finite query row also turns NaN the dK, dV of the
 * keys that share a backward tile (at most 128 keys) with it.
 * Calls that overlap on one stream are ordered; calls on different streams
 * that share output or workspace buffers race.
 */
#ifndef MIATTN_H
#define MIATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MIATTN_OK 0
#define MIATTN_ERR_INVALID_ARG (-1)
#define MIATTN_ERR_UNSUPPORTED (-2)
#define MIATTN_ERR_HIP (-3)
#define MIATTN_ERR_TOO_LARGE (-4)

/* Library version, major * 10000 + minor * 100 + patch. */
int miattn_version(void);

/* Static text for a status code (never NULL). */
const char* miattn_status_string(int status);

/* Forward, dense bf16.  q, k, v: [B,H,N,d] bf16 in; o: [B,H,N,d] bf16 out
 * (round-to-nearest-even); lse: [B,H,N] fp32 out (natural log, -inf for a row
 * with no visible key).  scale multiplies Q K^T (pass 1/sqrt(d) for the usual
 * attention); causal != 0 applies the causal mask.  Online-softmax forward of
 * "解析 FlashAttention（4）：FlashAttention-v2" section 四. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* Bytes of device workspace attn_bwd and its stages need: fp32 D [B,H,N]
 * (rounded up to 256 bytes).  Returns 0 for invalid sizes. */
size_t attn_bwd_workspace_bytes(int B, int H, int N, int d);

/* Bytes of device workspace attn_bwd_f32 needs: fp32 D [B,H,N] and an fp32
 * dQ accumulator [B,H,N,d].  Returns 0 for invalid sizes. */
size_t attn_bwd_f32_workspace_bytes(int B, int H, int N, int d);

/* Backward, dense bf16.  Inputs q, k, v, o (from attn_fwd), lse (from
 * attn_fwd), dO: upstream gradient [B,H,N,d] bf16.  Outputs dq, dk, dv:
 * [B,H,N,d] bf16 (fp32 accumulation, one final rounding).  workspace: at least
 * attn_bwd_workspace_bytes(B,H,N,d) bytes, 16-byte aligned, no initial
 * contents required; it is overwritten.  The LSE receives no gradient.
 * Runs attn_bwd_dq_preprocess, then attn_bwd_dkdv; the result equals, bit for
 * bit, attn_bwd_preprocess followed by attn_bwd_dkdv and attn_bwd_dq (the
 * last two independent of each other).  The result is bitwise reproducible:
 * no output is accumulated with atomics.
 * LSE-recompute backward of "解析 FlashAttention（4）" section 五. */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dO, void* dq, void* dk, void* dv,
             int B, int H, int N, int d, float scale, int causal,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Allocation-free form of attn_bwd, for callers that cannot allocate device
 * memory or pass a workspace (code under stream capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, kernels and
 * result (bit for bit) as attn_bwd without the workspace: D lives in a
 * scratch array built into the library, 32 MiB of device memory per GPU,
 * held from the library's load until the process ends.  Limit: B*H*N <=
 * attn_bwd_noalloc_max_rows() (8388608); larger problems return
 * MIATTN_ERR_TOO_LARGE before any launch.  Calls no allocating routine.  All
 * calls on one GPU share its scratch: calls that overlap on one GPU (other
 * streams, other host threads) race and must be serialised by the caller.
 * The first call on a device looks up the scratch's address on it (a HIP
 * error there returns MIATTN_ERR_HIP). */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dO, void* dq, void* dk, void* dv,
                     int B, int H, int N, int d, float scale, int causal, hipStream_t stream);
size_t attn_bwd_noalloc_max_rows(void);

/* The D pre-pass, stage 1 of the three-stage backward (attn_bwd itself forms
 * D inside its dQ pass, attn_bwd_dq_preprocess): D = rowsum(dO o O) in fp32
 * into the workspace ("解析 FlashAttention（4）" section 5.2). */
int attn_bwd_preprocess(const void* o, const void* dO, int B, int H, int N, int d,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The dK/dV stage of attn_bwd: the key-tile outer loop that rebuilds P and dS
 * and writes dk and dv ("解析 FlashAttention（4）" section 5.4).  Needs D in
 * the same workspace, from attn_bwd_preprocess or attn_bwd_dq_preprocess. */
int attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dO,
                  void* dk, void* dv, int B, int H, int N, int d, float scale, int causal,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The dQ stage of the three-stage backward: a query-tile outer loop that
 * rebuilds P and dS and writes dq = scale dS K ("解析 FlashAttention（4）"
 * sections 5.3-5.4, with the dQ sum taken per query tile instead of by atomic
 * adds).  Needs D in the same workspace (attn_bwd_preprocess). */
int attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dO, void* dq,
                int B, int H, int N, int d, float scale, int causal,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Stages 1 and 3 in one pass: the query-tile loop of attn_bwd_dq that first
 * forms D = rowsum(dO o O) of its own rows ("解析 FlashAttention（4）"
 * section 5.2), uses it and stores it in the workspace, bit for bit what
 * attn_bwd_preprocess stores; attn_bwd_dkdv may then run on the workspace.
 * Arguments as attn_bwd_dq plus o (from attn_fwd). */
int attn_bwd_dq_preprocess(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dO, void* dq, int B, int H, int N, int d, float scale, int causal,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward with grouped key/value heads (grouped-query attention; H_kv = 1 is
 * multi-query attention), dense bf16.  q, o: [B,H,N,d]; k, v: [B,H_kv,N,d];
 * lse: [B,H,N] fp32.  H_kv must divide H; query head h attends with key/value
 * head h / (H / H_kv).  Everything else as attn_fwd, which is the case
 * H_kv == H.  MQA and GQA are described in "第 18 章 FlashAttention" section
 * 18.2.2 (groups of query heads share one K/V head, loaded once and reused
 * across the group) and section 18.7.1 (an interface whose K/V carry fewer
 * heads than Q, broadcast when the query head count is a multiple of it).
 * MIATTN_ERR_INVALID_ARG also when H_kv <= 0 or H % H_kv != 0. */
int attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int H_kv, int N, int d, float scale, int causal, hipStream_t stream);

/* Backward with grouped key/value heads, dense bf16.  q, o, dO, dq:
 * [B,H,N,d]; k, v, dk, dv: [B,H_kv,N,d]; lse: [B,H,N].  dk and dv of a
 * key/value head are the sums over the H / H_kv query heads that read it
 * (taken in fp32 registers by one workgroup, no atomics; bitwise
 * reproducible).  workspace: attn_bwd_workspace_bytes(B,H,N,d) bytes. */
int attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dO, void* dq, void* dk, void* dv,
                 int B, int H, int H_kv, int N, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward with a sliding window, dense bf16, grouped key/value heads as in
 * attn_fwd_gqa (H_kv == H for plain multi-head attention).  Key j is visible
 * to query i iff i - window_left <= j <= i + window_right, a side given as -1
 * being unbounded; with causal != 0 the right side is 0 whatever
 * window_right says.  This is the window_size = (left, right) argument of the
 * flash-attn interface, (-1, -1) meaning global attention ("第 18 章
 * FlashAttention" section 18.7.1), the sliding-window pattern of section
 * 18.8.1 (Mistral, Longformer).  Key tiles wholly outside a query tile's
 * window are neither loaded nor computed.  A window that restricts nothing
 * runs exactly attn_fwd_gqa.  MIATTN_ERR_INVALID_ARG also for a side < -1. */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int H_kv, int N, int d, float scale, int causal,
                    int window_left, int window_right, hipStream_t stream);

/* Backward of attn_fwd_window; arguments as attn_bwd_gqa plus the window.
 * workspace: attn_bwd_workspace_bytes(B,H,N,d) bytes. */
int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv,
                    int B, int H, int H_kv, int N, int d, float scale, int causal,
                    int window_left, int window_right,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Block-sparse layout granularity: blocks of 128 query rows x 128 keys. */
#define MIATTN_SPARSE_BLOCK 128

/* Forward with a block-sparse layout, dense bf16, grouped key/value heads as
 * in attn_fwd_gqa.  Positions are cut into blocks of MIATTN_SPARSE_BLOCK
 * tokens, nb = ceil(N / MIATTN_SPARSE_BLOCK) of them (N <= 131072).  The
 * layout is a CSR list shared by every (batch, head), in device memory:
 * row_ptr int32 [nb + 1], col_idx int32 [nnz]; query block r attends the key
 * blocks col_idx[row_ptr[r] .. row_ptr[r+1]) ("第 18 章 FlashAttention"
 * section 18.8.1: a per-query-block list of the key blocks to compute, built
 * once per shape; the kernel loads only those blocks and the others add
 * nothing to the softmax).  A block listed twice counts once; entries outside
 * [0, nb) and positions past nnz are ignored (never read out of bounds); the
 * order within a row does not matter.  causal != 0 also applies the causal
 * mask.  A query row left with no key gets O = 0, LSE = -inf.
 * MIATTN_ERR_UNSUPPORTED when N > 131072. */
int attn_fwd_block_sparse(const void* q, const void* k, const void* v, void* o, float* lse,
                          int B, int H, int H_kv, int N, int d, float scale, int causal,
                          const int* row_ptr, const int* col_idx, int nnz, hipStream_t stream);

/* Workspace bytes for attn_bwd_block_sparse with a list of nnz entries: fp32
 * D (one per row), the list expanded to an nb x nb byte table, a balanced
 * work list and fp32 partial sums for key blocks that many query blocks list.
 * 0 for invalid sizes. */
size_t attn_bwd_block_sparse_workspace_bytes(int B, int H, int H_kv, int N, int d, int nnz);

/* Backward of attn_fwd_block_sparse; arguments as attn_bwd_gqa plus the
 * list.  The key-tile pass visits, for each key block, only the query blocks
 * that list it (read from the expanded table); a key block listed by more
 * query blocks than the average (such as a global block) is split
 * over several workgroups whose fp32 partial sums are then added in a fixed
 * order, so the result does not depend on scheduling.  dk, dv of a key block
 * no query block lists are 0. */
int attn_bwd_block_sparse(const void* q, const void* k, const void* v, const void* o, const float* lse,
                          const void* dO, void* dq, void* dk, void* dv,
                          int B, int H, int H_kv, int N, int d, float scale, int causal,
                          const int* row_ptr, const int* col_idx, int nnz,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for attn_decode (the pieces' running states); 0 for
 * invalid sizes. */
size_t attn_decode_workspace_bytes(int B, int H, int H_kv, int N_kv, int d);

/* Decoding attention, bf16: one new query token per sequence against a KV
 * cache ("第 18 章 FlashAttention" section 18.8.2, the decoding phase with
 * Q: [b, 1, d], and FlashDecoding).  q, o: [B,H,d]; k_cache, v_cache:
 * [B,H_kv,N_kv,d]; lse: [B,H] fp32.  Query head h of sequence b attends keys
 * 0 .. len_b - 1 of key/value head h / (H / H_kv), with len_b =
 * cache_seqlens[b] (device int32 [B], clamped to [0, N_kv]) or N_kv when
 * cache_seqlens is NULL; no other mask (the cached positions all precede the
 * new token, whose own K/V the caller has appended).  The cache is cut into
 * pieces processed in parallel, each keeping its own running max, sum and
 * unnormalised output, merged at the end with the online-softmax rule
 * (section 18.8.2, step 3).  A sequence with len_b = 0 gets O = 0, LSE = -inf.
 * workspace: attn_decode_workspace_bytes(B,H,H_kv,N_kv,d) bytes. */
int attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                int B, int H, int H_kv, int N_kv, int d, float scale, const int* cache_seqlens,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* FP8 (E4M3) attention ("第 18 章 FlashAttention" section 18.6.2: Q, K, V
 * converted to FP8 E4M3 with dynamic per-block scales s = max|X_block| / 448
 * for the load blocks of Q and K; S = QK^T and the softmax in fp32; O
 * dequantized).  Head dimension 128 only (MIATTN_ERR_UNSUPPORTED otherwise).
 * Codes are OCP E4M3FN (bias 7, largest magnitude 448), rounded to nearest
 * even; an all-zero block gets scale 1.
 *
 * attn_quantize_fp8_rows: x bf16 [B,H,N,128] -> x8 codes [B,H,N,128] and
 * scales fp32 [B,H,ceil(N/64)], one per block of 64 rows (for Q and for K).
 *
 * attn_quantize_fp8_vt: v bf16 [B,H,N,128] -> scales fp32 [B,H] (one per
 * head) and v8t codes [B,H,ceil(N/64),128,64]: tile t, feature f, position p
 * holds key 64t + k(p), k(p) = 32 (p%32/16) + 8 (p%16/4) + 4 (p/32) + p%4,
 * keys past N coded 0 (the order in which the forward's score accumulators
 * hold a tile's keys).  Queues three kernels: per-tile maxima (kept in v8t
 * until the codes overwrite them), the per-head scale, the codes. */
int attn_quantize_fp8_rows(const void* x, unsigned char* x8, float* scales, int B, int H, int N, int d,
                           hipStream_t stream);
int attn_quantize_fp8_vt(const void* v, unsigned char* v8t, float* scales, int B, int H, int N, int d,
                         hipStream_t stream);

/* FP8 forward, grouped key/value heads as attn_fwd_gqa: q8, q_scale from
 * attn_quantize_fp8_rows of Q [B,H,N,128]; k8, k_scale of K [B,H_kv,N,128];
 * v8t, v_scale from attn_quantize_fp8_vt of V [B,H_kv,N,128].  o bf16
 * [B,H,N,128], lse fp32 [B,H,N].  The P V product uses P multiplied by 2^6
 * and rounded to E4M3 (so every P >= 2^-12 is a normal E4M3 value), the 2^6
 * taken out again with 1/l; so O differs from exact attention on the
 * dequantized inputs by at most about 2^-4 sum_j P_ij |V_j| per element.
 * Scores come from FP8 matrix instructions whose accumulation of a score's
 * 128 products errs by at most 2^-13 of the sum of their magnitudes
 * (measured through single-key rows, where LSE is the score); LSE is that of
 * these fp32 scores.  Fully masked rows and errors as attn_fwd. */
int attn_fwd_fp8(const unsigned char* q8, const float* q_scale, const unsigned char* k8, const float* k_scale,
                 const unsigned char* v8t, const float* v_scale, void* o, float* lse,
                 int B, int H, int H_kv, int N, int d, float scale, int causal, hipStream_t stream);

/* fp32 forward: same contract as attn_fwd with fp32 q, k, v, o. */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int H, int N, int d, float scale, int causal, hipStream_t stream);

/* fp32 backward: same contract as attn_bwd with fp32 tensors; workspace size
 * from attn_bwd_f32_workspace_bytes.  dq is accumulated with float atomics
 * across key tiles, so it may differ in the last bits from run to run. */
int attn_bwd_f32(const float* q, const float* k, const float* v, const float* o, const float* lse,
                 const float* dO, float* dq, float* dk, float* dv,
                 int B, int H, int N, int d, float scale, int causal,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Forward over packed variable-length sequences, bf16.  q, k, v, o: [T,H,d];
 * lse: [H,T] fp32.  cu_seqlens: device int32 [nseq+1]; max_seqlen: the
 * longest sequence (rows past it are not computed); total_tokens: T.
 * key_valid: device uint8 [T] or NULL (all keys valid). */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int* cu_seqlens, int nseq, int max_seqlen, int total_tokens,
                    int H, int d, float scale, int causal, const unsigned char* key_valid,
                    hipStream_t stream);

/* Workspace bytes for attn_bwd_varlen: fp32 D [H,T]. */
size_t attn_bwd_varlen_workspace_bytes(int total_tokens, int H, int d);

/* Backward over packed variable-length sequences, bf16; arguments as in
 * attn_fwd_varlen plus those of attn_bwd. */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dO, void* dq, void* dk, void* dv,
                    const int* cu_seqlens, int nseq, int max_seqlen, int total_tokens,
                    int H, int d, float scale, int causal, const unsigned char* key_valid,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MIATTN_H */
