// Kernel launchers used by the C-ABI layer (internal to libmiattn).
#pragma once
#include <hip/hip_runtime.h>

namespace miattn {
struct AttnArgs;
struct DecodeArgs;
struct Fp8Args;

hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);
hipError_t launch_bwd_prep_bf16(const AttnArgs& a, int d, bool varlen, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);

// mask: kMaskWindow (causal already folded into the window) or kMaskBlocks
hipError_t launch_fwd_masked_bf16(const AttnArgs& a, int d, int mask, bool causal, hipStream_t stream);
hipError_t launch_bwd_dkdv_masked_bf16(const AttnArgs& a, int d, int mask, bool causal, hipStream_t stream);
hipError_t launch_bwd_dq_masked_bf16(const AttnArgs& a, int d, int mask, bool causal, hipStream_t stream);
// expands the block-sparse CSR list into a.blk_table (n_qblk x n_kblk bytes)
hipError_t launch_block_table(const AttnArgs& a, uint8_t* table, hipStream_t stream);
// balanced work list of the block-sparse key-tile pass (needs the table) and
// the sums of the chunks of the key blocks it cut
hipError_t launch_block_work(const AttnArgs& a, bool causal, int* work, int* slot, int* nch, hipStream_t stream);
hipError_t launch_block_reduce(const AttnArgs& a, int d, hipStream_t stream);

// split pass then merge pass of decoding against a KV cache
hipError_t launch_decode_bf16(const DecodeArgs& a, int d, hipStream_t stream);

// FP8: quantizers (bf16 -> E4M3 codes + scales) and the forward, D = 128
hipError_t launch_quant_rows_fp8(const void* x, void* x8, float* scales, int BH, int N, int d, hipStream_t stream);
hipError_t launch_quant_vt_fp8(const void* v, void* v8t, float* scales, int BH, int N, int d, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8Args& a, int d, bool causal, hipStream_t stream);

hipError_t launch_fwd_f32(const AttnArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_f32(const AttnArgs& a, int d, bool causal, hipStream_t stream);
}  // namespace miattn
