// Kernel launchers used by the C-ABI layer (internal to libmiattn).
#pragma once
#include <hip/hip_runtime.h>

namespace miattn {
struct AttnArgs;

hipError_t launch_fwd_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);
hipError_t launch_fwd_w4_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);
hipError_t launch_bwd_prep_bf16(const AttnArgs& a, int d, bool varlen, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const AttnArgs& a, int d, bool causal, bool varlen, hipStream_t stream);

hipError_t launch_fwd_f32(const AttnArgs& a, int d, bool causal, hipStream_t stream);
hipError_t launch_bwd_f32(const AttnArgs& a, int d, bool causal, hipStream_t stream);
}  // namespace miattn
