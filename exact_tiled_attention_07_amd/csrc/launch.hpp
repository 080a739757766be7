// Host-side launchers of the attention kernels (called by the C ABI layer
// after it has validated every argument).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace fa {

// Forward, fp16/bf16 with D in {64, 128}: MFMA kernel.
hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t stream);
// Stages of the backward pass, as a bit mask: the row statistics (D_i and the
// base-2 LSE) into the workspace, then dK/dV and dQ, which both read it and
// are independent of each other.
constexpr int kStagePrepare = 1;
constexpr int kStageDkdv = 2;
constexpr int kStageDq = 4;
constexpr int kStageAll = kStagePrepare | kStageDkdv | kStageDq;

// Backward, fp16/bf16 with D in {64, 128}: D_i preprocess, dK/dV and dQ kernels.
hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t stream, int stages);
// Forward and backward, fp32 with D <= 128 (D % 4 == 0): vector-ALU kernels.
hipError_t launch_fwd_f32(const AttnArgs& a, hipStream_t stream);
hipError_t launch_bwd_f32(const AttnArgs& a, hipStream_t stream, int stages);
// Attention against a KV cache (append, split key range, merge); fp16/bf16,
// D in {64, 128}.
hipError_t launch_kvcache(const KvArgs& k, hipStream_t stream);
// D_i = sum_c dout[i,c] * o[i,c] for every query row, any dtype.
hipError_t launch_bwd_preprocess(const AttnArgs& a, hipStream_t stream);

}  // namespace fa
