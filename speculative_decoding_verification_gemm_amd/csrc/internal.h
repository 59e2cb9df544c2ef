// Kernel launchers behind the C ABI. Arguments are validated by the caller
// (api.cpp); each launcher only queues work on `s` and returns the launch
// status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

// Largest number of verify positions handled by the vector-ALU streaming
// kernel; larger M uses the MFMA kernel.
constexpr int kMaxStreamM = 16;

hipError_t launch_gemm_stream(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                              int K, int N, hipStream_t s);
hipError_t launch_gemm_mfma(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                            int K, int N, hipStream_t s);

hipError_t launch_softmax_rows(const float* logits, int rows, int V, float* probs, float* row_max,
                               float* row_sumexp, hipStream_t s);
hipError_t launch_accept_probs(const float* p, const float* q, const int32_t* tokens,
                               const float* u_accept, int B, int K, int V, int32_t* n_accepted,
                               uint8_t* mask, hipStream_t s);
hipError_t launch_sample_probs(const float* p, const float* q, const int32_t* n_accepted,
                               const float* u_sample, int B, int K, int V, int32_t* token,
                               uint8_t* zero_residual, hipStream_t s);

// Fused sampling stage of spec_verify (logits in, tokens out).
size_t verify_workspace_bytes(int B, int K, int V);
hipError_t launch_verify_sampling(const float* target_logits, const float* draft_logits,
                                  const int32_t* tokens, const float* u_accept,
                                  const float* u_sample, int B, int K, int V, int32_t* out_tokens,
                                  int32_t* n_emitted, void* workspace, hipStream_t s);

}  // namespace specv
