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
// Largest M for the weight-streaming MFMA kernel (gemm_skinny.hip); larger M
// uses the tiled MFMA kernel.
constexpr int kMaxSkinnyM = 128;

// One linear of a streaming launch (single call, or one descriptor of a
// chain workspace, filled from spec_linear / spec_linear_w8).
struct StreamLinear {
  const uint16_t* x;
  const void* w;         // bf16 [N][K], or FP8 E4M3 codes [N][K]
  const float* w_scale;  // FP8 weights: scale of each output row; bf16: unused
  void* y;
  int K;         // d_in
  int N;         // d_out
  int out_bf16;  // SPEC_BF16 (1) or SPEC_F32 (0)
  int reserved;
};
static_assert(sizeof(StreamLinear) == 48, "descriptor layout");

// Header of a chain workspace; followed by `n` per-linear arrival counters
// (unsigned) and then the n descriptors (StreamLinear, 64-byte aligned).
struct ChainSync {
  unsigned gen;         // launches completed
  unsigned exit_count;  // workgroups that left, cumulative
  unsigned error;       // bit 0: a barrier wait gave up; bit 1: plan mismatch
  unsigned magic;
  int n;                // linears in the plan
  int M;                // rows of every x
  int grid;             // workgroups per launch (fixed by the device and M)
  int spin_limit;       // polls before a barrier wait gives up
  unsigned long long* trace;  // per-linear timestamps (diagnostic builds only; else null)
  int pad[6];           // header is one 64-byte line
};
static_assert(sizeof(ChainSync) == 64, "chain header is one cache line");
constexpr unsigned kChainMagic = 0x53504348u;    // "SPCH": bf16 weights
constexpr unsigned kChainMagicW8 = 0x53503848u;  // "SP8H": FP8 E4M3 weights
// Polls of a release flag (each followed by an s_sleep of about 256 clocks)
// before a barrier wait gives up and sets error bit 0: well under a second.
constexpr int kChainSpinLimit = 1 << 18;
// Chain workspace after the header: n arrival counters, then (64-byte
// aligned) per linear kReleaseLanes release flags and kArriveGroups group
// arrival counters, one 64-byte line each, then the descriptors.
constexpr int kReleaseLanes = 8;
constexpr int kArriveGroups = 8;
constexpr int kBarrierLines = kReleaseLanes + kArriveGroups;  // per linear
__host__ __device__ inline size_t chain_release_offset(int n) {  // in unsigned words from counts
  return (((size_t)n * 4 + 63) & ~(size_t)63) / 4;
}
__host__ __device__ inline size_t chain_counts_bytes(int n) {
  return chain_release_offset(n) * 4 + (size_t)n * kBarrierLines * 64;
}

// Softmax statistics of a logits linear, fused into the streaming kernel's
// epilogue: every workgroup folds the outputs of its row blocks into a
// running (max, sum of exp((l - max) * inv)) per output position -- or, for
// a greedy row, the first index of the maximum -- and writes one partial per
// position. Row m's partials are at [m * stride, m * stride + grid); a
// workgroup without row blocks writes (-inf, 0, INT_MAX).
struct LogitStats {
  float* pmax;    // nullptr: no statistics
  double* psum;
  int32_t* parg;
  double inv;     // inverse temperature (unused when greedy)
  int greedy;
  int stride;     // partials per position; at least the grid
};
// Most workgroups a fused-statistics launch may use (partials per position).
constexpr int kMaxStatParts = 1024;

size_t stream_rows_per_block(int M);
int stream_max_wgs_per_cu(int M, bool w8);
// Streaming kernel, one linear: bf16 weights (w_scale null) or FP8 E4M3
// weights with per-row scales (w8).
// `stats` (nullable): fused softmax statistics of y (fp32 y only).
hipError_t launch_gemm_stream(const uint16_t* x, const void* w, const float* w_scale, void* y,
                              bool out_bf16, bool w8, int M, int K, int N, int grid,
                              hipStream_t s, const LogitStats* stats = nullptr);
hipError_t launch_gemm_chain(const StreamLinear* chain, int n_lin, ChainSync* sync, int M, bool w8,
                             int grid, hipStream_t s);
hipError_t launch_gemm_skinny(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                              int K, int N, hipStream_t s);
hipError_t launch_gemm_mfma(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                            int K, int N, hipStream_t s);
// FP8 E4M3 weights with per-row scales on the tile kernel (K a multiple of
// 64; any M, used above kMaxStreamM).
// The per-linear tile kernel with its reduction split over workgroups into a
// caller workspace of gemm_split_workspace_bytes(M, K, N) bytes (0: the
// plan does not split, and launch_gemm_split runs launch_gemm_mfma).
size_t gemm_split_workspace_bytes(int M, int K, int N);
hipError_t launch_gemm_split(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M,
                             int K, int N, void* workspace, size_t workspace_bytes, hipStream_t s);
// The FP8 tile kernel with a split reduction (as launch_gemm_split).
size_t gemm_split_workspace_bytes_w8(int M, int K, int N);
hipError_t launch_gemm_split_w8(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                                bool out_bf16, int M, int K, int N, void* workspace,
                                size_t workspace_bytes, hipStream_t s);
hipError_t launch_gemm_tile_w8(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                               bool out_bf16, int M, int K, int N, hipStream_t s);

// Verify attention (attention.hip): head dimension 128, (K+1) * H / Hkv <= 32
// query rows per key/value head. The split count depends only on the shape;
// the workspace holds the split partials (0 bytes when there is one split).
int attention_splits(int B, int K1, int H, int Hkv, int T);
size_t attention_workspace_bytes(int B, int K1, int H, int Hkv, int n_split);
hipError_t launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   void* out, bool out_bf16, int B, int K1, int T, int H, int Hkv,
                                   float scale, void* workspace, hipStream_t s);

hipError_t launch_softmax_rows(const float* logits, int rows, int V, float* probs, float* row_max,
                               float* row_sumexp, hipStream_t s);
hipError_t launch_accept_probs(const float* p, const float* q, const int32_t* tokens,
                               const float* u_accept, int B, int K, int V, int32_t* n_accepted,
                               uint8_t* mask, hipStream_t s);
hipError_t launch_sample_probs(const float* p, const float* q, const int32_t* n_accepted,
                               const float* u_sample, int B, int K, int V, int32_t* token,
                               uint8_t* zero_residual, hipStream_t s);

// Probe kernels (probe.hip): the achievable HBM read bandwidth and dense
// bf16 MFMA rate. launch_probe_mfma's FLOPs per launch are
// grid * 4 waves * iters * 131072 (8 chains of 16x16x32 or 4 of 32x32x16).
hipError_t launch_probe_read(const void* buf, size_t bytes, int loads, unsigned* sink, int grid,
                             hipStream_t s);
hipError_t launch_probe_read_lds(const void* buf, size_t bytes, int loads, unsigned* sink,
                                 int grid, hipStream_t s);
hipError_t launch_probe_mfma(int shape, int iters, unsigned* sink, int grid, hipStream_t s);

// Fused sampling stage of spec_verify (logits in, tokens out).
size_t verify_workspace_bytes(int B, int K, int V);
// t_target, t_draft: temperatures (> 0), or 0 for greedy (one-hot at the
// row's first maximum).
// `target_stats` (nullable): the target rows' statistics were written by
// the lm-head launch (target_stats_slot), so only the draft rows are scanned
// for theirs; `parts` partials per target row.
hipError_t launch_verify_sampling(const float* target_logits, const float* draft_logits,
                                  const int32_t* tokens, const float* u_accept,
                                  const float* u_sample, int B, int K, int V, int32_t* out_tokens,
                                  int32_t* n_emitted, void* workspace, float t_target,
                                  float t_draft, hipStream_t s,
                                  const LogitStats* target_stats = nullptr, int parts = 0);
// Where the lm-head launch of spec_verify writes the target rows' fused
// statistics inside its workspace; pmax is nullptr when B * (K + 1) exceeds
// the streaming kernel's positions.
LogitStats target_stats_slot(void* workspace, int B, int K, int V, float t_target);

}  // namespace specv
