/*
 * spec_verify.h -- C ABI of libspecverify.so: the verification step of
 * speculative decoding on one AMD Instinct MI355X (gfx950).
 *
 * One verify step of speculative decoding feeds K+1 positions per sequence
 * (the last accepted token plus K draft tokens) through the target's linear
 * layers in a single read of the weights, then runs speculative sampling at
 * every position: softmax the target logits p and the draft logits q, accept
 * draft token x with probability min(1, p(x)/q(x)), stop at the first
 * rejection and resample there from norm(max(0, p - q)), or draw a bonus
 * token from p_{K+1} if every draft survived ("Speculative Decoding: Two
 * Models, One Voice", The idea, steps 1-3; "Speculative Decoding: Guess
 * Several Tokens, Check Them in One Pass", Steps 1-3).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every data pointer is a DEVICE pointer to row-major, contiguous memory
 *   owned by the caller. The library allocates no memory, keeps no state
 *   beyond a per-device property cache and a thread-local error string, and
 *   never synchronizes: work is queued on `stream` (a hipStream_t; NULL is
 *   the null stream) and outputs are valid once the caller has synchronized
 *   that stream. Every call can be captured into a HIP graph.
 * - bf16 data are passed as uint16_t bit patterns (IEEE bfloat16).
 * - Rows and indices: B sequences, K draft tokens (1 <= K <= 64), V the
 *   vocabulary. Target rows are [B][K+1][V]: row j of sequence b is the
 *   target's distribution for the slot after the last accepted token and the
 *   drafts x_1..x_j. Draft rows are [B][K][V]: row j is q_{j+1}, the
 *   distribution draft token x_{j+1} was drawn from.
 * - Randomness is supplied by the caller as uniforms in [0, 1):
 *   u_accept[b][j] drives the accept test of draft j; u_sample[b][j] drives
 *   the sample that ends the round at row j (j = number of accepted drafts),
 *   and is the only sample uniform consumed per sequence.
 * - Arguments are validated on the host before any HIP call; a failing call
 *   launches nothing. Device data are not validated on the host: a draft
 *   token outside [0, V) is treated as rejected (it cannot have been
 *   proposed), an n_accepted outside [0, K] yields token -1, and a row with
 *   no positive weight yields token -1. Device faults surface at the
 *   caller's synchronize. No C++ exception crosses this ABI.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 8

/* Status codes. */
#define SPEC_OK 0
#define SPEC_ERR_INVALID_ARGUMENT (-1) /* null required pointer, bad size or enum */
#define SPEC_ERR_ALIGNMENT (-2)        /* a pointer lacks the required alignment */
#define SPEC_ERR_UNSUPPORTED (-3)      /* current device is not gfx950 */
#define SPEC_ERR_WORKSPACE (-4)        /* workspace too small or misaligned */
#define SPEC_ERR_HIP (-5)              /* HIP runtime error; see spec_last_error() */

/* Output element types of spec_verify_gemm. */
#define SPEC_F32 0
#define SPEC_BF16 1

/* ABI version of the loaded library (SPEC_ABI_VERSION at build time). */
int spec_abi_version(void);

/* Static, human-readable name of a status code. */
const char* spec_status_string(int status);

/* Message of the last failing call made by this thread ("" if none). The
 * pointer stays valid until the thread's next library call. */
const char* spec_last_error(void);

/*
 * spec_verify_gemm -- one linear layer of the verify pass.
 *
 * y[M][d_out] = x[M][d_in] . w[d_out][d_in]^T with bf16 products and fp32
 * accumulation, reading w exactly once for all M = B*(K+1) rows
 * ("What Actually Happens During Speculative Decoding in LLMs": the weights
 * are loaded once and multiplied by a [5 x d] matrix instead of a [1 x d]
 * vector; "Speculative Decoding: Guess Several Tokens", Step 1).
 *
 *   x      bf16 [M][d_in], 16-byte aligned.
 *   w      bf16 [d_out][d_in] (nn.Linear layout), 16-byte aligned.
 *   y      [M][d_out], fp32 (y_dtype = SPEC_F32, 4-byte aligned) or bf16
 *          rounded to nearest even (SPEC_BF16, 2-byte aligned).
 *   Limits: 1 <= M <= 65536, 8 <= d_in <= 2^20 with d_in % 8 == 0,
 *   1 <= d_out <= 2^24.
 * Few rows on a large linear (M <= 8 with at least 2^26 weights, or
 * M <= 16 when d_in is not a multiple of 64) run a vector-ALU
 * weight-streaming kernel; every other shape runs a bf16 MFMA kernel (the
 * crossovers were measured on MI355X). Deterministic: the same inputs give
 * bitwise identical outputs.
 */
int spec_verify_gemm(const uint16_t* x, const uint16_t* w, void* y, int y_dtype,
                     int M, int d_in, int d_out, void* stream);

/*
 * spec_verify_gemm_workspace_bytes -- device workspace spec_verify_gemm_ws
 * needs for this shape, or 0 when it does not split the reduction there (or
 * the sizes are out of range). Depends on the shape only, not on the device;
 * no device call.
 */
size_t spec_verify_gemm_workspace_bytes(int M, int d_in, int d_out);

/*
 * spec_verify_gemm_ws -- spec_verify_gemm with the reduction over d_in
 * split across workgroups where a time model fitted on MI355X predicts
 * that to be faster: the same product y = x . w^T as spec_verify_gemm
 * ("What Actually Happens During Speculative Decoding in LLMs": the
 * weights are read once for all M positions), for shapes whose tiles alone
 * would leave compute units idle over a long reduction (a down projection,
 * d_in = 14336 into 4096, at M = 5 to 1280; measured 0.64 to 1.00 of the
 * unsplit time on the Llama-3.1-8B and 70B linears where it splits).
 *
 *   x, w, y, y_dtype, M, d_in, d_out  as for spec_verify_gemm.
 *   workspace        device memory of at least
 *                    spec_verify_gemm_workspace_bytes(M, d_in, d_out) bytes,
 *                    16-byte aligned, owned by the caller; may be NULL when
 *                    that size is 0. Overwritten: S fp32 partial outputs
 *                    [S][M][d_out], S the number of splits.
 *   workspace_bytes  its size in bytes.
 * When the size is 0 the call is exactly spec_verify_gemm. Otherwise two
 * kernels run on `stream`: the tile kernel writes each split's fp32 partial
 * sums, and a second kernel adds them in split order and rounds once, so
 * the result is deterministic (bitwise equal across launches), though its
 * fp32 rounding differs from spec_verify_gemm's single accumulator. Calls
 * sharing one workspace must be ordered on one stream.
 * Errors: as spec_verify_gemm; SPEC_ERR_WORKSPACE (before any device call)
 * if the workspace is NULL, smaller than needed or misaligned.
 */
int spec_verify_gemm_ws(const uint16_t* x, const uint16_t* w, void* y, int y_dtype,
                        int M, int d_in, int d_out, void* workspace,
                        size_t workspace_bytes, void* stream);

/*
 * spec_linear -- one linear of a chain (see spec_chain_prepare).
 *   x        bf16 [M][d_in], 16-byte aligned (read only after the previous
 *            linear of the chain has completed, so it may be that linear's y).
 *   w        bf16 [d_out][d_in], 16-byte aligned.
 *   y        [M][d_out], fp32 or bf16 as y_dtype says.
 *   d_in, d_out, y_dtype  as for spec_verify_gemm; reserved must be 0.
 */
typedef struct spec_linear {
  const uint16_t* x;
  const uint16_t* w;
  void* y;
  int32_t d_in;
  int32_t d_out;
  int32_t y_dtype;
  int32_t reserved;
} spec_linear;

/* Bytes of chain workspace for n linears; 0 if n is out of range. */
size_t spec_chain_workspace_bytes(int n);

/*
 * spec_chain_prepare -- validate a chain of n linears over the same M rows
 * and record it in `workspace` (device memory, 256-byte aligned, at least
 * spec_chain_workspace_bytes(n) bytes, owned by the caller and not used for
 * anything else while the chain is in use).
 *
 * `linears` is a HOST array; every descriptor is checked as spec_verify_gemm
 * checks its arguments. The call is synchronous (it copies the descriptors
 * to the device and resets the workspace's counters) and must not be
 * captured in a graph. 1 <= n <= 4096, 1 <= M <= 16 (the weight-streaming
 * regime).
 */
int spec_chain_prepare(const spec_linear* linears, int n, int M, void* workspace,
                       size_t workspace_bytes);

/*
 * spec_verify_gemm_chain -- run a prepared chain in one launch.
 *
 * Computes every linear of the chain in order, each exactly as
 * spec_verify_gemm would, in ONE pass that streams all weights: the K+1
 * verify positions cross the whole linear stack with a single read of every
 * weight ("What Actually Happens During Speculative Decoding in LLMs": the
 * weights are loaded once for all candidate positions). Linear i+1 reads its
 * x only after linear i's y is complete and visible (device-scope
 * release/acquire), as the next layer of a forward pass would; weight loads
 * of linear i+1, which depend on nothing, start before that point. n and M
 * must be those given to spec_chain_prepare (checked on the device: a
 * mismatch computes nothing and sets bit 1 of spec_chain_error). The call
 * is asynchronous and capturable; launches that use the same workspace must
 * be ordered (same stream).
 *
 * Precondition: the launch is one persistent workgroup per compute unit
 * (more where occupancy allows), and its barriers assume that all of them
 * are resident at once. A launch that shares the GPU with other work that
 * keeps compute units occupied for long may find some workgroups not yet
 * started; the waiting ones then give up after a bounded number of polls
 * (well under a second) instead of hanging, finish the launch, and set bit
 * 0 of spec_chain_error; the outputs of that launch are then not valid, and
 * spec_chain_reset brings the workspace back to a consistent state. The
 * call itself returns SPEC_OK in that case (the failure happens on the
 * device, after the call has returned): callers that cannot rule out such
 * sharing should read spec_chain_error after synchronizing.
 */
int spec_verify_gemm_chain(int n, int M, void* workspace, void* stream);

/*
 * Weight-only 8-bit storage (FP8 weights, bf16 activations and compute):
 * half the bytes per weight, so the weight-streaming verify pass moves half
 * as much and its FLOPs per byte double ("Speculative Decoding: The Algebra
 * and the Proof", Where it breaks). Each weight is an FP8 E4M3 code (OCP
 * 8-bit floating point: 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; 0x7F and 0xFF are NaN; largest finite 448), and each
 * output row n has one float32 scale:
 *
 *   y[m][n] = w_scale[n] * sum_k x[m][k] * e4m3(w[n][k])
 *
 * E4M3 values are exact in bf16, products are exact in fp32, and the sum is
 * accumulated in fp32 like spec_verify_gemm's; the scale multiplies the sum.
 *
 * spec_verify_gemm_w8 -- one linear.
 *   x        device, bf16 [M][d_in], 16-byte aligned.
 *   w        device, uint8 E4M3 codes [d_out][d_in], 16-byte aligned.
 *   w_scale  device, float32 [d_out], 4-byte aligned.
 *   y        device, [M][d_out] of y_dtype.
 *   d_in     multiple of 16, in [16, 2^20]; d_out in [1, 2^24].
 *   M        1..65536. Up to 16 positions a vector-ALU weight-streaming
 *            kernel runs (the regime where halving the bytes halves the
 *            time); above, the bf16 MFMA tile kernel with the codes widened
 *            exactly to bf16 on their way to the matrix cores, which needs
 *            d_in a multiple of 64 (else SPEC_ERR_UNSUPPORTED). There 8-bit
 *            weights double the FLOPs per weight byte, which halves the
 *            batch at which the pass stops being bound by the weight read
 *            (same page).
 * Errors as spec_verify_gemm. Nothing is allocated; the call is
 * asynchronous on `stream`.
 */
int spec_verify_gemm_w8(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                        int y_dtype, int M, int d_in, int d_out, void* stream);

/*
 * spec_verify_gemm_w8_workspace_bytes -- as spec_verify_gemm_workspace_bytes
 * for spec_verify_gemm_w8_ws (0: no split; always 0 at M <= 16).
 */
size_t spec_verify_gemm_w8_workspace_bytes(int M, int d_in, int d_out);

/*
 * spec_verify_gemm_w8_ws -- spec_verify_gemm_w8 with the reduction split
 * over workgroups where a time model fitted on MI355X predicts that to be
 * faster (M above 16; measured 0.42 to 0.99 of the unsplit time on the
 * Llama-3.1-8B and 70B linears where it splits, the down projections most).
 * Arguments as spec_verify_gemm_w8, plus `workspace` / `workspace_bytes`
 * as for spec_verify_gemm_ws. The fp32 partial sums are unscaled; the
 * second kernel adds them in split order, multiplies by w_scale[n] and
 * rounds once. Deterministic; errors as spec_verify_gemm_w8, and
 * SPEC_ERR_WORKSPACE as spec_verify_gemm_ws.
 */
int spec_verify_gemm_w8_ws(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                           int y_dtype, int M, int d_in, int d_out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* One linear of an FP8-weight chain: spec_linear with w_scale. */
typedef struct spec_linear_w8 {
  const uint16_t* x;
  const uint8_t* w;
  const float* w_scale;
  void* y;
  int32_t d_in;
  int32_t d_out;
  int32_t y_dtype;
  int32_t reserved;
} spec_linear_w8;

/*
 * spec_chain_prepare_w8 / spec_verify_gemm_chain_w8 -- spec_chain_prepare
 * and spec_verify_gemm_chain for a chain whose every linear has FP8 E4M3
 * weights (each checked as spec_verify_gemm_w8 checks its arguments). The
 * workspace is sized by spec_chain_workspace_bytes(n) as for a bf16 chain,
 * and M is limited to 16 as for a bf16 chain; a
 * workspace prepared by one kind of prepare call run by the other kind of
 * chain call computes nothing and sets bit 1 of spec_chain_error.
 */
int spec_chain_prepare_w8(const spec_linear_w8* linears, int n, int M, void* workspace,
                          size_t workspace_bytes);
int spec_verify_gemm_chain_w8(int n, int M, void* workspace, void* stream);

/*
 * spec_verify_attention -- the attention of the verify pass: the K+1 verify
 * positions of each sequence attend, through the causal mask, over that
 * sequence's KV cache, which is read once for all of them ("Speculative
 * Decoding: Guess Several Tokens, Check Them in One Pass", Step 1: the pass
 * works like a tiny prefill).
 *
 *   q        device, bf16 [B][K+1][n_heads][head_dim], 16-byte aligned.
 *   k_cache  device, bf16 [B][T][n_kv_heads][head_dim]: the keys of all T
 *            positions, the K+1 verify positions last; 16-byte aligned.
 *   v_cache  device, bf16, same layout as k_cache.
 *   out      device, [B][K+1][n_heads][head_dim] of out_dtype (SPEC_F32 or
 *            SPEC_BF16).
 *   Query position i (0..K) sits at position T-K-1+i and sees positions
 *   0..T-K-1+i; query head h reads key/value head h / (n_heads /
 *   n_kv_heads). out = softmax(scale * q . k) v, fp32 softmax and
 *   accumulation (the probabilities enter the value product as bf16).
 *   Limits: head_dim = 128; n_kv_heads divides n_heads;
 *   (K+1) * n_heads / n_kv_heads <= 32 query rows per key/value head
 *   (else SPEC_ERR_UNSUPPORTED); 0 <= K <= 64; K+1 <= T <= 2^24;
 *   1 <= B, n_kv_heads <= 65535; scale finite.
 *   workspace  device, at least spec_verify_attention_workspace_bytes(...)
 *            bytes (may be 0, then workspace may be null), 256-byte aligned,
 *            caller-owned; it holds the partial results of the context
 *            splits and is not read before being written.
 * Asynchronous on `stream`; allocates nothing.
 */
size_t spec_verify_attention_workspace_bytes(int B, int K, int T, int n_heads, int n_kv_heads,
                                             int head_dim);
int spec_verify_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                          void* out, int out_dtype, int B, int K, int T, int n_heads,
                          int n_kv_heads, int head_dim, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * spec_chain_error -- read and clear the device-side error word of a chain
 * workspace (synchronous). *error receives 0 if all is well; bit 0: a
 * workgroup gave up waiting at a barrier (its outputs are not valid); bit 1:
 * a launch did not match the prepared plan.
 */
int spec_chain_error(void* workspace, int* error);

/*
 * Measurement helpers: the achievable ceilings that the verify pass's
 * roofline fractions are quoted beside (the pass is priced against the
 * published 8 TB/s HBM and 2.5 PFLOP/s dense bf16 figures; "Speculative
 * Decoding: Guess Several Tokens, Check Them in One Pass", Step 1, and
 * "Speculative Decoding: The Algebra and the Proof", Where it breaks).
 *
 * spec_probe_read -- read `bytes` of device memory at `buf` once, front to
 * back, with 16-byte non-temporal loads from one persistent grid of
 * `wgs_per_cu` (1..4) workgroups of eight waves per compute unit, each lane
 * keeping `loads_per_lane` (1, 2, 4 or 8) loads in flight: 8 KB x loads x
 * workgroups in flight per compute unit. Nothing is written except,
 * in practice never, one word of `sink` (a device word the caller owns;
 * it keeps the loads from being optimised away). Time it with events on
 * `stream`; bytes / time is the achievable read bandwidth when `bytes` is
 * well above the 256 MB Infinity Cache (e.g. 4 GiB).
 *   buf   device, 16-byte aligned; bytes a positive multiple of 16.
 *
 * spec_probe_read_lds -- the same front-to-back read, one workgroup of
 * eight waves per compute unit, with the loads going straight to LDS
 * (global_load_lds, the path that feeds the tile kernels' operand rings):
 * each wave keeps `loads_per_lane` (1, 2, 4 or 8) one-kilobyte loads in
 * flight into a ring of as many LDS slots. bytes / time is the read
 * bandwidth that path can reach. Arguments, errors and sink as for
 * spec_probe_read.
 *
 * spec_probe_mfma -- independent chains of bf16 MFMAs on register operands
 * (no memory traffic): `iters` rounds per wave of eight independent
 * v_mfma_f32_16x16x32_bf16 (shape 16) or four v_mfma_f32_32x32x16_bf16
 * (shape 32), four waves per workgroup, two workgroups per compute unit. *flops
 * (host) receives the launch's floating-point operations; flops / time is
 * the achievable dense bf16 rate. sink as above.
 * Both are asynchronous on `stream` and allocate nothing.
 */
int spec_probe_read(const void* buf, size_t bytes, int loads_per_lane, int wgs_per_cu,
                    void* sink, void* stream);
int spec_probe_read_lds(const void* buf, size_t bytes, int loads_per_lane, void* sink,
                        void* stream);
int spec_probe_mfma(int shape, int iters, void* sink, double* flops, void* stream);

/*
 * spec_chain_reset -- set the barrier counters of a prepared chain workspace
 * to the values they hold after `generation` complete launches, and clear
 * its error word (synchronous; no launch may be using the workspace). The
 * descriptors are kept. After a barrier gave up (bit 0 of
 * spec_chain_error) the counters no longer agree with one another, and every
 * later launch would give up too; a reset makes the next launch consistent
 * again. Every counter advances by a fixed amount per launch and is compared
 * modulo 2^32, so any generation is valid, including those close to the
 * 32-bit wrap of the counters. Returns SPEC_ERR_INVALID_ARGUMENT if the
 * workspace holds no prepared chain.
 */
int spec_chain_reset(void* workspace, unsigned generation);

/*
 * spec_softmax -- p = softmax(logits) per row, T = 1.
 *
 * ("Speculative Decoding: Two Models, One Voice", Implementing it against a
 * real model: p = softmax(target logits), q = softmax(draft logits).)
 *
 *   logits      fp32 [rows][V].
 *   probs       fp32 [rows][V] or NULL: exp(l - max) / sumexp.
 *   row_max     fp32 [rows] or NULL: max_v l[v].
 *   row_sumexp  fp32 [rows] or NULL: sum_v exp(l[v] - max).
 * One pass over each row keeps a running max and a rescaled running sum; a
 * second pass writes probs when requested. Whichever outputs are non-NULL
 * are written. 1 <= rows <= 2^24, 1 <= V <= 2^26.
 */
int spec_softmax(const float* logits, int rows, int V, float* probs,
                 float* row_max, float* row_sumexp, void* stream);

/*
 * spec_accept_scan -- the accept test and the first rejection.
 *
 * For each sequence b and draft j: ratio = p_j(x_j) / q_j(x_j) (+inf if
 * q_j(x_j) = 0 < p_j(x_j); 0 if both are 0), accepted iff u_accept[b][j] <
 * ratio, which happens with probability min(1, p/q) ("Speculative
 * Decoding: Two Models, One Voice", The idea, step 3). n_accepted[b] is the
 * index of the first rejected draft, or K: later drafts are discarded, so the
 * accepted tokens form a prefix (same page, The rule that makes it exact).
 *
 *   p_probs       fp32 [B][K+1][V]   target probabilities.
 *   q_probs       fp32 [B][K][V]     draft probabilities.
 *   draft_tokens  int32 [B][K].
 *   u_accept      fp32 [B][K].
 *   n_accepted    int32 [B] (out).
 *   accept_mask   uint8 [B][K] or NULL (out): 1 where the test passed,
 *                 including positions after the first rejection.
 * The ratio is evaluated in fp64. 1 <= B <= 2^20, 1 <= K <= 64, V >= 1.
 */
int spec_accept_scan(const float* p_probs, const float* q_probs,
                     const int32_t* draft_tokens, const float* u_accept,
                     int B, int K, int V, int32_t* n_accepted,
                     uint8_t* accept_mask, void* stream);

/*
 * spec_residual_sample -- the token that ends the round.
 *
 * With n = n_accepted[b]: if n < K the token is drawn from
 * norm(max(0, p_n - q_n)) with u = u_sample[b][n]; if n = K it is the bonus
 * token drawn from p_K with u = u_sample[b][K] ("Speculative Decoding: Two
 * Models, One Voice", The idea, step 3). Inverse CDF in ascending token id:
 * the token is the smallest y whose running weight sum exceeds u * Z (Z the
 * total weight). If the residual has no mass the draw falls back to p_n and
 * zero_residual[b] is set ("What Actually Happens During Speculative
 * Decoding in LLMs", the reference sampler's guard; "Speculative Decoding:
 * The Algebra and the Proof" warns that p = q leaves nothing to normalise).
 * Weights and running sums are fp64.
 *
 *   p_probs, q_probs  as for spec_accept_scan.
 *   n_accepted        int32 [B].
 *   u_sample          fp32 [B][K+1].
 *   token             int32 [B] (out).
 *   zero_residual     uint8 [B] or NULL (out).
 * 1 <= B <= 2^20, 1 <= K <= 64, 1 <= V <= 2^26.
 */
int spec_residual_sample(const float* p_probs, const float* q_probs,
                         const int32_t* n_accepted, const float* u_sample,
                         int B, int K, int V, int32_t* token,
                         uint8_t* zero_residual, void* stream);

/* Bytes of device workspace spec_verify needs for (B, K, V); 0 on invalid
 * arguments. */
size_t spec_verify_workspace_bytes(int B, int K, int V);

/*
 * spec_verify -- the whole verify step after the stack: lm-head, softmax,
 * accept scan, residual or bonus sample, emit.
 *
 *   hidden        bf16 [B*(K+1)][d] or NULL; 16-byte aligned.
 *   lm_head       bf16 [V][d] or NULL; 16-byte aligned. When both are given,
 *                 target_logits = hidden . lm_head^T (fp32) is computed
 *                 first; when both are NULL, target_logits is an input.
 *   d             hidden size (ignored when lm_head is NULL).
 *   target_logits fp32 [B][K+1][V] (out or in, see above; left readable).
 *   draft_logits  fp32 [B][K][V].
 *   draft_tokens  int32 [B][K].
 *   u_accept      fp32 [B][K].
 *   u_sample      fp32 [B][K+1].
 *   out_tokens    int32 [B][K+1] (out): the accepted drafts, then the
 *                 sampled token, then -1 padding.
 *   n_emitted     int32 [B] (out): n_accepted + 1, between 1 and K+1
 *                 ("Speculative Decoding: Two Models, One Voice", Appendix
 *                 tool 2: every round emits N + 1 tokens).
 *   workspace     device memory of at least spec_verify_workspace_bytes(B,
 *                 K, V), 256-byte aligned; its contents are scratch.
 * Target and draft probabilities are never materialised: per-row max and
 * sum of exponentials are kept in the workspace and probabilities of the
 * few tokens the rule touches are evaluated in fp64 from the logits.
 * Limits as for the calls above, with V <= 2^26 and d as d_in of
 * spec_verify_gemm.
 */
int spec_verify(const uint16_t* hidden, const uint16_t* lm_head, int d,
                float* target_logits, const float* draft_logits,
                const int32_t* draft_tokens, const float* u_accept,
                const float* u_sample, int B, int K, int V,
                int32_t* out_tokens, int32_t* n_emitted, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * spec_verify_warped -- spec_verify on temperature-warped distributions:
 * p = softmax(target_logits / t_target), q = softmax(draft_logits /
 * t_draft). The accept test, the first rejection and the residual or bonus
 * draw are unchanged; they are exact for whatever distributions they are
 * given ("Speculative Decoding: Two Models, One Voice", Three remarks worth
 * internalizing; "Speculative Decoding: Guess Several Tokens, Check Them in
 * One Pass", What happens to the rejected tokens). t_draft must be the
 * temperature the drafts were drawn at ("Speculative Decoding: The Algebra
 * and the Proof", Where it breaks).
 *
 *   t_target, t_draft  finite, >= 0. A temperature of 0 is the one-hot law
 *                 of the row's first maximum: with t_target = 0 the step is
 *                 greedy verification -- a draft is kept iff it is the
 *                 target's argmax, and the round ends with the argmax of the
 *                 first mismatching (or the bonus) row; u_accept and
 *                 u_sample do not change the result ("Two Models, One
 *                 Voice", the same remarks). spec_verify is this call with
 *                 both temperatures 1.
 * Other arguments, limits and workspace as for spec_verify. A negative or
 * non-finite temperature returns SPEC_ERR_INVALID_ARGUMENT.
 */
int spec_verify_warped(const uint16_t* hidden, const uint16_t* lm_head, int d,
                       float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                       int B, int K, int V, float t_target, float t_draft, int32_t* out_tokens,
                       int32_t* n_emitted, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_noalloc -- spec_verify for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid allocation): the same arguments without the workspace, whose
 * role a static scratch array of the library takes. The call allocates
 * nothing and computes exactly what spec_verify computes.
 *
 * The scratch is a 4 MiB device array inside the library, one copy per GPU,
 * held until the process ends; its address is looked up once per device on
 * the first call made with that device current. Shapes whose
 * spec_verify_workspace_bytes(B, K, V) exceeds 4 MiB are rejected with
 * SPEC_ERR_WORKSPACE before anything is launched (at V = 128256 that is
 * about B > 440 at K = 8, B > 790 at K = 4). Every call on one GPU uses that
 * GPU's copy: calls that can overlap on one GPU (different streams, or
 * different host threads without ordering) race and must be serialized by
 * the caller. Nothing needs clearing between calls.
 */
int spec_verify_noalloc(const uint16_t* hidden, const uint16_t* lm_head, int d,
                        float* target_logits, const float* draft_logits,
                        const int32_t* draft_tokens, const float* u_accept,
                        const float* u_sample, int B, int K, int V, int32_t* out_tokens,
                        int32_t* n_emitted, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
