// Speculative sampling at every verified position: softmax, the accept test
// min(1, p/q) with the first rejection, and the residual / bonus draw.
//
// ("Speculative Decoding: Two Models, One Voice", The idea, step 3, and The
// rule that makes it exact; "Speculative Decoding: Guess Several Tokens,
// Check Them in One Pass", Step 3.)
//
// Row conventions (per sequence b, K drafts): target rows [B][K+1][V], draft
// rows [B][K][V]; u_accept[b][j] drives the test of draft j and
// u_sample[b][n] the draw that ends the round after n acceptances.
//
// Precision. Acceptance ratios and every weight of the final draw are fp64;
// running sums of the inverse CDF are fp64 in a fixed order, so results are
// deterministic. On the fused path (spec_verify) probabilities are never
// stored: per-row max and fp64 sum of exponentials are kept and each needed
// probability is exp(l - max) / sum evaluated in fp64 from the fp32 logit.

#include <limits.h>
#include <math.h>

#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kChunk = 4096;       // vocabulary entries per sampling chunk
constexpr int kScanThreads = 256;  // threads per chunk; 16 entries each
constexpr int kPerThread = kChunk / kScanThreads;

// ---------------------------------------------------------------------------
// Stage softmax: one workgroup per row
// ---------------------------------------------------------------------------

constexpr int kSoftmaxThreads = 512;

template <bool VEC>
__global__ __launch_bounds__(kSoftmaxThreads) void softmax_rows_kernel(
    const float* __restrict__ logits, int V, float* __restrict__ probs,
    float* __restrict__ row_max, float* __restrict__ row_sumexp) {
  __shared__ double red_d[kSoftmaxThreads / kWave];
  __shared__ float red_f[kSoftmaxThreads / kWave];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  const float* l = logits + row * (size_t)V;

  // One pass: running max m and running sum s of exp(l - m), rescaled
  // whenever the max grows.
  float m = -INFINITY;
  double s = 0.0;
  if (VEC) {
    const f32x4* l4 = reinterpret_cast<const f32x4*>(l);
    for (int i = tid; i < V / 4; i += kSoftmaxThreads) {
      const f32x4 v = l4[i];
      const float mx = fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
      if (mx > m) {
        s *= (double)expf(m - mx);
        m = mx;
      }
      s += (double)(expf(v.x - m) + expf(v.y - m)) + (double)(expf(v.z - m) + expf(v.w - m));
    }
  } else {
    for (int i = tid; i < V; i += kSoftmaxThreads) {
      const float v = l[i];
      if (v > m) {
        s *= (double)expf(m - v);
        m = v;
      }
      s += (double)expf(v - m);
    }
  }
  const float M = block_max_f32<kSoftmaxThreads>(m, red_f);
  const double part = (s > 0.0) ? s * (double)expf(m - M) : 0.0;
  const double S = block_sum_f64<kSoftmaxThreads>(part, red_d);
  if (tid == 0) {
    if (row_max) row_max[row] = M;
    if (row_sumexp) row_sumexp[row] = (float)S;
  }
  if (probs) {
    float* p = probs + row * (size_t)V;
    if (VEC) {
      const f32x4* l4 = reinterpret_cast<const f32x4*>(l);
      f32x4* p4 = reinterpret_cast<f32x4*>(p);
      for (int i = tid; i < V / 4; i += kSoftmaxThreads) {
        const f32x4 v = l4[i];
        p4[i] = f32x4{(float)((double)expf(v.x - M) / S), (float)((double)expf(v.y - M) / S),
                      (float)((double)expf(v.z - M) / S), (float)((double)expf(v.w - M) / S)};
      }
    } else {
      for (int i = tid; i < V; i += kSoftmaxThreads) p[i] = (float)((double)expf(l[i] - M) / S);
    }
  }
}

hipError_t launch_softmax_rows(const float* logits, int rows, int V, float* probs, float* row_max,
                               float* row_sumexp, hipStream_t s) {
  const bool vec = (V % 4 == 0) && ((uintptr_t)logits % 16 == 0) &&
                   (probs == nullptr || (uintptr_t)probs % 16 == 0);
  if (vec)
    hipLaunchKernelGGL(softmax_rows_kernel<true>, dim3(rows), dim3(kSoftmaxThreads), 0, s, logits,
                       V, probs, row_max, row_sumexp);
  else
    hipLaunchKernelGGL(softmax_rows_kernel<false>, dim3(rows), dim3(kSoftmaxThreads), 0, s,
                       logits, V, probs, row_max, row_sumexp);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Accept test and first rejection (wave ballot)
// ---------------------------------------------------------------------------

// ratio = p/q with q = 0 giving +inf when p > 0 and 0 otherwise; the test
// u < ratio accepts with probability min(1, p/q).
__device__ __forceinline__ bool accept_decision(double p, double q, float u) {
  double ratio;
  if (q > 0.0)
    ratio = p / q;
  else
    ratio = (p > 0.0) ? INFINITY : 0.0;
  return (double)u < ratio;
}

// n_accepted = index of the first lane in [0, K) whose test failed, or K.
__device__ __forceinline__ int first_rejection(bool acc, int K) {
  const unsigned long long mask = __ballot(acc);
  const unsigned long long rejected = ~mask;
  int n = rejected ? (__ffsll((long long)rejected) - 1) : kWave;
  return n < K ? n : K;
}

// One wave per sequence on probabilities.
__global__ __launch_bounds__(kWave) void accept_probs_kernel(
    const float* __restrict__ p, const float* __restrict__ q, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_accept, int K, int V, int32_t* __restrict__ n_accepted,
    uint8_t* __restrict__ mask) {
  const int b = blockIdx.x, j = threadIdx.x;
  bool acc = false;
  if (j < K) {
    const int x = tokens[(size_t)b * K + j];
    if (x >= 0 && x < V) {
      const double pp = p[((size_t)b * (K + 1) + j) * V + x];
      const double qq = q[((size_t)b * K + j) * V + x];
      acc = accept_decision(pp, qq, u_accept[(size_t)b * K + j]);
    }
    if (mask) mask[(size_t)b * K + j] = acc ? 1 : 0;
  }
  const int n = first_rejection(acc, K);
  if (j == 0) n_accepted[b] = n;
}

hipError_t launch_accept_probs(const float* p, const float* q, const int32_t* tokens,
                               const float* u_accept, int B, int K, int V, int32_t* n_accepted,
                               uint8_t* mask, hipStream_t s) {
  hipLaunchKernelGGL(accept_probs_kernel, dim3(B), dim3(kWave), 0, s, p, q, tokens, u_accept, K,
                     V, n_accepted, mask);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Inverse-CDF draw over one chunk
// ---------------------------------------------------------------------------

// Weights of one sampling row. residual: max(0, p - q); otherwise p.
struct ProbWeights {
  const float* p;
  const float* q;  // null for a plain draw from p
  __device__ __forceinline__ double operator()(int v) const {
    const double pv = p[v];
    if (!q) return pv;
    const double r = pv - (double)q[v];
    return r > 0.0 ? r : 0.0;
  }
};

// e^((l - m) * inv) for the bulk sums of the statistics, residual and draw
// passes, as 2^y with y = (l - m) * sc, sc = inv * log2(e), in fp32 and
// v_exp_f32. The error of y grows with |l - m|, but the terms that carry a
// sum (l - m above about -10 at inv = 1) keep a relative error under about
// 5e-7, more than an order under the 1e-5 band in which decisions count as
// ties; terms under 2^-126 of the maximum's flush to zero, far below what
// an fp64 sum of terms near 1 resolves. The sums themselves are fp64. The
// accept test's p(x) and q(x) use the fp64 exp.
__device__ __forceinline__ double exp_term(float l, float m, float sc) {
  return (double)exp2f((l - m) * sc);
}
__host__ __device__ inline float exp_scale(double inv) { return (float)(inv * 1.4426950408889634); }

// Weights of a draw from logits: p(v) = exp((l_p[v] - m_p) / T_p) / s_p,
// minus q(v) for a residual. ip, iq are the inverse temperatures (1 at
// T = 1); a greedy draft (T_q = 0) is one-hot at qarg. The residual pass and
// the draw evaluate the same weights, so the chunk sums that pick a chunk
// and the running sum inside it agree up to summation order.
struct LogitWeights {
  const float* lp;
  const float* lq;  // null for a plain draw from p
  float mp, mq;     // row maxima
  double sp, sq;    // row sums of exp((l - max) * inv)
  float scp, scq;   // exp_scale of the inverse temperatures
  int qarg = -1;    // >= 0: the draft is one-hot at this token
  __device__ __forceinline__ double operator()(int v) const {
    const double pv = exp_term(lp[v], mp, scp) * (1.0 / sp);
    if (!lq) return pv;
    const double qv = qarg >= 0 ? (v == qarg ? 1.0 : 0.0) : exp_term(lq[v], mq, scq) * (1.0 / sq);
    const double r = pv - qv;
    return r > 0.0 ? r : 0.0;
  }
};

// Fixed-order fp64 sum of the weights of chunk c (256 threads x 16 entries).
template <class Wt>
__device__ double chunk_sum(const Wt& wt, int c, int V, double* red) {
  const int v0 = c * kChunk + threadIdx.x * kPerThread;
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (v0 + i < V) t += wt(v0 + i);
  return block_sum_f64<kScanThreads>(t, red);
}

// Smallest token y in chunk c with w[y] > 0 and base + C_chunk[y] > T, where
// C_chunk is the running sum inside the chunk; if rounding leaves no such y,
// the largest y in the chunk with w[y] > 0; -1 if the chunk has no weight.
template <class Wt>
__device__ int chunk_draw(const Wt& wt, int c, int V, double base, double T, double* red_d,
                          int* red_i) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int v0 = c * kChunk + tid * kPerThread;
  double w[kPerThread];
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    w[i] = (v0 + i < V) ? wt(v0 + i) : 0.0;
    t += w[i];
  }
  // exclusive scan of the per-thread sums: wave inclusive scan, then waves
  double inc = t;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const double y = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += y;
  }
  if (lane == kWave - 1) red_d[wave] = inc;
  __syncthreads();
  double before = 0.0;
  for (int k = 0; k < wave; ++k) before += red_d[k];
  __syncthreads();
  double run = base + (before + (inc - t));
  int cand = 0x7fffffff, last = -1;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    if (w[i] > 0.0) {
      run += w[i];
      if (cand == 0x7fffffff && run > T) cand = v0 + i;
      last = v0 + i;
    }
  }
  // block min of cand, block max of last
  for (int o = 32; o > 0; o >>= 1) {
    cand = min(cand, __shfl_xor(cand, o, kWave));
    last = max(last, __shfl_xor(last, o, kWave));
  }
  if (lane == 0) {
    red_i[wave] = cand;
    red_i[kScanThreads / kWave + wave] = last;
  }
  __syncthreads();
  int bc = red_i[0], bl = red_i[kScanThreads / kWave];
  for (int k = 1; k < kScanThreads / kWave; ++k) {
    bc = min(bc, red_i[k]);
    bl = max(bl, red_i[kScanThreads / kWave + k]);
  }
  __syncthreads();
  return bc != 0x7fffffff ? bc : bl;
}

// Picks the chunk that holds T given the chunk sums sc[0..C) (read through
// `sum_of`), in ascending order. Returns the chunk and its base.
template <class SumOf>
__device__ __forceinline__ int pick_chunk(const SumOf& sum_of, int C, double T, double* base) {
  double run = 0.0;
  int last_pos = -1;
  double last_base = 0.0;
  for (int c = 0; c < C; ++c) {
    const double sc = sum_of(c);
    if (sc > 0.0) {
      if (run + sc > T) {
        *base = run;
        return c;
      }
      last_pos = c;
      last_base = run;
    }
    run += sc;
  }
  *base = last_base;
  return last_pos;
}

// ---------------------------------------------------------------------------
// Stage draw on probabilities: one workgroup per sequence
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kScanThreads) void sample_probs_kernel(
    const float* __restrict__ p, const float* __restrict__ q, const int32_t* __restrict__ n_acc,
    const float* __restrict__ u_sample, int K, int V, int32_t* __restrict__ token,
    uint8_t* __restrict__ zero_residual) {
  __shared__ double red_d[kScanThreads / kWave];
  __shared__ int red_i[2 * kScanThreads / kWave];
  const int b = blockIdx.x;
  const int n = n_acc[b];
  if (n < 0 || n > K) {
    if (threadIdx.x == 0) {
      token[b] = -1;
      if (zero_residual) zero_residual[b] = 0;
    }
    return;
  }
  const int C = (V + kChunk - 1) / kChunk;
  const float* prow = p + ((size_t)b * (K + 1) + n) * V;
  ProbWeights wt{prow, n < K ? q + ((size_t)b * K + n) * V : nullptr};
  // total mass, chunk by chunk in ascending order
  double Z = 0.0;
  for (int c = 0; c < C; ++c) Z += chunk_sum(wt, c, V, red_d);
  bool zero = false;
  if (!(Z > 0.0) && wt.q) {  // empty residual: fall back to p
    zero = true;
    wt.q = nullptr;
    Z = 0.0;
    for (int c = 0; c < C; ++c) Z += chunk_sum(wt, c, V, red_d);
  }
  int y = -1;
  if (Z > 0.0) {
    const double T = (double)u_sample[(size_t)b * (K + 1) + n] * Z;
    // second pass: running chunk sums (identical values) up to the crossing
    double run = 0.0, base = 0.0;
    int cc = -1;
    double last_base = 0.0;
    int last_c = -1;
    for (int c = 0; c < C; ++c) {
      const double sc = chunk_sum(wt, c, V, red_d);
      if (sc > 0.0) {
        if (run + sc > T) {
          cc = c;
          base = run;
          break;
        }
        last_c = c;
        last_base = run;
      }
      run += sc;
    }
    if (cc < 0) {
      cc = last_c;
      base = last_base;
    }
    if (cc >= 0) y = chunk_draw(wt, cc, V, base, T, red_d, red_i);
  }
  if (threadIdx.x == 0) {
    token[b] = y;
    if (zero_residual) zero_residual[b] = zero ? 1 : 0;
  }
}

hipError_t launch_sample_probs(const float* p, const float* q, const int32_t* n_accepted,
                               const float* u_sample, int B, int K, int V, int32_t* token,
                               uint8_t* zero_residual, hipStream_t s) {
  hipLaunchKernelGGL(sample_probs_kernel, dim3(B), dim3(kScanThreads), 0, s, p, q, n_accepted,
                     u_sample, K, V, token, zero_residual);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fused sampling stage of spec_verify (logits in)
// ---------------------------------------------------------------------------
//
// 1. stats_partial  grid R*C: per chunk of a row, max and fp64 sum of
//                   exp((l - max) / T); R = B*(K+1) target rows then B*K
//                   draft rows. A greedy row (T = 0) keeps the first index of
//                   the maximum instead.
// 2. verify_accept  grid B, one wave: combine the chunk partials of the
//                   sequence's 2K+1 rows into (max, sum) in a fixed order,
//                   then the accept test and the first rejection.
// 3. resid_partial  grid B*C: chunk sums of the terminating row's
//                   weights (the residual, and p for the empty-residual
//                   fallback).
// 4. verify_draw    grid B: pick the chunk, draw inside it, emit.

// Warping of the two distributions: inverse temperatures, and greedy
// (temperature 0: one-hot at the row's first maximum).
struct Warp {
  double it, id;  // 1 / T_target, 1 / T_draft (0 when greedy)
  int gt, gd;     // greedy target, greedy draft
};

struct VerifyWs {
  float* pmax;    // [R][C]
  double* psum;   // [R][C]
  int32_t* parg;  // [R][C] first index of the chunk maximum (greedy rows)
  float* fmax;    // [R]
  double* fsum;   // [R]
  int32_t* farg;  // [R] first index of the row maximum (greedy rows)
  int32_t* nacc;  // [B]
  double* rsum;   // [B][C] residual (or bonus p) chunk sums
  double* qsum;   // [B][C] p chunk sums for the empty-residual fallback
  // target rows' statistics fused into the lm-head launch: [B(K+1)][kMaxStatParts]
  // (null when B(K+1) exceeds the streaming kernel's positions)
  float* tmax;
  double* tsum;
  int32_t* targ;
};

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static VerifyWs carve(void* base, int B, int K, int V, size_t* total) {
  const size_t R = (size_t)B * (2 * K + 1);
  const size_t C = (V + kChunk - 1) / kChunk;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  VerifyWs ws;
  ws.pmax = reinterpret_cast<float*>(p + off);
  off = align256(off + R * C * sizeof(float));
  ws.psum = reinterpret_cast<double*>(p + off);
  off = align256(off + R * C * sizeof(double));
  ws.parg = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + R * C * sizeof(int32_t));
  ws.fmax = reinterpret_cast<float*>(p + off);
  off = align256(off + R * sizeof(float));
  ws.fsum = reinterpret_cast<double*>(p + off);
  off = align256(off + R * sizeof(double));
  ws.farg = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + R * sizeof(int32_t));
  ws.nacc = reinterpret_cast<int32_t*>(p + off);
  off = align256(off + (size_t)B * sizeof(int32_t));
  ws.rsum = reinterpret_cast<double*>(p + off);
  off = align256(off + (size_t)B * C * sizeof(double));
  ws.qsum = reinterpret_cast<double*>(p + off);
  off = align256(off + (size_t)B * C * sizeof(double));
  const size_t M = (size_t)B * (K + 1);
  ws.tmax = nullptr;
  ws.tsum = nullptr;
  ws.targ = nullptr;
  if (M <= (size_t)kMaxStreamM) {
    const size_t P = M * kMaxStatParts;
    ws.tmax = reinterpret_cast<float*>(p + off);
    off = align256(off + P * sizeof(float));
    ws.tsum = reinterpret_cast<double*>(p + off);
    off = align256(off + P * sizeof(double));
    ws.targ = reinterpret_cast<int32_t*>(p + off);
    off = align256(off + P * sizeof(int32_t));
  }
  if (total) *total = off;
  return ws;
}

LogitStats target_stats_slot(void* workspace, int B, int K, int V, float t_target) {
  const VerifyWs ws = carve(workspace, B, K, V, nullptr);
  LogitStats st{};
  st.pmax = ws.tmax;
  st.psum = ws.tsum;
  st.parg = ws.targ;
  st.greedy = t_target == 0.0f;
  st.inv = st.greedy ? 0.0 : 1.0 / (double)t_target;
  st.stride = kMaxStatParts;
  return st;
}

size_t verify_workspace_bytes(int B, int K, int V) {
  size_t total = 0;
  carve(nullptr, B, K, V, &total);
  return total;
}

// logits row of the fused layout: target rows first, then draft rows
__device__ __forceinline__ const float* verify_row(const float* tl, const float* dl, int row,
                                                   int B, int K, int V) {
  const int n_target = B * (K + 1);
  return row < n_target ? tl + (size_t)row * V : dl + (size_t)(row - n_target) * V;
}

// Entry of the chunk held in slot i of thread t. VEC (V a multiple of 4,
// 16-byte aligned rows): thread t holds entries 4 (t + 256 j) .. +3 for
// j = 0..3, so every load instruction of a wave reads 1 KB contiguous;
// otherwise entries t, t + 256, ... (256 contiguous bytes per instruction).
template <bool VEC>
__device__ __forceinline__ int chunk_entry(int c, int t, int i) {
  return VEC ? c * kChunk + ((i / 4) * kScanThreads + t) * 4 + (i % 4)
             : c * kChunk + t + i * kScanThreads;
}
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* __restrict__ l, int c, int t, int V,
                                           float (&x)[kPerThread]) {
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const int v = chunk_entry<true>(c, t, 4 * j);
      const float4 q = v < V ? *reinterpret_cast<const float4*>(l + v)
                             : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      x[4 * j] = q.x;
      x[4 * j + 1] = q.y;
      x[4 * j + 2] = q.z;
      x[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int v = chunk_entry<false>(c, t, i);
      x[i] = v < V ? l[v] : -INFINITY;
    }
  }
}

// row0: first row scanned (B(K+1) when the target rows' statistics come from
// the lm-head launch, so only draft rows are scanned). One pass over the
// chunk from memory into registers (load_chunk); the chunk maximum is
// reduced first, then the fp64 sums of exp((l - max) * inv) in a fixed order
// (per thread, a shuffle tree, then waves in order): deterministic.
template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void stats_partial_kernel(const float* __restrict__ tl,
                                                                     const float* __restrict__ dl,
                                                                     int B, int K, int V,
                                                                     VerifyWs ws, Warp wp,
                                                                     int row0) {
  __shared__ float red_m[kScanThreads / kWave];
  __shared__ double red_s[kScanThreads / kWave];
  __shared__ int red_i[kScanThreads / kWave];
  const int C = (V + kChunk - 1) / kChunk;
  const int row = row0 + (int)blockIdx.x / C, c = blockIdx.x - (row - row0) * C;
  const bool target = row < B * (K + 1);
  const bool greedy = target ? wp.gt : wp.gd;
  const double inv = target ? wp.it : wp.id;
  const float* l = verify_row(tl, dl, row, B, K, V);
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float x[kPerThread];
  load_chunk<VEC>(l, c, tid, V, x);
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) m = fmaxf(m, x[i]);
  if (greedy) {  // first index of the chunk maximum
    int first = INT_MAX;
#pragma unroll
    for (int i = kPerThread - 1; i >= 0; --i)  // slots hold ascending entries
      if (x[i] == m && x[i] != -INFINITY) first = chunk_entry<VEC>(c, tid, i);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float m2 = __shfl_xor(m, o, kWave);
      const int f2 = __shfl_xor(first, o, kWave);
      if (m2 > m || (m2 == m && f2 < first)) first = f2;
      m = fmaxf(m, m2);
    }
    if (lane == 0) {
      red_m[wave] = m;
      red_i[wave] = first;
    }
    __syncthreads();
    if (tid == 0) {
      float cm = red_m[0];
      int cf = red_i[0];
      for (int w = 1; w < kScanThreads / kWave; ++w)
        if (red_m[w] > cm || (red_m[w] == cm && red_i[w] < cf)) {
          cm = red_m[w];
          cf = red_i[w];
        }
      ws.pmax[(size_t)row * C + c] = cm;
      ws.psum[(size_t)row * C + c] = 1.0;
      ws.parg[(size_t)row * C + c] = cf;
    }
    return;
  }
  // the chunk maximum first (exact in fp32), then every sum relative to it
  const float cm = block_max_f32<kScanThreads>(m, red_m);
  const float sc = exp_scale(inv);
  double sum = 0.0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i)
    if (x[i] != -INFINITY) sum += exp_term(x[i], cm, sc);
  sum = block_sum_f64<kScanThreads>(sum, red_s);
  if (tid == 0) {
    ws.pmax[(size_t)row * C + c] = cm;
    ws.psum[(size_t)row * C + c] = sum;
  }
}

// Row statistics from partials: the maximum over partials, the fp64 sum of
// psum * exp((pmax - max) * inv) in a fixed order (lane-strided, then a
// fixed shuffle tree) and, for greedy rows, the smallest first-index among
// partials holding the maximum. Chunk partials (contiguous chunks) and the
// lm-head's per-workgroup partials merge alike; empty partials hold -inf.
__device__ __forceinline__ void merge_partials(const float* pm, const double* ps, const int32_t* pa,
                                               int n, bool greedy, double inv, float* M_out,
                                               double* S_out, int* arg_out) {
  const int lane = threadIdx.x & (kWave - 1);
  float M = -INFINITY;
  for (int c = lane; c < n; c += kWave) M = fmaxf(M, pm[c]);
  M = wave_max_f32(M);
  double S = 0.0;
  int arg = INT_MAX;
  if (greedy) {
    for (int c = lane; c < n; c += kWave)
      if (pm[c] == M) arg = min(arg, (int)pa[c]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) arg = min(arg, __shfl_xor(arg, o, kWave));
    S = 1.0;
  } else {
    for (int c = lane; c < n; c += kWave)
      if (pm[c] != -INFINITY) S += ps[c] * exp(((double)pm[c] - (double)M) * inv);
    S = wave_sum_f64(S);
  }
  *M_out = M;
  *S_out = S;
  *arg_out = greedy ? (arg == INT_MAX ? -1 : arg) : -1;
}

// tstats: the target rows' per-workgroup partials from the lm-head launch
// (tparts of them per row, stride kMaxStatParts), or tparts = 0 to use the
// chunk partials of stats_partial_kernel for every row.
constexpr int kAcceptWaves = 16;  // one wave per row up to K = 7; measured faster than 4 and 8

__global__ __launch_bounds__(kAcceptWaves * kWave) void verify_accept_kernel(
    const float* __restrict__ tl, const float* __restrict__ dl, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_accept, int B, int K, int V, VerifyWs ws, Warp wp, int tparts) {
  __shared__ float smax[2 * 64 + 1];
  __shared__ double ssum[2 * 64 + 1];
  __shared__ int sarg[2 * 64 + 1];
  const int b = blockIdx.x, lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int C = (V + kChunk - 1) / kChunk;
  // local index i: 0..K target rows, K+1..2K draft rows; each wave merges
  // whole rows' partials, rows dealt round-robin to the waves
  for (int i = wave; i < 2 * K + 1; i += kAcceptWaves) {
    const int row = i <= K ? b * (K + 1) + i : B * (K + 1) + b * K + (i - K - 1);
    const bool greedy = i <= K ? wp.gt : wp.gd;
    const double inv = i <= K ? wp.it : wp.id;
    float M;
    double S;
    int arg;
    if (i <= K && tparts > 0) {
      const size_t o = (size_t)row * kMaxStatParts;
      merge_partials(ws.tmax + o, ws.tsum + o, ws.targ + o, tparts, greedy, inv, &M, &S, &arg);
    } else {
      const size_t o = (size_t)row * C;
      merge_partials(ws.pmax + o, ws.psum + o, ws.parg + o, C, greedy, inv, &M, &S, &arg);
    }
    if (lane == 0) {
      ws.fmax[row] = M;
      ws.fsum[row] = S;
      ws.farg[row] = arg;
      smax[i] = M;
      ssum[i] = S;
      sarg[i] = arg;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  bool acc = false;
  if (lane < K) {
    const int x = tokens[(size_t)b * K + lane];
    if (x >= 0 && x < V) {
      const int trow = b * (K + 1) + lane, drow = b * K + lane;
      const double pp = wp.gt ? (x == sarg[lane] ? 1.0 : 0.0)
                              : exp(((double)tl[(size_t)trow * V + x] - (double)smax[lane]) * wp.it) /
                                    ssum[lane];
      const double qq =
          wp.gd ? (x == sarg[K + 1 + lane] ? 1.0 : 0.0)
                : exp(((double)dl[(size_t)drow * V + x] - (double)smax[K + 1 + lane]) * wp.id) /
                      ssum[K + 1 + lane];
      acc = accept_decision(pp, qq, u_accept[(size_t)b * K + lane]);
    }
  }
  const int n = first_rejection(acc, K);
  if (lane == 0) ws.nacc[b] = n;
}

__device__ __forceinline__ LogitWeights verify_weights(const float* tl, const float* dl, int b,
                                                       int n, int B, int K, int V,
                                                       const VerifyWs& ws, bool with_q,
                                                       const Warp& wp) {
  const int trow = b * (K + 1) + n;
  LogitWeights w;
  w.lp = tl + (size_t)trow * V;
  w.mp = ws.fmax[trow];
  w.sp = ws.fsum[trow];
  w.scp = exp_scale(wp.it);
  w.scq = exp_scale(wp.id);
  if (with_q && n < K) {
    const int drow = B * (K + 1) + b * K + n;
    w.lq = dl + (size_t)(b * K + n) * V;
    w.mq = ws.fmax[drow];
    w.sq = ws.fsum[drow];
    w.qarg = wp.gd ? ws.farg[drow] : -1;
  } else {
    w.lq = nullptr;
    w.mq = 0.0f;
    w.sq = 1.0;
  }
  return w;
}

template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void resid_partial_kernel(
    const float* __restrict__ tl, const float* __restrict__ dl, int B, int K, int V, VerifyWs ws,
    Warp wp) {
  __shared__ double red_d[kScanThreads / kWave];
  if (wp.gt) return;  // greedy target: the round ends with the row's argmax, no draw
  const int C = (V + kChunk - 1) / kChunk;
  const int b = blockIdx.x / C, c = blockIdx.x - b * C;
  const int n = ws.nacc[b];
  const LogitWeights w = verify_weights(tl, dl, b, n, B, K, V, ws, true, wp);
  const double isp = 1.0 / w.sp, isq = 1.0 / w.sq;
  // the chunk's logits as stats_partial loads them; each weight is computed
  // as LogitWeights computes it
  float xp[kPerThread], xq[kPerThread];
  load_chunk<VEC>(w.lp, c, threadIdx.x, V, xp);
  if (w.lq && w.qarg < 0) load_chunk<VEC>(w.lq, c, threadIdx.x, V, xq);
  double tr = 0.0, tp = 0.0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int v = chunk_entry<VEC>(c, threadIdx.x, i);
    if (v < V) {
      const double pv = exp_term(xp[i], w.mp, w.scp) * isp;
      tp += pv;
      if (w.lq) {
        const double qv = w.qarg >= 0 ? (v == w.qarg ? 1.0 : 0.0)
                                      : exp_term(xq[i], w.mq, w.scq) * isq;
        const double r = pv - qv;
        tr += r > 0.0 ? r : 0.0;
      }
    }
  }
  if (!w.lq) tr = tp;
  tr = block_sum_f64<kScanThreads>(tr, red_d);
  tp = block_sum_f64<kScanThreads>(tp, red_d);
  if (threadIdx.x == 0) {
    ws.rsum[(size_t)b * C + c] = tr;
    ws.qsum[(size_t)b * C + c] = tp;
  }
}

__global__ __launch_bounds__(kScanThreads) void verify_draw_kernel(
    const float* __restrict__ tl, const float* __restrict__ dl, const int32_t* __restrict__ tokens,
    const float* __restrict__ u_sample, int B, int K, int V, int32_t* __restrict__ out_tokens,
    int32_t* __restrict__ n_emitted, VerifyWs ws, Warp wp) {
  __shared__ double red_d[kScanThreads / kWave];
  __shared__ int red_i[2 * kScanThreads / kWave];
  __shared__ double s_base, s_T;
  __shared__ int s_chunk, s_use_p;
  const int b = blockIdx.x;
  const int C = (V + kChunk - 1) / kChunk;
  const int n = ws.nacc[b];
  if (wp.gt) {
    // greedy target: the rejected slot (or the bonus slot) gets the row's
    // argmax; the residual of a one-hot p is one-hot at the same token
    if (threadIdx.x == 0) {
      s_chunk = -2;
      s_use_p = 0;
    }
  } else if (threadIdx.x < kWave) {
    // The chunk that holds T = u * Z, found by the first wave: lane l sums
    // its own run of chunks, a shuffle scan gives each run's base, and the
    // first run that passes T is walked chunk by chunk (as pick_chunk would
    // walk all of them; only the rounding of the running sum differs).
    const int lane = threadIdx.x;
    const double* rs = ws.rsum + (size_t)b * C;
    const double* ps = ws.qsum + (size_t)b * C;
    const int per = (C + kWave - 1) / kWave;
    const int c0 = min(lane * per, C), c1 = min(c0 + per, C);
    double lr = 0.0, lp = 0.0;
    for (int c = c0; c < c1; ++c) {
      lr += rs[c];
      lp += ps[c];
    }
    double Z = wave_sum_f64(lr);
    const int use_p = !(Z > 0.0);  // empty residual: fall back to p of the same row
    if (use_p) Z = wave_sum_f64(lp);
    const double* sc = use_p ? ps : rs;
    const double loc = use_p ? lp : lr;
    const double T = (double)u_sample[(size_t)b * (K + 1) + n] * Z;
    double inc = loc;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const double y = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += y;
    }
    const double run0 = inc - loc;  // this lane's base
    const unsigned long long hit = __ballot(loc > 0.0 && run0 + loc > T);
    const unsigned long long pos = __ballot(loc > 0.0);
    // the lane that walks its run: the first that passes T, else (rounding)
    // the last with weight
    const int owner = hit ? __ffsll((long long)hit) - 1 : (pos ? 63 - __clzll((long long)pos) : -1);
    if (lane == 0) {
      s_T = T;
      s_use_p = use_p;
      s_chunk = -1;
      s_base = 0.0;
    }
    if (Z > 0.0 && lane == owner) {
      double run = run0, last_base = 0.0;
      int chunk = -1, last_pos = -1;
      for (int c = c0; c < c1; ++c) {
        const double w = sc[c];
        if (w > 0.0) {
          if (hit && run + w > T) {
            chunk = c;
            break;
          }
          last_pos = c;
          last_base = run;
        }
        run += w;
      }
      if (chunk < 0) {
        chunk = last_pos;
        run = last_base;
      }
      s_chunk = chunk;
      s_base = run;
    }
  }
  __syncthreads();
  const int chunk = s_chunk;
  int y = -1;
  if (chunk == -2) {
    y = ws.farg[b * (K + 1) + n];
  } else if (chunk >= 0) {
    const LogitWeights w = verify_weights(tl, dl, b, n, B, K, V, ws, !s_use_p, wp);
    y = chunk_draw(w, chunk, V, s_base, s_T, red_d, red_i);
  }
  for (int j = threadIdx.x; j < K + 1; j += kScanThreads) {
    int32_t t = -1;
    if (j < n)
      t = tokens[(size_t)b * K + j];
    else if (j == n)
      t = y;
    out_tokens[(size_t)b * (K + 1) + j] = t;
  }
  if (threadIdx.x == 0) n_emitted[b] = n + 1;
}

hipError_t launch_verify_sampling(const float* tl, const float* dl, const int32_t* tokens,
                                  const float* u_accept, const float* u_sample, int B, int K, int V,
                                  int32_t* out_tokens, int32_t* n_emitted, void* workspace,
                                  float t_target, float t_draft, hipStream_t s,
                                  const LogitStats* target_stats, int parts) {
  const VerifyWs ws = carve(workspace, B, K, V, nullptr);
  const int C = (V + kChunk - 1) / kChunk;
  const int R = B * (2 * K + 1);
  Warp wp;
  wp.gt = t_target == 0.0f;
  wp.gd = t_draft == 0.0f;
  wp.it = wp.gt ? 0.0 : 1.0 / (double)t_target;
  wp.id = wp.gd ? 0.0 : 1.0 / (double)t_draft;
  const bool fused = target_stats && target_stats->pmax && target_stats->pmax == ws.tmax &&
                     parts > 0 && parts <= kMaxStatParts;
  const int row0 = fused ? B * (K + 1) : 0;
  // 16-byte loads when every row starts on a 16-byte boundary
  const bool vec = V % 4 == 0 && ((reinterpret_cast<uintptr_t>(tl) | reinterpret_cast<uintptr_t>(dl)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(stats_partial_kernel<true>, dim3((R - row0) * C), dim3(kScanThreads), 0, s,
                       tl, dl, B, K, V, ws, wp, row0);
  else
    hipLaunchKernelGGL(stats_partial_kernel<false>, dim3((R - row0) * C), dim3(kScanThreads), 0, s,
                       tl, dl, B, K, V, ws, wp, row0);
  hipLaunchKernelGGL(verify_accept_kernel, dim3(B), dim3(kAcceptWaves * kWave), 0, s, tl, dl,
                     tokens, u_accept, B, K, V, ws, wp, fused ? parts : 0);
  if (vec)
    hipLaunchKernelGGL(resid_partial_kernel<true>, dim3(B * C), dim3(kScanThreads), 0, s, tl, dl, B,
                       K, V, ws, wp);
  else
    hipLaunchKernelGGL(resid_partial_kernel<false>, dim3(B * C), dim3(kScanThreads), 0, s, tl, dl, B,
                       K, V, ws, wp);
  hipLaunchKernelGGL(verify_draw_kernel, dim3(B), dim3(kScanThreads), 0, s, tl, dl, tokens,
                     u_sample, B, K, V, out_tokens, n_emitted, ws, wp);
  return hipGetLastError();
}

}  // namespace specv
