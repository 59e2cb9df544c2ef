// Verify attention: the K+1 verify positions of each sequence attend, through
// the causal mask, over its KV cache ("Speculative Decoding: Guess Several
// Tokens, Check Them in One Pass", Step 1: the pass is a tiny prefill and
// reads the cache once for all K+1 positions).
//
// Shapes: q [B][K+1][H][D], k/v cache [B][T][Hkv][D] (the K+1 verify
// positions are the last K+1 entries), out [B][K+1][H][D]; D = 128. Query
// position i sits at absolute position T-K-1+i; head h reads key/value head
// h / G, G = H / Hkv.
//
// The cache is read once and the work per byte is small (R = (K+1) * G query
// rows share every key/value row of a head), so HBM bounds the kernel:
//
//  * Grid (split, kv head, sequence): a split is a range of the cache's
//    tokens; splits give small batches enough workgroups. Within a
//    workgroup, each of four waves walks its own 32-token tiles with its own
//    running softmax (max, sum, output), and the waves are merged at the
//    end, then the splits in a second kernel, in a fixed order.
//  * A tile's keys and values come in as whole 256-byte rows (16 lanes x
//    16 bytes per row, 4 rows per load instruction) into registers, two
//    tiles ahead, and go to the wave's own LDS tile with an XOR swizzle of
//    the 16-byte units, so the operand reads below are free of bank
//    conflicts. No barrier is needed: a wave's LDS accesses run in order.
//  * S^T = K Q^T on the matrix cores (v_mfma_f32_16x16x32_bf16, A = 16 keys,
//    B = 16 query rows, reduction over D). Computing the transpose leaves
//    each lane with one query row's scores of 8 tokens: exactly the 8
//    reduction slots of the P operand of the next product, so the
//    probabilities need no shuffle.
//  * O^T += V^T P^T on the matrix cores: A = 16 value columns, gathered from
//    the LDS tile for the same 8 tokens per lane group.
//  * Softmax in base 2 (scale * log2 e folded into the scores), masked
//    entries -inf; a running max of -inf is replaced by 0 in the exponents
//    so that no -inf - -inf arises. P is rounded to bf16 for the product
//    and the row sums add the same rounded values.

#include <math.h>

#include "common.h"
#include "internal.h"

namespace specv {

constexpr int kAttD = 128;
constexpr int kAttWaves = 4;
constexpr int kAttThreads = kAttWaves * kWave;
constexpr int kAttTile = 32;                     // tokens per tile
constexpr int kAttRowBytes = kAttD * 2;          // 256 bytes per token and head
constexpr int kAttTileBytes = kAttTile * kAttRowBytes;      // 8 KB
constexpr int kAttWaveLds = 2 * kAttTileBytes;               // keys + values
constexpr int kAttLds = kAttWaves * kAttWaveLds;             // 64 KB
constexpr int kAttPartStride = kAttD + 2;        // o[D], m, l per partial row

#define SPECV_ATT_GLOBAL __attribute__((address_space(1)))

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  float* part;  // split partials [B][Hkv][n_split][16 * RT][kAttPartStride], or null
  int B, K1, T, H, Hkv, G, R;
  int n_split, split_len;  // tokens per split, a multiple of kAttTile * kAttWaves
  float scale_log2;        // scale * log2(e)
  int out_bf16;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_round(float v) {
  return __uint_as_float((uint32_t)f32_to_bf16_bits(v) << 16);
}

template <int RT>
__global__ __launch_bounds__(kAttThreads) void verify_attention_kernel(AttnArgs a) {
  extern __shared__ u32x4 att_lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row16 = lane & 15, grp = lane >> 4;
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int ts = split * a.split_len;
  const int te = min(ts + a.split_len, a.T);
  const int n_tiles = ts < te ? (te - ts + kAttTile - 1) / kAttTile : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + kAttWaves - 1) / kAttWaves : 0;

  // Q as the B operand of S^T: row r = i * G + qh of this kv head's group
  // (zero past R), reduction slots = D.
  u32x4 qf[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + row16;
    const bool ok = r < a.R;
    const int i = ok ? r / a.G : 0, qh = ok ? r - i * a.G : 0;
    const uint16_t* qrow = a.q + ((size_t)(b * a.K1 + i) * a.H + kvh * a.G + qh) * kAttD;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(qrow + ds * 32 + grp * 8);
      qf[rt][ds] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // last key position each of this lane's query rows may see
  int limit[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int r = rt * 16 + row16;
    limit[rt] = r < a.R ? a.T - a.K1 + r / a.G : a.T - 1;
  }

  char* wl = reinterpret_cast<char*>(att_lds) + wave * kAttWaveLds;  // this wave's tile
  const size_t head_stride = (size_t)a.Hkv * kAttD;                    // elements per token
  const uint16_t* kbase = a.k + (size_t)b * a.T * head_stride + (size_t)kvh * kAttD;
  const uint16_t* vbase = a.v + (size_t)b * a.T * head_stride + (size_t)kvh * kAttD;

  // Tile j of this wave covers tokens ts + (wave + kAttWaves j) * 32 + 0..31.
  // Loads of tiles past the wave's last one (and tokens past T) read clamped
  // valid rows; they are never used.
  struct Regs {
    u32x4 k[8], v[8];
  };
  auto load = [&](Regs& g, int j) __attribute__((always_inline)) {
    const int jc = my_tiles > 0 ? min(j, my_tiles - 1) : 0;
    const int t0 = ts + (wave + kAttWaves * jc) * kAttTile;
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int t = min(t0 + 4 * n + grp, a.T - 1);
      g.k[n] = __builtin_nontemporal_load(
          (const SPECV_ATT_GLOBAL u32x4*)(kbase + (size_t)t * head_stride) + row16);
      g.v[n] = __builtin_nontemporal_load(
          (const SPECV_ATT_GLOBAL u32x4*)(vbase + (size_t)t * head_stride) + row16);
    }
  };
  // 16-byte unit u of token t sits at t * 256 + ((u ^ (t & 7)) * 16)
  auto store_lds = [&](const Regs& g) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int t = 4 * n + grp;
      const int off = t * kAttRowBytes + ((row16 ^ (t & 7)) << 4);
      *reinterpret_cast<u32x4*>(wl + off) = g.k[n];
      *reinterpret_cast<u32x4*>(wl + kAttTileBytes + off) = g.v[n];
    }
  };

  float m_run[RT], l_run[RT];
  f32x4 acc_o[8][RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = -INFINITY;
    l_run[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc_o[dt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](int j) __attribute__((always_inline)) {
    const int t0 = ts + (wave + kAttWaves * j) * kAttTile;
    // S^T for tokens t0 + tt * 16 + 4 grp + e, query row rt * 16 + row16
    f32x4 s[2][RT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) s[tt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = tt * 16 + row16;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const int u = ds * 4 + grp;
        const u32x4 kv = *reinterpret_cast<const u32x4*>(wl + t * kAttRowBytes + ((u ^ (t & 7)) << 4));
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
          s[tt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, kv), __builtin_bit_cast(bf16x8, qf[rt][ds]), s[tt][rt],
              0, 0, 0);
      }
    }
    // masked, scaled scores; running max and sum per query row
    u32x4 pf[RT];
    float corr[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float mx = -INFINITY;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int ta = t0 + tt * 16 + 4 * grp + e;
          const bool vis = ta < te && ta <= limit[rt];
          s[tt][rt][e] = vis ? s[tt][rt][e] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, s[tt][rt][e]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run[rt], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      corr[rt] = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
      m_run[rt] = m_new;
      float p[8];
      float sum = 0.f;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = bf16_round(__builtin_amdgcn_exp2f(s[tt][rt][e] - m_use));
          p[tt * 4 + e] = pv;
          sum += pv;
        }
      sum += __shfl_xor(sum, 16, kWave);
      sum += __shfl_xor(sum, 32, kWave);
      l_run[rt] = l_run[rt] * corr[rt] + sum;
      // slot order of the P operand: tokens 4 grp + 0..3, then 16 + 4 grp + 0..3
      pf[rt] = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                     pack_bf16x2(p[6], p[7])};
    }
    // O^T[d][r] = corr * O^T + sum over the tile's tokens of V[t][d] P[r][t]
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const int d = dt * 16 + row16;
      const int u = d >> 3, w = d & 7;
      uint32_t h[4];
#pragma unroll
      for (int sl = 0; sl < 8; sl += 2) {
        const int ta = (sl < 4 ? 0 : 16) + 4 * grp + (sl & 3);
        const int tb = ta + 1;
        const uint16_t va = *reinterpret_cast<const uint16_t*>(
            wl + kAttTileBytes + ta * kAttRowBytes + ((u ^ (ta & 7)) << 4) + w * 2);
        const uint16_t vb = *reinterpret_cast<const uint16_t*>(
            wl + kAttTileBytes + tb * kAttRowBytes + ((u ^ (tb & 7)) << 4) + w * 2);
        h[sl >> 1] = (uint32_t)va | ((uint32_t)vb << 16);
      }
      const u32x4 vt{h[0], h[1], h[2], h[3]};
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        f32x4 c = acc_o[dt][rt];
        c[0] *= corr[rt];
        c[1] *= corr[rt];
        c[2] *= corr[rt];
        c[3] *= corr[rt];
        acc_o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, vt), __builtin_bit_cast(bf16x8, pf[rt]), c, 0, 0, 0);
      }
    }
  };

  // Two tiles of loads in flight; loads are issued on every path.
  Regs ra, rb;
  load(ra, 0);
  load(rb, 1);
  for (int j = 0; j < my_tiles; j += 2) {
    store_lds(ra);
    load(ra, j + 2);
    compute(j);
    store_lds(rb);
    load(rb, j + 3);
    if (j + 1 < my_tiles) compute(j + 1);
  }

  // ---- merge the four waves (fixed order), then store or write the partial
  __builtin_amdgcn_s_waitcnt(0);  // the unused loads past the last tile have landed
  __syncthreads();  // every wave is done with its tile; LDS is reused below
  constexpr int RP = 16 * RT;
  float* wm = reinterpret_cast<float*>(att_lds);          // [wave][RP]
  float* wlsum = wm + kAttWaves * RP;                      // [wave][RP]
  float* wo = wlsum + kAttWaves * RP;                      // [wave][RP][D]
  if (grp == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      wm[wave * RP + rt * 16 + row16] = m_run[rt];
      wlsum[wave * RP + rt * 16 + row16] = l_run[rt];
    }
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        wo[(wave * RP + rt * 16 + row16) * kAttD + dt * 16 + 4 * grp + e] = acc_o[dt][rt][e];
  __syncthreads();
  for (int x = tid; x < a.R * kAttD; x += kAttThreads) {
    const int r = x / kAttD, d = x - r * kAttD;
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) m = fmaxf(m, wm[w * RP + r]);
    const float m_use = m == -INFINITY ? 0.f : m;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w * RP + r] - m_use);
      o += wo[(w * RP + r) * kAttD + d] * f;
      l += wlsum[w * RP + r] * f;
    }
    const int i = r / a.G, h = kvh * a.G + (r - i * a.G);
    if (a.part) {
      float* pr = a.part +
                  ((((size_t)b * a.Hkv + kvh) * a.n_split + split) * RP + r) * kAttPartStride;
      pr[d] = o;
      if (d == 0) {
        pr[kAttD] = m;
        pr[kAttD + 1] = l;
      }
    } else {
      const size_t oi = ((size_t)(b * a.K1 + i) * a.H + h) * kAttD + d;
      const float v = o / l;
      if (a.out_bf16)
        reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(v);
      else
        reinterpret_cast<float*>(a.out)[oi] = v;
    }
  }
}

// Merge the splits of one (sequence, kv head, query row) in split order.
template <int RT>
__global__ __launch_bounds__(kAttD) void verify_attention_merge_kernel(AttnArgs a) {
  constexpr int RP = 16 * RT;
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const float* base = a.part + (((size_t)b * a.Hkv + kvh) * a.n_split * RP + r) * kAttPartStride;
  const size_t step = (size_t)RP * kAttPartStride;
  float m = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, base[s * step + kAttD]);
  const float m_use = m == -INFINITY ? 0.f : m;
  float o = 0.f, l = 0.f;
  for (int s = 0; s < a.n_split; ++s) {
    const float* p = base + s * step;
    const float f = __builtin_amdgcn_exp2f(p[kAttD] - m_use);
    o += p[d] * f;
    l += p[kAttD + 1] * f;
  }
  const int i = r / a.G, h = kvh * a.G + (r - i * a.G);
  const size_t oi = ((size_t)(b * a.K1 + i) * a.H + h) * kAttD + d;
  const float v = o / l;
  if (a.out_bf16)
    reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_bits(v);
  else
    reinterpret_cast<float*>(a.out)[oi] = v;
}

// Splits: about kAttTargetGroups workgroups in all (two per CU of the
// 256-CU part; a fixed target, so results do not depend on the device), a
// split being at least four tiles (one per wave) of tokens.
constexpr int kAttTargetGroups = 512;
int attention_splits(int B, int Hkv, int T) {
  const int per = kAttTile * kAttWaves;
  const int max_split = (T + per - 1) / per;
  const long long groups = (long long)B * Hkv;
  const int want = groups >= kAttTargetGroups ? 1 : (int)((kAttTargetGroups + groups - 1) / groups);
  return max(1, min(want, max_split));
}

size_t attention_workspace_bytes(int B, int K1, int H, int Hkv, int n_split) {
  if (n_split <= 1) return 0;
  const int R = K1 * (H / Hkv);
  const int RP = R <= 16 ? 16 : 32;
  return (size_t)B * Hkv * n_split * RP * kAttPartStride * sizeof(float);
}

template <int RT>
static hipError_t launch_att(const AttnArgs& a, hipStream_t s) {
  constexpr int RP = 16 * RT;
  const size_t lds = max((size_t)kAttLds, (size_t)(2 * kAttWaves * RP + kAttWaves * RP * kAttD) * 4);
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_attention_kernel<RT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((verify_attention_kernel<RT>), dim3(a.n_split, a.Hkv, a.B),
                     dim3(kAttThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split <= 1) return e;
  hipLaunchKernelGGL((verify_attention_merge_kernel<RT>), dim3(a.R, a.Hkv, a.B), dim3(kAttD), 0,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_verify_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                   void* out, bool out_bf16, int B, int K1, int T, int H, int Hkv,
                                   float scale, void* workspace, hipStream_t s) {
  AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.B = B;
  a.K1 = K1;
  a.T = T;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.R = K1 * a.G;
  const int per = kAttTile * kAttWaves;
  const int tiles = (T + per - 1) / per;
  const int n_split = attention_splits(B, Hkv, T);
  a.split_len = (tiles + n_split - 1) / n_split * per;
  a.n_split = (T + a.split_len - 1) / a.split_len;
  a.part = a.n_split > 1 ? static_cast<float*>(workspace) : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_bf16 = out_bf16 ? 1 : 0;
  return a.R <= 16 ? launch_att<1>(a, s) : launch_att<2>(a, s);
}

}  // namespace specv
