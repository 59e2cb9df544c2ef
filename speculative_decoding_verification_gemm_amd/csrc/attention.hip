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
//    16 bytes per row, 4 rows per load instruction) into registers, one or
//    two tiles ahead, and go to the wave's own LDS tile with an XOR swizzle of
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
constexpr int kAttQBytes = 32 * kAttRowBytes;                // query rows, after the tiles
constexpr int kAttPartStride = kAttD + 2;        // o[D], m, l per partial row

#define SPECV_ATT_GLOBAL __attribute__((address_space(1)))

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  void* out;
  float* part;  // split partials [B][Hkv][n_split][R][kAttPartStride], or null
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

// Waves and query rows: every wave computes one 16-row tile of the group's
// query rows. With up to 16 rows (RT = 1) each of the four waves walks its
// own token tiles; with 17..32 rows (RT = 2) two teams of two waves share
// token tiles, each wave of a team loading half of a tile (keys or values)
// into the team's double-buffered LDS tile, one barrier per tile step. Either
// way the registers allow two workgroups per CU.
template <int RT>
__global__ __launch_bounds__(kAttThreads, 2) void verify_attention_kernel(AttnArgs a) {
  extern __shared__ u32x4 att_lds[];
  constexpr int kTeams = kAttWaves / RT;         // groups of waves sharing token tiles
  constexpr int kLoads = 16 / RT;                // 16-byte loads per lane per tile and wave
  constexpr int kBufs = RT == 1 ? 1 : 2;         // LDS tiles per team
  static_assert(kTeams * kBufs * 2 * kAttTileBytes == kAttLds, "LDS tiles");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int row16 = lane & 15, grp = lane >> 4;
  const int team = wave % kTeams, rtw = wave / kTeams;  // token team, row tile of this wave
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int ts = split * a.split_len;
  const int te = min(ts + a.split_len, a.T);
  const int n_tiles = ts < te ? (te - ts + kAttTile - 1) / kAttTile : 0;
  const int team_tiles = n_tiles > team ? (n_tiles - team + kTeams - 1) / kTeams : 0;
  const int trips = n_tiles > 0 ? (n_tiles + kTeams - 1) / kTeams : 0;  // team 0's count

  // The group's query rows r = i * G + qh (zero past R) go to LDS once, in
  // the same swizzled layout as the tiles; the B operand of S^T is read from
  // there per tile.
  char* qlds = reinterpret_cast<char*>(att_lds) + kAttLds;
  for (int x = tid; x < 16 * RT * 16; x += kAttThreads) {
    const int r = x >> 4, u = x & 15;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (r < a.R) {
      const int i = r / a.G, qh = r - i * a.G;
      v = *reinterpret_cast<const u32x4*>(
          a.q + ((size_t)(b * a.K1 + i) * a.H + kvh * a.G + qh) * kAttD + u * 8);
    }
    *reinterpret_cast<u32x4*>(qlds + r * kAttRowBytes + ((u ^ (r & 7)) << 4)) = v;
  }
  __syncthreads();
  const int my_row = rtw * 16 + row16;  // this lane's query row
  const int limit = my_row < a.R ? a.T - a.K1 + my_row / a.G : a.T - 1;  // last visible key

  char* team_lds = reinterpret_cast<char*>(att_lds) + team * kBufs * 2 * kAttTileBytes;
  const size_t head_stride = (size_t)a.Hkv * kAttD;  // elements per token
  const uint16_t* kbase = a.k + (size_t)b * a.T * head_stride + (size_t)kvh * kAttD;
  const uint16_t* vbase = a.v + (size_t)b * a.T * head_stride + (size_t)kvh * kAttD;

  // Tile j of a team covers tokens ts + (team + kTeams j) * 32 + 0..31. Its
  // 16 load instructions (8 of keys, 8 of values; 4 whole token rows each)
  // are split over the team's waves. Tiles past the team's last one, and
  // tokens past T, load clamped valid rows that are never used.
  u32x4 regs[kLoads];
  auto load = [&](int j) __attribute__((always_inline)) {
    const int jc = team_tiles > 0 ? min(j, team_tiles - 1) : 0;
    const int t0 = ts + (team + kTeams * jc) * kAttTile;
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int ni = rtw * kLoads + n;  // instruction of the tile: 0..7 keys, 8..15 values
      const int t = min(t0 + 4 * (ni & 7) + grp, a.T - 1);
      const uint16_t* base = ni < 8 ? kbase : vbase;
      regs[n] = __builtin_nontemporal_load(
          (const SPECV_ATT_GLOBAL u32x4*)(base + (size_t)t * head_stride) + row16);
    }
  };
  // 16-byte unit u of token t sits at t * 256 + ((u ^ (t & 7)) * 16); the
  // values follow the keys
  auto store_lds = [&](char* tile) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < kLoads; ++n) {
      const int ni = rtw * kLoads + n;
      const int t = 4 * (ni & 7) + grp;
      *reinterpret_cast<u32x4*>(tile + (ni < 8 ? 0 : kAttTileBytes) + t * kAttRowBytes +
                                ((row16 ^ (t & 7)) << 4)) = regs[n];
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int j, const char* tile) __attribute__((always_inline)) {
    const int t0 = ts + (team + kTeams * j) * kAttTile;
    // S^T for tokens t0 + tt * 16 + 4 grp + e and this lane's query row
    f32x4 s[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int t = tt * 16 + row16;
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const int u = ds * 4 + grp;
        const u32x4 kv =
            *reinterpret_cast<const u32x4*>(tile + t * kAttRowBytes + ((u ^ (t & 7)) << 4));
        const u32x4 qv = *reinterpret_cast<const u32x4*>(qlds + my_row * kAttRowBytes +
                                                         ((u ^ (my_row & 7)) << 4));
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, kv), __builtin_bit_cast(bf16x8, qv), s[tt], 0, 0, 0);
      }
    }
    // masked, scaled scores; running max and sum of the row
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ta = t0 + tt * 16 + 4 * grp + e;
        const bool vis = ta < te && ta <= limit;
        s[tt][e] = vis ? s[tt][e] * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[tt][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    float p[8];
    float sum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = bf16_round(__builtin_amdgcn_exp2f(s[tt][e] - m_use));
        p[tt * 4 + e] = pv;
        sum += pv;
      }
    sum += __shfl_xor(sum, 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    l_run = l_run * corr + sum;
    // slot order of the P operand: tokens 4 grp + 0..3, then 16 + 4 grp + 0..3
    const u32x4 pf{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                   pack_bf16x2(p[6], p[7])};
    // O^T[d][r] = corr * O^T + sum over the tile's tokens of V[t][d] P[r][t]
    const char* vt_lds = tile + kAttTileBytes;
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
            vt_lds + ta * kAttRowBytes + ((u ^ (ta & 7)) << 4) + w * 2);
        const uint16_t vb = *reinterpret_cast<const uint16_t*>(
            vt_lds + tb * kAttRowBytes + ((u ^ (tb & 7)) << 4) + w * 2);
        h[sl >> 1] = (uint32_t)va | ((uint32_t)vb << 16);
      }
      const u32x4 vt{h[0], h[1], h[2], h[3]};
      f32x4 c = acc_o[dt];
      c[0] *= corr;
      c[1] *= corr;
      c[2] *= corr;
      c[3] *= corr;
      acc_o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, vt), __builtin_bit_cast(bf16x8, pf), c, 0, 0, 0);
    }
  };

  // Loads are issued on every path (clamped), so the compiler's waits on
  // them are exact; one tile of loads is in flight while a tile is computed.
  load(0);
  if constexpr (RT == 1) {
    // a wave's LDS accesses run in order: no barrier between its own tiles
    for (int j = 0; j < team_tiles; ++j) {
      store_lds(team_lds);
      load(j + 1);
      compute(j, team_lds);
    }
  } else {
    // the team's two waves fill one tile together: a barrier before it is
    // read; alternate buffers make a second barrier unnecessary (a buffer is
    // refilled two steps later, after every wave passed the barrier between)
    for (int j = 0; j < trips; ++j) {
      char* tile = team_lds + (j & 1) * 2 * kAttTileBytes;
      store_lds(tile);
      load(j + 1);
      __syncthreads();
      if (j < team_tiles) compute(j, tile);
    }
  }

  // ---- merge the waves of each row tile (fixed order), then store or write
  // the split's partial
  __builtin_amdgcn_s_waitcnt(0);  // the unused loads past the last tile have landed
  __syncthreads();  // every wave is done with its tiles; LDS is reused below
  float* wm = reinterpret_cast<float*>(att_lds);  // [wave][16]
  float* wlsum = wm + kAttWaves * 16;              // [wave][16]
  float* wo = wlsum + kAttWaves * 16;              // [wave][16][D]
  if (grp == 0) {
    wm[wave * 16 + row16] = m_run;
    wlsum[wave * 16 + row16] = l_run;
  }
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      wo[(wave * 16 + row16) * kAttD + dt * 16 + 4 * grp + e] = acc_o[dt][e];
  __syncthreads();
  for (int x = tid; x < a.R * kAttD; x += kAttThreads) {
    const int r = x / kAttD, d = x - r * kAttD;
    const int w0 = (r >> 4) * kTeams, rl = r & 15;  // waves of row tile r / 16: w0 .. w0 + kTeams - 1
    float m = -INFINITY;
#pragma unroll
    for (int t = 0; t < kTeams; ++t) m = fmaxf(m, wm[(w0 + t) * 16 + rl]);
    const float m_use = m == -INFINITY ? 0.f : m;
    float o = 0.f, l = 0.f;
#pragma unroll
    for (int t = 0; t < kTeams; ++t) {
      const float f = __builtin_amdgcn_exp2f(wm[(w0 + t) * 16 + rl] - m_use);
      o += wo[((w0 + t) * 16 + rl) * kAttD + d] * f;
      l += wlsum[(w0 + t) * 16 + rl] * f;
    }
    const int i = r / a.G, h = kvh * a.G + (r - i * a.G);
    if (a.part) {
      float* pr = a.part +
                  ((((size_t)b * a.Hkv + kvh) * a.n_split + split) * a.R + r) * kAttPartStride;
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

// Merge the splits of one (sequence, kv head, query row) in split order. The
// splits' maxima and sums are read in parallel into LDS first; each thread
// then merges one output column.
constexpr int kAttMaxSplit = 4096;
__global__ __launch_bounds__(kAttD) void verify_attention_merge_kernel(AttnArgs a) {
  __shared__ float sm[kAttMaxSplit], sl[kAttMaxSplit];
  const int r = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z, d = threadIdx.x;
  const float* base = a.part + (((size_t)b * a.Hkv + kvh) * a.n_split * a.R + r) * kAttPartStride;
  const size_t step = (size_t)a.R * kAttPartStride;
  for (int s = d; s < a.n_split; s += kAttD) {
    sm[s] = base[s * step + kAttD];
    sl[s] = base[s * step + kAttD + 1];
  }
  __syncthreads();
  float m = -INFINITY;
  for (int s = 0; s < a.n_split; ++s) m = fmaxf(m, sm[s]);
  const float m_use = m == -INFINITY ? 0.f : m;
  float o = 0.f, l = 0.f;
#pragma unroll 8
  for (int s = 0; s < a.n_split; ++s) {
    const float f = __builtin_amdgcn_exp2f(sm[s] - m_use);
    o += base[s * step + d] * f;
    l += sl[s] * f;
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
  return max(1, min(min(want, max_split), kAttMaxSplit));
}

size_t attention_workspace_bytes(int B, int K1, int H, int Hkv, int n_split) {
  if (n_split <= 1) return 0;
  const int R = K1 * (H / Hkv);
  return (size_t)B * Hkv * n_split * R * kAttPartStride * sizeof(float);
}

template <int RT>
static hipError_t launch_att(const AttnArgs& a, hipStream_t s) {
  static_assert((2 * kAttWaves * 16 + kAttWaves * 16 * kAttD) * 4 <= kAttLds,
                "the merge buffers fit in the tile region");
  const size_t lds = kAttLds + kAttQBytes;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(&verify_attention_kernel<RT>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((verify_attention_kernel<RT>), dim3(a.n_split, a.Hkv, a.B),
                     dim3(kAttThreads), lds, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split <= 1) return e;
  hipLaunchKernelGGL(verify_attention_merge_kernel, dim3(a.R, a.Hkv, a.B), dim3(kAttD), 0, s, a);
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
