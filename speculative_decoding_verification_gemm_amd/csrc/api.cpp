// C ABI of libspecverify: argument validation, device check and dispatch.
// Every argument is checked before the first HIP call, so a failing call
// launches nothing and the checks run on hosts without a GPU.

#include <hip/hip_runtime.h>
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <stddef.h>

#include <atomic>

#include "../../include/spec_verify.h"
#include "chain_sync.h"
#include "internal.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Per-device answer to "is this a gfx950?" (0 unknown, 1 yes, -1 no) and
// its compute-unit count.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

int check_device(int* cus = nullptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_ERR_UNSUPPORTED, "device index %d", dev);
  int ok = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (ok == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(SPEC_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    g_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                     std::memory_order_relaxed);
    ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_arch_ok[dev].store(ok, std::memory_order_relaxed);
  }
  if (ok < 0) return fail(SPEC_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  if (cus) *cus = g_cus[dev].load(std::memory_order_relaxed);
  return SPEC_OK;
}

// Resident workgroups per CU for the streaming kernel: the occupancy limit,
// capped at 2 (measured best for the Llama-shaped linears). Diagnostic
// builds (SPECV_DIAGNOSTICS) let SPECV_STREAM_WGS_PER_CU override the cap.
std::atomic<int> g_stream_occ[2][17];
int stream_wgs_per_cu(int M, bool w8 = false) {
  int occ = g_stream_occ[w8][M].load(std::memory_order_relaxed);
  if (occ == 0) {
    occ = specv::stream_max_wgs_per_cu(M, w8);
    g_stream_occ[w8][M].store(occ, std::memory_order_relaxed);
  }
  int cap = 2;
#if defined(SPECV_DIAGNOSTICS)
  if (const char* env = getenv("SPECV_STREAM_WGS_PER_CU")) {
    const int v = atoi(env);
    if (v > 0) cap = v;
  }
#endif
  return occ < cap ? occ : cap;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return SPEC_OK;
}

constexpr int kMaxM = 65536;
constexpr int kMaxDin = 1 << 20;
constexpr int kMaxDout = 1 << 24;
constexpr int kMaxRows = 1 << 24;
constexpr int kMaxV = 1 << 26;
constexpr int kMaxB = 1 << 20;
constexpr int kMaxK = 64;
// fused-stage grid bound: rows * chunks of 4096 entries
constexpr size_t kMaxVerifyBlocks = (size_t)1 << 22;

int check_gemm_args(const uint16_t* x, const uint16_t* w, const void* y, int y_dtype, int M,
                    int d_in, int d_out) {
  if (!x || !w || !y) return fail(SPEC_ERR_INVALID_ARGUMENT, "null pointer (x, w or y)");
  if (y_dtype != SPEC_F32 && y_dtype != SPEC_BF16)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "y_dtype %d is neither SPEC_F32 nor SPEC_BF16", y_dtype);
  if (M < 1 || M > kMaxM) return fail(SPEC_ERR_INVALID_ARGUMENT, "M=%d outside [1, %d]", M, kMaxM);
  if (d_in < 8 || d_in > kMaxDin || d_in % 8 != 0)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "d_in=%d must be a multiple of 8 in [8, %d]", d_in,
                kMaxDin);
  if (d_out < 1 || d_out > kMaxDout)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "d_out=%d outside [1, %d]", d_out, kMaxDout);
  if (!aligned(x, 16) || !aligned(w, 16))
    return fail(SPEC_ERR_ALIGNMENT, "x and w must be 16-byte aligned");
  if (!aligned(y, y_dtype == SPEC_F32 ? 4 : 2))
    return fail(SPEC_ERR_ALIGNMENT, "y is not aligned to its element size");
  return SPEC_OK;
}

// FP8 weights: as check_gemm_args, plus the scale vector and d_in a multiple
// of 16 (one 16-byte load holds 16 weights); above the streaming kernel's
// positions (M > 16) the tile kernel needs d_in a multiple of 64.
int check_gemm_w8_args(const uint16_t* x, const uint8_t* w, const float* w_scale, const void* y,
                       int y_dtype, int M, int d_in, int d_out) {
  if (!w_scale) return fail(SPEC_ERR_INVALID_ARGUMENT, "null w_scale");
  int rc = check_gemm_args(x, reinterpret_cast<const uint16_t*>(w), y, y_dtype, M, d_in, d_out);
  if (rc != SPEC_OK) return rc;
  if (d_in % 16 != 0)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "d_in=%d must be a multiple of 16 for FP8 weights",
                d_in);
  if (!aligned(w_scale, 4)) return fail(SPEC_ERR_ALIGNMENT, "w_scale is not 4-byte aligned");
  if (M > specv::kMaxStreamM && d_in % 64 != 0)
    return fail(SPEC_ERR_UNSUPPORTED,
                "FP8 weights with M > %d need d_in a multiple of 64 (got M=%d, d_in=%d)",
                specv::kMaxStreamM, M, d_in);
  return SPEC_OK;
}

int check_bkv(int B, int K, int V) {
  if (B < 1 || B > kMaxB) return fail(SPEC_ERR_INVALID_ARGUMENT, "B=%d outside [1, %d]", B, kMaxB);
  if (K < 1 || K > kMaxK) return fail(SPEC_ERR_INVALID_ARGUMENT, "K=%d outside [1, %d]", K, kMaxK);
  if (V < 1 || V > kMaxV) return fail(SPEC_ERR_INVALID_ARGUMENT, "V=%d outside [1, %d]", V, kMaxV);
  return SPEC_OK;
}

// Which kernel a single launch uses when d_in is a multiple of 64 (other
// d_in stream up to kMaxStreamM positions). The streaming kernel's dot
// products grow with M while the tile kernel's MFMA work does not, and the
// streaming kernel is at its best on long linears, where every CU walks many
// row blocks. Measured on the Llama-3.1-8B linears: from 9 positions up the
// tile kernel is faster on every linear (the whole stack at M = 10: 3.26
// against 4.60 ms; at 16: 3.34 against 6.14 ms); at 1 to 8 positions it is
// faster on QKV, O and down (at M = 5: 13.4 against 18.9 us, 10.2 against
// 14.9, 26.2 against 28.5) and slower on gate/up and the lm-head (47.1
// against 45.0 us, 179 against 164), which hold 2^26 weights or more.
constexpr int kMaxStreamGemmM = 8;
constexpr long long kStreamMinWeights = 1LL << 26;
bool use_stream(int M, int d_in, int d_out) {
  if (M > specv::kMaxStreamM) return false;
  if (d_in % 64 != 0) return true;
  return M <= kMaxStreamGemmM && (long long)d_in * d_out >= kStreamMinWeights;
}

int run_gemm(const uint16_t* x, const uint16_t* w, void* y, bool out_bf16, int M, int d_in,
             int d_out, int cus, hipStream_t s) {
  hipError_t e;
  if (use_stream(M, d_in, d_out))
    e = specv::launch_gemm_stream(x, w, nullptr, y, out_bf16, false, M, d_in, d_out,
                                  cus * stream_wgs_per_cu(M), s);
  else if (d_in % 64 == 0 || M > specv::kMaxSkinnyM)
    // the pipelined tile kernel when d_in is a multiple of 64 (measured
    // faster than the weight-streaming MFMA kernel at every M from 17 up),
    // else the register-staged tile kernel
    e = specv::launch_gemm_mfma(x, w, y, out_bf16, M, d_in, d_out, s);
  else
    e = specv::launch_gemm_skinny(x, w, y, out_bf16, M, d_in, d_out, s);
  return launched(e, "spec_verify_gemm");
}

constexpr int kMaxChain = 4096;

size_t chain_counts_offset() { return sizeof(specv::ChainSync); }
size_t chain_desc_offset(int n) {
  return (chain_counts_offset() + specv::chain_counts_bytes(n) + 63) & ~(size_t)63;
}
size_t chain_bytes(int n) {
  return (chain_desc_offset(n) + (size_t)n * sizeof(specv::StreamLinear) + 255) & ~(size_t)255;
}

// Validates the n descriptors (fill(i, &desc) checks linear i and writes its
// internal descriptor), then uploads header, zeroed counters and
// descriptors. The header's magic records the weight format.
template <class Fill>
int chain_prepare(int n, int M, void* workspace, size_t workspace_bytes, bool w8, Fill&& fill) {
  if (!workspace) return fail(SPEC_ERR_INVALID_ARGUMENT, "null workspace");
  if (n < 1 || n > kMaxChain)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "n=%d outside [1, %d]", n, kMaxChain);
  if (M < 1 || M > specv::kMaxStreamM)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "chain M=%d outside [1, %d]", M, specv::kMaxStreamM);
  const size_t bytes = chain_bytes(n);
  char* img = static_cast<char*>(calloc(1, bytes));
  if (!img) return fail(SPEC_ERR_HIP, "host staging allocation failed");
  specv::StreamLinear* descs = reinterpret_cast<specv::StreamLinear*>(img + chain_desc_offset(n));
  for (int i = 0; i < n; ++i) {
    int rc = fill(i, &descs[i]);
    if (rc != SPEC_OK) {
      free(img);
      char msg[512];
      snprintf(msg, sizeof(msg), "linear %d: %s", i, g_err);
      return fail(rc, "%s", msg);
    }
  }
  if (workspace_bytes < bytes) {
    free(img);
    return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, bytes);
  }
  if (!aligned(workspace, 256)) {
    free(img);
    return fail(SPEC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  int rc = SPEC_OK;
  int cus = 0;
  if ((rc = check_device(&cus)) != SPEC_OK) {
    free(img);
    return rc;
  }
  specv::ChainSync hdr{};
  hdr.magic = w8 ? specv::kChainMagicW8 : specv::kChainMagic;
  hdr.n = n;
  hdr.M = M;
  hdr.grid = cus * stream_wgs_per_cu(M, w8);
  hdr.spin_limit = specv::kChainSpinLimit;
#if defined(SPECV_DIAGNOSTICS)
  // Diagnostics: SPECV_CHAIN_TRACE=<device address of n * grid * 4 uint64>
  // records, per linear and workgroup, the wall clock (100 MHz ticks) at
  // arrival, at the end of the wait for the previous linear, and when the
  // first activation chunk is staged, and when the last output stores of
  // the linear have been issued.
  // The address must lie in one device allocation that holds
  // (n + 1) * grid * 4 records; anything else is rejected.
  if (const char* env = getenv("SPECV_CHAIN_TRACE")) {
    void* const v = reinterpret_cast<void*>(strtoull(env, nullptr, 0));
    const size_t need = (size_t)(n + 1) * hdr.grid * 4 * sizeof(uint64_t);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, v) != hipSuccess ||
        static_cast<char*>(v) + need > static_cast<char*>(base) + size) {
      free(img);
      (void)hipGetLastError();
      return fail(SPEC_ERR_INVALID_ARGUMENT,
                  "SPECV_CHAIN_TRACE is not a device buffer of %zu bytes", need);
    }
    hdr.trace = static_cast<unsigned long long*>(v);
  }
#endif
  memcpy(img, &hdr, sizeof(hdr));
  hipError_t e = hipMemcpy(workspace, img, bytes, hipMemcpyHostToDevice);
  free(img);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "chain upload: %s", hipGetErrorString(e));
  return SPEC_OK;
}

int chain_run(int n, int M, void* workspace, bool w8, void* stream) {
  if (!workspace) return fail(SPEC_ERR_INVALID_ARGUMENT, "null workspace");
  if (n < 1 || n > kMaxChain)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "n=%d outside [1, %d]", n, kMaxChain);
  if (M < 1 || M > specv::kMaxStreamM)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "chain M=%d outside [1, %d]", M, specv::kMaxStreamM);
  if (!aligned(workspace, 256)) return fail(SPEC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc != SPEC_OK) return rc;
  char* base = static_cast<char*>(workspace);
  return launched(specv::launch_gemm_chain(
                      reinterpret_cast<const specv::StreamLinear*>(base + chain_desc_offset(n)), n,
                      reinterpret_cast<specv::ChainSync*>(base), M, w8,
                      cus * stream_wgs_per_cu(M, w8), static_cast<hipStream_t>(stream)),
                  w8 ? "spec_verify_gemm_chain_w8" : "spec_verify_gemm_chain");
}

}  // namespace

extern "C" {

int spec_abi_version(void) { return SPEC_ABI_VERSION; }

const char* spec_status_string(int status) {
  switch (status) {
    case SPEC_OK: return "SPEC_OK";
    case SPEC_ERR_INVALID_ARGUMENT: return "SPEC_ERR_INVALID_ARGUMENT";
    case SPEC_ERR_ALIGNMENT: return "SPEC_ERR_ALIGNMENT";
    case SPEC_ERR_UNSUPPORTED: return "SPEC_ERR_UNSUPPORTED";
    case SPEC_ERR_WORKSPACE: return "SPEC_ERR_WORKSPACE";
    case SPEC_ERR_HIP: return "SPEC_ERR_HIP";
    default: return "SPEC_ERR_UNKNOWN";
  }
}

const char* spec_last_error(void) { return g_err; }

int spec_verify_gemm(const uint16_t* x, const uint16_t* w, void* y, int y_dtype, int M, int d_in,
                     int d_out, void* stream) {
  clear_error();
  int rc = check_gemm_args(x, w, y, y_dtype, M, d_in, d_out);
  if (rc != SPEC_OK) return rc;
  int cus = 0;
  if ((rc = check_device(&cus)) != SPEC_OK) return rc;
  return run_gemm(x, w, y, y_dtype == SPEC_BF16, M, d_in, d_out, cus,
                  static_cast<hipStream_t>(stream));
}

// The tile path's reduction split applies where the per-linear call would
// run the pipelined tile kernel (d_in a multiple of 64, no streaming).
size_t split_bytes(int M, int d_in, int d_out) {
  if (M < 1 || M > kMaxM || d_in < 64 || d_in > kMaxDin || d_out < 1 || d_out > kMaxDout)
    return 0;
  if (d_in % 64 != 0 || use_stream(M, d_in, d_out)) return 0;
  return specv::gemm_split_workspace_bytes(M, d_in, d_out);
}

size_t spec_verify_gemm_workspace_bytes(int M, int d_in, int d_out) {
  return split_bytes(M, d_in, d_out);
}

int spec_verify_gemm_ws(const uint16_t* x, const uint16_t* w, void* y, int y_dtype, int M,
                        int d_in, int d_out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  clear_error();
  int rc = check_gemm_args(x, w, y, y_dtype, M, d_in, d_out);
  if (rc != SPEC_OK) return rc;
  const size_t need = split_bytes(M, d_in, d_out);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SPEC_ERR_WORKSPACE,
                "workspace of %zu bytes (%s) is smaller than the %zu bytes M=%d, d_in=%d, "
                "d_out=%d needs",
                workspace_bytes, workspace ? "non-null" : "null", need, M, d_in, d_out);
  if (need > 0 && !aligned(workspace, 16))
    return fail(SPEC_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  int cus = 0;
  if ((rc = check_device(&cus)) != SPEC_OK) return rc;
  if (need == 0)
    return run_gemm(x, w, y, y_dtype == SPEC_BF16, M, d_in, d_out, cus,
                    static_cast<hipStream_t>(stream));
  return launched(specv::launch_gemm_split(x, w, y, y_dtype == SPEC_BF16, M, d_in, d_out,
                                           workspace, workspace_bytes,
                                           static_cast<hipStream_t>(stream)),
                  "spec_verify_gemm_ws");
}

size_t spec_chain_workspace_bytes(int n) {
  if (n < 1 || n > kMaxChain) return 0;
  return chain_bytes(n);
}

int spec_chain_prepare(const spec_linear* linears, int n, int M, void* workspace,
                       size_t workspace_bytes) {
  clear_error();
  if (!linears) return fail(SPEC_ERR_INVALID_ARGUMENT, "null linears");
  return chain_prepare(n, M, workspace, workspace_bytes, false,
                       [&](int i, specv::StreamLinear* d) {
                         const spec_linear& l = linears[i];
                         int rc = check_gemm_args(l.x, l.w, l.y, l.y_dtype, M, l.d_in, l.d_out);
                         if (rc == SPEC_OK && l.reserved != 0)
                           rc = fail(SPEC_ERR_INVALID_ARGUMENT, "reserved != 0");
                         *d = specv::StreamLinear{l.x, l.w, nullptr, l.y, l.d_in, l.d_out,
                                                  l.y_dtype == SPEC_BF16 ? 1 : 0, 0};
                         return rc;
                       });
}

int spec_chain_prepare_w8(const spec_linear_w8* linears, int n, int M, void* workspace,
                          size_t workspace_bytes) {
  clear_error();
  if (!linears) return fail(SPEC_ERR_INVALID_ARGUMENT, "null linears");
  return chain_prepare(n, M, workspace, workspace_bytes, true,
                       [&](int i, specv::StreamLinear* d) {
                         const spec_linear_w8& l = linears[i];
                         int rc = check_gemm_w8_args(l.x, l.w, l.w_scale, l.y, l.y_dtype, M,
                                                     l.d_in, l.d_out);
                         if (rc == SPEC_OK && l.reserved != 0)
                           rc = fail(SPEC_ERR_INVALID_ARGUMENT, "reserved != 0");
                         *d = specv::StreamLinear{l.x, l.w, l.w_scale, l.y, l.d_in, l.d_out,
                                                  l.y_dtype == SPEC_BF16 ? 1 : 0, 0};
                         return rc;
                       });
}

int spec_verify_gemm_chain(int n, int M, void* workspace, void* stream) {
  clear_error();
  return chain_run(n, M, workspace, false, stream);
}

int spec_verify_gemm_chain_w8(int n, int M, void* workspace, void* stream) {
  clear_error();
  return chain_run(n, M, workspace, true, stream);
}

}  // extern "C"

namespace {
// Shape checks shared by the attention entry points (SPEC_OK or an error).
int check_attention_shape(int B, int K, int T, int H, int Hkv, int D) {
  if (B < 1 || B > 65535) return fail(SPEC_ERR_INVALID_ARGUMENT, "B=%d outside [1, 65535]", B);
  if (K < 0 || K > kMaxK) return fail(SPEC_ERR_INVALID_ARGUMENT, "K=%d outside [0, %d]", K, kMaxK);
  if (T < K + 1 || T > (1 << 24))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "T=%d outside [K+1, 2^24]", T);
  if (H < 1 || Hkv < 1 || Hkv > 65535 || H % Hkv != 0)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "n_heads=%d, n_kv_heads=%d: kv heads must divide heads",
                H, Hkv);
  if (D != 128) return fail(SPEC_ERR_UNSUPPORTED, "head_dim=%d (implemented: 128)", D);
  if ((long long)(K + 1) * (H / Hkv) > 32)
    return fail(SPEC_ERR_UNSUPPORTED, "(K+1) * n_heads / n_kv_heads = %lld query rows > 32",
                (long long)(K + 1) * (H / Hkv));
  return SPEC_OK;
}
}  // namespace

extern "C" {

size_t spec_verify_attention_workspace_bytes(int B, int K, int T, int n_heads, int n_kv_heads,
                                             int head_dim) {
  if (check_attention_shape(B, K, T, n_heads, n_kv_heads, head_dim) != SPEC_OK) return 0;
  const size_t n = specv::attention_workspace_bytes(
      B, K + 1, n_heads, n_kv_heads, specv::attention_splits(B, K + 1, n_heads, n_kv_heads, T));
  return (n + 255) & ~(size_t)255;
}

int spec_verify_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                          void* out, int out_dtype, int B, int K, int T, int n_heads,
                          int n_kv_heads, int head_dim, float scale, void* workspace,
                          size_t workspace_bytes, void* stream) {
  clear_error();
  if (!q || !k_cache || !v_cache || !out)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "null pointer (q, k_cache, v_cache or out)");
  if (out_dtype != SPEC_F32 && out_dtype != SPEC_BF16)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "out_dtype %d is neither SPEC_F32 nor SPEC_BF16",
                out_dtype);
  int rc = check_attention_shape(B, K, T, n_heads, n_kv_heads, head_dim);
  if (rc != SPEC_OK) return rc;
  if (!std::isfinite(scale)) return fail(SPEC_ERR_INVALID_ARGUMENT, "scale is not finite");
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
    return fail(SPEC_ERR_ALIGNMENT, "q, k_cache and v_cache must be 16-byte aligned");
  if (!aligned(out, out_dtype == SPEC_F32 ? 4 : 2))
    return fail(SPEC_ERR_ALIGNMENT, "out is not aligned to its element size");
  const size_t need = spec_verify_attention_workspace_bytes(B, K, T, n_heads, n_kv_heads, head_dim);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(SPEC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  if ((rc = check_device()) != SPEC_OK) return rc;
  return launched(specv::launch_verify_attention(q, k_cache, v_cache, out, out_dtype == SPEC_BF16,
                                                 B, K + 1, T, n_heads, n_kv_heads, scale,
                                                 workspace, static_cast<hipStream_t>(stream)),
                  "spec_verify_attention");
}

int spec_verify_gemm_w8(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                        int y_dtype, int M, int d_in, int d_out, void* stream) {
  clear_error();
  int rc = check_gemm_w8_args(x, w, w_scale, y, y_dtype, M, d_in, d_out);
  if (rc != SPEC_OK) return rc;
  int cus = 0;
  if ((rc = check_device(&cus)) != SPEC_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (M > specv::kMaxStreamM)  // a dense contraction: the MFMA tile kernel
    return launched(specv::launch_gemm_tile_w8(x, w, w_scale, y, y_dtype == SPEC_BF16, M, d_in,
                                               d_out, s),
                    "spec_verify_gemm_w8");
  return launched(specv::launch_gemm_stream(x, w, w_scale, y, y_dtype == SPEC_BF16, true, M, d_in,
                                            d_out, cus * stream_wgs_per_cu(M, true), s),
                  "spec_verify_gemm_w8");
}

// FP8 weights: the split applies to the tile kernel (M above the streaming
// kernel's positions; d_in a multiple of 64 is then required anyway).
size_t split_bytes_w8(int M, int d_in, int d_out) {
  if (M <= specv::kMaxStreamM || M > kMaxM || d_in < 64 || d_in > kMaxDin || d_in % 64 != 0 ||
      d_out < 1 || d_out > kMaxDout)
    return 0;
  return specv::gemm_split_workspace_bytes_w8(M, d_in, d_out);
}

size_t spec_verify_gemm_w8_workspace_bytes(int M, int d_in, int d_out) {
  return split_bytes_w8(M, d_in, d_out);
}

int spec_verify_gemm_w8_ws(const uint16_t* x, const uint8_t* w, const float* w_scale, void* y,
                           int y_dtype, int M, int d_in, int d_out, void* workspace,
                           size_t workspace_bytes, void* stream) {
  clear_error();
  int rc = check_gemm_w8_args(x, w, w_scale, y, y_dtype, M, d_in, d_out);
  if (rc != SPEC_OK) return rc;
  const size_t need = split_bytes_w8(M, d_in, d_out);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(SPEC_ERR_WORKSPACE,
                "workspace of %zu bytes (%s) is smaller than the %zu bytes M=%d, d_in=%d, "
                "d_out=%d needs",
                workspace_bytes, workspace ? "non-null" : "null", need, M, d_in, d_out);
  if (need > 0 && !aligned(workspace, 16))
    return fail(SPEC_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  if (need == 0) return spec_verify_gemm_w8(x, w, w_scale, y, y_dtype, M, d_in, d_out, stream);
  int cus = 0;
  if ((rc = check_device(&cus)) != SPEC_OK) return rc;
  return launched(specv::launch_gemm_split_w8(x, w, w_scale, y, y_dtype == SPEC_BF16, M, d_in,
                                              d_out, workspace, workspace_bytes,
                                              static_cast<hipStream_t>(stream)),
                  "spec_verify_gemm_w8_ws");
}

int spec_probe_read(const void* buf, size_t bytes, int loads_per_lane, int wgs_per_cu,
                    void* sink, void* stream) {
  clear_error();
  if (!buf || !sink) return fail(SPEC_ERR_INVALID_ARGUMENT, "null buf or sink");
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "loads_per_lane=%d (1, 2, 4 or 8)", loads_per_lane);
  if (wgs_per_cu < 1 || wgs_per_cu > 4)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "wgs_per_cu=%d outside [1, 4]", wgs_per_cu);
  if (bytes < 16 || bytes % 16 != 0)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "bytes=%zu must be a positive multiple of 16", bytes);
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(SPEC_ERR_ALIGNMENT, "buf must be 16-byte and sink 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc != SPEC_OK) return rc;
  return launched(specv::launch_probe_read(buf, bytes, loads_per_lane,
                                           static_cast<unsigned*>(sink), wgs_per_cu * cus,
                                           static_cast<hipStream_t>(stream)),
                  "spec_probe_read");
}

int spec_probe_read_lds(const void* buf, size_t bytes, int loads_per_lane, void* sink,
                        void* stream) {
  clear_error();
  if (!buf || !sink) return fail(SPEC_ERR_INVALID_ARGUMENT, "null buf or sink");
  if (loads_per_lane != 1 && loads_per_lane != 2 && loads_per_lane != 4 && loads_per_lane != 8)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "loads_per_lane=%d (1, 2, 4 or 8)", loads_per_lane);
  if (bytes < 16 || bytes % 16 != 0)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "bytes=%zu must be a positive multiple of 16", bytes);
  if (!aligned(buf, 16) || !aligned(sink, 4))
    return fail(SPEC_ERR_ALIGNMENT, "buf must be 16-byte and sink 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc != SPEC_OK) return rc;
  return launched(specv::launch_probe_read_lds(buf, bytes, loads_per_lane,
                                               static_cast<unsigned*>(sink), cus,
                                               static_cast<hipStream_t>(stream)),
                  "spec_probe_read_lds");
}

int spec_probe_mfma(int shape, int iters, void* sink, double* flops, void* stream) {
  clear_error();
  if (shape != 16 && shape != 32)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "shape=%d (16 or 32)", shape);
  if (iters < 1 || iters > (1 << 24))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "iters=%d outside [1, 2^24]", iters);
  if (!sink || !flops) return fail(SPEC_ERR_INVALID_ARGUMENT, "null sink or flops");
  if (!aligned(sink, 4)) return fail(SPEC_ERR_ALIGNMENT, "sink must be 4-byte aligned");
  int cus = 0;
  int rc = check_device(&cus);
  if (rc != SPEC_OK) return rc;
  const int grid = 2 * cus;  // two workgroups of four waves: two waves per SIMD
  // per wave and iteration: 8 x 16x16x32 or 4 x 32x32x16, 131072 FLOPs either way
  *flops = (double)grid * 4 * iters * 131072.0;
  return launched(specv::launch_probe_mfma(shape, iters, static_cast<unsigned*>(sink), grid,
                                           static_cast<hipStream_t>(stream)),
                  "spec_probe_mfma");
}

int spec_chain_reset(void* workspace, unsigned generation) {
  clear_error();
  if (!workspace) return fail(SPEC_ERR_INVALID_ARGUMENT, "null workspace");
  if (!aligned(workspace, 256)) return fail(SPEC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  int rc = check_device();
  if (rc != SPEC_OK) return rc;
  specv::ChainSync hdr;
  hipError_t e = hipMemcpy(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "chain header read: %s", hipGetErrorString(e));
  if ((hdr.magic != specv::kChainMagic && hdr.magic != specv::kChainMagicW8) || hdr.n < 1 ||
      hdr.n > kMaxChain || hdr.grid < 1)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "workspace holds no prepared chain");
  // Every counter as it stands after `generation` complete launches (the
  // invariants of chain_sync.h), and the error word cleared.
  const int n = hdr.n, G = hdr.grid;
  const int n_groups = G < specv::kArriveGroups ? G : specv::kArriveGroups;
  const size_t words = specv::chain_counts_bytes(n) / 4;
  unsigned* img = static_cast<unsigned*>(calloc(words, sizeof(unsigned)));
  if (!img) return fail(SPEC_ERR_HIP, "host staging allocation failed");
  const size_t rel = specv::chain_release_offset(n);
  for (int l = 0; l < n; ++l) {
    img[l] = generation * (unsigned)n_groups;
    for (int x = 0; x < specv::kReleaseLanes; ++x)
      img[rel + ((size_t)l * specv::kBarrierLines + x) * 16] = specv::chain_target(generation, G);
    for (int g = 0; g < specv::kArriveGroups; ++g)
      img[rel + ((size_t)l * specv::kBarrierLines + specv::kReleaseLanes + g) * 16] =
          generation * specv::chain_group_size(G, g, specv::kArriveGroups);
  }
  hdr.gen = generation;
  hdr.exit_count = specv::chain_target(generation, G);
  hdr.error = 0;
  char* base = static_cast<char*>(workspace);
  e = hipMemcpy(base + chain_counts_offset(), img, words * 4, hipMemcpyHostToDevice);
  free(img);
  if (e == hipSuccess) e = hipMemcpy(base, &hdr, sizeof(hdr), hipMemcpyHostToDevice);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "chain reset: %s", hipGetErrorString(e));
  return SPEC_OK;
}

int spec_chain_error(void* workspace, int* error) {
  clear_error();
  if (!workspace || !error) return fail(SPEC_ERR_INVALID_ARGUMENT, "null workspace or error");
  if (!aligned(workspace, 256)) return fail(SPEC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  int rc = check_device();
  if (rc != SPEC_OK) return rc;
  specv::ChainSync hdr;
  hipError_t e = hipMemcpy(&hdr, workspace, sizeof(hdr), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "chain error read: %s", hipGetErrorString(e));
  *error = (int)hdr.error;
  if (hdr.error) {
    const unsigned zero = 0;
    e = hipMemcpy(static_cast<char*>(workspace) + offsetof(specv::ChainSync, error), &zero,
                  sizeof(zero), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(SPEC_ERR_HIP, "chain error clear: %s", hipGetErrorString(e));
  }
  return SPEC_OK;
}

int spec_softmax(const float* logits, int rows, int V, float* probs, float* row_max,
                 float* row_sumexp, void* stream) {
  clear_error();
  if (!logits) return fail(SPEC_ERR_INVALID_ARGUMENT, "null logits");
  if (rows < 1 || rows > kMaxRows)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "rows=%d outside [1, %d]", rows, kMaxRows);
  if (V < 1 || V > kMaxV) return fail(SPEC_ERR_INVALID_ARGUMENT, "V=%d outside [1, %d]", V, kMaxV);
  if (!aligned(logits, 4) || (probs && !aligned(probs, 4)) || (row_max && !aligned(row_max, 4)) ||
      (row_sumexp && !aligned(row_sumexp, 4)))
    return fail(SPEC_ERR_ALIGNMENT, "fp32 arrays must be 4-byte aligned");
  if (!probs && !row_max && !row_sumexp) return SPEC_OK;
  int rc = check_device();
  if (rc != SPEC_OK) return rc;
  return launched(specv::launch_softmax_rows(logits, rows, V, probs, row_max, row_sumexp,
                                             static_cast<hipStream_t>(stream)),
                  "spec_softmax");
}

int spec_accept_scan(const float* p_probs, const float* q_probs, const int32_t* draft_tokens,
                     const float* u_accept, int B, int K, int V, int32_t* n_accepted,
                     uint8_t* accept_mask, void* stream) {
  clear_error();
  if (!p_probs || !q_probs || !draft_tokens || !u_accept || !n_accepted)
    return fail(SPEC_ERR_INVALID_ARGUMENT,
                "null pointer (p_probs, q_probs, draft_tokens, u_accept or n_accepted)");
  int rc = check_bkv(B, K, V);
  if (rc != SPEC_OK) return rc;
  if (!aligned(p_probs, 4) || !aligned(q_probs, 4) || !aligned(draft_tokens, 4) ||
      !aligned(u_accept, 4) || !aligned(n_accepted, 4))
    return fail(SPEC_ERR_ALIGNMENT, "32-bit arrays must be 4-byte aligned");
  if ((rc = check_device()) != SPEC_OK) return rc;
  return launched(specv::launch_accept_probs(p_probs, q_probs, draft_tokens, u_accept, B, K, V,
                                             n_accepted, accept_mask,
                                             static_cast<hipStream_t>(stream)),
                  "spec_accept_scan");
}

int spec_residual_sample(const float* p_probs, const float* q_probs, const int32_t* n_accepted,
                         const float* u_sample, int B, int K, int V, int32_t* token,
                         uint8_t* zero_residual, void* stream) {
  clear_error();
  if (!p_probs || !q_probs || !n_accepted || !u_sample || !token)
    return fail(SPEC_ERR_INVALID_ARGUMENT,
                "null pointer (p_probs, q_probs, n_accepted, u_sample or token)");
  int rc = check_bkv(B, K, V);
  if (rc != SPEC_OK) return rc;
  if (!aligned(p_probs, 4) || !aligned(q_probs, 4) || !aligned(n_accepted, 4) ||
      !aligned(u_sample, 4) || !aligned(token, 4))
    return fail(SPEC_ERR_ALIGNMENT, "32-bit arrays must be 4-byte aligned");
  if ((rc = check_device()) != SPEC_OK) return rc;
  return launched(specv::launch_sample_probs(p_probs, q_probs, n_accepted, u_sample, B, K, V,
                                             token, zero_residual,
                                             static_cast<hipStream_t>(stream)),
                  "spec_residual_sample");
}

}  // extern "C"

namespace {

// The scratch of spec_verify_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends. Kernels receive the address that
// hipGetSymbolAddress returns on the current device (the array's name is
// only a host-side stand-in in host code); it is looked up once per device
// and kept. Every spec_verify_noalloc call on a GPU uses that GPU's copy, so
// calls that overlap on one GPU race. The sampler writes every scratch word
// it reads within the same call, so nothing needs clearing between calls.
constexpr size_t kScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
std::atomic<void*> g_scratch[kMaxDevices];

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SPEC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SPEC_ERR_UNSUPPORTED, "device index %d", dev);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SPEC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev].store(p, std::memory_order_release);  // same value if two threads race here
  }
  *out = p;
  return SPEC_OK;
}

int verify_impl(const uint16_t* hidden, const uint16_t* lm_head, int d, float* target_logits,
                const float* draft_logits, const int32_t* draft_tokens, const float* u_accept,
                const float* u_sample, int B, int K, int V, float t_target, float t_draft,
                int32_t* out_tokens, int32_t* n_emitted, void* workspace, size_t workspace_bytes,
                bool use_scratch, void* stream);

}  // namespace

extern "C" {

size_t spec_verify_workspace_bytes(int B, int K, int V) {
  if (B < 1 || B > kMaxB || K < 1 || K > kMaxK || V < 1 || V > kMaxV) return 0;
  return specv::verify_workspace_bytes(B, K, V);
}

int spec_verify(const uint16_t* hidden, const uint16_t* lm_head, int d, float* target_logits,
                const float* draft_logits, const int32_t* draft_tokens, const float* u_accept,
                const float* u_sample, int B, int K, int V, int32_t* out_tokens,
                int32_t* n_emitted, void* workspace, size_t workspace_bytes, void* stream) {
  return spec_verify_warped(hidden, lm_head, d, target_logits, draft_logits, draft_tokens, u_accept,
                            u_sample, B, K, V, 1.0f, 1.0f, out_tokens, n_emitted, workspace,
                            workspace_bytes, stream);
}

int spec_verify_warped(const uint16_t* hidden, const uint16_t* lm_head, int d,
                       float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, const float* u_accept, const float* u_sample,
                       int B, int K, int V, float t_target, float t_draft, int32_t* out_tokens,
                       int32_t* n_emitted, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return verify_impl(hidden, lm_head, d, target_logits, draft_logits, draft_tokens, u_accept,
                     u_sample, B, K, V, t_target, t_draft, out_tokens, n_emitted, workspace,
                     workspace_bytes, false, stream);
}

int spec_verify_noalloc(const uint16_t* hidden, const uint16_t* lm_head, int d,
                        float* target_logits, const float* draft_logits,
                        const int32_t* draft_tokens, const float* u_accept,
                        const float* u_sample, int B, int K, int V, int32_t* out_tokens,
                        int32_t* n_emitted, void* stream) {
  clear_error();
  return verify_impl(hidden, lm_head, d, target_logits, draft_logits, draft_tokens, u_accept,
                     u_sample, B, K, V, 1.0f, 1.0f, out_tokens, n_emitted, nullptr, 0, true,
                     stream);
}

}  // extern "C"

namespace {

// spec_verify_warped, and spec_verify_noalloc (use_scratch: the library's
// static scratch array stands in for the workspace).
int verify_impl(const uint16_t* hidden, const uint16_t* lm_head, int d, float* target_logits,
                const float* draft_logits, const int32_t* draft_tokens, const float* u_accept,
                const float* u_sample, int B, int K, int V, float t_target, float t_draft,
                int32_t* out_tokens, int32_t* n_emitted, void* workspace, size_t workspace_bytes,
                bool use_scratch, void* stream) {
  if (!(t_target >= 0.0f) || !(t_draft >= 0.0f) || !std::isfinite(t_target) ||
      !std::isfinite(t_draft))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "temperatures must be finite and >= 0 (got %g, %g)",
                (double)t_target, (double)t_draft);
  if (!target_logits || !draft_logits || !draft_tokens || !u_accept || !u_sample || !out_tokens ||
      !n_emitted || (!workspace && !use_scratch))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "null required pointer");
  if ((hidden == nullptr) != (lm_head == nullptr))
    return fail(SPEC_ERR_INVALID_ARGUMENT, "hidden and lm_head must be both given or both NULL");
  int rc = check_bkv(B, K, V);
  if (rc != SPEC_OK) return rc;
  const size_t chunks = ((size_t)V + 4095) / 4096;
  if ((size_t)B * (2 * K + 1) * chunks > kMaxVerifyBlocks)
    return fail(SPEC_ERR_INVALID_ARGUMENT, "B*(2K+1)*ceil(V/4096) exceeds %zu", kMaxVerifyBlocks);
  const int M = B * (K + 1);
  if (lm_head) {
    if (M > kMaxM) return fail(SPEC_ERR_INVALID_ARGUMENT, "B*(K+1)=%d exceeds %d", M, kMaxM);
    if ((rc = check_gemm_args(hidden, lm_head, target_logits, SPEC_F32, M, d, V)) != SPEC_OK)
      return rc;
  }
  if (!aligned(target_logits, 4) || !aligned(draft_logits, 4) || !aligned(draft_tokens, 4) ||
      !aligned(u_accept, 4) || !aligned(u_sample, 4) || !aligned(out_tokens, 4) ||
      !aligned(n_emitted, 4))
    return fail(SPEC_ERR_ALIGNMENT, "32-bit arrays must be 4-byte aligned");
  const size_t need = specv::verify_workspace_bytes(B, K, V);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(SPEC_ERR_WORKSPACE,
                  "(B, K, V) = (%d, %d, %d) needs %zu bytes of scratch; the library's static "
                  "scratch holds %zu (use spec_verify with a workspace)",
                  B, K, V, need, kScratchBytes);
  } else {
    if (workspace_bytes < need)
      return fail(SPEC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    if (!aligned(workspace, 256))
      return fail(SPEC_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  }
  int cus = 0;
  if ((rc = check_device(&cus)) != SPEC_OK) return rc;
  if (use_scratch && (rc = scratch_address(&workspace)) != SPEC_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // With the streaming lm-head (where spec_verify_gemm would use it) the
  // target rows' softmax statistics are folded into the GEMM's epilogue, so
  // the logits are never re-read for them.
  specv::LogitStats tstats{};
  int parts = 0;
  if (lm_head && use_stream(M, d, V)) {
    tstats = specv::target_stats_slot(workspace, B, K, V, t_target);
    parts = cus * stream_wgs_per_cu(M);
    if (!tstats.pmax || parts > specv::kMaxStatParts) {
      tstats = specv::LogitStats{};
      parts = 0;
    }
  }
  if (lm_head) {
    if (parts > 0)
      rc = launched(specv::launch_gemm_stream(hidden, lm_head, nullptr, target_logits, false,
                                              false, M, d, V, parts, s, &tstats),
                    "spec_verify lm-head");
    else
      rc = run_gemm(hidden, lm_head, target_logits, false, M, d, V, cus, s);
    if (rc != SPEC_OK) return rc;
  }
  return launched(specv::launch_verify_sampling(target_logits, draft_logits, draft_tokens, u_accept,
                                                u_sample, B, K, V, out_tokens, n_emitted,
                                                workspace, t_target, t_draft, s,
                                                parts > 0 ? &tstats : nullptr, parts),
                  "spec_verify sampling");
}

}  // namespace
