// C ABI of the attention library: argument checks and kernel dispatch.
// Every check runs on the host before any HIP call, so a rejected call has
// no device side effect.  The library allocates nothing; its only state is
// the fixed scratch array of attn_bwd_static (below) and the per-device
// addresses of that array.
#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/attn.h"
#include "launch.h"

// Scratch memory of attn_bwd_static: the backward pass's row statistic
// D_i = sum_c dO_ic O_ic, B*H*N floats, which attn_bwd takes from the caller.
// Each GPU the library runs on holds its own copy for the life of the
// process.  Host code never uses this name as an address: it looks up the
// device address once per device (hipGetSymbolAddress) and passes that.
static __device__ __align__(256) float scratch[ATTN_STATIC_SCRATCH_FLOATS];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point; returns ATTN_OK, an error, or 1
// for "nothing to do".
int check_shape(int B, int H, int N, int d) {
  if (B < 0 || H < 0 || N < 0) return ATTN_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return ATTN_ERR_INVALID_ARG;
  if (N >= (1 << 30)) return ATTN_ERR_INVALID_ARG;
  const int64_t bh = static_cast<int64_t>(B) * H;
  if (bh >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  // grid: one workgroup per (b, h, 64-row block) at most
  if (bh * ((static_cast<int64_t>(N) + 63) / 64) >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (B == 0 || H == 0 || N == 0) return 1;
  return ATTN_OK;
}

// The softmax scale: finite and > 0 as given, or 0 for the scaled
// dot-product's 1/sqrt(d) (page "Self-Attention, CUDA kernels and
// FlashAttention", section 1).
int resolve_scale(float scale, int d, float* out) {
  if (scale == 0.f) {
    *out = 1.f / std::sqrt(static_cast<float>(d));
    return ATTN_OK;
  }
  if (!(std::isfinite(scale) && scale > 0.f)) return ATTN_ERR_INVALID_ARG;
  *out = scale;
  return ATTN_OK;
}

int check_ptrs(const void* q, const void* k, const void* v, const void* o, const void* lse) {
  if (!q || !k || !v || !o) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return ATTN_ERR_INVALID_ARG;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with it current) and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

int scratch_address(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return ATTN_OK;
}

// Checks shared by attn_bwd and attn_bwd_static (all but the scratch
// pointer); returns ATTN_OK, an error, or 1 for "nothing to do".
int bwd_check(const void* q, const void* k, const void* v, const void* o, const void* dout,
              const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
              float* scale, int dtype) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (resolve_scale(*scale, d, scale) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  const void* ps[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return ATTN_ERR_INVALID_ARG;
  if (!lse || (reinterpret_cast<uintptr_t>(lse) & 3u)) return ATTN_ERR_INVALID_ARG;
  return st;
}

int fwd_common(bool simple, const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (resolve_scale(scale, d, &scale) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (check_ptrs(q, k, v, o, lse) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (st == 1) return ATTN_OK;
  attn127::LaunchArgs a{q, k, v, o, lse, B, H, N, d, scale, causal ? 1 : 0, dtype, stream};
  if (simple || dtype == ATTN_F32) return status_of(attn127::launch_simple(a));
  return status_of(attn127::launch_mfma_bf16(a));
}

}  // namespace

namespace {
int fp8_prepare_common(bool mx, const float* q, const float* k, const float* v, const float* R,
                       uint8_t* q8, uint8_t* k8, uint8_t* v8, void* q_scale, void* k_scale,
                       void* v_scale, int B, int H, int N, int d, void* stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  // work items (tensor, b*h, 128-token tile) are indexed in 32 bits
  if (3 * static_cast<int64_t>(B) * H * ((static_cast<int64_t>(N) + 127) / 128) >= (int64_t(1) << 30))
    return ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !R || !q8 || !k8 || !v8 || !q_scale || !k_scale || !v_scale)
    return ATTN_ERR_INVALID_ARG;
  const void* ps[] = {q, k, v, R, q8, k8, v8};
  for (const void* p : ps)
    if (!aligned16(p)) return ATTN_ERR_INVALID_ARG;
  const void* ss[] = {q_scale, k_scale, v_scale};
  for (const void* p : ss)   // per-tile float scales: 4-byte alignment; E8M0 rows: d/32 bytes
    if (reinterpret_cast<uintptr_t>(p) & static_cast<uintptr_t>(mx ? (d / 32 - 1) : 3)) return ATTN_ERR_INVALID_ARG;
  if (st == 1) return ATTN_OK;
  attn127::Fp8PrepArgs a{q, k, v, R, q8, k8, v8, q_scale, k_scale, v_scale, B, H, N, d, mx ? 1 : 0, stream};
  return status_of(attn127::launch_fp8_prepare(a));
}

int fp8_fwd_common(bool mx, const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                   const void* q_scale, const void* k_scale, const void* v_scale, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal, void* stream) {
  int st = check_shape(B, H, N, d);
  if (st < 0) return st;
  if (resolve_scale(scale, d, &scale) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (check_ptrs(q8, k8, v8, o, lse) != ATTN_OK) return ATTN_ERR_INVALID_ARG;
  if (!q_scale || !k_scale || !v_scale) return ATTN_ERR_INVALID_ARG;
  const void* ss[] = {q_scale, k_scale, v_scale};
  for (const void* p : ss)
    if (reinterpret_cast<uintptr_t>(p) & static_cast<uintptr_t>(mx ? (d / 32 - 1) : 3)) return ATTN_ERR_INVALID_ARG;
  if (st == 1) return ATTN_OK;
  attn127::Fp8Args a{q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale,
                     causal ? 1 : 0, mx ? 1 : 0, stream};
  return status_of(attn127::launch_fp8_fwd(a));
}
int w4_check(const void* qweight, const void* scales, const void* zeros, const void* out,
             int M, int N, int K, int group, bool gemm, const void* x) {
  if (M < 0 || N < 0 || K < 0) return ATTN_ERR_INVALID_ARG;
  if (gemm && M > 16) return ATTN_ERR_INVALID_ARG;
  if (K % 8 != 0) return ATTN_ERR_INVALID_ARG;
  if (group != 128) return ATTN_ERR_UNSUPPORTED;
  if (K > 32768) return ATTN_ERR_UNSUPPORTED;   // the groups' scales of 32 rows stay in 32 KB of LDS
  if (K % group != 0) return ATTN_ERR_INVALID_ARG;
  // packed weights and activations are addressed with 32-bit byte offsets
  if (static_cast<int64_t>(N) * (K / 2) >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (static_cast<int64_t>(K) * 2 * 16 >= (int64_t(1) << 31)) return ATTN_ERR_INVALID_ARG;
  if (!qweight || !scales || !zeros || !out || (gemm && !x)) return ATTN_ERR_INVALID_ARG;
  if (!aligned16(qweight) || (reinterpret_cast<uintptr_t>(scales) & 1u)) return ATTN_ERR_INVALID_ARG;
  if (gemm ? (!aligned16(x) || (reinterpret_cast<uintptr_t>(out) & 7u)) : !aligned16(out))
    return ATTN_ERR_INVALID_ARG;
  if (N == 0 || K == 0 || (gemm && M == 0)) return 1;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
             int N, int d, float scale, int causal, int dtype, void* stream) {
  return fwd_common(false, q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream);
}

int attn_fwd_simple(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  return fwd_common(true, q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream);
}


int attn_fp8_prepare(const float* q, const float* k, const float* v, const float* R, uint8_t* q8,
                     uint8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, float* v_scale,
                     int B, int H, int N, int d, void* stream) {
  return fp8_prepare_common(false, q, k, v, R, q8, k8, v8, q_scale, k_scale, v_scale, B, H, N, d, stream);
}

int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const float* q_scale,
                 const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, void* stream) {
  return fp8_fwd_common(false, q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale,
                        causal, stream);
}

int attn_mxfp8_prepare(const float* q, const float* k, const float* v, const float* R, uint8_t* q8,
                       uint8_t* k8, uint8_t* v8, uint8_t* q_scale, uint8_t* k_scale,
                       uint8_t* v_scale, int B, int H, int N, int d, void* stream) {
  return fp8_prepare_common(true, q, k, v, R, q8, k8, v8, q_scale, k_scale, v_scale, B, H, N, d, stream);
}

int attn_fwd_mxfp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8, const uint8_t* q_scale,
                   const uint8_t* k_scale, const uint8_t* v_scale, void* o, float* lse, int B, int H,
                   int N, int d, float scale, int causal, void* stream) {
  return fp8_fwd_common(true, q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N, d, scale,
                        causal, stream);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, float* delta, void* dq, void* dk, void* dv, int B, int H, int N,
             int d, float scale, int causal, int dtype, void* stream) {
  const int st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, &scale, dtype);
  if (st < 0) return st;
  if (!delta || (reinterpret_cast<uintptr_t>(delta) & 3u)) return ATTN_ERR_INVALID_ARG;
  if (st == 1) return ATTN_OK;
  attn127::BwdArgs a{q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, scale,
                     causal ? 1 : 0, stream};
  return status_of(attn127::launch_bwd(a));
}

int attn_bwd_static(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                    float scale, int causal, int dtype, void* stream) {
  const int st = bwd_check(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, &scale, dtype);
  if (st < 0) return st;
  if (static_cast<int64_t>(B) * H * N > ATTN_STATIC_SCRATCH_FLOATS) return ATTN_ERR_TOO_LARGE;
  if (st == 1) return ATTN_OK;
  float* delta = nullptr;
  const int sa = scratch_address(&delta);
  if (sa != ATTN_OK) return sa;
  // D is written in full by the first of the three launches before the
  // other two read it, so nothing left by an earlier call needs clearing
  attn127::BwdArgs a{q, k, v, o, dout, lse, delta, dq, dk, dv, B, H, N, d, scale,
                     causal ? 1 : 0, stream};
  return status_of(attn127::launch_bwd(a));
}

int w4a16_gemm(const void* x, const uint32_t* qweight, const void* scales, const uint8_t* zeros,
               void* y, int M, int N, int K, int group, void* stream) {
  const int st = w4_check(qweight, scales, zeros, y, M, N, K, group, true, x);
  if (st != ATTN_OK) return st == 1 ? ATTN_OK : st;
  attn127::W4Args a{x, qweight, scales, zeros, y, M, N, K, stream};
  return status_of(attn127::launch_w4a16(a));
}

int w4a16_dequantize(const uint32_t* qweight, const void* scales, const uint8_t* zeros, void* w,
                     int N, int K, int group, void* stream) {
  const int st = w4_check(qweight, scales, zeros, w, 0, N, K, group, false, nullptr);
  if (st != ATTN_OK) return st == 1 ? ATTN_OK : st;
  attn127::W4Args a{nullptr, qweight, scales, zeros, w, 0, N, K, stream};
  return status_of(attn127::launch_w4a16_dequant(a));
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size, dtype or scale)";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_HIP: return "HIP runtime error at launch";
    case ATTN_ERR_TOO_LARGE: return "request exceeds the library's fixed scratch buffer (attn_bwd_static: B*H*N > ATTN_STATIC_SCRATCH_FLOATS)";
    default: return "unknown status";
  }
}

}  // extern "C"
