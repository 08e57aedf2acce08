// Host-side launch descriptors shared by the C ABI and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn127 {

// Tokens per fp8 quantisation tile (one float32 scale per (b, h, tile)),
// shared by the prepare and the forward kernels.
constexpr int kFp8Tile = 128;

// Causal launches walk an XCD's share of heads (the dispatcher sends
// workgroup i to XCD i mod 8) in chunks whose per-head streamed bytes total
// about 16 MB, so that the blocks running side by side on an XCD read the
// same keys (or queries) from its L2 and the last-level cache instead of
// every CU streaming a different head from HBM.  Measured on the bf16
// forward: 1.30 -> 1.14 ms at B=8 H=32 N=4096, 2.24 -> 2.08 ms at B=4 H=32
// N=8192.  The chunk divides the XCD's share of heads.
inline int causal_head_chunk(int BH, int64_t head_bytes) {
  const int hx = BH % 8 == 0 ? BH / 8 : 1;
  int64_t hc = (int64_t(16) << 20) / (head_bytes > 0 ? head_bytes : 1);
  hc = hc < 1 ? 1 : (hc > hx ? hx : hc);
  int h = static_cast<int>(hc);
  while (hx % h) --h;
  return h;
}

struct LaunchArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;          // nullable
  int B, H, N, d;
  float scale;
  int causal;
  int dtype;           // attn_dtype
  void* stream;
};

struct Fp8Args {
  const uint8_t* q8;
  const uint8_t* k8;
  const uint8_t* v8;
  const void* sq;      // float32 per 128-token tile, or E8M0 bytes per 32 channels (mx)
  const void* sk;
  const void* sv;
  void* o;             // bf16
  float* lse;          // nullable
  int B, H, N, d;
  float scale;
  int causal;
  int mx;              // 1: MXFP8 (E8M0 scale per 32 channels of a token)
  void* stream;
};

struct Fp8PrepArgs {
  const float* q;
  const float* k;
  const float* v;
  const float* R;
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8;
  void* sq;            // float32 per 128-token tile, or E8M0 bytes per 32 channels (mx)
  void* sk;
  void* sv;
  int B, H, N, d;
  int mx;
  void* stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;        // caller's scratch, B*H*N floats
  void* dq;
  void* dk;
  void* dv;
  int B, H, N, d;
  float scale;
  int causal;
  void* stream;
};

hipError_t launch_simple(const LaunchArgs& a);
hipError_t launch_mfma_bf16(const LaunchArgs& a);
hipError_t launch_fp8_prepare(const Fp8PrepArgs& a);
hipError_t launch_fp8_fwd(const Fp8Args& a);
hipError_t launch_bwd(const BwdArgs& a);

struct W4Args {
  const void* x;           // fp16 [M][K]
  const uint32_t* qweight; // [N][K/8]
  const void* scales;      // fp16 [N][K/128]
  const uint8_t* zeros;    // [N][K/128]
  void* y;                 // fp16 [M][N] (dequantise: fp16 weights [N][K])
  int M, N, K;
  void* stream;
};

hipError_t launch_w4a16(const W4Args& a);
hipError_t launch_w4a16_dequant(const W4Args& a);

}  // namespace attn127
