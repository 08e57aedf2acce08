// Plain tiled attention forward with float32 vector arithmetic.
//
// The second device path of the library: no matrix cores and no rounding of
// P, so for float32 inputs every step stays in float32.  It follows the same
// algorithm as the matrix-core kernel -- query rows held on chip for the
// whole key loop, key/value tiles staged through LDS, an online softmax with
// a running maximum and running normaliser that rescales the partial output
// as each tile arrives (page "Self-Attention, CUDA kernels and
// FlashAttention", section 3), and one division by the normaliser after the
// last tile (page "FlashAttention scaling, multi-GPU training and weight
// quantization", section 1) -- but with one query row per lane (two lanes per
// row when d = 128) instead of MFMA tiles.
#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int kSimpleKeys = 32;     // keys per LDS tile
constexpr int kSimpleStep = 16;     // keys per softmax update

template <typename T>
__device__ __forceinline__ float load_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_bits_to_f32(p[i]);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, int64_t i, float x) {
  p[i] = static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xFFFFu);
}

// One wave per block of 64 / LPQ query rows of one (b, h).  Lane owns DL = 64
// channels of one query row; with d = 128 two neighbouring lanes share a row.
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(64)
attn_simple_kernel(const T* __restrict__ q, const T* __restrict__ k,
                   const T* __restrict__ v, T* __restrict__ o,
                   float* __restrict__ lse, int N, float c /* scale*log2e */) {
  constexpr int LPQ = D / 64;          // lanes per query row
  constexpr int QPB = 64 / LPQ;        // query rows per block
  constexpr int DL = 64;               // channels per lane
  __shared__ float ks[kSimpleKeys][D];
  __shared__ float vs[kSimpleKeys][D];

  const int lane = threadIdx.x;
  const int half = lane % LPQ;
  const int nqb = (N + QPB - 1) / QPB;
  const int bh = blockIdx.x / nqb;
  const int q0 = (blockIdx.x % nqb) * QPB;
  const int qi = q0 + lane / LPQ;
  const int64_t base = static_cast<int64_t>(bh) * N * D;

  float qr[DL], acc[DL];
#pragma unroll
  for (int t = 0; t < DL; ++t) {
    qr[t] = (qi < N) ? load_elem<T>(q, base + static_cast<int64_t>(qi) * D + half * DL + t) : 0.f;
    acc[t] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  int kend = N;
  if (CAUSAL) kend = min(N, q0 + QPB);   // last query of the block sees keys < q0+QPB
  for (int k0 = 0; k0 < kend; k0 += kSimpleKeys) {
    __syncthreads();
    for (int e = lane; e < kSimpleKeys * D; e += 64) {
      const int r = e / D, col = e % D;
      const int key = k0 + r;
      const bool ok = key < N;
      const int64_t off = base + static_cast<int64_t>(key) * D + col;
      ks[r][col] = ok ? load_elem<T>(k, off) : 0.f;
      vs[r][col] = ok ? load_elem<T>(v, off) : 0.f;
    }
    __syncthreads();
    for (int j0 = 0; j0 < kSimpleKeys; j0 += kSimpleStep) {
      float s[kSimpleStep];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kSimpleStep; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int t = 0; t < DL; ++t) dot = fmaf(qr[t], ks[j0 + j][half * DL + t], dot);
        if (LPQ == 2) dot += __shfl_xor(dot, 1);
        const int key = k0 + j0 + j;
        const bool masked = key >= N || (CAUSAL && key > qi);
        s[j] = masked ? -INFINITY : dot * c;
        mx = fmaxf(mx, s[j]);
      }
      const float mnew = fmaxf(m, mx);
      // A row whose keys so far are all masked keeps m = -inf; use 0 as the
      // reference so exp2 gives 0 rather than NaN.
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(m - mref);
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < kSimpleStep; ++j) {
        s[j] = fast_exp2(s[j] - mref);
        psum += s[j];
      }
      l = l * alpha + psum;
      m = mnew;
#pragma unroll
      for (int t = 0; t < DL; ++t) {
        float a = acc[t] * alpha;
#pragma unroll
        for (int j = 0; j < kSimpleStep; ++j) a = fmaf(s[j], vs[j0 + j][half * DL + t], a);
        acc[t] = a;
      }
    }
  }
  if (qi < N) {
    const float inv = 1.f / l;
#pragma unroll
    for (int t = 0; t < DL; ++t)
      store_elem<T>(o, base + static_cast<int64_t>(qi) * D + half * DL + t, acc[t] * inv);
    if (lse != nullptr && half == 0)
      lse[static_cast<int64_t>(bh) * N + qi] = (m + __log2f(l)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(const LaunchArgs& a) {
  constexpr int QPB = 64 / (D / 64);
  const int64_t blocks = static_cast<int64_t>((a.N + QPB - 1) / QPB) * a.B * a.H;
  dim3 grid(static_cast<unsigned>(blocks));   // < 2^31, checked by the caller
  hipLaunchKernelGGL((attn_simple_kernel<T, D, CAUSAL>), grid, dim3(64), 0,
                     static_cast<hipStream_t>(a.stream),
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                     static_cast<const T*>(a.v), static_cast<T*>(a.o), a.lse, a.N,
                     a.scale * kLog2e);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dtype(const LaunchArgs& a) {
  if (a.d == 64) return a.causal ? launch_one<T, 64, true>(a) : launch_one<T, 64, false>(a);
  return a.causal ? launch_one<T, 128, true>(a) : launch_one<T, 128, false>(a);
}

}  // namespace

hipError_t launch_simple(const LaunchArgs& a) {
  return a.dtype == 0 ? launch_dtype<float>(a) : launch_dtype<uint16_t>(a);
}

}  // namespace attn127
