// Plain tiled attention forward with float32 vector arithmetic.
//
// The second device path of the library: no matrix cores and no rounding of
// P, so for float32 inputs every step stays in float32.  It follows the same
// algorithm as the matrix-core kernel -- query rows held on chip for the
// whole key loop, key/value tiles staged through LDS, an online softmax with
// a running maximum and running normaliser that rescales the partial output
// as each tile arrives (page "Self-Attention, CUDA kernels and
// FlashAttention", section 3), and one division by the normaliser after the
// last key (page "FlashAttention scaling, multi-GPU training and weight
// quantization", section 1) -- but with four lanes per query row (each
// holding a quarter of its channels) instead of MFMA tiles.
//
// A workgroup of KS waves handles one block of query rows; wave s runs the
// online softmax over the s-th of KS equal key ranges, and the KS partial
// results (running maximum, normaliser and unnormalised output of every row)
// are merged once at the end through LDS:  M = max_s m_s,
// l = sum_s l_s 2^(m_s - M), O = sum_s O_s 2^(m_s - M) / l.  This is the same
// rescaling the online softmax applies between tiles, so the result is the
// one exact softmax; splitting the keys only gives a short sequence (the
// 196-token ViT image) KS times more waves.  Four lanes per row (16 rows
// per wave) spread the work of a short sequence over four times as many
// waves again, and cut the LDS bytes every lane reads per key by four.
#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int kSplit = 8;           // waves (key ranges) per workgroup
constexpr int kSimpleStep = 16;     // keys per softmax update

template <int D>
struct SimpleCfg {
  static constexpr int LPQ = 4;                  // lanes per query row
  static constexpr int QPB = 64 / LPQ;           // query rows per workgroup
  static constexpr int DL = D / LPQ;             // channels per lane
  static constexpr int TK = D == 64 ? 32 : 16;   // keys per LDS tile of one wave
  static constexpr int STAGE = TK * D;           // floats of one K (or V) tile
  // floats of LDS per wave: its K and V tiles, later its 64 lanes' partial
  // outputs in rows of DL+1 floats (the pad spreads lanes over banks)
  static constexpr int PW = 2 * STAGE > 64 * (DL + 1) ? 2 * STAGE : 64 * (DL + 1);
  static_assert(TK % kSimpleStep == 0, "whole softmax steps per tile");
  static_assert(PW % 4 == 0, "16-byte aligned wave regions");
};

template <typename T>
__device__ __forceinline__ f32x4 load4(const T* p, int64_t i);
template <>
__device__ __forceinline__ f32x4 load4<float>(const float* p, int64_t i) {
  return *reinterpret_cast<const f32x4*>(p + i);
}
template <>
__device__ __forceinline__ f32x4 load4<uint16_t>(const uint16_t* p, int64_t i) {
  const u32x2 w = *reinterpret_cast<const u32x2*>(p + i);
  return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xFFFF0000u),
               __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xFFFF0000u)};
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, int64_t i, float x);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, int64_t i, float x) { p[i] = x; }
template <>
__device__ __forceinline__ void store_elem<uint16_t>(uint16_t* p, int64_t i, float x) {
  p[i] = static_cast<uint16_t>(pack_bf16x2(x, 0.f) & 0xFFFFu);
}

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kSplit)
attn_simple_kernel(const T* __restrict__ q, const T* __restrict__ k,
                   const T* __restrict__ v, T* __restrict__ o,
                   float* __restrict__ lse, int N, float c /* scale*log2e */) {
  using C = SimpleCfg<D>;
  constexpr int DL = C::DL, TK = C::TK;
  __shared__ __attribute__((aligned(16))) float smem[kSplit * C::PW];
  __shared__ float part_ml[kSplit][64][2];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int quarter = lane % C::LPQ;     // which quarter of the row's channels
  const int nqb = (N + C::QPB - 1) / C::QPB;
  const int bh = blockIdx.x / nqb;
  const int q0 = (blockIdx.x % nqb) * C::QPB;
  const int qi = q0 + lane / C::LPQ;
  const int64_t base = static_cast<int64_t>(bh) * N * D;

  float qr[DL], acc[DL];
#pragma unroll
  for (int t = 0; t < DL; t += 4) {
    const f32x4 x = (qi < N) ? load4<T>(q, base + static_cast<int64_t>(qi) * D + quarter * DL + t) : f32x4{};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      qr[t + u] = x[u];
      acc[t + u] = 0.f;
    }
  }
  float m = -INFINITY, l = 0.f;

  // this wave's key range: the workgroup's keys split into kSplit whole tiles
  const int kend = CAUSAL ? min(N, q0 + C::QPB) : N;
  const int ntile = (kend + TK - 1) / TK;
  const int per = (ntile + kSplit - 1) / kSplit;
  const int t0 = wave * per, t1 = min(ntile, t0 + per);
  float* ks = smem + wave * C::PW;
  float* vs = ks + C::STAGE;

  for (int tt = t0; tt < t1; ++tt) {
    const int k0 = tt * TK;
    // stage K and V rows [k0, k0+TK) of this head, 4 floats per lane and step
#pragma unroll
    for (int e = lane * 4; e < C::STAGE; e += 256) {
      const int r = e / D, col = e % D;
      const int key = k0 + r;
      const int64_t off = base + static_cast<int64_t>(key) * D + col;
      const f32x4 kx = key < N ? load4<T>(k, off) : f32x4{};
      const f32x4 vx = key < N ? load4<T>(v, off) : f32x4{};
      *reinterpret_cast<f32x4*>(ks + e) = kx;
      *reinterpret_cast<f32x4*>(vs + e) = vx;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // this wave's LDS writes are visible
    __builtin_amdgcn_wave_barrier();
    for (int j0 = 0; j0 < TK; j0 += kSimpleStep) {
      float s[kSimpleStep];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < kSimpleStep; ++j) {
        // every lane of a row group reads the same K row: broadcast reads
        const float* krow = ks + (j0 + j) * D + quarter * DL;
        float dot = 0.f;
#pragma unroll
        for (int t = 0; t < DL; t += 4) {
          const f32x4 kk = *reinterpret_cast<const f32x4*>(krow + t);
          dot = fmaf(qr[t], kk[0], dot);
          dot = fmaf(qr[t + 1], kk[1], dot);
          dot = fmaf(qr[t + 2], kk[2], dot);
          dot = fmaf(qr[t + 3], kk[3], dot);
        }
        dot += __shfl_xor(dot, 1);       // the row's four lanes: lane bits 0 and 1
        dot += __shfl_xor(dot, 2);
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
      for (int t = 0; t < DL; ++t) acc[t] *= alpha;
#pragma unroll
      for (int j = 0; j < kSimpleStep; ++j) {
        const float* vrow = vs + (j0 + j) * D + quarter * DL;
#pragma unroll
        for (int t = 0; t < DL; t += 4) {
          const f32x4 vv = *reinterpret_cast<const f32x4*>(vrow + t);
          acc[t] = fmaf(s[j], vv[0], acc[t]);
          acc[t + 1] = fmaf(s[j], vv[1], acc[t + 1]);
          acc[t + 2] = fmaf(s[j], vv[2], acc[t + 2]);
          acc[t + 3] = fmaf(s[j], vv[3], acc[t + 3]);
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");   // reads done before the next tile's writes
    __builtin_amdgcn_wave_barrier();
  }

  // ---- merge the kSplit partial results of every row ----
  __syncthreads();                                  // every wave is done with its tiles
  float* mine = smem + wave * C::PW + lane * (DL + 1);
#pragma unroll
  for (int t = 0; t < DL; ++t) mine[t] = acc[t];
  part_ml[wave][lane][0] = m;
  part_ml[wave][lane][1] = l;
  __syncthreads();
  // wave w writes channels [w*DL/kSplit, (w+1)*DL/kSplit) of every row of the block
  float mm = -INFINITY;
#pragma unroll
  for (int s2 = 0; s2 < kSplit; ++s2) mm = fmaxf(mm, part_ml[s2][lane][0]);
  const float mref = (mm == -INFINITY) ? 0.f : mm;
  float ltot = 0.f, wgt[kSplit];
#pragma unroll
  for (int s2 = 0; s2 < kSplit; ++s2) {
    wgt[s2] = fast_exp2(part_ml[s2][lane][0] - mref);   // 0 for an empty range (m = -inf)
    ltot += wgt[s2] * part_ml[s2][lane][1];
  }
  if (qi < N) {
    const float inv = 1.f / ltot;
    constexpr int CW = DL / kSplit;
#pragma unroll
    for (int t = wave * CW; t < (wave + 1) * CW; ++t) {
      float x = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < kSplit; ++s2) x = fmaf(wgt[s2], smem[s2 * C::PW + lane * (DL + 1) + t], x);
      store_elem<T>(o, base + static_cast<int64_t>(qi) * D + quarter * DL + t, x * inv);
    }
    if (lse != nullptr && quarter == 0 && wave == 0)     // one lane per row
      lse[static_cast<int64_t>(bh) * N + qi] = (mm + __log2f(ltot)) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_one(const LaunchArgs& a) {
  constexpr int QPB = SimpleCfg<D>::QPB;
  const int64_t blocks = static_cast<int64_t>((a.N + QPB - 1) / QPB) * a.B * a.H;
  dim3 grid(static_cast<unsigned>(blocks));   // < 2^31, checked by the caller
  hipLaunchKernelGGL((attn_simple_kernel<T, D, CAUSAL>), grid, dim3(64 * kSplit), 0,
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
