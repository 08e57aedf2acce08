// fp8 (OCP e4m3) path, first half: block quantisation with incoherent
// processing of Q, K, V (gfx950).
//
// Page "FlashAttention scaling, multi-GPU training and weight quantization",
// section 1, the FP8 bullet: low-precision matrix units double the matmul
// rate, and two measures keep outliers from ruining accuracy -- an
// independent scale for each small tile (block quantisation) and
// multiplying Q and K by a random orthogonal matrix first (incoherent
// processing), which leaves Q K^T unchanged.
//
// attn_fp8_prepare: a workgroup of four waves takes one tile of 128 tokens
// of one (tensor, batch*head) at a time, each wave 32 tokens.  Q and K are
// rotated on the float32 matrix cores as (x R)^T = R^T x^T, so each lane
// holds one token's outputs; then the tile's largest magnitude gives
// s = amax/448 and the codes are e4m3(y/s), nearest-even, by the hardware
// conversion (|y/s| <= 448, so nothing saturates).  attn_mxfp8_prepare
// instead takes one power-of-two scale per 32 channels of each token.  The
// grid strides over (tensor, batch*head, tile) items with the tensor varying
// fastest, so the matrix-core work of rotating Q and K overlaps the memory
// traffic of V.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int kTile8 = kFp8Tile;     // tokens per quantisation tile
constexpr float kE4m3Max = 448.0f;

// Four waves of 32 tokens: one 128-token quantisation tile per step.
constexpr int kPrepWaves = 4;
constexpr int kPrepThreads = kPrepWaves * 64;
constexpr int kPrepGrid = 512;       // two resident workgroups on each of 256 CUs
static_assert(kPrepWaves * 32 == kTile8, "a step covers one quantisation tile");

// v_mfma_f32_32x32x2_f32 layout: the contraction index of step s is channel
// KS*h + s in lane half h (h = lane/32), so a lane reads KS contiguous
// channels of its token; R^T sits in LDS with a padded row per output channel.
template <int D>
struct PrepCfg {
  static constexpr int KS = D / 2;     // contraction steps
  static constexpr int NX = KS / 4;    // 16-byte loads of x per lane
  static constexpr int NB = D / 32;    // 32-channel output blocks
  static constexpr int RT = D + 4;     // floats per LDS row of R^T
};

#if defined(__HIP_DEVICE_COMPILE__)
// MXFP8 scale exponent of a block whose largest magnitude is am:
// e = ceil(log2(am / 448)) clamped to [-127, 127], -127 for am = 0.  With
// am = 1.m * 2^E (448 = 1.75 * 2^8): e = E - 8, plus one when 1.m > 1.75.
__device__ __forceinline__ int mx_exponent(float am) {
  const uint32_t b = __float_as_uint(am);
  const int et = static_cast<int>((b >> 23) & 0xFFu);
  if (!(am > 0.f) || et == 0) return -127;          // zero or below 2^-126
  const int e = (et - 127) - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return max(-127, min(127, e));
}
#endif

#if defined(__HIP_DEVICE_COMPILE__)
template <int D>
__device__ __forceinline__ void prep_load_x(f32x4 (&x)[PrepCfg<D>::NX], const float* src,
                                           int64_t row, bool valid, int h) {
#pragma unroll
  for (int j = 0; j < PrepCfg<D>::NX; ++j)
    x[j] = valid ? *reinterpret_cast<const f32x4*>(src + row + h * PrepCfg<D>::KS + 4 * j)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
}

// Four e4m3 codes (a in the low byte) by the hardware conversion: OCP E4M3FN,
// nearest-even, subnormals kept.  Callers pass values of magnitude <= 448.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// Rotated block ob of a token: lane half h holds channels 32*ob + 8*g + 4*h + j
// (g, j = 0..3) as acc[4*g + j].  Codes of channel groups g and g+1 are
// exchanged across the halves so that each lane stores 8 consecutive bytes.
__device__ __forceinline__ void store_rotated_block(uint8_t* row, int ob, const uint32_t (&wd)[4],
                                                    int h, bool valid) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t send = h ? wd[2 * p] : wd[2 * p + 1];
    const uint32_t got = static_cast<uint32_t>(__shfl_xor(static_cast<int>(send), 32));
    const uint32_t lo = h ? got : wd[2 * p];
    const uint32_t hi = h ? wd[2 * p + 1] : got;
    if (valid) *reinterpret_cast<u32x2*>(row + 32 * ob + 16 * p + 8 * h) = u32x2{lo, hi};
  }
}
#endif

// MX = false: one float32 scale per 128-token tile (s = amax/448).
// MX = true: one E8M0 byte per 32 channels of each token (scale 2^e).
// Work items are (tensor, batch*head, tile); the grid strides over them and
// each wave loads its next tile's rows while it works on the current one.
#if defined(__HIP_DEVICE_COMPILE__)
// x / s rounded to nearest float32, from r = 1/s rounded to nearest: q =
// x r is within an ulp of x/s, the remainder x - s q is exact in one fma,
// and q + (x - s q) r rounds to the correctly rounded quotient (Markstein's
// theorem; no overflow here, |x/s| <= 448, and quotients in the float32
// subnormal range encode as e4m3 zero either way).  The sign is x's (s > 0):
// for x = -0 the correction would otherwise produce +0.  Four vector
// instructions where a division takes about ten.
__device__ __forceinline__ float quot_rn(float x, float s, float r) {
  const float q = x * r;
  return copysignf(fmaf(fmaf(-s, q, x), r, q), x);
}
#endif

template <int D, bool MX>
__global__ void __launch_bounds__(kPrepThreads, 2)
fp8_prepare_kernel(const float* __restrict__ q, const float* __restrict__ k,
                   const float* __restrict__ v, const float* __restrict__ R,
                   uint8_t* __restrict__ q8, uint8_t* __restrict__ k8, uint8_t* __restrict__ v8,
                   void* __restrict__ sq, void* __restrict__ sk, void* __restrict__ sv,
                   int N, int BH, int ntq) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = PrepCfg<D>;
  __shared__ __attribute__((aligned(16))) float rt[D * C::RT];   // rt[o*RT + c] = R[c][o]
  __shared__ float red[2][kPrepWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h = lane >> 5, col = lane & 31;
  for (int e = tid * 4; e < D * D; e += kPrepThreads * 4) {
    const int c = e / D, o = e % D;
    const f32x4 r4 = *reinterpret_cast<const f32x4*>(R + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) rt[(o + j) * C::RT + c] = r4[j];
  }
  __syncthreads();

  const int total = 3 * BH * ntq;
  // this lane's token row of work item `id`; the tensor varies fastest, so a
  // workgroup's items mix rotated tiles (matrix-core bound) with V tiles
  // (memory bound)
  auto locate = [&](int id, int& tensor, int& bh, int& tile, int& t, bool& valid) {
    const int rem = id / 3;
    tensor = id - 3 * rem;
    bh = rem / ntq;
    tile = rem - bh * ntq;
    t = tile * kTile8 + 32 * w + col;
    valid = t < N;
  };
  auto source = [&](int tensor) { return tensor == 0 ? q : (tensor == 1 ? k : v); };

  int id = static_cast<int>(blockIdx.x);
  f32x4 x[C::NX];
  {
    int tensor, bh, tile, t; bool valid;
    locate(id, tensor, bh, tile, t, valid);
    prep_load_x<D>(x, source(tensor), (static_cast<int64_t>(bh) * N + t) * D, valid, h);
  }
  int par = 0;
  for (; id < total; id += gridDim.x) {
    int tensor, bh, tile, t; bool valid;
    locate(id, tensor, bh, tile, t, valid);
    const int64_t row = (static_cast<int64_t>(bh) * N + t) * D;
    uint8_t* dst = (tensor == 0 ? q8 : (tensor == 1 ? k8 : v8)) + row;
    void* scale_out = tensor == 0 ? sq : (tensor == 1 ? sk : sv);

    f32x4 xn[C::NX];
    const int nid = id + static_cast<int>(gridDim.x);
    if (nid < total) {
      int tn, bn, tln, tt; bool vn;
      locate(nid, tn, bn, tln, tt, vn);
      prep_load_x<D>(xn, source(tn), (static_cast<int64_t>(bn) * N + tt) * D, vn, h);
    }

    if (tensor < 2) {
      // y^T = R^T x^T on 32x32x2 float32 MFMA: A = R^T rows (output channels), B = x^T
      f32x16 acc[C::NB];
#pragma unroll
      for (int ob = 0; ob < C::NB; ++ob)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ob][r] = 0.f;
#pragma unroll
      for (int s4 = 0; s4 < C::NX; ++s4) {
        f32x4 a4[C::NB];
#pragma unroll
        for (int ob = 0; ob < C::NB; ++ob)
          a4[ob] = *reinterpret_cast<const f32x4*>(rt + (32 * ob + col) * C::RT + h * C::KS + 4 * s4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int ob = 0; ob < C::NB; ++ob)
            acc[ob] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[ob][j], x[s4][j], acc[ob], 0, 0, 0);
      }
      if constexpr (MX) {
        uint8_t* sc = static_cast<uint8_t*>(scale_out);
#pragma unroll
        for (int ob = 0; ob < C::NB; ++ob) {
          float am = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(acc[ob][r]));
          am = fmaxf(am, __shfl_xor(am, 32));
          const int e = mx_exponent(am);
          const float mul = ldexpf(1.f, -e);         // exact power of two
          uint32_t wd[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            wd[g] = pack4_e4m3(acc[ob][4 * g] * mul, acc[ob][4 * g + 1] * mul,
                               acc[ob][4 * g + 2] * mul, acc[ob][4 * g + 3] * mul);
          store_rotated_block(dst, ob, wd, h, valid);
          if (valid && h == 0)
            sc[(static_cast<int64_t>(bh) * N + t) * C::NB + ob] = static_cast<uint8_t>(e + 127);
        }
      } else {
        float am = 0.f;
#pragma unroll
        for (int ob = 0; ob < C::NB; ++ob)
#pragma unroll
          for (int r = 0; r < 16; ++r) am = fmaxf(am, fabsf(acc[ob][r]));
        for (int m = 32; m > 0; m >>= 1) am = fmaxf(am, __shfl_xor(am, m));
        if (lane == 0) red[par][w] = am;
        __syncthreads();
        am = red[par][0];
#pragma unroll
        for (int i = 1; i < kPrepWaves; ++i) am = fmaxf(am, red[par][i]);
        par ^= 1;
        const float sc = am > 0.f ? am / kE4m3Max : 1.f;
        const float rsc = 1.f / sc;
        if (tid == 0) static_cast<float*>(scale_out)[static_cast<int64_t>(bh) * ntq + tile] = sc;
#pragma unroll
        for (int ob = 0; ob < C::NB; ++ob) {
          uint32_t wd[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            wd[g] = pack4_e4m3(quot_rn(acc[ob][4 * g], sc, rsc), quot_rn(acc[ob][4 * g + 1], sc, rsc),
                               quot_rn(acc[ob][4 * g + 2], sc, rsc), quot_rn(acc[ob][4 * g + 3], sc, rsc));
          store_rotated_block(dst, ob, wd, h, valid);
        }
      }
    } else {
      // V: no rotation; the lane's KS channels are contiguous
      uint8_t* out = dst + h * C::KS;
      if constexpr (MX) {
        uint8_t* sc = static_cast<uint8_t*>(scale_out);
        constexpr int BPL = C::KS / 32;              // whole 32-channel blocks per lane
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
          float am = 0.f;
#pragma unroll
          for (int j = 8 * b; j < 8 * b + 8; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(x[j][i]));
          const int e = mx_exponent(am);
          const float mul = ldexpf(1.f, -e);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            u32x4 cw;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const f32x4 xv = x[8 * b + 4 * m + i];
              cw[i] = pack4_e4m3(xv[0] * mul, xv[1] * mul, xv[2] * mul, xv[3] * mul);
            }
            if (valid) *reinterpret_cast<u32x4*>(out + 32 * b + 16 * m) = cw;
          }
          if (valid)
            sc[(static_cast<int64_t>(bh) * N + t) * C::NB + h * BPL + b] = static_cast<uint8_t>(e + 127);
        }
      } else {
        float am = 0.f;
#pragma unroll
        for (int j = 0; j < C::NX; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) am = fmaxf(am, fabsf(x[j][i]));
        for (int m = 32; m > 0; m >>= 1) am = fmaxf(am, __shfl_xor(am, m));
        if (lane == 0) red[par][w] = am;
        __syncthreads();
        am = red[par][0];
#pragma unroll
        for (int i = 1; i < kPrepWaves; ++i) am = fmaxf(am, red[par][i]);
        par ^= 1;
        const float sc = am > 0.f ? am / kE4m3Max : 1.f;
        const float rsc = 1.f / sc;
        if (tid == 0) static_cast<float*>(scale_out)[static_cast<int64_t>(bh) * ntq + tile] = sc;
#pragma unroll
        for (int m = 0; m < C::NX / 4; ++m) {
          u32x4 cw;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f32x4 xv = x[4 * m + i];
            cw[i] = pack4_e4m3(quot_rn(xv[0], sc, rsc), quot_rn(xv[1], sc, rsc), quot_rn(xv[2], sc, rsc),
                               quot_rn(xv[3], sc, rsc));
          }
          if (valid) *reinterpret_cast<u32x4*>(out + 16 * m) = cw;
        }
      }
    }
    if (nid < total) {
#pragma unroll
      for (int j = 0; j < C::NX; ++j) x[j] = xn[j];
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool MX>
hipError_t prep_one(const Fp8PrepArgs& a) {
  const int BH = a.B * a.H;
  const int ntq = (a.N + kTile8 - 1) / kTile8;
  const int64_t items = 3LL * BH * ntq;
  const int64_t blocks = items < kPrepGrid ? items : kPrepGrid;
  hipLaunchKernelGGL((fp8_prepare_kernel<D, MX>), dim3(static_cast<unsigned>(blocks)), dim3(kPrepThreads), 0,
                     static_cast<hipStream_t>(a.stream), a.q, a.k, a.v, a.R, a.q8, a.k8, a.v8,
                     a.sq, a.sk, a.sv, a.N, BH, ntq);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_prepare(const Fp8PrepArgs& a) {
  if (a.mx) return a.d == 64 ? prep_one<64, true>(a) : prep_one<128, true>(a);
  return a.d == 64 ? prep_one<64, false>(a) : prep_one<128, false>(a);
}

}  // namespace attn127
