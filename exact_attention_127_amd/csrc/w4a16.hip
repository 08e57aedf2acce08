// W4A16 decode product on gfx950: Y = X W^T with 4-bit weights.
//
// Page "FlashAttention scaling, multi-GPU training and weight quantization",
// section 3 (quantisation and on-the-fly dequantisation kernels): the
// weights stay packed, eight 4-bit integers per 32-bit word, on their way
// from HBM; each lane unpacks its words in registers with shifts and masks,
// applies the group's scale and zero point to get FP16 values, and hands
// them straight to the matrix cores with the FP16 activations.  The expanded
// weights never reach memory.
//
// Layout: X fp16 [M][K] (M <= 16 tokens), qweight uint32 [N][K/8] (value i of
// a word in bits 4i..4i+3, eight consecutive k of one output row), scales
// fp16 [N][K/128], zero points uint8 [N][K/128], Y fp16 [M][N].
//
// v_mfma_f32_16x16x32_f16 with A = W rows (16 output channels) and B = X^T
// (16 tokens, zero past M): lane l supplies 8 consecutive k of row l%16 for
// quad l/16, which is exactly one packed word.  Per 128-k group a lane loads
// the four words of its quad (16 bytes) and uses one per MFMA step.
// Unpacking: (word >> 4i) & 0x000F000F | 0x64006400 is the fp16 pair
// (1024 + q_i, 1024 + q_{i+4}); subtracting 1024 + z gives q - z exactly and
// one multiplication by s rounds once, to fp16(s (q - z)).  The k order
// inside a step is therefore (0,4,1,5,2,6,3,7), and each X fragment is
// permuted to the same order with v_perm_b32.
// Four waves split K; their float32 partial sums meet in LDS in a fixed
// order, so results are deterministic.
#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int kW4Waves = 4;                  // waves per workgroup (split K)
constexpr int kW4RowTiles = 2;               // 16-row tiles per wave
constexpr int kW4Rows = 16 * kW4RowTiles;    // output rows per workgroup
constexpr int kW4Group = 128;                // k per scale group

#if defined(__HIP_DEVICE_COMPILE__)
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// Eight fp16 weights of one packed word in the step order (0,4,1,5,2,6,3,7).
__device__ __forceinline__ h8 dequant_word(uint32_t w, h2 zb, h2 s) {
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = (w >> (4 * i)) & 0x000F000Fu;
    const h2 v = (as_h2(b | 0x64006400u) - zb) * s;    // exact difference, one rounding
    p[i] = as_u(v);
  }
  return __builtin_bit_cast(h8, u32x4{p[0], p[1], p[2], p[3]});
}

// Eight activations x[k0 .. k0+7] (four dwords) in the step order.
__device__ __forceinline__ h8 permute_x(u32x4 d) {
  const uint32_t a = __builtin_amdgcn_perm(d[2], d[0], 0x05040100u);   // (x0, x4)
  const uint32_t b = __builtin_amdgcn_perm(d[2], d[0], 0x07060302u);   // (x1, x5)
  const uint32_t c = __builtin_amdgcn_perm(d[3], d[1], 0x05040100u);   // (x2, x6)
  const uint32_t e = __builtin_amdgcn_perm(d[3], d[1], 0x07060302u);   // (x3, x7)
  return __builtin_bit_cast(h8, u32x4{a, b, c, e});
}
#endif

__global__ void __launch_bounds__(kW4Waves * 64)
w4a16_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
             const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
             uint16_t* __restrict__ y, int M, int N, int K) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ f32x4 red[kW4Waves][kW4RowTiles][64];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15;                 // A: row in the tile; B: token
  const int quad = lane >> 4;                // k quad of the step
  const int n0 = static_cast<int>(blockIdx.x) * kW4Rows;
  const int ngroups = K / kW4Group;
  const int per = (ngroups + kW4Waves - 1) / kW4Waves;
  const int g0 = wave * per;
  const int g1 = min(ngroups, g0 + per);
  const int kw = K / 8;                      // words per weight row
  const bool tok = col < M;
  const uint16_t* xrow = x + static_cast<int64_t>(tok ? col : 0) * K;

  f32x4 acc[kW4RowTiles];
#pragma unroll
  for (int rt = 0; rt < kW4RowTiles; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g = g0; g < g1; ++g) {
    u32x4 wv[kW4RowTiles];
    h2 zb[kW4RowTiles], sc[kW4RowTiles];
#pragma unroll
    for (int rt = 0; rt < kW4RowTiles; ++rt) {
      const int n = n0 + 16 * rt + col;
      if (n < N) {
        wv[rt] = *reinterpret_cast<const u32x4*>(qw + static_cast<int64_t>(n) * kw + g * 16 + 4 * quad);
        const uint32_t s = scales[static_cast<int64_t>(n) * ngroups + g];
        const uint32_t z = zeros[static_cast<int64_t>(n) * ngroups + g];
        sc[rt] = as_h2(s | (s << 16));
        zb[rt] = as_h2((0x6400u | z) * 0x00010001u);
      } else {
        wv[rt] = u32x4{0u, 0u, 0u, 0u};
        sc[rt] = as_h2(0u);
        zb[rt] = as_h2(0x64006400u);
      }
    }
    u32x4 xv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
      xv[t] = tok ? *reinterpret_cast<const u32x4*>(xrow + g * kW4Group + 8 * (4 * quad + t))
                  : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const h8 b = permute_x(xv[t]);
#pragma unroll
      for (int rt = 0; rt < kW4RowTiles; ++rt) {
        const h8 a = dequant_word(wv[rt][t], zb[rt], sc[rt]);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[rt], 0, 0, 0);
      }
    }
  }

  // partial sums of the four K slices, added in wave order
#pragma unroll
  for (int rt = 0; rt < kW4RowTiles; ++rt) red[wave][rt][lane] = acc[rt];
  __syncthreads();
  if (wave < kW4RowTiles) {
    const int rt = wave;
    f32x4 s = red[0][rt][lane];
#pragma unroll
    for (int w = 1; w < kW4Waves; ++w) s += red[w][rt][lane];
    // C layout: lane holds token col, output rows 4*quad + r of the tile
    const int nb = n0 + 16 * rt + 4 * quad;
    if (tok && nb < N) {
      uint16_t* out = y + static_cast<int64_t>(col) * N + nb;
      if ((N & 3) == 0 && nb + 3 < N) {          // 8-byte aligned
        const h2 lo = h2{static_cast<_Float16>(s[0]), static_cast<_Float16>(s[1])};
        const h2 hi = h2{static_cast<_Float16>(s[2]), static_cast<_Float16>(s[3])};
        *reinterpret_cast<u32x2*>(out) = u32x2{as_u(lo), as_u(hi)};
      } else {
        for (int r = 0; r < 4 && nb + r < N; ++r)
          out[r] = __builtin_bit_cast(uint16_t, static_cast<_Float16>(s[r]));
      }
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// The fp16 weights themselves, written out: the unfused path the fused
// product avoids, kept for checking the dequantisation bit for bit.
__global__ void __launch_bounds__(256)
w4a16_dequant_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
                     const uint8_t* __restrict__ zeros, uint16_t* __restrict__ w, int N, int K) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int64_t words = static_cast<int64_t>(N) * (K / 8);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= words) return;
  const int n = static_cast<int>(i / (K / 8));
  const int k0 = static_cast<int>(i % (K / 8)) * 8;
  const int g = k0 / kW4Group;
  const uint32_t s = scales[static_cast<int64_t>(n) * (K / kW4Group) + g];
  const uint32_t z = zeros[static_cast<int64_t>(n) * (K / kW4Group) + g];
  const h8 v = dequant_word(qw[i], as_h2((0x6400u | z) * 0x00010001u), as_h2(s | (s << 16)));
  // step order (0,4,1,5,2,6,3,7) back to k order
  const h8 o = __builtin_shufflevector(v, v, 0, 2, 4, 6, 1, 3, 5, 7);
  *reinterpret_cast<u32x4*>(w + static_cast<int64_t>(n) * K + k0) = __builtin_bit_cast(u32x4, o);
#endif
}

}  // namespace

hipError_t launch_w4a16(const W4Args& a) {
  const unsigned blocks = static_cast<unsigned>((a.N + kW4Rows - 1) / kW4Rows);
  hipLaunchKernelGGL(w4a16_kernel, dim3(blocks), dim3(kW4Waves * 64), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x), a.qweight,
                     static_cast<const uint16_t*>(a.scales), a.zeros, static_cast<uint16_t*>(a.y),
                     a.M, a.N, a.K);
  return hipGetLastError();
}

hipError_t launch_w4a16_dequant(const W4Args& a) {
  const int64_t words = static_cast<int64_t>(a.N) * (a.K / 8);
  const unsigned blocks = static_cast<unsigned>((words + 255) / 256);
  hipLaunchKernelGGL(w4a16_dequant_kernel, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(a.stream), a.qweight,
                     static_cast<const uint16_t*>(a.scales), a.zeros, static_cast<uint16_t*>(a.y),
                     a.N, a.K);
  return hipGetLastError();
}

}  // namespace attn127
