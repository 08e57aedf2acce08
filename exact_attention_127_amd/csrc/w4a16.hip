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
//
// Memory: the packed words stream through buffer loads whose per-lane
// offsets are fixed and whose group advances in the scalar offset, two
// groups ahead of the matrix cores; the scales and zero points of the
// workgroup's rows are staged in LDS once with coalesced loads (read per
// lane from global memory they cost more time than the weights).  Four
// waves split K; their float32 partial sums meet in LDS in a fixed order, so
// results are deterministic.
#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int kW4Waves = 4;                  // waves per workgroup (split K)
constexpr int kW4Group = 128;                // k per scale group

#if defined(__HIP_DEVICE_COMPILE__)
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// (a & m) | c in one instruction.  gfx950's three-operand encoding has no
// 32-bit literal, so the compiler splits the expression when m and c are
// constants; here they arrive in registers.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(m), "v"(c));
  return r;
}

// Eight fp16 weights of one packed word in the step order (0,4,1,5,2,6,3,7).
// m = 0x000F000F and c = 0x64006400 (the fp16 pair 1024, 1024) come in
// registers.
__device__ __forceinline__ h8 dequant_word(uint32_t w, h2 zb, h2 s, uint32_t m, uint32_t c) {
  uint32_t p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t b = and_or(w >> (4 * i), m, c);          // (1024 + q_i, 1024 + q_{i+4})
    p[i] = as_u((as_h2(b) - zb) * s);                        // exact difference, one rounding
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

// What one lane loads for one 128-k group: its four words of each row tile,
// the raw scale and zero point of those rows, and its X fragment.  Kept raw
// so that no arithmetic on them forces a wait before the next loads issue.
template <int RT>
struct W4Raw {
  u32x4 w[RT];
  u32x4 x[4];
};

// Loads go through buffer resources.  Each lane's offset into a buffer is
// fixed for the whole loop (its row, token and quad); the group enters
// through the instruction's scalar offset.  Offsets at or past a buffer's
// end read as zeros: a lane whose row is past N or whose token is past M
// starts at the end, and a group past the wave's slice gets a scalar offset
// at the end, so no branch surrounds a load (branches around loads make the
// compiler wait for every load in flight at the join).
template <int RT>
struct W4Src {
  __amdgpu_buffer_rsrc_t qw, x;
  uint32_t qw_end, x_end;                   // buffer sizes in bytes
  uint32_t vw[RT], vx;                      // per-lane offsets
};

template <int RT>
__device__ __forceinline__ void w4_load(W4Raw<RT>& r, const W4Src<RT>& src, int g, bool live) {
  const uint32_t gw = live ? static_cast<uint32_t>(g) * 64u : src.qw_end;
  const uint32_t gx = live ? static_cast<uint32_t>(g) * (2u * kW4Group) : src.x_end;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    r.w[rt] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.qw, src.vw[rt], gw, 0));
#pragma unroll
  for (int t = 0; t < 4; ++t)
    r.x[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(src.x, src.vx + 16 * t, gx, 0));
}

// RT row tiles of 16 outputs per wave: two for a few tokens (more waves in
// flight), four for up to 16 tokens (each X fragment feeds more rows).
template <int RT>
__global__ void __launch_bounds__(kW4Waves * 64)
w4a16_kernel(const uint16_t* __restrict__ x, const uint32_t* __restrict__ qw,
             const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros,
             uint16_t* __restrict__ y, int M, int N, int K) {
#if defined(__HIP_DEVICE_COMPILE__)
  __shared__ f32x4 red[kW4Waves][RT][64];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;   // wave-uniform
  const int col = lane & 15;                 // A: row in the tile; B: token
  const int quad = lane >> 4;                // k quad of the step
  const int n0 = static_cast<int>(blockIdx.x) * (16 * RT);
  const int ngroups = K / kW4Group;
  const int per = (ngroups + kW4Waves - 1) / kW4Waves;
  const int g0 = wave * per;
  const int g1 = min(ngroups, g0 + per);
  const int kw = K / 8;                      // words per weight row
  const bool tok = col < M;
  // scale and zero point of every (row, group) of the workgroup, staged in
  // LDS once with coalesced loads as s | z << 16; rows padded by one word
  extern __shared__ uint32_t szs[];
  const int szrow = ngroups + 1;
  for (int i = tid; i < (16 * RT) * ngroups; i += kW4Waves * 64) {
    const int r = i / ngroups, g = i - r * ngroups;
    const int n = n0 + r;
    uint32_t v = 0u;
    if (n < N) {
      const int64_t o = static_cast<int64_t>(n) * ngroups + g;
      v = static_cast<uint32_t>(scales[o]) | (static_cast<uint32_t>(zeros[o]) << 16);
    }
    szs[r * szrow + g] = v;
  }

  W4Src<RT> src;
  // the ABI keeps N*K/2 and M*K*2 below 2^31 bytes, so an offset at the end
  // plus any scalar offset stays below 2^32
  src.qw_end = static_cast<uint32_t>(N) * kw * 4u;
  src.x_end = static_cast<uint32_t>(M) * K * 2u;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const uint32_t n = static_cast<uint32_t>(n0 + 16 * rt + col);
    src.vw[rt] = n < static_cast<uint32_t>(N) ? (n * kw + 4 * quad) * 4u : src.qw_end;
  }
  src.vx = tok ? (static_cast<uint32_t>(col) * K + 32 * quad) * 2u : src.x_end;
  const uint32_t kmask = 0x000F000Fu, kmagic = 0x64006400u;
  src.qw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(qw), 0, static_cast<int>(src.qw_end), 0x00020000);
  src.x = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), 0, static_cast<int>(src.x_end), 0x00020000);

  f32x4 acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // software pipeline: the loads of group g+2 are issued before group g is
  // computed, so each wave keeps two groups (about 4 KB) in flight.  Three
  // buffers take turns (unrolled by three) so that no register holding a
  // pending load is ever copied, which would force a wait.
  auto compute = [&](const W4Raw<RT>& r, int g) __attribute__((always_inline)) {
    h2 zb[RT], sc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const uint32_t v = szs[(16 * rt + col) * szrow + g];
      const uint32_t sv = v & 0xFFFFu, zv = v >> 16;
      sc[rt] = as_h2(sv | (sv << 16));
      zb[rt] = as_h2((0x6400u | zv) * 0x00010001u);
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const h8 b = permute_x(r.x[t]);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const h8 a = dequant_word(r.w[rt][t], zb[rt], sc[rt], kmask, kmagic);
        acc[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[rt], 0, 0, 0);
      }
    }
  };
  auto load = [&](W4Raw<RT>& r, int g) __attribute__((always_inline)) {
    w4_load<RT>(r, src, g, g < g1);
  };
  W4Raw<RT> ra, rb, rc;
  load(ra, g0);
  load(rb, g0 + 1);
  __syncthreads();                           // scales and zero points staged
  for (int g = g0; g < g1; g += 3) {
    load(rc, g + 2);
    compute(ra, g);
    if (g + 1 >= g1) break;
    load(ra, g + 3);
    compute(rb, g + 1);
    if (g + 2 >= g1) break;
    load(rb, g + 4);
    compute(rc, g + 2);
  }

  // partial sums of the four K slices, added in wave order
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) red[wave][rt][lane] = acc[rt];
  __syncthreads();
  for (int rt = wave; rt < RT; rt += kW4Waves) {
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
  const h8 v = dequant_word(qw[i], as_h2((0x6400u | z) * 0x00010001u), as_h2(s | (s << 16)),
                            0x000F000Fu, 0x64006400u);
  // step order (0,4,1,5,2,6,3,7) back to k order
  const h8 o = __builtin_shufflevector(v, v, 0, 2, 4, 6, 1, 3, 5, 7);
  *reinterpret_cast<u32x4*>(w + static_cast<int64_t>(n) * K + k0) = __builtin_bit_cast(u32x4, o);
#endif
}

template <int RT>
hipError_t launch_w4a16_rt(const W4Args& a) {
  const unsigned blocks = static_cast<unsigned>((a.N + 16 * RT - 1) / (16 * RT));
  const size_t lds = static_cast<size_t>(16 * RT) * (a.K / kW4Group + 1) * 4;   // staged scales
  hipLaunchKernelGGL(w4a16_kernel<RT>, dim3(blocks), dim3(kW4Waves * 64), lds,
                     static_cast<hipStream_t>(a.stream), static_cast<const uint16_t*>(a.x), a.qweight,
                     static_cast<const uint16_t*>(a.scales), a.zeros, static_cast<uint16_t*>(a.y),
                     a.M, a.N, a.K);
  return hipGetLastError();
}

}  // namespace

// Four row tiles per wave for more than four tokens when its LDS (the
// staged scales of 64 rows plus the reduction buffer) stays within 64 KB.
hipError_t launch_w4a16(const W4Args& a) {
  const size_t lds4 = static_cast<size_t>(64) * (a.K / kW4Group + 1) * 4 + sizeof(f32x4) * kW4Waves * 4 * 64;
  return (a.M > 4 && lds4 <= 65536) ? launch_w4a16_rt<4>(a) : launch_w4a16_rt<2>(a);
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
