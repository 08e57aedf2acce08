// Fused exact attention forward on bf16 matrix cores (gfx950).
//
// Algorithm (page "Self-Attention, CUDA kernels and FlashAttention",
// section 3; page "FlashAttention scaling, multi-GPU training and weight
// quantization", section 1, FlashAttention-2 bullets): one workgroup per
// (batch*head, block of BR query rows) -- the outer loop over query blocks is
// the grid, so even one head fills the machine at long sequence length --
// and an inner loop over key/value tiles of BC keys.  Per tile:
//   S^T = K Q^T        bf16 MFMA 32x32x16, float32 accumulate
//   online softmax     running row maximum m and normaliser l in registers,
//                      p = exp2(S*c - m) with c = scale*log2(e)
//   O^T += V^T P^T     P rounded to bf16, bf16 MFMA, float32 accumulate
// and after the last tile O /= l once, O rounded to bf16, LSE = ln2*(m+log2 l).
// S and P live only in registers; nothing N x N reaches memory.
//
// gfx950 mapping:
//  * Scores are computed transposed (keys x queries): in the 32x32
//    accumulator layout each lane then holds 16 keys of ONE query (column
//    lane%32), so the row maximum and row sum are in-lane reductions plus one
//    v_permlane32_swap between the two lane halves.
//  * Those probabilities feed the second product directly as its B operand;
//    its A operand (V^T) comes from row-major V in LDS through
//    ds_read_b64_tr_b16, which hands each lane four keys of one channel, read
//    in exactly the key order the accumulator registers hold.
//  * K and V tiles go from HBM straight into LDS (buffer_load ... lds, 16
//    bytes per lane, no register staging), double-buffered so tile t+1 is in
//    flight while tile t is computed; one barrier per tile.  Out-of-range
//    rows of the last tile read as zero (buffer bounds).  16-byte chunks are
//    XOR-swizzled per row so the matrix-operand reads hit distinct banks.
//  * The running maximum used as the exponent reference is only raised when
//    some row's tile maximum exceeds it by more than 2^kTau (base 2); p then
//    stays <= 2^kTau, the normaliser and the partial output carry the same
//    reference, and the single division at the end cancels it exactly.  Most
//    tiles of a long row therefore skip the rescale of the partial output.
//  * Work items are grouped by XCD (dispatch is round-robin over the 8 XCDs)
//    so the query blocks of one head share one L2, heaviest causal blocks
//    first.
#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int NW = 4;            // waves per workgroup
constexpr int BRW = 32;          // query rows per wave
constexpr int BR = NW * BRW;     // query rows per workgroup
constexpr int BC = 64;           // keys per tile
constexpr int NT = NW * 64;      // threads per workgroup
constexpr float kTau = 8.0f;     // allowed growth of p above 1, as a power of two
constexpr int kXcds = 8;

template <int D>
struct Cfg {
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;      // rows per 1 KB load block
  static constexpr int TILEB = BC * ROWB;      // bytes of one K (or V) tile
  static constexpr int BLK = TILEB / 1024;     // 1 KB blocks per tile
  static constexpr int BPW = BLK / NW;         // blocks per wave per tile
  static_assert(BPW * NW == BLK, "tile must split evenly over the waves");
};

// Chunk swizzles (XOR on the 16-byte chunk index within a row).  K: the 16
// rows read together by one operand load land on 16 different chunk
// positions.  V: the 4 rows x 4 chunks read by one transposing load of half
// a wave land on 16 different chunk positions.
template <int D>
__device__ __forceinline__ int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int vswz(int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

// Device-only helpers (gfx950 builtins have no host-side meaning).
#if defined(__HIP_DEVICE_COMPILE__)
typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// generic pointer into a __shared__ array -> LDS address space (C-style cast:
// the address-space change is not expressible with the C++ casts)
__device__ __forceinline__ lds_void* as_lds(const char* p) { return (lds_void*)(const_cast<char*>(p)); }
__device__ __forceinline__ v4i16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<char*>(p)));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Start the HBM -> LDS copy of K and V rows [kv0, kv0+BC) into one stage.
template <int D>
__device__ __forceinline__ void issue_tile(char* kst, char* vst, const uint16_t* kbase,
                                           const uint16_t* vbase, int kv0, int N, int wave,
                                           int lane) {
  using C = Cfg<D>;
  const int rows = min(BC, N - kv0);
  const uint32_t bytes = static_cast<uint32_t>(rows) * C::ROWB;
  const auto rk = make_rsrc(kbase + static_cast<int64_t>(kv0) * D, bytes);
  const auto rv = make_rsrc(vbase + static_cast<int64_t>(kv0) * D, bytes);
#pragma unroll
  for (int b = 0; b < C::BPW; ++b) {
    const int blk = wave * C::BPW + b;
    const int row = blk * C::RPB + lane / C::CPR;
    const int pos = lane % C::CPR;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rk, as_lds(kst + blk * 1024), 16,
        row * C::ROWB + ((pos ^ kswz<D>(row)) << 4), 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rv, as_lds(vst + blk * 1024), 16,
        row * C::ROWB + ((pos ^ vswz<D>(row)) << 4), 0, 0, 0);
  }
}

// v_permlane32_swap with both operands = x: lanes 0..31 get (own, partner),
// lanes 32..63 get (partner, own), partner being the lane 32 away; combining
// the pair gives the same two-lane reduction on every lane.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct WaveState {
  bf16x8 qr[D / 16];          // Q^T operand: channels ks*16 + 8h .. +7 of the lane's row
  f32x16 oacc[D / 32];        // O^T accumulator: 32 channels x 32 rows per block
  float m;                    // exponent reference (base 2), -inf before the first tile
  float lsum;                 // this lane half's share of the normaliser
};

// One key tile for one wave: scores, masks, online softmax, P V.
template <int D, bool CAUSAL>
__device__ __forceinline__ void tile_step(WaveState<D>& w, const char* kst, const char* vst,
                                          int kv0, int N, int q0w, int qrow, int j, int h,
                                          int lane, float c) {
  using C = Cfg<D>;
  // ---- S^T = K Q^T (two 32-key blocks) ----
  f32x16 sacc[BC / 32];
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb) {
    const int row = kb * 32 + j;
    const char* krow = kst + row * C::ROWB;
    const int sw = kswz<D>(row);
    bf16x8 a[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      a[ks] = *reinterpret_cast<const bf16x8*>(krow + (((2 * ks + h) ^ sw) << 4));
    sacc[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], w.qr[ks], sacc[kb], 0, 0, 0);
  }
  // ---- masks: keys past the diagonal (causal), keys past the end ----
  const bool need_mask = (CAUSAL && kv0 + BC - 1 > q0w) || (kv0 + BC > N);
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool masked = (key >= N) || (CAUSAL && key > qrow);
        sacc[kb][r] = masked ? -INFINITY : sacc[kb][r];
      }
  }
  // ---- online softmax (base 2), reference raised only when needed ----
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  const float mt = halves_max(mx) * c;
  if (__builtin_amdgcn_ballot_w64(mt > w.m + kTau) != 0) {
    const float mnew = fmaxf(w.m, mt);
    const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(w.m - mnew);
    w.lsum *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) w.oacc[db] *= alpha;
    w.m = mnew;
  }
  const float mref = (w.m == -INFINITY) ? 0.f : w.m;
  uint32_t pw[BC / 16][4];
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(fmaf(sacc[kb][r], c, -mref));
      const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], c, -mref));
      // the normaliser sums the float32 p (two chains for latency)
      ls0 += p0;
      ls1 += p1;
      // accumulator registers 8c'..8c'+7 of block kb form operand 2kb+c'
      pw[kb * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
    }
  w.lsum += ls0 + ls1;
  bf16x8 pb[BC / 16];
#pragma unroll
  for (int c16 = 0; c16 < BC / 16; ++c16)
    pb[c16] = __builtin_bit_cast(bf16x8, u32x4{pw[c16][0], pw[c16][1], pw[c16][2], pw[c16][3]});
  // ---- O^T += V^T P^T: A operand through transposing LDS reads ----
  const int g16 = lane >> 4, r16 = lane & 15;
  const int b16 = g16 & 1;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int chunk = db * 4 + 2 * b16 + ((r16 & 3) >> 1);
    const int half8 = (r16 & 1) << 3;
#pragma unroll
    for (int c16 = 0; c16 < BC / 16; ++c16) {
      const int key0 = c16 * 16 + 4 * h + (r16 >> 2);
      const int key1 = key0 + 8;
      const v4i16 lo = ds_read_tr16(vst + key0 * C::ROWB + ((chunk ^ vswz<D>(key0)) << 4) + half8);
      const v4i16 hi = ds_read_tr16(vst + key1 * C::ROWB + ((chunk ^ vswz<D>(key1)) << 4) + half8);
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c16], w.oacc[db], 0, 0, 0);
    }
  }
}

#endif  // __HIP_DEVICE_COMPILE__

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT, 2)
attn_mfma_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                      float* __restrict__ lse, int N, int BH, int nqb, float c) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D>;
  // two stages, each a separate array so the compiler can tell the copy in
  // flight from the tile being read
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILEB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;        // query column inside the wave's 32 rows
  const int h = lane >> 5;        // lane half

  // ---- work item: XCD-grouped heads, heaviest causal blocks first ----
  const int id = static_cast<int>(blockIdx.x);
  int bh, qb;
  if (BH % kXcds == 0) {
    const int x = id % kXcds, s = id / kXcds, hx = BH / kXcds;
    if (CAUSAL) { qb = nqb - 1 - s / hx; bh = x + kXcds * (s % hx); }
    else        { bh = x + kXcds * (s / nqb); qb = s % nqb; }
  } else if (CAUSAL) {
    qb = nqb - 1 - id / BH; bh = id % BH;
  } else {
    bh = id / nqb; qb = id % nqb;
  }
  const int q0 = qb * BR;
  const int q0w = q0 + wave * BRW;
  const int qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint16_t* kbase = k + base;
  const uint16_t* vbase = v + base;

  WaveState<D> w;
  {
    const int rows = max(0, min(BRW, N - q0w));
    const auto rq = make_rsrc(q + base + static_cast<int64_t>(min(q0w, N)) * D,
                              static_cast<uint32_t>(rows) * C::ROWB);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rq, j * C::ROWB + (ks * 16 + 8 * h) * 2, 0, 0);
      w.qr[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }
#pragma unroll
  for (int db = 0; db < D / 32; ++db) w.oacc[db] = f32x16{};
  w.m = -INFINITY;
  w.lsum = 0.f;

  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const bool wave_live = q0w < N;

  issue_tile<D>(k0s, v0s, kbase, vbase, 0, N, wave, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Two tiles per trip so each stage is a fixed array.
  for (int t = 0; t < ntiles; t += 2) {
    {
      const int kv0 = t * BC;
      if (t + 1 < ntiles) issue_tile<D>(k1s, v1s, kbase, vbase, kv0 + BC, N, wave, lane);
      if (wave_live && (!CAUSAL || kv0 <= q0w + BRW - 1))
        tile_step<D, CAUSAL>(w, k0s, v0s, kv0, N, q0w, qrow, j, h, lane, c);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    if (t + 1 < ntiles) {
      const int kv0 = (t + 1) * BC;
      if (t + 2 < ntiles) issue_tile<D>(k0s, v0s, kbase, vbase, kv0 + BC, N, wave, lane);
      if (wave_live && (!CAUSAL || kv0 <= q0w + BRW - 1))
        tile_step<D, CAUSAL>(w, k1s, v1s, kv0, N, q0w, qrow, j, h, lane, c);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
  }

  // ---- epilogue: the deferred division, bf16 output, LSE ----
  const float ltot = halves_sum(w.lsum);
  if (qrow < N) {
    const float inv = 1.f / ltot;
    uint16_t* orow = o + base + static_cast<int64_t>(qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = db * 32 + 8 * g + 4 * h;
        u32x2 wv;
        wv[0] = pack_bf16x2(w.oacc[db][4 * g + 0] * inv, w.oacc[db][4 * g + 1] * inv);
        wv[1] = pack_bf16x2(w.oacc[db][4 * g + 2] * inv, w.oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + col) = wv;
      }
    if (lse != nullptr && h == 0)
      lse[static_cast<int64_t>(bh) * N + qrow] = (w.m + __log2f(ltot)) * kLn2;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool CAUSAL>
hipError_t launch_one(const LaunchArgs& a) {
  const int BH = a.B * a.H;
  const int nqb = (a.N + BR - 1) / BR;
  const int64_t blocks = static_cast<int64_t>(nqb) * BH;
  hipLaunchKernelGGL((attn_mfma_bf16_kernel<D, CAUSAL>), dim3(static_cast<unsigned>(blocks)),
                     dim3(NT), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                     a.N, BH, nqb, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_mfma_bf16(const LaunchArgs& a) {
  if (a.d == 64) return a.causal ? launch_one<64, true>(a) : launch_one<64, false>(a);
  return a.causal ? launch_one<128, true>(a) : launch_one<128, false>(a);
}

}  // namespace attn127
