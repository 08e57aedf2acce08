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
//                      p = exp2(S*c - m) with c = scale*log2(e), the partial
//                      output rescaled by exp2(m_old - m_new)
//   O^T += V^T P^T     P rounded to bf16, bf16 MFMA, float32 accumulate
// and after the last tile O /= l once, O rounded to bf16, LSE = ln2*(m+log2 l).
// S and P live only in registers; nothing N x N reaches memory.
//
// Layout choices (gfx950, wave64):
//  * Scores are computed transposed (keys x queries), so in the 32x32
//    accumulator layout each lane holds 16 keys of ONE query (column
//    lane%32); the row maximum and row sum are in-lane reductions plus one
//    v_permlane32_swap between the two lane halves.
//  * Those probabilities feed the second product directly as the B operand
//    (keys x queries); the key order inside each 16-key MFMA step is the
//    accumulator's order, so V^T is written to LDS in that same permuted key
//    order and every A-operand read is one 16-byte ds_read.
//  * Q is loaded once into registers (B operand of the first product); K is
//    staged row-major in LDS, V transposed; both double-buffered so tile t+1
//    is fetched from HBM while tile t is computed, with one barrier per tile.
//  * Rows are padded by 16 bytes so the 16-byte A-operand reads of 16 lanes
//    cover all LDS banks once.
#include "common.h"
#include "launch.h"

namespace attn127 {
namespace {

constexpr int NW = 4;            // waves per workgroup
constexpr int BRW = 32;          // query rows per wave
constexpr int BR = NW * BRW;     // query rows per workgroup
constexpr int BC = 64;           // keys per tile
constexpr int NT = NW * 64;      // threads per workgroup

template <int D>
struct Smem {
  static constexpr int KROW = D * 2 + 16;           // bytes per K row in LDS
  static constexpr int VROW = BC * 2 + 16;          // bytes per V^T row in LDS
  static constexpr int KBYTES = BC * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int TOTAL = 2 * STAGE;
  static constexpr int KCHUNKS = BC * D / 8 / NT;   // 16-byte K chunks per thread
  static constexpr int VTHREADS = (BC / 4) * (D / 8);  // threads owning a 4x8 V block
};

// Position of key kk (0..BC-1) inside the V^T row: within each 16-key group
// the 4-key groups 1 and 2 trade places, matching which keys a lane's
// accumulator registers 8c'..8c'+7 hold.
__device__ __forceinline__ int vt_pos(int kk) {
  const int g = (kk >> 2) & 3;
  const int sg = (g == 1) ? 2 : (g == 2 ? 1 : g);
  return (kk & ~15) | (sg << 2) | (kk & 3);
}

template <int D>
struct TileRegs {
  u32x4 kr[Smem<D>::KCHUNKS];
  u32x4 vr[4];
};

template <int D>
__device__ __forceinline__ void load_tile(TileRegs<D>& r, const uint16_t* __restrict__ kbase,
                                          const uint16_t* __restrict__ vbase, int kv0, int N,
                                          int tid) {
  using S = Smem<D>;
#pragma unroll
  for (int i = 0; i < S::KCHUNKS; ++i) {
    const int id = i * NT + tid;
    const int row = id / (D / 8), col8 = id % (D / 8);
    const int key = kv0 + row;
    r.kr[i] = (key < N) ? *reinterpret_cast<const u32x4*>(kbase + static_cast<int64_t>(key) * D + col8 * 8)
                        : u32x4{0, 0, 0, 0};
  }
  if (tid < S::VTHREADS) {
    const int kgrp = tid % (BC / 4), dchunk = tid / (BC / 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = kv0 + kgrp * 4 + e;
      r.vr[e] = (key < N) ? *reinterpret_cast<const u32x4*>(vbase + static_cast<int64_t>(key) * D + dchunk * 8)
                          : u32x4{0, 0, 0, 0};
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& r, char* stage, int tid) {
  using S = Smem<D>;
#pragma unroll
  for (int i = 0; i < S::KCHUNKS; ++i) {
    const int id = i * NT + tid;
    const int row = id / (D / 8), col8 = id % (D / 8);
    *reinterpret_cast<u32x4*>(stage + row * S::KROW + col8 * 16) = r.kr[i];
  }
  if (tid < S::VTHREADS) {
    const int kgrp = tid % (BC / 4), dchunk = tid / (BC / 4);
    char* vt = stage + S::KBYTES + vt_pos(kgrp * 4) * 2;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // channels 2w (low halves) and 2w+1 (high halves) of the 4 keys
      const uint32_t lo01 = __builtin_amdgcn_perm(r.vr[1][w], r.vr[0][w], 0x05040100u);
      const uint32_t lo23 = __builtin_amdgcn_perm(r.vr[3][w], r.vr[2][w], 0x05040100u);
      const uint32_t hi01 = __builtin_amdgcn_perm(r.vr[1][w], r.vr[0][w], 0x07060302u);
      const uint32_t hi23 = __builtin_amdgcn_perm(r.vr[3][w], r.vr[2][w], 0x07060302u);
      *reinterpret_cast<u32x2*>(vt + (dchunk * 8 + 2 * w) * S::VROW) = u32x2{lo01, lo23};
      *reinterpret_cast<u32x2*>(vt + (dchunk * 8 + 2 * w + 1) * S::VROW) = u32x2{hi01, hi23};
    }
  }
}

// v_permlane32_swap with both operands = x: lanes 0..31 get (own, partner),
// lanes 32..63 get (partner, own), where partner is the lane 32 away; the
// combination of the pair is therefore the same reduction on every lane.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(NT, 2)
attn_mfma_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                      float* __restrict__ lse, int N, int BH, int nqb, float c) {
  using S = Smem<D>;
  __shared__ __attribute__((aligned(16))) char smem[S::TOTAL];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int j = lane & 31;        // query column inside the wave's 32
  const int h = lane >> 5;        // lane half

  // Work item: causal blocks are issued heaviest (last query block) first.
  int bh, qb;
  if (CAUSAL) {
    qb = nqb - 1 - static_cast<int>(blockIdx.x / BH);
    bh = static_cast<int>(blockIdx.x % BH);
  } else {
    bh = static_cast<int>(blockIdx.x / nqb);
    qb = static_cast<int>(blockIdx.x % nqb);
  }
  const int q0 = qb * BR;
  const int q0w = q0 + wave * BRW;
  const int qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint16_t* kbase = k + base;
  const uint16_t* vbase = v + base;

  // Q^T as the B operand: lane (j, h) holds channels ks*16 + 8h .. +7 of row qrow.
  bf16x8 qr[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    u32x4 x = (qrow < N) ? *reinterpret_cast<const u32x4*>(q + base + static_cast<int64_t>(qrow) * D + ks * 16 + 8 * h)
                         : u32x4{0, 0, 0, 0};
    qr[ks] = __builtin_bit_cast(bf16x8, x);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  const int kend = CAUSAL ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  const bool wave_live = q0w < N;

  TileRegs<D> regs;
  load_tile<D>(regs, kbase, vbase, 0, N, tid);
  store_tile<D>(regs, smem, tid);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BC;
    const bool more = t + 1 < ntiles;
    if (more) load_tile<D>(regs, kbase, vbase, kv0 + BC, N, tid);
    const char* stage = smem + (t & 1) * S::STAGE;

    const bool wave_needs = wave_live && (!CAUSAL || kv0 <= q0w + BRW - 1);
    if (wave_needs) {
      // ---- S^T = K Q^T for the tile's BC keys (two 32-key blocks) ----
      f32x16 sacc[BC / 32];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
        sacc[kb] = f32x16{};
        const char* krow = stage + (kb * 32 + j) * S::KROW + 16 * h;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(krow + ks * 32);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[ks], sacc[kb], 0, 0, 0);
        }
      }
      // ---- masks: causal diagonal tiles, keys past the sequence end ----
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > q0w) || (kv0 + BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
            const bool masked = (key >= N) || (CAUSAL && key > qrow);
            if (masked) sacc[kb][r] = -INFINITY;
          }
      }
      // ---- online softmax (base 2) ----
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = halves_max(mx);
      const float mnew = fmaxf(m, mx * c);
      const float mref = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(m - mref);
      m = mnew;
      float psum = 0.f;
      uint32_t pw[BC / 16][4];
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(sacc[kb][r], c, -mref));
          const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], c, -mref));
          psum += p0 + p1;
          // accumulator registers 8c'..8c'+7 of block kb form operand 2kb+c'
          pw[kb * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
        }
      }
      bf16x8 pb[BC / 16];
#pragma unroll
      for (int c16 = 0; c16 < BC / 16; ++c16)
        pb[c16] = __builtin_bit_cast(bf16x8, u32x4{pw[c16][0], pw[c16][1], pw[c16][2], pw[c16][3]});
      lsum = lsum * alpha + psum;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      // ---- O^T += V^T P^T ----
      const char* vt = stage + S::KBYTES;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const char* vrow = vt + (db * 32 + j) * S::VROW + 16 * h;
#pragma unroll
        for (int c16 = 0; c16 < BC / 16; ++c16) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vrow + c16 * 32);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[c16], oacc[db], 0, 0, 0);
        }
      }
    }
    if (more) store_tile<D>(regs, smem + ((t + 1) & 1) * S::STAGE, tid);
    __syncthreads();
  }

  // ---- epilogue: the deferred division, bf16 output, LSE ----
  const float ltot = halves_sum(lsum);
  if (qrow < N) {
    const float inv = 1.f / ltot;
    uint16_t* orow = o + base + static_cast<int64_t>(qrow) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = db * 32 + 8 * g + 4 * h;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + col) = w;
      }
    if (lse != nullptr && h == 0)
      lse[static_cast<int64_t>(bh) * N + qrow] = (m + __log2f(ltot)) * kLn2;
  }
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
