// Backward pass of exact attention on bf16 matrix cores (gfx950).
//
// The page "Self-Attention, CUDA kernels and FlashAttention", section 3:
// the backward pass keeps only the small per-row statistics of the forward
// pass (here the natural-log LSE) and recomputes the attention tiles on chip.
// With c = scale*log2(e), per head:
//   P   = exp2(c*Q K^T - log2(e)*LSE)        recomputed tile by tile (masked)
//   dV  = P^T dO
//   dP  = dO V^T
//   D_i = sum_c dO_ic O_ic                   (equals sum_j P_ij dP_ij)
//   dS  = P * (dP - D)
//   dQ  = scale * dS K,   dK = scale * dS^T Q
// Nothing N x N reaches memory.  Three launches, no atomics:
//  * bwd_delta_kernel: D for every row (HBM-bound).
//  * bwd_dkdv_kernel: one workgroup per (b*h, block of keys); each wave keeps
//    its keys' K rows in registers and the block's V sits in LDS; Q / dO
//    tiles stream through a two-slot ring shared by the workgroup.  Each
//    wave owns 32 keys, so S = Q K^T and dP = dO V^T are computed with the
//    key in the accumulator column: every lane holds 16 queries of one key,
//    which is the B-operand layout that dV^T += dO^T P and dK^T += Q^T dS
//    need (dO^T, Q^T come from transposing LDS reads).
//  * bwd_dq_kernel: one workgroup per (b*h, block of queries), laid out like
//    the forward kernel: S^T = K Q^T and dP^T = V dO^T put the query in the
//    column, so LSE and D are one register per lane, and dQ^T += K^T dS^T
//    reads K^T through transposing LDS reads.
// K, V, Q and dO tiles are each read both row-wise (16-byte reads) and
// transposed (ds_read_b64_tr_b16); one XOR swizzle of the 16-byte chunks
// keeps both patterns free of LDS bank conflicts.
#include <type_traits>

#include "common.h"
#include "launch.h"
#if defined(__HIP_DEVICE_COMPILE__)
#include "device_util.h"
#endif

namespace attn127 {
namespace {

constexpr int BT = 64;        // rows per streamed tile (keys in dQ, queries in dK/dV)
constexpr int kXcdsB = 8;     // XCDs the dispatcher round-robins over
constexpr int kRingB = 3;     // K (and V) tiles resident in the dQ kernel's LDS

template <int D>
struct BTile {
  static constexpr int ROWB = 2 * D;          // bytes per bf16 row
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;     // rows per 1 KB copy block
  static constexpr int TILEB = BT * ROWB;     // bytes of one tile
  static constexpr int BLK = TILEB / 1024;    // 1 KB blocks per tile
};

// Chunk swizzle of row `row`.  d=128 (16 chunks, 256-byte rows): the
// row-wise reads of 16 consecutive rows need 16 distinct chunk positions
// (the two 2-bit fields of the row's low nibble, swapped, are a bijection),
// and the 4 rows x 2 chunks of one transposing read need 8 (the row's low
// two bits move the chunk's high bits).  d=64 (8 chunks, 128-byte rows, two
// rows per bank window): the same two requirements per row parity.
template <int D>
__host__ __device__ constexpr int bswz(int row) {
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 1) | (((row >> 2) & 1) << 2) | ((row >> 3) & 1));
}

#if defined(__HIP_DEVICE_COMPILE__)
// Buffer descriptor forced into scalar registers (the copy instructions take
// it as a scalar operand; every field is the same on all lanes).
__device__ __forceinline__ i32x4 uniform_desc(const void* base, uint32_t bytes) {
  const i32x4 d = buffer_desc(base, bytes);
  return i32x4{__builtin_amdgcn_readfirstlane(d[0]), __builtin_amdgcn_readfirstlane(d[1]),
               __builtin_amdgcn_readfirstlane(d[2]), __builtin_amdgcn_readfirstlane(d[3])};
}

// One 4-byte-per-lane HBM -> LDS copy: lane i's word lands at lds + 4*i.
__device__ __forceinline__ void dma4(const i32x4& desc, const char* lds_block, int voffset) {
  const uint32_t m = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(as_lds(lds_block))));
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(m), "v"(voffset), "s"(desc) : "memory", "m0");
#pragma clang diagnostic pop
}

// Rows [r0, r0+BT) of a [N][D] bf16 slice -> one LDS tile (rows past N read
// as zero); the workgroup's NW waves share the tile's 1 KB blocks.
template <int D, int NW>
__device__ __forceinline__ void copy_tile(char* dst, const uint16_t* src, int r0, int N, int wave,
                                          int lane) {
  using T = BTile<D>;
  static_assert(T::BLK % NW == 0, "tile must split evenly over the waves");
  constexpr int BPW = T::BLK / NW;
  const int rows = min(BT, N - r0);
  const i32x4 desc = uniform_desc(src + static_cast<int64_t>(r0) * D,
                                  static_cast<uint32_t>(max(rows, 0)) * T::ROWB);
#pragma unroll
  for (int b = 0; b < BPW; ++b) {
    const int blk = wave * BPW + b;
    const int row = blk * T::RPB + lane / T::CPR;
    const int pos = lane % T::CPR;
    dma16(desc, dst + blk * 1024, row * T::ROWB + ((pos ^ bswz<D>(row)) << 4));
  }
}

// Lane-constant LDS offsets.  Row reads (operand rows j and j+32 of a tile,
// channels 16ks+8h..+7): rofs[ks].  Transposing reads of channel block db:
// rows key0 + 8i (+16 per 16-row group), tofs[db][i]; the swizzle of those
// rows depends only on i.
template <int D>
struct BLane {
  int rofs[D / 16];
  int tofs[D / 32][2];
  __device__ __forceinline__ BLane(int j, int h, int lane) {
    using T = BTile<D>;
    const int sj = bswz<D>(j);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) rofs[ks] = j * T::ROWB + (((2 * ks + h) ^ sj) << 4);
    const int r16 = lane & 15, b16 = (lane >> 4) & 1;
    const int key0 = 4 * h + (r16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int chunk = db * 4 + 2 * b16 + ((r16 & 3) >> 1);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = key0 + 8 * i;
        tofs[db][i] = row * T::ROWB + ((chunk ^ bswz<D>(row)) << 4) + ((r16 & 1) << 3);
      }
    }
  }
};

__device__ __forceinline__ bf16x8 lds_row(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }

// Transposed operand: channels 32db + lane%32, 16 rows of group g16 (rows
// 16 g16 .. +15 of the tile) in the order of a 32x32 accumulator's rows.
template <int D>
__device__ __forceinline__ bf16x8 lds_trans(const char* tile, const BLane<D>& la, int db, int g16) {
  const int off = g16 * 16 * BTile<D>::ROWB;
  const v4i16 lo = ds_read_tr16(tile + la.tofs[db][0] + off);
  const v4i16 hi = ds_read_tr16(tile + la.tofs[db][1] + off);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Store a 32x32 accumulator block (rows: channels 32db + 8g + 4h + 0..3;
// columns: the wave's 32 rows r0 .. r0+31 of a [N][D] output), times `mul`,
// as bf16 through LDS: the rows go to the wave's own
// idle LDS region `stage` (rows of 2D bytes, 16-byte chunks swizzled by the
// row so that one instruction's 8-byte writes spread over the banks) and
// are stored in row order, each store instruction writing whole rows (1 KB
// contiguous) instead of 8-byte pieces of 32 rows.  Rows at or past N are
// not stored.
template <int D>
__device__ __forceinline__ void store_rows_lds(uint16_t* out, int r0, int N, const f32x16 (&acc)[D / 32],
                                               float mul, char* stage, int j, int h, int lane) {
  constexpr int RB = 2 * D, CPR = RB / 16, RPI = 64 / CPR;
  char* row = stage + j * RB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = db * 4 + g;             // chunk of channels 8c..8c+7; the lane holds 8c + 4h .. +3
      u32x2 wv;
      wv[0] = pack_bf16x2(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul);
      wv[1] = pack_bf16x2(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
      *reinterpret_cast<u32x2*>(row + ((c ^ (j % CPR)) << 4) + 8 * h) = wv;
    }
  // stores through a descriptor that covers the valid rows only: rows at or
  // past N are dropped by its range check, without a branch
  const int r0u = __builtin_amdgcn_readfirstlane(r0);
  const int rows = max(0, min(32, N - r0u));
  const auto rs = uniform_rsrc(out + static_cast<int64_t>(min(r0u, N)) * D, rows * RB);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, c = lane % CPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * RB + ((c ^ (r % CPR)) << 4));
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, r * RB + c * 16, 0, 0);
  }
}
#endif  // __HIP_DEVICE_COMPILE__

// ---- D_i = sum_c dO_ic O_ic, float32, one row per D/8 lanes ----
template <int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int LPR = D / 8;          // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  const int64_t row = static_cast<int64_t>(blockIdx.x) * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(o + row * D + part * 8);
    const u32x4 b = *reinterpret_cast<const u32x4*>(dout + row * D + part * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc = fmaf(__uint_as_float(a[w] << 16), __uint_as_float(b[w] << 16), acc);
      acc = fmaf(__uint_as_float(a[w] & 0xFFFF0000u), __uint_as_float(b[w] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (row < rows && part == 0) delta[row] = acc;
#endif
}

// ---- dQ: query-major, K/V tiles streamed through three-slot rings ----
//
// Per 32-key block b of the wave: A_b = the products S^T = K Q^T and
// dP^T = V dO^T (16 MFMAs at d=128), V_b = the vector work dS^T = P^T
// (dP^T - D) with P^T = exp2(S^T c - LSE) (8 pairs of scores per lane),
// C_b = dQ^T += K^T dS^T (8 MFMAs).  The blocks are software-pipelined: phase
// b runs A_{b+1} slot by slot beside V_b (one MFMA, its operand read two
// ahead and a share of the vector work per slot, closed by a scheduling
// barrier; empty asm uses keep the vector work in its slot), then C_b.  So
// the matrix cores and the vector ALU work side by side in one wave, where
// the eight waves, held in step by the per-tile barrier, would otherwise all
// wait on the same unit.  Tile t carries blocks 2t and 2t+1; iteration t runs
// phases 2t-1 and 2t, which read K of tiles t-1 and t, hence three K slots.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1)
bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
              const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
              const float* __restrict__ lse, const float* __restrict__ delta,
              uint16_t* __restrict__ dq, int N, int BH, int nqb, float c, float scale,
              int causal_arg, int hc) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = BTile<D>;
  constexpr int BR = NW * 32;
  const bool causal = causal_arg != 0;
  __shared__ __attribute__((aligned(1024))) char smem[2 * kRingB * T::TILEB];   // K ring, then V ring
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, j = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);   // the same value, known uniform

  // work item: whole heads per XCD, heaviest causal query blocks first
  const int id = static_cast<int>(blockIdx.x);
  int bh, qb;
  if (BH % kXcdsB == 0) {
    const int x = id % kXcdsB, s = id / kXcdsB;
    if (causal) {   // chunks of hc heads, each chunk's blocks heaviest first
      const int per = hc * nqb, ch = s / per, r = s - ch * per;
      qb = nqb - 1 - r / hc; bh = x + kXcdsB * (ch * hc + r % hc);
    } else {
      bh = x + kXcdsB * (s / nqb); qb = s % nqb;
    }
  } else if (causal) {
    qb = nqb - 1 - id / BH; bh = id % BH;
  } else {
    bh = id / nqb; qb = id % nqb;
  }
  // row blocks r and 7-r share a SIMD (waves w and w+4 do), so the causal
  // diagonal leaves every SIMD the same idle work, as in the forward kernel
  const int rgp = NW == 8 ? (wave < 4 ? wave : 11 - wave) : wave;
  const int q0 = qb * BR, q0w = q0 + rgp * 32, qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint16_t* kbase = k + base;
  const uint16_t* vbase = v + base;

  const int kend = causal ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BT - 1) / BT;
  // last 32-key block this wave needs (-1: its rows are all past the end)
  int lb = -1;
  if (q0w < N) lb = causal ? min((N - 1) / 32, (q0w + 31) / 32) : (N - 1) / 32;
  auto kslot = [&](int r) __attribute__((always_inline)) -> const char* { return smem + r * T::TILEB; };           // r = tile % 3
  auto vslot = [&](int r) __attribute__((always_inline)) -> const char* { return smem + (kRingB + r) * T::TILEB; };
  if (ntiles > 0) {
    copy_tile<D, NW>(smem, kbase, 0, N, wave_u, lane);
    copy_tile<D, NW>(smem + kRingB * T::TILEB, vbase, 0, N, wave_u, lane);
  }
  // this lane's Q and dO row as B operands (rows past N read as zero)
  bf16x8 qr[D / 16], dor[D / 16];
  {
    const int rows = max(0, min(32, N - q0w));
    const int64_t r0 = base + static_cast<int64_t>(min(q0w, N)) * D;
    const auto rq = uniform_rsrc(q + r0, rows * T::ROWB);
    const auto rd = uniform_rsrc(dout + r0, rows * T::ROWB);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int off = j * T::ROWB + (ks * 16 + 8 * h) * 2;
      qr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      dor[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0));
    }
  }
  float lse2 = 0.f, dl = 0.f;
  if (qrow < N) {
    lse2 = lse[static_cast<int64_t>(bh) * N + qrow] * kLog2e;
    dl = delta[static_cast<int64_t>(bh) * N + qrow];
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};
  const BLane<D> la(j, h, lane);
  wait_vmcnt<0>();
  __syncthreads();

  constexpr int NA = 2 * (D / 16);              // MFMAs of A (S^T, then dP^T)
  constexpr int NC = 2 * (D / 32);              // MFMAs of C
  // A operand of MFMA i of block b: a K row (S^T) or a V row (dP^T)
  auto a_op = [&](const char* kst, const char* vst, int kb, int i) __attribute__((always_inline)) {
    return i < D / 16 ? lds_row(kst + kb * 32 * T::ROWB + la.rofs[i])
                      : lds_row(vst + kb * 32 * T::ROWB + la.rofs[i - D / 16]);
  };
  auto a_mfma = [&](f32x16& sacc, f32x16& dpacc, const bf16x8& a, int i) __attribute__((always_inline)) {
    if (i < D / 16) sacc = mfma(a, qr[i], i == 0 ? f32x16{} : sacc);
    else dpacc = mfma(a, dor[i - D / 16], i == D / 16 ? f32x16{} : dpacc);
  };
  // keys of block b past the sequence end or (causal) past this lane's row
  // get S = -inf, so P = 0 and dS = 0 there
  auto mask_block = [&](f32x16& sacc, int b) __attribute__((always_inline)) {
    const int base_key = 32 * b + 4 * h;
    const int lim = causal ? min(N - 1, qrow) - base_key : N - 1 - base_key;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = (8 * (r >> 2) + (r & 3)) > lim ? -INFINITY : sacc[r];
  };
  auto needs_mask = [&](int b) __attribute__((always_inline)) { return (causal && 32 * b + 31 > q0w) || 32 * b + 32 > N; };
  // dS^T for pair pr (accumulator registers 2pr, 2pr+1) into operand word dsw
  auto ds_pair = [&](uint32_t (&dsw)[2][4], const f32x16& sacc, const f32x16& dpacc, int pr) __attribute__((always_inline)) {
    const int r = 2 * pr;
    const float d0 = fast_exp2(fmaf(sacc[r], c, -lse2)) * (dpacc[r] - dl);
    const float d1 = fast_exp2(fmaf(sacc[r + 1], c, -lse2)) * (dpacc[r + 1] - dl);
    dsw[r >> 3][(r & 7) >> 1] = pack_bf16x2(d0, d1);
  };
  auto c_mfmas = [&](const uint32_t (&dsw)[2][4], const char* kst, int kb) __attribute__((always_inline)) {
    bf16x8 ktr[NC];
    ktr[0] = lds_trans<D>(kst, la, 0, 2 * kb);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if (i + 1 < NC) ktr[i + 1] = lds_trans<D>(kst, la, (i + 1) % (D / 32), 2 * kb + (i + 1) / (D / 32));
      const int cg = i / (D / 32), db = i % (D / 32);
      const bf16x8 dsb = __builtin_bit_cast(bf16x8, u32x4{dsw[cg][0], dsw[cg][1], dsw[cg][2], dsw[cg][3]});
      acc[db] = mfma(ktr[i], dsb, acc[db]);
    }
  };
  auto pin = [](auto x) __attribute__((always_inline)) { asm volatile("" ::"v"(x)); };
  // phase b: A_{b+1} beside V_b, then C_b.  (sc, dpc): products of block b;
  // (sn, dpn): receive those of block b+1.  ks*/vs*: LDS tiles of the two blocks.
  auto phase = [&](int b, auto kbc, f32x16& sc, f32x16& dpc, f32x16& sn, f32x16& dpn,
                   const char* kst_b, const char* kst_n, const char* vst_n) __attribute__((always_inline)) {
    constexpr int kb = decltype(kbc)::value, kbn = 1 - kb;   // b & 1, (b + 1) & 1
    const bool do_a = b + 1 <= lb, do_vc = b >= 0 && b <= lb;
    uint32_t dsw[2][4];
    if (do_vc && needs_mask(b)) mask_block(sc, b);
    if (do_a && do_vc) {
      bf16x8 aop[NA];
      __builtin_amdgcn_sched_barrier(0);
      aop[0] = a_op(kst_n, vst_n, kbn, 0);
      aop[1] = a_op(kst_n, vst_n, kbn, 1);
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + 2 < NA) aop[i + 2] = a_op(kst_n, vst_n, kbn, i + 2);
        a_mfma(sn, dpn, aop[i], i);
#pragma unroll
        for (int pr = 0; pr < 8; ++pr) {
          if ((pr * NA) / 8 != i) continue;
          ds_pair(dsw, sc, dpc, pr);
          pin(dsw[pr >> 2][pr & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      c_mfmas(dsw, kst_b, kb);
    } else if (do_a) {
#pragma unroll
      for (int i = 0; i < NA; ++i) a_mfma(sn, dpn, a_op(kst_n, vst_n, kbn, i), i);
    } else if (do_vc) {
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) ds_pair(dsw, sc, dpc, pr);
      c_mfmas(dsw, kst_b, kb);
    }
  };

  // iteration t (R = t mod 3, a compile-time slot index): copy tile t+1,
  // run phases 2t-1 (A of block 2t, C of block 2t-1) and 2t (A of block
  // 2t+1, C of block 2t)
  f32x16 se = f32x16{}, dpe = f32x16{}, so = f32x16{}, dpo = f32x16{};   // even / odd blocks
  auto iteration = [&](int t, auto rc) __attribute__((always_inline)) {
    constexpr int R = decltype(rc)::value;
    constexpr int RP = (R + 2) % 3, RN = (R + 1) % 3;
    if (t + 1 < ntiles) {
      copy_tile<D, NW>(smem + RN * T::TILEB, kbase, (t + 1) * BT, N, wave_u, lane);
      copy_tile<D, NW>(smem + (kRingB + RN) * T::TILEB, vbase, (t + 1) * BT, N, wave_u, lane);
    }
    phase(2 * t - 1, std::integral_constant<int, 1>{}, so, dpo, se, dpe, kslot(RP), kslot(R), vslot(R));
    phase(2 * t, std::integral_constant<int, 0>{}, se, dpe, so, dpo, kslot(R), kslot(R), vslot(R));
    wait_vmcnt<0>();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 3) {
    iteration(t, std::integral_constant<int, 0>{});
    if (t + 1 < ntiles) iteration(t + 1, std::integral_constant<int, 1>{});
    if (t + 2 < ntiles) iteration(t + 2, std::integral_constant<int, 2>{});
  }
  // the last block's vector work and C (its tile is still in LDS)
  if (ntiles > 0) {
    const int r = (ntiles - 1) % 3;
    phase(2 * ntiles - 1, std::integral_constant<int, 1>{}, so, dpo, se, dpe, kslot(r), kslot(r), vslot(r));
  }
  __syncthreads();   // every wave is done with the rings (the last block read its K tile)
  static_assert(NW * 32 * 2 * D <= static_cast<int>(sizeof(smem)), "dQ staging fits the rings");
  store_rows_lds<D>(dq + base, q0w, N, acc, scale, smem + wave_u * (32 * 2 * D), j, h, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---- dK, dV: key-major; each wave's K and V rows in registers, Q/dO tiles streamed ----
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1)
bwd_dkdv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                const float* __restrict__ lse, const float* __restrict__ delta,
                uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int N, int BH, int nkb,
                float c, float scale, int causal_arg, int hc) {
#if defined(__HIP_DEVICE_COMPILE__)
  using T = BTile<D>;
  constexpr int BK = NW * 32;                  // keys per workgroup
  constexpr int SB = 2 * BT * 4;               // LSE and D of one query tile
  const bool causal = causal_arg != 0;
  constexpr int VB = BK * T::ROWB;             // V rows of the block
  static_assert(BK % BT == 0, "key block is whole tiles");
  __shared__ __attribute__((aligned(1024))) char smem[VB + 4 * T::TILEB + 2 * SB];
  char* const vt = smem;
  char* const qring = smem + VB;
  char* const dring = qring + 2 * T::TILEB;
  char* const sring = dring + 2 * T::TILEB;    // [slot][LSE BT floats | D BT floats]
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, j = lane & 31, h = lane >> 5;

  // work item: whole heads per XCD; causal: the first key blocks see the
  // most query tiles, so they go first
  const int id = static_cast<int>(blockIdx.x);
  int bh, kb;
  if (BH % kXcdsB == 0) {
    const int x = id % kXcdsB, s = id / kXcdsB;
    if (causal) {   // chunks of hc heads, each chunk's key blocks heaviest first
      const int per = hc * nkb, ch = s / per, r = s - ch * per;
      kb = r / hc; bh = x + kXcdsB * (ch * hc + r % hc);
    } else {
      bh = x + kXcdsB * (s / nkb); kb = s % nkb;
    }
  } else if (causal) {
    kb = id / BH; bh = id % BH;
  } else {
    bh = id / nkb; kb = id % nkb;
  }
  const int k0 = kb * BK, k0w = k0 + wave * 32, key = k0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const int64_t sbase = static_cast<int64_t>(bh) * N;
  const uint16_t* qbase = q + base;
  const uint16_t* dbase = dout + base;

  const int nqt = (N + BT - 1) / BT;
  const int qt0 = causal ? k0 / BT : 0;
  // V of the block into LDS; this lane's K row (key k0w + j) as B operands
  // (rows past N read as zero)
#pragma unroll
  for (int cpy = 0; cpy < BK / BT; ++cpy)
    if (k0 + cpy * BT < N) copy_tile<D, NW>(vt + cpy * T::TILEB, v + base, k0 + cpy * BT, N, wave, lane);
  bf16x8 kr[D / 16];
  {
    const int rows = max(0, min(32, N - k0w));
    const int64_t r0 = base + static_cast<int64_t>(min(k0w, N)) * D;
    const auto rk = uniform_rsrc(k + r0, rows * T::ROWB);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int off = j * T::ROWB + (ks * 16 + 8 * h) * 2;
      kr[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
    }
  }
  const char* vw = vt + wave * 32 * T::ROWB;   // this wave's 32 V rows
  auto copy_qtile = [&](int qt, int slot) {
    copy_tile<D, NW>(qring + slot * T::TILEB, qbase, qt * BT, N, wave, lane);
    copy_tile<D, NW>(dring + slot * T::TILEB, dbase, qt * BT, N, wave, lane);
    if (wave == 0) {
      const uint32_t bytes = static_cast<uint32_t>(min(BT, N - qt * BT)) * 4u;
      dma4(uniform_desc(lse + sbase + qt * BT, bytes), sring + slot * SB, lane * 4);
      dma4(uniform_desc(delta + sbase + qt * BT, bytes), sring + slot * SB + BT * 4, lane * 4);
    }
  };
  // wave 0 copied a tile's LSE row; once it has landed, the same wave turns
  // it into base-2 units in place (one multiply per query instead of one per
  // score), before the barrier that publishes the tile
  auto lse_to_base2 = [&](int slot) {
    if (wave == 0) {
      float* l = reinterpret_cast<float*>(sring + slot * SB);
      l[lane] *= kLog2e;
    }
  };
  if (qt0 < nqt) copy_qtile(qt0, 0);
  f32x16 dka[D / 32], dva[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) { dka[db] = f32x16{}; dva[db] = f32x16{}; }
  const BLane<D> la(j, h, lane);
  wait_vmcnt<0>();
  if (qt0 < nqt) lse_to_base2(0);
  __syncthreads();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int slot = (qt - qt0) & 1;
    const char* qst = qring + slot * T::TILEB;
    const char* dst = dring + slot * T::TILEB;
    const char* sst = sring + slot * SB;
    if (qt + 1 < nqt) copy_qtile(qt + 1, slot ^ 1);
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qs = qt * BT + sb * 32;
      if (qs >= N || k0w >= N || (causal && qs + 31 < k0w)) continue;   // wave-uniform
      // S then dP, one product per slot, each slot reading the LDS operands
      // of the product two slots ahead (left to the compiler, every product
      // waited on reads issued just before it: 3.258 -> 3.238 ms at 16k,
      // 3.636 -> 3.608 ms at B=8 H=32 N=4096, side by side; one slot ahead
      // was slower and three spill)
      f32x16 s = f32x16{}, dp = f32x16{};
      {
        constexpr int NS = D / 16, RA = 2;
        bf16x8 qa[NS], da[NS], va[NS];
        auto rd = [&](int i) __attribute__((always_inline)) {
          if (i < NS) {
            qa[i] = lds_row(qst + sb * 32 * T::ROWB + la.rofs[i]);
          } else if (i < 2 * NS) {
            da[i - NS] = lds_row(dst + sb * 32 * T::ROWB + la.rofs[i - NS]);
            va[i - NS] = lds_row(vw + la.rofs[i - NS]);
          }
        };
#pragma unroll
        for (int i = 0; i < RA; ++i) rd(i);
#pragma unroll
        for (int i = 0; i < 2 * NS; ++i) {
          rd(i + RA);
          if (i < NS) s = mfma(qa[i], kr[i], s);
          else dp = mfma(da[i - NS], va[i - NS], dp);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // Only sub-blocks that reach the causal diagonal or the sequence end
      // (wave-uniform test) carry a mask: the score becomes -inf there, so P
      // and dS are exactly 0.
      if ((qs + 31 >= N) || (k0w + 31 >= N) || (causal && k0w + 31 > qs)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qq = qs + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool masked = (qq >= N) || (key >= N) || (causal && key > qq);
          s[r] = masked ? -INFINITY : s[r];
        }
      }
      // P and dS for this lane's key and the 16 queries 8g + 4h + (0..3);
      // the tile's LSE values were turned into base-2 units in LDS
      uint32_t pw[2][4], dsw[2][4];
      auto group = [&](int g) __attribute__((always_inline)) {
        const f32x4 lg = *reinterpret_cast<const f32x4*>(sst + (sb * 32 + 8 * g + 4 * h) * 4);
        const f32x4 dg = *reinterpret_cast<const f32x4*>(sst + BT * 4 + (sb * 32 + 8 * g + 4 * h) * 4);
        float pv[4], dsv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = 4 * g + x;
          pv[x] = fast_exp2(fmaf(s[r], c, -lg[x]));
          dsv[x] = pv[x] * (dp[r] - dg[x]);
        }
        pw[g >> 1][(g & 1) * 2 + 0] = pack_bf16x2(pv[0], pv[1]);
        pw[g >> 1][(g & 1) * 2 + 1] = pack_bf16x2(pv[2], pv[3]);
        dsw[g >> 1][(g & 1) * 2 + 0] = pack_bf16x2(dsv[0], dsv[1]);
        dsw[g >> 1][(g & 1) * 2 + 1] = pack_bf16x2(dsv[2], dsv[3]);
      };
      group(0);
      group(1);
      // dV and dK of the first operand half (queries of groups 0, 1), slot
      // by slot beside groups 2 and 3 (one group per four MFMAs; empty asm
      // uses keep that work in its slot), then the second half
#pragma unroll
      for (int cg = 0; cg < 2; ++cg) {
        const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pw[cg][0], pw[cg][1], pw[cg][2], pw[cg][3]});
        const bf16x8 dsb = __builtin_bit_cast(bf16x8, u32x4{dsw[cg][0], dsw[cg][1], dsw[cg][2], dsw[cg][3]});
        if (cg == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dva[db] = mfma(lds_trans<D>(dst, la, db, 2 * sb + cg), pb, dva[db]);
          dka[db] = mfma(lds_trans<D>(qst, la, db, 2 * sb + cg), dsb, dka[db]);
          if (cg == 0 && (db == 0 || db == D / 64)) {
            const int g = db == 0 ? 2 : 3;
            group(g);
            asm volatile("" ::"v"(pw[1][(g & 1) * 2]), "v"(pw[1][(g & 1) * 2 + 1]),
                         "v"(dsw[1][(g & 1) * 2]), "v"(dsw[1][(g & 1) * 2 + 1]));
          }
          if (cg == 0) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    wait_vmcnt<0>();
    if (qt + 1 < nqt) lse_to_base2(slot ^ 1);
    __syncthreads();
  }
  // the loop's last barrier left the LDS idle: each wave stages dK, then dV,
  // in its own 32-row region
  static_assert(NW * 32 * 2 * D <= static_cast<int>(sizeof(smem)), "dK/dV staging fits the LDS");
  char* stage = smem + wave * (32 * 2 * D);
  store_rows_lds<D>(dk + base, k0w, N, dka, scale, stage, j, h, lane);
  store_rows_lds<D>(dv + base, k0w, N, dva, 1.f, stage, j, h, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a) {
  const int BH = a.B * a.H;
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const float c = a.scale * kLog2e;
  const auto* q = static_cast<const uint16_t*>(a.q);
  const auto* k = static_cast<const uint16_t*>(a.k);
  const auto* v = static_cast<const uint16_t*>(a.v);
  const auto* o = static_cast<const uint16_t*>(a.o);
  const auto* dout = static_cast<const uint16_t*>(a.dout);
  const int64_t rows = static_cast<int64_t>(BH) * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3(static_cast<unsigned>((rows + RPB - 1) / RPB)),
                     dim3(256), 0, st, o, dout, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  constexpr int NWK = D == 128 ? 8 : 4;        // dK/dV: 256 (d=128) or 128 keys per workgroup
  const int nkb = (a.N + NWK * 32 - 1) / (NWK * 32);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, NWK>), dim3(static_cast<unsigned>(static_cast<int64_t>(nkb) * BH)),
                     dim3(NWK * 64), 0, st, q, k, v, dout, a.lse, a.delta,
                     static_cast<uint16_t*>(a.dk), static_cast<uint16_t*>(a.dv), a.N, BH, nkb, c,
                     a.scale, a.causal, causal_head_chunk(BH, 4LL * a.N * D));   // Q and dO bytes of a head
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  constexpr int NWQ = D == 128 ? 8 : 4;        // dQ: as the forward kernel
  const int nqb = (a.N + NWQ * 32 - 1) / (NWQ * 32);
  hipLaunchKernelGGL((bwd_dq_kernel<D, NWQ>), dim3(static_cast<unsigned>(static_cast<int64_t>(nqb) * BH)),
                     dim3(NWQ * 64), 0, st, q, k, v, dout, a.lse, a.delta,
                     static_cast<uint16_t*>(a.dq), a.N, BH, nqb, c, a.scale, a.causal,
                     causal_head_chunk(BH, 4LL * a.N * D));   // K and V bytes of a head
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const BwdArgs& a) {
  return a.d == 64 ? launch_bwd_d<64>(a) : launch_bwd_d<128>(a);
}

}  // namespace attn127
