// fp8 (OCP e4m3) path: the fused attention forward on fp8 matrix cores
// (gfx950); the quantisation that feeds it is in attn_fp8_prepare.hip.
//
// Page "FlashAttention scaling, multi-GPU training and weight quantization",
// section 1, the FP8 bullet: low-precision matrix units double the matmul
// rate, and two measures keep outliers from ruining accuracy -- an
// independent scale for each small tile (block quantisation) and
// multiplying Q and K by a random orthogonal matrix first (incoherent
// processing), which leaves Q K^T unchanged.
//
// Both kernels keep the bf16 kernel's structure (transposed scores,
// in-register online softmax, deferred normalisation, HBM -> LDS copies)
// with the scores on v_mfma_scale_f32_32x32x64_f8f6f4: S^T = K^ Q^^T.
//
// attn_fp8_kernel (one float32 scale per 128-token tile): the Q and K tile
// scales fold into the exponent's multiplier.  The second product runs on
// fp16 matrix cores.  V stays e4m3 in LDS; each V^T operand is read with a
// transposing 8-bit LDS read (8 keys of one channel per lane) and widened
// to fp16 in registers (exact: every e4m3 value is an fp16 value), and the
// V tile's scale, relative to the largest V tile scale of the head, rides
// on P: p * s_v / s_vmax is rounded to fp16 (2^-11 of each weight; it stays
// below 2^8, far inside fp16's range).  Rounding P to e4m3 instead would
// cost up to 2^-4 of every weight and bf16 2^-8; where the x40 outlier
// channels of V cancel in O, a 2^-8 weight error reaches 9% of |O|
// (measured on the fp8 workload against float64 attention on the
// dequantised codes), 2^-11 about 1%.
//
// attn_mxfp8_kernel (MXFP8: one E8M0 scale per 32 channels of a token): the
// score MFMA applies the K and Q block scales itself, and V is widened to
// bf16 with its block scale into a bf16 LDS tile, since the widened values
// span bf16's exponent range and a V^T operand's 8 keys carry 8 different
// scales.
#include <float.h>
#include <math.h>

#include "common.h"
#include "launch.h"
#if defined(__HIP_DEVICE_COMPILE__)
#include "device_util.h"
#endif

namespace attn127 {
namespace {

constexpr int kTile8 = kFp8Tile;     // tokens per quantisation tile

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------
// Four waves per workgroup, 32 query rows each.  Per-tile scales: with V
// widened per operand there is no shared conversion pass, and independent
// four-wave workgroups (two or three per CU) overlap each other's matrix
// and vector work; the earlier eight-wave design, which shared one widened
// fp16 V tile over 256 rows, measured 3.24-3.34 ms against 3.11-3.13 ms on
// 4x32x8192 and 0.460-0.475 against 0.41 ms causal at 2x16x8192.  MXFP8: 8
// waves measured 27% slower (its per-block scale loads and widening stall
// all eight waves at each tile's barrier).
constexpr int kNW8 = 4;              // waves per workgroup
constexpr int kXcds8 = 8;            // XCDs the dispatcher round-robins over
constexpr int BC8 = 64;              // keys per tile (half a quantisation tile)
constexpr float kTau8 = 8.0f;        // p <= 2^kTau8 (exponent reference raised lazily)
static_assert(kTile8 % 32 == 0, "a wave's 32 rows share one Q scale");

template <int D>
struct Cfg8 {
  static constexpr int ROWB = D;               // bytes per fp8 K/V row
  static constexpr int ROWB16 = 2 * D;         // bytes per bf16 V row
  static constexpr int CPR = D / 16;           // 16-byte chunks per fp8 row
  static constexpr int RPB = 1024 / ROWB;      // fp8 rows per 1 KB copy block
  static constexpr int TILEB = BC8 * ROWB;     // fp8 tile
  static constexpr int TILEB16 = BC8 * ROWB16; // bf16 V tile
  static constexpr int BLK = TILEB / 1024;
  static constexpr int BPW = BLK / kNW8;
  static_assert(BPW * kNW8 == BLK, "tile must split evenly over the waves");
};

// fp8 rows: chunk swizzle spreading the rows that one K operand read touches
// over distinct LDS bank groups (two rows share a 256-byte bank window at
// D=128, four at D=64).  The same swizzle spreads the 8 keys that one
// transposing V^T read of 16 lanes touches.
template <int D>
__device__ __forceinline__ int swz8(int row) { return D == 128 ? ((row >> 1) & 7) : ((row >> 2) & 3); }
// bf16 V rows: the swizzle under which the 4 rows x 4 chunks of one
// transposing read of half a wave hit distinct banks.
template <int D>
__device__ __forceinline__ int swz16(int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

// Work item: workgroups are dispatched round-robin over the 8 XCDs, so item
// id lands on XCD id % 8; giving each XCD whole heads keeps a head's K/V
// tiles in one L2.  Causal: chunks of hc heads, each chunk's query blocks
// heaviest first.
template <bool CAUSAL>
__device__ __forceinline__ void work_item8(int id, int BH, int nqb, int hc, int& bh, int& qb) {
  if (BH % kXcds8 == 0) {
    const int x = id % kXcds8, s = id / kXcds8;
    if (CAUSAL) {
      const int per = hc * nqb, ch = s / per, r = s - ch * per;
      qb = nqb - 1 - r / hc; bh = x + kXcds8 * (ch * hc + r % hc);
    } else {
      bh = x + kXcds8 * (s / nqb); qb = s % nqb;
    }
  } else if (CAUSAL) {
    qb = nqb - 1 - id / BH; bh = id % BH;
  } else {
    bh = id / nqb; qb = id % nqb;
  }
}

#if defined(__HIP_DEVICE_COMPILE__)
template <int D>
__device__ __forceinline__ void issue_copy8(char* dst, const uint8_t* src, int kv0, int N, int wave, int lane) {
  using C = Cfg8<D>;
  const int rows = min(BC8, N - kv0);
  const i32x4 desc = buffer_desc(src + static_cast<int64_t>(kv0) * D, static_cast<uint32_t>(rows) * C::ROWB);
#pragma unroll
  for (int b = 0; b < C::BPW; ++b) {
    const int blk = wave * C::BPW + b;
    const int row = blk * C::RPB + lane / C::CPR;
    const int pos = lane % C::CPR;
    dma16(desc, dst + blk * 1024, row * C::ROWB + ((pos ^ swz8<D>(row)) << 4));
  }
}

__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // operand formats 0/0 = e4m3; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// Block-scaled form: each lane's 32 codes of A (B) are multiplied by
// 2^(sa-127) (2^(sb-127)); sa, sb are E8M0 bytes in bits 7:0.
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, const f32x16& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

__device__ __forceinline__ i32x8 join8(const u32x4& lo, const u32x4& hi) {
  return i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]), static_cast<int>(lo[3]),
               static_cast<int>(hi[0]), static_cast<int>(hi[1]), static_cast<int>(hi[2]), static_cast<int>(hi[3])};
}

// Keys past the sequence end or (causal) past the row -> -inf.  Accumulator
// register r of key block kb holds key kv0 + kb*32 + 8(r/4) + 4h + r%4.
template <bool CAUSAL>
__device__ __forceinline__ void mask8(f32x16 (&sacc)[2], int kv0, int N, int qrow, int h) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kv0 + kb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      const bool masked = (key >= N) || (CAUSAL && key > qrow);
      sacc[kb][r] = masked ? -INFINITY : sacc[kb][r];
    }
}

// The reference moves only when a tile's maximum exceeds it by more than
// kTau8 (every p stays below 2^kTau8); the partial output and normaliser
// are rescaled then.
template <int D>
__device__ __forceinline__ void update_reference(const f32x16 (&sacc)[2], float ct, float& m, float& lsum,
                                                 f32x16 (&oacc)[D / 32]) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  const float mt = halves_max(mx) * ct;
  if (__builtin_amdgcn_ballot_w64(mt > m + kTau8) != 0) {
    const float mnew = fmaxf(m, mt);
    const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(m - mnew);
    m = mnew;
    lsum *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
  }
}

// Epilogue: O = acc * oscale / l in bf16, LSE in natural log.  The wave's
// 32 bf16 rows go through its own LDS region (rows of 2D bytes, 16-byte
// chunks swizzled by the row) and are stored in row order, each store
// instruction writing whole rows (1 KB contiguous) instead of 8-byte pieces
// of 32 rows.  The region must be idle (ring space after the last barrier).
template <int D>
__device__ __forceinline__ void store_rows8(const f32x16 (&oacc)[D / 32], float m, float lsum, float oscale,
                                            char* stage, uint16_t* o, float* lse, int64_t base, int bh, int N,
                                            int q0w, int j, int h, int lane) {
  constexpr int RB = 2 * D, CPR = RB / 16, RPI = 64 / CPR;
  const float ltot = halves_sum(lsum);
  const float inv = oscale / ltot;
  char* row = stage + j * RB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = db * 4 + g;             // chunk of channels 8c..8c+7; the lane holds 8c + 4h .. +3
      u32x2 wv;
      wv[0] = pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      wv[1] = pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(row + ((c ^ (j % CPR)) << 4) + 8 * h) = wv;
    }
  if (lse != nullptr && h == 0 && q0w + j < N)
    lse[static_cast<int64_t>(bh) * N + q0w + j] = (m + __log2f(ltot)) * kLn2;
  // stores through a descriptor that covers the valid rows only: rows at or
  // past N are dropped by its range check, without a branch
  const int r0u = __builtin_amdgcn_readfirstlane(q0w);
  const int rows = max(0, min(32, N - r0u));
  const auto rs = uniform_rsrc(o + base + static_cast<int64_t>(min(r0u, N)) * D, rows * RB);
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CPR, c = lane % CPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * RB + ((c ^ (r % CPR)) << 4));
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, r * RB + c * 16, 0, 0);
  }
}
#endif

// ---------------------------------------------------------------------------
// per-tile scales
// ---------------------------------------------------------------------------
// Scores on fp8 MFMA; P V on fp16 MFMA with each V^T operand read as e4m3
// from LDS and widened in registers, and the V tile scale, relative to the
// head's largest V tile scale s_vmax, carried by P (p * s_v / s_vmax rounded
// to fp16); O is the accumulated product times s_vmax over the normaliser.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kNW8 * 64, 2)
attn_fp8_kernel(const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
                const uint8_t* __restrict__ v8, const float* __restrict__ sqv,
                const float* __restrict__ skv, const float* __restrict__ svv,
                uint16_t* __restrict__ o, float* __restrict__ lse, int N, int BH, int nqb,
                int ntq, float c0, int hc) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg8<D>;
  __shared__ __attribute__((aligned(1024))) char kring[2 * C::TILEB];     // e4m3 K, two slots
  __shared__ __attribute__((aligned(1024))) char vring[2 * C::TILEB];     // e4m3 V, two slots

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h = lane >> 5;

  int bh, qbk;
  work_item8<CAUSAL>(static_cast<int>(blockIdx.x), BH, nqb, hc, bh, qbk);
  const int q0 = qbk * (kNW8 * 32);
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint8_t* kbase = k8 + base;
  const uint8_t* vbase = v8 + base;
  // the key and value tile scales of this head, and the multiplier
  // s_q * scale * log2(e) of this wave's rows (a wave past the end reads
  // the last tile's)
  const float* skh = skv + static_cast<int64_t>(bh) * ntq;
  const float* svh = svv + static_cast<int64_t>(bh) * ntq;
  const float cq = c0 * sqv[static_cast<int64_t>(bh) * ntq + min(q0w, N - 1) / kTile8];

  const int kend = CAUSAL ? min(N, q0 + kNW8 * 32) : N;
  const int ntiles = (kend + BC8 - 1) / BC8;
  int last = -1;
  if (q0w < N) last = CAUSAL ? min(ntiles - 1, (q0w + 31) / BC8) : ntiles - 1;

  issue_copy8<D>(kring, kbase, 0, N, wave, lane);
  issue_copy8<D>(vring, vbase, 0, N, wave, lane);
  // Q^ as the B operand: k-step ks holds channels ks*64 + 32h .. +31
  i32x8 qr[D / 64];
  {
    const int rows = max(0, min(32, N - q0w));
    const auto rq = uniform_rsrc(q8 + base + static_cast<int64_t>(min(q0w, N)) * D, rows * D);
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      const int lo_c = ks * 64 + 32 * h;
      qr[ks] = join8(__builtin_amdgcn_raw_buffer_load_b128(rq, j * D + lo_c, 0, 0),
                     __builtin_amdgcn_raw_buffer_load_b128(rq, j * D + lo_c + 16, 0, 0));
    }
  }
  // the head's largest V tile scale (every lane of every wave computes the same)
  float svmax;
  {
    float mxs = 0.f;
    for (int t = lane; t < ntq; t += 64) mxs = fmaxf(mxs, svh[t]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mxs = fmaxf(mxs, __shfl_xor(mxs, off));
    svmax = mxs;
  }
  wait_vmcnt<0>();
  __syncthreads();

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  // lane-constant LDS offsets.  K operand reads: rows j and 32+j share the
  // swizzle.  V^T operand reads (ds_read_b64_tr_b8, probed on the chip): in
  // each group of 16 lanes, lane s loads 8 bytes, and after the transpose
  // lane i holds byte b of lane 2b + i/8 at position i%8.  So lane s loads 8
  // channels, 32db + 16(g&1) + 8(s&1) .. +7 (g = lane/16), of key
  // kk = 4h + {0,1,2,3,8,9,10,11}[s/2], and lane i then holds channel
  // 32db + (lane%32) of 8 keys in the key order of the P operand built from
  // the score accumulators.
  const int ksw = swz8<D>(j);
  const int s16 = lane & 15, g16 = lane >> 4;
  const int kk = 4 * h + ((s16 >> 1) & 3) + 8 * (s16 >> 3);
  const int vsw = swz8<D>(kk);                    // equals swz8 of kk + 16 c16
  int vb8[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
    vb8[db] = kk * C::ROWB + (((2 * db + (g16 & 1)) ^ vsw) << 4) + 8 * (s16 & 1);

  // At the top of iteration t, K and V of tile t are in ring slot t&1; the
  // iteration copies tile t+1 into the other slot, which every wave left at
  // the previous barrier.
  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BC8;
    const char* kst = kring + (t & 1) * C::TILEB;
    const char* vst = vring + (t & 1) * C::TILEB;
    if (t + 1 < ntiles) {
      issue_copy8<D>(kring + ((t + 1) & 1) * C::TILEB, kbase, kv0 + BC8, N, wave, lane);
      issue_copy8<D>(vring + ((t + 1) & 1) * C::TILEB, vbase, kv0 + BC8, N, wave, lane);
    }
    if (t <= last) {
      // ---- S^T = K^ Q^^T, two 32-key blocks ----
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const char* krow = kst + (kb * 32 + j) * C::ROWB;
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
          const int clo = 4 * ks + 2 * h;            // 16-byte chunks, as for Q
          const u32x4 lo = *reinterpret_cast<const u32x4*>(krow + ((clo ^ ksw) << 4));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(krow + (((clo + 1) ^ ksw) << 4));
          sacc[kb] = mfma_fp8(join8(lo, hi), qr[ks], sacc[kb]);
        }
      }
      if ((CAUSAL && kv0 + BC8 - 1 > q0w) || kv0 + BC8 > N) mask8<CAUSAL>(sacc, kv0, N, qrow, h);
      // ---- online softmax; the key tile's scale enters the multiplier ----
      const float ct = cq * skh[kv0 / kTile8];
      update_reference<D>(sacc, ct, m, lsum, oacc);
      // operand p' = p * s_v / s_vmax = exp2(s*ct - m - log2(s_vmax / s_v));
      // the normaliser takes sum(p') * s_vmax / s_v.  The ratio comes from the
      // hardware reciprocal (within 1 ulp; two IEEE divisions per tile cost
      // 4 % of the kernel's time), capped so that a zero sum stays zero.
      const float rsv = fminf(svmax * __builtin_amdgcn_rcpf(svh[kv0 / kTile8]), FLT_MAX);
      const float mref = ((m == -INFINITY) ? 0.f : m) + __log2f(rsv);
      uint32_t pw[4][4];
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(sacc[kb][r], ct, -mref));
          const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], ct, -mref));
          ls0 += p0;
          ls1 += p1;
          pw[kb * 2 + (r >> 3)][(r & 7) >> 1] = pack_f16x2(p0, p1);
        }
      lsum += (ls0 + ls1) * rsv;
      // ---- O^T += V^T P'^T on fp16 ----
      // The wave raises its issue priority for its P V products, so that of
      // the three waves sharing a SIMD the one with matrix work ready goes
      // first (1-2 % faster than equal priorities).
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c16 = 0; c16 < 4; ++c16) {
        const u32x4 pwv = u32x4{pw[c16][0], pw[c16][1], pw[c16][2], pw[c16][3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const v2i32 x = ds_read_tr8(vst + vb8[db] + c16 * 16 * C::ROWB);
          u32x4 a;
          a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.f, false));
          a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[0], 1.f, true));
          a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.f, false));
          a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x[1], 1.f, true));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                            __builtin_bit_cast(f16x8, pwv), oacc[db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (t + 1 < ntiles) wait_vmcnt<0>();          // this wave's copies of tile t+1 landed
    __syncthreads();
  }

  // waves 0-1 stage O in the K ring, waves 2-3 in the V ring
  static_assert(2 * 32 * 2 * D <= 2 * C::TILEB, "O staging fits the rings");
  store_rows8<D>(oacc, m, lsum, svmax, (wave < 2 ? kring : vring) + (wave & 1) * (32 * 2 * D), o, lse, base, bh,
                 N, q0w, j, h, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

// ---------------------------------------------------------------------------
// MXFP8
// ---------------------------------------------------------------------------
#if defined(__HIP_DEVICE_COMPILE__)
// The block of a V tile this wave copied, e4m3 codes -> bf16 with the
// block's power-of-two scale (exact), into the bf16 tile.  Lane i's 16
// codes are channels 16c..16c+15 of one row.
// Row and channel chunk (16 codes) that lane `lane` converts in block b.
template <int D>
__device__ __forceinline__ void convert_slot(int wave, int lane, int b, int& row, int& c) {
  using C = Cfg8<D>;
  const int blk = wave * C::BPW + b;
  row = blk * C::RPB + lane / C::CPR;
  c = (lane % C::CPR) ^ swz8<D>(row);
}

template <int D>
__device__ __forceinline__ void convert_v_mx(char* dst16, const char* src8, int wave, int lane,
                                             const float (&vscale)[Cfg8<D>::BPW]) {
  using C = Cfg8<D>;
#pragma unroll
  for (int b = 0; b < C::BPW; ++b) {
    const int blk = wave * C::BPW + b;
    int row, c;
    convert_slot<D>(wave, lane, b, row, c);
    const u32x4 x = *reinterpret_cast<const u32x4*>(src8 + blk * 1024 + lane * 16);
    const float sc = vscale[b];
    u32x4 lo, hi;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      lo[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], sc, false));
      lo[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w], sc, true));
      hi[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w + 2], sc, false));
      hi[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x[w + 2], sc, true));
    }
    char* r16 = dst16 + row * C::ROWB16;
    *reinterpret_cast<u32x4*>(r16 + (((2 * c) ^ swz16<D>(row)) << 4)) = lo;
    *reinterpret_cast<u32x4*>(r16 + (((2 * c + 1) ^ swz16<D>(row)) << 4)) = hi;
  }
}

// E8M0 bytes of one token row (D/32 of them, packed little-endian) from a
// [rows][D/32] byte array; rows past the descriptor's range read as zero.
template <int D>
__device__ __forceinline__ uint32_t load_row_scales(__amdgpu_buffer_rsrc_t r, int row) {
  if constexpr (D == 128) return __builtin_amdgcn_raw_buffer_load_b32(r, row * 4, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b16(r, row * 2, 0, 0);
}
#endif

// Every token row carries one E8M0 scale per 32 channels.  The score MFMA
// applies the K and Q block scales itself (each lane's 32 codes are one
// block), V is widened to bf16 with its block scale (exact) into an LDS
// tile, and P V runs on bf16 matrix cores with P carrying no scale.  Each
// lane loads the scale bytes it needs with the tile copies, so they are
// covered by the same wait.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kNW8 * 64, 2)
attn_mxfp8_kernel(const uint8_t* __restrict__ q8, const uint8_t* __restrict__ k8,
                  const uint8_t* __restrict__ v8, const uint8_t* __restrict__ sq,
                  const uint8_t* __restrict__ sk, const uint8_t* __restrict__ sv,
                  uint16_t* __restrict__ o, float* __restrict__ lse, int N, int BH, int nqb,
                  float c0, int hc) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg8<D>;
  __shared__ __attribute__((aligned(1024))) char kring[2 * C::TILEB];     // e4m3 K, two slots
  __shared__ __attribute__((aligned(1024))) char vstage[C::TILEB];        // e4m3 V landing area
  __shared__ __attribute__((aligned(1024))) char vring[2 * C::TILEB16];   // bf16 V, two slots

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h = lane >> 5;

  int bh, qbk;
  work_item8<CAUSAL>(static_cast<int>(blockIdx.x), BH, nqb, hc, bh, qbk);
  const int q0 = qbk * (kNW8 * 32);
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint8_t* kbase = k8 + base;
  const uint8_t* vbase = v8 + base;
  constexpr int SPR = D / 32;                    // scale bytes per row
  const int64_t sbase = static_cast<int64_t>(bh) * N * SPR;
  const auto rks = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sk + sbase), 0, N * SPR, 0x00020000);
  const auto rvs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sv + sbase), 0, N * SPR, 0x00020000);
  uint32_t kscw[2] = {0u, 0u};                   // this lane's K row scales, current tile
  float vsc[C::BPW];                             // V block scales of the tile being converted
  auto load_tile_scales = [&](int kv0n, uint32_t (&kw)[2], float (&vs)[C::BPW]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) kw[kb] = load_row_scales<D>(rks, kv0n + kb * 32 + j);
#pragma unroll
    for (int b = 0; b < C::BPW; ++b) {
      int row, cch;
      convert_slot<D>(wave, lane, b, row, cch);
      const uint32_t e = __builtin_amdgcn_raw_buffer_load_b8(rvs, (kv0n + row) * SPR + cch / 2, 0, 0);
      vs[b] = static_cast<float>(e);             // exponent byte; widened after the wait
    }
  };
  auto widen = [&](float (&vs)[C::BPW]) {
#pragma unroll
    for (int b = 0; b < C::BPW; ++b) vs[b] = ldexpf(1.f, static_cast<int>(vs[b]) - 127);
  };

  const int kend = CAUSAL ? min(N, q0 + kNW8 * 32) : N;
  const int ntiles = (kend + BC8 - 1) / BC8;
  int last = -1;
  if (q0w < N) last = CAUSAL ? min(ntiles - 1, (q0w + 31) / BC8) : ntiles - 1;

  issue_copy8<D>(kring, kbase, 0, N, wave, lane);
  issue_copy8<D>(vstage, vbase, 0, N, wave, lane);
  load_tile_scales(0, kscw, vsc);
  // Q block scales of this lane's row, k-step ks: block 2 ks + h
  int qsc[D / 64];
  {
    uint32_t qw = 0u;
    if (qrow < N) qw = D == 128 ? *reinterpret_cast<const uint32_t*>(sq + sbase + static_cast<int64_t>(qrow) * SPR)
                                : *reinterpret_cast<const uint16_t*>(sq + sbase + static_cast<int64_t>(qrow) * SPR);
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) qsc[ks] = static_cast<int>((qw >> (8 * (2 * ks + h))) & 0xFFu);
  }
  // Q^ as the B operand.  The block-scaled instruction takes a lane's bytes
  // 0-15 into the k-step's first 32-channel block and bytes 16-31 into the
  // second (each block scaled by the low / high half-wave's scale), so a
  // lane holds channels 16h..+15 and 32+16h..+15 of the step.
  i32x8 qr[D / 64];
  {
    const int rows = max(0, min(32, N - q0w));
    const auto rq = uniform_rsrc(q8 + base + static_cast<int64_t>(min(q0w, N)) * D, rows * D);
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
      qr[ks] = join8(__builtin_amdgcn_raw_buffer_load_b128(rq, j * D + ks * 64 + 16 * h, 0, 0),
                     __builtin_amdgcn_raw_buffer_load_b128(rq, j * D + ks * 64 + 32 + 16 * h, 0, 0));
  }
  wait_vmcnt<0>();
  widen(vsc);
  convert_v_mx<D>(vring, vstage, wave, lane, vsc);     // this wave's own copied blocks
  __syncthreads();

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, lsum = 0.f;

  // lane-constant LDS offsets
  const int ksw = swz8<D>(j);                     // rows j and 32+j share it
  const int r16 = lane & 15, b16 = (lane >> 4) & 1;
  const int vkey0 = 4 * h + (r16 >> 2);
  const int vs16 = swz16<D>(vkey0);               // equals swz16 of every vkey0 + 8i
  int vbase16[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int chunk = db * 4 + 2 * b16 + ((r16 & 3) >> 1);
    vbase16[db] = vkey0 * C::ROWB16 + ((chunk ^ vs16) << 4) + ((r16 & 1) << 3);
  }

  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BC8;
    const char* kst = kring + (t & 1) * C::TILEB;
    const char* vst = vring + (t & 1) * C::TILEB16;
    uint32_t kscw_next[2] = {0u, 0u};
    if (t + 1 < ntiles) {
      issue_copy8<D>(kring + ((t + 1) & 1) * C::TILEB, kbase, kv0 + BC8, N, wave, lane);
      issue_copy8<D>(vstage, vbase, kv0 + BC8, N, wave, lane);
      load_tile_scales(kv0 + BC8, kscw_next, vsc);
    }
    if (t <= last) {
      // ---- S^T = K^ Q^^T, two 32-key blocks, block scales on the MFMA ----
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        const char* krow = kst + (kb * 32 + j) * C::ROWB;
#pragma unroll
        for (int ks = 0; ks < D / 64; ++ks) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(krow + (((4 * ks + h) ^ ksw) << 4));
          const u32x4 hi = *reinterpret_cast<const u32x4*>(krow + (((4 * ks + 2 + h) ^ ksw) << 4));
          sacc[kb] = mfma_mx(join8(lo, hi), qr[ks], sacc[kb],
                             static_cast<int>((kscw[kb] >> (8 * (2 * ks + h))) & 0xFFu), qsc[ks]);
        }
      }
      if ((CAUSAL && kv0 + BC8 - 1 > q0w) || kv0 + BC8 > N) mask8<CAUSAL>(sacc, kv0, N, qrow, h);
      // ---- online softmax ----
      update_reference<D>(sacc, c0, m, lsum, oacc);
      const float mref = (m == -INFINITY) ? 0.f : m;
      uint32_t pw[4][4];
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float p0 = fast_exp2(fmaf(sacc[kb][r], c0, -mref));
          const float p1 = fast_exp2(fmaf(sacc[kb][r + 1], c0, -mref));
          ls0 += p0;
          ls1 += p1;
          pw[kb * 2 + (r >> 3)][(r & 7) >> 1] = pack_bf16x2(p0, p1);
        }
      lsum += ls0 + ls1;
      // ---- O^T += V^T P^T on bf16 ----
#pragma unroll
      for (int c16 = 0; c16 < 4; ++c16) {
        const u32x4 pwv = u32x4{pw[c16][0], pw[c16][1], pw[c16][2], pw[c16][3]};
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const v4i16 lo = ds_read_tr16(vst + vbase16[db] + (c16 * 16) * C::ROWB16);
          const v4i16 hi = ds_read_tr16(vst + vbase16[db] + (c16 * 16 + 8) * C::ROWB16);
          const v8i16 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                             __builtin_bit_cast(bf16x8, pwv), oacc[db], 0, 0, 0);
        }
      }
    }
    if (t + 1 < ntiles) {
      // this wave's copies of tile t+1 have landed: publish its K, convert
      // its V blocks into the free bf16 slot (tile t-1's, read before the
      // previous barrier)
      wait_vmcnt<0>();
      widen(vsc);
      convert_v_mx<D>(vring + ((t + 1) & 1) * C::TILEB16, vstage, wave, lane, vsc);
      kscw[0] = kscw_next[0];
      kscw[1] = kscw_next[1];
    }
    __syncthreads();
  }

  // the bf16 V ring holds the four waves' staged O
  static_assert(4 * 32 * 2 * D <= 2 * C::TILEB16, "O staging fits the V ring");
  store_rows8<D>(oacc, m, lsum, 1.f, vring + wave * (32 * 2 * D), o, lse, base, bh, N, q0w, j, h, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, bool CAUSAL>
hipError_t fwd_tile(const Fp8Args& a) {
  const int BH = a.B * a.H;
  const int nqb = (a.N + kNW8 * 32 - 1) / (kNW8 * 32);
  const int ntq = (a.N + kTile8 - 1) / kTile8;
  const int64_t blocks = static_cast<int64_t>(nqb) * BH;
  const int hc = causal_head_chunk(BH, 2LL * a.N * D);      // fp8 K and V bytes of a head
  hipLaunchKernelGGL((attn_fp8_kernel<D, CAUSAL>), dim3(static_cast<unsigned>(blocks)), dim3(kNW8 * 64), 0,
                     static_cast<hipStream_t>(a.stream), a.q8, a.k8, a.v8, static_cast<const float*>(a.sq),
                     static_cast<const float*>(a.sk), static_cast<const float*>(a.sv),
                     static_cast<uint16_t*>(a.o), a.lse, a.N, BH, nqb, ntq, a.scale * kLog2e, hc);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t fwd_mx(const Fp8Args& a) {
  const int BH = a.B * a.H;
  const int nqb = (a.N + kNW8 * 32 - 1) / (kNW8 * 32);
  const int64_t blocks = static_cast<int64_t>(nqb) * BH;
  const int hc = causal_head_chunk(BH, 2LL * a.N * D);
  hipLaunchKernelGGL((attn_mxfp8_kernel<D, CAUSAL>), dim3(static_cast<unsigned>(blocks)), dim3(kNW8 * 64), 0,
                     static_cast<hipStream_t>(a.stream), a.q8, a.k8, a.v8, static_cast<const uint8_t*>(a.sq),
                     static_cast<const uint8_t*>(a.sk), static_cast<const uint8_t*>(a.sv),
                     static_cast<uint16_t*>(a.o), a.lse, a.N, BH, nqb, a.scale * kLog2e, hc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8_fwd(const Fp8Args& a) {
  if (a.mx) {
    if (a.d == 64) return a.causal ? fwd_mx<64, true>(a) : fwd_mx<64, false>(a);
    return a.causal ? fwd_mx<128, true>(a) : fwd_mx<128, false>(a);
  }
  if (a.d == 64) return a.causal ? fwd_tile<64, true>(a) : fwd_tile<64, false>(a);
  return a.causal ? fwd_tile<128, true>(a) : fwd_tile<128, false>(a);
}

}  // namespace attn127
