// Fused exact attention forward on bf16 matrix cores (gfx950).
//
// Algorithm (page "Self-Attention, CUDA kernels and FlashAttention",
// section 3; page "FlashAttention scaling, multi-GPU training and weight
// quantization", section 1, FlashAttention-2 bullets): one workgroup per
// (batch*head, block of BR query rows) -- the outer loop over query blocks is
// the grid, so even one head fills the machine at long sequence length --
// and an inner loop over key/value tiles of BC keys.  Per tile:
//   S^T = K Q^T        bf16 MFMA 32x32x16, float32 accumulate
//   online softmax     exponent reference m and normaliser l per row in
//                      registers, p = exp2(S*c - m) with c = scale*log2(e)
//   O^T += V^T P^T     P rounded to bf16, bf16 MFMA, float32 accumulate
// and after the last tile O /= l once, O rounded to bf16, LSE = ln2*(m+log2 l).
// S and P live only in registers; nothing N x N reaches memory.
//
// gfx950 mapping:
//  * Scores are computed transposed (keys x queries): in the 32x32
//    accumulator layout each lane then holds 16 keys of ONE query (column
//    lane%32), so row reductions (the first tile's maximum, the sum) are
//    in-lane reductions plus one v_permlane32_swap between the lane halves.
//  * Those probabilities feed the second product directly as its B operand;
//    its A operand (V^T) comes from row-major V in LDS through
//    ds_read_b64_tr_b16, which hands each lane four keys of one channel, read
//    in exactly the key order the accumulator registers hold.
//  * Each wave software-pipelines its tiles in two phases: while the matrix
//    cores compute the scores of tile t+1, the vector ALUs run the
//    exponentials of tile t's first three P operands; while they compute P V
//    of tile t, the vector ALUs scale tile t+1's scores into exponents and
//    form its last P operand.  Both phases are written slot by slot (one
//    MFMA, its operand read and a share of the vector work per slot, closed
//    by a scheduling barrier and pinned by empty asm uses), which is what
//    lets MFMA and VALU work overlap inside one wave.
//  * K and V tiles go from HBM straight into LDS (buffer_load ... lds, 16
//    bytes per lane, no register staging) in two-slot rings: K of tile t+2
//    and V of tile t+1 are copied while tile t is processed; one barrier per
//    tile.  Out-of-range rows read as zero (buffer bounds).  16-byte chunks
//    are XOR-swizzled per row so the operand reads hit distinct LDS banks.
//  * The exponent reference is the first tile's row maximum and moves only
//    when a tile's numerators would grow past 2^16, detected from their sum
//    (which the normaliser needs anyway) instead of a per-element maximum;
//    the normaliser and the partial output carry the same reference, and the
//    single division at the end cancels it exactly.  Most tiles of a long
//    row therefore skip both the maximum and the rescale.
//  * d=128: one workgroup of eight waves (two per SIMD) per CU shares each
//    K/V tile over 256 query rows; d=64: two workgroups of four waves per
//    CU.  Work items are grouped by XCD (dispatch is round-robin over the 8
//    XCDs) so the query blocks of one head share one L2, heaviest causal
//    blocks first.
#include "common.h"
#include "launch.h"
#if defined(__HIP_DEVICE_COMPILE__)
#include "device_util.h"
#endif

namespace attn127 {
namespace {

constexpr int BRW = 32;          // query rows per wave
constexpr int BC = 64;           // keys per tile
constexpr int kXcds = 8;

// NW waves per workgroup: 8 (two per SIMD, sharing each K/V tile) or 4
// (one per SIMD, two workgroups per CU).
template <int D, int NW>
struct Cfg {
  static constexpr int NT = NW * 64;           // threads per workgroup
  static constexpr int BR = NW * BRW;          // query rows per workgroup
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int RPB = 1024 / ROWB;      // rows per 1 KB copy block
  static constexpr int TILEB = BC * ROWB;      // bytes of one K (or V) tile
  static constexpr int BLK = TILEB / 1024;     // 1 KB blocks per tile
  static constexpr int BPW = BLK / NW;         // blocks of one tile copied per wave
  static_assert(BPW * NW == BLK, "tile must split evenly over the waves");
  static_assert(2 * BPW < 16, "vmcnt field");
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
// Copy rows [kv0, kv0+BC) of one (b,h) slice of K or V into an LDS tile;
// each wave copies BPW one-kilobyte blocks.
// dst: the tile's LDS byte address (wave-uniform).
template <int D, int NW, bool IS_V>
__device__ __forceinline__ void issue_copy(uint32_t dst, const uint16_t* src, int kv0, int N,
                                           int wave, int lane) {
  using C = Cfg<D, NW>;
  const int rows = min(BC, N - kv0);
  const i32x4 desc = buffer_desc(src + static_cast<int64_t>(kv0) * D,
                                 static_cast<uint32_t>(rows) * C::ROWB);
#pragma unroll
  for (int b = 0; b < C::BPW; ++b) {
    const int blk = wave * C::BPW + b;
    const int row = blk * C::RPB + lane / C::CPR;
    const int pos = lane % C::CPR;
    const int sw = IS_V ? vswz<D>(row) : kswz<D>(row);
    dma16(desc, dst + static_cast<uint32_t>(blk * 1024), row * C::ROWB + ((pos ^ sw) << 4));
  }
}

template <int D>
struct WaveState {
  bf16x8 qr[D / 16];          // Q^T operand: channels ks*16 + 8h .. +7 of the lane's row
  f32x16 oacc[D / 32];        // O^T accumulator: 32 channels x 32 rows per block
  float m;                    // exponent reference (base 2), -inf before the first tile
  float lsum;                 // this lane half's share of the normaliser
};

// Lane-constant parts of the LDS operand addresses.  K operand reads: one
// byte offset per 16-channel step (the row swizzle makes them irregular; the
// second 32-key block adds a constant).  V transposing reads: one base per
// 32-channel block; keys enter as compile-time offsets because the V swizzle
// depends only on key bits that are the same for all of a lane's reads.
template <int D>
struct LaneAddr {
  int kofs[D / 16];
  int vbase[D / 32];
  __device__ __forceinline__ LaneAddr(int j, int h, int lane) {
    using C = Cfg<D, 4>;        // only the row size is used
    const int ksw = kswz<D>(j);   // rows j and 32+j share the swizzle
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) kofs[ks] = j * C::ROWB + (((2 * ks + h) ^ ksw) << 4);
    const int g16 = lane >> 4, r16 = lane & 15, b16 = g16 & 1;
    const int key0 = 4 * h + (r16 >> 2);                 // key of the first read in chunk 0
    const int vs = vswz<D>(key0);                         // equals vswz of every key0 + 8i
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int chunk = db * 4 + 2 * b16 + ((r16 & 3) >> 1);
      vbase[db] = key0 * C::ROWB + ((chunk ^ vs) << 4) + ((r16 & 1) << 3);
    }
  }
};

// MFMA counts per tile: both products take (BC/32)*(D/16) = (D/32)*(BC/16)
// instructions, and each lane holds BC/4 pairs of scores (two keys of one
// query), so every MFMA slot of a phase carries PPS pairs of vector work.
template <int D>
struct Ops {
  static constexpr int NM = (BC / 32) * (D / 16);
  static constexpr int PAIRS = BC / 4;
  static constexpr int PPS = PAIRS / NM;
  static_assert(NM == (D / 32) * (BC / 16) && PPS * NM == PAIRS, "phase shapes");
};

// A operand of score MFMA i (key block i / (D/16), channel step i % (D/16)).
template <int D>
__device__ __forceinline__ bf16x8 k_operand(const char* kst, const LaneAddr<D>& la, int i) {
  const int kb = i / (D / 16), ks = i % (D / 16);
  return *reinterpret_cast<const bf16x8*>(kst + kb * 32 * (2 * D) + la.kofs[ks]);
}

// A operand (V^T) of output MFMA i (channel block i / (BC/16), key step i % (BC/16)).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char* vst, const LaneAddr<D>& la, int i) {
  const int db = i / (BC / 16), c16 = i % (BC / 16);
  const v4i16 lo = ds_read_tr16(vst + la.vbase[db] + (c16 * 16) * (2 * D));
  const v4i16 hi = ds_read_tr16(vst + la.vbase[db] + (c16 * 16 + 8) * (2 * D));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// S^T = K Q^T for one tile (two 32-key blocks), K from LDS.
template <int D>
__device__ __forceinline__ void scores(f32x16 (&sacc)[BC / 32], const WaveState<D>& w,
                                       const LaneAddr<D>& la, const char* kst) {
#pragma unroll
  for (int i = 0; i < Ops<D>::NM; ++i) {
    const int kb = i / (D / 16), ks = i % (D / 16);
    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand<D>(kst, la, i), w.qr[ks],
                                                       ks == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
  }
}

// Accumulator register r of key block kb holds key kv0 + 4h + key_off(kb, r)
// (a compile-time offset below BC).  A key is visible when it is below N and,
// causal, not past the query row, i.e. when key_off <= key_limit.
__device__ __forceinline__ constexpr int key_off(int kb, int r) { return kb * 32 + 8 * (r >> 2) + (r & 3); }
__device__ __forceinline__ int key_limit(int kv0, int N, int qrow, int h, bool causal) {
  const int base = kv0 + 4 * h;
  return causal ? min(N - 1, qrow) - base : N - 1 - base;
}

// Keys past the diagonal (causal) or past the sequence end -> -inf.
__device__ __forceinline__ void apply_mask(f32x16 (&sacc)[BC / 32], int kv0, int N, int qrow, int h,
                                           bool causal) {
  const int lim = key_limit(kv0, N, qrow, h, causal);
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[kb][r] = key_off(kb, r) > lim ? -INFINITY : sacc[kb][r];
}

__device__ __forceinline__ float tile_max(const f32x16 (&sacc)[BC / 32]) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
  return mx;
}

// A tile's 16 score pairs per lane form 4 P operands of 4 packed words each
// (pair pr -> word pr%4 of operand pr/4).  The last operand of tile t+1 (its
// "early" pairs, keys 48..63) is formed in the P V phase of tile t, right
// after that tile's exponents are known; the other pairs ("late") follow in
// the score phase of tile t+1.  This moves a quarter of the exponential work
// to the phase whose vector pipe is otherwise less loaded (measured on an
// instruction-level model of the tile: 1096 -> 1022 ns; moving 3, 5, 6 or 7
// pairs instead measured slower in the kernel).
constexpr int kOps = BC / 16;                           // P operands per tile
constexpr int kPairs = BC / 4;                          // score pairs per lane and tile
constexpr int kEarly = 4;                               // pairs formed early
constexpr int kLate = kPairs - kEarly;                  // pairs formed in the score phase
constexpr int kEarlyP0 = kLate;                         // first early pair

// k-th early pair / k-th late pair of a tile, and whether a pair is early
__device__ __forceinline__ constexpr int early_pair(int k) { return kEarlyP0 + k; }
__device__ __forceinline__ constexpr int late_pair(int k) { return k; }
__device__ __forceinline__ constexpr bool is_early(int pr) { return pr >= kEarlyP0; }

// Packed bf16 numerators of a tile: the early words (formed one phase ahead)
// and the late words (indexed by pair; only late pairs are used).
struct EarlyWords {
  uint32_t w[kEarly];
};
struct LateWords {
  uint32_t w[kPairs];
};

// p = exp2(t) for pair pr of a tile (two keys of the lane's query: scores
// r and r+1 of key block kb).  The float32 p go into the normaliser, the
// bf16-rounded p into the pair's packed word (accumulator registers
// 8c'..8c'+7 of key block kb form operand 2kb+c').
__device__ __forceinline__ void exp2_pair(float& p0, float& p1, const f32x16 (&t)[BC / 32], int pr) {
  const int kb = pr / 8, r = (pr % 8) * 2;
  p0 = fast_exp2(t[kb][r]);
  p1 = fast_exp2(t[kb][r + 1]);
}
__device__ __forceinline__ void sum_pack(uint32_t& word, float& ls0, float& ls1, float p0, float p1) {
  ls0 += p0;
  ls1 += p1;
  word = pack_bf16x2(p0, p1);
}
// The first pair of a sum starts it (p >= +0, so 0 + p = p: same bits).
__device__ __forceinline__ void sum_pack_first(uint32_t& word, float& ls0, float& ls1, float p0, float p1) {
  ls0 = p0;
  ls1 = p1;
  word = pack_bf16x2(p0, p1);
}
__device__ __forceinline__ void exp_pair(uint32_t& word, float& ls0, float& ls1, const f32x16 (&t)[BC / 32],
                                         int pr, bool first = false) {
  float p0, p1;
  exp2_pair(p0, p1, t, pr);
  if (first) sum_pack_first(word, ls0, ls1, p0, p1);
  else sum_pack(word, ls0, ls1, p0, p1);
}

// All early pairs of a tile at once (first tile, and after a reference shift).
__device__ __forceinline__ void early_words(EarlyWords& pe, float& le, const f32x16 (&t)[BC / 32]) {
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int k = 0; k < kEarly; ++k) exp_pair(pe.w[k], l0, l1, t, early_pair(k), k == 0);
  le = l0 + l1;
}

// First tile: the exponent reference becomes the row's scaled maximum, the
// scores become exponents t = s*c - m in place, and the early words form.
template <int D>
__device__ __forceinline__ void first_reference(WaveState<D>& w, f32x16 (&s)[BC / 32], float c,
                                                EarlyWords& pe, float& le) {
  w.m = halves_max(tile_max(s)) * c;
  const float mref = (w.m == -INFINITY) ? 0.f : w.m;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], c, -mref);
  early_words(pe, le, s);
}

// Later tiles arrive as exponents t = s*c - m against the current reference
// m, which only moves when a tile would overflow it: the guard is the
// per-lane sum of the tile's numerators (every p <= that sum), computed
// anyway for the normaliser, so no per-element maximum is needed.  When a
// lane's sum exceeds 2^kGuard (or is not finite), the tile's exact maximum
// becomes the reference: the partial output and the normaliser of earlier
// tiles are rescaled, the tile's exponents shifted, and its numerators
// formed again.  p therefore stays below 2^kGuard, which float32 sums and
// bf16 operands carry without loss of relative precision, and the final
// division cancels the reference exactly.
constexpr float kGuard = 65536.f;      // 2^16

template <int D>
__device__ __forceinline__ bool tile_overflows(float lsum_tile) {
  return __builtin_amdgcn_ballot_w64(!(lsum_tile <= kGuard)) != 0;
}

// Numerators of a tile's late pairs at once (the last tile, which is not
// pipelined, and the overflow path); ll receives their sum.
__device__ __forceinline__ void late_words(LateWords& pl, float& ll, const f32x16 (&t)[BC / 32]) {
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int j = 0; j < kLate; ++j) exp_pair(pl.w[late_pair(j)], ls0, ls1, t, late_pair(j), j == 0);
  ll = ls0 + ls1;
}

// Overflow path: the tile's exact maximum exponent becomes the reference
// (rows whose maximum is not above it keep theirs).
template <int D>
__device__ __forceinline__ void rebase_tile(WaveState<D>& w, f32x16 (&t)[BC / 32], LateWords& pl,
                                            EarlyWords& pe, float& le, float& ll) {
  const float delta = fmaxf(halves_max(tile_max(t)), 0.f);
  const float alpha = fast_exp2(-delta);
  w.lsum *= alpha;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) w.oacc[db] *= alpha;
  w.m += delta;
#pragma unroll
  for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) t[kb][r] -= delta;
  early_words(pe, le, t);
  late_words(pl, ll, t);
}

// The guard and the normaliser update of a tile whose numerators are formed.
template <int D>
__device__ __forceinline__ void commit_tile(WaveState<D>& w, f32x16 (&t)[BC / 32], LateWords& pl,
                                            EarlyWords& pe, float& le, float ll) {
  if (tile_overflows<D>(ll + le)) rebase_tile<D>(w, t, pl, pe, le, ll);
  w.lsum += ll + le;
}

// P operand c16 of a tile: its four packed words, early or late.
__device__ __forceinline__ uint32_t p_word(const LateWords& pl, const EarlyWords& pe, int pr) {
  return is_early(pr) ? pe.w[pr - kEarlyP0] : pl.w[pr];
}
__device__ __forceinline__ bf16x8 p_operand(const LateWords& pl, const EarlyWords& pe, int c16) {
  return __builtin_bit_cast(bf16x8, u32x4{p_word(pl, pe, 4 * c16), p_word(pl, pe, 4 * c16 + 1),
                                          p_word(pl, pe, 4 * c16 + 2), p_word(pl, pe, 4 * c16 + 3)});
}

// O^T += V^T P^T for one tile, V^T through transposing LDS reads.
template <int D>
__device__ __forceinline__ void pv_tile(WaveState<D>& w, const LateWords& pl, const EarlyWords& pe,
                                        const LaneAddr<D>& la, const char* vst) {
#pragma unroll
  for (int i = 0; i < Ops<D>::NM; ++i) {
    const int db = i / (BC / 16), c16 = i % (BC / 16);
    w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(vst, la, i), p_operand(pl, pe, c16),
                                                         w.oacc[db], 0, 0, 0);
  }
}

// An empty volatile use: the value must be computed before this point, so
// code sinking cannot move a slot's vector work out of its slot (the
// scheduling barriers only act after instruction selection).
template <typename T>
__device__ __forceinline__ void pin(T x) { asm volatile("" ::"v"(x)); }

// The two phases of a pipelined tile are written slot by slot: slot i holds
// MFMA i, the LDS read of the operand a few MFMAs ahead, and a share of the
// vector work, and a scheduling barrier closes every slot, so the matrix and
// vector pipes are fed side by side in one wave instead of as two blocks
// (measured on an instruction-level model of the tile: 1474 ns as blocks,
// 1096 ns slotted).
constexpr int kReadAheadK = 3;   // score operands in flight
constexpr int kReadAheadV = 2;   // output operands in flight (two reads each)

// Phase A: scores of the next tile on the matrix cores beside the
// exponentials, normaliser and bf16 packing of the current tile's late
// pairs (spread evenly over the slots).  A pair's normaliser sum and bf16
// pack run one slot after its exponentials, so they never wait on the
// transcendental unit's result (measured: 0.909 -> 0.889 ms at N=16384,
// identical results).
template <int D>
__device__ __forceinline__ void phase_a(WaveState<D>& w, f32x16 (&snext)[BC / 32], LateWords& pl, float& ll,
                                        const f32x16 (&tcur)[BC / 32], const LaneAddr<D>& la,
                                        const char* kst_next) {
  constexpr int NM = Ops<D>::NM, KA = kReadAheadK;
  bf16x8 kop[NM];
  float pp[kLate][2];
  float ls0 = 0.f, ls1 = 0.f;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < KA; ++i) kop[i] = k_operand<D>(kst_next, la, i);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i + KA < NM) kop[i + KA] = k_operand<D>(kst_next, la, i + KA);
    const int kb = i / (D / 16), ks = i % (D / 16);
    snext[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i], w.qr[ks],
                                                        ks == 0 ? f32x16{} : snext[kb], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < kLate; ++j) {
      const int pr = late_pair(j), sl = (j * NM) / kLate;
      if (sl == i - 1) {
        if (j == 0) sum_pack_first(pl.w[pr], ls0, ls1, pp[j][0], pp[j][1]);
        else sum_pack(pl.w[pr], ls0, ls1, pp[j][0], pp[j][1]);
        pin(pl.w[pr]);
      }
      if (sl == i) {
        exp2_pair(pp[j][0], pp[j][1], tcur, pr);
        pin(pp[j][0]);
        pin(pp[j][1]);
      }
    }
    pin(ls0);
    pin(ls1);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int j = 0; j < kLate; ++j) {
    const int pr = late_pair(j);
    if ((j * NM) / kLate == NM - 1) sum_pack(pl.w[pr], ls0, ls1, pp[j][0], pp[j][1]);
  }
  ll = ls0 + ls1;
}

// Phase B: P V of the current tile on the matrix cores beside the scaling
// (t = s*c - m) of the next tile, whose masked keys (causal diagonal,
// sequence end) were set to -inf before the phase, and the next tile's
// early pairs.  The early pairs are scaled first.
template <int D>
__device__ __forceinline__ void phase_b(WaveState<D>& w, f32x16 (&snext)[BC / 32], const LateWords& pl,
                                         const EarlyWords& pecur, EarlyWords& penext, float& lenext,
                                         const LaneAddr<D>& la, const char* vst, float c) {
  constexpr int NM = Ops<D>::NM, PPS = Ops<D>::PPS, VA = kReadAheadV;
  constexpr int S0 = (kEarly + PPS - 1) / PPS;   // slots that scale the early pairs
  static_assert(S0 < NM, "early pairs leave slots for their exponentials");
  bf16x8 vop[NM];
  float pp[kEarly][2];
  float l0 = 0.f, l1 = 0.f;
  const float mref = w.m;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < VA; ++i) vop[i] = v_operand<D>(vst, la, i);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i + VA < NM) vop[i + VA] = v_operand<D>(vst, la, i + VA);
    const int db = i / (BC / 16), c16 = i % (BC / 16);
    w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[i], p_operand(pl, pecur, c16), w.oacc[db], 0, 0, 0);
#pragma unroll
    for (int u = 0; u < PPS; ++u) {
      // scaling order: the early pairs, then the late ones
      const int q = i * PPS + u;
      const int pr = q < kEarly ? early_pair(q) : late_pair(q - kEarly);
      const int kb = pr / 8, r = (pr % 8) * 2;
      snext[kb][r] = fmaf(snext[kb][r], c, -mref);           // -inf stays -inf (c > 0)
      snext[kb][r + 1] = fmaf(snext[kb][r + 1], c, -mref);
      pin(snext[kb][r]);
      pin(snext[kb][r + 1]);
    }
#pragma unroll
    for (int k = 0; k < kEarly; ++k) {
      const int pr = early_pair(k);
      const int sl = S0 + (k * (NM - S0)) / kEarly;
      if (sl == i - 1) {
        if (k == 0) sum_pack_first(penext.w[k], l0, l1, pp[k][0], pp[k][1]);
        else sum_pack(penext.w[k], l0, l1, pp[k][0], pp[k][1]);
        pin(penext.w[k]);
        pin(l0);
        pin(l1);
      }
      if (sl == i) {
        exp2_pair(pp[k][0], pp[k][1], snext, pr);
        pin(pp[k][0]);
        pin(pp[k][1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int k = 0; k < kEarly; ++k) {
    if (S0 + (k * (NM - S0)) / kEarly == NM - 1) sum_pack(penext.w[k], l0, l1, pp[k][0], pp[k][1]);
  }
  lenext = l0 + l1;
}

// Work item of workgroup `id`: XCD-grouped heads, heaviest causal blocks
// first.  When B*H is a multiple of 8, XCD x takes heads x, x+8, ...;
// causal launches walk them in chunks of hc heads, each chunk's query blocks
// heaviest first and interleaved across its heads.
__device__ __forceinline__ void work_item(int id, int BH, int nqb, bool causal, int hc, int& bh, int& qb) {
  if (BH % kXcds == 0) {
    const int x = id % kXcds, s = id / kXcds;
    if (causal) {
      const int per = hc * nqb, ch = s / per, r = s - ch * per;
      qb = nqb - 1 - r / hc;
      bh = x + kXcds * (ch * hc + r % hc);
    } else {
      bh = x + kXcds * (s / nqb); qb = s % nqb;
    }
  } else if (causal) {
    qb = nqb - 1 - id / BH; bh = id % BH;
  } else {
    bh = id / nqb; qb = id % nqb;
  }
}

// The wave's 32 Q rows (the B operands of the score products) copied into
// an LDS region laid out like the first 32 rows of a K tile (same
// swizzle): one 1 KB block of whole rows per copy instruction, where
// loading the operands from global memory directly takes 32-byte pieces of
// 32 rows per instruction.  Rows past the end read as zero.  dst: the
// region's LDS byte address (wave-uniform).
template <int D>
__device__ __forceinline__ void issue_q_copy(uint32_t dst, const uint16_t* q, int64_t base, int q0w, int N,
                                             int lane) {
  using C = Cfg<D, 4>;
  constexpr int NB = BRW * C::ROWB / 1024;
  const int rows = max(0, min(BRW, N - q0w));
  i32x4 desc = buffer_desc(q + base + static_cast<int64_t>(min(q0w, N)) * D,
                           static_cast<uint32_t>(rows) * C::ROWB);
#pragma unroll
  for (int k = 0; k < 4; ++k) desc[k] = __builtin_amdgcn_readfirstlane(desc[k]);   // wave-uniform
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int row = b * C::RPB + lane / C::CPR;
    const int pos = lane % C::CPR;
    dma16(desc, dst + static_cast<uint32_t>(b * 1024), row * C::ROWB + ((pos ^ kswz<D>(row)) << 4));
  }
}

// Epilogue through LDS.  The wave's 32 rows of bf16 O go to its own LDS
// region (rows of 2D bytes, 16-byte chunks swizzled by the row so that the
// 8-byte writes of one instruction spread over the banks), then come back
// in row order: each global store instruction writes whole rows, 64 lanes x
// 16 contiguous bytes, instead of 16-byte pieces of 32 rows.  The region
// must not be in use by another wave (callers pass K/V ring space after the
// loop's last barrier).
template <int D>
__device__ __forceinline__ void store_rows_lds(const WaveState<D>& w, char* stage, uint16_t* o, float* lse,
                                               int64_t base, int bh, int N, int q0w, int j, int h, int lane) {
  constexpr int RB = 2 * D;                 // bytes per row
  constexpr int CPR = RB / 16;              // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;             // rows per store instruction
  const float ltot = halves_sum(w.lsum);
  const float inv = 1.f / ltot;
  char* row = stage + j * RB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c = db * 4 + g;             // chunk of channels 8c..8c+7; the lane holds 8c + 4h .. +3
      u32x2 wv;
      wv[0] = pack_bf16x2(w.oacc[db][4 * g + 0] * inv, w.oacc[db][4 * g + 1] * inv);
      wv[1] = pack_bf16x2(w.oacc[db][4 * g + 2] * inv, w.oacc[db][4 * g + 3] * inv);
      *reinterpret_cast<u32x2*>(row + ((c ^ (j % CPR)) << 4) + 8 * h) = wv;
    }
  if (lse != nullptr && h == 0 && q0w + j < N)
    lse[static_cast<int64_t>(bh) * N + q0w + j] = (w.m + __log2f(ltot)) * kLn2;
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

// ---- one tile at a time (the d=64 kernel; the last tile of a pipelined wave) ----
constexpr int kSeqReadAhead = 3;   // LDS operands in flight

// S^T for the first NKB 32-key blocks of a tile, operand reads 3 MFMAs ahead.
template <int D, int NKB>
__device__ __forceinline__ void scores_seq(f32x16 (&sacc)[BC / 32], const WaveState<D>& w,
                                           const LaneAddr<D>& la, const char* kst) {
  constexpr int NM = NKB * (D / 16), RA = kSeqReadAhead;
  bf16x8 kop[NM];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < RA && i < NM; ++i) kop[i] = k_operand<D>(kst, la, i);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    if (i + RA < NM) kop[i + RA] = k_operand<D>(kst, la, i + RA);
    const int kb = i / (D / 16), ks = i % (D / 16);
    sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[i], w.qr[ks], ks == 0 ? f32x16{} : sacc[kb], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// O^T += V^T P^T over the first NKB 32-key blocks (key steps c16 < 2*NKB).
template <int D, int NKB>
__device__ __forceinline__ void pv_seq(WaveState<D>& w, const LateWords& pl, const EarlyWords& pe,
                                       const LaneAddr<D>& la, const char* vst) {
  constexpr int NM = (D / 32) * 2 * NKB, RA = kSeqReadAhead;
  // n-th product: channel block n / (2*NKB), key step n % (2*NKB)
  auto op_index = [](int n) { return (n / (2 * NKB)) * (BC / 16) + n % (2 * NKB); };
  bf16x8 vop[NM];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int n = 0; n < RA && n < NM; ++n) vop[n] = v_operand<D>(vst, la, op_index(n));
#pragma unroll
  for (int n = 0; n < NM; ++n) {
    if (n + RA < NM) vop[n + RA] = v_operand<D>(vst, la, op_index(n + RA));
    const int i = op_index(n), db = i / (BC / 16), c16 = i % (BC / 16);
    w.oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[n], p_operand(pl, pe, c16), w.oacc[db], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NKB>
__device__ __forceinline__ float tile_max_seq(const f32x16 (&s)[BC / 32]) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  return mx;
}

// Numerators of the pairs in the first NKB key blocks, summed in the same
// grouping as the pipelined kernel (late pairs, then early pairs): p = 0 for
// the skipped block, so both kernels give the same bits.
template <int NKB>
__device__ __forceinline__ void words_seq(LateWords& pl, EarlyWords& pe, float& ll, float& le,
                                          const f32x16 (&t)[BC / 32]) {
  float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
  for (int j = 0; j < kLate; ++j)
    if (late_pair(j) / 8 < NKB) exp_pair(pl.w[late_pair(j)], ls0, ls1, t, late_pair(j), j == 0);
  ll = ls0 + ls1;
  float l0 = 0.f, l1 = 0.f;
#pragma unroll
  for (int k = 0; k < kEarly; ++k)
    if (early_pair(k) / 8 < NKB) exp_pair(pe.w[k], l0, l1, t, early_pair(k), k == 0);
  le = l0 + l1;
}

// One tile: scores, mask, exponents against the reference (the first tile's
// maximum; moved only when the numerators would pass 2^16, as in the
// pipelined kernel), numerators, P V.
template <int D, int NKB>
__device__ __forceinline__ void tile_seq(WaveState<D>& w, const LaneAddr<D>& la, const char* kst,
                                         const char* vst, int kv0, int N, int qrow, int h, bool causal,
                                         bool need_mask, bool first, float c) {
  f32x16 s[BC / 32];
  scores_seq<D, NKB>(s, w, la, kst);
  if (need_mask) {
    const int lim = key_limit(kv0, N, qrow, h, causal);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = key_off(kb, r) > lim ? -INFINITY : s[kb][r];
  }
  if (first) w.m = halves_max(tile_max_seq<NKB>(s)) * c;
  const float mref = (w.m == -INFINITY) ? 0.f : w.m;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = fmaf(s[kb][r], c, -mref);
  LateWords pl;
  EarlyWords pe;
  float ll, le;
  words_seq<NKB>(pl, pe, ll, le, s);
  if (tile_overflows<D>(ll + le)) {
    const float delta = fmaxf(halves_max(tile_max_seq<NKB>(s)), 0.f);
    const float alpha = fast_exp2(-delta);
    w.lsum *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) w.oacc[db] *= alpha;
    w.m += delta;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
    words_seq<NKB>(pl, pe, ll, le, s);
  }
  w.lsum += ll + le;
  pv_seq<D, NKB>(w, pl, pe, la, vst);
}
#endif  // __HIP_DEVICE_COMPILE__

// The causal flag is a run-time argument: the causal and non-causal launches
// share one compiled loop (a compile-time flag let the compiler allocate the
// non-causal loop into register spills).
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64, NW == 4 ? 2 : 1)
attn_mfma_bf16_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                      const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                      float* __restrict__ lse, int N, int BH, int nqb, float c, int causal_arg, int hc) {
#if defined(__HIP_DEVICE_COMPILE__)
  using C = Cfg<D, NW>;
  constexpr int BR = C::BR;
  const bool causal = causal_arg != 0;
  // two-slot rings for K and V tiles
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILEB];
  char* const kring = smem;
  char* const vring = smem + 2 * C::TILEB;
  // Q staging: the registers already limit a CU to one workgroup, so these
  // 64 KB of LDS are otherwise unused
  __shared__ __attribute__((aligned(1024))) char qstage[NW * BRW * C::ROWB];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);   // the same value, known uniform
  const int lane = tid & 63;
  const int j = lane & 31;        // query column inside the wave's 32 rows
  const int h = lane >> 5;        // lane half

  int bh, qb;
  work_item(static_cast<int>(blockIdx.x), BH, nqb, causal, hc, bh, qb);
  const int q0 = qb * BR;
  // Row block of this wave.  The waves of a workgroup are placed on the four
  // SIMDs in turn (waves w and w+4 share one), and under the causal mask a
  // block's lower rows need fewer tiles; pairing row blocks r and 7-r on a
  // SIMD gives every SIMD the same number of idle wave-tiles at the diagonal
  // (measured: 4k layer 1.0547 -> 1.0485 ms, 16k 0.9167 -> 0.9145 ms).
  const int rgp = NW == 8 ? (wave < 4 ? wave : 11 - wave) : wave;
  const int q0w = q0 + rgp * BRW;
  const int qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint16_t* kbase = k + base;
  const uint16_t* vbase = v + base;

  WaveState<D> w;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) w.oacc[db] = f32x16{};
  w.m = -INFINITY;
  w.lsum = 0.f;
  const LaneAddr<D> la(j, h, lane);

  const int kend = causal ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  // last tile this wave needs (-1: the wave's rows are all past the end),
  // and its last visible key
  int last = -1;
  if (q0w < N) last = causal ? min(ntiles - 1, (q0w + BRW - 1) / BC) : ntiles - 1;
  const int kmax = causal ? min(N - 1, q0w + BRW - 1) : N - 1;

  // ---- prologue: K0, V0, K1 and Q in flight (Q copied through LDS in whole
  // rows, then read as operands); scores of tile 0 ----
  const uint32_t kring_a = lds_addr(kring), vring_a = lds_addr(vring);   // LDS byte addresses
  issue_copy<D, NW, false>(kring_a, kbase, 0, N, wave_u, lane);
  issue_copy<D, NW, true>(vring_a, vbase, 0, N, wave_u, lane);
  if (ntiles > 1) issue_copy<D, NW, false>(kring_a + C::TILEB, kbase, BC, N, wave_u, lane);
  const char* qst = qstage + wave_u * (BRW * C::ROWB);
  issue_q_copy<D>(lds_addr(qst), q, base, q0w, N, lane);
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) w.qr[ks] = *reinterpret_cast<const bf16x8*>(qst + la.kofs[ks]);
  __syncthreads();

  f32x16 sa[BC / 32], sb[BC / 32];   // scores of the current and the next tile
  EarlyWords pea, peb;               // their early numerators ...
  float lea = 0.f, leb = 0.f;        // ... and those operands' normaliser shares
  LateWords pb;
  if (last >= 0) {
    scores<D>(sa, w, la, kring);
    if ((causal && BC - 1 > q0w) || BC > N) apply_mask(sa, 0, N, qrow, h, causal);
    first_reference<D>(w, sa, c, pea, lea);
  }
  __syncthreads();   // every wave is done with K0 before its slot is refilled

  // ---- main loop: at the top of iteration t the scores of tile t are in
  // registers (masked, reference updated), K of tile t+1 and V of tile t are
  // in LDS.  Iteration t copies V of t+1 and K of t+2.
  // The score buffers alternate roles each tile; two tiles per trip keep
  // that choice static.
  auto iteration = [&](int t, f32x16 (&scur)[BC / 32], f32x16 (&snext)[BC / 32], EarlyWords& pecur,
                       EarlyWords& penext, float& lecur, float& lenext) {
    const char* kst_next = kring + ((t + 1) & 1) * C::TILEB;
    const char* vst = vring + (t & 1) * C::TILEB;
    if (t + 1 < ntiles) issue_copy<D, NW, true>(vring_a + ((t + 1) & 1) * C::TILEB, vbase, (t + 1) * BC, N, wave_u, lane);
    if (t + 2 < ntiles) issue_copy<D, NW, false>(kring_a + (t & 1) * C::TILEB, kbase, (t + 2) * BC, N, wave_u, lane);
    if (t < last) {
      const int kv0n = (t + 1) * BC;
      float ll;
      // A wave issues its score phase at raised priority and its P V phase
      // at the normal one, so when the two waves of a SIMD drift apart the
      // one starting a tile's score products goes first: 0.3-0.7 % faster
      // than equal priorities on every shape tried (16k 0.9018 -> 0.8954
      // ms); raising the P V phase instead gains nothing.
      __builtin_amdgcn_s_setprio(1);
      phase_a<D>(w, snext, pb, ll, scur, la, kst_next);
      __builtin_amdgcn_s_setprio(0);
      commit_tile<D>(w, scur, pb, pecur, lecur, ll);
      const bool mask_next = (causal && kv0n + BC - 1 > q0w) || (kv0n + BC > N);
      if (mask_next) apply_mask(snext, kv0n, N, qrow, h, causal);
      phase_b<D>(w, snext, pb, pecur, penext, lenext, la, vst, c);
    } else if (t == last) {
      // the last tile is not pipelined; when its second 32-key block is
      // masked for all of the wave's rows (the causal diagonal of every
      // other wave, a short sequence end), that block's numerators are
      // zero and its P V products are skipped
      float ll;
      if (t * BC + 32 > kmax) {
        float l0 = 0.f, l1 = 0.f;
#pragma unroll
        for (int jj = 0; jj < kLate; ++jj)
          if (late_pair(jj) / 8 == 0) exp_pair(pb.w[late_pair(jj)], l0, l1, scur, late_pair(jj), jj == 0);
        ll = l0 + l1;
        commit_tile<D>(w, scur, pb, pecur, lecur, ll);
        pv_seq<D, 1>(w, pb, pecur, la, vst);
      } else {
        late_words(pb, ll, scur);
        commit_tile<D>(w, scur, pb, pecur, lecur, ll);
        pv_tile<D>(w, pb, pecur, la, vst);
      }
    }
    wait_vmcnt<0>();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    iteration(t, sa, sb, pea, peb, lea, leb);
    if (t + 1 < ntiles) iteration(t + 1, sb, sa, peb, pea, leb, lea);
  }

  // the rings are free after the last barrier: waves 0-3 stage O in the K
  // ring, waves 4-7 in the V ring (32 rows x 2D bytes each)
  static_assert(NW <= 8 && 4 * BRW * 2 * D <= 2 * C::TILEB, "O staging fits the rings");
  store_rows_lds<D>(w, (wave < 4 ? kring : vring) + (wave & 3) * BRW * 2 * D, o, lse, base, bh, N, q0w, j, h, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, int NW>
hipError_t launch_one(const LaunchArgs& a) {
  using C = Cfg<D, NW>;
  const int BH = a.B * a.H;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  const int64_t blocks = static_cast<int64_t>(nqb) * BH;
  const int hc = causal_head_chunk(BH, 4LL * a.N * D);      // K and V bytes of a head
  hipLaunchKernelGGL((attn_mfma_bf16_kernel<D, NW>), dim3(static_cast<unsigned>(blocks)),
                     dim3(C::NT), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                     a.N, BH, nqb, a.scale * kLog2e, a.causal, hc);
  return hipGetLastError();
}


// ---- one tile at a time: d = 64, and short rows at d = 128 ----
//
// At d=64 a 32x32x16 product covers half as many channels, so each score
// costs half the matrix work but the same vector work (scaling, exp2,
// normaliser, bf16 pack) as at d=128; the short rows of an image model add a
// prologue and a masked last tile per handful of tiles.  Software pipelining
// inside a wave needs two score buffers (182 VGPRs at d=64, two waves per
// SIMD); running each wave's tiles one after another needs 154, so three
// four-wave workgroups share a CU and the SIMDs overlap one wave's matrix
// work with another's vector work instead.  Measured side by side against
// the pipelined kernel at d=64, identical results: B=64 H=12 N=196 0.0280
// -> 0.0233 ms (0.0257 -> 0.0212 causal); N=512 to 8192, causal or not, 2-7
// % faster.  At d=128 (256 VGPRs, two workgroups per CU) it wins only on
// short rows (launch_mfma_bf16).  A wave also skips the second 32-key block
// of a tile (its score and P V products and exponentials) when every key in
// it is masked for all its rows: the last tile of a 196-key row holds 4 keys.

template <int D>
__global__ void __launch_bounds__(256, D == 64 ? 3 : 2)
attn_mfma_bf16_seq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                          const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
                          float* __restrict__ lse, int N, int BH, int nqb, float c, int causal_arg, int hc) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = 4;
  using C = Cfg<D, NW>;
  constexpr int BR = C::BR;
  const bool causal = causal_arg != 0;
  // two-slot rings for K and V tiles
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILEB];
  char* const kring = smem;
  char* const vring = smem + 2 * C::TILEB;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int j = lane & 31;
  const int h = lane >> 5;

  int bh, qb;
  work_item(static_cast<int>(blockIdx.x), BH, nqb, causal, hc, bh, qb);
  const int q0 = qb * BR;
  // Row block of this wave.  The waves of a workgroup are placed on the four
  // SIMDs in turn (waves w and w+4 share one), and under the causal mask a
  // block's lower rows need fewer tiles; pairing row blocks r and 7-r on a
  // SIMD gives every SIMD the same number of idle wave-tiles at the diagonal
  // (measured: 4k layer 1.0547 -> 1.0485 ms, 16k 0.9167 -> 0.9145 ms).
  const int rgp = NW == 8 ? (wave < 4 ? wave : 11 - wave) : wave;
  const int q0w = q0 + rgp * BRW;
  const int qrow = q0w + j;
  const int64_t base = static_cast<int64_t>(bh) * N * D;
  const uint16_t* kbase = k + base;
  const uint16_t* vbase = v + base;

  WaveState<D> w;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) w.oacc[db] = f32x16{};
  w.m = -INFINITY;
  w.lsum = 0.f;
  const LaneAddr<D> la(j, h, lane);

  const int kend = causal ? min(N, q0 + BR) : N;
  const int ntiles = (kend + BC - 1) / BC;
  // last tile this wave needs (-1: the wave's rows are all past the end),
  // and its last visible key
  int last = -1;
  if (q0w < N) last = causal ? min(ntiles - 1, (q0w + BRW - 1) / BC) : ntiles - 1;
  const int kmax = causal ? min(N - 1, q0w + BRW - 1) : N - 1;

  const uint32_t kring_a = lds_addr(kring), vring_a = lds_addr(vring);
  issue_copy<D, NW, false>(kring_a, kbase, 0, N, wave, lane);
  issue_copy<D, NW, true>(vring_a, vbase, 0, N, wave, lane);
  // Q through the second ring slots (free until the first iteration's
  // copies): waves 0-1 in the K slot, waves 2-3 in the V slot, 32 rows each
  static_assert(2 * BRW * C::ROWB == C::TILEB, "two waves' Q rows fill a slot");
  const int qoff = C::TILEB + (wave & 1) * (BRW * C::ROWB);
  const char* qst = (wave < 2 ? kring : vring) + qoff;
  issue_q_copy<D>((wave < 2 ? kring_a : vring_a) + qoff, q, base, q0w, N, lane);
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) w.qr[ks] = *reinterpret_cast<const bf16x8*>(qst + la.kofs[ks]);
  __syncthreads();   // K0/V0 landed for every wave; every wave holds its Q before slot 1 is refilled

  // At the top of iteration t, K and V of tile t are in ring slot t&1; the
  // iteration copies tile t+1 into the other slot, which every wave left at
  // the previous barrier.
  for (int t = 0; t < ntiles; ++t) {
    const int kv0 = t * BC;
    if (t + 1 < ntiles) {
      issue_copy<D, NW, false>(kring_a + ((t + 1) & 1) * C::TILEB, kbase, kv0 + BC, N, wave, lane);
      issue_copy<D, NW, true>(vring_a + ((t + 1) & 1) * C::TILEB, vbase, kv0 + BC, N, wave, lane);
    }
    if (t <= last) {
      const char* kst = kring + (t & 1) * C::TILEB;
      const char* vst = vring + (t & 1) * C::TILEB;
      const bool need_mask = (causal && kv0 + BC - 1 > q0w) || (kv0 + BC > N);
      if (kv0 + 32 > kmax)
        tile_seq<D, 1>(w, la, kst, vst, kv0, N, qrow, h, causal, need_mask, t == 0, c);
      else
        tile_seq<D, 2>(w, la, kst, vst, kv0, N, qrow, h, causal, need_mask, t == 0, c);
    }
    wait_vmcnt<0>();
    __syncthreads();
  }

  static_assert(NW * BRW * 2 * D <= 4 * C::TILEB, "O staging fits the rings");
  store_rows_lds<D>(w, smem + wave * BRW * 2 * D, o, lse, base, bh, N, q0w, j, h, lane);
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D>
hipError_t launch_seq(const LaunchArgs& a) {
  using C = Cfg<D, 4>;
  const int BH = a.B * a.H;
  const int nqb = (a.N + C::BR - 1) / C::BR;
  const int64_t blocks = static_cast<int64_t>(nqb) * BH;
  const int hc = causal_head_chunk(BH, 4LL * a.N * D);      // K and V bytes of a head
  hipLaunchKernelGGL((attn_mfma_bf16_seq_kernel<D>), dim3(static_cast<unsigned>(blocks)),
                     dim3(C::NT), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
                     static_cast<const uint16_t*>(a.v), static_cast<uint16_t*>(a.o), a.lse,
                     a.N, BH, nqb, a.scale * kLog2e, a.causal, hc);
  return hipGetLastError();
}

}  // namespace

// d = 128: the pipelined kernel with eight waves (two per SIMD, one K/V tile
// copy shared by 256 query rows), measured faster than four, except on
// short rows (at most 8 tiles of keys per query block on average), where
// the one-tile-at-a-time kernel at two four-wave workgroups per CU wins:
// measured side by side, N=512 0.1022 -> 0.0974 ms (causal 0.0863 ->
// 0.0762), causal N=1024 0.1179 -> 0.1101, N=196 0.0497 -> 0.0450, while
// N=1024 non-causal (0.1528 against 0.1578) and N=2048 stay pipelined.
// d = 64: the one-tile-at-a-time kernel, three four-wave workgroups per CU.
hipError_t launch_mfma_bf16(const LaunchArgs& a) {
  if (a.d == 64) return launch_seq<64>(a);
  const int64_t row_keys = a.causal ? a.N / 2 : a.N;     // keys of an average row
  return row_keys <= 512 ? launch_seq<128>(a) : launch_one<128, 8>(a);
}

}  // namespace attn127
