/*
 * attn.h -- C ABI of the fused exact-attention library (gfx950): forward,
 * fp8 and MXFP8 forward, and backward.
 *
 * The operation (page "Self-Attention, CUDA kernels and FlashAttention",
 * section 1): for every batch b and head h, with Q, K, V the N x d slices
 * [b][h],
 *
 *     S = Q K^T * scale,   P = row-softmax(S),   O = P V
 *
 * and (same page, section 3) only O and one small statistic per query row
 * are written: the natural-log log-sum-exp of that row's scaled, masked
 * scores, LSE_i = ln sum_j exp(S_ij).  The N x N matrices S and P never go to
 * device memory.  Heads are independent and run in parallel (section 1,
 * multi-head paragraph); query blocks of one head run in parallel too
 * (page "FlashAttention scaling, multi-GPU training and weight
 * quantization", section 1, the sequence-length-parallelism bullet).
 *
 * Common conventions
 *   Layout     q, k, v, o: contiguous row-major [B][H][N][d]; lse: [B][H][N].
 *              Element (b,h,i,c) sits at ((b*H + h)*N + i)*d + c.
 *   Causal     causal != 0 masks key j for query i when j > i (square
 *              self-attention: row i sees keys 0..i).
 *   Scale      scale must be finite and > 0, or exactly 0 to select
 *              1/sqrt(d), the scaled dot-product's own factor (page
 *              "Self-Attention, CUDA kernels and FlashAttention", section 1).
 *   Sizes      B, H, N >= 0 (any zero makes the call a no-op that returns
 *              ATTN_OK); d must be 64 or 128; B*H*N*d < 2^31 is not needed
 *              (offsets are 64-bit), but B*H < 2^31 and N < 2^30.
 *   Pointers   device pointers, 16-byte aligned, owned by the caller; the
 *              library allocates, frees and retains nothing and keeps no
 *              global state, so calls on different streams are independent.
 *              The one exception is attn_bwd_static, which keeps a fixed
 *              scratch array per GPU (see there).  lse may be NULL (the
 *              statistic is then not written).  Inputs must not alias
 *              outputs.
 *   Stream     a hipStream_t passed as void* (NULL = the null stream).  Every
 *              call only enqueues work and returns; the caller synchronises.
 *   Errors     a negative attn_status.  Arguments are checked on the host
 *              before any HIP call, so a rejected call has no device side
 *              effect.  ATTN_ERR_HIP reports a failed launch; faults during
 *              execution surface at the caller's synchronisation.
 */
#ifndef ATTN127_ATTN_H
#define ATTN127_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,   /* q, k, v, o are float32                                  */
  ATTN_BF16 = 1   /* q, k, v, o are bfloat16 (bit pattern in uint16)        */
} attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = -1,  /* null / misaligned pointer, bad size or scale */
  ATTN_ERR_UNSUPPORTED = -2,  /* valid request this build has no kernel for  */
  ATTN_ERR_HIP = -3,          /* the HIP runtime rejected a launch            */
  ATTN_ERR_TOO_LARGE = -4     /* request exceeds a fixed buffer of the library */
} attn_status;

/*
 * attn_fwd -- O = softmax(Q K^T * scale) V and LSE for all B*H heads.
 *
 * dtype ATTN_BF16 runs the matrix-core kernel: both products on bf16 MFMA
 * with float32 accumulation, the online softmax (a running normaliser and a
 * per-row exponent reference -- the first key tile's maximum, moved to a
 * later tile's maximum only when that tile's numerators would grow past
 * 2^16 -- with the partial output rescaled whenever the reference moves;
 * page "Self-Attention, CUDA kernels and FlashAttention", section 3) in
 * float32, P rounded to bf16 (nearest-even) as the second product's operand,
 * the 1/normaliser division done once after the last key tile (page
 * "FlashAttention scaling, multi-GPU training and weight quantization",
 * section 1, the bullet on fewer non-matmul operations), O rounded to bf16
 * (nearest-even).  dtype ATTN_F32 keeps every step in float32 (no bf16
 * rounding anywhere).  lse is float32 in both cases.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int N, int d, float scale, int causal, int dtype,
             void* stream);

/*
 * attn_fwd_simple -- the same operation and contract as attn_fwd, computed
 * by a plain tiled kernel with float32 vector arithmetic (no matrix cores,
 * no bf16 rounding of P).  A second, structurally different device path,
 * kept for cross-checking; not tuned.
 */
int attn_fwd_simple(const void* q, const void* k, const void* v, void* o,
                    float* lse, int B, int H, int N, int d, float scale,
                    int causal, int dtype, void* stream);

/* Tokens per fp8 quantisation tile: one float32 scale per (b, h, tile). */
#define ATTN_FP8_TILE 128

/*
 * attn_fp8_prepare -- block quantisation with incoherent processing (page
 * "FlashAttention scaling, multi-GPU training and weight quantization",
 * section 1, the FP8 bullet).
 *
 *   q', k' = q R, k R      R: float32 [d][d] row-major, orthogonal (caller's
 *                          seeded draw; the product is not checked); v is
 *                          not rotated.
 *   For each (b, h, t) with tile t = tokens [128 t, 128 t + 128) of all d
 *   channels:  s = amax / 448 (s = 1 when amax = 0), code = e4m3(x / s)
 *   (OCP E4M3FN, nearest-even, saturating to +-448).
 *
 * q, k, v: float32 [B][H][N][d].  q8, k8, v8: uint8 codes [B][H][N][d].
 * q_scale, k_scale, v_scale: float32 [B][H][ceil(N/128)].
 * The rotation runs on float32 matrix cores (products exact, float32
 * accumulation).  ATTN_ERR_INVALID_ARG also when 3*B*H*ceil(N/128) >= 2^30
 * (the work items are indexed in 32 bits; such inputs exceed device memory).
 */
int attn_fp8_prepare(const float* q, const float* k, const float* v,
                     const float* R, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                     float* q_scale, float* k_scale, float* v_scale,
                     int B, int H, int N, int d, void* stream);

/*
 * attn_fwd_fp8 -- attention on the e4m3 tensors attn_fp8_prepare writes
 * (page "FlashAttention scaling, multi-GPU training and weight
 * quantization", section 1, the FP8 bullet: the score product on FP8 matrix
 * units, inputs block-quantised with one scale per tile).
 * Value of an input element = decode(code) * scale of its 128-token tile.
 * Q K^T runs on fp8 MFMA (e4m3 x e4m3, float32 accumulation) with the Q and
 * K tile scales folded into the exponent's multiplier.  P V runs on fp16
 * MFMA: each e4m3 V operand is widened to fp16 (exact) in registers, and P,
 * carrying the V tile's scale relative to the head's largest V tile scale,
 * is rounded to fp16 (nearest-even).  o is bf16
 * [B][H][N][d]; lse (nullable) float32 [B][H][N].  The tile scales must be
 * positive normal floats, as attn_fp8_prepare writes them; they live in
 * device memory and are not checked.  Other conventions as attn_fwd.
 */
int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                 const float* q_scale, const float* k_scale,
                 const float* v_scale, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, void* stream);

/* Channels per MXFP8 block: one E8M0 scale per (b, h, token, block). */
#define ATTN_MX_BLOCK 32

/*
 * attn_mxfp8_prepare -- MXFP8 block quantisation (page "Efficient MoE
 * training for biological foundation models", the section on memory and
 * quantisation costs: 8-bit values with one scale per block of 32 values)
 * after the same incoherent processing as attn_fp8_prepare (q' = q R,
 * k' = k R; v not rotated).  For every token and every 32 consecutive
 * channels: e = ceil(log2(amax / 448)) clamped to [-127, 127] (e = -127 when
 * amax = 0), scale byte = e + 127 (E8M0), code = e4m3(x / 2^e) (OCP E4M3FN,
 * nearest-even; no saturation occurs since amax / 2^e <= 448).
 *
 * q, k, v: float32 [B][H][N][d].  q8, k8, v8: uint8 codes [B][H][N][d].
 * q_scale, k_scale, v_scale: uint8 [B][H][N][d/32], aligned to d/32 bytes.
 */
int attn_mxfp8_prepare(const float* q, const float* k, const float* v,
                       const float* R, uint8_t* q8, uint8_t* k8, uint8_t* v8,
                       uint8_t* q_scale, uint8_t* k_scale, uint8_t* v_scale,
                       int B, int H, int N, int d, void* stream);

/*
 * attn_fwd_mxfp8 -- attention on the MXFP8 tensors attn_mxfp8_prepare
 * writes.  Value of an element = decode(code) * 2^(scale byte - 127) of its
 * 32-channel block.  Q K^T runs on the block-scaled fp8 MFMA, which applies
 * the Q and K block scales (every lane's 32 codes form one block); P V runs on
 * bf16 MFMA with each V block widened to bf16 with its scale (exact) and P
 * rounded to bf16.  o is bf16 [B][H][N][d]; lse (nullable) float32 [B][H][N].
 * Other conventions as attn_fwd.
 */
int attn_fwd_mxfp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8,
                   const uint8_t* q_scale, const uint8_t* k_scale,
                   const uint8_t* v_scale, void* o, float* lse, int B, int H,
                   int N, int d, float scale, int causal, void* stream);

/*
 * attn_bwd -- gradients of attn_fwd (page "Self-Attention, CUDA kernels and
 * FlashAttention", section 3: the backward pass keeps only the per-row
 * statistic and recomputes the attention tiles on chip).  Given dO, the
 * gradient of a loss with respect to O, for every head:
 *
 *     P = exp(S - LSE)  (recomputed, masked as in the forward pass)
 *     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
 *     dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
 *
 * q, k, v, o, dout: bf16 [B][H][N][d], o and lse exactly as attn_fwd wrote
 * them for the same q, k, v, scale and causal.  dq, dk, dv: bf16
 * [B][H][N][d], written.  lse: float32 [B][H][N], read (4-byte aligned).
 * delta: float32 [B][H][N], the caller's scratch (4-byte aligned), receives D.
 * All products on bf16 MFMA with float32 accumulation; P and dS rounded to
 * bf16 (nearest-even) as operands; outputs rounded to bf16.  dtype must be
 * ATTN_BF16 (ATTN_F32 returns ATTN_ERR_UNSUPPORTED).  Three launches on
 * `stream`, no atomics: results are deterministic.  Other conventions as
 * attn_fwd; lse and delta may not be NULL.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, float* delta, void* dq,
             void* dk, void* dv, int B, int H, int N, int d, float scale,
             int causal, int dtype, void* stream);

/* Floats of device scratch attn_bwd_static holds per GPU (16 MiB). */
#define ATTN_STATIC_SCRATCH_FLOATS 4194304

/*
 * attn_bwd_static -- attn_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, kernels and results, without the delta
 * scratch argument.  D lives instead in a fixed array of
 * ATTN_STATIC_SCRATCH_FLOATS floats that the library holds on every GPU it
 * runs on until the process ends; the first call on a device looks up that
 * device's copy (the current device at the call).  The call allocates
 * nothing.  B*H*N above ATTN_STATIC_SCRATCH_FLOATS returns ATTN_ERR_TOO_LARGE
 * before any HIP call.  Every call on one GPU uses that GPU's single array:
 * calls that overlap on one GPU (different streams, or host threads without
 * ordering) race and must not be issued; calls in order on one stream are
 * safe.  Other arguments, conventions and errors as attn_bwd.
 */
int attn_bwd_static(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk,
                    void* dv, int B, int H, int N, int d, float scale,
                    int causal, int dtype, void* stream);

/* Weights per scale group of the W4A16 product. */
#define W4A16_GROUP 128

/*
 * w4a16_gemm -- Y = X W^T with 4-bit weights dequantised in registers (page
 * "FlashAttention scaling, multi-GPU training and weight quantization",
 * section 3: packed INT4 weights read from HBM, unpacked with shifts and
 * masks, scale and zero point applied to give FP16 values that go straight
 * to the matrix cores; the expanded weights are never written to memory).
 *
 *   w[n][k] = fp16(s[n][k/128] * (q[n][k] - z[n][k/128]))   (rounded once)
 *   Y[m][n] = fp16(sum_k X[m][k] w[n][k])                    (float32 sums)
 *
 * x: fp16 [M][K], 1 <= M <= 16 (tokens of a decode step), 16-byte aligned.
 * qweight: uint32 [N][K/8]; word (n, j) holds q[n][8j + i] in bits 4i..4i+3;
 * 16-byte aligned.  scales: fp16 [N][K/128], 2-byte aligned.  zeros: uint8
 * [N][K/128], values 0..15.  y: fp16 [M][N], 8-byte aligned.
 * group must be 128 and K at most 32768 (ATTN_ERR_UNSUPPORTED otherwise);
 * K a multiple of 128;
 * the packed weights below 2 GiB (N*K/2 < 2^31) and K < 2^26.
 * M, N or K = 0: no-op.  M > 16, a bad size, pointer or alignment:
 * ATTN_ERR_INVALID_ARG before any HIP call.  Asynchronous on stream;
 * deterministic (the four K slices of a row block are summed in a fixed
 * order).  The caller owns all memory; nothing is allocated.
 */
int w4a16_gemm(const void* x, const uint32_t* qweight, const void* scales,
               const uint8_t* zeros, void* y, int M, int N, int K, int group,
               void* stream);

/*
 * w4a16_dequantize -- the fp16 weights w[n][k] of w4a16_gemm written out to
 * w (fp16 [N][K], 16-byte aligned): the unfused path the product avoids,
 * for checking the dequantisation bit for bit.  Other arguments and errors
 * as w4a16_gemm.
 */
int w4a16_dequantize(const uint32_t* qweight, const void* scales,
                     const uint8_t* zeros, void* w, int N, int K, int group,
                     void* stream);

/* Static, human-readable text for a status code (never NULL). */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN127_ATTN_H */
