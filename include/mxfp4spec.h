/*
 * mxfp4spec.h — C ABI of the MX-FP4 speculative verification library (AMD gfx950).
 *
 * The library implements the two parts of the target model's verification step
 * in speculative decoding:
 *
 *   1. a weight-streaming GEMM over OCP MX-FP4 weights that reads every weight
 *      once and applies it to the T = K+1 draft positions, and
 *   2. the rejection-sampling acceptance step over the target and draft logits.
 *
 * Sources (the pages this library follows):
 *   [M11]  "Module 11. Speculative Decoding and Quantization" (Modern LLMs
 *          lecture): §4 acceptance rule a(x) = min(1, p/q), first-rejection
 *          stop, residual r = norm((p - q)+), bonus token; §5 edge cases
 *          (q(t) = 0, zero draw); §12 E2M1 / E8M0 / 32-element MX blocks and
 *          4.25 bits per value; §13 validation refuses, never repairs.
 *   [NEWS] "Next-Gen Speculative Decoding and FP4 Quantization Shake Up LLM
 *          Inference Economics", section "Microscaling FP4 (MX-FP4)
 *          Integration": packed weights [N, K/2] and scales [N, K/32], fp32
 *          accumulation, one verification pass over all K candidates.
 *
 * Conventions for every entry point
 *   - Every data pointer is a DEVICE pointer, allocated and owned by the caller.
 *     The library allocates no memory, keeps no mutable global state and is
 *     safe to call from several host threads. The one exception is
 *     spec_accept_noalloc, whose workspace is a static device array of the
 *     library (calls on one GPU share it and must not overlap).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream)
 *     and runs asynchronously: the caller synchronizes before reading outputs.
 *   - Arrays are row-major and contiguous.
 *   - Errors that the host can see (NULL pointers, sizes, alignment, workspace
 *     size) are returned BEFORE any HIP call, and nothing is enqueued.
 *     MXS_ERR_DEVICE is returned when no HIP device is usable or the current
 *     device is not gfx950; MXS_ERR_LAUNCH when a kernel launch fails.
 *   - Conditions only the device can see are OR-ed into the caller's
 *     `*dev_flags` word (device memory) with the MXS_FLAG_* bits. The library
 *     never clears it: zero it before a call to read that call's flags alone.
 *     `dev_flags` may be NULL, in which case nothing is reported.
 */
#ifndef MXFP4SPEC_H
#define MXFP4SPEC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mxs_status {
  MXS_OK = 0,
  MXS_ERR_NULL = 1,      /* a required pointer is NULL */
  MXS_ERR_SHAPE = 2,     /* a size is out of range (see each entry point) */
  MXS_ERR_ALIGN = 3,     /* a pointer is not aligned as documented */
  MXS_ERR_WORKSPACE = 4, /* the workspace is smaller than the query returns */
  MXS_ERR_DEVICE = 5,    /* no usable HIP device, or it is not gfx950 */
  MXS_ERR_LAUNCH = 6,    /* a kernel launch failed */
  MXS_ERR_VALUE = 7      /* an argument value is out of range (see each entry point) */
} mxs_status;

/* Device-detected conditions (bits of *dev_flags). */
#define MXS_FLAG_NONFINITE 1     /* NaN/+inf input (or a logit row with no finite value) */
#define MXS_FLAG_TOKEN_RANGE 2   /* a draft token outside [0, V) */
#define MXS_FLAG_Q_ZERO 4        /* a draft token with draft probability 0 */
#define MXS_FLAG_RESIDUAL_ZERO 8 /* a rejection whose residual (p - q)+ had zero mass */

/* Activation formats of the W4A8 / W4A4 product (the element-format numbers of the
   block-scaled matrix instruction). */
#define MXS_ACT_FP8 0  /* MX-FP8: E4M3 elements, E8M0 scale per 32 */
#define MXS_ACT_FP4 4  /* MX-FP4: E2M1 elements, E8M0 scale per 32 */

#define MXS_ABI_VERSION 1

/* Human-readable name of a status code (static storage; never NULL). */
const char* mxs_status_string(int status);

/* MXS_ABI_VERSION of the built library. */
int mxs_abi_version(void);

/*
 * mxfp4_quantize — fp32 W[n, k] -> MX-FP4 (E2M1 codes + one E8M0 scale per
 * 32 consecutive elements of a row). [M11 §12] fixes the format; the block
 * exponent follows the OCP MX v1.0 rule the lecture cites:
 *   e = floor(log2(max |v|)) - 2, clamped to [-127, 127] (an all-zero block
 *   gets e = -127), scale byte = e + 127 (value 2^(s-127));
 *   each element v * 2^-e is rounded to the nearest E2M1 value
 *   {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even encoding, magnitudes above
 *   6 saturate to 6; the sign bit is the sign bit of v (so -0 -> code 8).
 *   A block holding a NaN or infinity gets scale byte 0xFF (the E8M0 NaN),
 *   codes 0, and sets MXS_FLAG_NONFINITE.
 *
 * w       [n, k] fp32, 16-byte aligned.
 * n, k    n >= 1, k >= 32, k % 32 == 0.
 * codes   [n, k/2] bytes, 16-byte aligned. Element (r, c) is the nibble of
 *         byte r*k/2 + c/2: the low nibble when c is even. [NEWS] layout.
 * scales  [n, k/32] bytes (E8M0), any alignment.
 * Returns MXS_ERR_NULL (w, codes, scales), MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status mxfp4_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes,
                          uint8_t* scales, int32_t* dev_flags, void* stream);

/*
 * mxfp4_verify_gemm — Y[m, n] = X[m, k] · Ŵ[n, k]ᵀ with
 * Ŵ = E2M1(code) · 2^(scale - 127) decoded in registers and products summed in
 * fp32. The verification pass reads every weight once for all m = B·T
 * activation rows ([M11 §4, §10]; [NEWS] fp32-accumulated MX-FP4 GEMV).
 * Weights are decoded exactly; activations are taken exactly; only the fp32
 * summation rounds. Dequantized weights below 2^-126 in magnitude (scale
 * bytes 0 and 1) may be flushed to zero by the matrix cores.
 *
 * codes   [n, k/2] bytes as written by mxfp4_quantize, 16-byte aligned.
 * scales  [n, k/32] E8M0 bytes, any alignment.
 * n, k    n >= 1, k >= 32, k % 32 == 0.
 * x       [m, k] bf16 bit patterns (uint16), 16-byte aligned.
 * m       1 <= m <= 65536 (rows are sequences × positions, sequence-major).
 * y       [m, n] fp32, 4-byte aligned. Fully overwritten.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status mxfp4_verify_gemm(const uint8_t* codes, const uint8_t* scales, int64_t n,
                             int64_t k, const uint16_t* x, int64_t m, float* y,
                             void* stream);

/*
 * mxfp4_verify_gemm_grouped — several independent verify GEMMs with the same k
 * and m in one launch where possible: Y_i = X_i · Ŵ_iᵀ for i < count, each as
 * mxfp4_verify_gemm defines it (same numerics, same layouts and alignment).
 * This is the verification pass over a layer's projections that read the same
 * input (q, k, v; gate, up) without concatenating their weights [M11 §4, §10].
 * Groups of up to 8 products share one launch; larger counts use several.
 *
 * problems  HOST array of `count` descriptors, read during the call only.
 * count     1 <= count <= 65536.
 * k, m      shared by all products: k >= 32, k % 32 == 0; 1 <= m <= 65536.
 * Returns MXS_ERR_NULL (problems or any pointer in it), MXS_ERR_SHAPE, MXS_ERR_ALIGN;
 * nothing is enqueued when any descriptor is invalid.
 */
typedef struct mxs_gemm_problem {
  const uint8_t* codes;  /* [n, k/2], 16-byte aligned */
  const uint8_t* scales; /* [n, k/32] */
  const uint16_t* x;     /* [m, k] bf16, 16-byte aligned */
  float* y;              /* [m, n] fp32, 4-byte aligned */
  int64_t n;             /* output rows of this product, >= 1 */
} mxs_gemm_problem;

mxs_status mxfp4_verify_gemm_grouped(const mxs_gemm_problem* problems, int32_t count, int64_t k,
                                     int64_t m, void* stream);

/*
 * nvfp4_quantize — fp32 W[n, k] -> NVFP4 [M11 §12: E2M1 values, one E4M3 scale
 * per 16 values, one fp32 scale for the tensor; 4.5 bits/value counting the
 * block scales].
 *
 * g = amax(|W|) / (6 * 448) over the finite entries (1 for an all-zero tensor);
 * block scale = E4M3 (bias 7, subnormals, NaN = 0x7F, largest 448) of
 * amax_block / (6 g), nearest with ties to the even fraction, saturating; each
 * value is coded from w / (E4M3 * g) as mxfp4_quantize codes (nearest, ties to
 * even, saturating at 6, sign of zero kept). Each step is one correctly rounded
 * fp32 operation. A block holding a NaN or +-inf gets scale 0x7F and codes 0,
 * and raises MXS_FLAG_NONFINITE; such entries are left out of amax.
 *
 * w             [n, k] fp32, 16-byte aligned; k % 16 == 0, k >= 16.
 * codes         [n, k/2] bytes as mxfp4_quantize (low nibble = even column), 2-byte aligned.
 * scales        [n, k/16] E4M3 bytes.
 * global_scale  one fp32 in device memory: g (written; also used as scratch).
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status nvfp4_quantize(const float* w, int64_t n, int64_t k, uint8_t* codes, uint8_t* scales,
                          float* global_scale, int32_t* dev_flags, void* stream);

/*
 * nvfp4_verify_gemm — Y[m, n] = X[m, k] · Ŵ[n, k]ᵀ with
 * Ŵ = E2M1(code) * E4M3(scale) * g [M11 §12], fp32 accumulation of exact bf16
 * products (E2M1 * E4M3 is exact in bf16), g applied to each output once.
 * Layouts as nvfp4_quantize; x bf16 [m, k] row-major; y fp32 [m, n].
 * k % 512 == 0 (no other k is supported by this kernel), 1 <= m <= 65536
 * (positions beyond 16 run as further 16-position tiles that re-read the
 * weights: the batched dense path is MX-FP4 only). codes, scales, x 16-byte
 * aligned; y, global_scale 4-byte aligned.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status nvfp4_verify_gemm(const uint8_t* codes, const uint8_t* scales, const float* global_scale,
                             int64_t n, int64_t k, const uint16_t* x, int64_t m, float* y,
                             void* stream);

/*
 * nvfp4_verify_gemm_grouped — several independent NVFP4 products with the same k and m
 * (the projections of a layer that read the same input), up to 8 per launch, as
 * mxfp4_verify_gemm_grouped does for MX-FP4. Each product has its own tensor scale.
 * Same argument rules as nvfp4_verify_gemm for every product.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
typedef struct mxs_nvfp4_problem {
  const uint8_t* codes;       /* [n, k/2] */
  const uint8_t* scales;      /* [n, k/16] E4M3 */
  const float* global_scale;  /* one fp32 in device memory */
  const uint16_t* x;          /* [m, k] bf16 */
  float* y;                   /* [m, n] fp32 */
  int64_t n;
} mxs_nvfp4_problem;

mxs_status nvfp4_verify_gemm_grouped(const mxs_nvfp4_problem* problems, int32_t count, int64_t k, int64_t m,
                                     void* stream);

/*
 * nvfp4_verify_gemm_grouped_tiled — nvfp4_verify_gemm_grouped with each product's codes
 * in the tiled layout of mxfp4_tile_codes (NVFP4 codes pack E2M1 values as MX-FP4 codes
 * do; the E4M3 scales stay in the row layout [n, k/16]). Every wave-wide code load then
 * reads 1 KiB contiguously [the byte order is this library's choice]. Same rules, errors
 * and kernel; the result is bit-identical to nvfp4_verify_gemm_grouped's. One product is
 * a group of one. n <= 2^31 - 16.
 */
mxs_status nvfp4_verify_gemm_grouped_tiled(const mxs_nvfp4_problem* problems, int32_t count, int64_t k, int64_t m,
                                           void* stream);

/*
 * mx_quantize_act — bf16 activations X[m, k] -> MX-FP8 or MX-FP4 [M11 §11: W4A8 /
 * W4A4 quantize activations as well as weights; §12: E4M3 = 8-bit float with 4
 * exponent and 3 fraction bits, E8M0 power-of-two scale; news page, "Microscaling
 * FP4 (MX-FP4) Integration": 32 values per scale].
 *
 * Per 32-value block along k: e = floor(log2 amax) - emax (8 for E4M3, whose
 * largest value is 448 = 1.75 * 2^8; 2 for E2M1), clamped to [-127, 127], scale
 * byte e + 127 (0 for an all-zero block); each value v * 2^-e goes to the nearest
 * element value with ties to the even fraction, saturating (at 448 or 6), sign
 * kept on zeros. A block holding a NaN or +-inf gets scale 0xFF and codes 0, and
 * raises MXS_FLAG_NONFINITE.
 *
 * x       [m, k] bf16, 16-byte aligned; k % 32 == 0.
 * fmt     MXS_ACT_FP8 or MXS_ACT_FP4 (else MXS_ERR_VALUE).
 * codes   FP8: [m, k] E4M3 bytes, 8-byte aligned. FP4: [m, k/2] as mxfp4_quantize
 *         (low nibble = even column), 4-byte aligned.
 * scales  [m, k/32] E8M0 bytes.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN, MXS_ERR_VALUE.
 */
mxs_status mx_quantize_act(const uint16_t* x, int64_t m, int64_t k, int32_t fmt, uint8_t* codes,
                           uint8_t* scales, int32_t* dev_flags, void* stream);

/*
 * mx_verify_gemm_act — Y[m, n] = X^[m, k] · Ŵ[n, k]ᵀ: MX-FP4 weights (mxfp4_quantize
 * layout) times MX-quantized activations (mx_quantize_act layout, format fmt), the
 * W4A8 / W4A4 forms of the verify GEMM [M11 §11, §12]. Products of the two decoded
 * operands (element × element × 2^(sw + sx - 254)) are exact; they are summed in
 * fp32 by the block-scaled matrix instruction, so Y is the product of the QUANTIZED
 * activations (a different result from mxfp4_verify_gemm on the bf16 ones).
 * Built for the batched verification (m = sequences × positions); any 1 <= m <= 65536
 * is accepted.
 *
 * k % 128 == 0, k <= 2^24; codes and act_codes 16-byte aligned; scales and act_scales
 * 4-byte aligned; y fp32 [m, n], 4-byte aligned. Returns MXS_ERR_NULL, MXS_ERR_SHAPE,
 * MXS_ERR_ALIGN, MXS_ERR_VALUE (fmt).
 */
mxs_status mx_verify_gemm_act(const uint8_t* codes, const uint8_t* scales, int64_t n, int64_t k,
                              const uint8_t* act_codes, const uint8_t* act_scales, int32_t fmt, int64_t m,
                              float* y, void* stream);

/*
 * mxfp4_tile_codes — MX-FP4 codes in the mxfp4_quantize row layout [n, k/2] -> the
 * tiled layout read by mx_verify_gemm_act_tiled, mxfp4_verify_gemm_tiled,
 * mxfp4_verify_gemm_grouped_tiled and (for NVFP4 codes, which pack E2M1 values the same way)
 * nvfp4_verify_gemm_grouped_tiled. This is a byte permutation done once at weight-prep time, like the quantization itself [M11 §12
 * fixes the values; the byte order in memory is this library's choice]. The scales have
 * a tiled layout of their own (mxfp4_tile_scales).
 *
 * Tiled layout: one 1 KiB tile per (16-row tile t, 128-k group q), at byte
 * (t * (k/128) + q) * 1024. Its 16-byte unit L = 16 * g + r (g = 0..3, r = 0..15)
 * holds the 16 bytes of row 16 t + r, MX block 4 q + g (columns 128 q + 32 g ..
 * + 31, low nibble = even column, as in the row layout). Rows past n (up to the
 * next multiple of 16) are zero.
 *
 * codes   [n, k/2], 16-byte aligned; k % 128 == 0, k >= 128.
 * tiled   mxfp4_tiled_bytes(n, k) bytes (= ceil(n/16) * 16 * k/2), 16-byte aligned.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
size_t mxfp4_tiled_bytes(int64_t n, int64_t k); /* 0 when the sizes are out of range */
mxs_status mxfp4_tile_codes(const uint8_t* codes, int64_t n, int64_t k, uint8_t* tiled, void* stream);

/*
 * mxfp4_tile_scales — E8M0 scales in the row layout [n, k/32] -> the tiled scale layout
 * read by mx_verify_gemm_act_tiled, mxfp4_verify_gemm_tiled and
 * mxfp4_verify_gemm_grouped_tiled: 2 KiB per (128-row tile t, 512-k window w) at byte
 * (t * ceil(k/512) + w) * 2048. Its 16-byte unit r holds the scale bytes of columns
 * 512 w .. 512 w + 511 (bytes 16 w .. 16 w + 15 of the row) of row 128 t + r. Bytes
 * past k/32 and rows past n are zero.
 *
 * scales  [n, k/32], 4-byte aligned; k % 128 == 0, k >= 128.
 * tiled   mxfp4_tiled_scale_bytes(n, k) bytes, 16-byte aligned.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
size_t mxfp4_tiled_scale_bytes(int64_t n, int64_t k); /* 0 when the sizes are out of range */
mxs_status mxfp4_tile_scales(const uint8_t* scales, int64_t n, int64_t k, uint8_t* tiled, void* stream);

/*
 * mx_verify_gemm_act_tiled — mx_verify_gemm_act with the weight codes in the tiled
 * layout of mxfp4_tile_codes and the weight scales in that of mxfp4_tile_scales. Every
 * wave-wide weight load then reads 1 KiB contiguously instead of 64 bytes from each of
 * 16 rows, and a window's weight scales arrive in two 1 KiB loads. The result is
 * bit-identical to mx_verify_gemm_act on the same weights. Same arguments, rules and
 * errors; tiled_scales must be 16-byte aligned.
 */
mxs_status mx_verify_gemm_act_tiled(const uint8_t* tiled_codes, const uint8_t* tiled_scales, int64_t n, int64_t k,
                                    const uint8_t* act_codes, const uint8_t* act_scales, int32_t fmt, int64_t m,
                                    float* y, void* stream);

/*
 * mxfp4_verify_gemm_tiled — mxfp4_verify_gemm with the weight codes in the tiled
 * layout of mxfp4_tile_codes and the weight scales in that of mxfp4_tile_scales
 * [M11 §4, §10; the byte order is this library's choice]. Every wave-wide weight load
 * then reads 1 KiB contiguously instead of 64 bytes from each of 16 rows. Same product
 * and numerics. Kernels: for m <= 32 with k % 512 == 0 the skinny kernel of
 * mxfp4_verify_gemm, otherwise its dense kernel (any m, k % 128 == 0). Where
 * mxfp4_verify_gemm runs the same kernel (m <= 32 with k % 512 == 0 and 16-byte
 * aligned row-layout scales; m > 32) the result is bit-identical to it.
 *
 * tiled_codes   mxfp4_tiled_bytes(n, k) bytes, 16-byte aligned.
 * tiled_scales  mxfp4_tiled_scale_bytes(n, k) bytes, 16-byte aligned.
 * n, k          1 <= n <= 2^31 - 16; 128 <= k <= 2^23, k % 128 == 0.
 * x             [m, k] bf16 bit patterns, 16-byte aligned.
 * m             1 <= m <= 65536, and ceil(n/1024) * 8 * ceil(m/80) <= 2^23 - 1 (the
 *               launch grid: n up to about 1M rows at m = 65536).
 * y             [m, n] fp32, 4-byte aligned. Fully overwritten.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status mxfp4_verify_gemm_tiled(const uint8_t* tiled_codes, const uint8_t* tiled_scales, int64_t n, int64_t k,
                                   const uint16_t* x, int64_t m, float* y, void* stream);

/*
 * mxfp4_verify_gemm_grouped_tiled — mxfp4_verify_gemm_grouped on tiled weights: each
 * descriptor's codes and scales are the mxfp4_tile_codes / mxfp4_tile_scales outputs of
 * that product's weights. Per product the rules, kernels and result are those of
 * mxfp4_verify_gemm_tiled; up to 8 products share one launch of the skinny kernel, and
 * with the dense kernel each product has its own launch [M11 §4, §10].
 *
 * problems  HOST array of `count` descriptors, read during the call only.
 * count     1 <= count <= 65536.
 * k, m      as mxfp4_verify_gemm_tiled, for every product.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status mxfp4_verify_gemm_grouped_tiled(const mxs_gemm_problem* problems, int32_t count, int64_t k, int64_t m,
                                           void* stream);

/*
 * spec_accept_workspace_bytes — device workspace spec_accept needs for
 * (b, kd, v). Returns 0 when the sizes are out of range.
 */
size_t spec_accept_workspace_bytes(int32_t b, int32_t kd, int32_t v);

/*
 * spec_accept — one verification cycle for b independent sequences [M11 §4].
 *
 * For each sequence, with p_i = softmax(target row i) and q_i = softmax(draft
 * row i) (temperature 1, no filtering; -inf logits are allowed and mean
 * probability 0):
 *   for i = 0 .. kd-1: a_i = min(1, p_i(x_i) / q_i(x_i)), or 0 when
 *     q_i(x_i) = 0 (MXS_FLAG_Q_ZERO) or x_i is outside [0, v)
 *     (MXS_FLAG_TOKEN_RANGE); accept x_i iff u_i < a_i; stop at the first
 *     rejection n = i.
 *   If all kd are accepted, n = kd and the final weights are w = p_kd
 *   (bonus token); otherwise w = (p_n - q_n)+ (residual; if it has zero
 *   mass, MXS_FLAG_RESIDUAL_ZERO and w = p_n).
 *   Final token t* = min{ t : u_kd · Z < C_t } with C the inclusive prefix
 *   sums of w and Z = sum w; if rounding leaves no such t, the last t with
 *   w_t > 0. Probabilities and prefix sums are computed in fp64.
 *   A sequence with a NaN/+inf logit, or a row whose logits are all -inf, is
 *   refused: MXS_FLAG_NONFINITE, n = 0 and every output token -1.
 *
 * target_logits   [b, kd+1, v] fp32; row kd is the next-position (bonus) law.
 * draft_logits    [b, kd, v] fp32 (may be NULL when kd == 0).
 * draft_tokens    [b, kd] int32, drawn from the draft laws by the caller
 *                 (may be NULL when kd == 0).
 * uniforms        [b, kd+1] fp32 in [0, 1): u_i for acceptance test i and
 *                 u_kd for the single final draw.
 * b, kd, v        1 <= b <= 65535, 0 <= kd <= 32, 2 <= v <= 2^26.
 * out_tokens      [b, kd+1] int32: the n accepted drafts, then t*, then -1.
 * out_num_accepted[b] int32: n.
 * workspace       device scratch of at least spec_accept_workspace_bytes(b, kd, v)
 *                 bytes, 16-byte aligned; its contents on entry do not matter.
 * Logit pointers must be 4-byte aligned (16-byte alignment with v % 4 == 0
 * enables vector loads).
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN, MXS_ERR_WORKSPACE.
 */
mxs_status spec_accept(const float* target_logits, const float* draft_logits,
                       const int32_t* draft_tokens, const float* uniforms, int32_t b,
                       int32_t kd, int32_t v, int32_t* out_tokens,
                       int32_t* out_num_accepted, void* workspace, size_t workspace_bytes,
                       int32_t* dev_flags, void* stream);

/*
 * spec_accept_noalloc — spec_accept with a built-in workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It calls no hipMalloc / hipFree and allocates nothing: the
 * workspace is a static device array of MXS_NOALLOC_SCRATCH_BYTES in the library, one
 * copy per GPU, held until the process ends; its address is looked up once per device on
 * the first call made with that device current. Same rule, arguments (minus the
 * workspace), outputs and errors as spec_accept, and bit-identical results.
 *
 * The array is shared by every call on one GPU and keeps the last call's contents
 * (which no call depends on: every word a call reads it first writes). Calls that
 * overlap on one GPU (two host threads, or two streams without ordering between them)
 * race on it and give undefined results: serialize them, or use spec_accept with a
 * workspace each.
 *
 * Returns MXS_ERR_WORKSPACE when spec_accept_workspace_bytes(b, kd, v) exceeds
 * MXS_NOALLOC_SCRATCH_BYTES (e.g. b = 64, kd = 4, v = 128256 needs about 0.43 MB; the
 * limit admits b up to ~590 at that kd and v), before any HIP call; MXS_ERR_DEVICE when
 * the array's device address cannot be obtained; otherwise as spec_accept.
 */
#define MXS_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
mxs_status spec_accept_noalloc(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms, int32_t b,
                               int32_t kd, int32_t v, int32_t* out_tokens,
                               int32_t* out_num_accepted, int32_t* dev_flags, void* stream);

/*
 * spec_accept_sampled_workspace_bytes — device workspace spec_accept_sampled
 * needs for (b, kd, v): spec_accept's plus ~80 KB per logit row for the top-k /
 * top-p selection. Returns 0 when the sizes are out of range.
 */
size_t spec_accept_sampled_workspace_bytes(int32_t b, int32_t kd, int32_t v);

/*
 * spec_accept_sampled — spec_accept on transformed laws [M11 §4: the laws p_i
 * and q_i are the ones tokens are actually sampled from, so temperature,
 * top-k, top-p and a grammar mask apply to both, or the cycle is not exact].
 *
 * Every target and draft row is transformed alike, in this order:
 *   mask       token t of position i is removed when bit t % 32 of word t / 32
 *              of mask row i is 0 (target row i and draft row i share mask row
 *              i; the bonus row kd uses mask row kd);
 *   temperature the logits are divided by temperature;
 *   top-k      a token stays iff fewer than top_k remaining tokens have a
 *              strictly larger logit (ties at the k-th value all stay);
 *   top-p      with e_t = exp((z_t - max z) / temperature) over the tokens
 *              top-k left and S their sum, a token stays iff the e-mass of
 *              those with a strictly larger logit is below top_p * S (the
 *              smallest most-probable set reaching top_p, boundary ties kept).
 * The law of a row is e_t / sum over the remaining tokens; then the cycle of
 * spec_accept runs unchanged on these laws (a draft token the transformed
 * draft law gives probability 0 raises MXS_FLAG_Q_ZERO; a row with no
 * remaining finite logit refuses its sequence with MXS_FLAG_NONFINITE). The
 * draft tokens must come from the transformed draft laws.
 *
 * temperature     > 0 and finite (1: none).
 * top_k           >= 0 (0: none; >= v: none).
 * top_p           in (0, 1] (1: none). The top-p boundary sums are fp64 with
 *                 an unspecified summation order, so a token whose strictly-
 *                 larger mass is within ~1e-15 * S of top_p * S can fall on
 *                 either side. With top-p alone, the kept law's normaliser is
 *                 summed in such an order too: its last bits can differ between
 *                 calls, which moves a decision only where u * q(x) lies within
 *                 ~1e-15 of p(x).
 * mask            [b, kd+1, ceil(v/32)] uint32 device bits, 4-byte aligned; or
 *                 NULL (no mask).
 * workspace       at least spec_accept_sampled_workspace_bytes(b, kd, v) bytes;
 *                 other arguments as spec_accept.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_VALUE (temperature, top_k,
 * top_p), MXS_ERR_ALIGN, MXS_ERR_WORKSPACE.
 */
mxs_status spec_accept_sampled(const float* target_logits, const float* draft_logits,
                               const int32_t* draft_tokens, const float* uniforms, int32_t b,
                               int32_t kd, int32_t v, float temperature, int32_t top_k,
                               float top_p, const uint32_t* mask, int32_t* out_tokens,
                               int32_t* out_num_accepted, void* workspace,
                               size_t workspace_bytes, int32_t* dev_flags, void* stream);

/*
 * spec_sampling_thresholds_workspace_bytes — device workspace spec_sampling_thresholds
 * needs for `rows` rows (~80 KB per row). Returns 0 when the sizes are out of range.
 */
size_t spec_sampling_thresholds_workspace_bytes(int32_t rows, int32_t v);

/*
 * spec_sampling_thresholds — the top-k / top-p selection of spec_accept_sampled on its own,
 * for `rows` independent logit rows [M11 §4: the draft's tokens must be drawn from the same
 * transformed law the acceptance test uses, so a draft sampler needs these sets too].
 *
 * A row's kept set is {t : mask bit t set, logit finite, key(z_t) >= out_thresholds[row]},
 * where key is the order-preserving map of an fp32 logit to uint32 (bits | 0x80000000 for
 * z >= 0, ~bits for z < 0; -0 maps as +0). It is the set spec_accept_sampled's rule gives:
 * mask, then top-k (ties at the k-th value all stay), then top-p on the law top-k left, with
 * masses exp((z - max z) / temperature). A threshold of 0 keeps every allowed finite token
 * (also returned when top-k and top-p are both off, or the row has no allowed finite logit).
 *
 * logits          [rows, v] fp32 device, row-major, 4-byte aligned.
 * temperature     > 0 and finite; top_k >= 0 (0 or >= v: off); top_p in (0, 1] (1: off).
 *                 The top-p boundary sums are fp64; when top-p is on without top-k, the mass
 *                 above the boundary's bucket is summed in an unspecified order, so a token
 *                 whose strictly-larger mass is within ~1e-15 * S of top_p * S can fall on
 *                 either side.
 * mask            [rows, ceil(v/32)] uint32 device bits (1 = allowed), or NULL.
 * out_thresholds  [rows] uint32 device, written.
 * workspace       at least spec_sampling_thresholds_workspace_bytes(rows, v) device bytes,
 *                 16-byte aligned, no initial contents required.
 * stream          hipStream_t or NULL. Asynchronous; host errors come back before any launch:
 *                 MXS_ERR_NULL, MXS_ERR_SHAPE (rows outside [1, 2^22], v outside [2, 2^26]),
 *                 MXS_ERR_VALUE (temperature, top_k, top_p), MXS_ERR_ALIGN,
 *                 MXS_ERR_WORKSPACE, MXS_ERR_DEVICE.
 */
mxs_status spec_sampling_thresholds(const float* logits, int32_t rows, int32_t v, float temperature,
                                    int32_t top_k, float top_p, const uint32_t* mask,
                                    uint32_t* out_thresholds, void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * spec_accept_tree_workspace_bytes — device workspace spec_accept_tree needs for this tree
 * (parent: HOST array of `nodes` entries, as spec_accept_tree takes it), b sequences and
 * vocabulary v. Returns 0 when the sizes or the tree are out of range.
 */
size_t spec_accept_tree_workspace_bytes(const int32_t* parent, int32_t nodes, int32_t b, int32_t v);

/*
 * spec_accept_tree — one verification cycle over a tree of draft tokens for each of b
 * sequences [M11 §4, applied at every node; §8: a tree verified by typical acceptance loses
 * §4's guarantee, so this rule keeps §4's]. The tree is shared by the sequences; node i has
 * parent parent[i] (-1 = the root, else a node before i) and draft token draft_tokens[s][i],
 * drawn by the caller from the draft law of its parent's history, siblings independently.
 *
 * Laws: row 0 of target_logits / draft_logits is the root's history, row i + 1 the history
 * ending in node i (softmax of the fp32 logits, temperature 1; -inf allowed). At the current
 * node (the root first), with p = its target law and q = its draft law, the children are tried
 * in index order: child j is accepted iff u_j < min(1, L_j(x_j) / q(x_j)), with L_1 = p and,
 * after each rejection, L_{j+1} = norm((L_j - q)+) (0 when q(x_j) = 0: MXS_FLAG_Q_ZERO; 0 when
 * x_j is outside [0, v): MXS_FLAG_TOKEN_RANGE); an accepted child becomes the current node.
 * When every child is rejected, or the node is a leaf, the final token is drawn from the
 * current law by inverse CDF on u[N]: t* = min{t : u * Z < C_t} over the law's prefix sums
 * (the last positive token if rounding leaves none). A residual with no mass left (rounding)
 * raises MXS_FLAG_RESIDUAL_ZERO and the draw uses the law before that try. A chain (one
 * child per node) is spec_accept's rule. A sequence with a NaN / +inf logit or an all -inf
 * row anywhere in its tree is refused: MXS_FLAG_NONFINITE, n = 0, all outputs -1.
 * Probabilities and prefix sums are fp64.
 *
 * parent          HOST [nodes] int32, read during the call; nodes <= 64, at most 16 children
 *                 per node (else MXS_ERR_VALUE). D below = the tree's depth (nodes on its
 *                 longest root-to-leaf path).
 * target_logits   [b, nodes+1, v] fp32.  draft_logits  [b, nodes+1, v] fp32 (leaf rows are
 *                 examined for validity only).
 * draft_tokens    [b, nodes] int32 (may be NULL when nodes == 0).
 * uniforms        [b, nodes+1] fp32 in [0, 1): u[i] for node i's test, u[nodes] for the draw.
 * b, v            1 <= b <= 65535, 2 <= v <= 2^26.
 * out_tokens      [b, D+1] int32: the accepted path's tokens, then the final token, then -1.
 * out_nodes       [b, D] int32: the accepted path's node indices, then -1 (may be NULL when
 *                 nodes == 0).
 * out_num_accepted[b] int32: accepted drafts n (the path length).
 * workspace       spec_accept_tree_workspace_bytes(parent, nodes, b, v) bytes, 16-byte
 *                 aligned; its contents on entry do not matter.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_VALUE (the tree), MXS_ERR_ALIGN,
 * MXS_ERR_WORKSPACE.
 */
mxs_status spec_accept_tree(const float* target_logits, const float* draft_logits, const int32_t* parent,
                            int32_t nodes, const int32_t* draft_tokens, const float* uniforms, int32_t b,
                            int32_t v, int32_t* out_tokens, int32_t* out_nodes, int32_t* out_num_accepted,
                            void* workspace, size_t workspace_bytes, int32_t* dev_flags, void* stream);

/*
 * mxfp4_kv_append — write t tokens' key (or value) vectors into an MX-FP4 KV cache [NEWS,
 * "Microscaling FP4 (MX-FP4) Integration": the KV cache tensors are held in 4-bit MX
 * values with an E8M0 scale per 32 elements, the FP4 KV cache pool of its pipeline figure].
 * The cache is [capacity, heads, d] coded as the weights are (mxfp4_quantize's rule and
 * layout with row = slot * heads + head): 32-element blocks run along d inside one token's
 * one head, so appending a token codes only its own blocks and never touches other entries.
 * Token i's vectors go to entry slots[i].
 *
 * kv        [t, heads, d] bf16 bit patterns, 16-byte aligned.
 * t, heads  >= 1; d >= 32, d % 32 == 0; capacity >= 1 (entries of the cache).
 * slots     [t] int32 device array: the cache entry of each token. A slot outside
 *           [0, capacity) writes nothing and raises MXS_FLAG_TOKEN_RANGE.
 * codes     [capacity, heads, d/2] bytes (low nibble = even element), 4-byte aligned.
 * scales    [capacity, heads, d/32] E8M0 bytes.
 * A block holding a NaN or infinity gets scale 0xFF and codes 0 and raises
 * MXS_FLAG_NONFINITE. Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status mxfp4_kv_append(const uint16_t* kv, int64_t t, int64_t heads, int64_t d, const int32_t* slots,
                           int64_t capacity, uint8_t* codes, uint8_t* scales, int32_t* dev_flags, void* stream);

/*
 * mxfp4_kv_attention_workspace_bytes — device workspace mxfp4_kv_attention needs (the
 * per-workgroup partial results). Returns 0 when the sizes are out of range.
 */
size_t mxfp4_kv_attention_workspace_bytes(int32_t b, int32_t t, int32_t hq, int32_t hkv, int64_t max_len);

/*
 * mxfp4_kv_attention — the verification pass's attention over an MX-FP4 KV cache [M11 §4:
 * the target scores every draft position in one pass and stays causal, a row sees only its
 * own history; NEWS, "Microscaling FP4 (MX-FP4) Integration": the KV cache held in MX-FP4].
 * For each sequence s, query position i < t and query head h (KV head h / G, G = hq / hkv):
 *   out[s, i, h] = sum_l softmax_l(scale * q[s, i, h] . K^[s, l, h/G]) V^[s, l, h/G]
 * over the visible cache entries l: every l < ctx_len[s] (the committed prefix) and the new
 * entry ctx_len[s] + r when bit r of masks[i] is set (a lower-triangular mask for a chain of
 * drafts; a position's ancestors and itself for a tree). The t new entries must have been
 * written (mxfp4_kv_append) at ctx_len[s] .. ctx_len[s] + t - 1 before the call. K^ and V^ are
 * the entries decoded exactly (E2M1 x 2^(s-127)); scores, softmax and sums are fp32 (the
 * probabilities enter the value product as a bf16 pair, error ~2^-17 relative). Every
 * position must see at least one entry.
 *
 * q           [b, t, hq, d] bf16, 16-byte aligned.
 * k_codes, v_codes    [b, capacity, hkv, d/2] (mxfp4_kv_append layout per sequence), 16-byte aligned.
 * k_scales, v_scales  [b, capacity, hkv, d/32].
 * ctx_len     [b] int32 device: committed entries of each sequence. A sequence with ctx_len < 0
 *             or ctx_len + t > max_len is refused: its outputs are NaN, MXS_FLAG_TOKEN_RANGE.
 * b, t        1 <= b <= 65535; 1 <= t <= 64 with t * hq / hkv <= 64 (query rows per KV head).
 * hq, hkv     hq a multiple of hkv. d = 128.
 * capacity    entries per sequence in the caches; max_len (host bound on ctx_len + t, sizes the
 *             launch): t <= max_len <= capacity.
 * masks       HOST [t] uint64, read during the call: bit r of masks[i] lets position i see new
 *             entry r; bits >= t are refused (MXS_ERR_VALUE).
 * scale       > 0 and finite (1/sqrt(d) for plain attention).
 * out         [b, t, hq, d] fp32, 4-byte aligned.
 * workspace   mxfp4_kv_attention_workspace_bytes(b, t, hq, hkv, max_len) bytes, 16-byte aligned.
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_VALUE, MXS_ERR_ALIGN, MXS_ERR_WORKSPACE.
 */
mxs_status mxfp4_kv_attention(const uint16_t* q, const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v_codes,
                              const uint8_t* v_scales, const int32_t* ctx_len, int32_t b, int32_t t, int32_t hq,
                              int32_t hkv, int32_t d, int64_t capacity, int64_t max_len, const uint64_t* masks,
                              float scale, float* out, void* workspace, size_t workspace_bytes, int32_t* dev_flags,
                              void* stream);

/*
 * mxs_stream_read — read `bytes` of device memory once and discard them: the measured
 * ceiling of the weight stream. A verification step that streams all weights is bounded by
 * Q <= BW / W [M11 §1]; this plain read-only kernel measures the BW one kernel draws from
 * HBM on the current device, against which the verify GEMM's achieved bandwidth is read
 * (timing is the caller's: events around the call on `stream`).
 *
 * buf    device memory, 16-byte aligned, read only.
 * bytes  >= 16, a multiple of 16.
 * sink   one device uint32, 4-byte aligned: OR-ed with 1 only if the XOR of all words read
 *        equals 0x9E3779B9 (it keeps the loads live; its value carries no meaning).
 * Returns MXS_ERR_NULL, MXS_ERR_SHAPE, MXS_ERR_ALIGN.
 */
mxs_status mxs_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4SPEC_H */
