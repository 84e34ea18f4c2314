/*
 * fp8bs.h -- C ABI of the block-scaled FP8 linear library for AMD MI355X
 * (gfx950).  Every entry point takes plain device pointers, sizes and a HIP
 * stream, enqueues its kernels on that stream and returns without waiting.
 *
 * Conventions shared by all entry points
 *   - Tensors are dense, row-major and contiguous; sizes are element counts.
 *   - "e4m3" is the OCP float8 E4M3 "fn" byte format (torch.float8_e4m3fn):
 *     bias 7, no infinities, 0x7F/0xFF are NaN, largest magnitude 448.
 *   - "bf16" tensors are passed as their 16-bit patterns (torch.bfloat16).
 *   - Block size is 128 everywhere: activations carry one float32 scale per
 *     1 x 128 block along K, weights one per 128 x 128 block.  A scale is the
 *     dequantisation multiplier: real value = decode(code) * scale.
 *   - The caller owns all memory.  The library never allocates or frees
 *     device memory, creates no streams or events, and keeps no state
 *     between calls beyond a per-device cache of the compute-unit count.  It
 *     is safe to call from several host threads.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream) on the
 *     current HIP device; all pointers must be device (or managed) memory of
 *     that device.
 *   - Arguments are validated on the host before any HIP call.  A non-zero
 *     status means nothing was enqueued (except FP8BS_ERR_HIP, returned when
 *     a kernel launch itself fails).  Faults inside kernels are reported
 *     asynchronously by HIP, as for any kernel.
 *   - Inputs holding NaN are outside the contract (NaN propagates; payloads
 *     are not specified).
 *
 * The operations follow the DeepSeek-V3 inference pages: "DeepSeek-V3
 * Administrator & Developer Guide" sections 8.5.1 (act_quant_kernel), 8.5.2
 * (weight_dequant_kernel), 8.5.3 (fp8_gemm_kernel), 6.3 (the FP8 path and
 * the weight scale shape), 6.4 (MoE expert loop); "DeepSeek-V3 User Guide"
 * section 7 FAQ (scale_fmt ue8m0) and section 6 (K must be a multiple of 128).
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define FP8BS_OK          0
#define FP8BS_ERR_NULL    1  /* a required pointer is NULL */
#define FP8BS_ERR_SHAPE   2  /* negative size, K not a multiple of 128, size limit */
#define FP8BS_ERR_ALIGN   3  /* a pointer is not 16-byte aligned */
#define FP8BS_ERR_ENUM    4  /* unknown scale_fmt / out_dtype */
#define FP8BS_ERR_HIP     5  /* a HIP launch failed */
#define FP8BS_ERR_ALIAS   6  /* an output overlaps an input */

/* Scale formats for activation quantisation. */
#define FP8BS_SCALE_FP32  0  /* s = max(amax, 1e-4) / 448 as float32 */
#define FP8BS_SCALE_UE8M0 1  /* s rounded up to the next power of two */

/* Output element types of the GEMMs. */
#define FP8BS_OUT_BF16    0
#define FP8BS_OUT_F32     1

/* Human-readable name of a status code (static string, never NULL). */
const char* fp8bs_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int fp8bs_version(void);

/*
 * act_quant -- per-1x128-block activation quantisation.
 * Admin guide 8.5.1; ue8m0 per the User guide FAQ.
 *
 * For every row m and block j (columns 128j .. 128j+127):
 *   amax = max |x|,  s = RN32(max(amax, 1e-4f) / 448)   (IEEE division),
 *   ue8m0: s = smallest power of two >= s,
 *   q = e4m3(RN32(x / s))  (correctly rounded division, then round to nearest
 *   even onto the e4m3 grid, saturating at +-448).
 *
 *   x_bf16  in   bf16 [M, K]
 *   q_e4m3  out  e4m3 [M, K]          (must not overlap x)
 *   s       out  float32 [M, K/128]
 *   M >= 0 (0 = no-op), K >= 0 with K % 128 == 0 (else FP8BS_ERR_SHAPE).
 *   One launch covers at most 2^32 - 1 threads, 32 blocks per 256 threads:
 *   M * (K / 128) <= 536870880 (M * K up to about 2^36); larger shapes
 *   return FP8BS_ERR_SHAPE.
 *   All three pointers 16-byte aligned except `s` (4-byte).
 *   x must be finite: a block holding +-Inf or NaN gets an unspecified scale
 *   and unspecified codes (the rule above is not defined for it).
 */
int fp8bs_act_quant(const void* x_bf16, void* q_e4m3, float* s, int64_t M, int64_t K,
                    int scale_fmt, void* stream);

/*
 * e4m3_encode -- the float32 -> e4m3 step of act_quant and weight_quant on
 * its own (the cast to float8_e4m3fn of Admin guide 8.5.1): q[i] is x[i]
 * rounded to the nearest e4m3 value, ties to even mantissa, magnitudes
 * above 448 saturating to +-448 (464, the midpoint to the next binade,
 * rounds to 448); the sign of a zero result follows x.  Exposed so that
 * the hardware conversion can be checked against a reference over every
 * float32 input.
 *
 *   x       in   float32 [n] (16-byte aligned)
 *   q_e4m3  out  e4m3 [n] (4-byte aligned, must not overlap x)
 *   n >= 0; n <= 2^34 - 1024 (one launch), else FP8BS_ERR_SHAPE.
 *   NaN inputs are outside the contract.
 */
int fp8bs_e4m3_encode(const float* x, void* q_e4m3, int64_t n, void* stream);

/*
 * weight_quant -- 128x128-block weight quantisation with the same rule as
 * act_quant (fp32 scale format).  The pages ship weights already quantised
 * (Admin guide 6.3: one float32 scale per 128 x 128 block, shape
 * ceil(N/128) x ceil(K/128)); this entry point produces that form from a
 * bf16 weight.  A partial edge block uses the amax of its own elements.
 *
 *   w_bf16  in   bf16 [N, K]
 *   q_e4m3  out  e4m3 [N, K]
 *   s       out  float32 [ceil(N/128), ceil(K/128)]
 *   N, K >= 0, any values.
 */
int fp8bs_weight_quant(const void* w_bf16, void* q_e4m3, float* s, int64_t N, int64_t K,
                       void* stream);

/*
 * weight_dequant -- Admin guide 8.5.2:
 *   y[n, k] = bf16_RNE( RN32( decode(w[n, k]) * s[n/128, k/128] ) ).
 *
 *   w_e4m3  in   e4m3 [N, K]
 *   s       in   float32 [ceil(N/128), ceil(K/128)]
 *   y_bf16  out  bf16 [N, K]
 *   N, K >= 0, ragged edge blocks allowed.  One launch covers at most 2^32 - 1
 *   threads: N*K + 255 < 2^32 when K % 16 != 0, and ceil(N/4) * ceil(K/1024)
 *   < 2^24 workgroups when K % 16 == 0 (N*K up to about 2^36); larger shapes
 *   return FP8BS_ERR_SHAPE.
 */
int fp8bs_weight_dequant(const void* w_e4m3, const float* s, void* y_bf16, int64_t N, int64_t K,
                         void* stream);

/*
 * gemm -- block-scaled FP8 GEMM, Admin guide 8.5.3 (nn.Linear layout):
 *   C[m, n] = sum_kb ( sum_{k in block kb} a[m, k] * b[n, k] )
 *                    * a_s[m, kb] * b_s[n / 128, kb]
 * with float32 accumulation; each 128-wide K block's partial product is
 * scaled once and added to the accumulator.
 *
 *   a    in   e4m3 [M, K]              (activations, from fp8bs_act_quant)
 *   a_s  in   float32 [M, K/128]
 *   b    in   e4m3 [N, K]              (weight, out x in)
 *   b_s  in   float32 [ceil(N/128), K/128]
 *   c    out  [M, N], bf16 (RNE) or float32 per out_dtype
 *   M >= 0 (0 = no-op), N >= 0, K >= 128 with K % 128 == 0;
 *   (M + 256) * K < 2^32 and (N + 256) * K < 2^32 (32-bit operand offsets).
 *   a, b, c 16-byte aligned; a_s, b_s 4-byte aligned.
 *
 * Accuracy.  Let S[m, n] = sum_kb sum_{k in kb} |a[m,k] * b[n,k]| * a_s[m,kb]
 * * b_s[n/128,kb] (the sum of the absolute scaled products) and ref the exact
 * sum.  M <= 64 runs on bf16 matrix instructions over exactly decoded codes;
 * its float32 result carries only the float32 rounding of the accumulation,
 * within about (K/128 + 16) * 2^-24 * S of ref.  M > 64 runs on the FP8 matrix instruction
 * (K = 128 per instruction), whose internal sum of a block's 128 products is
 * not exact in float32: measured on gfx950 its error per block reaches about
 * 1.4e-5 of the block's sum of |products| on normally distributed codes and
 * 2^-13.6 of it with 1% of activations scaled by 50.  The float32 result
 * then satisfies |err| <= 1e-2 * |ref| + 1e-3 + 2^-11 * S.  Where products
 * cancel (|ref| much smaller than S) the first two terms alone can be missed:
 * with 1% x50 activation outliers about 1 output in 10^4 did (211 of 1.57 M
 * at 1024 x 1536 x 7168); on N(0,1) activations none were seen.  A bf16
 * output adds its own rounding, 2^-9 * |ref|.
 */
int fp8bs_gemm(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
               int64_t M, int64_t N, int64_t K, int out_dtype, void* stream);

/*
 * moe_gemm -- grouped block-scaled FP8 GEMM over E experts in one launch,
 * the per-expert products of the MoE loop (Admin guide 6.4), each computed as
 * in fp8bs_gemm.  Rows [offsets[e], offsets[e+1]) of `a` (grouped by expert)
 * are multiplied by expert e's weight:
 *   C[r, n] = sum_kb (sum_k a[r, k] * b[e, n, k]) * a_s[r, kb] * b_s[e, n/128, kb].
 *
 *   a        in   e4m3 [R, K]
 *   a_s      in   float32 [R, K/128]
 *   b        in   e4m3 [E, N, K]
 *   b_s      in   float32 [E, ceil(N/128), K/128]
 *   offsets  in   DEVICE int32 [E+1]: offsets[0] = 0, non-decreasing,
 *                 offsets[E] = R (precondition, not checked on the host so
 *                 that no device->host copy is needed; the kernel clamps
 *                 every range to [0, R] so a violation cannot write outside c)
 *   c        out  [R, N] bf16 or float32; rows not covered by any expert are
 *                 left untouched
 *   R, E >= 0 (either 0 = no-op), N >= 0, K >= 128 with K % 128 == 0;
 *   (R + 256) * K < 2^32 and (N + 256) * K < 2^32.
 * One launch on `stream`: experts with more than 64 rows run on the 256 x 256
 * tiles of fp8bs_gemm, the others on 64 x 256 tiles that stream the weight
 * once, the two kinds of tiles sharing the grid.  The grid is sized on the
 * host from R and E alone (each workgroup finds its tile from the device
 * offsets, so no device-to-host copy is needed); experts with no rows cost
 * nothing.  Accuracy as fp8bs_gemm for M > 64 (both tile kinds use the FP8
 * matrix instruction).
 */
int fp8bs_moe_gemm(const void* a, const float* a_s, const void* b, const float* b_s,
                   const int32_t* offsets, void* c, int64_t R, int64_t E, int64_t N, int64_t K,
                   int out_dtype, void* stream);

/*
 * gemm_ue8m0 -- fp8bs_gemm for operands whose scales are all powers of two
 * (act_quant with FP8BS_SCALE_UE8M0 and fp8bs_weight_quant_ue8m0), the ue8m0
 * variant of the pages (User guide FAQ; Admin guide 8.5.1).  The result is the
 * same sum; the kernel passes each scale's exponent to the MFMA
 * (v_mfma_scale_f32_16x16x128_f8f6f4, E8M0 scales) instead of folding the
 * scales in with VALU instructions.  Arguments as fp8bs_gemm.
 * PRECONDITION (not checked on the host: the scales live on the device):
 * every a_s and b_s value is 2^k with -126 <= k <= 127; only the exponent
 * field is read, so other values give wrong results, not faults.
 * Accuracy as fp8bs_gemm: M > 64 uses the same FP8 matrix instruction
 * (scaled form) and has the same 2^-11 * S term beyond
 * 1e-2 * |ref| + 1e-3; M <= 64 runs fp8bs_gemm's bf16 decode kernel.
 */
int fp8bs_gemm_ue8m0(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
                     int64_t M, int64_t N, int64_t K, int out_dtype, void* stream);

/*
 * weight_quant_ue8m0 -- fp8bs_weight_quant with each block scale rounded up
 * to a power of two (act_quant's ue8m0 rule on 128 x 128 blocks); a harness
 * option: the pages round only activation scales.  Arguments as
 * fp8bs_weight_quant.
 */
int fp8bs_weight_quant_ue8m0(const void* w_bf16, void* q_e4m3, float* s, int64_t N, int64_t K,
                             void* stream);

/*
 * w8a16_gemm -- the BF16 path of the linear (Admin guide 6.3, gemm_impl
 * "bf16"): C = x . weight_dequant(w, w_s)^T with the weight dequantised as
 * fp8bs_weight_dequant does (bf16(RN32(decode(q) * s))) but never stored:
 * the kernel dequantises in registers and multiplies with bf16 MFMA,
 * accumulating in float32.
 *
 *   x_bf16   in   bf16 [M, K]
 *   w_e4m3   in   e4m3 [N, K] (nn.Linear out x in)
 *   w_s      in   float32 [ceil(N/128), K/128]
 *   c        out  [M, N] bf16 or float32 (out_dtype)
 *   M, N >= 0 (either 0 = no-op), K >= 128 with K % 128 == 0;
 *   (M + 256) * 2K < 2^32 and (N + 256) * K < 2^32.
 * x, w and c 16-byte aligned, w_s 4-byte aligned; c must not overlap an input.
 */
int fp8bs_w8a16_gemm(const void* x_bf16, const void* w_e4m3, const float* w_s, void* c, int64_t M,
                     int64_t N, int64_t K, int out_dtype, void* stream);

/*
 * MoE dispatch and combine -- the steps around fp8bs_moe_gemm in the expert
 * loop of the Admin guide (6.4; the annotated forward pass in 8.4): hit
 * counts of the routed expert ids, each expert's (token, slot) pairs in token
 * order, the expert run on those tokens' rows, and the expert outputs scaled
 * by the routing weight of their (token, slot) and summed per token.
 *
 * moe_route_workspace_size -- bytes of device workspace fp8bs_moe_route
 * needs for T tokens, topk slots and E experts (4 * ceil(T*topk/512) * E;
 * 0 when T*topk == 0).  Returns -1 for sizes fp8bs_moe_route rejects.
 */
int64_t fp8bs_moe_route_workspace_size(int64_t T, int64_t topk, int64_t E);

/*
 * moe_route -- stable counting sort of the routed expert ids by expert.
 *
 *   indices    in   DEVICE int32 [T, topk]: the expert of each (token, slot)
 *   offsets    out  DEVICE int32 [E+1]: expert e owns rows [offsets[e],
 *                   offsets[e+1]); offsets[E] = R, the number of pairs whose
 *                   id lies in [0, E)
 *   row_token  out  DEVICE int32 [T*topk]: the token of each row r < R, rows
 *                   of one expert in (token, slot) order (the order the
 *                   pages' per-expert index lookup yields); entries >= R
 *                   untouched
 *   row_of     out  DEVICE int32 [T, topk]: the row of each (token, slot), or
 *                   -1 when its id is outside [0, E) (such a pair is not
 *                   routed and takes no row)
 *   workspace  tmp  DEVICE, >= fp8bs_moe_route_workspace_size bytes, 4-byte
 *                   aligned; its contents are scratch (nothing needs clearing)
 *   T >= 0, 1 <= topk, 1 <= E, T*topk < 2^31.  Two kernel launches (four
 *   when ceil(T*topk/512) * E > 65536 or E > 2048); the result does not
 *   depend on timing (its only atomics are on-chip adds and ORs, whose order
 *   does not change it).
 */
int fp8bs_moe_route(const int32_t* indices, int64_t T, int64_t topk, int64_t E, int32_t* offsets,
                    int32_t* row_token, int32_t* row_of, void* workspace,
                    int64_t workspace_bytes, void* stream);

/*
 * moe_route_noalloc -- fp8bs_moe_route with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  The count table
 * lives in a 1 MiB device array inside the library (one per GPU, held until
 * the process ends); the call allocates nothing.  Limit:
 * fp8bs_moe_route_workspace_size(T, topk, E) <= 1048576 bytes, i.e.
 * ceil(T*topk/512) * E <= 262144 (e.g. 4096 tokens x top-8 with up to 4096
 * experts), else FP8BS_ERR_SHAPE.  Every call on one GPU uses the same
 * table: calls that overlap in time on one GPU (on different streams, or
 * from several host threads without ordering) race and give wrong results.
 * Other arguments, results and errors as fp8bs_moe_route.
 */
int fp8bs_moe_route_noalloc(const int32_t* indices, int64_t T, int64_t topk, int64_t E,
                            int32_t* offsets, int32_t* row_token, int32_t* row_of, void* stream);

/*
 * moe_quant_scatter -- the expert inputs: act_quant (as fp8bs_act_quant) of
 * every token row of x, written to each row its (token, slot) pairs were
 * routed to.  Quantisation is row local, so row r holds act_quant of
 * x[row_token[r]].
 *
 *   x        in   bf16 [T, K], K % 128 == 0
 *   row_of   in   DEVICE int32 [T, topk] (from fp8bs_moe_route); entries
 *                 outside [0, R) are skipped
 *   q        out  e4m3 [R, K]; s out float32 [R, K/128]; rows no pair maps
 *                 to are left untouched
 *   scale_fmt     FP8BS_SCALE_FP32 or FP8BS_SCALE_UE8M0
 * Alignment as fp8bs_act_quant; row_of 4-byte aligned.  If row_of maps two
 * pairs to one row, that row receives one of the two (identical for a
 * token's own duplicates).  Launch limit as fp8bs_act_quant with M = T:
 * T * (K / 128) <= 536870880, else FP8BS_ERR_SHAPE.
 */
int fp8bs_moe_quant_scatter(const void* x_bf16, const int32_t* row_of, void* q_e4m3, float* s,
                            int64_t T, int64_t topk, int64_t R, int64_t K, int scale_fmt,
                            void* stream);

/*
 * moe_combine -- y[t, n] = sum_k w[t, k] * out[row_of[t, k], n], summed in
 * float32 in slot order (the pages accumulate y in place, expert by expert;
 * here a token's at most topk terms are summed once and rounded once).
 *
 *   out      in   bf16 [R, N]: expert outputs in routed-row order
 *   w        in   float32 [T, topk]: routing weights
 *   row_of   in   DEVICE int32 [T, topk]; pairs outside [0, R) contribute 0
 *   y        out  [T, N] bf16 or float32 (out_dtype); overwritten, not
 *                 accumulated into
 * out and y 16-byte aligned, w and row_of 4-byte aligned; N >= 0, T >= 0,
 * topk >= 1, R >= 0.
 */
int fp8bs_moe_combine(const void* out_bf16, const float* w, const int32_t* row_of, void* y,
                      int64_t T, int64_t topk, int64_t R, int64_t N, int out_dtype, void* stream);

/*
 * MLA absorb with an FP8 wkv_b -- the two products of the absorb attention
 * (Admin guide 8.3, steps 5 and 7) that use the up-projection wkv_b
 * [H*(dn+dv), R] viewed per head as [H, dn+dv, R].  With an FP8 wkv_b the
 * pages dequantise the whole weight (weight_dequant, 8.5.2) on every forward
 * step and then run the einsums; here the kernels dequantise in registers
 * with the same rounding (bf16(RN32(decode(q) * s))) and multiply with bf16
 * MFMA, accumulating in float32; the bf16 weight is never stored.
 *
 * mla_absorb_key -- q_nope carried into the latent space by the key rows:
 *   out[t, h, c] = sum_{d < dn} q[t, h, d] * Wd[h*(dn+dv) + d, c]
 * mla_absorb_value -- the attention-weighted latent turned into values by
 * the value rows:
 *   out[t, h, d] = sum_{c < R} x[t, h, c] * Wd[h*(dn+dv) + dn + d, c]
 *
 *   q_bf16 / x_bf16  in   bf16, element (t, h, i) at [t*ld_t + h*ld_h + i]
 *                         for i < dn (key) or i < R (value); ld_t, ld_h >= 0
 *                         and multiples of 8 (so the q_nope slice of a
 *                         [T, H, dn + rope] q can be passed in place)
 *   wkv_b            in   e4m3 [H*(dn+dv), R]
 *   wkv_b_s          in   float32 [H*(dn+dv)/128, R/128]
 *   out              out  contiguous [T, H, R] (key) or [T, H, dv] (value),
 *                         bf16 or float32 (out_dtype)
 *   dn, dv, R positive multiples of 128 (the pages' configurations all use
 *   128, 128, 512); key side: dn is 128 or 256; value side: R <= 512.
 *   T, H >= 0 (either 0 = no-op); the weight, the output and the input's
 *   extent below 2^31 elements.
 * Input, wkv_b and out 16-byte aligned, wkv_b_s 4-byte aligned; out must not
 * overlap an input (FP8BS_ERR_ALIAS).
 */
int fp8bs_mla_absorb_key(const void* q_bf16, int64_t ld_t, int64_t ld_h, const void* wkv_b,
                         const float* wkv_b_s, void* out, int64_t T, int64_t H, int64_t dn,
                         int64_t dv, int64_t R, int out_dtype, void* stream);
int fp8bs_mla_absorb_value(const void* x_bf16, int64_t ld_t, int64_t ld_h, const void* wkv_b,
                           const float* wkv_b_s, void* out, int64_t T, int64_t H, int64_t dn,
                           int64_t dv, int64_t R, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
