/*
 * fp8bs_oracle.c -- CPU oracle for the block-scaled FP8 linear.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, obviously-correct
 * model of what the GPU library computes.  Only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark load it; the product path
 * never does.  It shares no code, header, table or constant with the HIP
 * library: every value it needs is derived here from the definitions.
 *
 * Sources (the method as described on the DeepSeek-V3 pages):
 *   - "DeepSeek-V3 Administrator & Developer Guide", section 8.5.1
 *     (act_quant_kernel), 8.5.2 (weight_dequant_kernel), 8.5.3
 *     (fp8_gemm_kernel), 6.3 (the FP8 path: weight scale shape
 *     ceil(out/128) x ceil(in/128)), 6.4 and 8.4 (MoE expert loop, and the
 *     dispatch and combine around it).
 *   - "DeepSeek-V3 User Guide", section 7 FAQ (scale_fmt ue8m0: the scale is
 *     rounded up to a power of two) and section 6 (K must be a multiple of
 *     the 128 block size).
 *   - The OCP 8-bit floating point specification for the E4M3 ("fn": no
 *     infinities, one NaN mantissa pattern) encoding, which the pages name
 *     only as torch.float8_e4m3fn with maximum magnitude 448.
 *
 * Arithmetic conventions (all in IEEE binary64 unless stated):
 *   - A quotient of two binary32 values is formed in binary64 and rounded
 *     once to binary32.  Because 53 >= 2*24 + 2, this double rounding equals
 *     the correctly rounded binary32 quotient (Figueroa, "When is double
 *     rounding innocuous?", 1995).  So RN32(a/b) is exact-IEEE here.
 *   - A product of an e4m3 value (4 significant bits) and a binary32 value
 *     (24 bits) is exact in binary64.
 *   - A sum of 128 products of two e4m3 values is exact in binary64: each
 *     product is an integer multiple of 2^-18 below 2^18 in magnitude, so the
 *     running sum is a multiple of 2^-18 below 2^25, i.e. under 2^43 units.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math: the arithmetic
 * above relies on strict IEEE evaluation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BLOCK 128
#define ORC_FMT_FP32 0
#define ORC_FMT_UE8M0 1

/* ------------------------------------------------------------------------ */
/* Scalar helpers                                                            */
/* ------------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> binary32: a bf16 value is the top half of a binary32 pattern. */
float orc_bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* binary32 -> bf16, round to nearest, ties to the even significand.
 * Written as an explicit choice between the two neighbouring bf16 values:
 * `lo` (the pattern truncated toward zero) and `hi` (the next pattern away
 * from zero), whichever is nearer; on a tie the one whose last kept bit is 0. */
uint16_t orc_f32_to_bf16(float f) {
    uint32_t u = bits_from_f32(f);
    if (isnan(f)) return (uint16_t)((u >> 16) | 0x0040u);   /* stays a (quiet) NaN */
    uint32_t lo = u & 0xFFFF0000u;
    uint32_t hi = lo + 0x00010000u;
    double a = fabs((double)f);
    double vlo = fabs((double)f32_from_bits(lo));
    /* If `hi` would be the infinity pattern, its value for rounding purposes is 2^128. */
    double vhi = ((hi & 0x7FFFFFFFu) == 0x7F800000u) ? ldexp(1.0, 128)
                                                      : fabs((double)f32_from_bits(hi));
    double dlo = a - vlo, dhi = vhi - a;
    uint32_t pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = hi;
    else pick = ((lo >> 16) & 1u) ? hi : lo;
    return (uint16_t)(pick >> 16);
}

/* ------------------------------------------------------------------------ */
/* E4M3 ("fn") decode and encode                                             */
/* ------------------------------------------------------------------------ */

/* Decode one e4m3fn code: sign bit 7, exponent bits 6..3 (bias 7), mantissa
 * bits 2..0.  Exponent field 0 is subnormal (m * 2^-9).  The pattern with all
 * exponent and mantissa bits set (0x7F / 0xFF) is NaN; there are no
 * infinities, so exponent field 15 with mantissa 0..6 is finite (up to 448). */
double orc_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* The 127 finite non-negative magnitudes, indexed by code 0x00..0x7E; they are
 * strictly increasing in the code. */
static double g_mag[127];
static int g_mag_ready = 0;
static void mag_init(void) {
    if (g_mag_ready) return;
    for (int c = 0; c < 127; ++c) g_mag[c] = orc_e4m3_decode((uint8_t)c);
    g_mag_ready = 1;
}

/* Encode a real y to e4m3fn: round to the nearest finite magnitude by explicit
 * comparison with the midpoint of the two neighbours; an exact midpoint goes
 * to the even code (the code's last bit is the mantissa's last bit).  Any
 * magnitude >= 448 saturates to 448 (0x7E).  The sign is kept, so negative
 * values that round to zero give 0x80.  NaN gives 0x7F. */
uint8_t orc_e4m3_encode(double y) {
    mag_init();
    if (isnan(y)) return 0x7F;
    uint8_t sign = signbit(y) ? 0x80 : 0x00;
    double a = fabs(y);
    /* c = largest code with g_mag[c] <= a (binary search on the sorted table). */
    int lo = 0, hi = 126;
    if (a >= g_mag[126]) return (uint8_t)(sign | 126);
    while (lo < hi) {               /* invariant: g_mag[lo] <= a < g_mag[hi+1] */
        int mid = (lo + hi + 1) / 2;
        if (g_mag[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    double midpoint = 0.5 * (g_mag[c] + g_mag[c + 1]);   /* exact in binary64 */
    int code;
    if (a < midpoint) code = c;
    else if (a > midpoint) code = c + 1;
    else code = (c % 2 == 0) ? c : c + 1;
    return (uint8_t)(sign | code);
}

void orc_e4m3_encode_f32_array(const float* y, uint8_t* q, int64_t n) {
    mag_init();
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) q[i] = orc_e4m3_encode((double)y[i]);
}

void orc_e4m3_decode_array(const uint8_t* q, double* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_decode(q[i]);
}

/* ------------------------------------------------------------------------ */
/* Block scale rule (Admin guide 8.5.1; User guide FAQ on ue8m0)             */
/* ------------------------------------------------------------------------ */

/* s = RN32(max(amax, 1e-4) / 448), with the 1e-4 floor taken as the binary32
 * value nearest 1e-4.  For ue8m0, s becomes the smallest power of two that is
 * >= s (kept if s already is one). */
float orc_block_scale(float amax, int fmt) {
    const float floor32 = 1e-4f;
    float a = amax < floor32 ? floor32 : amax;
    float s = (float)((double)a / 448.0);
    if (fmt == ORC_FMT_UE8M0) {
        int e;
        double f = frexp((double)s, &e);      /* s = f * 2^e, f in [0.5, 1) */
        s = (f == 0.5) ? s : (float)ldexp(1.0, e);
    }
    return s;
}

/* y = RN32(x / s), then the e4m3 code of y. */
static uint8_t quant_one(float x, float s) {
    float y = (float)((double)x / (double)s);
    return orc_e4m3_encode((double)y);
}

/* ------------------------------------------------------------------------ */
/* act_quant: 1 x 128 blocks along the last dimension (Admin guide 8.5.1)    */
/* ------------------------------------------------------------------------ */

/* x: bf16 bit patterns [M, K] row-major, K % 128 == 0.
 * q: e4m3 codes [M, K];  s: binary32 [M, K/128]. */
void orc_act_quant(const uint16_t* x, int64_t M, int64_t K, int fmt, uint8_t* q, float* s) {
    mag_init();
    int64_t nb = K / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t j = 0; j < nb; ++j) {
            const uint16_t* xb = x + m * K + j * ORC_BLOCK;
            float amax = 0.0f;
            for (int k = 0; k < ORC_BLOCK; ++k) {
                float v = fabsf(orc_bf16_to_f32(xb[k]));
                if (v > amax) amax = v;
            }
            float sc = orc_block_scale(amax, fmt);
            s[m * nb + j] = sc;
            for (int k = 0; k < ORC_BLOCK; ++k)
                q[m * K + j * ORC_BLOCK + k] = quant_one(orc_bf16_to_f32(xb[k]), sc);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Weight quantisation, 128 x 128 blocks (harness input; not on the pages,   */
/* which ship weights already quantised: same rule as act_quant, applied to  */
/* a 2-D block; a partial edge block uses its own amax)                      */
/* ------------------------------------------------------------------------ */

/* w: bf16 [N, K]; q: e4m3 [N, K]; s: binary32 [ceil(N/128), ceil(K/128)]. */
/* fmt selects the scale rule as for act_quant: float32 or rounded up to a
 * power of two (ue8m0).  The pages round only activation scales; power-of-two
 * weight scales are a harness option for the ue8m0 fast path, where both
 * operands carry power-of-two scales. */
void orc_weight_quant_fmt(const uint16_t* w, int64_t N, int64_t K, int fmt, uint8_t* q, float* s) {
    mag_init();
    int64_t nbn = (N + ORC_BLOCK - 1) / ORC_BLOCK, nbk = (K + ORC_BLOCK - 1) / ORC_BLOCK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bn = 0; bn < nbn; ++bn) {
        for (int64_t bk = 0; bk < nbk; ++bk) {
            int64_t n0 = bn * ORC_BLOCK, n1 = n0 + ORC_BLOCK < N ? n0 + ORC_BLOCK : N;
            int64_t k0 = bk * ORC_BLOCK, k1 = k0 + ORC_BLOCK < K ? k0 + ORC_BLOCK : K;
            float amax = 0.0f;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t k = k0; k < k1; ++k) {
                    float v = fabsf(orc_bf16_to_f32(w[n * K + k]));
                    if (v > amax) amax = v;
                }
            float sc = orc_block_scale(amax, fmt);
            s[bn * nbk + bk] = sc;
            for (int64_t n = n0; n < n1; ++n)
                for (int64_t k = k0; k < k1; ++k)
                    q[n * K + k] = quant_one(orc_bf16_to_f32(w[n * K + k]), sc);
        }
    }
}

void orc_weight_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* s) {
    orc_weight_quant_fmt(w, N, K, ORC_FMT_FP32, q, s);
}

/* ------------------------------------------------------------------------ */
/* weight_dequant (Admin guide 8.5.2): out = bf16(RN32(decode(q) * s))       */
/* ------------------------------------------------------------------------ */

void orc_weight_dequant(const uint8_t* q, const float* s, int64_t N, int64_t K, uint16_t* out) {
    int64_t nbk = (K + ORC_BLOCK - 1) / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double sc = (double)s[(n / ORC_BLOCK) * nbk + (k / ORC_BLOCK)];
            float prod = (float)(orc_e4m3_decode(q[n * K + k]) * sc);  /* exact, then RN32 */
            out[n * K + k] = orc_f32_to_bf16(prod);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* fp8_gemm (Admin guide 8.5.3):                                             */
/*   C[m,n] = sum_kb ( sum_{k in kb} A[m,k] B[n,k] ) * a_s[m,kb] * b_s[n/128,kb] */
/* A e4m3 [M,K], a_s [M,K/128]; B e4m3 [N,K] (out x in), b_s [ceil(N/128),K/128]. */
/* ------------------------------------------------------------------------ */

static double gemm_point(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
                         int64_t K, int64_t m, int64_t n, const double* dec) {
    int64_t nbk = K / ORC_BLOCK;
    double acc = 0.0;
    for (int64_t kb = 0; kb < nbk; ++kb) {
        double p = 0.0;                          /* exact block partial */
        const uint8_t* ar = a + m * K + kb * ORC_BLOCK;
        const uint8_t* br = b + n * K + kb * ORC_BLOCK;
        for (int k = 0; k < ORC_BLOCK; ++k) p += dec[ar[k]] * dec[br[k]];
        acc += p * (double)a_s[m * nbk + kb] * (double)b_s[(n / ORC_BLOCK) * nbk + kb];
    }
    return acc;
}

static void decode_table(double* dec) {
    for (int c = 0; c < 256; ++c) dec[c] = orc_e4m3_decode((uint8_t)c);
}

void orc_gemm(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
              int64_t M, int64_t N, int64_t K, double* c) {
    double dec[256];
    decode_table(dec);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            c[m * N + n] = gemm_point(a, a_s, b, b_s, K, m, n, dec);
}

/* C at a list of (row, col) points only -- used for full-size checks. */
void orc_gemm_points(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
                     int64_t K, const int64_t* rows, const int64_t* cols, int64_t npts, double* out) {
    double dec[256];
    decode_table(dec);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i)
        out[i] = gemm_point(a, a_s, b, b_s, K, rows[i], cols[i], dec);
}

/* ------------------------------------------------------------------------ */
/* Grouped MoE GEMM (Admin guide 6.4: each expert multiplies the rows routed */
/* to it by its own weight).  Rows [off[e], off[e+1]) of A belong to expert   */
/* e; B is [E, N, K] with scales [E, ceil(N/128), K/128].                    */
/* ------------------------------------------------------------------------ */

void orc_moe_gemm(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
                  const int32_t* off, int64_t R, int64_t E, int64_t N, int64_t K, double* c) {
    double dec[256];
    decode_table(dec);
    int64_t nbk = K / ORC_BLOCK, nbn = (N + ORC_BLOCK - 1) / ORC_BLOCK;
    (void)R;
    for (int64_t e = 0; e < E; ++e) {
        const uint8_t* be = b + e * N * K;
        const float* bse = b_s + e * nbn * nbk;
        int64_t r0 = off[e], r1 = off[e + 1];
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t m = r0; m < r1; ++m)
            for (int64_t n = 0; n < N; ++n)
                c[m * N + n] = gemm_point(a, a_s, be, bse, K, m, n, dec);
    }
}

/* MoE output at (row, col) points; the expert of a row is found from off[]. */
void orc_moe_gemm_points(const uint8_t* a, const float* a_s, const uint8_t* b, const float* b_s,
                         const int32_t* off, int64_t E, int64_t N, int64_t K,
                         const int64_t* rows, const int64_t* cols, int64_t npts, double* out) {
    double dec[256];
    decode_table(dec);
    int64_t nbk = K / ORC_BLOCK, nbn = (N + ORC_BLOCK - 1) / ORC_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i) {
        int64_t e = 0;
        while (e + 1 < E && off[e + 1] <= rows[i]) ++e;   /* expert owning the row */
        out[i] = gemm_point(a, a_s, b + e * N * K, b_s + e * nbn * nbk, K, rows[i], cols[i], dec);
    }
}

/* ------------------------------------------------------------------------ */
/* The BF16 path of the linear (Admin guide 6.3: with gemm_impl "bf16" the   */
/* FP8 weight is dequantised by weight_dequant (8.5.2) and the product runs   */
/* as a BF16 F.linear): C[m, n] = sum_k x[m, k] * Wd[n, k], x bf16 [M, K],    */
/* Wd = weight_dequant(q, s) bf16 [N, K].  Each product of two bf16 values is */
/* exact in binary64 (8 + 8 significant bits) and the sum of K of them is    */
/* formed in binary64 in k order (exact while K * 2^16 * 2^(e-range) fits;   */
/* in any case within a few binary64 ulps).                                  */
/* ------------------------------------------------------------------------ */
static double w8a16_point(const uint16_t* x, const uint16_t* wd, int64_t K, int64_t m, int64_t n) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k)
        acc += (double)orc_bf16_to_f32(x[m * K + k]) * (double)orc_bf16_to_f32(wd[n * K + k]);
    return acc;
}

void orc_w8a16_gemm(const uint16_t* x, const uint8_t* q, const float* s, int64_t M, int64_t N,
                    int64_t K, double* c) {
    uint16_t* wd = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * K > 0 ? N * K : 1));
    orc_weight_dequant(q, s, N, K, wd);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) c[m * N + n] = w8a16_point(x, wd, K, m, n);
    free(wd);
}

/* The same at (row, col) points. */
void orc_w8a16_gemm_points(const uint16_t* x, const uint8_t* q, const float* s, int64_t N, int64_t K,
                           const int64_t* rows, const int64_t* cols, int64_t npts, double* out) {
    uint16_t* wd = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * K > 0 ? N * K : 1));
    orc_weight_dequant(q, s, N, K, wd);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i) out[i] = w8a16_point(x, wd, K, rows[i], cols[i]);
    free(wd);
}

/* ------------------------------------------------------------------------ */
/* MLA "absorb" with an FP8 wkv_b (Admin guide 8.3, steps 5 and 7; the FP8   */
/* weight is dequantised by weight_dequant (8.5.2), then used in the two      */
/* einsums).  wkv_b [H*(dn+dv), R] viewed as [H, dn+dv, R]: the first dn     */
/* rows of head h absorb q_nope into the latent space, the last dv rows turn  */
/* the attention-weighted latent into the head's values:                     */
/*   key side   out[t,h,c] = sum_{d<dn} q[t,h,d] * Wd[h(dn+dv) + d, c]        */
/*   value side out[t,h,d] = sum_{c<R}  x[t,h,c] * Wd[h(dn+dv) + dn + d, c]   */
/* q [T,H,dn] and x [T,H,R] are bf16, products are exact in binary64 and the  */
/* sums run in binary64 in index order.                                      */
/* ------------------------------------------------------------------------ */
static double mla_point(int side, const uint16_t* in, const uint16_t* wd, int64_t H, int64_t dn,
                        int64_t dv, int64_t R, int64_t t, int64_t h, int64_t col) {
    double acc = 0.0;
    if (side == 0) {            /* key side: col = c, sum over d */
        for (int64_t d = 0; d < dn; ++d)
            acc += (double)orc_bf16_to_f32(in[(t * H + h) * dn + d]) *
                   (double)orc_bf16_to_f32(wd[(h * (dn + dv) + d) * R + col]);
    } else {                    /* value side: col = d, sum over c */
        for (int64_t c = 0; c < R; ++c)
            acc += (double)orc_bf16_to_f32(in[(t * H + h) * R + c]) *
                   (double)orc_bf16_to_f32(wd[(h * (dn + dv) + dn + col) * R + c]);
    }
    return acc;
}

static uint16_t* mla_dequant(const uint8_t* w, const float* s, int64_t H, int64_t dn, int64_t dv,
                             int64_t R) {
    int64_t n = H * (dn + dv);
    uint16_t* wd = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(n * R > 0 ? n * R : 1));
    orc_weight_dequant(w, s, n, R, wd);
    return wd;
}

/* side 0: q [T,H,dn] -> out [T,H,R]; side 1: x [T,H,R] -> out [T,H,dv]. */
void orc_mla_absorb(int side, const uint16_t* in, const uint8_t* w, const float* s, int64_t T,
                    int64_t H, int64_t dn, int64_t dv, int64_t R, double* out) {
    uint16_t* wd = mla_dequant(w, s, H, dn, dv, R);
    int64_t ncol = side == 0 ? R : dv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t col = 0; col < ncol; ++col)
                out[(t * H + h) * ncol + col] = mla_point(side, in, wd, H, dn, dv, R, t, h, col);
    free(wd);
}

/* The same at (t, h, col) points. */
void orc_mla_absorb_points(int side, const uint16_t* in, const uint8_t* w, const float* s,
                           int64_t H, int64_t dn, int64_t dv, int64_t R, const int64_t* ts,
                           const int64_t* hs, const int64_t* cols, int64_t npts, double* out) {
    uint16_t* wd = mla_dequant(w, s, H, dn, dv, R);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < npts; ++i)
        out[i] = mla_point(side, in, wd, H, dn, dv, R, ts[i], hs[i], cols[i]);
    free(wd);
}

/* ------------------------------------------------------------------------ */
/* MoE dispatch and combine around the expert GEMMs (Admin guide 6.4 and     */
/* 8.4: per-expert hit counts; for each expert with hits, the (token, slot)  */
/* pairs whose routed expert it is, in token order as the pages' index       */
/* lookup yields them; the expert runs on those tokens' rows; its output     */
/* is scaled by the routing weight of that (token, slot) and summed into the */
/* token's output, which starts at zero).                                     */
/* ------------------------------------------------------------------------ */

/* Stable counting sort of the routed expert ids idx [T, topk] by expert.
 * Expert e owns rows [off[e], off[e+1]); within it, rows follow (token,
 * slot) order.  row_token/row_slot [R] give each row's source pair and
 * row_of [T, topk] the row of each pair.  Ids outside [0, E) are not routed:
 * their row_of is -1 and they take no row.  Returns R = off[E]. */
int64_t orc_moe_route(const int32_t* idx, int64_t T, int64_t topk, int64_t E, int32_t* off,
                      int32_t* row_token, int32_t* row_slot, int32_t* row_of) {
    /* pass 1: hit counts per expert */
    for (int64_t e = 0; e <= E; ++e) off[e] = 0;
    for (int64_t i = 0; i < T * topk; ++i)
        if (idx[i] >= 0 && idx[i] < E) off[idx[i] + 1] += 1;
    /* exclusive prefix: first row of each expert */
    for (int64_t e = 0; e < E; ++e) off[e + 1] += off[e];
    /* pass 2: place every pair at its expert's next free row, in (t, s) order */
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    for (int64_t e = 0; e < E; ++e) next[e] = off[e];
    for (int64_t t = 0; t < T; ++t)
        for (int64_t k = 0; k < topk; ++k) {
            int32_t e = idx[t * topk + k];
            if (e < 0 || e >= E) {
                row_of[t * topk + k] = -1;
                continue;
            }
            int32_t r = next[e]++;
            row_token[r] = (int32_t)t;
            row_slot[r] = (int32_t)k;
            row_of[t * topk + k] = r;
        }
    free(next);
    return off[E];
}

/* The expert inputs: act_quant of every token row of x [T, K], placed at the
 * rows its (token, slot) pairs were routed to.  The quantisation is row-local,
 * so this is the quantisation of the gathered rows x[row_token[r]]. */
void orc_moe_quant_scatter(const uint16_t* x, int64_t T, int64_t K, int fmt, const int32_t* row_of,
                           int64_t topk, int64_t R, uint8_t* q, float* s) {
    int64_t nb = K / ORC_BLOCK;
    uint8_t* qt = (uint8_t*)malloc((size_t)K);
    float* st = (float*)malloc(sizeof(float) * (size_t)nb);
    for (int64_t t = 0; t < T; ++t) {
        orc_act_quant(x + t * K, 1, K, fmt, qt, st);
        for (int64_t k = 0; k < topk; ++k) {
            int32_t r = row_of[t * topk + k];
            if (r < 0 || r >= R) continue;
            memcpy(q + (int64_t)r * K, qt, (size_t)K);
            memcpy(s + (int64_t)r * nb, st, sizeof(float) * (size_t)nb);
        }
    }
    free(qt);
    free(st);
}

/* The combine: y[t, n] = sum over slots k of w[t, k] * out[row_of[t, k], n],
 * with out given as bf16 bit patterns [R, N] and w as binary32.  Each term
 * is exact in binary64 (8 + 24 significant bits); the sum of at most topk
 * terms is formed in binary64 in slot order.  Pairs that were not routed
 * (row_of < 0) contribute nothing. */
void orc_moe_combine(const uint16_t* out, const float* w, const int32_t* row_of, int64_t T,
                     int64_t topk, int64_t R, int64_t N, double* y) {
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < topk; ++k) {
                int32_t r = row_of[t * topk + k];
                if (r < 0 || r >= R) continue;
                acc += (double)w[t * topk + k] * (double)orc_bf16_to_f32(out[(int64_t)r * N + n]);
            }
            y[t * N + n] = acc;
        }
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
