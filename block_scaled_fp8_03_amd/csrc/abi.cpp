// abi.cpp -- the C entry points declared in include/fp8bs.h.  Each one checks
// its arguments on the host (no HIP call happens before the checks pass) and
// then enqueues the kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8bs.h"
#include "launch.h"

namespace {

// The tile kernels address operands with 32-bit byte offsets and may touch up
// to 256 rows past the end of an operand (those loads return zeros), so
// (rows + 256) * K must stay below 2^32 for A and for (each expert's) B.
constexpr int64_t kLimit32 = (int64_t)1 << 32;
constexpr int64_t kLimitInt = ((int64_t)1 << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// [p, p + n) and [q, q + m) intersect (empty ranges never do)
bool overlap(const void* p, int64_t n, const void* q, int64_t m) {
  if (n <= 0 || m <= 0) return false;
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)m && b < a + (uintptr_t)n;
}

// product of non-negative sizes, or -1 on int64 overflow
int64_t mul(int64_t a, int64_t b) {
  if (a == 0 || b == 0) return 0;
  if (a > INT64_MAX / b) return -1;
  return a * b;
}

int status_of(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_ERR_HIP; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL: return "a required pointer is NULL";
    case FP8BS_ERR_SHAPE: return "invalid shape (negative size, K not a multiple of 128, or size limit exceeded)";
    case FP8BS_ERR_ALIGN: return "a pointer is not aligned as required (16 bytes for tensors, 4 for scales)";
    case FP8BS_ERR_ENUM: return "unknown scale_fmt or out_dtype";
    case FP8BS_ERR_HIP: return "HIP kernel launch failed";
    case FP8BS_ERR_ALIAS: return "an output buffer overlaps an input buffer";
    default: return "unknown status";
  }
}

int fp8bs_version(void) { return 10000; }

int fp8bs_act_quant(const void* x_bf16, void* q_e4m3, float* s, int64_t M, int64_t K,
                    int scale_fmt, void* stream) {
  if (M < 0 || K < 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (scale_fmt != FP8BS_SCALE_FP32 && scale_fmt != FP8BS_SCALE_UE8M0) return FP8BS_ERR_ENUM;
  const int64_t n = mul(M, K);
  if (n < 0 || mul(n, 2) < 0 || !fp8bs::act_quant_fits(M, K)) return FP8BS_ERR_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (!x_bf16 || !q_e4m3 || !s) return FP8BS_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(s, 4)) return FP8BS_ERR_ALIGN;
  const int64_t ns = n / 128;
  if (overlap(q_e4m3, n, x_bf16, 2 * n) || overlap(s, 4 * ns, x_bf16, 2 * n) ||
      overlap(q_e4m3, n, s, 4 * ns))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_act_quant(x_bf16, q_e4m3, s, M, K,
                                           scale_fmt == FP8BS_SCALE_UE8M0, (hipStream_t)stream));
}

int fp8bs_e4m3_encode(const float* x, void* q_e4m3, int64_t n, void* stream) {
  if (n < 0 || !fp8bs::e4m3_encode_fits(n)) return FP8BS_ERR_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (!x || !q_e4m3) return FP8BS_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q_e4m3, 4)) return FP8BS_ERR_ALIGN;
  if (overlap(q_e4m3, n, x, 4 * n)) return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_e4m3_encode(x, q_e4m3, n, (hipStream_t)stream));
}

static int weight_quant_entry(bool ue8m0, const void* w_bf16, void* q_e4m3, float* s, int64_t N,
                              int64_t K, void* stream) {
  if (N < 0 || K < 0) return FP8BS_ERR_SHAPE;
  const int64_t n = mul(N, K);
  if (n < 0 || mul(n, 2) < 0 || cdiv(N, 128) > 65535 || cdiv(K, 128) > kLimitInt)
    return FP8BS_ERR_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (!w_bf16 || !q_e4m3 || !s) return FP8BS_ERR_NULL;
  if (!aligned(w_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(s, 4)) return FP8BS_ERR_ALIGN;
  const int64_t ns = cdiv(N, 128) * cdiv(K, 128);
  if (overlap(q_e4m3, n, w_bf16, 2 * n) || overlap(s, 4 * ns, w_bf16, 2 * n) ||
      overlap(q_e4m3, n, s, 4 * ns))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_weight_quant(w_bf16, q_e4m3, s, N, K, ue8m0, (hipStream_t)stream));
}

int fp8bs_weight_quant(const void* w_bf16, void* q_e4m3, float* s, int64_t N, int64_t K,
                       void* stream) {
  return weight_quant_entry(false, w_bf16, q_e4m3, s, N, K, stream);
}

int fp8bs_weight_quant_ue8m0(const void* w_bf16, void* q_e4m3, float* s, int64_t N, int64_t K,
                             void* stream) {
  return weight_quant_entry(true, w_bf16, q_e4m3, s, N, K, stream);
}

int fp8bs_weight_dequant(const void* w_e4m3, const float* s, void* y_bf16, int64_t N, int64_t K,
                         void* stream) {
  if (N < 0 || K < 0) return FP8BS_ERR_SHAPE;
  const int64_t n = mul(N, K);
  if (n < 0 || mul(n, 2) < 0 || !fp8bs::weight_dequant_fits(N, K)) return FP8BS_ERR_SHAPE;
  if (n == 0) return FP8BS_OK;
  if (!w_e4m3 || !s || !y_bf16) return FP8BS_ERR_NULL;
  if (!aligned(w_e4m3, 16) || !aligned(y_bf16, 16) || !aligned(s, 4)) return FP8BS_ERR_ALIGN;
  const int64_t ns = cdiv(N, 128) * cdiv(K, 128);
  if (overlap(y_bf16, 2 * n, w_e4m3, n) || overlap(y_bf16, 2 * n, s, 4 * ns)) return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_weight_dequant(w_e4m3, s, y_bf16, N, K, (hipStream_t)stream));
}

static int gemm_entry(bool ue8m0, const void* a, const float* a_s, const void* b, const float* b_s,
                      void* c, int64_t M, int64_t N, int64_t K, int out_dtype, void* stream) {
  if (M < 0 || N < 0 || K < 128 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_F32) return FP8BS_ERR_ENUM;
  if (M > kLimitInt || N > kLimitInt || K > kLimitInt) return FP8BS_ERR_SHAPE;
  const int64_t na = mul(M, K), nb = mul(N, K), nc = mul(M, N);
  if (na < 0 || nb < 0 || nc < 0 || mul(M + 256, K) >= kLimit32 || mul(N + 256, K) >= kLimit32 ||
      mul(nc, 4) < 0)
    return FP8BS_ERR_SHAPE;
  if (nc == 0) return FP8BS_OK;
  if (!a || !a_s || !b || !b_s || !c) return FP8BS_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16) || !aligned(a_s, 4) ||
      !aligned(b_s, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t cb = nc * (out_dtype == FP8BS_OUT_F32 ? 4 : 2);
  const int64_t nas = M * (K / 128) * 4, nbs = cdiv(N, 128) * (K / 128) * 4;
  if (overlap(c, cb, a, na) || overlap(c, cb, b, nb) || overlap(c, cb, a_s, nas) ||
      overlap(c, cb, b_s, nbs))
    return FP8BS_ERR_ALIAS;
  const bool f32 = out_dtype == FP8BS_OUT_F32;
  return status_of(ue8m0 ? fp8bs::launch_gemm_ue8m0(a, a_s, b, b_s, c, M, N, K, f32, (hipStream_t)stream)
                         : fp8bs::launch_gemm(a, a_s, b, b_s, c, M, N, K, f32, (hipStream_t)stream));
}

int fp8bs_gemm(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
               int64_t M, int64_t N, int64_t K, int out_dtype, void* stream) {
  return gemm_entry(false, a, a_s, b, b_s, c, M, N, K, out_dtype, stream);
}

int fp8bs_gemm_ue8m0(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
                     int64_t M, int64_t N, int64_t K, int out_dtype, void* stream) {
  return gemm_entry(true, a, a_s, b, b_s, c, M, N, K, out_dtype, stream);
}

int fp8bs_moe_gemm(const void* a, const float* a_s, const void* b, const float* b_s,
                   const int32_t* offsets, void* c, int64_t R, int64_t E, int64_t N, int64_t K,
                   int out_dtype, void* stream) {
  if (R < 0 || E < 0 || N < 0 || K < 128 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_F32) return FP8BS_ERR_ENUM;
  if (R > kLimitInt || E > kLimitInt || N > kLimitInt || K > kLimitInt) return FP8BS_ERR_SHAPE;
  const int64_t na = mul(R, K), nbe = mul(N, K), nb = mul(E, nbe), nc = mul(R, N);
  if (na < 0 || nbe < 0 || nb < 0 || nc < 0 || mul(R + 256, K) >= kLimit32 ||
      mul(N + 256, K) >= kLimit32 || mul(nc, 4) < 0)
    return FP8BS_ERR_SHAPE;
  // the launch grid is at most (R / 256 + 2 E) * ceil(N / 256) + 16 workgroups
  if (mul(R / 64 + 2 * E, cdiv(N, 256)) > kLimitInt - 16) return FP8BS_ERR_SHAPE;
  if (nc == 0 || E == 0) return FP8BS_OK;
  if (!a || !a_s || !b || !b_s || !offsets || !c) return FP8BS_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16) || !aligned(a_s, 4) ||
      !aligned(b_s, 4) || !aligned(offsets, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t cb = nc * (out_dtype == FP8BS_OUT_F32 ? 4 : 2);
  const int64_t nas = R * (K / 128) * 4, nbs = E * cdiv(N, 128) * (K / 128) * 4;
  if (overlap(c, cb, a, na) || overlap(c, cb, b, nb) || overlap(c, cb, a_s, nas) ||
      overlap(c, cb, b_s, nbs) || overlap(c, cb, offsets, 4 * (E + 1)))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_moe_gemm(a, a_s, b, b_s, offsets, c, R, E, N, K,
                                          out_dtype == FP8BS_OUT_F32, (hipStream_t)stream));
}

int fp8bs_w8a16_gemm(const void* x_bf16, const void* w_e4m3, const float* w_s, void* c, int64_t M,
                     int64_t N, int64_t K, int out_dtype, void* stream) {
  if (M < 0 || N < 0 || K < 128 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_F32) return FP8BS_ERR_ENUM;
  if (M > kLimitInt || N > kLimitInt || K > kLimitInt) return FP8BS_ERR_SHAPE;
  const int64_t nx = mul(M, K), nw = mul(N, K), nc = mul(M, N);
  if (nx < 0 || nw < 0 || nc < 0 || mul(M + 256, 2 * K) >= kLimit32 || mul(N + 256, K) >= kLimit32 ||
      mul(nc, 4) < 0 || mul(cdiv(M, 256), cdiv(N, 256)) > kLimitInt)
    return FP8BS_ERR_SHAPE;
  if (nc == 0) return FP8BS_OK;
  if (!x_bf16 || !w_e4m3 || !w_s || !c) return FP8BS_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(w_e4m3, 16) || !aligned(c, 16) || !aligned(w_s, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t cb = nc * (out_dtype == FP8BS_OUT_F32 ? 4 : 2);
  const int64_t nws = cdiv(N, 128) * (K / 128) * 4;
  if (overlap(c, cb, x_bf16, 2 * nx) || overlap(c, cb, w_e4m3, nw) || overlap(c, cb, w_s, nws))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_w8a16_gemm(x_bf16, w_e4m3, w_s, c, M, N, K,
                                            out_dtype == FP8BS_OUT_F32, (hipStream_t)stream));
}

static int mla_entry(bool value_side, const void* in, int64_t ld_t, int64_t ld_h, const void* w,
                     const float* w_s, void* out, int64_t T, int64_t H, int64_t dn, int64_t dv,
                     int64_t R, int out_dtype, void* stream) {
  if (T < 0 || H < 0 || ld_t < 0 || ld_h < 0 || dn <= 0 || dv <= 0 || R <= 0 || dn % 128 != 0 ||
      dv % 128 != 0 || R % 128 != 0)
    return FP8BS_ERR_SHAPE;
  if (value_side ? R > 512 : (dn != 128 && dn != 256)) return FP8BS_ERR_SHAPE;
  if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_F32) return FP8BS_ERR_ENUM;
  if (ld_t % 8 != 0 || ld_h % 8 != 0) return FP8BS_ERR_ALIGN;
  const int64_t width = value_side ? R : dn, ncol = value_side ? dv : R;
  const int64_t nrows = mul(H, dn + dv), nw = mul(nrows, R), nout = mul(mul(T, H), ncol);
  // every element offset the kernels form fits an int
  if (nrows < 0 || nw < 0 || nout < 0 || nw > kLimitInt || nout > kLimitInt || ld_t > kLimitInt ||
      ld_h > kLimitInt || dn + dv > kLimitInt)
    return FP8BS_ERR_SHAPE;
  if (nout == 0) return FP8BS_OK;
  const int64_t nin = mul(T - 1, ld_t) + mul(H - 1, ld_h) + width;   // input extent (elements)
  if (nin > kLimitInt || mul(H, cdiv(T, 256)) > kLimitInt) return FP8BS_ERR_SHAPE;
  if (!in || !w || !w_s || !out) return FP8BS_ERR_NULL;
  if (!aligned(in, 16) || !aligned(w, 16) || !aligned(out, 16) || !aligned(w_s, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t ob = nout * (out_dtype == FP8BS_OUT_F32 ? 4 : 2);
  const int64_t nws = (nrows / 128) * (R / 128) * 4;
  if (overlap(out, ob, in, 2 * nin) || overlap(out, ob, w, nw) || overlap(out, ob, w_s, nws))
    return FP8BS_ERR_ALIAS;
  const bool f32 = out_dtype == FP8BS_OUT_F32;
  return status_of(value_side
                       ? fp8bs::launch_mla_absorb_value(in, ld_t, ld_h, w, w_s, out, T, H, dn, dv,
                                                        R, f32, (hipStream_t)stream)
                       : fp8bs::launch_mla_absorb_key(in, ld_t, ld_h, w, w_s, out, T, H, dn, dv, R,
                                                      f32, (hipStream_t)stream));
}

int fp8bs_mla_absorb_key(const void* q_bf16, int64_t ld_t, int64_t ld_h, const void* wkv_b,
                         const float* wkv_b_s, void* out, int64_t T, int64_t H, int64_t dn,
                         int64_t dv, int64_t R, int out_dtype, void* stream) {
  return mla_entry(false, q_bf16, ld_t, ld_h, wkv_b, wkv_b_s, out, T, H, dn, dv, R, out_dtype,
                   stream);
}

int fp8bs_mla_absorb_value(const void* x_bf16, int64_t ld_t, int64_t ld_h, const void* wkv_b,
                           const float* wkv_b_s, void* out, int64_t T, int64_t H, int64_t dn,
                           int64_t dv, int64_t R, int out_dtype, void* stream) {
  return mla_entry(true, x_bf16, ld_t, ld_h, wkv_b, wkv_b_s, out, T, H, dn, dv, R, out_dtype,
                   stream);
}

int64_t fp8bs_moe_route_workspace_size(int64_t T, int64_t topk, int64_t E) {
  if (T < 0 || topk < 1 || E < 1 || E > kLimitInt) return -1;
  const int64_t P = mul(T, topk);
  if (P < 0 || P > kLimitInt) return -1;
  const int64_t bytes = mul(mul(cdiv(P, 512), E), 4);
  return bytes < 0 ? -1 : bytes;
}

int fp8bs_moe_route(const int32_t* indices, int64_t T, int64_t topk, int64_t E, int32_t* offsets,
                    int32_t* row_token, int32_t* row_of, void* workspace,
                    int64_t workspace_bytes, void* stream) {
  const int64_t need = fp8bs_moe_route_workspace_size(T, topk, E);
  if (need < 0) return FP8BS_ERR_SHAPE;
  if (workspace_bytes < need) return FP8BS_ERR_SHAPE;
  const int64_t P = T * topk;
  if (!offsets) return FP8BS_ERR_NULL;
  if (P > 0 && (!indices || !row_token || !row_of || !workspace)) return FP8BS_ERR_NULL;
  if (!aligned(indices, 4) || !aligned(offsets, 4) || !aligned(row_token, 4) ||
      !aligned(row_of, 4) || !aligned(workspace, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t ob = 4 * (E + 1), pb = 4 * P;
  if (overlap(offsets, ob, indices, pb) || overlap(row_token, pb, indices, pb) ||
      overlap(row_of, pb, indices, pb) || overlap(offsets, ob, row_token, pb) ||
      overlap(offsets, ob, row_of, pb) || overlap(row_token, pb, row_of, pb) ||
      overlap(workspace, need, indices, pb) || overlap(workspace, need, offsets, ob) ||
      overlap(workspace, need, row_token, pb) || overlap(workspace, need, row_of, pb))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_moe_route(indices, T, topk, E, offsets, row_token, row_of,
                                           workspace, (hipStream_t)stream));
}

int fp8bs_moe_route_noalloc(const int32_t* indices, int64_t T, int64_t topk, int64_t E,
                            int32_t* offsets, int32_t* row_token, int32_t* row_of, void* stream) {
  const int64_t need = fp8bs_moe_route_workspace_size(T, topk, E);
  if (need < 0 || need > fp8bs::kRouteScratchBytes) return FP8BS_ERR_SHAPE;
  const int64_t P = T * topk;
  if (!offsets) return FP8BS_ERR_NULL;
  if (P > 0 && (!indices || !row_token || !row_of)) return FP8BS_ERR_NULL;
  if (!aligned(indices, 4) || !aligned(offsets, 4) || !aligned(row_token, 4) || !aligned(row_of, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t ob = 4 * (E + 1), pb = 4 * P;
  if (overlap(offsets, ob, indices, pb) || overlap(row_token, pb, indices, pb) ||
      overlap(row_of, pb, indices, pb) || overlap(offsets, ob, row_token, pb) ||
      overlap(offsets, ob, row_of, pb) || overlap(row_token, pb, row_of, pb))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_moe_route_noalloc(indices, T, topk, E, offsets, row_token, row_of,
                                                   (hipStream_t)stream));
}

int fp8bs_moe_quant_scatter(const void* x_bf16, const int32_t* row_of, void* q_e4m3, float* s,
                            int64_t T, int64_t topk, int64_t R, int64_t K, int scale_fmt,
                            void* stream) {
  if (T < 0 || topk < 1 || R < 0 || K < 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (scale_fmt != FP8BS_SCALE_FP32 && scale_fmt != FP8BS_SCALE_UE8M0) return FP8BS_ERR_ENUM;
  const int64_t nx = mul(T, K), nq = mul(R, K), P = mul(T, topk);
  if (nx < 0 || nq < 0 || P < 0 || P > kLimitInt || mul(nx, 2) < 0 || R > kLimitInt ||
      !fp8bs::act_quant_fits(T, K))
    return FP8BS_ERR_SHAPE;
  if (nx == 0 || nq == 0) return FP8BS_OK;
  if (!x_bf16 || !row_of || !q_e4m3 || !s) return FP8BS_ERR_NULL;
  if (!aligned(x_bf16, 16) || !aligned(q_e4m3, 16) || !aligned(s, 4) || !aligned(row_of, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t ns = 4 * (nq / 128);
  if (overlap(q_e4m3, nq, x_bf16, 2 * nx) || overlap(s, ns, x_bf16, 2 * nx) ||
      overlap(q_e4m3, nq, s, ns) || overlap(q_e4m3, nq, row_of, 4 * P) ||
      overlap(s, ns, row_of, 4 * P))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_moe_quant_scatter(x_bf16, row_of, q_e4m3, s, T, topk, R, K,
                                                   scale_fmt == FP8BS_SCALE_UE8M0,
                                                   (hipStream_t)stream));
}

int fp8bs_moe_combine(const void* out_bf16, const float* w, const int32_t* row_of, void* y,
                      int64_t T, int64_t topk, int64_t R, int64_t N, int out_dtype, void* stream) {
  if (T < 0 || topk < 1 || R < 0 || N < 0) return FP8BS_ERR_SHAPE;
  if (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_F32) return FP8BS_ERR_ENUM;
  const int64_t no = mul(R, N), ny = mul(T, N), P = mul(T, topk);
  if (no < 0 || ny < 0 || P < 0 || P > kLimitInt || mul(no, 2) < 0 || mul(ny, 4) < 0 ||
      R > kLimitInt)
    return FP8BS_ERR_SHAPE;
  if (ny == 0) return FP8BS_OK;
  if (!w || !row_of || !y || (no > 0 && !out_bf16)) return FP8BS_ERR_NULL;
  if (!aligned(out_bf16, 16) || !aligned(y, 16) || !aligned(w, 4) || !aligned(row_of, 4))
    return FP8BS_ERR_ALIGN;
  const int64_t yb = ny * (out_dtype == FP8BS_OUT_F32 ? 4 : 2);
  if (overlap(y, yb, out_bf16, 2 * no) || overlap(y, yb, w, 4 * P) || overlap(y, yb, row_of, 4 * P))
    return FP8BS_ERR_ALIAS;
  return status_of(fp8bs::launch_moe_combine(out_bf16, w, row_of, y, T, topk, R, N,
                                             out_dtype == FP8BS_OUT_F32, (hipStream_t)stream));
}

}  // extern "C"
