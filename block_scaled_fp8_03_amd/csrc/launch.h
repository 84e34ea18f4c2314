// launch.h -- internal kernel launchers (host side).  Arguments have been
// validated by the C ABI layer before these are called; each returns the
// hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

// Whether one act_quant (or moe_quant_scatter) launch covers `rows` rows of
// K columns (its grid's thread limit).
bool act_quant_fits(int64_t rows, int64_t K);
hipError_t launch_act_quant(const void* x, void* q, float* s, int64_t M, int64_t K, bool ue8m0,
                            hipStream_t stream);
// The float32 -> e4m3 conversion of act_quant / weight_quant on its own.
bool e4m3_encode_fits(int64_t n);
hipError_t launch_e4m3_encode(const float* x, void* q, int64_t n, hipStream_t stream);
hipError_t launch_weight_quant(const void* w, void* q, float* s, int64_t N, int64_t K, bool ue8m0,
                               hipStream_t stream);
// Whether one weight_dequant launch covers [N, K] (its grid's thread limit).
bool weight_dequant_fits(int64_t N, int64_t K);
hipError_t launch_weight_dequant(const void* w, const float* s, void* y, int64_t N, int64_t K,
                                 hipStream_t stream);
hipError_t launch_gemm(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
                       int64_t M, int64_t N, int64_t K, bool out_f32, hipStream_t stream);
hipError_t launch_moe_gemm(const void* a, const float* a_s, const void* b, const float* b_s,
                           const int32_t* offsets, void* c, int64_t R, int64_t E, int64_t N,
                           int64_t K, bool out_f32, hipStream_t stream);

hipError_t launch_gemm_ue8m0(const void* a, const float* a_s, const void* b, const float* b_s,
                             void* c, int64_t M, int64_t N, int64_t K, bool out_f32,
                             hipStream_t stream);
hipError_t launch_w8a16_gemm(const void* x, const void* w, const float* w_s, void* c, int64_t M,
                             int64_t N, int64_t K, bool out_f32, hipStream_t stream);
hipError_t launch_moe_quant_scatter(const void* x, const int32_t* row_of, void* q, float* s,
                                    int64_t T, int64_t topk, int64_t R, int64_t K, bool ue8m0,
                                    hipStream_t stream);
int64_t moe_route_workspace_bytes(int64_t T, int64_t topk, int64_t E);
hipError_t launch_moe_route(const int32_t* indices, int64_t T, int64_t topk, int64_t E,
                            int32_t* offsets, int32_t* row_token, int32_t* row_of, void* workspace,
                            hipStream_t stream);
// fp8bs_moe_route_noalloc: the count table in a file-scope device array of
// kRouteScratchBytes per GPU instead of a caller workspace.
constexpr int64_t kRouteScratchBytes = (int64_t)1 << 20;
hipError_t launch_moe_route_noalloc(const int32_t* indices, int64_t T, int64_t topk, int64_t E,
                                    int32_t* offsets, int32_t* row_token, int32_t* row_of,
                                    hipStream_t stream);
hipError_t launch_moe_combine(const void* out, const float* w, const int32_t* row_of, void* y,
                              int64_t T, int64_t topk, int64_t R, int64_t N, bool out_f32,
                              hipStream_t stream);
hipError_t launch_mla_absorb_key(const void* q, int64_t ld_t, int64_t ld_h, const void* w,
                                 const float* ws, void* out, int64_t T, int64_t H, int64_t dn,
                                 int64_t dv, int64_t R, bool out_f32, hipStream_t stream);
hipError_t launch_mla_absorb_value(const void* x, int64_t ld_t, int64_t ld_h, const void* w,
                                   const float* ws, void* out, int64_t T, int64_t H, int64_t dn,
                                   int64_t dv, int64_t R, bool out_f32, hipStream_t stream);

}  // namespace fp8bs
