// device_common.h -- small gfx950 device helpers shared by the HIP kernels of
// the block-scaled FP8 library.  CDNA4 only: 64-lane wavefronts, OCP E4M3
// conversions in hardware, fp8 MFMA with K = 128.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

constexpr int kBlock = 128;          // quantisation block edge (1x128 and 128x128)
constexpr float kE4m3Max = 448.0f;   // largest finite e4m3fn magnitude
constexpr float kAmaxFloor = 1e-4f;  // amax floor of the scale rule

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bits_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t f32_bits(float f) { return __float_as_uint(f); }

// Streaming (read-once / write-once) memory accesses: the non-temporal hint
// keeps data that is not reused from displacing what is.  It pays where a
// store instruction writes whole cache lines (a wave's lanes covering
// contiguous bytes) or a load streams data read once: act_quant's input and
// codes, the MoE quant_scatter and combine, weight_dequant's output (after
// its lanes were remapped so each store writes 1 KB contiguous), the GEMM's
// bf16 C tile written as whole rows from LDS, the MLA key output staged the
// same way, and the weight DMA of the decode and small-expert MoE tiles.
// Where lanes write 8-16 bytes at a row stride (a store covering part of
// every line it touches) the hint made the stores several times slower, so
// such stores stay plain.  kNonTemporal is the cache-policy operand of the
// raw buffer load builtins (the `nt` bit on gfx950).
constexpr int kNonTemporal = 2;
template <typename T>
__device__ __forceinline__ void store_nt(T* p, const T& v);
template <>
__device__ __forceinline__ void store_nt<uint2>(uint2* p, const uint2& v) {
  __builtin_nontemporal_store(v.x, &((uint32_t*)p)[0]);
  __builtin_nontemporal_store(v.y, &((uint32_t*)p)[1]);
}
template <>
__device__ __forceinline__ void store_nt<uint4>(uint4* p, const uint4& v) {
  __builtin_nontemporal_store(v.x, &((uint32_t*)p)[0]);
  __builtin_nontemporal_store(v.y, &((uint32_t*)p)[1]);
  __builtin_nontemporal_store(v.z, &((uint32_t*)p)[2]);
  __builtin_nontemporal_store(v.w, &((uint32_t*)p)[3]);
}

// Two bf16 values packed in one dword -> two floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bits_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bits_f32(w & 0xFFFF0000u); }

// Maximum over the 16 lanes of a DPP row (lanes 16r .. 16r+15) of a
// non-negative float given as its bit pattern (unsigned order == float order
// for non-negative values).  Every lane of the row receives the result.
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xF, 0xF, false));  // row_ror 4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false));  // row_ror 8
  return v;
}

// Full-wave (64 lanes) maximum of a non-negative float bit pattern.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = row16_max_u32(v);
  v = max(v, (uint32_t)__shfl_xor((int)v, 16));
  v = max(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// Block scale: s = RN32(max(amax, 1e-4) / 448) with an IEEE division; for
// the ue8m0 format the smallest power of two >= s (s is always a normal
// number here, so bumping the exponent field is exact).
template <bool UE8M0>
__device__ __forceinline__ float block_scale(float amax) {
  float s = __fdiv_rn(fmaxf(amax, kAmaxFloor), kE4m3Max);
  if (UE8M0) {
    uint32_t u = f32_bits(s);
    if (u & 0x007FFFFFu) u = (u & 0xFF800000u) + 0x00800000u;
    s = bits_f32(u);
  }
  return s;
}

// Correctly rounded x / s (s > 0) given r = RN(1/s): Markstein's correction
// step.  q0 = RN(x*r) is within one ulp of x/s; the residual x - q0*s is exact
// in an FMA; RN(q0 + residual*r) is then the correctly rounded quotient
// (P. Markstein, IBM J. Res. Dev. 34(1), 1990; Muller et al., Handbook of
// Floating-Point Arithmetic, section on FMA-based division).  The correction
// turns a zero quotient of a negative x into +0 (fma(+0, r, -0) = +0); the
// IEEE quotient keeps the sign of x, so it is copied back.
__device__ __forceinline__ float div_markstein(float x, float s, float r) {
  float q0 = __fmul_rn(x, r);
  float e = __builtin_fmaf(-q0, s, x);
  return __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
}

// Four floats -> four e4m3 bytes (RNE), after clamping to [-448, 448], which
// makes out-of-range values saturate whatever the converter does with them.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -kE4m3Max, kE4m3Max);
  b = __builtin_amdgcn_fmed3f(b, -kE4m3Max, kE4m3Max);
  c = __builtin_amdgcn_fmed3f(c, -kE4m3Max, kE4m3Max);
  d = __builtin_amdgcn_fmed3f(d, -kE4m3Max, kE4m3Max);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);   // bytes 0,1
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);        // bytes 2,3
  return (uint32_t)w;
}

// Two floats -> packed bf16x2 (round to nearest even), low half = a.
// An fptrunc of a float pair to bf16, which gfx950 performs with one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2f f = {a, b};
  v2bf r = __builtin_convertvector(f, v2bf);
  return __builtin_bit_cast(uint32_t, r);
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// 8 e4m3 codes (two dwords, byte order = element order) times a block scale
// -> 8 bf16, with weight_dequant's rounding: the float32 product (exact
// decode, one RN32 multiply) then bf16 round-to-nearest-even.
__device__ __forceinline__ v8bf dequant8_bf16(uint32_t w0, uint32_t w1, float sc) {
  const v2f a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false);
  const v2f b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const v2f c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false);
  const v2f d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
  const v4u_t u = {pack2_bf16(__fmul_rn(a.x, sc), __fmul_rn(a.y, sc)),
                   pack2_bf16(__fmul_rn(b.x, sc), __fmul_rn(b.y, sc)),
                   pack2_bf16(__fmul_rn(c.x, sc), __fmul_rn(c.y, sc)),
                   pack2_bf16(__fmul_rn(d.x, sc), __fmul_rn(d.y, sc))};
  return __builtin_bit_cast(v8bf, u);
}

}  // namespace fp8bs
