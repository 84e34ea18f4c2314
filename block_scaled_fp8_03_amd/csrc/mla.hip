// mla.hip -- MLA "absorb" projections through an FP8 wkv_b for gfx950
// ("DeepSeek-V3 Administrator & Developer Guide" 8.3, steps 5 and 7: with the
// absorb attention, q_nope is carried into the latent space by the key rows of
// wkv_b, and the attention-weighted latent is turned into the head's values by
// its value rows; an FP8 wkv_b is dequantised by weight_dequant (8.5.2) before
// both einsums, on every forward step).  Here the weight is dequantised in
// registers with weight_dequant's rounding (float32 product, bf16 RNE) and
// multiplied on the bf16 MFMA with float32 accumulation; no bf16 copy of the
// weight is ever written.
//
// wkv_b [H*(dn+dv), R] e4m3 with 128x128 block scales [H*(dn+dv)/128, R/128];
// head h owns rows h(dn+dv) .. h(dn+dv)+dn-1 (key) and the dv rows after them
// (value).  dn, dv and R are multiples of 128, so every head's key and value
// rows start on a scale block.
//
//   key   out[t,h,c] = sum_{d<dn} q[t,h,d] Wd[h(dn+dv)+d, c]       c < R
//   value out[t,h,d] = sum_{c<R}  x[t,h,c] Wd[h(dn+dv)+dn+d, c]    d < dv
//
// MFMA: v_mfma_f32_16x16x32_bf16, D[16 x 16] = X[16 x 32] . Y[32 x 16].  Lane l
// supplies row l % 16 of X and column l % 16 of Y, each with 8 of the 32 K
// values chosen by l / 16 (any fixed choice works when both operands use it);
// the result lane l, register r is D[4 (l / 16) + r][l % 16].  In both kernels
// X is the weight and Y the activation, so a lane's results share one token.
//
// Both kernels are HBM-bound at every size (the weight is read once per
// T-chunk, the activations once, the outputs written once); the weight of a
// wave lives in registers for its whole T-chunk.
#include <algorithm>
#include <cstdint>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_bf16(v8bf x, v8bf y, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
}

__device__ __forceinline__ v8bf load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(p));
}

struct MlaParams {
  const uint16_t* in;     // q [.., dn] (key) or x [.., R] (value), bf16 bits
  const uint8_t* w;       // wkv_b e4m3 [H*(dn+dv), R]
  const float* ws;        // [H*(dn+dv)/128, R/128]
  void* out;              // key [T, H, R], value [T, H, dv]
  int T, H, dn, dv, R;
  int ld_t, ld_h;         // element strides of the input between tokens / heads
  int tch;                // tokens per workgroup (multiple of 16)
  int n_tch;              // number of token chunks
};

// ---------------------------------------------------------------------------
// Key side.  Wave = one head, 64 latent columns c0 .. c0+63, a chunk of tokens.
// The contraction runs over the weight's row index d, so the weight operand
// is read transposed: for K step s, lane (j = l % 16, g = l / 16) loads the
// dword at rows 32s + 8g + i (i = 0..7), columns c0 + 4j .. c0 + 4j + 3, and a
// byte transpose turns those 8 dwords into 4 fragments; fragment u holds
// column c0 + 4j + u over the 8 rows (K values 8g + i).  The MFMA row index
// of fragment u is j, so output register r of lane (g', t) is column
// c0 + 4 (4g' + r) + u = c0 + 16 g' + 4 r + u: across its four accumulators a
// lane owns the 16 consecutive columns c0 + 16 g' .. c0 + 16 g' + 15 of token t.
// ---------------------------------------------------------------------------

// 4 x 4 byte transpose: out[u] byte i = byte u of w[i]  (v_perm_b32: S1
// supplies bytes 0..3 of the selection, S0 bytes 4..7).
__device__ __forceinline__ void transpose4x4_b8(const uint32_t w[4], uint32_t o[4]) {
  const uint32_t a_lo = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);   // w0.0 w1.0 w0.1 w1.1
  const uint32_t a_hi = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);   // w0.2 w1.2 w0.3 w1.3
  const uint32_t b_lo = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
  const uint32_t b_hi = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
  o[0] = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u);
  o[1] = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
  o[2] = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
  o[3] = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
}

template <int DN, bool OUT_F32>
__global__ void __launch_bounds__(512) mla_key_kernel(MlaParams p) {
  constexpr int KS = DN / 32;                       // MFMA K steps
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int c0 = (blockIdx.y * (blockDim.x >> 6) + wave) * 64;
  if (c0 >= p.R) return;                            // no barriers in this kernel
  const int h = blockIdx.x % p.H;
  const int t_begin = (blockIdx.x / p.H) * p.tch;
  const int t_end = min(p.T, t_begin + p.tch);
  const int row0 = h * (p.dn + p.dv);

  // the first token tile's q is requested before the weight, so both round
  // trips overlap; inside the loop the next tile's q is requested before the
  // current tile's MFMAs
  auto load_q = [&](int t0, v8bf (&qf)[KS]) {
    const int tl = min(t0 + j, t_end - 1);          // rows past the end load a valid row
    const uint16_t* q = p.in + (size_t)tl * p.ld_t + (size_t)h * p.ld_h + 8 * g;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = load_bf16x8(q + 32 * s);
  };
  v8bf qcur[KS];
  load_q(t_begin, qcur);

  // weight fragments, dequantised once for the whole token chunk
  v8bf wf[KS][4];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const float sc = p.ws[((row0 + 32 * s) >> 7) * (p.R >> 7) + (c0 >> 7)];
    const uint8_t* base = p.w + (size_t)(row0 + 32 * s + 8 * g) * p.R + c0 + 4 * j;
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wd[i] = *reinterpret_cast<const uint32_t*>(base + (size_t)i * p.R);
    uint32_t lo[4], hi[4];
    transpose4x4_b8(wd, lo);
    transpose4x4_b8(wd + 4, hi);
#pragma unroll
    for (int u = 0; u < 4; ++u) wf[s][u] = dequant8_bf16(lo[u], hi[u], sc);
  }

  // The prefetch is unconditional (the last tile reloads itself) and the
  // stores below are not under a branch: otherwise the compiler's wait count,
  // merged over both paths, covers the loads just issued and the previous
  // tile's stores (vmcnt counts both), which serialises the q stream and the
  // output stream.
  const int t_last = t_begin + ((t_end - t_begin - 1) / 16) * 16;
  for (int t0 = t_begin; t0 < t_end; t0 += 16) {
    const int t = t0 + j;
    v8bf qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = qcur[s];
    load_q(min(t0 + 16, t_last), qcur);
    v4f acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = mfma_bf16(wf[s][u], qf[s], acc[u]);
    // Rows past the end loaded the last row's q, so their results equal that
    // row's: they are stored there (the same bytes twice), which keeps the
    // stores out of a branch.
    const int ts = min(t, t_end - 1);
    // lane (g, t) owns columns c0 + 16g + e, e = 4r + u
    const size_t o = ((size_t)ts * p.H + h) * p.R + c0 + 16 * g;
    if (OUT_F32) {
      float* out = reinterpret_cast<float*>(p.out) + o;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        *reinterpret_cast<v4f*>(out + 4 * r) = v4f{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
    } else {
      uint16_t* out = reinterpret_cast<uint16_t*>(p.out) + o;
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        const v4u v = {pack2_bf16(acc[0][r], acc[1][r]), pack2_bf16(acc[2][r], acc[3][r]),
                       pack2_bf16(acc[0][r + 1], acc[1][r + 1]), pack2_bf16(acc[2][r + 1], acc[3][r + 1])};
        *reinterpret_cast<v4u*>(out + 4 * r) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Value side.  Wave = one head, 32 value columns d0 .. d0+31 (two MFMA row
// tiles), a chunk of tokens.  The contraction runs along the weight's rows
// (c), so both operands are read straight: for each 64-wide slice s' of c,
// lane (j, g) loads the 16 weight bytes [64s' + 16g, +16) of row d0 + 16ct + j
// (K steps 2s' and 2s'+1 take bytes 0..7 and 8..15) and the 16 bf16 of x at
// the same c.  Output register r of lane (g', t) is column d0 + 16ct + 4g' + r.
// ---------------------------------------------------------------------------
// Two waves per SIMD: with the weight in registers (16 RK VGPRs) a third
// wave left the compiler too few registers for a tile's x fragments, and it
// loaded them one at a time with a full wait after each.
template <int RK, bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_value_kernel(MlaParams p) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int d0 = (blockIdx.y * (blockDim.x >> 6) + wave) * 32;
  if (d0 >= p.dv) return;                           // no barriers in this kernel
  const int h = blockIdx.x % p.H;
  const int t_begin = (blockIdx.x / p.H) * p.tch;
  const int t_end = min(p.T, t_begin + p.tch);
  const int vrow0 = h * (p.dn + p.dv) + p.dn + d0;  // first weight row of the wave

  // x is not prefetched across token tiles: with the weight in registers a
  // second x buffer would leave one wave per SIMD, which measured slower
  auto load_x = [&](int t0, v8bf (&xf)[RK][2]) {
    const int tl = min(t0 + j, t_end - 1);          // rows past the end load a valid row
    const uint16_t* x = p.in + (size_t)tl * p.ld_t + (size_t)h * p.ld_h + 16 * g;
#pragma unroll
    for (int s = 0; s < RK; ++s) {
      xf[s][0] = load_bf16x8(x + 64 * s);
      xf[s][1] = load_bf16x8(x + 64 * s + 8);
    }
  };

  v8bf wf[2][RK][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const uint8_t* base = p.w + (size_t)(vrow0 + 16 * ct + j) * p.R + 16 * g;
    const float* sc = p.ws + (size_t)(vrow0 >> 7) * (p.R >> 7);
#pragma unroll
    for (int s = 0; s < RK; ++s) {
      const v4u wv = *reinterpret_cast<const v4u*>(base + 64 * s);
      const float scale = sc[s >> 1];
      wf[ct][s][0] = dequant8_bf16(wv.x, wv.y, scale);
      wf[ct][s][1] = dequant8_bf16(wv.z, wv.w, scale);
    }
  }

  for (int t0 = t_begin; t0 < t_end; t0 += 16) {
    const int t = t0 + j;
    v8bf xf[RK][2];
    load_x(t0, xf);
    // all of the tile's x loads are issued before the first MFMA (otherwise
    // the scheduler pairs each load with its MFMA, two loads in flight)
    __builtin_amdgcn_sched_barrier(0);
    v4f acc[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct][0] = acc[ct][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < RK; ++s)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[ct][k] = mfma_bf16(wf[ct][s][k], xf[s][k], acc[ct][k]);
    const int ts = min(t, t_end - 1);                   // as in the key kernel
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const v4f v = acc[ct][0] + acc[ct][1];
      const size_t o = ((size_t)ts * p.H + h) * p.dv + d0 + 16 * ct + 4 * g;
      if (OUT_F32) {
        *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + o) = v;
      } else {
        typedef uint32_t v2u __attribute__((ext_vector_type(2)));
        *reinterpret_cast<v2u*>(reinterpret_cast<uint16_t*>(p.out) + o) =
            v2u{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
      }
    }
  }
}

// Token chunking: at most 256 tokens per workgroup, evenly split, a multiple
// of 16.
void chunk_tokens(MlaParams& p) {
  p.n_tch = std::max(1, (p.T + 255) / 256);
  const int per = (p.T + p.n_tch - 1) / p.n_tch;
  p.tch = (per + 15) / 16 * 16;
  p.n_tch = (p.T + p.tch - 1) / p.tch;
}

}  // namespace

hipError_t launch_mla_absorb_key(const void* q, int64_t ld_t, int64_t ld_h, const void* w,
                                 const float* ws, void* out, int64_t T, int64_t H, int64_t dn,
                                 int64_t dv, int64_t R, bool out_f32, hipStream_t stream) {
  MlaParams p{static_cast<const uint16_t*>(q), static_cast<const uint8_t*>(w), ws, out, (int)T,
              (int)H, (int)dn, (int)dv, (int)R, (int)ld_t, (int)ld_h, 0, 0};
  chunk_tokens(p);
  // above 64 tokens one workgroup per (head, token chunk) covers up to 512
  // latent columns, so the chunk's q rows are read once and shared by its
  // waves (4096 tokens: 265 -> 248 us); at decode sizes four-wave workgroups
  // spread the weight over more CUs
  const int waves = T > 64 ? (int)std::min<int64_t>(8, R / 64) : 4;
  const dim3 grid((unsigned)(H * p.n_tch), (unsigned)((R / 64 + waves - 1) / waves));
  const dim3 block(64 * waves);
  if (dn == 128) {
    if (out_f32) hipLaunchKernelGGL((mla_key_kernel<128, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla_key_kernel<128, false>), grid, block, 0, stream, p);
  } else {
    if (out_f32) hipLaunchKernelGGL((mla_key_kernel<256, true>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((mla_key_kernel<256, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_mla_absorb_value(const void* x, int64_t ld_t, int64_t ld_h, const void* w,
                                   const float* ws, void* out, int64_t T, int64_t H, int64_t dn,
                                   int64_t dv, int64_t R, bool out_f32, hipStream_t stream) {
  MlaParams p{static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w), ws, out, (int)T,
              (int)H, (int)dn, (int)dv, (int)R, (int)ld_t, (int)ld_h, 0, 0};
  chunk_tokens(p);
  // one wave per workgroup when few tokens (more workgroups to spread the
  // weight over the CUs); four (one head's 128 value columns) otherwise, so
  // the waves that read the same x rows share a CU
  const int waves = T <= 64 ? 1 : 4;
  const dim3 grid((unsigned)(H * p.n_tch), (unsigned)((dv / 32 + waves - 1) / waves));
  const dim3 block(64 * waves);
#define FP8BS_MLA_V(RK_)                                                                       \
  case RK_:                                                                                    \
    if (out_f32) hipLaunchKernelGGL((mla_value_kernel<RK_, true>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((mla_value_kernel<RK_, false>), grid, block, 0, stream, p);        \
    break;
  switch (R / 64) {
    FP8BS_MLA_V(2)
    FP8BS_MLA_V(4)
    FP8BS_MLA_V(6)
    FP8BS_MLA_V(8)
    default: return hipErrorInvalidValue;
  }
#undef FP8BS_MLA_V
  return hipGetLastError();
}

}  // namespace fp8bs
