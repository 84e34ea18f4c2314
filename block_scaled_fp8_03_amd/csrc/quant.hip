// quant.hip -- block quantisation kernels for gfx950:
//   act_quant      1 x 128 activation blocks -> e4m3 + float32 scale
//                  ("DeepSeek-V3 Administrator & Developer Guide" 8.5.1;
//                  ue8m0 per the "DeepSeek-V3 User Guide" FAQ)
//   weight_quant   128 x 128 weight blocks, same rule (scale layout of
//                  Admin guide 6.3)
//   weight_dequant e4m3 x block scale -> bf16 (Admin guide 8.5.2)
// All three are HBM-streaming kernels: every lane moves 16-byte vectors,
// a 16-lane DPP row owns one 128-element activation block, and the per-block
// reductions stay inside registers.
#include "device_common.h"
#include "launch.h"

namespace fp8bs {

// ----------------------------------------------------------------------------
// act_quant
// ----------------------------------------------------------------------------
// The input is a flat sequence of 128-element blocks (K % 128 == 0, row-major),
// and block b's scale lives at s[b] ([M, K/128] row-major is that order).
// A 16-lane row handles one block: lane i holds elements 8i .. 8i+7 (16 bytes
// of bf16) and writes their 8 e4m3 bytes.  A workgroup of THREADS threads
// covers THREADS / 16 blocks per pass and PASSES passes, all loads issued
// before any use.  Two launch shapes, by size (graph-replayed back-to-back
// launches over inputs rotated past the Infinity Cache, same box, us):
//   256 threads x 2 passes: 1024 x 7168 ue8m0 5.87, 32 x 7168 2.13 -- best
//     on the small launches (a device copy of the same bytes: 6.34, 2.05);
//   64 threads x 4 passes: 4096 x 7168 17.9 (256 x 2: 19.7), 4096 x 18432
//     38.0 (42.3), 32768 x 2048 34.3 (37.2) -- best on the streaming ones
//     (128 x 4, 256 x 4 within 2%; 256 x 1 and 128 x 2 slower).
// Inputs of at least kAqLargeElems elements take the second shape.
constexpr int kAqThreads = 256;
constexpr int kAqPasses = 2;
constexpr int kAqBlocksPerWg = (kAqThreads / 16) * kAqPasses;
constexpr int kAqLargeThreads = 64;
constexpr int kAqLargePasses = 4;
constexpr int64_t kAqLargeElems = (int64_t)16 << 20;

// SCATTER: x is the token matrix [T, K] and the codes and scale of token t's
// block j go to every row r = row_of[t * topk + k] (k < topk, 0 <= r < R) of
// q [R, K] / s [R, K/128] instead of to row t -- the expert inputs of the MoE
// dispatch (quantisation is row local, so this equals quantising the
// gathered rows).
template <bool UE8M0, bool SCATTER, int THREADS, int PASSES>
__global__ __launch_bounds__(THREADS) void act_quant_kernel(const uint4* __restrict__ x,
                                                               uint2* __restrict__ q,
                                                               float* __restrict__ s,
                                                               int64_t nblocks,
                                                               const int32_t* __restrict__ row_of,
                                                               int topk, int64_t nb, int64_t R) {
  constexpr int BPW = (THREADS / 16) * PASSES;             // blocks per workgroup
  const int lane16 = threadIdx.x & 15;
  const int row = threadIdx.x >> 4;
  const int64_t wg_first = (int64_t)blockIdx.x * BPW;
  const int64_t first = wg_first + row;
  // Loads through a buffer resource over this workgroup's blocks: blocks past
  // the end read zeros without a branch, so all passes' loads are in flight
  // together (bounds checks under branches had made the compiler wait for the
  // first two before issuing the rest).
  const int64_t wg_blocks = min<int64_t>(nblocks - wg_first, BPW);
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(x + wg_first * 16), (short)0, (int)(uint32_t)(wg_blocks * 256), 0x00020000);
  uint4 v[PASSES];
#pragma unroll
  for (int u = 0; u < PASSES; ++u) {
    const uint32_t off = (uint32_t)(((row + u * (THREADS / 16)) * 16 + lane16) * 16);
    v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kNonTemporal));
  }
#pragma unroll
  for (int u = 0; u < PASSES; ++u) {
    const int64_t b = first + u * (THREADS / 16);
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = max(m, f32_bits(f[i]) & 0x7FFFFFFFu);
    m = row16_max_u32(m);                      // amax of the whole 128-block
    const float sc = block_scale<UE8M0>(bits_f32(m));
    const float r = __fdiv_rn(1.0f, sc);
    uint2 o;
    o.x = pack4_e4m3(div_markstein(f[0], sc, r), div_markstein(f[1], sc, r),
                     div_markstein(f[2], sc, r), div_markstein(f[3], sc, r));
    o.y = pack4_e4m3(div_markstein(f[4], sc, r), div_markstein(f[5], sc, r),
                     div_markstein(f[6], sc, r), div_markstein(f[7], sc, r));
    if (b < nblocks) {
      if (!SCATTER) {
        store_nt(q + b * 16 + lane16, o);
        if (lane16 == 0) s[b] = sc;
      } else {
        // the token's routed rows, up to 8 read together, then the stores
        const int64_t t = b / nb, j = b - t * nb;
        for (int k0 = 0; k0 < topk; k0 += 8) {
          int32_t rr[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) rr[k] = row_of[t * topk + min(k0 + k, topk - 1)];
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int64_t r = rr[k];
            if (k0 + k >= topk || r < 0 || r >= R) continue;
            store_nt(q + (r * nb + j) * 16 + lane16, o);
            if (lane16 == 0) s[r * nb + j] = sc;
          }
        }
      }
    }
  }
}

// The grid is one-dimensional: at most 2^32 - 1 threads per launch.  The
// 256 x 2 shape takes the most threads per block (8), so its limit,
// nblocks <= floor((2^32 - 1) / 256) * 32, holds for both shapes.
bool act_quant_fits(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0) return true;
  const int64_t max_wg = (((int64_t)1 << 32) - 1) / kAqThreads;
  const int64_t nb = K / kBlock;
  return rows <= max_wg * kAqBlocksPerWg / nb;
}

// One launch of the kernel for nblocks blocks of x (T token rows for SCATTER).
template <bool UE8M0, bool SCATTER>
void launch_aq(const void* x, void* q, float* s, int64_t nblocks, const int32_t* row_of, int topk,
               int64_t nb, int64_t R, hipStream_t stream) {
  if (nblocks * kBlock >= kAqLargeElems) {
    constexpr int BPW = (kAqLargeThreads / 16) * kAqLargePasses;
    const int64_t grid = (nblocks + BPW - 1) / BPW;
    act_quant_kernel<UE8M0, SCATTER, kAqLargeThreads, kAqLargePasses>
        <<<dim3((unsigned)grid), dim3(kAqLargeThreads), 0, stream>>>((const uint4*)x, (uint2*)q, s, nblocks,
                                                                     row_of, topk, nb, R);
  } else {
    const int64_t grid = (nblocks + kAqBlocksPerWg - 1) / kAqBlocksPerWg;
    act_quant_kernel<UE8M0, SCATTER, kAqThreads, kAqPasses>
        <<<dim3((unsigned)grid), dim3(kAqThreads), 0, stream>>>((const uint4*)x, (uint2*)q, s, nblocks,
                                                                row_of, topk, nb, R);
  }
}

hipError_t launch_act_quant(const void* x, void* q, float* s, int64_t M, int64_t K, bool ue8m0,
                            hipStream_t stream) {
  const int64_t nblocks = M * (K / kBlock);
  if (nblocks == 0) return hipSuccess;
  if (!act_quant_fits(M, K)) return hipErrorInvalidConfiguration;
  if (ue8m0) launch_aq<true, false>(x, q, s, nblocks, nullptr, 0, 0, 0, stream);
  else launch_aq<false, false>(x, q, s, nblocks, nullptr, 0, 0, 0, stream);
  return hipGetLastError();
}

hipError_t launch_moe_quant_scatter(const void* x, const int32_t* row_of, void* q, float* s,
                                    int64_t T, int64_t topk, int64_t R, int64_t K, bool ue8m0,
                                    hipStream_t stream) {
  const int64_t nb = K / kBlock;
  const int64_t nblocks = T * nb;
  if (nblocks == 0 || R == 0) return hipSuccess;
  if (!act_quant_fits(T, K)) return hipErrorInvalidConfiguration;
  if (ue8m0) launch_aq<true, true>(x, q, s, nblocks, row_of, (int)topk, nb, R, stream);
  else launch_aq<false, true>(x, q, s, nblocks, row_of, (int)topk, nb, R, stream);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// e4m3_encode: the float32 -> e4m3 step of act_quant and weight_quant alone
// ----------------------------------------------------------------------------
// q[i] = pack4_e4m3's encoding of x[i]: clamp to [-448, 448], then the
// hardware conversion (round to nearest, ties to even).  Thread t encodes
// x[4t .. 4t+3] with one 16-byte load and one 4-byte store; a partial last
// group goes element by element.
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ x,
                                                          uint8_t* __restrict__ q, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    const float4 v = *(const float4*)(x + i);
    *(uint32_t*)(q + i) = pack4_e4m3(v.x, v.y, v.z, v.w);
  } else if (i < n) {
    for (int64_t k = i; k < n; ++k) q[k] = (uint8_t)(pack4_e4m3(x[k], 0.0f, 0.0f, 0.0f) & 0xFFu);
  }
}

bool e4m3_encode_fits(int64_t n) {
  return n <= ((((int64_t)1 << 32) - 1) / 256) * 256 * 4;
}

hipError_t launch_e4m3_encode(const float* x, void* q, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  if (!e4m3_encode_fits(n)) return hipErrorInvalidConfiguration;
  const int64_t grid = (n + 1023) / 1024;
  e4m3_encode_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(x, (uint8_t*)q, n);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// weight_quant: one 256-thread workgroup per 128 x 128 block.  Thread t owns
// row t/2 and the 64 columns (t%2)*64 .. +63 of the block.
// ----------------------------------------------------------------------------
__device__ __forceinline__ float block_amax_256(uint32_t m, uint32_t* red) {
  m = wave_max_u32(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  return bits_f32(m);
}

// UE8M0: power-of-two block scales (act_quant's ue8m0 rule per 128 x 128
// block), a harness option for the ue8m0 fast path of the GEMM.
template <bool UE8M0>
__global__ __launch_bounds__(256) void weight_quant_kernel(const uint16_t* __restrict__ w,
                                                           uint8_t* __restrict__ q,
                                                           float* __restrict__ s, int64_t N,
                                                           int64_t K) {
  __shared__ uint32_t red[4];
  const int64_t bk = blockIdx.x, bn = blockIdx.y;
  const int64_t nbk = (K + kBlock - 1) / kBlock;
  const int64_t n = bn * kBlock + (threadIdx.x >> 1);
  const int64_t k0 = bk * kBlock + (threadIdx.x & 1) * 64;
  const bool full = (bn + 1) * kBlock <= N && (bk + 1) * kBlock <= K && (K % 16) == 0;
  if (full) {
    // Interior block with 16-byte aligned rows: vector path.
    const uint4* src = (const uint4*)(w + n * K + k0);
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = src[i];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t ws[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        m = max(m, max(f32_bits(bf16_lo(ws[j])) & 0x7FFFFFFFu, f32_bits(bf16_hi(ws[j])) & 0x7FFFFFFFu));
    }
    const float sc = block_scale<UE8M0>(block_amax_256(m, red));
    const float r = __fdiv_rn(1.0f, sc);
    uint4* dst = (uint4*)(q + n * K + k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a[4] = {v[2 * i].x, v[2 * i].y, v[2 * i].z, v[2 * i].w};
      const uint32_t b[4] = {v[2 * i + 1].x, v[2 * i + 1].y, v[2 * i + 1].z, v[2 * i + 1].w};
      uint4 o;
      o.x = pack4_e4m3(div_markstein(bf16_lo(a[0]), sc, r), div_markstein(bf16_hi(a[0]), sc, r),
                       div_markstein(bf16_lo(a[1]), sc, r), div_markstein(bf16_hi(a[1]), sc, r));
      o.y = pack4_e4m3(div_markstein(bf16_lo(a[2]), sc, r), div_markstein(bf16_hi(a[2]), sc, r),
                       div_markstein(bf16_lo(a[3]), sc, r), div_markstein(bf16_hi(a[3]), sc, r));
      o.z = pack4_e4m3(div_markstein(bf16_lo(b[0]), sc, r), div_markstein(bf16_hi(b[0]), sc, r),
                       div_markstein(bf16_lo(b[1]), sc, r), div_markstein(bf16_hi(b[1]), sc, r));
      o.w = pack4_e4m3(div_markstein(bf16_lo(b[2]), sc, r), div_markstein(bf16_hi(b[2]), sc, r),
                       div_markstein(bf16_lo(b[3]), sc, r), div_markstein(bf16_hi(b[3]), sc, r));
      dst[i] = o;
    }
    if (threadIdx.x == 0) s[bn * nbk + bk] = sc;
  } else {
    // Edge block or unaligned rows: element by element, masked.
    uint32_t m = 0;
    if (n < N)
      for (int j = 0; j < 64; ++j)
        if (k0 + j < K) m = max(m, f32_bits(bf16_lo(w[n * K + k0 + j])) & 0x7FFFFFFFu);
    const float sc = block_scale<UE8M0>(block_amax_256(m, red));
    const float r = __fdiv_rn(1.0f, sc);
    if (n < N)
      for (int j = 0; j < 64; j += 4) {
        float f[4];
        for (int t = 0; t < 4; ++t)
          f[t] = (k0 + j + t < K) ? div_markstein(bf16_lo(w[n * K + k0 + j + t]), sc, r) : 0.0f;
        const uint32_t o = pack4_e4m3(f[0], f[1], f[2], f[3]);
        for (int t = 0; t < 4; ++t)
          if (k0 + j + t < K) q[n * K + k0 + j + t] = (uint8_t)(o >> (8 * t));
      }
    if (threadIdx.x == 0) s[bn * nbk + bk] = sc;
  }
}

hipError_t launch_weight_quant(const void* w, void* q, float* s, int64_t N, int64_t K, bool ue8m0,
                               hipStream_t stream) {
  if (N == 0 || K == 0) return hipSuccess;
  const int64_t nbn = (N + kBlock - 1) / kBlock, nbk = (K + kBlock - 1) / kBlock;
  if (ue8m0)
    weight_quant_kernel<true><<<dim3((unsigned)nbk, (unsigned)nbn), dim3(256), 0, stream>>>(
        (const uint16_t*)w, (uint8_t*)q, s, N, K);
  else
    weight_quant_kernel<false><<<dim3((unsigned)nbk, (unsigned)nbn), dim3(256), 0, stream>>>(
        (const uint16_t*)w, (uint8_t*)q, s, N, K);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// weight_dequant
// ----------------------------------------------------------------------------
// Vector path (K % 16 == 0): a one-dimensional grid of ceil(N / kDqRows) x
// ceil(K / 1024) workgroups, the column span fastest (bx = span, by = row
// group).  Wave w converts row by*kDqRows + w over 1024 columns; lane l takes
// the 8-column chunks bx*128 + l and bx*128 + l + 64 (8 e4m3 bytes in, 16 bf16 bytes out; a
// chunk never straddles a 128-column scale block).  Each of a wave's two
// 16-byte stores then writes 1 KB of contiguous output, whole cache lines;
// the earlier mapping (one 16-byte load and two 16-byte stores per lane for
// 16 consecutive columns) left every store instruction writing half of each
// line it touched.  The stores carry the non-temporal hint.  N x 7168 with
// two weights in rotation, same box, us (before / remap / remap + hint):
// N = 4096 15.4 / 14.1 / 13.9, 9216 38.8 / 35.8 / 29.7, 16384 63.3 / 60.1 /
// 52.5, 18432 70.8 / 67.7 / 59.2, 36864 137.7 / 133.0 / 129.3; non-temporal
// loads as well cost (18432: 62.3).  Four rows per workgroup (one per wave)
// measured fastest in the earlier mapping: 82.5 / 76.1 / 71.0 us at 16 / 8 /
// 4 rows, 86.6 at 32.
constexpr int kDqRows = 4;

__global__ __launch_bounds__(64 * kDqRows) void weight_dequant_kernel(const uint2* __restrict__ w,
                                                                      const float* __restrict__ s,
                                                                      uint4* __restrict__ y,
                                                                      int64_t N, int64_t K) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t kc8 = K / 8;                                 // 8-column chunks per row
  const int64_t spans = (kc8 + 127) / 128;
  const int64_t c0 = ((int64_t)blockIdx.x % spans) * 128 + lane;
  const int64_t n = ((int64_t)blockIdx.x / spans) * kDqRows + wave;
  if (c0 >= kc8 || n >= N) return;
  const bool has1 = c0 + 64 < kc8;
  const int64_t nbk = (K + kBlock - 1) / kBlock;
  const float* srow = s + (n / kBlock) * nbk;
  const uint2 v0 = w[n * kc8 + c0];
  const uint2 v1 = has1 ? w[n * kc8 + c0 + 64] : make_uint2(0, 0);
  const float s0 = srow[(c0 * 8) / kBlock];
  const float s1 = has1 ? srow[((c0 + 64) * 8) / kBlock] : 0.0f;
  const uint4 o0 = __builtin_bit_cast(uint4, dequant8_bf16(v0.x, v0.y, s0));
  const uint4 o1 = __builtin_bit_cast(uint4, dequant8_bf16(v1.x, v1.y, s1));
  store_nt(y + n * kc8 + c0, o0);
  if (has1) store_nt(y + n * kc8 + c0 + 64, o1);
}

// Generic path (any K): one element per thread.
__global__ __launch_bounds__(256) void weight_dequant_scalar_kernel(const uint8_t* __restrict__ w,
                                                                    const float* __restrict__ s,
                                                                    uint16_t* __restrict__ y,
                                                                    int64_t N, int64_t K) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * K) return;
  const int64_t n = i / K, k = i % K;
  const int64_t nbk = (K + kBlock - 1) / kBlock;
  const v2f f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
  const float p = __fmul_rn(f.x, s[(n / kBlock) * nbk + k / kBlock]);
  y[i] = (uint16_t)(pack2_bf16(p, 0.0f) & 0xFFFFu);
}

// Both grids are one-dimensional: at most 2^32 - 1 threads.
bool weight_dequant_fits(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return true;
  const int64_t limit = ((int64_t)1 << 32) - 1;
  if (K % 16 == 0) {
    const int64_t spans = (K / 8 + 127) / 128, groups = (N + kDqRows - 1) / kDqRows;
    return groups <= limit / (64 * kDqRows) / spans;
  }
  return N <= (limit - 255) / K;
}

hipError_t launch_weight_dequant(const void* w, const float* s, void* y, int64_t N, int64_t K,
                                 hipStream_t stream) {
  if (N == 0 || K == 0) return hipSuccess;
  if (!weight_dequant_fits(N, K)) return hipErrorInvalidConfiguration;
  if (K % 16 == 0) {
    const int64_t spans = (K / 8 + 127) / 128, groups = (N + kDqRows - 1) / kDqRows;
    const dim3 grid((unsigned)(spans * groups)), block(64 * kDqRows);
    weight_dequant_kernel<<<grid, block, 0, stream>>>((const uint2*)w, s, (uint4*)y, N, K);
  } else {
    const int64_t grid = (N * K + 255) / 256;
    weight_dequant_scalar_kernel<<<dim3((unsigned)grid), dim3(256), 0, stream>>>(
        (const uint8_t*)w, s, (uint16_t*)y, N, K);
  }
  return hipGetLastError();
}

}  // namespace fp8bs
