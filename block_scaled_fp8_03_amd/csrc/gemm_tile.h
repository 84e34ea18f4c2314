// gemm_tile.h -- pieces shared by the FP8 tile kernels (gemm.hip, gemm_e8.hip):
// the MFMA and DMA helpers, the kernel parameters, the tile order, the LDS
// swizzle and the staged bf16 epilogue.  The orientation and operand layout
// of the MFMA are described at the top of gemm.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "device_common.h"

namespace fp8bs {

// One K = 128 FP8 MFMA with a zero accumulator.  With all scale operands 0
// the compiler emits the unscaled v_mfma_f32_16x16x128_f8f6f4, which computes
// the plain product and issues faster than the scaled encoding (measured on
// gfx950: ~10% more MFMA throughput).
__device__ __forceinline__ v4f mfma_k128(v8i x, v8i y) {
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(x, y, z, 0, 0, 0, 0, 0, 0);
}

// s_waitcnt that waits until at most n vector-memory operations of this wave
// are outstanding (gfx9 encoding: vmcnt split over bits 3:0 and 15:14;
// expcnt and lgkmcnt left at their "no wait" maxima).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that orders LDS accesses only (global memory traffic in
// flight, e.g. prefetches, is not waited for).
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 128-bit buffer resource for raw (untyped) loads of `bytes` bytes from
// `base`; loads at offsets >= bytes return zeros instead of faulting.
typedef int v4i __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  v4i r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xFFFFu));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = 0x00020000;                                                   // 32-bit data format
  return r;
}

// Direct buffer -> LDS loads: lane i's bytes land at LDS address
// lds + size * i.  Written as inline assembly so the compiler does not treat
// every later LDS read as dependent on every load in flight; completion is
// tracked explicitly with wait_vmcnt() before the barrier that publishes a
// stage.  The LDS address is wave-uniform (it goes to M0); readfirstlane
// keeps it in an SGPR whatever register the compiler chose for it.
__device__ __forceinline__ void dma_b128(v4i rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory", "m0");
}
// The same with the non-temporal hint, for data read exactly once (the
// weight stream of the decode kernel): measured 27.4 vs 29.4 us on the
// decode-shaped GEMM.
__device__ __forceinline__ void dma_b128_nt(v4i rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(v4i rsrc, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc) : "memory", "m0");
}

// The loads above with a wave-uniform byte offset in the instruction's
// scalar offset field (and a non-temporal form of the 16-byte one): the K position of a tile's loads advances in an SGPR
// instead of one VALU add per load and K block.  Every such offset stays
// inside the row that `voff` addresses (or `voff` alone is already past the
// end of the buffer), so the range check zero-fills exactly the loads it did
// without the scalar offset.
__device__ __forceinline__ void dma_b128s(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
__device__ __forceinline__ void dma_b128s_nt(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32s(v4i rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :: "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(rsrc),
                  "s"(__builtin_amdgcn_readfirstlane(soff)) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// ----------------------------------------------------------------------------
// Tile kernel
// ----------------------------------------------------------------------------
// A workgroup of 4 waves computes a BM x BN tile of C (BM rows of A, BN rows
// of B); wave (wm, wn) computes a WM x WN sub-tile as (WN/16) x (WM/16) MFMA
// tiles.  Each K block moves through a ring of ST LDS stages:
//   stage = [A tile BM x 128 bytes][B tile BN x 128 bytes][a_s column, 256 floats]
//           [b_s of each wave's weight block, 4 x 64 floats]
// filled by direct buffer->LDS loads, so no VGPRs are spent on staging.
// Rows are 128 bytes, their 16-byte chunks permuted by an XOR swizzle of the
// row index (below) so the MFMA operand reads are free of bank conflicts.
// Rows past the end of an operand read as zeros (buffer range check) and
// their results are never stored.

struct GemmParams {
  const uint8_t* a;       // [rows, K] e4m3
  const float* a_s;       // [rows, K/128]
  const uint8_t* b;       // [N, K] or [E, N, K]
  const float* b_s;       // [ceil(N/128), K/128] or [E, ...]
  void* c;                // [rows, N]
  const int32_t* offsets; // MoE: [E+1] device row offsets
  int rows;               // M (dense) or R (MoE)
  int N, K;
  int E;                  // MoE experts
  int num_m;              // dense: m tiles
  int num_n;              // n tiles
  int n0;                 // dense: first output column of this launch's tiles (a multiple of 128)
  int small_bn;           // MoE: column width of the small-expert tiles (64, 128 or 256)
  int large_sh;           // MoE: log2 of the large-expert tiles' side (8: 256 x 256, 7: 128 x 128)
};

// Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
// that each XCD receives a contiguous range of logical tiles, which then
// share operands in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int q = total / 8, r = total % 8;
  const int x = id % 8, k = id / 8;
  return x * q + min(x, r) + k;
}

// LDS tiles hold 128-byte rows; the 16-byte chunk c of row r sits at chunk
// position c ^ swz(r).  Measured on gfx950, a ds_read_b128 is served in four
// cycles of 16 lanes -- the lanes of one half-wave with equal parity of lane
// bits 2..4 -- over 64 four-byte banks (one cycle per 256 bytes), so a cycle
// is conflict-free when its 16 lanes touch 16 distinct 16-byte positions
// modulo 256 bytes.  In the MFMA operand read, lane l takes row l % 16 and
// chunk 2 (l / 16) (+1), and
//   SW = 2: swz(r) = r1 | r2 << 2 (bits of r)
// makes every cycle conflict-free.  SW = 0 (swz(r) = r % 8) and SW = 1
// (swz(r) = (r / 2) % 8) leave two-way conflicts.  Each DMA instruction
// writes 8 whole rows (8 lanes per 128-byte row, contiguous in LDS), so
// global reads stay line-sized whatever the swizzle.
template <int SW>
__device__ __forceinline__ int swz(int r) {
  return SW == 0 ? (r & 7) : SW == 1 ? ((r >> 1) & 7) : (((r >> 1) & 1) | (r & 4));
}

// Row `r` of a tile, lane group g: the 32 bytes of logical chunks 2g and 2g+1
// (two 16-byte reads at their swizzled positions).
template <int SW>
__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int r, int g) {
  const int sw = swz<SW>(r);
  const uint4 lo = *(const uint4*)(tile + r * 128 + (((2 * g) ^ sw) << 4));
  const uint4 hi = *(const uint4*)(tile + r * 128 + (((2 * g + 1) ^ sw) << 4));
  v8i v;
  v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
  v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
  return v;
}

// bf16 C tile out through LDS.  Lane (r16, g) of wave (wm, wn) holds
// C[row][col .. col+3] for row = wm*WM + 16t + r16, col = wn*WN + 16j + 4g;
// written straight to global memory, each store instruction would cover 32
// bytes of each of 16 rows, a quarter of every line it touches.  Instead the
// tile goes into the (drained) stage buffers as BM rows of BN bf16, 16-byte
// chunk c of row r at c ^ (r mod 16) (conflict-free for both the 8-byte
// writes and the 16-byte reads), then every thread writes whole 16-byte
// chunks of consecutive columns, a wave covering whole rows, with the
// non-temporal hint.  Rows from m_end and columns from N are not stored
// (N % 8 == 0, so a chunk is all in or all out).  Same box, bit-identical
// outputs (us, before -> after): 4096x18432x7168 500 -> 491, 1024x16384x512
// 18.6 -> 15.7, MoE up / down 1050 / 1157 -> 1016 / 1114; the down GEMM
// 4096x7168x18432 unchanged (485.5 -> 485.1).  The caller guarantees that no
// wave still reads the stage buffers' operands (the barrier below) and that
// no DMA into them is in flight.
template <int BM, int BN, int WM, int WN, int NW, int MT, int NT>
__device__ __forceinline__ void store_c_tile_bf16(uint8_t* smem, const v4f (&acc)[NT][MT], int tid,
                                                  int wm, int wn, void* c_out, int N, int m_base,
                                                  int m_end, int n_base) {
  constexpr int CPRC = BN / 8;                                // 16-byte chunks per C row
  constexpr int SWM = CPRC >= 16 ? 15 : CPRC - 1;
  constexpr int PASSES = BM * CPRC / (NW * 64);
  static_assert((CPRC & (CPRC - 1)) == 0, "power-of-two row chunks");
  static_assert(BM * CPRC % (NW * 64) == 0, "whole passes");
  const int lane = tid & 63, g = lane >> 4, r16 = lane & 15;
  __syncthreads();
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = wm * WM + 16 * t + r16;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int c = (wn * WN + 16 * j) / 8 + (g >> 1);
      const uint32_t lo = pack2_bf16(acc[j][t][0], acc[j][t][1]);
      const uint32_t hi = pack2_bf16(acc[j][t][2], acc[j][t][3]);
      *(uint2*)(smem + row * (BN * 2) + ((c ^ (row & SWM)) << 4) + 8 * (g & 1)) = make_uint2(lo, hi);
    }
  }
  __syncthreads();
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int q = tid + ps * NW * 64;
    const int row = q / CPRC, c = q % CPRC;
    const int m = m_base + row, n = n_base + 8 * c;
    const uint4 v = *(const uint4*)(smem + row * (BN * 2) + ((c ^ (row & SWM)) << 4));
    if (m < m_end && n < N) store_nt((uint4*)((uint16_t*)c_out + (int64_t)m * N + n), v);
  }
}

// LDS bytes of one tile configuration (stages, a_s chunk buffers, dummy area).
template <int BM, int BN, int ST, int NW, bool ASCH>
constexpr int tile_lds_bytes() {
  return ST * (BM * 128 + BN * 128 + (ASCH ? 0 : NW * 256) + NW * 256) + (ASCH ? 2 * NW * 1024 : 0) +
         ((ASCH && ST > 2) ? 256 : 0);
}

// The ue8m0 main tile kernel (four waves, gemm_e8.hip): one launch of `grid`
// 256 x 256 tiles in the dense tile order.
hipError_t launch_gemm_e8_tile(const GemmParams& p, bool out_f32, int grid, hipStream_t stream);

}  // namespace fp8bs
