// gemm_e8.hip -- the ue8m0 GEMM's main tile on four waves.  The FP8 GEMM of
// "DeepSeek-V3 Administrator & Developer Guide" 8.5.3 for operands whose
// block scales are all powers of two (the ue8m0 scale format of the
// "DeepSeek-V3 User Guide" FAQ): each K block's 128-wide products are scaled
// by the MFMA itself (v_mfma_scale_f32_16x16x128_f8f6f4 with the E8M0
// exponents of the activation row and the weight block) and accumulated in
// float32, K block after K block, so there is no VALU fold and no VALU
// instruction ever reads the accumulators before the epilogue: they can live
// in AGPRs, which VALU instructions cannot address.
//
// Layout.  A 256 x 256 tile of C per workgroup of four waves, one per SIMD;
// wave (wm, wn) owns rows 128 wm .. +127 and columns 128 wn .. +127, i.e. 8 x
// 8 MFMA tiles and 256 float32 accumulators per lane, which the compiler keeps
// in AGPRs.  Its 128 columns lie in one weight block, so one weight scale per
// K block.  Two LDS stages of [A 256 x 128 B][B 256 x 128 B][a_s][b_s], the
// same swizzled row layout, DMA and tile order as the eight-wave tile of
// gemm.hip (shared through gemm_tile.h), so the results are bit-identical to
// it: every accumulator sees the same MFMAs in the same K order.
//
// Schedule.  With one wave per SIMD, every wait of that wave idles the matrix
// pipe.  So the MFMAs of each K block's last CR row blocks are issued after
// the next workgroup barrier, from registers, and cover the reads of the new
// stage's weight fragments (reloaded one fragment at a time into the
// registers the carried MFMAs free) and the issue of the next stage's DMA.
// Same box, rounds alternating, weights resident, bit-identical outputs,
// against the eight-wave tile (us): 4096 x 18432 x 7168 423.6 -> 396.9,
// 4096 x 16384 x 7168 367.0 -> 346.2, 4096 x 7168 x 18432 424.9 -> 387.4;
// weights rotated over two copies: 439.5 -> 439.6, 367.4 -> 343.2,
// 439.6 -> 448.4.  Carrying 2 / 3 / 5 row blocks measured slower than 4, and
// one DMA part after every carried MFMA slower than two per weight fragment.
//
// This file is compiled without -amdgpu-mfma-vgpr-form (the rest of the
// GEMMs fold with VALU FMAs and keep their MFMA results in VGPRs).
#include <algorithm>
#include <cstdint>

#include "device_common.h"
#include "gemm_tile.h"

namespace fp8bs {

template <bool ASCH, bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_e8w4_kernel(GemmParams p) {
  constexpr int BM = 256, BN = 256, WM = 128, WN = 128, NW = 4, SW = 2, ST = 2;
  constexpr int MT = WM / 16, NT = WN / 16;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, BS_BYTES = NW * 256;
  constexpr int AS_BYTES = ASCH ? 0 : NW * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES;
  constexpr int A_LOADS = A_BYTES / (NW * 1024), B_LOADS = B_BYTES / (NW * 1024);
  constexpr int ASC = ASCH ? NW * 256 / BM : 1;
  constexpr int CHUNK_BYTES = ASCH ? NW * 1024 : 0;
  static_assert(MT == 8 && NT == 8, "shape");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<BM, BN, ST, NW, ASCH>() + 1024];

  int m_base, n_base;
  {
    const int t = xcd_remap(blockIdx.x, gridDim.x);
    constexpr int GM = 4;
    const int group = GM * p.num_n;
    const int gid = t / group, first_m = gid * GM;
    const int gsz = min(p.num_m - first_m, GM);
    const int in = t % group;
    m_base = (first_m + in % gsz) * BM;
    n_base = p.n0 + (in / gsz) * BN;
  }
  const int m_end = p.rows;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % 2, wn = wave / 2;
  const int K = p.K, N = p.N;
  const int nkb = K / 128;
  const int nbn = (N + 127) / 128;

  const v4i a_rsrc = make_rsrc(p.a, (uint32_t)((int64_t)p.rows * K));
  const v4i b_rsrc = make_rsrc(p.b, (uint32_t)((int64_t)N * K));
  const v4i as_rsrc = make_rsrc(p.a_s, (uint32_t)((int64_t)p.rows * nkb * 4));
  const v4i bs_rsrc = make_rsrc(p.b_s, (uint32_t)((int64_t)nbn * nkb * 4));
  const int lrow = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ swz<SW>(lrow);
  const uint32_t a_voff = (uint32_t)(m_base + lrow) * K + 16 * lchunk;
  const uint32_t b_voff = (uint32_t)(n_base + lrow) * K + 16 * lchunk;
  const uint32_t as_voff = (uint32_t)(m_base + (tid % BM)) * nkb * 4;
  const uint32_t bs_voff = (uint32_t)((n_base + wn * WN) / 128) * nkb * 4;
  const uint32_t rowstep = 8u * NW * (uint32_t)K;
  const uint32_t smem_lds = lds_addr(smem);
  constexpr int LPR = ASCH ? ASC / 4 : 1;
  const int as_idx = 64 * wave + lane;
  const uint32_t asc_voff = ((uint32_t)(m_base + as_idx / LPR) * nkb + 4 * (as_idx % LPR)) * 4;
  const uint32_t chunk_lds = smem_lds + ST * STAGE + wave * 1024;
  const uint32_t dummy_lds = smem_lds + tile_lds_bytes<BM, BN, ST, NW, ASCH>();

  // DMA part i of K block kb into stage st: A row group i (i < 8), B row
  // group i - 8 (i < 16), the activation scales (16), the weight block scale
  // (17).  Row group i is the 8 rows 8 (4 i + wave) .. +7 of the tile, lane
  // l taking row l / 8 and chunk (l % 8) ^ swz(row), as in gemm.hip.  When
  // a_s comes in chunks, the stages that start none load out of range into
  // a dummy area (zero-fill, no traffic), so the issue has no branch.
  constexpr int PARTS = A_LOADS + B_LOADS + 2;
  auto issue_part = [&](int kb, int st, int i) {
    const uint32_t base = smem_lds + st * STAGE + wave * 1024;
    const uint32_t koff = (uint32_t)kb * 128;
    if (i < A_LOADS) {
      dma_b128s(a_rsrc, base + i * NW * 1024, a_voff + i * rowstep, koff);
    } else if (i < A_LOADS + B_LOADS) {
      const int k = i - A_LOADS;
      dma_b128s(b_rsrc, base + A_BYTES + k * NW * 1024, b_voff + k * rowstep, koff);
    } else if (i == A_LOADS + B_LOADS) {
      if (ASCH) {
        const bool start = kb % ASC == 0;
        dma_b128s(as_rsrc, start ? chunk_lds + ((kb / ASC) & 1) * CHUNK_BYTES : dummy_lds,
                  start ? asc_voff : 0xF0000000u, start ? (uint32_t)kb * 4 : 0u);
      } else {
        dma_b32s(as_rsrc, smem_lds + st * STAGE + A_BYTES + B_BYTES + wave * 256, as_voff, (uint32_t)kb * 4);
      }
    } else {
      dma_b32s(bs_rsrc, smem_lds + st * STAGE + A_BYTES + B_BYTES + AS_BYTES + wave * 256, bs_voff,
               (uint32_t)kb * 4);
    }
  };

  v4f acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  const int g = lane >> 4, r16 = lane & 15;
  const int fsw = swz<SW>(r16);
  const uint32_t f_lo = r16 * 128 + (((2 * g) ^ fsw) << 4);
  const uint32_t f_hi = r16 * 128 + (((2 * g + 1) ^ fsw) << 4);
  const uint32_t a_lo = wm * WM * 128 + f_lo, a_hi = wm * WM * 128 + f_hi;
  const uint32_t b_lo = A_BYTES + wn * WN * 128 + f_lo, b_hi = A_BYTES + wn * WN * 128 + f_hi;
  const uint32_t as_lane = (uint32_t)(wm * WM + r16) * ASC * 4;

  auto frag = [&](const uint8_t* sb, uint32_t lo, uint32_t hi, int i) {
    const uint4 x = *(const uint4*)(sb + lo + i * 2048);
    const uint4 y = *(const uint4*)(sb + hi + i * 2048);
    v8i v;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
    return v;
  };
  // E8M0 exponent of this lane's activation row in row block t, and of the
  // wave's weight block
  auto ea_of = [&](int kb, const uint8_t* sb, int t) {
    const uint8_t* asb = (ASCH ? smem + ST * STAGE + ((kb / ASC) & 1) * CHUNK_BYTES : sb + A_BYTES + B_BYTES) +
                         as_lane + (ASCH ? (kb % ASC) * 4 : 0);
    return (int)(f32_bits(*(const float*)(asb + t * 16 * ASC * 4)) >> 23);
  };
  auto eb_of = [&](const uint8_t* sb) {
    return (int)(f32_bits(((const float*)(sb + A_BYTES + B_BYTES + AS_BYTES))[wave * 64]) >> 23);
  };

  // The last CR row blocks of each K block are carried past the next
  // barrier (their activation fragments ac and exponents eac in registers).
  constexpr int CR = 4;
  v8i bf[NT], ac[CR];
  int eac[CR], ebd = 0;
#pragma unroll
  for (int r = 0; r < CR; ++r) eac[r] = 0;

  // K block kb from stage kb % 2.  After the barrier: this K block's scale
  // exponents first (LDS reads return in order, so these never hold up an
  // MFMA), then for each weight fragment j the carried MFMAs of the previous
  // K block that read it, its reload with this K block's fragment j, and two
  // parts of the next K block's DMA; then row blocks 0 .. MT - CR - 1, each
  // reading the next row block's activation fragment ahead of its MFMAs.
  // The next K block's DMA goes into the other stage, whose last reads (the
  // carried fragments) completed before this barrier.  The last K block
  // reloads itself there (harmless: that stage is done with, and the loads
  // are waited for before the epilogue), which keeps the loop body one
  // basic block and the sched_barrier order intact.
  auto kblock = [&](int kb, bool carry) {
    wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* sb = smem + (kb & 1) * STAGE;
    int ea[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) ea[t] = ea_of(kb, sb, t);
    const int eb = eb_of(sb);
    v8i a_next = frag(sb, a_lo, a_hi, 0);
    const int kn = min(kb + 1, nkb - 1), sn = (kb + 1) & 1;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      if (carry) {
#pragma unroll
        for (int r = 0; r < CR; ++r)
          acc[j][MT - CR + r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], ac[r], acc[j][MT - CR + r], 0, 0, 0, ebd, 0, eac[r]);
      }
      __builtin_amdgcn_sched_barrier(0);
      bf[j] = frag(sb, b_lo, b_hi, j);
      __builtin_amdgcn_sched_barrier(0);
      issue_part(kn, sn, j);
      issue_part(kn, sn, A_LOADS + j);
      __builtin_amdgcn_sched_barrier(0);
    }
    issue_part(kn, sn, A_LOADS + B_LOADS);
    issue_part(kn, sn, A_LOADS + B_LOADS + 1);
#pragma unroll
    for (int t = 0; t < MT - CR; ++t) {
      const v8i a = a_next;
      a_next = frag(sb, a_lo, a_hi, t + 1);
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], a, acc[j][t], 0, 0, 0, eb, 0, ea[t]);
    }
    ac[0] = a_next;
#pragma unroll
    for (int r = 1; r < CR; ++r) ac[r] = frag(sb, a_lo, a_hi, MT - CR + r);
#pragma unroll
    for (int r = 0; r < CR; ++r) eac[r] = ea[MT - CR + r];
    ebd = eb;
  };

#pragma unroll
  for (int i = 0; i < PARTS; ++i) issue_part(0, 0, i);
  kblock(0, false);
  for (int kb = 1; kb < nkb; ++kb) kblock(kb, true);
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < CR; ++r)
      acc[j][MT - CR + r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], ac[r], acc[j][MT - CR + r], 0, 0, 0, ebd, 0, eac[r]);
  wait_vmcnt<0>();   // the last K block's reload into the other stage

  if constexpr (!OUT_F32) {
    if ((N & 7) == 0) {
      store_c_tile_bf16<BM, BN, WM, WN, NW, MT, NT>(smem, acc, tid, wm, wn, p.c, N, m_base, m_end, n_base);
      return;
    }
  }
  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m_base + wm * WM + 16 * t + r16;
    if (m >= m_end) continue;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int n = n_base + wn * WN + 16 * j + 4 * g;
      if (n >= N) continue;
      if (OUT_F32) {
        float* cp = (float*)p.c + (int64_t)m * N + n;
        if (vec_ok && n + 3 < N) {
          *(float4*)cp = make_float4(acc[j][t][0], acc[j][t][1], acc[j][t][2], acc[j][t][3]);
        } else {
          for (int r = 0; r < 4; ++r)
            if (n + r < N) cp[r] = acc[j][t][r];
        }
      } else {
        uint16_t* cp = (uint16_t*)p.c + (int64_t)m * N + n;
        const uint32_t lo = pack2_bf16(acc[j][t][0], acc[j][t][1]);
        const uint32_t hi = pack2_bf16(acc[j][t][2], acc[j][t][3]);
        if (vec_ok && n + 3 < N) {
          *(uint2*)cp = make_uint2(lo, hi);
        } else {
          const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
          for (int r = 0; r < 4; ++r)
            if (n + r < N) cp[r] = h[r];
        }
      }
    }
  }
}


hipError_t launch_gemm_e8_tile(const GemmParams& p, bool out_f32, int grid, hipStream_t stream) {
  // a_s in chunks of four K blocks (16 bytes per lane) needs K / 128 % 4 == 0
  // and 16-byte aligned rows
  const bool chunked = (p.K / 128) % 4 == 0 && ((uintptr_t)p.a_s & 15) == 0;
  const dim3 g((unsigned)grid), blk(256);
  if (chunked) {
    if (out_f32) gemm_e8w4_kernel<true, true><<<g, blk, 0, stream>>>(p);
    else gemm_e8w4_kernel<true, false><<<g, blk, 0, stream>>>(p);
  } else {
    if (out_f32) gemm_e8w4_kernel<false, true><<<g, blk, 0, stream>>>(p);
    else gemm_e8w4_kernel<false, false><<<g, blk, 0, stream>>>(p);
  }
  return hipGetLastError();
}

}  // namespace fp8bs
