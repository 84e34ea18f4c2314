// gemm.hip -- block-scaled FP8 GEMM kernels for gfx950 ("DeepSeek-V3
// Administrator & Developer Guide" 8.5.3: an FP8 tiled matmul with a float32
// accumulator, where each 128-wide K block's product is scaled by the row's
// activation scale and the weight block's scale before being added), and the
// grouped form used for the MoE experts (Admin guide 6.4).
//
// Orientation.  C = A . B^T with A [M, K] activations and B [N, K] weights.
// The MFMA computes D[16 x 16] = X[16 x 128] . Y[128 x 16] with X taken from
// the weights (rows = n) and Y from the activations (columns = m).  A lane
// then holds four consecutive n of one m: those four share one weight scale,
// so the scale applied to a lane's 16x16 partial is the single number
// a_s[m, kb] * b_s[n/128, kb].
//
// MFMA operand layout (v_mfma_scale_f32_16x16x128_f8f6f4, fp8 e4m3 operands,
// unit E8M0 scales): lane l supplies row (l % 16) of its operand and 32 of
// the 128 K bytes, chosen by l / 16.  A K-block's dot product is the same
// whichever 32 bytes each lane group carries, as long as both operands use
// the same choice, so lane group g carries K bytes [32g, 32g + 32).  The
// result lane l, register r is D[4 (l / 16) + r][l % 16].
#include <algorithm>
#include <cstdint>

#include "device_common.h"
#include "gemm_tile.h"
#include "launch.h"

namespace fp8bs {

// Activation scales.  With ASCH = false each stage carries the tile's a_s
// column for its K block, fetched as one float per row: a 64-byte memory
// request per row and K block.  With ASCH = true (needs K/128 % 4 == 0 and a
// 16-byte aligned a_s) the scales come in chunks of ASC = NW*256/BM
// consecutive K blocks, BM rows x ASC floats, loaded 16 bytes per lane
// (ASC/4 lanes per row) into one of two LDS chunk buffers.  Chunk c is issued
// together with the DMA of stage ASC*c, so it is complete whenever that stage
// is; it overwrites chunk c-2, whose last K block ASC*(c-1)-1 is finished by
// every wave once the barrier before that issue has passed (ASC >= ST - 1).
// Stages that start no chunk issue an out-of-range dummy load (no memory
// traffic) when ST > 2 so that every stage has the same number of DMA ops.
// OCC workgroups share a CU (register budget set for OCC * NW / 4 waves per SIMD).
// E8: every a_s and b_s value is a power of two; the MFMA applies them itself
// (v_mfma_scale_f32_16x16x128_f8f6f4 with each lane's E8M0 exponent: the
// weight block's for the weight operand, its activation row's for the other)
// and accumulates straight into the fp32 accumulators -- no VALU fold.
// One BM x BN tile of C: rows [m_base, m_base + BM) of A (results stored
// for rows < m_end) times rows [n_base, n_base + BN) of the weight B with
// block scales Bs.  `smem` is the workgroup's LDS, at least
// tile_lds_bytes<BM, BN, ST, NW, ASCH>() bytes, 1024-byte aligned.  Every
// wave of the workgroup calls it with the same arguments.
// NT_B: the weight DMA carries the non-temporal hint.
// HALF: the tile holds at most BM / 2 rows (rows [m_base + BM / 2, m_base +
// BM) are all past m_end).  Its waves are then laid out so that the two waves
// of a SIMD hold different m halves, and the waves of the second half skip
// every fragment read, MFMA and fold: they issue their share of the loads and
// meet every barrier, so each SIMD does the work of its one busy wave.
template <int BM, int BN, int WM, int WN, int ST, int NW, int SW, bool ASCH, bool OUT_F32, bool NT_B,
          bool E8, bool HALF = false>
__device__ __forceinline__ void gemm_tile(const GemmParams& p, uint8_t* smem, int m_base, int m_end,
                                          int n_base, const uint8_t* B, const float* Bs) {
  constexpr int WAVES_M = BM / WM, WAVES_N = BN / WN;
  static_assert(WAVES_M * WAVES_N == NW && (NW == 4 || NW == 8), "4 or 8 waves per workgroup");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's n range lies in one weight block");
  constexpr int MT = WM / 16, NT = WN / 16;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128, BS_BYTES = NW * 256;
  constexpr int AS_BYTES = ASCH ? 0 : NW * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + BS_BYTES;
  constexpr int A_LOADS = A_BYTES / (NW * 1024), B_LOADS = B_BYTES / (NW * 1024);  // per thread
  constexpr int LPS = A_LOADS + B_LOADS + 2;                          // DMA ops per stage
  static_assert(A_LOADS >= 1 && B_LOADS >= 1 && BM <= NW * 64, "tile shape");
  static_assert(ST >= 2, "at least double buffering");
  constexpr int ASC = ASCH ? NW * 256 / BM : 1;                       // K blocks per a_s chunk
  static_assert(!ASCH || (ASC % 4 == 0 && ASC >= ST - 1), "a_s chunk shape");
  constexpr int CHUNK_BYTES = ASCH ? NW * 1024 : 0;
  static_assert(tile_lds_bytes<BM, BN, ST, NW, ASCH>() <= 160 * 1024, "LDS");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  static_assert(!HALF || WAVES_M == 2, "HALF splits the tile's two m halves");
  const int wm = HALF ? wave / WAVES_N : wave % WAVES_M;
  const int wn = HALF ? wave % WAVES_N : wave / WAVES_M;
  const int K = p.K, N = p.N;
  const int nkb = K / 128;
  const int nbn = (N + 127) / 128;

  // ---- DMA sources.  Load i of this wave covers the 8 rows 8*(NW*i+wave)
  // .. +7 of the tile; lane l takes row l/8 of those and the logical chunk
  // (l % 8) ^ swz(row).  Offsets grow by 8*NW rows per load (which keeps
  // row % 16, hence the chunk choice) and 128 bytes per K block.
  const v4i a_rsrc = make_rsrc(p.a, (uint32_t)((int64_t)p.rows * K));
  const v4i b_rsrc = make_rsrc(B, (uint32_t)((int64_t)N * K));
  const v4i as_rsrc = make_rsrc(p.a_s, (uint32_t)((int64_t)p.rows * nkb * 4));
  const v4i bs_rsrc = make_rsrc(Bs, (uint32_t)((int64_t)nbn * nkb * 4));
  const int lrow = 8 * wave + (lane >> 3);
  const int lchunk = (lane & 7) ^ swz<SW>(lrow);
  const uint32_t a_voff = (uint32_t)(m_base + lrow) * K + 16 * lchunk;
  const uint32_t b_voff = (uint32_t)(n_base + lrow) * K + 16 * lchunk;
  const uint32_t as_voff = (uint32_t)(m_base + (tid % BM)) * nkb * 4;
  const uint32_t bs_voff = (uint32_t)((n_base + wn * WN) / 128) * nkb * 4;  // this wave's block row
  const uint32_t rowstep = 8u * NW * (uint32_t)K;
  const uint32_t smem_lds = lds_addr(smem);
  // a_s chunk piece of this lane: row (64 wave + lane) / (ASC/4), K blocks
  // 4 ((64 wave + lane) % (ASC/4)) .. +3 of the chunk; lands at byte
  // 16 (64 wave + lane) of the chunk buffer, i.e. row-major [BM][ASC].
  constexpr int LPR = ASCH ? ASC / 4 : 1;                              // lanes per a_s row
  const int as_idx = 64 * wave + lane;
  const uint32_t asc_voff = ((uint32_t)(m_base + as_idx / LPR) * nkb + 4 * (as_idx % LPR)) * 4;
  const uint32_t chunk_lds = smem_lds + ST * STAGE + wave * 1024;
  const uint32_t dummy_lds = smem_lds + ST * STAGE + 2 * CHUNK_BYTES;

  auto issue = [&](int kb, int st) {
    const uint32_t base = smem_lds + st * STAGE + wave * 1024;
    const uint32_t koff = (uint32_t)kb * 128;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      dma_b128s(a_rsrc, base + i * NW * 1024, a_voff + i * rowstep, koff);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      // NT_B: the weight is read exactly once (the small-expert MoE tiles:
      // at most 64 rows per expert, one m tile): non-temporal DMA (measured
      // on the 4096-token MoE: up 1062 -> 1030 us, down 1169 -> 1124 us; the
      // same hint on the 256-row tiles of single-tile experts did not help).
      if (NT_B) dma_b128s_nt(b_rsrc, base + A_BYTES + i * NW * 1024, b_voff + i * rowstep, koff);
      else dma_b128s(b_rsrc, base + A_BYTES + i * NW * 1024, b_voff + i * rowstep, koff);
    }
    if (ASCH) {
      if (kb % ASC == 0)
        dma_b128s(as_rsrc, chunk_lds + ((kb / ASC) & 1) * CHUNK_BYTES, asc_voff, (uint32_t)kb * 4);
      else if (ST > 2)
        dma_b32(as_rsrc, dummy_lds, 0xF0000000u);
    } else {
      // a_s: thread t fetches row t % BM into slot t (slots >= BM hold copies)
      dma_b32s(as_rsrc, smem_lds + st * STAGE + A_BYTES + B_BYTES + wave * 256, as_voff, (uint32_t)kb * 4);
    }
    // every lane of the wave fetches the same b_s value of its weight block
    dma_b32s(bs_rsrc, smem_lds + st * STAGE + A_BYTES + B_BYTES + AS_BYTES + wave * 256,
             bs_voff, (uint32_t)kb * 4);
  };

  v4f acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  const int g = lane >> 4, r16 = lane & 15;

  // Lane-constant parts of the fragment reads.  Fragment rows are 16 apart
  // and every row block of a tile starts at a multiple of 16, so the swizzle
  // of row 16 i + r16 is that of r16: each read is one of four lane bases
  // plus a compile-time offset (the ds_read offset field), with no
  // per-fragment address arithmetic in the loop.
  const int fsw = swz<SW>(r16);
  const uint32_t f_lo = r16 * 128 + (((2 * g) ^ fsw) << 4);
  const uint32_t f_hi = r16 * 128 + (((2 * g + 1) ^ fsw) << 4);
  const uint32_t a_lo = wm * WM * 128 + f_lo, a_hi = wm * WM * 128 + f_hi;
  const uint32_t b_lo = A_BYTES + wn * WN * 128 + f_lo, b_hi = A_BYTES + wn * WN * 128 + f_hi;
  const uint32_t as_lane = (uint32_t)(wm * WM + r16) * ASC * 4;

  // prologue
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nkb) issue(s, s);

  // The fold of a K block's last row block is deferred to just after the
  // next barrier: its MFMAs then run on through the barrier wait instead of
  // draining the matrix pipe before it.
  v4f pend[NT];
  float pend_sc = 0.0f;
#pragma unroll
  for (int j = 0; j < NT; ++j) pend[j] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  if (HALF && wm == 1) {
    // the empty second m half: the same loads, waits and barriers, no compute
    // (its accumulators stay zero and its rows are never stored)
    for (int kb = 0; kb < nkb; ++kb) {
      if (kb + ST - 2 < nkb) wait_vmcnt<(ST - 2) * LPS>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds();
      __builtin_amdgcn_sched_barrier(0);
      if (kb + ST - 1 < nkb) issue(kb + ST - 1, (kb + ST - 1) % ST);
    }
  } else
  for (int kb = 0; kb < nkb; ++kb) {
    const int st = kb % ST;
    // DMA for kb is complete once at most the later stages' ops are pending.
    if (kb + ST - 2 < nkb) wait_vmcnt<(ST - 2) * LPS>();
    else wait_vmcnt<0>();
    __builtin_amdgcn_sched_barrier(0);
    barrier_lds();
    __builtin_amdgcn_sched_barrier(0);

    const uint8_t* sbase = smem + st * STAGE;
    // fragment rows 16 i .. 16 i + 15 from the lane bases (lo, hi)
    auto frag = [&](uint32_t lo, uint32_t hi, int i) {
      const uint4 x = *(const uint4*)(sbase + lo + i * 2048);
      const uint4 y = *(const uint4*)(sbase + hi + i * 2048);
      v8i v;
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
      v[4] = y.x; v[5] = y.y; v[6] = y.z; v[7] = y.w;
      return v;
    };
    // this lane's activation scale of fragment row block t: a_s[row][as_col]
    // of the [BM][ASC] chunk (or the stage's [BM] column when ASC = 1)
    const uint8_t* asb = (ASCH ? smem + ST * STAGE + ((kb / ASC) & 1) * CHUNK_BYTES
                               : sbase + A_BYTES + B_BYTES) + as_lane + (ASCH ? (kb % ASC) * 4 : 0);
    const float bsv = ((const float*)(sbase + A_BYTES + B_BYTES + AS_BYTES))[wave * 64];
    v8i bf[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) bf[j] = frag(b_lo, b_hi, j);
    const v8i af0 = frag(a_lo, a_hi, 0);
    // The next stage's DMA goes out after the operand reads of this K block's
    // first MFMAs, so those reads do not queue behind the workgroup's burst of
    // DMA instructions.  It fills the other stage (and possibly the other a_s
    // chunk buffer), which every wave finished reading before the barrier.
    if (kb + ST - 1 < nkb) issue(kb + ST - 1, (kb + ST - 1) % ST);
    if (!E8) {
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        acc[j][MT - 1][0] = __builtin_fmaf(pend[j][0], pend_sc, acc[j][MT - 1][0]);
        acc[j][MT - 1][1] = __builtin_fmaf(pend[j][1], pend_sc, acc[j][MT - 1][1]);
        acc[j][MT - 1][2] = __builtin_fmaf(pend[j][2], pend_sc, acc[j][MT - 1][2]);
        acc[j][MT - 1][3] = __builtin_fmaf(pend[j][3], pend_sc, acc[j][MT - 1][3]);
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v8i af = t == 0 ? af0 : frag(a_lo, a_hi, t);
      const float as_t = *(const float*)(asb + t * 16 * ASC * 4);
      if (E8) {
        // E8M0 exponents: the biased exponent field of each power-of-two scale
        const int ea = (int)(f32_bits(as_t) >> 23);
        const int eb = (int)(f32_bits(bsv) >> 23);
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[j][t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af, acc[j][t], 0, 0, 0, eb, 0, ea);
        continue;
      }
      const float sc = as_t * bsv;
      if (t == MT - 1) {
#pragma unroll
        for (int j = 0; j < NT; ++j) pend[j] = mfma_k128(bf[j], af);
        pend_sc = sc;
        continue;
      }
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const v4f pr = mfma_k128(bf[j], af);
        acc[j][t][0] = __builtin_fmaf(pr[0], sc, acc[j][t][0]);
        acc[j][t][1] = __builtin_fmaf(pr[1], sc, acc[j][t][1]);
        acc[j][t][2] = __builtin_fmaf(pr[2], sc, acc[j][t][2]);
        acc[j][t][3] = __builtin_fmaf(pr[3], sc, acc[j][t][3]);
      }
    }
  }
  if (!E8) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc[j][MT - 1][0] = __builtin_fmaf(pend[j][0], pend_sc, acc[j][MT - 1][0]);
      acc[j][MT - 1][1] = __builtin_fmaf(pend[j][1], pend_sc, acc[j][MT - 1][1]);
      acc[j][MT - 1][2] = __builtin_fmaf(pend[j][2], pend_sc, acc[j][MT - 1][2]);
      acc[j][MT - 1][3] = __builtin_fmaf(pend[j][3], pend_sc, acc[j][MT - 1][3]);
    }
  }

  // ---- epilogue: lane holds C[m][n .. n+3] for each (j, t)
  if constexpr (!OUT_F32) {
    if ((N & 7) == 0) {
      static_assert(BM * BN * 2 <= ST * STAGE, "the C tile fits the stage buffers");
      store_c_tile_bf16<BM, BN, WM, WN, NW, MT, NT>(smem, acc, tid, wm, wn, p.c, N, m_base, m_end,
                                                    n_base);
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
          const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                 (uint16_t)(hi >> 16)};
          for (int r = 0; r < 4; ++r)
            if (n + r < N) cp[r] = h[r];
        }
      }
    }
  }
}

// Dense GEMM: one tile per workgroup.  OCC workgroups share a CU (register
// budget set for OCC * NW / 4 waves per SIMD).
template <int BM, int BN, int WM, int WN, int ST, int NW, int SW, bool ASCH, bool OUT_F32, int OCC,
          bool E8 = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC * NW / 4, OCC * NW / 4)))
gemm_tile_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[tile_lds_bytes<BM, BN, ST, NW, ASCH>()];
  // Groups of GM m-tiles sweep across n (consecutive tiles share B or A).
  const int t = xcd_remap(blockIdx.x, gridDim.x);
  constexpr int GM = 4;
  const int group = GM * p.num_n;
  const int gid = t / group, first_m = gid * GM;
  const int gsz = min(p.num_m - first_m, GM);
  const int in = t % group;
  const int mt = first_m + in % gsz, nt = in / gsz;
  gemm_tile<BM, BN, WM, WN, ST, NW, SW, ASCH, OUT_F32, false, E8>(p, smem, mt * BM, p.rows,
                                                                   p.n0 + nt * BN, p.b, p.b_s);
}

// ----------------------------------------------------------------------------
// Grouped MoE GEMM: both expert classes in one launch
// ----------------------------------------------------------------------------
// Experts are classed by their row count.  Experts with more than kMoeSplit
// rows are dense GEMMs in their own right and take the 256 x 256 tile of the
// dense path (bound by the matrix cores); the others -- most experts under
// skewed routing, and most of the weight bytes -- take one 64 x 256 tile per
// weight slice, three LDS stages, the weight read once with the
// non-temporal hint (bound by HBM).  Both shapes run in eight-wave
// workgroups of one kernel, so the two classes share the CUs in one grid:
// while some CUs multiply the large experts, the others stream the small
// experts' weights.
//
// Schedule.  The grid is an upper bound on the tile count, sized on the host
// from R and E alone.  Every workgroup counts the real m tiles of each class
// from the device offsets (wave prefix sums over the experts).  Each class's
// tiles -- (expert, m tile) pairs in expert order, n-minor, so consecutive
// tiles share an expert's activation rows -- are cut into eight contiguous
// parts, one per XCD (workgroups are dealt to the XCDs round-robin, so
// workgroup b runs on XCD b % 8 as its (b / 8)-th): an XCD reads an
// activation slab once for all its n tiles and an expert's weight on the one
// or two XCDs that hold its m tiles.  Within an XCD the large tiles are
// spread evenly over the first L + S * kMoeMix / 256 positions of its
// sequence and the small tiles fill the rest, so the long compute-bound tiles
// are all dispatched before the sequence ends in short streaming tiles.
constexpr int kMoeSplit = 64;
constexpr int kMoeMix = 160;

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d);
    if (lane >= d) v += u;
  }
  return v;
}

// m tiles of an expert with n_rows rows in class `large` (large tiles of
// 1 << lsh rows).
__device__ __forceinline__ int class_mtiles(int n_rows, bool large, int lsh) {
  return large ? (n_rows > kMoeSplit ? (n_rows + (1 << lsh) - 1) >> lsh : 0)
               : ((n_rows > 0 && n_rows <= kMoeSplit) ? 1 : 0);
}

// Rows of the experts e0 + 64 j + lane (j < 4), ranges clamped to [0, R]
// (0 past the last expert).  The eight offset loads are issued together:
// every workgroup runs this before its tile while its CU waits, so it costs
// one memory round trip per 256 experts instead of one per 64.
__device__ __forceinline__ void expert_rows4(const GemmParams& p, int e0, int lane, int (&rows)[4]) {
  int lo[4], hi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ee = min(e0 + 64 * j + lane, p.E - 1);
    lo[j] = p.offsets[ee];
    hi[j] = p.offsets[ee + 1];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int l = min(max(lo[j], 0), p.rows);
    rows[j] = e0 + 64 * j + lane < p.E ? min(max(hi[j], l), p.rows) - l : 0;
  }
}

template <bool ASCH, bool OUT_F32>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
moe_gemm_kernel(GemmParams p) {
  constexpr int LB = tile_lds_bytes<256, 256, 2, 8, ASCH>(), SB = tile_lds_bytes<64, 256, 3, 8, ASCH>();
  constexpr int ST64 = ASCH ? 7 : 6, ST128 = ASCH ? 5 : 4;   // narrow small-expert tiles' stages
  constexpr int S64 = tile_lds_bytes<64, 64, ST64, 8, ASCH>(), S128 = tile_lds_bytes<64, 128, ST128, 8, ASCH>();
  constexpr int L128 = tile_lds_bytes<128, 128, 3, 8, ASCH>();
  static_assert(S64 <= LB && S128 <= LB && SB <= LB && L128 <= LB, "the 256 x 256 layout is the largest");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[LB];
  const int lane = threadIdx.x & 63;
  const int lsh = p.large_sh;                             // large tiles: 1 << lsh square
  const int nn = (p.N + (1 << lsh) - 1) >> lsh;           // large tiles' n tiles
  const int nns = (p.N + p.small_bn - 1) / p.small_bn;    // small tiles' n tiles

  // real m tiles of each class (the first 256 experts' row counts are kept)
  int rows0[4];
  expert_rows4(p, 0, lane, rows0);
  int ml = 0, ms = 0;
  for (int e0 = 0; e0 < p.E; e0 += 256) {
    int rows[4];
    if (e0 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rows[j] = rows0[j];
    } else {
      expert_rows4(p, e0, lane, rows);
    }
    int cl = 0, cs = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cl += class_mtiles(rows[j], true, lsh);
      cs += class_mtiles(rows[j], false, lsh);
    }
    ml += __shfl(wave_incl_scan(cl, lane), 63);
    ms += __shfl(wave_incl_scan(cs, lane), 63);
  }
  const int64_t L = (int64_t)__builtin_amdgcn_readfirstlane(ml) * nn;
  const int64_t S = (int64_t)__builtin_amdgcn_readfirstlane(ms) * nns;

  // this XCD's parts of both lists and this workgroup's place in its sequence
  const int x = blockIdx.x % 8, k = blockIdx.x / 8;
  const int64_t l0 = L * x / 8, lx = L * (x + 1) / 8 - l0;
  const int64_t s0 = S * x / 8, sx = S * (x + 1) / 8 - s0;
  if (k >= lx + sx) return;                               // no real tile (uniform)
  const int64_t pl = lx + sx * kMoeMix / 256;             // positions holding the large tiles
  bool large;
  int64_t idx;
  if (k < pl) {
    const int64_t before = (int64_t)k * lx / pl;          // large tiles at positions < k
    large = ((int64_t)(k + 1) * lx / pl) > before;
    idx = large ? l0 + before : s0 + (k - before);
  } else {
    large = false;
    idx = s0 + (k - lx);
  }
  const int nc = large ? nn : nns;
  const int nt = (int)(idx % nc), gm = (int)(idx / nc);

  // the expert and m tile of class m tile gm: experts in index order, so
  // expert e0 + 64 j + lane comes after all of chunk j - 1 of its 256
  int e = -1, mt = 0, before = 0;
  for (int e0 = 0; e0 < p.E && e < 0; e0 += 256) {
    int rows[4];
    if (e0 == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) rows[j] = rows0[j];
    } else {
      expert_rows4(p, e0, lane, rows);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int cnt = class_mtiles(rows[j], large, lsh);
      const int incl = wave_incl_scan(cnt, lane);
      const int excl = before + incl - cnt;
      const unsigned long long ball = __ballot(gm >= excl && gm < excl + cnt);
      if (ball && e < 0) {
        const int src = __ffsll((long long)ball) - 1;
        e = e0 + 64 * j + src;
        mt = gm - __shfl(excl, src);
      }
      before += __shfl(incl, 63);
    }
  }
  e = __builtin_amdgcn_readfirstlane(e);
  mt = __builtin_amdgcn_readfirstlane(mt);
  if (e < 0) return;                                      // unreachable for valid offsets (uniform)
  const int lo = __builtin_amdgcn_readfirstlane(min(max(p.offsets[e], 0), p.rows));
  const int hi = __builtin_amdgcn_readfirstlane(min(max(p.offsets[e + 1], lo), p.rows));
  const int nbn = (p.N + 127) / 128, nkb = p.K / 128;
  const uint8_t* B = p.b + (int64_t)e * p.N * p.K;
  const float* Bs = p.b_s + (int64_t)e * nbn * nkb;
  // A large expert's m tile with at most 128 rows (its last, or its only one)
  // skips the MFMAs of the empty half (in the Zipf routing of the 4096-token
  // workload, 57 of 155 such m tiles; up 1013 -> 963-979 us, down 1086-1097 ->
  // 1038-1067 us, same box, bit-identical).
  if (large && lsh == 7) {
    // few experts: 128 x 128 tiles (eight waves of 64 x 32), HALF when the
    // m tile holds at most 64 rows
    if (hi - (lo + mt * 128) > 64)
      gemm_tile<128, 128, 64, 32, 3, 8, 2, ASCH, OUT_F32, false, false>(p, smem, lo + mt * 128, hi, nt * 128, B, Bs);
    else
      gemm_tile<128, 128, 64, 32, 3, 8, 2, ASCH, OUT_F32, false, false, true>(p, smem, lo + mt * 128, hi, nt * 128,
                                                                             B, Bs);
  } else if (large) {
    if (hi - (lo + mt * 256) > 128)
      gemm_tile<256, 256, 128, 64, 2, 8, 2, ASCH, OUT_F32, false, false>(p, smem, lo + mt * 256, hi, nt * 256, B, Bs);
    else
      gemm_tile<256, 256, 128, 64, 2, 8, 2, ASCH, OUT_F32, false, false, true>(p, smem, lo + mt * 256, hi, nt * 256,
                                                                              B, Bs);
  }
  else if (p.small_bn == 64)
    gemm_tile<64, 64, 32, 16, ST64, 8, 2, ASCH, OUT_F32, true, false>(p, smem, lo, hi, nt * 64, B, Bs);
  else if (p.small_bn == 128)
    gemm_tile<64, 128, 32, 32, ST128, 8, 2, ASCH, OUT_F32, true, false>(p, smem, lo, hi, nt * 128, B, Bs);
  else
    gemm_tile<64, 256, 64, 32, 3, 8, 2, ASCH, OUT_F32, true, false>(p, smem, lo, hi, nt * 256, B, Bs);
}

// ----------------------------------------------------------------------------
// Helpers for the HBM-bound decode kernel
// ----------------------------------------------------------------------------
// bf16 MFMA on decoded e4m3 operands.  The FP8 MFMA sums its 128 products in
// a reduced-precision internal format (measured on gfx950: errors up to
// ~1.4e-5 of the sum of |products| on normal data and ~2.3e-4 with 50x
// outliers), while the bf16 MFMA on the same values is accurate to ~2e-8.
// The decode kernel is bound by HBM, not by the matrix cores, so it decodes
// the e4m3 bytes to bf16 in registers (exact: every e4m3 value is a bf16
// value) and runs four K = 32 bf16 MFMAs per 128-wide K block; the block's
// partial is then scaled and added in fp32 as in the tile kernel.  K mapping:
// instruction i, lane group g takes the bytes [32g + 8i, 32g + 8i + 8) of the
// block for both operands.

// Eight e4m3 bytes (two dwords, byte order = element order) -> eight bf16.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t w0, uint32_t w1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  v8bf r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// ----------------------------------------------------------------------------
// Decode kernel (M <= 16*MT): HBM-bound weight streaming through LDS.
// ----------------------------------------------------------------------------
// One workgroup per CU: workgroup g owns the `rows` (a multiple of 8, at most
// 80) consecutive weight rows starting at g*rows, chosen on the host so the
// rows are spread evenly over the CUs, plus all M (<= 16*MT) activation rows.
// Each LDS stage holds KPS = 2 consecutive K blocks of both operands, filled
// by direct buffer->LDS loads whose every wave instruction covers 8 rows x one
// whole 128-byte line; the two K blocks of the same 8 rows are issued back to
// back, so each row is read 256 contiguous bytes at a time (the access pattern
// that streamed fastest on gfx950).  Five stages (~145 KB for M <= 32) keep
// four stages -- ~73 KB of weights per CU -- in flight.  Row groups past
// `rows` are requested at an out-of-range offset, which the buffer unit
// returns as zeros without touching memory.
// Wave w computes K block (w % 2) of every stage for the three 16-row tiles
// 3 (w / 2) .. 3 (w / 2) + 2 (tiles past `rows` read unused LDS and are never
// stored); the two waves of a pair are summed through LDS at the end.
// Arithmetic: e4m3 decoded to bf16, four K = 32 bf16 MFMAs per K block, one
// scale fold per K block in fp32 (see the helpers above).
constexpr int kDecodeMaxRows = 80;

template <int MT, bool OUT_F32>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
gemm_decode_kernel(GemmParams p, int rows) {
  constexpr int NW = 4, KPS = 2, MR = 16 * MT;
  constexpr int ST = MT <= 2 ? 5 : 3;
  constexpr int OCT = kDecodeMaxRows / 8;                        // row groups per K block
  constexpr int B_TILE = kDecodeMaxRows * 128, A_TILE = MR * 128;  // one K block
  constexpr int B_BYTES = KPS * B_TILE, A_BYTES = KPS * A_TILE;
  constexpr int AS_BYTES = NW * 256, BS_BYTES = NW * 256;
  constexpr int STAGE = B_BYTES + A_BYTES + AS_BYTES + BS_BYTES;
  constexpr int B_LOADS = KPS * OCT / NW, A_LOADS = A_BYTES / (NW * 1024);
  constexpr int LPS = B_LOADS + A_LOADS + 2;
  constexpr int NTW = 3;                                          // tiles per wave
  static_assert((KPS * OCT) % NW == 0 && A_LOADS >= 1 && MR <= 64, "shape");
  static_assert(ST * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int M = p.rows, N = p.N, K = p.K;
  const int nkb = K / 128, nkc = (nkb + KPS - 1) / KPS;
  const int n_base = blockIdx.x * rows;
  const int n_end = min(n_base + rows, N);
  const int q = wave & 1;                                 // this wave's K block in a stage
  const int jt0 = NTW * (wave >> 1);                      // this wave's first tile

  const v4i a_rsrc = make_rsrc(p.a, (uint32_t)((int64_t)M * K));
  const v4i b_rsrc = make_rsrc(p.b, (uint32_t)((int64_t)N * K));
  const v4i as_rsrc = make_rsrc(p.a_s, (uint32_t)((int64_t)M * nkb * 4));
  const int nbn = (N + 127) / 128;
  const v4i bs_rsrc = make_rsrc(p.b_s, (uint32_t)((int64_t)nbn * nkb * 4));
  // DMA instruction u = NW i + wave covers row group u / KPS of K block
  // u % KPS = q; lane l takes row l / 8 of the group and logical chunk
  // (l % 8) ^ (l / 8) (the row's swizzle, row % 8 = l / 8).
  const int lchunk = (lane & 7) ^ (lane >> 3);
  const int grp0 = wave >> 1;                             // row group of i = 0; +2 per i
  uint32_t b_voff[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int grp = grp0 + 2 * i;
    b_voff[i] = 8 * grp < rows
                    ? (uint32_t)(n_base + 8 * grp + (lane >> 3)) * K + 16 * lchunk + 128 * q
                    : 0xF0000000u;                       // past the buffer: zeros
  }
  const uint32_t a_voff = (uint32_t)(8 * grp0 + (lane >> 3)) * K + 16 * lchunk + 128 * q;
  const uint32_t as_voff = (uint32_t)lane * nkb * 4 + 4 * q;       // lane = activation row
  // lanes 0 and 1 fetch the scales of the (at most two) weight blocks the
  // workgroup's rows touch
  const uint32_t bs_voff = (uint32_t)(n_base / 128 + (lane & 1)) * nkb * 4 + 4 * q;
  const uint32_t step16 = 16u * (uint32_t)K;              // 2 row groups per i
  const uint32_t smem_lds = lds_addr(smem);

  auto issue = [&](int kc, int st) {
    const uint32_t base = smem_lds + st * STAGE;
    const uint32_t koff = (uint32_t)kc * (KPS * 128);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      dma_b128(b_rsrc, base + q * B_TILE + (grp0 + 2 * i) * 1024, b_voff[i] + koff);
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      dma_b128(a_rsrc, base + B_BYTES + q * A_TILE + (grp0 + 2 * i) * 1024, a_voff + i * step16 + koff);
    dma_b32(as_rsrc, base + B_BYTES + A_BYTES + wave * 256, as_voff + kc * (KPS * 4));
    dma_b32(bs_rsrc, base + B_BYTES + A_BYTES + AS_BYTES + wave * 256, bs_voff + kc * (KPS * 4));
  };

  v4f acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nkc) issue(s, s);

  for (int kc = 0; kc < nkc; ++kc) {
    const int st = kc % ST;
    if (kc + ST - 2 < nkc) wait_vmcnt<(ST - 2) * LPS>();
    else wait_vmcnt<0>();
    barrier_lds();
    if (kc + ST - 1 < nkc) issue(kc + ST - 1, (kc + ST - 1) % ST);
    if (kc * KPS + q >= nkb) continue;                   // odd tail: no second K block
    const uint8_t* base = smem + st * STAGE;
    const uint8_t* bt = base + q * B_TILE;
    const uint8_t* at = base + B_BYTES + q * A_TILE;
    const float* ast = (const float*)(base + B_BYTES + A_BYTES + wave * 256);
    const float* bst = (const float*)(base + B_BYTES + A_BYTES + AS_BYTES + wave * 256);
    v8bf af[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v8i f = lds_frag<0>(at, 16 * t + r16, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[t][i] = e4m3x8_to_bf16(f[2 * i], f[2 * i + 1]);
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      // rows of tile jt0 + j past the B region read the A region (unused results)
      const v8i f = lds_frag<0>(bt, 16 * (jt0 + j) + r16, g);
      // this lane's four rows share one weight block
      const int nl = n_base + 16 * (jt0 + j) + 4 * g;
      const float bsv = bst[(nl / 128 - n_base / 128) & 1];
      v8bf bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bf[i] = e4m3x8_to_bf16(f[2 * i], f[2 * i + 1]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        v4f pr = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[i], af[t][i], pr, 0, 0, 0);
        const float sc = ast[16 * t + r16] * bsv;
        acc[j][t][0] = __builtin_fmaf(pr[0], sc, acc[j][t][0]);
        acc[j][t][1] = __builtin_fmaf(pr[1], sc, acc[j][t][1]);
        acc[j][t][2] = __builtin_fmaf(pr[2], sc, acc[j][t][2]);
        acc[j][t][3] = __builtin_fmaf(pr[3], sc, acc[j][t][3]);
      }
    }
  }

  // ---- pairwise reduction (waves w and w ^ 1 hold the same tiles), store
  constexpr int NV = NTW * MT * 4;
  float* red = (float*)smem;                             // [NW][NV][64], reused
  barrier_lds();
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * NV + (j * MT + t) * 4 + r) * 64 + lane] = acc[j][t][r];
  barrier_lds();
  if (q == 0) {
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      const int n = n_base + 16 * (jt0 + j) + 4 * g;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = 16 * t + r16;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = acc[j][t][r] + red[((wave + 1) * NV + (j * MT + t) * 4 + r) * 64 + lane];
        if (m >= M || n >= n_end) continue;
        if (OUT_F32) {
          float* cp = (float*)p.c + (int64_t)m * N + n;
          if ((N % 4) == 0 && n + 3 < n_end) *(float4*)cp = make_float4(v[0], v[1], v[2], v[3]);
          else for (int r = 0; r < 4; ++r) if (n + r < n_end) cp[r] = v[r];
        } else {
          uint16_t* cp = (uint16_t*)p.c + (int64_t)m * N + n;
          const uint32_t lo = pack2_bf16(v[0], v[1]), hi = pack2_bf16(v[2], v[3]);
          if ((N % 4) == 0 && n + 3 < n_end) *(uint2*)cp = make_uint2(lo, hi);
          else {
            const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
            for (int r = 0; r < 4; ++r) if (n + r < n_end) cp[r] = h[r];
          }
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Decode kernel, eight-wave form (M <= 32).
// ----------------------------------------------------------------------------
// Workgroup g owns `rows` (<= 72, a multiple of 8) consecutive weight rows and
// all M activation rows, one workgroup per CU.  A stage holds KPS = 4
// consecutive K blocks: the weight rows ([4][72 rows][128 B], non-temporal
// DMA), the activations ([4][16 MT rows][128 B]), their scales ([4][64]) and
// the (at most two) weight block scales the rows touch -- 54.5 KB for
// M <= 32, three stages (two in flight, ~107 KB per CU).  The activation
// scales of a stage come as 16 bytes per row (one load; CH = true, needs K/128
// a multiple of 4 and a 16-byte aligned a_s) or as four column loads; the two
// weight block scales are read with scalar loads.  Every wave issues exactly
// LPS DMA instructions per stage (the real ones padded with zero-filling
// out-of-range loads into a 256-byte dummy area), so one vmcnt bound fits all
// waves.
// Wave w computes K block w % 4 of each stage for the 16-row weight tiles
// 0..2 (w < 4) or 3..4 (w >= 4): the two waves that share a SIMD cover all
// five tiles of one K block (72 rows; rows 72..79 of tile 4 read other LDS
// data and are never stored).  The four waves of a tile set are summed
// through LDS at the end.  Arithmetic as in the four-wave kernel: e4m3 to
// bf16 (exact), bf16 MFMA, one scale fold per K block.
constexpr int kDecode8Rows = 72;

template <int MT, bool OUT_F32, bool CH>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
gemm_decode8_kernel(GemmParams p, int rows) {
  constexpr int NW = 8, KPS = 4, ST = 3, MR = 16 * MT;
  constexpr int GRP = kDecode8Rows / 8;                           // weight row groups per K block
  constexpr int AGRP = MR / 8;                                    // activation row groups
  constexpr int B_TILE = kDecode8Rows * 128, A_TILE = MR * 128;   // one K block
  constexpr int B_BYTES = KPS * B_TILE, A_BYTES = KPS * A_TILE;
  constexpr int AS_BYTES = KPS * 256;                             // [row][4] or [4][row]
  constexpr int STAGE = B_BYTES + A_BYTES + AS_BYTES;
  constexpr int N_AS = CH ? 1 : KPS;
  constexpr int N_B = KPS * GRP, N_A = KPS * AGRP;
  constexpr int IB = (N_B + NW - 1) / NW, IA = (N_A + NW - 1) / NW;  // load slots per wave
  constexpr int LPS = IB + IA + 1;                                // + one for the activation scales
  constexpr int NTW = 3;                                          // tiles per wave (set 1: 2)
  static_assert(N_A == NW * IA && N_AS <= NW && MR <= 32, "shape");
  static_assert(ST * STAGE + 1024 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * STAGE + 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NW);
  const int g = lane >> 4, r16 = lane & 15;
  const int M = p.rows, N = p.N, K = p.K;
  const int nkb = K / 128, nkc = (nkb + KPS - 1) / KPS;
  const int n_base = blockIdx.x * rows;
  const int n_end = min(n_base + rows, N);
  const int q = wave & 3;                                 // this wave's K block in a stage
  const int jt0 = 3 * (wave >> 2);                        // this wave's first tile
  const int ntw = wave < 4 ? 3 : 2;

  const v4i a_rsrc = make_rsrc(p.a, (uint32_t)((int64_t)M * K));
  const v4i b_rsrc = make_rsrc(p.b, (uint32_t)((int64_t)N * K));
  const v4i as_rsrc = make_rsrc(p.a_s, (uint32_t)((int64_t)M * nkb * 4));
  const int nbn = (N + 127) / 128;
  typedef const float __attribute__((address_space(4)))* const_f32_ptr;
  const const_f32_ptr bs_const = (const_f32_ptr)(uintptr_t)p.b_s;
  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t dummy_lds = smem_lds + ST * STAGE;

  // The LPS DMA instructions of a wave in a stage have a type fixed by their
  // slot i, so the issue is straight-line code (a per-load type chosen at run
  // time had compiled to a chain of scalar branches in front of every load,
  // all on the path from the barrier to the next stage's requests):
  //   i < IB        weight rows, u = wave + NW i < N_B: K block u / GRP, row
  //                 group u % GRP (u >= N_B: padding);
  //   i < IB + IA   activations, v = wave + NW (i - IB): K block v / AGRP,
  //                 row group v % AGRP;
  //   i = IB + IA   a_s: CH: wave 0, lane = row, its 4 K blocks (16 bytes);
  //                 else waves 0 .. KPS - 1, K block `wave`, lane = row.
  // Padding loads are out of range (zeros) into the 1 KB dummy area.  16-byte
  // loads: lane l takes row l / 8 of its group and logical chunk
  // (l % 8) ^ (l / 8), the row's swizzle (row % 8 = l / 8).  The stage's K
  // position goes in the scalar offset field.
  const int lchunk = (lane & 7) ^ (lane >> 3);
  uint32_t voff[LPS], lds_off[LPS];
  bool real[LPS];
#pragma unroll
  for (int i = 0; i < LPS; ++i) {
    if (i < IB) {
      const int u = wave + NW * i, kq = u / GRP, grp = u % GRP;
      real[i] = u < N_B;
      voff[i] = real[i] && 8 * grp < rows
                    ? (uint32_t)(n_base + 8 * grp + (lane >> 3)) * K + 16 * lchunk + 128 * kq
                    : 0xF0000000u;
      lds_off[i] = kq * B_TILE + grp * 1024;
    } else if (i < IB + IA) {
      const int v = wave + NW * (i - IB), kq = v / AGRP, grp = v % AGRP;
      real[i] = true;
      voff[i] = (uint32_t)(8 * grp + (lane >> 3)) * K + 16 * lchunk + 128 * kq;
      lds_off[i] = B_BYTES + kq * A_TILE + grp * 1024;
    } else {
      const int kq = CH ? 0 : wave;
      real[i] = wave < N_AS;
      voff[i] = real[i] ? (uint32_t)lane * nkb * 4 + 4 * kq : 0xF0000000u;
      lds_off[i] = B_BYTES + A_BYTES + kq * 256;
    }
  }

  auto issue = [&](int kc, int st) {
    const uint32_t base = smem_lds + st * STAGE;
    const uint32_t kofs = (uint32_t)kc * (KPS * 128), sofs = (uint32_t)kc * (KPS * 4);
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const uint32_t lds = real[i] ? base + lds_off[i] : dummy_lds;
      if (i < IB) dma_b128s_nt(b_rsrc, lds, voff[i], kofs);
      else if (i < IB + IA) dma_b128s(a_rsrc, lds, voff[i], kofs);
      else if (CH) dma_b128s(as_rsrc, lds, voff[i], sofs);
      else dma_b32s(as_rsrc, lds, voff[i], sofs);
    }
  };

  v4f acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nkc) issue(s, s);

  for (int kc = 0; kc < nkc; ++kc) {
    const int st = kc % ST;
    if (kc + ST - 2 < nkc) wait_vmcnt<(ST - 2) * LPS>();
    else wait_vmcnt<0>();
    barrier_lds();
    if (kc + ST - 1 < nkc) issue(kc + ST - 1, (kc + ST - 1) % ST);
    if (kc * KPS + q >= nkb) continue;                   // tail stage: K block past the end
    const uint8_t* base = smem + st * STAGE;
    const uint8_t* bt = base + q * B_TILE;
    const uint8_t* at = base + B_BYTES + q * A_TILE;
    const float* ast = (const float*)(base + B_BYTES + A_BYTES);
    // the (at most two) weight block scales of this K block, read with scalar
    // loads (constant address space, wave-uniform index) so that no vector
    // load -- and no compiler-inserted vmcnt wait -- enters the K loop; the
    // second index is clamped (when the rows do not reach a second block no
    // lane uses it)
    const int kbq = kc * KPS + q;
    const int blk0 = n_base / 128, blk1 = min(blk0 + 1, nbn - 1);
    const float bs0 = bs_const[__builtin_amdgcn_readfirstlane(blk0 * nkb + kbq)];
    const float bs1 = bs_const[__builtin_amdgcn_readfirstlane(blk1 * nkb + kbq)];
    v8bf af[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const v8i f = lds_frag<0>(at, 16 * t + r16, g);
#pragma unroll
      for (int i = 0; i < 4; ++i) af[t][i] = e4m3x8_to_bf16(f[2 * i], f[2 * i + 1]);
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      if (j >= ntw) break;                                 // wave-uniform
      const v8i f = lds_frag<0>(bt, 16 * (jt0 + j) + r16, g);
      const int nl = n_base + 16 * (jt0 + j) + 4 * g;      // this lane's four rows share a block
      const float bsv = ((nl / 128 - n_base / 128) & 1) ? bs1 : bs0;
      v8bf bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bf[i] = e4m3x8_to_bf16(f[2 * i], f[2 * i + 1]);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        v4f pr = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < 4; ++i) pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[i], af[t][i], pr, 0, 0, 0);
        const int m = 16 * t + r16;
        const float sc = (CH ? ast[4 * m + q] : ast[64 * q + m]) * bsv;
        acc[j][t][0] = __builtin_fmaf(pr[0], sc, acc[j][t][0]);
        acc[j][t][1] = __builtin_fmaf(pr[1], sc, acc[j][t][1]);
        acc[j][t][2] = __builtin_fmaf(pr[2], sc, acc[j][t][2]);
        acc[j][t][3] = __builtin_fmaf(pr[3], sc, acc[j][t][3]);
      }
    }
  }

  // ---- reduction over the four K-block waves of each tile set, then store
  constexpr int NV = NTW * MT * 4;
  float* red = (float*)smem;                             // [NW][NV][64], reused
  static_assert(NW * NV * 64 * 4 <= ST * STAGE, "reduction area");
  barrier_lds();
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * NV + (j * MT + t) * 4 + r) * 64 + lane] = acc[j][t][r];
  barrier_lds();
  if (q != 0) return;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    if (j >= ntw) break;
    const int n = n_base + 16 * (jt0 + j) + 4 * g;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = 16 * t + r16;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = acc[j][t][r];
#pragma unroll
        for (int w = 1; w < 4; ++w) v[r] += red[((wave + w) * NV + (j * MT + t) * 4 + r) * 64 + lane];
      }
      if (m >= M || n >= n_end) continue;
      if (OUT_F32) {
        float* cp = (float*)p.c + (int64_t)m * N + n;
        if ((N % 4) == 0 && n + 3 < n_end) *(float4*)cp = make_float4(v[0], v[1], v[2], v[3]);
        else for (int r = 0; r < 4; ++r) if (n + r < n_end) cp[r] = v[r];
      } else {
        uint16_t* cp = (uint16_t*)p.c + (int64_t)m * N + n;
        const uint32_t lo = pack2_bf16(v[0], v[1]), hi = pack2_bf16(v[2], v[3]);
        if ((N % 4) == 0 && n + 3 < n_end) *(uint2*)cp = make_uint2(lo, hi);
        else {
          const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
          for (int r = 0; r < 4; ++r) if (n + r < n_end) cp[r] = h[r];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Decode kernel for few weight rows (M <= 32): K split over the waves.
// ----------------------------------------------------------------------------
// With a small N the streaming kernel above gives each workgroup a few rows
// and walks all K blocks in one sequence of stages, so its time is that
// sequence's latency, not its bytes (32 x 1536 x 7168: 16.8 us for 11 MB).
// Here a workgroup owns 16 weight rows n0 .. n0+15 and its eight waves deal
// the K blocks round-robin (wave w: K blocks w, w + 8, ...).  A wave loads
// its operand fragments straight into registers with range-checked buffer
// loads, two K blocks ahead.  Every load is unconditional: a K block past the
// end (and rows past N or M) read zeros at an out-of-range offset and add
// nothing, so the compiler's in-order wait counts keep the next block in
// flight.  The codes are decoded to bf16 and multiplied on the bf16 MFMA,
// with one fold per K block, as in the kernel above (same fragment and K
// mapping: lane (r16, g) holds bytes 32g .. 32g + 31 of its row's block); the
// eight waves' sums meet in LDS and wave 0 adds them in wave order.
// BF16X: the BF16 path (W8A16): x is bf16 (p.a, no a_s), each weight code is
// dequantised with its block scale (weight_dequant's rounding) and the
// products accumulate with no fold, as in w8a16_decode8_kernel.
template <int MT, bool OUT_F32, bool BF16X = false>
__global__ void __launch_bounds__(512) gemm_decode_splitk_kernel(GemmParams p) {
  constexpr int NW = 8;
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int M = p.rows, N = p.N, K = p.K, nkb = K / 128;
  const int n0 = blockIdx.x * 16;
  const int nbn = (N + 127) / 128;
  const uint32_t bad = 0xF0000000u;                      // out of every range: zeros
  constexpr int XB = BF16X ? 2 : 1;                      // bytes per activation element
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.a), (short)0, (int)(uint32_t)((int64_t)M * K * XB), 0x00020000);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.b), (short)0, (int)(uint32_t)((int64_t)N * K), 0x00020000);
  const __amdgpu_buffer_rsrc_t as_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.a_s), (short)0, (int)(uint32_t)((int64_t)M * nkb * 4), 0x00020000);
  const __amdgpu_buffer_rsrc_t bs_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.b_s), (short)0, (int)(uint32_t)((int64_t)nbn * nkb * 4), 0x00020000);
  const uint32_t b_row = (uint32_t)(n0 + r16) * K + 32 * g;
  uint32_t a_row[MT], as_row[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    a_row[t] = (uint32_t)(16 * t + r16) * K * XB + 32 * XB * g;
    as_row[t] = (uint32_t)(16 * t + r16) * nkb * 4;
  }
  const uint32_t bs_row = (uint32_t)(n0 / 128) * nkb * 4;  // the 16 rows lie in one block row

  constexpr int NA = 2 * XB;                             // 16-byte activation loads per row
  struct Frag {
    u4 b[2];
    u4 a[MT][NA];
    float as[MT];
    float bs;
  };
  auto load = [&](Frag& f, int kb) {
    const bool ok = kb < nkb;                              // wave-uniform
    const uint32_t ko = (uint32_t)kb * 128;
    f.b[0] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(b_rs, ok ? b_row + ko : bad, 0, kNonTemporal));
    f.b[1] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(b_rs, ok ? b_row + ko + 16 : bad, 0, kNonTemporal));
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        f.a[t][i] = __builtin_bit_cast(
            u4, __builtin_amdgcn_raw_buffer_load_b128(a_rs, ok ? a_row[t] + XB * ko + 16 * i : bad, 0, 0));
      if constexpr (!BF16X)
        f.as[t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(as_rs, ok ? as_row[t] + 4 * kb : bad, 0, 0));
    }
    f.bs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bs_rs, ok ? bs_row + 4 * kb : bad, 0, 0));
  };
  v4f acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const Frag& f) {
    if constexpr (BF16X) {
      // lane (r16, g), step i: codes 32g + 8i .. + 8 of its weight row and
      // the same K range of token 16t + r16 (bytes 64g + 16i of the x row)
      v8bf bf[4];
      bf[0] = dequant8_bf16(f.b[0].x, f.b[0].y, f.bs);
      bf[1] = dequant8_bf16(f.b[0].z, f.b[0].w, f.bs);
      bf[2] = dequant8_bf16(f.b[1].x, f.b[1].y, f.bs);
      bf[3] = dequant8_bf16(f.b[1].z, f.b[1].w, f.bs);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[i], __builtin_bit_cast(v8bf, f.a[t][i]), acc[t], 0, 0, 0);
    } else {
    v8bf bf[4];
    bf[0] = e4m3x8_to_bf16(f.b[0].x, f.b[0].y);
    bf[1] = e4m3x8_to_bf16(f.b[0].z, f.b[0].w);
    bf[2] = e4m3x8_to_bf16(f.b[1].x, f.b[1].y);
    bf[3] = e4m3x8_to_bf16(f.b[1].z, f.b[1].w);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      v4f pr = {0.0f, 0.0f, 0.0f, 0.0f};
      pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[0], e4m3x8_to_bf16(f.a[t][0].x, f.a[t][0].y), pr, 0, 0, 0);
      pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[1], e4m3x8_to_bf16(f.a[t][0].z, f.a[t][0].w), pr, 0, 0, 0);
      pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[2], e4m3x8_to_bf16(f.a[t][1].x, f.a[t][1].y), pr, 0, 0, 0);
      pr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[3], e4m3x8_to_bf16(f.a[t][1].z, f.a[t][1].w), pr, 0, 0, 0);
      const float sc = f.as[t] * f.bs;
      acc[t][0] = __builtin_fmaf(pr[0], sc, acc[t][0]);
      acc[t][1] = __builtin_fmaf(pr[1], sc, acc[t][1]);
      acc[t][2] = __builtin_fmaf(pr[2], sc, acc[t][2]);
      acc[t][3] = __builtin_fmaf(pr[3], sc, acc[t][3]);
    }
    }
  };
  // K blocks per wave, rounded up to whole pairs (uniform; the extra ones are zeros)
  const int iters = 2 * ((nkb + 2 * NW - 1) / (2 * NW));
  Frag f0, f1;
  load(f0, wave);
  load(f1, wave + NW);
  for (int it = 0; it < iters; it += 2) {
    compute(f0);
    load(f0, wave + NW * (it + 2));
    compute(f1);
    load(f1, wave + NW * (it + 3));
  }

  __shared__ float red[NW][MT * 4][64];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][t * 4 + r][lane] = acc[t][r];
  __syncthreads();
  if (wave != 0) return;
  const int n = n0 + 4 * g;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + r16;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      v[r] = red[0][t * 4 + r][lane];
#pragma unroll
      for (int w = 1; w < NW; ++w) v[r] += red[w][t * 4 + r][lane];
    }
    if (m >= M || n >= N) continue;
    if (OUT_F32) {
      float* cp = (float*)p.c + (int64_t)m * N + n;
      if ((N % 4) == 0 && n + 3 < N) *(float4*)cp = make_float4(v[0], v[1], v[2], v[3]);
      else for (int r = 0; r < 4; ++r) if (n + r < N) cp[r] = v[r];
    } else {
      uint16_t* cp = (uint16_t*)p.c + (int64_t)m * N + n;
      const uint32_t lo = pack2_bf16(v[0], v[1]), hi = pack2_bf16(v[2], v[3]);
      if ((N % 4) == 0 && n + 3 < N) *(uint2*)cp = make_uint2(lo, hi);
      else {
        const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
        for (int r = 0; r < 4; ++r) if (n + r < N) cp[r] = h[r];
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Decode kernel of the BF16 path (W8A16, M <= 32), eight waves.
// ----------------------------------------------------------------------------
// The streaming structure of gemm_decode8_kernel with the BF16 path's
// arithmetic: x is bf16, the weight codes are dequantised in registers with
// weight_dequant's rounding (float32 product, bf16 RNE) and multiplied on the
// bf16 MFMA; the block scale is inside the operand, so there is no fold.  A
// stage holds KPS = 2 K blocks: the weight rows ([2][72][128 B],
// non-temporal) and the bf16 activation rows ([2][16 MT][256 B]); four
// stages (three in flight).  The 256-byte x rows put 16-byte chunk c of row
// r at c ^ (r & 11), which makes the fragment reads conflict-free under the
// measured bank rule (four cycles of 16 lanes: half-wave x parity of lane
// bits 2..4).  Wave w computes K block w % 2 for tile set w / 2: tiles {0, 1},
// {2}, {3} or {4}; the two K-block waves of a set are summed at the end.
__device__ __forceinline__ int swz256(int r) { return r & 11; }

template <int MT, bool OUT_F32>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
w8a16_decode8_kernel(GemmParams p, int rows) {
  constexpr int NW = 8, KPS = 2, ST = 4, MR = 16 * MT;
  constexpr int GRP = kDecode8Rows / 8;                           // 8-row weight groups
  constexpr int AGRP = MR / 4;                                    // 4-row x groups (1 KB each)
  constexpr int B_TILE = kDecode8Rows * 128, A_TILE = MR * 256;   // one K block
  constexpr int B_BYTES = KPS * B_TILE, A_BYTES = KPS * A_TILE;
  constexpr int STAGE = B_BYTES + A_BYTES;
  constexpr int N_B = KPS * GRP, N_A = KPS * AGRP;
  constexpr int IB = (N_B + NW - 1) / NW, IA = N_A / NW;          // load slots per wave
  constexpr int LPS = IB + IA;
  constexpr int NTW = 2;                                          // tiles per wave (sets 1-3: 1)
  static_assert(MR <= 32 && N_A == NW * IA, "shape");
  static_assert(ST * STAGE + 1024 <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * STAGE + 1024];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  __builtin_assume(wave >= 0 && wave < NW);
  const int g = lane >> 4, r16 = lane & 15;
  const int M = p.rows, N = p.N, K = p.K;
  const int nkb = K / 128, nkc = (nkb + KPS - 1) / KPS;
  const int n_base = blockIdx.x * rows;
  const int n_end = min(n_base + rows, N);
  const int q = wave & 1;                                 // this wave's K block in a stage
  const int set = wave >> 1;
  const int jt0 = set == 0 ? 0 : set + 1;                 // first tile of the set
  const int ntw = set == 0 ? 2 : 1;

  const v4i a_rsrc = make_rsrc(p.a, (uint32_t)((int64_t)M * K * 2));
  const v4i b_rsrc = make_rsrc(p.b, (uint32_t)((int64_t)N * K));
  const int nbn = (N + 127) / 128;
  typedef const float __attribute__((address_space(4)))* const_f32_ptr;
  const const_f32_ptr bs_const = (const_f32_ptr)(uintptr_t)p.b_s;
  const uint32_t smem_lds = lds_addr(smem);
  const uint32_t dummy_lds = smem_lds + ST * STAGE;

  // The LPS DMA instructions of a wave in a stage have a type fixed by their
  // slot i (straight-line issue, as in gemm_decode8_kernel):
  //   i < IB   weight rows, u = wave + NW i < N_B: K block u / GRP, 8-row group
  //            u % GRP; lane l takes row l / 8, logical chunk (l % 8) ^ (l / 8)
  //            (u >= N_B: padding, out of range into the 1 KB dummy area);
  //   else     x rows, v = wave + NW (i - IB): K block v / AGRP, 4-row group
  //            v % AGRP; lane l takes row l / 16, logical chunk
  //            (l % 16) ^ swz256(row).
  // The stage's K position goes in the scalar offset field.
  uint32_t voff[LPS], lds_off[LPS];
  bool real[LPS];
#pragma unroll
  for (int i = 0; i < LPS; ++i) {
    if (i < IB) {
      const int u = wave + NW * i, kq = u / GRP, grp = u % GRP;
      const int lchunk = (lane & 7) ^ (lane >> 3);
      real[i] = u < N_B;
      voff[i] = real[i] && 8 * grp < rows
                    ? (uint32_t)(n_base + 8 * grp + (lane >> 3)) * K + 16 * lchunk + 128 * kq
                    : 0xF0000000u;
      lds_off[i] = kq * B_TILE + grp * 1024;
    } else {
      const int v = wave + NW * (i - IB), kq = v / AGRP, grp = v % AGRP;
      const int r = 4 * grp + (lane >> 4);
      const int lchunk = (lane & 15) ^ swz256(r & 15);
      real[i] = true;
      voff[i] = (uint32_t)r * (2 * K) + 16 * lchunk + 256 * kq;   // rows >= M read zeros
      lds_off[i] = B_BYTES + kq * A_TILE + grp * 1024;
    }
  }

  auto issue = [&](int kc, int st) {
    const uint32_t base = smem_lds + st * STAGE;
    const uint32_t bofs = (uint32_t)kc * (KPS * 128), xofs = (uint32_t)kc * (KPS * 256);
#pragma unroll
    for (int i = 0; i < LPS; ++i) {
      const uint32_t lds = real[i] ? base + lds_off[i] : dummy_lds;
      if (i < IB) dma_b128s_nt(b_rsrc, lds, voff[i], bofs);
      else dma_b128s(a_rsrc, lds, voff[i], xofs);
    }
  };

  v4f acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nkc) issue(s, s);

  for (int kc = 0; kc < nkc; ++kc) {
    const int st = kc % ST;
    if (kc + ST - 2 < nkc) wait_vmcnt<(ST - 2) * LPS>();
    else if (kc + 1 < nkc) wait_vmcnt<LPS>();
    else wait_vmcnt<0>();
    barrier_lds();
    if (kc + ST - 1 < nkc) issue(kc + ST - 1, (kc + ST - 1) % ST);
    const int kbq = kc * KPS + q;
    if (kbq >= nkb) continue;                            // tail stage: K block past the end
    const uint8_t* base = smem + st * STAGE;
    const uint8_t* bt = base + q * B_TILE;
    const uint8_t* at = base + B_BYTES + q * A_TILE;
    // the (at most two) weight block scales of this K block (scalar loads;
    // the second index is clamped: when the rows do not reach a second block
    // no lane uses it)
    const int blk0 = n_base / 128, blk1 = min(blk0 + 1, nbn - 1);
    const float bs0 = bs_const[__builtin_amdgcn_readfirstlane(blk0 * nkb + kbq)];
    const float bs1 = bs_const[__builtin_amdgcn_readfirstlane(blk1 * nkb + kbq)];
    // x: lane (r16, g) holds K [32 g + 8 i, +8) of token 16 t + r16 for step i
    v8bf xf[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const uint8_t* row = at + (16 * t + r16) * 256;
      const int sw = swz256(r16);
#pragma unroll
      for (int i = 0; i < 4; ++i) xf[t][i] = __builtin_bit_cast(v8bf, *(const v4i*)(row + (((4 * g + i) ^ sw) << 4)));
    }
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      if (j >= ntw) break;                                 // wave-uniform
      const int jt = jt0 + j;
      const v8i f = lds_frag<0>(bt, 16 * jt + r16, g);     // weight row 16 jt + r16, K [32 g, +32)
      const int nrow = n_base + 16 * jt + r16;
      const float sc = ((nrow / 128 - blk0) & 1) ? bs1 : bs0;
      v8bf bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bf[i] = dequant8_bf16(f[2 * i], f[2 * i + 1], sc);
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[i], xf[t][i], acc[j][t], 0, 0, 0);
    }
  }

  // ---- sum the two K-block waves of each tile set, then store
  constexpr int NV = NTW * MT * 4;
  float* red = (float*)smem;                             // [NW][NV][64], reused
  static_assert(NW * NV * 64 * 4 <= ST * STAGE, "reduction area");
  barrier_lds();
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[(wave * NV + (j * MT + t) * 4 + r) * 64 + lane] = acc[j][t][r];
  barrier_lds();
  if (q != 0) return;
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    if (j >= ntw) break;
    const int n = n_base + 16 * (jt0 + j) + 4 * g;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int m = 16 * t + r16;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = acc[j][t][r] + red[((wave + 1) * NV + (j * MT + t) * 4 + r) * 64 + lane];
      if (m >= M || n >= n_end) continue;
      if (OUT_F32) {
        float* cp = (float*)p.c + (int64_t)m * N + n;
        if ((N % 4) == 0 && n + 3 < n_end) *(float4*)cp = make_float4(v[0], v[1], v[2], v[3]);
        else for (int r = 0; r < 4; ++r) if (n + r < n_end) cp[r] = v[r];
      } else {
        uint16_t* cp = (uint16_t*)p.c + (int64_t)m * N + n;
        const uint32_t lo = pack2_bf16(v[0], v[1]), hi = pack2_bf16(v[2], v[3]);
        if ((N % 4) == 0 && n + 3 < n_end) *(uint2*)cp = make_uint2(lo, hi);
        else {
          const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi, (uint16_t)(hi >> 16)};
          for (int r = 0; r < 4; ++r) if (n + r < n_end) cp[r] = h[r];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// BF16 path (W8A16): C = x . weight_dequant(W)^T with x bf16, W e4m3 + 128x128
// block scales ("DeepSeek-V3 Administrator & Developer Guide" 6.3: with
// gemm_impl "bf16" the FP8 weight is dequantised (8.5.2) and the linear runs
// in BF16).  The dequantised weight is never stored: each wave decodes the
// weight codes of its fragments in registers -- RN32(decode(q) * s), then
// bf16 round-to-nearest-even, exactly the weight_dequant rounding -- and feeds
// them to v_mfma_f32_16x16x32_bf16, which accumulates in fp32 (no per-block
// fold: the scale is inside the dequantised operand).
//
// Workgroup: 8 waves, 256 (m) x 256 (n) tile, wave 128 x 64 as in the FP8
// tile kernel.  A stage is a 64-wide K slice: [x 256 rows x 128 bytes][W 256
// rows x 64 bytes][b_s per wave]; three stages (150 KB).  K mapping of one
// slice: MFMA step s (0, 1), lane group g takes K [16g + 8s, 16g + 8s + 8), so
// a lane's weight codes for both steps are the 16 contiguous bytes [16g,
// 16g + 16) of its row, and its x values for step s the 16 bytes at 32g + 16s.
// The 128-byte x rows use the swizzle of the FP8 kernel; the 64-byte weight
// rows put chunk c of row r at c ^ ((r >> 1) & 2), which keeps the weight
// fragment reads conflict-free under the same bank rule.
__device__ __forceinline__ int swz64(int r) { return (r >> 1) & 2; }


template <int BM, int BN, int WM, int WN, int NW, int ST, int OCC, bool OUT_F32>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(OCC * NW / 4, OCC * NW / 4)))
w8a16_tile_kernel(GemmParams p) {
  constexpr int WAVES_M = BM / WM;
  static_assert(WAVES_M * (BN / WN) == NW && (NW == 4 || NW == 8), "4 or 8 waves");
  static_assert(WN <= 128 && 128 % WN == 0, "a wave's n range lies in one weight block");
  constexpr int MT = WM / 16, NT = WN / 16;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 64, BS_BYTES = NW * 256;
  constexpr int STAGE = A_BYTES + B_BYTES + BS_BYTES;
  constexpr int A_LOADS = A_BYTES / (NW * 1024), B_LOADS = B_BYTES / (NW * 1024);
  constexpr int LPS = A_LOADS + B_LOADS + 1;
  static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile shape");
  static_assert(OCC * ST * STAGE <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[ST * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int K = p.K, N = p.N;
  const int nks = K / 64;                                    // 64-wide K slices
  const int nbk = K / 128;

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

  const v4i a_rsrc = make_rsrc(p.a, (uint32_t)((int64_t)p.rows * K * 2));
  const v4i b_rsrc = make_rsrc(p.b, (uint32_t)((int64_t)N * K));
  const v4i bs_rsrc = make_rsrc(p.b_s, (uint32_t)((int64_t)((N + 127) / 128) * nbk * 4));
  // x: load i of this wave covers rows 8 (NW i + wave) .. +7, 8 lanes per row
  const int arow = 8 * wave + (lane >> 3);
  const uint32_t a_voff = (uint32_t)(m_base + arow) * (uint32_t)(2 * K) + 16 * ((lane & 7) ^ swz<2>(arow));
  const uint32_t a_step = 8u * NW * (uint32_t)(2 * K);
  // W: load i covers rows 16 (NW i + wave) .. +15, 4 lanes per row
  const int brow = 16 * wave + (lane >> 2);
  const uint32_t b_voff = (uint32_t)(n_base + brow) * (uint32_t)K + 16 * ((lane & 3) ^ swz64(brow));
  const uint32_t b_step = 16u * NW * (uint32_t)K;
  const uint32_t bs_voff = (uint32_t)((n_base + wn * WN) / 128) * nbk * 4;
  const uint32_t smem_lds = lds_addr(smem);

  auto issue = [&](int ks, int st) {
    const uint32_t base = smem_lds + st * STAGE + wave * 1024;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
      dma_b128s(a_rsrc, base + i * NW * 1024, a_voff + i * a_step, (uint32_t)ks * 128);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      dma_b128s(b_rsrc, base + A_BYTES + i * NW * 1024, b_voff + i * b_step, (uint32_t)ks * 64);
    dma_b32s(bs_rsrc, smem_lds + st * STAGE + A_BYTES + B_BYTES + wave * 256, bs_voff, (uint32_t)(ks / 2) * 4);
  };

  v4f acc[NT][MT];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[j][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  const int g = lane >> 4, r16 = lane & 15;
  // lane bases of the fragment reads (row blocks start at multiples of 16,
  // so both swizzles depend on r16 only): x chunk 2g + s of row 16t + r16 at
  // xa[s] + 2048 t, the weight chunk g of row 16j + r16 at wb + 1024 j
  const uint32_t xa0 = (uint32_t)(wm * WM + r16) * 128 + (((2 * g) ^ swz<2>(r16)) << 4);
  const uint32_t xa1 = (uint32_t)(wm * WM + r16) * 128 + (((2 * g + 1) ^ swz<2>(r16)) << 4);
  const uint32_t wb = A_BYTES + (uint32_t)(wn * WN + r16) * 64 + ((g ^ swz64(r16)) << 4);

#pragma unroll
  for (int s0 = 0; s0 < ST - 1; ++s0)
    if (s0 < nks) issue(s0, s0);

  for (int ks = 0; ks < nks; ++ks) {
    const int st = ks % ST;
    if (ks + ST - 2 < nks) wait_vmcnt<(ST - 2) * LPS>();
    else wait_vmcnt<0>();
    barrier_lds();

    const uint8_t* at = smem + st * STAGE;
    const float bsv = ((const float*)(at + A_BYTES + B_BYTES))[wave * 64];
    uint4 wr[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) wr[j] = *(const uint4*)(at + wb + j * 1024);
    const uint4 x00 = *(const uint4*)(at + xa0);
    // the next stage's DMA after the first operand reads (as in the FP8 tile
    // kernel); it fills a stage every wave finished reading before the barrier
    if (ks + ST - 1 < nks) issue(ks + ST - 1, (ks + ST - 1) % ST);
    v8bf bf[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      bf[j][0] = dequant8_bf16(wr[j].x, wr[j].y, bsv);
      bf[j][1] = dequant8_bf16(wr[j].z, wr[j].w, bsv);
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const v8bf af = __builtin_bit_cast(
            v8bf, (t == 0 && s == 0) ? x00 : *(const uint4*)(at + (s ? xa1 : xa0) + t * 2048));
#pragma unroll
        for (int j = 0; j < NT; ++j)
          acc[j][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j][s], af, acc[j][t], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds C[m][n .. n+3] for each (j, t)
  if constexpr (!OUT_F32) {
    if ((N & 7) == 0) {
      static_assert(BM * BN * 2 <= ST * STAGE, "the C tile fits the stage buffers");
      store_c_tile_bf16<BM, BN, WM, WN, NW, MT, NT>(smem, acc, tid, wm, wn, p.c, N, m_base, p.rows,
                                                    n_base);
      return;
    }
  }
  const bool vec_ok = (N % 4) == 0;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m_base + wm * WM + 16 * t + r16;
    if (m >= p.rows) continue;
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
          const uint16_t h[4] = {(uint16_t)lo, (uint16_t)(lo >> 16), (uint16_t)hi,
                                 (uint16_t)(hi >> 16)};
          for (int r = 0; r < 4; ++r)
            if (n + r < N) cp[r] = h[r];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Launchers
// ----------------------------------------------------------------------------
namespace {

template <int BM, int BN, int WM, int WN, int ST, int NW, int SW, bool ASCH, int OCC, bool E8>
void launch_tile(const GemmParams& p, bool out_f32, int grid, hipStream_t stream) {
  if (out_f32)
    gemm_tile_kernel<BM, BN, WM, WN, ST, NW, SW, ASCH, true, OCC, E8><<<dim3(grid), dim3(NW * 64), 0, stream>>>(p);
  else
    gemm_tile_kernel<BM, BN, WM, WN, ST, NW, SW, ASCH, false, OCC, E8><<<dim3(grid), dim3(NW * 64), 0, stream>>>(p);
}

// Chunked a_s loads (16 bytes per lane) need every row of a_s to start on a
// 16-byte boundary.
template <int BM, int BN, int WM, int WN, int ST, int NW, int SW, int OCC = 1, bool E8 = false>
hipError_t run_tile(const GemmParams& p, bool out_f32, int grid, hipStream_t stream) {
  const bool chunked = (p.K / 128) % 4 == 0 && ((uintptr_t)p.a_s & 15) == 0;
  if (chunked)
    launch_tile<BM, BN, WM, WN, ST, NW, SW, true, OCC, E8>(p, out_f32, grid, stream);
  else
    launch_tile<BM, BN, WM, WN, ST, NW, SW, false, OCC, E8>(p, out_f32, grid, stream);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

// Decode GEMMs with N up to this take the split-K kernel.  Same box, us,
// streaming kernel -> split-K kernel, K = 7168: N = 1536 at M = 1 / 16 / 32
// 13.7 / 13.9 / 17.5 -> 7.2 / 10.8 / 16.0, N = 576 13.4 / 13.5 / 17.3 -> 7.5 /
// 11.1 / 16.1, N = 4096 13.6 / 13.8 / 17.8 -> 9.6 / 12.0 / 16.5; 1 x 1536 x
// 2048 5.8 -> 4.2.  Above it the streaming kernel wins (7168 x 16384 at
// M = 32: 39 us against 61; 18432 x 7168: 26 against 72).  Four K blocks in
// flight per wave, or sixteen waves per workgroup, ran 0.3 - 1.5 us slower.
constexpr int kSplitkMaxN = 4096;

template <int MT>
hipError_t run_decode(const GemmParams& p, bool out_f32, hipStream_t stream) {
  const int cus = device_cus();
  const int groups = (p.N + 7) / 8;
  if constexpr (MT <= 2) {
    if (p.N <= kSplitkMaxN) {
      const int grid = (p.N + 15) / 16;
      if (out_f32) gemm_decode_splitk_kernel<MT, true><<<dim3(grid), dim3(512), 0, stream>>>(p);
      else gemm_decode_splitk_kernel<MT, false><<<dim3(grid), dim3(512), 0, stream>>>(p);
      return hipGetLastError();
    }
    // eight-wave kernel: rows per workgroup a multiple of 8, at most 72
    const int rows = 8 * std::min(kDecode8Rows / 8, (groups + cus - 1) / cus);
    const int grid = (p.N + rows - 1) / rows;
    // a_s as 16 bytes per row and stage: whole stages and 16-byte rows
    const bool ch = (p.K / 128) % 4 == 0 && ((uintptr_t)p.a_s & 15) == 0;
    if (out_f32) {
      if (ch) gemm_decode8_kernel<MT, true, true><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
      else gemm_decode8_kernel<MT, true, false><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
    } else {
      if (ch) gemm_decode8_kernel<MT, false, true><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
      else gemm_decode8_kernel<MT, false, false><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
    }
    return hipGetLastError();
  }
  // rows per workgroup: a multiple of 8 that spreads N over the CUs, at most 80
  const int rows = 8 * std::min(kDecodeMaxRows / 8, (groups + cus - 1) / cus);
  const int grid = (p.N + rows - 1) / rows;
  if (out_f32)
    gemm_decode_kernel<MT, true><<<dim3(grid), dim3(256), 0, stream>>>(p, rows);
  else
    gemm_decode_kernel<MT, false><<<dim3(grid), dim3(256), 0, stream>>>(p, rows);
  return hipGetLastError();
}

}  // namespace

// Time of a round of 128 x 128 tail tiles (two workgroups per CU) relative
// to a round of 256 x 256 tiles of the same K (measured ~65 vs ~108 us at
// K = 7168).
constexpr double kTailCost = 0.6;

template <bool E8>
hipError_t dense_gemm(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
                      int64_t M, int64_t N, int64_t K, bool out_f32, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a = (const uint8_t*)a; p.a_s = a_s; p.b = (const uint8_t*)b; p.b_s = b_s; p.c = c;
  p.offsets = nullptr; p.rows = (int)M; p.N = (int)N; p.K = (int)K; p.E = 0;
  if (M <= 16) return run_decode<1>(p, out_f32, stream);
  if (M <= 32) return run_decode<2>(p, out_f32, stream);
  if (M <= 64) return run_decode<4>(p, out_f32, stream);
  // The main tile: 256 x 256, eight waves of 128 (m) x 64 (n), two LDS
  // stages, the conflict-free swizzle (ue8m0: four waves of 128 x 128).
  constexpr int BM = 256, BN = 256;
  // Smaller GEMMs whose 256 x 256 tiles cannot fill the CUs, by their count
  // of 128 x 128 tiles t:
  //   t < CUs / 2, or 64 x 64 tiles that fit one round at two per CU ...
  //     64 x 64 tiles, four LDS stages, two workgroups per CU (measured:
  //     1024 x 1536 x 7168 104 -> 30 us against one 256 x 256 tile per CU,
  //     then 30.2 -> 27.9 us with four stages instead of three; these tiles
  //     are bound by operand fetch, 17 KB per 1 MFLOP K block; at t = CUs / 2
  //     they beat half the CUs on 128 x 128 tiles: 512 x 4096 x 7168 40.3 ->
  //     34.6 us, 512 x 4096 x 2048 14.3 -> 10.2 us);
  //   t <= CUs ....... 128 x 128 tiles, four stages, one workgroup per CU
  //     (three in flight: M x 18432 x 7168, M = 65 41.4 -> 39.9 us against
  //     three stages, 1000 x 2100 x 7168 42.2 -> 40.7 us);
  //   t <= 2 CUs ..... 128 x 128 tiles, two stages, two workgroups per CU: one
  //     round instead of two (M x 18432 x 7168, us: M = 192 87.7 -> 69.6,
  //     256 90.0 -> 79.0, 384 92.5 -> 76.1);
  //   beyond ......... the 256 x 256 tiles below, one partial round (M = 512:
  //     135.0 -> 107.1 us against three rounds of 128 x 128 tiles).
  const int cus = device_cus();
  auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (tiles(BM, BN) < cus && tiles(128, 128) <= 2 * cus) {
    const int t128 = tiles(128, 128);
    if (t128 > cus) {
      p.num_m = (int)((M + 127) / 128);
      p.num_n = (int)((N + 127) / 128);
      return run_tile<128, 128, 64, 64, 2, 4, 2, 2, E8>(p, out_f32, t128, stream);
    }
    if (t128 >= cus / 2 && tiles(64, 64) > 2 * cus) {
      p.num_m = (int)((M + 127) / 128);
      p.num_n = (int)((N + 127) / 128);
      return run_tile<128, 128, 64, 64, 4, 4, 2, 1, E8>(p, out_f32, t128, stream);
    }
    p.num_m = (int)((M + 63) / 64);
    p.num_n = (int)((N + 63) / 64);
    return run_tile<64, 64, 32, 32, 4, 4, 2, 2, E8>(p, out_f32, p.num_m * p.num_n, stream);
  }
  p.num_m = (int)((M + BM - 1) / BM);
  p.num_n = (int)((N + BN - 1) / BN);
  // One workgroup per CU, so a launch takes ceil(tiles / CUs) rounds of
  // equal tiles.  When the last round would be partly empty, the columns
  // past the last full round run as a second launch of 128 x 128 tiles, two
  // workgroups per CU (four times as many tiles, each a quarter of the work),
  // if the model full rounds + tail rounds x kTailCost beats one more full
  // round.
  const int64_t T = (int64_t)p.num_m * p.num_n;
  const int64_t full = T / cus * cus;
  if (BM == 256 && BN == 256 && T > cus && full != T && full % p.num_m == 0) {
    const int n_main = (int)(full / p.num_m);
    const int64_t tail_cols = N - (int64_t)n_main * BN;
    const int64_t tail_tiles = ((M + 127) / 128) * ((tail_cols + 127) / 128);
    const double split_cost = (double)(full / cus) + (double)((tail_tiles + 2 * cus - 1) / (2 * cus)) * kTailCost;
    if (split_cost < (double)((T + cus - 1) / cus)) {
      p.num_n = n_main;
      hipError_t e;
      if constexpr (E8) e = launch_gemm_e8_tile(p, out_f32, (int)full, stream);
      else e = run_tile<256, 256, 128, 64, 2, 8, 2, 1, E8>(p, out_f32, (int)full, stream);
      if (e != hipSuccess) return e;
      GemmParams q = p;
      q.n0 = n_main * BN;
      q.num_m = (int)((M + 127) / 128);
      q.num_n = (int)((tail_cols + 127) / 128);
      // 128 x 128 tiles of four waves (64 x 64 each), two stages, two
      // workgroups per CU (74 KB of LDS each): a barrier spans four waves
      // and the two workgroups fill each other's waits.  Measured against
      // one workgroup per CU of 128 x 256 tiles (eight waves, three stages):
      // prefill 513.6 -> 500.9 us, N = 18000 509.2 -> 493.9 us, ue8m0
      // prefill 468.3 -> 455.8 us.
      return run_tile<128, 128, 64, 64, 2, 4, 2, 2, E8>(q, out_f32, q.num_m * q.num_n, stream);
    }
  }
  // The ue8m0 path's 256 x 256 tiles run on four waves (gemm_e8.hip).
  if constexpr (E8) return launch_gemm_e8_tile(p, out_f32, p.num_m * p.num_n, stream);
  else return run_tile<256, 256, 128, 64, 2, 8, 2, 1, E8>(p, out_f32, p.num_m * p.num_n, stream);
}

hipError_t launch_gemm(const void* a, const float* a_s, const void* b, const float* b_s, void* c,
                       int64_t M, int64_t N, int64_t K, bool out_f32, hipStream_t stream) {
  return dense_gemm<false>(a, a_s, b, b_s, c, M, N, K, out_f32, stream);
}

// The ue8m0 fast path: the same tile choice, scales applied by the MFMA; its
// 256 x 256 tiles run on the four-wave kernel of gemm_e8.hip (decode-sized M
// keeps the decode kernel, which handles any scales).
hipError_t launch_gemm_ue8m0(const void* a, const float* a_s, const void* b, const float* b_s,
                             void* c, int64_t M, int64_t N, int64_t K, bool out_f32,
                             hipStream_t stream) {
  return dense_gemm<true>(a, a_s, b, b_s, c, M, N, K, out_f32, stream);
}

hipError_t launch_moe_gemm(const void* a, const float* a_s, const void* b, const float* b_s,
                           const int32_t* offsets, void* c, int64_t R, int64_t E, int64_t N,
                           int64_t K, bool out_f32, hipStream_t stream) {
  if (R == 0 || E == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a = (const uint8_t*)a; p.a_s = a_s; p.b = (const uint8_t*)b; p.b_s = b_s; p.c = c;
  p.offsets = offsets; p.rows = (int)R; p.N = (int)N; p.K = (int)K; p.E = (int)E;
  // Few experts: the small-expert tiles are 64 or 128 columns wide when even
  // every expert holding rows would give no more such tiles than CUs, so the
  // weight stream spreads over more CUs in one round.  A narrow tile streams
  // less per CU than a 64 x 256 one (its fixed per-K-block cost is spread
  // over fewer bytes), so it pays only when it needs no second round:
  // 8 experts x 16 rows, N = 2048, K = 7168: 56.6 -> 38.4 us with 64-column
  // tiles, 16 experts 67.1 -> 44.2 us with 128-column ones, while 31 experts
  // on 64-column tiles (four rounds) went 78.8 -> 139.3 us.
  const int64_t cus = device_cus();
  p.small_bn = E * ((N + 63) / 64) <= cus ? 64 : E * ((N + 127) / 128) <= cus ? 128 : 256;
  const int64_t nns = (N + p.small_bn - 1) / p.small_bn;
  // Upper bounds on each class's m tiles: the large experts' sum of
  // ceil(rows / side) <= R / side + (number of such experts), with at most
  // R / (kMoeSplit + 1) of them; one small tile per expert with rows.
  const int64_t nlarge = std::min<int64_t>(E, R / (kMoeSplit + 1));
  // The large experts' tiles are 128 x 128 when there can be no more than
  // two rounds of them (N = 2048, K = 7168, us: 8 experts x 200 rows 90.8 ->
  // 53.2, 4 x 300 88.4 -> 45.9, 16 x 100 71.4 -> 55.1), else 256 x 256: with
  // more 128 x 128 rounds the narrower tiles lose (12 x 300 94.9 -> 117.9,
  // 8 x 700 97.2 -> 130.9).  Below K = 4096 a tile's fixed cost weighs more
  // against its K loop and only one round is allowed (N = 7168, K = 2048:
  // 1 x 1000 rows 32.8 -> 35.1 and 2 x 500 31.8 -> 33.8 us with two).
  const int64_t rounds = K >= 4096 ? 2 : 1;
  p.large_sh = (R / 128 + nlarge) * ((N + 127) / 128) <= rounds * cus ? 7 : 8;
  const int64_t ml = (R >> p.large_sh) + nlarge;
  p.num_n = (int)((N + (1 << p.large_sh) - 1) >> p.large_sh);
  const int64_t ms = std::min<int64_t>(E, R);
  // each XCD's part of a class list is at most ceil(tiles / 8)
  const int64_t grid = 8 * ((ml * p.num_n + 7) / 8 + (ms * nns + 7) / 8);
  const bool chunked = (K / 128) % 4 == 0 && ((uintptr_t)a_s & 15) == 0;
  const dim3 g((unsigned)grid), blk(512);
  if (chunked) {
    if (out_f32) moe_gemm_kernel<true, true><<<g, blk, 0, stream>>>(p);
    else moe_gemm_kernel<true, false><<<g, blk, 0, stream>>>(p);
  } else {
    if (out_f32) moe_gemm_kernel<false, true><<<g, blk, 0, stream>>>(p);
    else moe_gemm_kernel<false, false><<<g, blk, 0, stream>>>(p);
  }
  return hipGetLastError();
}

// The grid of p.num_m x p.num_n tiles (columns from p.n0 on).
template <int BM, int BN, int WM, int WN, int NW, int ST, int OCC>
hipError_t run_w8a16_grid(const GemmParams& p, bool out_f32, hipStream_t stream) {
  const dim3 grid((unsigned)(p.num_m * p.num_n)), block(NW * 64);
  if (out_f32)
    w8a16_tile_kernel<BM, BN, WM, WN, NW, ST, OCC, true><<<grid, block, 0, stream>>>(p);
  else
    w8a16_tile_kernel<BM, BN, WM, WN, NW, ST, OCC, false><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int NW, int ST, int OCC>
hipError_t run_w8a16(GemmParams p, bool out_f32, hipStream_t stream) {
  p.num_m = (int)((p.rows + BM - 1) / BM);
  p.num_n = (int)((p.N + BN - 1) / BN);
  return run_w8a16_grid<BM, BN, WM, WN, NW, ST, OCC>(p, out_f32, stream);
}

// Tile choice: decode-sized M streams the weight through 64-column tiles
// (two workgroups per CU, six stages); GEMMs whose 256 x 256 tiles cannot
// fill the CUs use 64-row tiles while 128 x 128 ones would not reach half
// the CUs, then 128 x 128 tiles, one workgroup per CU while those fit the
// CUs and two per CU (three stages) up to twice that (one round instead of
// two: M x 18432 x 7168, M = 192 166.2 -> 101.1 us, 256 166.4 -> 103.9, 384
// 173.8 -> 118.4); beyond, and for the rest, the 256 x 256 eight-wave tile
// (M = 512: 248.6 -> 175.3 us against three rounds of 128 x 128 tiles).
hipError_t launch_w8a16_gemm(const void* x, const void* w, const float* w_s, void* c, int64_t M,
                             int64_t N, int64_t K, bool out_f32, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  GemmParams p{};
  p.a = (const uint8_t*)x; p.a_s = nullptr; p.b = (const uint8_t*)w; p.b_s = w_s; p.c = c;
  p.offsets = nullptr; p.rows = (int)M; p.N = (int)N; p.K = (int)K; p.E = 0;
  if (M <= 32 && N <= kSplitkMaxN) {
    // few weight rows: K split over the waves (gemm_decode_splitk_kernel),
    // the FP8 path's rule.  Same box, us, streaming -> split-K, K = 7168:
    // N = 1536 at M = 1 / 16 / 32 21.5 / 21.8 / 24.7 -> 7.8 / 12.6 / 21.1,
    // N = 4096 22.1 / 22.0 / 24.5 -> 9.7 / 13.6 / 22.6; 1 x 1536 x 2048
    // 8.0 -> 4.4.
    const int grid = (int)((N + 15) / 16);
    if (M <= 16) {
      if (out_f32) gemm_decode_splitk_kernel<1, true, true><<<dim3(grid), dim3(512), 0, stream>>>(p);
      else gemm_decode_splitk_kernel<1, false, true><<<dim3(grid), dim3(512), 0, stream>>>(p);
    } else {
      if (out_f32) gemm_decode_splitk_kernel<2, true, true><<<dim3(grid), dim3(512), 0, stream>>>(p);
      else gemm_decode_splitk_kernel<2, false, true><<<dim3(grid), dim3(512), 0, stream>>>(p);
    }
    return hipGetLastError();
  }
  if (M <= 32) {
    // eight-wave streaming kernel: rows per workgroup a multiple of 8, at most 72
    const int cus = device_cus();
    const int rows = 8 * std::min(kDecode8Rows / 8, ((int)((N + 7) / 8) + cus - 1) / cus);
    const int grid = (int)((N + rows - 1) / rows);
    if (M <= 16) {
      if (out_f32) w8a16_decode8_kernel<1, true><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
      else w8a16_decode8_kernel<1, false><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
    } else {
      if (out_f32) w8a16_decode8_kernel<2, true><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
      else w8a16_decode8_kernel<2, false><<<dim3(grid), dim3(512), 0, stream>>>(p, rows);
    }
    return hipGetLastError();
  }
  if (M <= 64) return run_w8a16<64, 64, 64, 16, 4, 6, 2>(p, out_f32, stream);
  const int cus = device_cus();
  const int64_t big_tiles = ((M + 255) / 256) * ((N + 255) / 256);
  if (big_tiles < cus) {
    const int64_t t128 = ((M + 127) / 128) * ((N + 127) / 128);
    // too few 128 x 128 tiles for half the CUs, or 64-row tiles that fit one
    // round at two per CU: the 64-row tiles (128 x 7168 x 18432 208.7 ->
    // 109.6 us, 100 x 4096 x 7168 83.2 -> 43.7, 512 x 4096 x 7168 86.7 -> 56.5)
    const int64_t t64 = ((M + 63) / 64) * ((N + 63) / 64);
    if (t128 < cus / 2 || t64 <= 2 * cus) return run_w8a16<64, 64, 64, 16, 4, 6, 2>(p, out_f32, stream);
    if (t128 <= cus) return run_w8a16<128, 128, 64, 64, 4, 4, 1>(p, out_f32, stream);
    if (t128 <= 2 * cus) return run_w8a16<128, 128, 64, 64, 4, 3, 2>(p, out_f32, stream);
  }
  // As in the FP8 GEMM: when the last round of 256 x 256 tiles would be
  // partly empty, the columns past the last full round run as a second launch
  // of 128 x 128 tiles (four waves, three stages) two workgroups per CU, if
  // full rounds + tail rounds x kTailCost beats one more full round.
  p.num_m = (int)((M + 255) / 256);
  p.num_n = (int)((N + 255) / 256);
  const int64_t full = big_tiles / cus * cus;
  if (full != big_tiles && full % p.num_m == 0) {
    const int n_main = (int)(full / p.num_m);
    const int64_t tail_cols = N - (int64_t)n_main * 256;
    const int64_t tail_tiles = ((M + 127) / 128) * ((tail_cols + 127) / 128);
    const double split_cost = (double)(full / cus) + (double)((tail_tiles + 2 * cus - 1) / (2 * cus)) * kTailCost;
    if (split_cost < (double)((big_tiles + cus - 1) / cus)) {
      p.num_n = n_main;
      hipError_t e = run_w8a16_grid<256, 256, 128, 64, 8, 3, 1>(p, out_f32, stream);
      if (e != hipSuccess) return e;
      GemmParams q = p;
      q.n0 = n_main * 256;
      q.num_m = (int)((M + 127) / 128);
      q.num_n = (int)((tail_cols + 127) / 128);
      return run_w8a16_grid<128, 128, 64, 64, 4, 3, 2>(q, out_f32, stream);
    }
  }
  return run_w8a16_grid<256, 256, 128, 64, 8, 3, 1>(p, out_f32, stream);
}

}  // namespace fp8bs
