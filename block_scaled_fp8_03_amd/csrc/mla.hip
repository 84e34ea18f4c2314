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
//
// bf16 outputs leave through LDS: each 16-token tile of the workgroup's
// columns is staged there and written out as whole contiguous rows, so every
// store instruction covers whole cache lines.  The large stream of a launch
// (the key side's output, the value side's input) takes the non-temporal hint
// when it is at least the 256 MiB of the Infinity Cache, which it could not
// stay in anyway; below that the cache absorbs it and the hint costs time.
// Same-box timings, 128 heads, R = 512, bf16 out (us; before -> after):
// key 4096 tokens 157.5 -> 102.0, 2048 tokens 101.2 -> 52.2, 1536 tokens
// 49.1 -> 43.7, 1000 tokens 31.6 -> 29.5; value 4096 tokens 129.4 -> 117.1,
// 2048 tokens 66.7 -> 62.2, 1536 and 1000 tokens unchanged (45.0 -> 42.7,
// 28.9 -> 28.8).  Below the cut the hint cost: key 1536 tokens 47.5 us with
// it, value 1536 tokens 50.9.
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

// The q tile of 16 tokens (16 rows of DN bf16) is shared by the workgroup's
// waves through a double-buffered LDS tile, chunk c of row r at c ^ r (as in
// the value kernel; conflict-free for these reads too): the threads load it
// one tile ahead into registers (threads past the tile's chunks load
// duplicates, which write the same bytes), so no wave loads what the others
// also need.  A bf16 result tile (16 tokens x the workgroup's 64 NWK columns)
// is staged in a second double-buffered LDS tile, 16-byte chunk c of row r at
// c ^ r, and written out after the barrier that ends the iteration; NT puts
// the non-temporal hint on those stores.
template <int DN, int NWK, bool OUT_F32, bool NT>
__global__ void __launch_bounds__(64 * NWK) mla_key_kernel(MlaParams p) {
  constexpr int KS = DN / 32;                       // MFMA K steps
  constexpr int CPR = DN / 8;                       // 16-byte chunks per q row
  constexpr int ROW_BYTES = CPR * 16;
  constexpr int TOTAL = 16 * CPR;                   // chunks per tile
  constexpr int NL = (TOTAL + 64 * NWK - 1) / (64 * NWK);
  constexpr int OCPR = NWK * 8;                     // 16-byte chunks per staged bf16 row
  static_assert(OCPR % 16 == 0, "row swizzle");
  __shared__ __attribute__((aligned(16))) uint8_t qs[2][16 * ROW_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t os[2][OUT_F32 ? 16 : 16 * OCPR * 16];

  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int c0 = (blockIdx.y * NWK + wave) * 64;
  const bool active = c0 < p.R;                     // idle waves still load and sync
  const int cw = active ? c0 : 0;
  const int h = blockIdx.x % p.H;
  const int t_begin = (blockIdx.x / p.H) * p.tch;
  const int t_end = min(p.T, t_begin + p.tch);
  const int ntiles = (t_end - t_begin + 15) / 16;
  const int row0 = h * (p.dn + p.dv);

  auto load_tile = [&](int tile, v4u (&qr)[NL]) {
    const int t0 = t_begin + 16 * tile;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = (threadIdx.x + 64 * NWK * i) % TOTAL;
      const int tl = min(t0 + q / CPR, t_end - 1);  // rows past the end load the last row
      const uint16_t* src = p.in + (size_t)tl * p.ld_t + (size_t)h * p.ld_h + 8 * (q % CPR);
      qr[i] = *reinterpret_cast<const v4u*>(src);
    }
  };
  auto store_tile = [&](int b, const v4u (&qr)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = (threadIdx.x + 64 * NWK * i) % TOTAL;
      const int r = q / CPR, c = q % CPR;
      *reinterpret_cast<v4u*>(&qs[b][r * ROW_BYTES + ((c ^ r) << 4)]) = qr[i];
    }
  };

  v4u qr[NL];
  load_tile(0, qr);

  // weight fragments, dequantised once for the whole token chunk
  v8bf wf[KS][4];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    const float sc = p.ws[((row0 + 32 * s) >> 7) * (p.R >> 7) + (cw >> 7)];
    const uint8_t* base = p.w + (size_t)(row0 + 32 * s + 8 * g) * p.R + cw + 4 * j;
    uint32_t wd[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wd[i] = *reinterpret_cast<const uint32_t*>(base + (size_t)i * p.R);
    uint32_t lo[4], hi[4];
    transpose4x4_b8(wd, lo);
    transpose4x4_b8(wd + 4, hi);
#pragma unroll
    for (int u = 0; u < 4; ++u) wf[s][u] = dequant8_bf16(lo[u], hi[u], sc);
  }

  store_tile(0, qr);
  load_tile(min(1, ntiles - 1), qr);
  __syncthreads();

  // One token tile; `next` stages the next tile and loads the one after it.
  // The last tile is peeled off without them: its iteration then does not
  // wait for a reload nobody reads before its barrier and stores.
  auto iter = [&](int it, bool next) {
    const int b = it & 1;
    if (active) {
      const uint8_t* row = qs[b] + j * ROW_BYTES;
      v4f acc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int c = 4 * s + g;                      // d = 32 s + 8 g .. + 8
        const v8bf qf = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(row + ((c ^ j) << 4)));
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = mfma_bf16(wf[s][u], qf, acc[u]);
      }
      // lane (g, t) owns columns c0 + 16g + e, e = 4r + u
      if (OUT_F32) {
        // Rows past the end computed the last row's q, so their results equal
        // that row's: they are stored there (the same bytes twice), which
        // keeps the stores out of a branch.
        const int ts = min(t_begin + 16 * it + j, t_end - 1);
        float* out = reinterpret_cast<float*>(p.out) + ((size_t)ts * p.H + h) * p.R + c0 + 16 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<v4f*>(out + 4 * r) = v4f{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
      } else {
#pragma unroll
        for (int r = 0; r < 4; r += 2) {
          const v4u v = {pack2_bf16(acc[0][r], acc[1][r]), pack2_bf16(acc[2][r], acc[3][r]),
                         pack2_bf16(acc[0][r + 1], acc[1][r + 1]), pack2_bf16(acc[2][r + 1], acc[3][r + 1])};
          const int ch = wave * 8 + 2 * g + (r >> 1);
          *reinterpret_cast<v4u*>(&os[b][j * (OCPR * 16) + ((ch ^ j) << 4)]) = v;
        }
      }
    }
    if (next) {
      store_tile(b ^ 1, qr);
      load_tile(min(it + 2, ntiles - 1), qr);
    }
    __syncthreads();
    if (!OUT_F32) {
      // The staged tile out, two chunks per thread.  Chunks past R (idle
      // waves) clamp to the row's last real chunk and rows past the end to
      // the last row, whose results they hold: every store writes bytes that
      // are correct for its address, with no branch.  os[b] is written again
      // two iterations on, after the next barrier.
      const int cbase = blockIdx.y * NWK * 64;
      const int last_ch = min(OCPR, (p.R - cbase) / 8) - 1;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        const int q = threadIdx.x + 64 * NWK * pass;
        const int r = q / OCPR;
        const int ch = min(q % OCPR, last_ch);
        const int ts = min(t_begin + 16 * it + r, t_end - 1);
        const v4u v = *reinterpret_cast<const v4u*>(&os[b][r * (OCPR * 16) + ((ch ^ r) << 4)]);
        uint16_t* dst = reinterpret_cast<uint16_t*>(p.out) + ((size_t)ts * p.H + h) * p.R + cbase + 8 * ch;
        if (NT) store_nt(reinterpret_cast<uint4*>(dst), __builtin_bit_cast(uint4, v));
        else *reinterpret_cast<v4u*>(dst) = v;
      }
    }
  };
  for (int it = 0; it + 1 < ntiles; ++it) iter(it, true);
  iter(ntiles - 1, false);
}

// ---------------------------------------------------------------------------
// Value side.  Wave = one head, 32 value columns d0 .. d0+31 (two MFMA row
// tiles), a chunk of tokens; the NWV waves of a workgroup take consecutive
// 32-column groups of the same head and tokens.  The contraction runs along
// the weight's rows (c): for each 64-wide slice s' of c, lane (j, g) holds the
// 16 weight bytes [64s' + 16g, +16) of row d0 + 16ct + j (K steps 2s' and
// 2s'+1 take bytes 0..7 and 8..15) and the 16 bf16 of x at the same c.
// Output register r of lane (g', t) is column d0 + 16ct + 4g' + r.
// The x tile of 16 tokens (16 rows of R bf16) is shared through LDS: each
// wave loads 16/NWV of its rows into registers one tile ahead and writes them
// to a double-buffered LDS tile, 16-byte chunk c of row r at c ^ r (found by
// exhaustive search to keep the fragment reads conflict-free under the
// measured bank rule); every wave then reads its fragments from LDS (before,
// each wave loaded the whole tile itself: four times the load instructions).
// NT puts the non-temporal hint on the x loads.  A bf16 result tile (16
// tokens x the workgroup's 32 NWV columns) is staged in LDS, chunk c of row r
// at c ^ (r mod chunks per row), and written out as whole rows after the
// barrier that ends the iteration.
// ---------------------------------------------------------------------------
template <int RK, int NWV, bool OUT_F32, bool NT>
__global__ void __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2, 2)))
mla_value_kernel(MlaParams p) {
  constexpr int CPR = RK * 8;                       // 16-byte chunks per x row (R / 8)
  constexpr int ROW_BYTES = CPR * 16;
  constexpr int TILE_BYTES = 16 * ROW_BYTES;
  constexpr int NL = 16 * CPR / (64 * NWV);         // 16-byte loads per lane per tile
  static_assert(16 * CPR % (64 * NWV) == 0, "tile split");
  constexpr int OCPR = NWV * 4;                     // 16-byte chunks per staged bf16 row
  static_assert(16 * OCPR == 64 * NWV, "one staged chunk per thread");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t os[2][OUT_F32 ? 16 : 16 * OCPR * 16];

  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int d0 = (blockIdx.y * NWV + wave) * 32;
  const bool active = d0 < p.dv;                    // idle waves still load and sync
  const int h = blockIdx.x % p.H;
  const int t_begin = (blockIdx.x / p.H) * p.tch;
  const int t_end = min(p.T, t_begin + p.tch);
  const int ntiles = (t_end - t_begin + 15) / 16;
  const int vrow0 = h * (p.dn + p.dv) + p.dn + (active ? d0 : 0);

  // this thread's share of a tile: load q = tid + 64 NWV i, row q / CPR,
  // chunk q % CPR (rows past the end load the last row)
  auto load_tile = [&](int tile, v4u (&xr)[NL]) {
    const int t0 = t_begin + 16 * tile;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = threadIdx.x + 64 * NWV * i;
      const int tl = min(t0 + q / CPR, t_end - 1);
      const uint16_t* x = p.in + (size_t)tl * p.ld_t + (size_t)h * p.ld_h + 8 * (q % CPR);
      if (NT) xr[i] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(x));
      else xr[i] = *reinterpret_cast<const v4u*>(x);
    }
  };
  auto store_tile = [&](int b, const v4u (&xr)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = threadIdx.x + 64 * NWV * i;
      const int r = q / CPR, c = q % CPR;
      *reinterpret_cast<v4u*>(&xs[b][r * ROW_BYTES + ((c ^ r) << 4)]) = xr[i];
    }
  };

  v4u xr[NL];
  load_tile(0, xr);

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

  store_tile(0, xr);
  load_tile(min(1, ntiles - 1), xr);
  __syncthreads();

  // One token tile; the last is peeled off without staging or loading a
  // next one (as in the key kernel).
  auto iter = [&](int i, bool next) {
    const int b = i & 1;
    if (active) {
      const uint8_t* row = xs[b] + j * ROW_BYTES;
      v4f acc[2][2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[ct][0] = acc[ct][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < RK; ++s)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int c = 8 * s + 2 * g + k;            // x[16 s' ... ] chunk of this lane
          const v8bf xf = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(row + ((c ^ j) << 4)));
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) acc[ct][k] = mfma_bf16(wf[ct][s][k], xf, acc[ct][k]);
        }
      const int ts = min(t_begin + 16 * i + j, t_end - 1);   // as in the key kernel
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const v4f v = acc[ct][0] + acc[ct][1];
        if (OUT_F32) {
          const size_t o = ((size_t)ts * p.H + h) * p.dv + d0 + 16 * ct + 4 * g;
          *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + o) = v;
        } else {
          // columns d0 + 16 ct + 4 g .. + 3: half g & 1 of staged chunk c
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          const int c = wave * 4 + 2 * ct + (g >> 1);
          *reinterpret_cast<v2u*>(&os[b][j * (OCPR * 16) + ((c ^ (j & (OCPR - 1))) << 4) + 8 * (g & 1)]) =
              v2u{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
        }
      }
    }
    // the next tile into the other buffer (last read one iteration ago, behind
    // the barrier that ended it), then the loads of the tile after it
    if (next) {
      store_tile(b ^ 1, xr);
      load_tile(min(i + 2, ntiles - 1), xr);
    }
    __syncthreads();
    if (!OUT_F32) {
      // the staged tile out, one chunk per thread, clamped as in the key
      // kernel (chunks past dv to the row's last real chunk, rows past the
      // end to the last row)
      const int cbase = blockIdx.y * NWV * 32;
      const int last_ch = min(OCPR, (p.dv - cbase) / 8) - 1;
      const int r = threadIdx.x / OCPR;
      const int ch = min((int)threadIdx.x % OCPR, last_ch);
      const int tr = min(t_begin + 16 * i + r, t_end - 1);
      const v4u v = *reinterpret_cast<const v4u*>(&os[b][r * (OCPR * 16) + ((ch ^ (r & (OCPR - 1))) << 4)]);
      *reinterpret_cast<v4u*>(reinterpret_cast<uint16_t*>(p.out) + ((size_t)tr * p.H + h) * p.dv + cbase + 8 * ch) = v;
    }
  };
  for (int i = 0; i + 1 < ntiles; ++i) iter(i, true);
  iter(ntiles - 1, false);
}

// Value side at decode sizes (T <= 64): a workgroup of NS waves owns one
// head, 32 value columns d0 .. d0+31 and the token chunk, and wave w takes
// the latent slices w RK/NS .. (w+1) RK/NS - 1 of the contraction.  With one
// wave per 32 columns (the kernel above on one-wave workgroups, as this size
// ran before), 128 heads gave 512 waves that each loaded 16 KB of weight
// before any compute; here four (two) times as many waves each wait for a
// quarter (half) of that.  The x tile is shared through LDS as in the kernel
// above.  After each
// token tile's MFMAs the waves' partial sums meet in LDS, and after the
// tile's barrier wave 0 adds them in wave order and writes the 16 x 32
// result (bf16: staged in LDS and stored as whole 64-byte rows).  Same box,
// 128 heads, R = 512, bf16 out, graph-replayed, us (one-wave kernel -> this):
// 32 tokens 5.82-5.93 -> 4.31-4.47, 64 tokens 7.96-7.99 -> 5.70-5.75,
// 1 token 4.50-4.52 -> 3.51-3.52; eight waves of one slice each: 4.68 at 32
// tokens.  (The key side split the same way over its d rows ran slower,
// 4.04 -> 5.93 us at 32 tokens: its 16 x 64 result per tile is four times
// the partial sums to meet in LDS, and one wave to write out.)
// ---------------------------------------------------------------------------
template <int RK, int NS, bool OUT_F32>
__global__ void __launch_bounds__(64 * NS) mla_value_split_kernel(MlaParams p) {
  constexpr int CPR = RK * 8;                       // 16-byte chunks per x row (R / 8)
  constexpr int ROW_BYTES = CPR * 16;
  constexpr int TILE_BYTES = 16 * ROW_BYTES;
  constexpr int NL = 16 * CPR / (64 * NS);          // 16-byte loads per lane per tile
  constexpr int SPW = RK / NS;                      // latent slices per wave
  static_assert(RK % NS == 0 && 16 * CPR % (64 * NS) == 0, "split");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][TILE_BYTES];
  __shared__ __attribute__((aligned(16))) v4f red[2][NS][2][64];
  __shared__ __attribute__((aligned(16))) uint8_t os[2][OUT_F32 ? 16 : 16 * 64];

  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int d0 = blockIdx.y * 32;                   // dv % 32 == 0: every column is real
  const int h = blockIdx.x % p.H;
  const int t_begin = (blockIdx.x / p.H) * p.tch;
  const int t_end = min(p.T, t_begin + p.tch);
  const int ntiles = (t_end - t_begin + 15) / 16;
  const int vrow0 = h * (p.dn + p.dv) + p.dn + d0;
  const int s0 = wave * SPW;

  auto load_tile = [&](int tile, v4u (&xr)[NL]) {
    const int t0 = t_begin + 16 * tile;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = threadIdx.x + 64 * NS * i;
      const int tl = min(t0 + q / CPR, t_end - 1);
      xr[i] = *reinterpret_cast<const v4u*>(p.in + (size_t)tl * p.ld_t + (size_t)h * p.ld_h + 8 * (q % CPR));
    }
  };
  auto store_tile = [&](int b, const v4u (&xr)[NL]) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int q = threadIdx.x + 64 * NS * i;
      const int r = q / CPR, c = q % CPR;
      *reinterpret_cast<v4u*>(&xs[b][r * ROW_BYTES + ((c ^ r) << 4)]) = xr[i];
    }
  };

  v4u xr[NL];
  load_tile(0, xr);

  v8bf wf[2][SPW][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const uint8_t* base = p.w + (size_t)(vrow0 + 16 * ct + j) * p.R + 16 * g;
    const float* sc = p.ws + (size_t)(vrow0 >> 7) * (p.R >> 7);
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int s = s0 + u;
      const v4u wv = *reinterpret_cast<const v4u*>(base + 64 * s);
      const float scale = sc[s >> 1];
      wf[ct][u][0] = dequant8_bf16(wv.x, wv.y, scale);
      wf[ct][u][1] = dequant8_bf16(wv.z, wv.w, scale);
    }
  }

  store_tile(0, xr);
  load_tile(min(1, ntiles - 1), xr);
  __syncthreads();

  auto iter = [&](int i, bool next) {
    const int b = i & 1;
    const uint8_t* row = xs[b] + j * ROW_BYTES;
    v4f acc[2][2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[ct][0] = acc[ct][1] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < SPW; ++u)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int c = 8 * (s0 + u) + 2 * g + k;
        const v8bf xf = __builtin_bit_cast(v8bf, *reinterpret_cast<const v4u*>(row + ((c ^ j) << 4)));
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[ct][k] = mfma_bf16(wf[ct][u][k], xf, acc[ct][k]);
      }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) red[b][wave][ct][lane] = acc[ct][0] + acc[ct][1];
    if (next) {
      store_tile(b ^ 1, xr);
      load_tile(min(i + 2, ntiles - 1), xr);
    }
    __syncthreads();
    if (wave == 0) {
      const int ts = min(t_begin + 16 * i + j, t_end - 1);   // rows past the end: the last row's result
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        v4f v = red[b][0][ct][lane];
#pragma unroll
        for (int w = 1; w < NS; ++w) v += red[b][w][ct][lane];
        if (OUT_F32) {
          const size_t o = ((size_t)ts * p.H + h) * p.dv + d0 + 16 * ct + 4 * g;
          *reinterpret_cast<v4f*>(reinterpret_cast<float*>(p.out) + o) = v;
        } else {
          // columns 16 ct + 4 g .. + 3: half g & 1 of chunk 2 ct + (g >> 1) of row j
          typedef uint32_t v2u __attribute__((ext_vector_type(2)));
          const int c = 2 * ct + (g >> 1);
          *reinterpret_cast<v2u*>(&os[b][j * 64 + ((c ^ (j & 3)) << 4) + 8 * (g & 1)]) =
              v2u{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
        }
      }
      if (!OUT_F32) {
        // the wave's own LDS writes above are complete before its reads
        __builtin_amdgcn_s_waitcnt(0xc07f);          // lgkmcnt(0)
        __builtin_amdgcn_wave_barrier();
        const int r = lane >> 2, ch = lane & 3;
        const int tr = min(t_begin + 16 * i + r, t_end - 1);
        const v4u v = *reinterpret_cast<const v4u*>(&os[b][r * 64 + ((ch ^ (r & 3)) << 4)]);
        *reinterpret_cast<v4u*>(reinterpret_cast<uint16_t*>(p.out) + ((size_t)tr * p.H + h) * p.dv + d0 + 8 * ch) = v;
      }
    }
  };
  for (int i = 0; i + 1 < ntiles; ++i) iter(i, true);
  iter(ntiles - 1, false);
}

// Token chunking, evenly split, a multiple of 16: the largest chunk of 1024,
// 512 or 256 tokens that still gives at least 512 workgroups (two per CU)
// over the heads, else 256, or less when even that leaves CUs idle (below).  Longer chunks load each head's weight fewer
// times (measured, 128 heads: 4096 tokens key 167.3 -> 157.5 us and value
// 131.4 -> 127.4 us with 1024-token chunks against 256; 2048 tokens value
// 64.6 -> 62.0 us with 512), but a grid below two workgroups per CU lost
// more than that (1000 tokens in 1024-token chunks: 30 -> 57 us).
// Streams at least this large (the 256 MiB Infinity Cache) take the
// non-temporal hint.
constexpr int64_t kStreamBytes = int64_t(256) << 20;

void chunk_tokens(MlaParams& p) {
  int cap = 256;
  for (int c : {1024, 512})
    if ((int64_t)p.H * ((p.T + c - 1) / c) >= 512) {
      cap = c;
      break;
    }
  // Fewer 256-token workgroups than CUs: 128- or 64-token chunks, re-reading
  // the weight per chunk rather than leaving CUs idle (128 heads, us, key /
  // value: 72 tokens 7.54 / 7.39 -> 6.60 / 6.27, 128 tokens 9.80 / 9.57 ->
  // 8.19 / 7.34, 256 tokens 14.9 / 14.7 -> 11.2 / 10.7; asking for two
  // workgroups per CU at every size lost at 384 and 640 tokens, 13.5 -> 15.7
  // and 20.0 -> 22.6 us on the key side).
  if (cap == 256 && (int64_t)p.H * ((p.T + 255) / 256) < 256)
    cap = (int64_t)p.H * ((p.T + 127) / 128) >= 256 ? 128 : 64;
  p.n_tch = std::max(1, (p.T + cap - 1) / cap);
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
  // latent columns (eight waves), so the chunk's q tile is loaded once for
  // all of them; at decode sizes four-wave workgroups spread the weight over
  // more CUs
  const bool wide = T > 64 && R >= 512;
  const int waves = wide ? 8 : 4;
  const dim3 grid((unsigned)(H * p.n_tch), (unsigned)((R / 64 + waves - 1) / waves));
  const dim3 block(64 * waves);
  // the bf16 output is the launch's large stream
  const bool nt = !out_f32 && T * H * R * 2 >= kStreamBytes;
#define FP8BS_MLA_K(DN_)                                                                              \
  if (wide) {                                                                                       \
    if (out_f32) hipLaunchKernelGGL((mla_key_kernel<DN_, 8, true, false>), grid, block, 0, stream, p); \
    else if (nt) hipLaunchKernelGGL((mla_key_kernel<DN_, 8, false, true>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((mla_key_kernel<DN_, 8, false, false>), grid, block, 0, stream, p);     \
  } else {                                                                                          \
    if (out_f32) hipLaunchKernelGGL((mla_key_kernel<DN_, 4, true, false>), grid, block, 0, stream, p); \
    else hipLaunchKernelGGL((mla_key_kernel<DN_, 4, false, false>), grid, block, 0, stream, p);    \
  }
  if (dn == 128) {
    FP8BS_MLA_K(128)
  } else {
    FP8BS_MLA_K(256)
  }
#undef FP8BS_MLA_K
  return hipGetLastError();
}

hipError_t launch_mla_absorb_value(const void* x, int64_t ld_t, int64_t ld_h, const void* w,
                                   const float* ws, void* out, int64_t T, int64_t H, int64_t dn,
                                   int64_t dv, int64_t R, bool out_f32, hipStream_t stream) {
  MlaParams p{static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(w), ws, out, (int)T,
              (int)H, (int)dn, (int)dv, (int)R, (int)ld_t, (int)ld_h, 0, 0};
  chunk_tokens(p);
  // at most 64 tokens: the latent split over two or four waves of a
  // workgroup per 32 value columns (mla_value_split_kernel); otherwise four
  // waves (one head's 128 value columns), so the waves that use the same x
  // rows share them through LDS
  const bool wide = T > 64;
  const int ns = (R / 64) % 4 == 0 ? 4 : 2;
  const int waves = wide ? 4 : 1;
  const dim3 grid((unsigned)(H * p.n_tch), (unsigned)((dv / 32 + waves - 1) / waves));
  const dim3 block(64 * (wide ? waves : ns));
  // x is the launch's large stream
  const bool nt = T * H * R * 2 >= kStreamBytes;
#define FP8BS_MLA_V4(RK_, F32_)                                                                     \
  if (nt) hipLaunchKernelGGL((mla_value_kernel<RK_, 4, F32_, true>), grid, block, 0, stream, p);    \
  else hipLaunchKernelGGL((mla_value_kernel<RK_, 4, F32_, false>), grid, block, 0, stream, p);
#define FP8BS_MLA_V(RK_)                                                                            \
  case RK_:                                                                                         \
    if (wide) {                                                                                     \
      if (out_f32) {                                                                                \
        FP8BS_MLA_V4(RK_, true)                                                                     \
      } else {                                                                                      \
        FP8BS_MLA_V4(RK_, false)                                                                    \
      }                                                                                             \
    } else {                                                                                        \
      constexpr int NS_ = RK_ % 4 == 0 ? 4 : 2;                                                   \
      if (out_f32) hipLaunchKernelGGL((mla_value_split_kernel<RK_, NS_, true>), grid, block, 0, stream, p); \
      else hipLaunchKernelGGL((mla_value_split_kernel<RK_, NS_, false>), grid, block, 0, stream, p); \
    }                                                                                               \
    break;
  switch (R / 64) {
    FP8BS_MLA_V(2)
    FP8BS_MLA_V(4)
    FP8BS_MLA_V(6)
    FP8BS_MLA_V(8)
    default: return hipErrorInvalidValue;
  }
#undef FP8BS_MLA_V
#undef FP8BS_MLA_V4
  return hipGetLastError();
}

}  // namespace fp8bs
