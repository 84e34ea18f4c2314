// moe_dispatch.hip -- the MoE steps around the grouped expert GEMM, after the
// expert loop of the "DeepSeek-V3 Administrator & Developer Guide" (6.4 and
// the annotated forward pass in 8.4): per-expert hit counts of the routed
// expert ids, each expert's (token, slot) pairs in token order, the expert
// run on those tokens' rows, and each output scaled by the routing weight of
// its (token, slot) and summed into the token's output.
//
//   route    stable counting sort of ids [T, topk] by expert -> offsets
//            [E+1], row_token [R] and row_of [T, topk] (one launch each for
//            chunk histograms, their scan, and the placement; the only
//            atomics are LDS adds and ORs, whose order does not change the
//            result, so it is deterministic)
//   combine  y[t, :] = sum_k w[t, k] * out[row_of[t, k], :] in fp32, slot
//            order, one rounding at the store
// (The expert inputs -- act_quant of each token written to its routed rows --
// are the scatter variant of act_quant in quant.hip.)
#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace fp8bs {

// ----------------------------------------------------------------------------
// route
// ----------------------------------------------------------------------------
// The P = T * topk (token, slot) pairs are cut into chunks of kRouteChunk in
// (token, slot) order.  Pass 1 counts, per chunk, the pairs of every expert;
// pass 2 turns the [chunks][E] counts into the first row of each (chunk,
// expert) -- expert e's rows start at offsets[e], and within them chunk c's
// pairs come after those of chunks < c; pass 3 gives each pair of a chunk, in
// order, the next row of its expert.  Passes 2 and 3 run as one launch when
// the table is small and E <= kFusedMaxE, else as three (below).
constexpr int kRouteChunk = 512;
constexpr int kRouteThreads = 256;
constexpr int kScanThreads = 1024;

__device__ __forceinline__ int load_chunk_ids(const int32_t* __restrict__ idx, int64_t P,
                                              int32_t* ids) {
  const int64_t p0 = (int64_t)blockIdx.x * kRouteChunk;
  const int n = (int)min<int64_t>(kRouteChunk, P - p0);
  for (int i = threadIdx.x; i < kRouteChunk; i += kRouteThreads) ids[i] = i < n ? idx[p0 + i] : -1;
  __syncthreads();
  return n;
}

// Pass 1.  The chunk's ids go into an LDS histogram with atomic adds (a count
// does not depend on the order of the adds, so the table is deterministic),
// kCountLdsMaxE experts at a time: one pass over the chunk per window of
// experts.
constexpr int kCountLdsMaxE = 8192;

__global__ __launch_bounds__(kRouteThreads) void moe_route_count_kernel(
    const int32_t* __restrict__ idx, int64_t P, int E, int32_t* __restrict__ hist) {
  __shared__ int32_t h[kCountLdsMaxE];
  const int64_t p0 = (int64_t)blockIdx.x * kRouteChunk;
  int id[kRouteChunk / kRouteThreads];
#pragma unroll
  for (int k = 0; k < kRouteChunk / kRouteThreads; ++k) {
    const int64_t p = p0 + threadIdx.x + k * kRouteThreads;
    id[k] = p < P ? idx[p] : -1;
  }
  for (int e0 = 0; e0 < E; e0 += kCountLdsMaxE) {
    const int ew = min(kCountLdsMaxE, E - e0);
    for (int e = threadIdx.x; e < ew; e += kRouteThreads) h[e] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kRouteChunk / kRouteThreads; ++k)
      if (id[k] >= e0 && id[k] < e0 + ew) atomicAdd(&h[id[k] - e0], 1);
    __syncthreads();
    for (int e = threadIdx.x; e < ew; e += kRouteThreads) hist[(int64_t)blockIdx.x * E + e0 + e] = h[e];
    __syncthreads();                                   // the next window reuses h
  }
}

// Pair-parallel placement of one chunk, for E <= kFusedMaxE.  base[e] (LDS)
// holds expert e's next free row; wmask is LDS scratch [4][E] of 64-bit lane
// masks, zero on entry and on return.  The chunk goes in rounds of 256 pairs,
// wave w taking pairs 64w .. 64w+63 of the round.  Each valid pair sets its
// lane's bit in wmask[w][id] (an atomic OR: the result does not depend on the
// order of the ORs, so the placement is deterministic).  A pair's row is then
// base[id] + (pairs of the same expert in earlier waves of the round: the
// popcounts of their masks) + (earlier lanes of its own wave with the same
// expert: the popcount of its mask below its lane).
constexpr int kFusedMaxE = 2048;

__device__ void place_chunk(const int32_t* ids, int n, int64_t p0, int topk, int E, int32_t* base,
                            unsigned long long* wmask, int32_t* __restrict__ row_token,
                            int32_t* __restrict__ row_of) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long below = (1ull << lane) - 1;
  for (int r0 = 0; r0 < kRouteChunk; r0 += kRouteThreads) {
    const int i = r0 + threadIdx.x;
    const int id = i < n ? ids[i] : -1;
    const bool valid = id >= 0 && id < E;
    if (valid) atomicOr(&wmask[wave * E + id], 1ull << lane);
    __syncthreads();
    if (valid) {
      int pos = base[id] + __popcll(wmask[wave * E + id] & below);
      for (int w = 0; w < wave; ++w) pos += __popcll(wmask[w * E + id]);
      const int64_t p = p0 + i;
      row_token[pos] = (int32_t)(p / topk);
      row_of[p] = pos;
    } else if (i < n) {
      row_of[p0 + i] = -1;
    }
    __syncthreads();                                  // every lane has read base and wmask
    for (int e = threadIdx.x; e < E; e += kRouteThreads) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        c += __popcll(wmask[w * E + e]);
        wmask[w * E + e] = 0;
      }
      base[e] += c;
    }
    __syncthreads();
  }
}

// Passes 2 and 3 in one launch (when E <= kFusedMaxE and C * E is small):
// every placement workgroup reads the whole [C][E] count table (from L2),
// forms each expert's total and the count of its own earlier chunks, scans the
// totals over the experts itself, and places its chunk.  Workgroup 0 also
// writes offsets.  The count table is only read, so the workgroups need no
// ordering among themselves.
constexpr int64_t kFusedMaxTable = 1 << 16;

__global__ __launch_bounds__(kRouteThreads) void moe_route_scan_place_kernel(
    const int32_t* __restrict__ idx, int64_t P, int topk, int E, int C,
    const int32_t* __restrict__ hist, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  __shared__ __attribute__((aligned(16))) int32_t ids[kRouteChunk];
  __shared__ int32_t base[kFusedMaxE];
  __shared__ unsigned long long wmask[4 * kFusedMaxE];
  __shared__ int32_t part[kRouteThreads];
  __shared__ int32_t carry;
  const int c = blockIdx.x;
  const int n = load_chunk_ids(idx, P, ids);
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  constexpr int kBatch = 32;
  for (int e0 = 0; e0 < E; e0 += kRouteThreads) {
    const int e = e0 + threadIdx.x;
    int tot = 0, pre = 0;                               // all chunks; chunks before c
    if (e < E)
      for (int c0 = 0; c0 < C; c0 += kBatch) {
        int v[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < C ? hist[(int64_t)(c0 + j) * E + e] : 0;
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
          tot += v[j];
          pre += c0 + j < c ? v[j] : 0;
        }
      }
    part[threadIdx.x] = tot;
    __syncthreads();
    for (int d = 1; d < kRouteThreads; d <<= 1) {
      const int v = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int first = carry + part[threadIdx.x] - tot;
    if (e < E) {
      base[e] = first + pre;
      if (c == 0) offsets[e] = first;
#pragma unroll
      for (int w = 0; w < 4; ++w) wmask[w * E + e] = 0;
    }
    __syncthreads();                                   // every thread has read carry
    if (threadIdx.x == kRouteThreads - 1) carry += part[threadIdx.x];
    __syncthreads();
  }
  if (c == 0 && threadIdx.x == 0) offsets[E] = carry;
  place_chunk(ids, n, (int64_t)c * kRouteChunk, topk, E, base, wmask, row_token, row_of);
}

// Passes 2 and 3 for larger tables or E > kFusedMaxE: pass 2 split over the
// experts, pass 3 independent of E.
//   colscan: thread e (one per expert, 256 per workgroup) turns column e of
//            the [C][E] counts into its exclusive prefix over the chunks and
//            writes the column's total to offsets[e];
//   totscan: one workgroup turns offsets[0 .. E) into the exclusive prefix of
//            the totals and writes offsets[E];
//   place:   one thread per pair; its row is offsets[id] + its chunk's first
//            row of id (the column prefix) + the pairs of id earlier in its
//            chunk, counted by scanning the chunk's ids in LDS (every lane
//            reads the same word, a broadcast).
// Measured (4096 tokens x top-8, uniform ids, us): E = 2048 35.4 -> 24.3 and
// E = 8192 998 -> 32.5 against a one-workgroup scan and a thread-per-expert
// placement; 65536 tokens over 256 experts 119.5 -> 86.5.
__global__ __launch_bounds__(kRouteThreads) void moe_route_colscan_kernel(int32_t* __restrict__ hist,
                                                                          int C, int E,
                                                                          int32_t* __restrict__ offsets) {
  const int e = blockIdx.x * kRouteThreads + threadIdx.x;
  if (e >= E) return;
  constexpr int kBatch = 16;                           // column loads in flight per thread
  int run = 0;
  for (int c0 = 0; c0 < C; c0 += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) v[j] = c0 + j < C ? hist[(int64_t)(c0 + j) * E + e] : 0;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int x = v[j];
      v[j] = run;
      run += x;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (c0 + j < C) hist[(int64_t)(c0 + j) * E + e] = v[j];
  }
  offsets[e] = run;
}

__global__ __launch_bounds__(kScanThreads) void moe_route_totscan_kernel(int E, int32_t* __restrict__ offsets) {
  // thread t owns the totals [L t, L t + L) of each pass of kScanThreads * L
  constexpr int L = 8;
  __shared__ int32_t part[kScanThreads];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += kScanThreads * L) {
    const int eb = e0 + L * threadIdx.x;
    int v[L], sum = 0;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      v[j] = eb + j < E ? offsets[eb + j] : 0;
      sum += v[j];
    }
    part[threadIdx.x] = sum;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
      const int x = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
      __syncthreads();
      part[threadIdx.x] += x;
      __syncthreads();
    }
    int run = carry + part[threadIdx.x] - sum;
#pragma unroll
    for (int j = 0; j < L; ++j) {
      if (eb + j < E) offsets[eb + j] = run;
      run += v[j];
    }
    __syncthreads();                                   // every thread has read carry
    if (threadIdx.x == kScanThreads - 1) carry += part[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[E] = carry;
}

__global__ __launch_bounds__(kRouteChunk) void moe_route_place_many_kernel(
    const int32_t* __restrict__ idx, int64_t P, int topk, int E, const int32_t* __restrict__ first,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  // one thread per pair of the chunk
  __shared__ __attribute__((aligned(16))) int32_t ids[kRouteChunk];
  const int i = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * kRouteChunk + i;
  const int id = p < P ? idx[p] : -1;
  ids[i] = id;
  __syncthreads();
  // pairs before i with the same id
  const int4* ids4 = (const int4*)ids;
  int rank = 0;
#pragma unroll 8
  for (int q = 0; q < kRouteChunk / 4; ++q) {
    const int4 v = ids4[q];
    rank += (4 * q + 0 < i && v.x == id) + (4 * q + 1 < i && v.y == id) + (4 * q + 2 < i && v.z == id) +
            (4 * q + 3 < i && v.w == id);
  }
  if (p >= P) return;
  if (id >= 0 && id < E) {
    const int pos = offsets[id] + first[(int64_t)blockIdx.x * E + id] + rank;
    row_token[pos] = (int32_t)(p / topk);
    row_of[p] = pos;
  } else {
    row_of[p] = -1;
  }
}

int64_t moe_route_workspace_bytes(int64_t T, int64_t topk, int64_t E) {
  const int64_t chunks = (T * topk + kRouteChunk - 1) / kRouteChunk;
  return chunks * E * (int64_t)sizeof(int32_t);
}

hipError_t launch_moe_route(const int32_t* indices, int64_t T, int64_t topk, int64_t E,
                            int32_t* offsets, int32_t* row_token, int32_t* row_of, void* workspace,
                            hipStream_t stream) {
  const int64_t P = T * topk;
  const int C = (int)((P + kRouteChunk - 1) / kRouteChunk);
  int32_t* hist = (int32_t*)workspace;
  if (C > 0) {
    moe_route_count_kernel<<<dim3(C), dim3(kRouteThreads), 0, stream>>>(indices, P, (int)E, hist);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (E <= kFusedMaxE && (int64_t)C * E <= kFusedMaxTable) {
      moe_route_scan_place_kernel<<<dim3(C), dim3(kRouteThreads), 0, stream>>>(
          indices, P, (int)topk, (int)E, C, hist, offsets, row_token, row_of);
      return hipGetLastError();
    }
  }
  // (with no pairs, C = 0: the column scan writes zero totals and the
  // offsets come out all zero)
  moe_route_colscan_kernel<<<dim3((unsigned)((E + kRouteThreads - 1) / kRouteThreads)), dim3(kRouteThreads), 0,
                             stream>>>(hist, C, (int)E, offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  moe_route_totscan_kernel<<<dim3(1), dim3(kScanThreads), 0, stream>>>((int)E, offsets);
  err = hipGetLastError();
  if (err != hipSuccess || C == 0) return err;
  moe_route_place_many_kernel<<<dim3(C), dim3(kRouteChunk), 0, stream>>>(indices, P, (int)topk, (int)E, hist,
                                                                         offsets, row_token, row_of);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// route without a caller workspace
// ----------------------------------------------------------------------------
// For callers that cannot allocate (code under stream capture, serving loops,
// harnesses that forbid allocation): the route's [chunks][E] count table
// lives in a file-scope device array of kRouteScratchBytes instead of a
// caller workspace.  Every GPU the library runs on holds its own copy until
// the process ends.  In host code `scratch` names a host-side stand-in, so
// the array's device address is looked up once per device (with that device
// current) and only that address is ever passed to a kernel.  The count
// kernel overwrites every table entry the later kernels read, so nothing is
// cleared between calls; two calls that overlap on one GPU share the table
// and race.
static __device__ __align__(256) int32_t scratch[kRouteScratchBytes / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}
}  // namespace

hipError_t launch_moe_route_noalloc(const int32_t* indices, int64_t T, int64_t topk, int64_t E,
                                    int32_t* offsets, int32_t* row_token, int32_t* row_of,
                                    hipStream_t stream) {
  if (moe_route_workspace_bytes(T, topk, E) > kRouteScratchBytes) return hipErrorInvalidValue;
  void* table = nullptr;
  const hipError_t err = scratch_address(&table);
  if (err != hipSuccess) return err;
  return launch_moe_route(indices, T, topk, E, offsets, row_token, row_of, table, stream);
}

// ----------------------------------------------------------------------------
// combine
// ----------------------------------------------------------------------------
// Vector path (N % 8 == 0, 16-byte aligned buffers, topk <= KMAX, R*N*2 <
// 2^32): a thread owns 8 consecutive columns of one token and issues all its
// row loads (16 bytes of bf16 each) before using any.  Slots k >= topk and
// pairs outside [0, R) load through an out-of-range buffer offset, which
// returns zeros without touching memory, and carry weight 0, so every load is
// unconditional; the sum runs in fp32 in slot order.
constexpr int kCombineThreads = 256;
typedef int v4i_t __attribute__((ext_vector_type(4)));

template <int KMAX, bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void moe_combine_vec_kernel(
    const void* __restrict__ out, const float* __restrict__ w, const int32_t* __restrict__ row_of,
    void* __restrict__ y, int64_t T, int topk, int64_t R, int64_t nv) {
  const int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (i >= T * nv) return;
  const int64_t t = i / nv, v = i - t * nv;
  // raw buffer over out (R rows of nv 16-byte vectors), 32-bit data format
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(out), (short)0, (int)(uint32_t)(R * nv * 16), 0x00020000);
  int r[KMAX];
  float wk[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int kk = k < topk ? k : topk - 1;              // in-range index for the load
    r[k] = row_of[t * topk + kk];
    wk[k] = w[t * topk + kk];
  }
  v4i_t o[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const bool ok = k < topk && r[k] >= 0 && r[k] < R;
    const uint32_t off = ok ? (uint32_t)(((int64_t)r[k] * nv + v) * 16) : 0xF0000000u;
    o[k] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, kNonTemporal);
    if (!ok) wk[k] = 0.0f;
  }
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t h = (uint32_t)o[k][j];
      acc[2 * j] = __builtin_fmaf(wk[k], bf16_lo(h), acc[2 * j]);
      acc[2 * j + 1] = __builtin_fmaf(wk[k], bf16_hi(h), acc[2 * j + 1]);
    }
  }
  if (OUT_F32) {
    uint4* yp = (uint4*)y + 2 * i;
    store_nt(yp, make_uint4(f32_bits(acc[0]), f32_bits(acc[1]), f32_bits(acc[2]), f32_bits(acc[3])));
    store_nt(yp + 1, make_uint4(f32_bits(acc[4]), f32_bits(acc[5]), f32_bits(acc[6]), f32_bits(acc[7])));
  } else {
    store_nt((uint4*)y + i, make_uint4(pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]),
                                       pack2_bf16(acc[4], acc[5]), pack2_bf16(acc[6], acc[7])));
  }
}

// Element path (any N, any topk): one thread per output element.
template <bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void moe_combine_elem_kernel(
    const uint16_t* __restrict__ out, const float* __restrict__ w,
    const int32_t* __restrict__ row_of, void* __restrict__ y, int64_t T, int topk, int64_t R,
    int64_t N) {
  const int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (i >= T * N) return;
  const int64_t t = i / N, n = i - t * N;
  float acc = 0.0f;
  for (int k = 0; k < topk; ++k) {
    const int64_t r = row_of[t * topk + k];
    if (r < 0 || r >= R) continue;
    acc = __builtin_fmaf(w[t * topk + k], bits_f32((uint32_t)out[r * N + n] << 16), acc);
  }
  if (OUT_F32)
    ((float*)y)[i] = acc;
  else
    ((uint16_t*)y)[i] = (uint16_t)pack2_bf16(acc, 0.0f);
}

hipError_t launch_moe_combine(const void* out, const float* w, const int32_t* row_of, void* y,
                              int64_t T, int64_t topk, int64_t R, int64_t N, bool out_f32,
                              hipStream_t stream) {
  if (T == 0 || N == 0) return hipSuccess;
  const bool vec = N % 8 == 0 && topk <= 16 && ((uintptr_t)out & 15) == 0 &&
                   ((uintptr_t)y & 15) == 0 && R * N * 2 < ((int64_t)1 << 32) - ((int64_t)1 << 28);
  if (vec) {
    const int64_t nv = N / 8, total = T * nv;
    const dim3 grid((unsigned)((total + kCombineThreads - 1) / kCombineThreads)), block(kCombineThreads);
    if (topk <= 8) {
      if (out_f32)
        moe_combine_vec_kernel<8, true><<<grid, block, 0, stream>>>(out, w, row_of, y, T, (int)topk, R, nv);
      else
        moe_combine_vec_kernel<8, false><<<grid, block, 0, stream>>>(out, w, row_of, y, T, (int)topk, R, nv);
    } else {
      if (out_f32)
        moe_combine_vec_kernel<16, true><<<grid, block, 0, stream>>>(out, w, row_of, y, T, (int)topk, R, nv);
      else
        moe_combine_vec_kernel<16, false><<<grid, block, 0, stream>>>(out, w, row_of, y, T, (int)topk, R, nv);
    }
  } else {
    const int64_t total = T * N;
    const dim3 grid((unsigned)((total + kCombineThreads - 1) / kCombineThreads));
    if (out_f32)
      moe_combine_elem_kernel<true><<<grid, dim3(kCombineThreads), 0, stream>>>(
          (const uint16_t*)out, w, row_of, y, T, (int)topk, R, N);
    else
      moe_combine_elem_kernel<false><<<grid, dim3(kCombineThreads), 0, stream>>>(
          (const uint16_t*)out, w, row_of, y, T, (int)topk, R, N);
  }
  return hipGetLastError();
}

}  // namespace fp8bs
