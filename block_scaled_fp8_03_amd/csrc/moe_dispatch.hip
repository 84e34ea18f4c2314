// moe_dispatch.hip -- the MoE steps around the grouped expert GEMM, after the
// expert loop of the "DeepSeek-V3 Administrator & Developer Guide" (6.4 and
// the annotated forward pass in 8.4): per-expert hit counts of the routed
// expert ids, each expert's (token, slot) pairs in token order, the expert
// run on those tokens' rows, and each output scaled by the routing weight of
// its (token, slot) and summed into the token's output.
//
//   route    stable counting sort of ids [T, topk] by expert -> offsets
//            [E+1], row_token [R] and row_of [T, topk] (one launch each for
//            chunk histograms, their scan, and the placement; no atomics, so
//            the result is deterministic)
//   combine  y[t, :] = sum_k w[t, k] * out[row_of[t, k], :] in fp32, slot
//            order, one rounding at the store
// (The expert inputs -- act_quant of each token written to its routed rows --
// are the scatter variant of act_quant in quant.hip.)
#include <algorithm>

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
// pairs come after those of chunks < c; pass 3 walks each chunk in order and
// gives each pair the next row of its expert.  In passes 1 and 3 a thread owns
// experts e = tid, tid + 256, ... and scans the chunk's ids from LDS (every
// lane reads the same word, a broadcast).
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

__global__ __launch_bounds__(kRouteThreads) void moe_route_count_kernel(
    const int32_t* __restrict__ idx, int64_t P, int E, int32_t* __restrict__ hist) {
  __shared__ __attribute__((aligned(16))) int32_t ids[kRouteChunk];
  load_chunk_ids(idx, P, ids);
  const int4* ids4 = (const int4*)ids;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int cnt = 0;
    for (int i = 0; i < kRouteChunk / 4; ++i) {        // padding ids are -1: never an expert
      const int4 v = ids4[i];
      cnt += (v.x == e) + (v.y == e) + (v.z == e) + (v.w == e);
    }
    hist[(int64_t)blockIdx.x * E + e] = cnt;
  }
}

// One workgroup.  hist [C][E] counts -> first rows; offsets [E+1].
__global__ __launch_bounds__(kScanThreads) void moe_route_scan_kernel(int32_t* __restrict__ hist,
                                                                      int C, int E,
                                                                      int32_t* __restrict__ offsets) {
  __shared__ int32_t part[kScanThreads];
  __shared__ int32_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int e0 = 0; e0 < E; e0 += kScanThreads) {
    const int e = e0 + threadIdx.x;
    // exclusive prefix of expert e's column over the chunks; tot = its hits
    int tot = 0;
    if (e < E)
      for (int c = 0; c < C; ++c) {
        const int v = hist[(int64_t)c * E + e];
        hist[(int64_t)c * E + e] = tot;
        tot += v;
      }
    // exclusive prefix of the totals over the experts of this round
    part[threadIdx.x] = tot;
    __syncthreads();
    for (int d = 1; d < kScanThreads; d <<= 1) {
      const int v = threadIdx.x >= d ? part[threadIdx.x - d] : 0;
      __syncthreads();
      part[threadIdx.x] += v;
      __syncthreads();
    }
    const int first = carry + part[threadIdx.x] - tot;
    if (e < E) {
      offsets[e] = first;
      for (int c = 0; c < C; ++c) hist[(int64_t)c * E + e] += first;
    }
    __syncthreads();                                   // every thread has read carry
    if (threadIdx.x == kScanThreads - 1) carry += part[threadIdx.x];
    __syncthreads();
  }
  if (threadIdx.x == 0) offsets[E] = carry;
}

__global__ __launch_bounds__(kRouteThreads) void moe_route_place_kernel(
    const int32_t* __restrict__ idx, int64_t P, int topk, int E, const int32_t* __restrict__ first,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  __shared__ __attribute__((aligned(16))) int32_t ids[kRouteChunk];
  const int n = load_chunk_ids(idx, P, ids);
  const int64_t p0 = (int64_t)blockIdx.x * kRouteChunk;
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int pos = first[(int64_t)blockIdx.x * E + e];
    for (int i = 0; i < n; ++i)
      if (ids[i] == e) {
        const int64_t p = p0 + i;
        row_token[pos] = (int32_t)(p / topk);
        row_of[p] = pos;
        ++pos;
      }
  }
  for (int i = threadIdx.x; i < n; i += kRouteThreads)
    if (ids[i] < 0 || ids[i] >= E) row_of[p0 + i] = -1;
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
  }
  moe_route_scan_kernel<<<dim3(1), dim3(kScanThreads), 0, stream>>>(hist, C, (int)E, offsets);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || C == 0) return err;
  moe_route_place_kernel<<<dim3(C), dim3(kRouteThreads), 0, stream>>>(indices, P, (int)topk, (int)E,
                                                                      hist, row_token, row_of);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------
// combine
// ----------------------------------------------------------------------------
// Vector path (N % 8 == 0, 16-byte aligned buffers): a thread owns 8
// consecutive columns of one token, issues the topk row loads (16 bytes of
// bf16 each) before using any, and sums w * out in fp32 in slot order.
constexpr int kCombineThreads = 256;
constexpr int kCombineMaxTopk = 16;

template <bool OUT_F32>
__global__ __launch_bounds__(kCombineThreads) void moe_combine_vec_kernel(
    const uint4* __restrict__ out, const float* __restrict__ w, const int32_t* __restrict__ row_of,
    void* __restrict__ y, int64_t T, int topk, int64_t R, int64_t nv) {
  const int64_t i = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  if (i >= T * nv) return;
  const int64_t t = i / nv, v = i - t * nv;
  uint4 o[kCombineMaxTopk];
  float wk[kCombineMaxTopk];
#pragma unroll
  for (int k = 0; k < kCombineMaxTopk; ++k) {
    wk[k] = 0.0f;
    o[k] = make_uint4(0, 0, 0, 0);
    if (k < topk) {
      const int64_t r = row_of[t * topk + k];
      if (r >= 0 && r < R) {
        wk[k] = w[t * topk + k];
        o[k] = out[r * nv + v];
      }
    }
  }
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int k = 0; k < kCombineMaxTopk; ++k) {
    if (k >= topk) break;
    const uint32_t h[4] = {o[k].x, o[k].y, o[k].z, o[k].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = __builtin_fmaf(wk[k], bf16_lo(h[j]), acc[2 * j]);
      acc[2 * j + 1] = __builtin_fmaf(wk[k], bf16_hi(h[j]), acc[2 * j + 1]);
    }
  }
  if (OUT_F32) {
    float4* yp = (float4*)y + 2 * i;
    yp[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    yp[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else {
    ((uint4*)y)[i] = make_uint4(pack2_bf16(acc[0], acc[1]), pack2_bf16(acc[2], acc[3]),
                                pack2_bf16(acc[4], acc[5]), pack2_bf16(acc[6], acc[7]));
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
  const bool vec = N % 8 == 0 && topk <= kCombineMaxTopk && ((uintptr_t)out & 15) == 0 &&
                   ((uintptr_t)y & 15) == 0;
  if (vec) {
    const int64_t nv = N / 8, total = T * nv;
    const dim3 grid((unsigned)((total + kCombineThreads - 1) / kCombineThreads));
    if (out_f32)
      moe_combine_vec_kernel<true><<<grid, dim3(kCombineThreads), 0, stream>>>(
          (const uint4*)out, w, row_of, y, T, (int)topk, R, nv);
    else
      moe_combine_vec_kernel<false><<<grid, dim3(kCombineThreads), 0, stream>>>(
          (const uint4*)out, w, row_of, y, T, (int)topk, R, nv);
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
