// k_topk.hip — the two full-history passes of the exact top-K (gfx950).
//
// The DSA indexer keeps the 2,048 best history positions and the selection must
// be exact (page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
// Offloading", sections "Separate historical capacity from the current working
// set" and "Decision one: should the CPU store history and run the indexer?").
// Ranking is by the IEEE totalOrder key of the fp32 score, ties to the lower
// position.  The cut is found by radix selection on the 32-bit key:
//
//   pass 1 (k_topk_hist):   histogram of the top 12 key bits per unit, built in
//                           LDS per workgroup and merged with global atomics;
//   pass 2 (k_topk_filter): every workgroup locates the bin holding the K-th
//                           key, then compacts its chunk: positions in higher
//                           bins go to `above` (always selected, < K of them),
//                           positions in the cut bin go to `cand` with their key.
//
// The remaining 20 key bits and the position tie-break are resolved on the
// (small) candidate list by k_select.  Both passes are HBM-bound streaming reads
// of 4 B per position; grid = (chunks of 8,192 positions) x (units).
#include "hc_internal.h"

namespace hc {

constexpr int kScanThreads = 256;
constexpr int kPerThread = kScanChunk / kScanThreads;  // 32 scores per thread

// Loads this thread's scores of the chunk: element j of the thread is position
// base + idx(j); positions >= n are reported invalid.
template <bool VEC>
__device__ __forceinline__ void load_chunk(const float* src, int n, float (&x)[kPerThread],
                                           int (&pos)[kPerThread]) {
  const int tid = threadIdx.x;
  if (VEC) {
    // float4 j of this thread covers chunk positions 4 * (tid + 256 j) + [0, 4).
    const float4* s4 = reinterpret_cast<const float4*>(src);
#pragma unroll
    for (int j = 0; j < kPerThread / 4; ++j) {
      const int q = tid + kScanThreads * j;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (4 * q < n) v = s4[q];
      x[4 * j + 0] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
#pragma unroll
      for (int c = 0; c < 4; ++c) pos[4 * j + c] = 4 * q + c;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
      const int q = tid + kScanThreads * j;
      x[j] = q < n ? src[q] : 0.f;
      pos[j] = q;
    }
  }
}

template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void k_topk_hist(DevState d, StepArgs a,
                                                            const float* __restrict__ scores,
                                                            uint64_t stride) {
  __shared__ uint32_t h[kBins1];
  const int u = blockIdx.y;
  const int64_t H = a.hist_len[u / d.G];
  const int64_t base = (int64_t)blockIdx.x * kScanChunk;
  if (base >= H) return;
  const int n = (int)(H - base < kScanChunk ? H - base : kScanChunk);

  for (int b = threadIdx.x; b < kBins1; b += kScanThreads) h[b] = 0;
  __syncthreads();

  float x[kPerThread];
  int pos[kPerThread];
  load_chunk<VEC>(scores + (uint64_t)u * stride + base, n, x, pos);
#pragma unroll
  for (int j = 0; j < kPerThread; ++j)
    if (pos[j] < n) atomicAdd(&h[order_key(x[j]) >> (32 - kBin1Bits)], 1u);
  __syncthreads();

  uint32_t* gh = d.hist + (size_t)u * kBins1;
  for (int b = threadIdx.x; b < kBins1; b += kScanThreads)
    if (h[b]) atomicAdd(&gh[b], h[b]);
}

// Inclusive prefix sum over the 256 threads of the block (thread order).
__device__ __forceinline__ int block_incl_scan256(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += wtot[i];
  __syncthreads();
  return x + off;
}

template <bool VEC>
__global__ __launch_bounds__(kScanThreads) void k_topk_filter(DevState d, StepArgs a,
                                                              const float* __restrict__ scores,
                                                              uint64_t stride) {
  __shared__ int wtot[kScanThreads / 64];
  __shared__ uint32_t cut_bin;
  __shared__ int off_above, off_cand;
  const int u = blockIdx.y;
  const int64_t H = a.hist_len[u / d.G];
  const int64_t base = (int64_t)blockIdx.x * kScanChunk;
  if (base >= H) return;
  const int n = (int)(H - base < kScanChunk ? H - base : kScanChunk);
  const int tid = threadIdx.x;

  // 1. The cut bin: the highest bin b with (count of keys in bins >= b) >= K.
  //    Thread i owns bins [kBins1 - 16 (i + 1), kBins1 - 16 i), scanned top-down.
  constexpr int kPer = kBins1 / kScanThreads;
  const uint32_t* gh = d.hist + (size_t)u * kBins1;
  const int top = kBins1 - 1 - kPer * tid;
  uint32_t hb[kPer];
  if (tid == 0) cut_bin = 0;  // ordered before the search by the scan's barriers
  int sum = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    hb[i] = gh[top - i];
    sum += (int)hb[i];
  }
  const int incl = block_incl_scan256(sum, wtot);
  const int excl = incl - sum;
  if (excl < d.K && d.K <= incl) {
    int cum = excl;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (cum + (int)hb[i] >= d.K) {
        cut_bin = (uint32_t)(top - i);
        break;
      }
      cum += (int)hb[i];
    }
  }
  __syncthreads();
  const uint32_t b1 = cut_bin;
  if (blockIdx.x == 0 && tid == 0) d.cnt[u * kCnt + kCntBin1] = (int32_t)b1;

  // 2. Classify this thread's scores and compact them.
  float x[kPerThread];
  int pos[kPerThread];
  load_chunk<VEC>(scores + (uint64_t)u * stride + base, n, x, pos);
  uint32_t key[kPerThread];
  int na = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    key[j] = order_key(x[j]);
    const uint32_t b = key[j] >> (32 - kBin1Bits);
    const bool ok = pos[j] < n;
    na += ok && b > b1;
    nc += ok && b == b1;
  }
  // both counts fit 16 bits (at most 8,192 per block): scan them packed
  const int packed = (na << 16) | nc;
  const int pincl = block_incl_scan256(packed, wtot);
  if (tid == kScanThreads - 1) {
    off_above = atomicAdd(&d.cnt[u * kCnt + kCntAbove], pincl >> 16);
    off_cand = atomicAdd(&d.cnt[u * kCnt + kCntCand], pincl & 0xFFFF);
  }
  __syncthreads();
  int ia = off_above + ((pincl - packed) >> 16);
  int ic = off_cand + ((pincl - packed) & 0xFFFF);
  int32_t* above = d.above + (size_t)u * d.K;
  uint2* cand = d.cand + (size_t)u * d.hcap;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (pos[j] >= n) continue;
    const uint32_t b = key[j] >> (32 - kBin1Bits);
    const int32_t p = (int32_t)(base + pos[j]);
    // the cut bin bounds both lists (< K above, <= H candidates); the guards
    // only keep a corrupted histogram from writing out of bounds
    if (b > b1) {
      if (ia < d.K) above[ia] = p;
      ++ia;
    } else if (b == b1) {
      if (ic < d.hcap) cand[ic] = make_uint2(key[j], (uint32_t)p);
      ++ic;
    }
  }
}

hipError_t launch_topk_hist(const DevState& d, const StepArgs& a, const float* scores,
                            uint64_t stride, int n_chunks, bool vec4, hipStream_t st) {
  dim3 grid(n_chunks, d.S * d.G);
  if (vec4)
    hipLaunchKernelGGL(k_topk_hist<true>, grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  else
    hipLaunchKernelGGL(k_topk_hist<false>, grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  return hipGetLastError();
}

hipError_t launch_topk_filter(const DevState& d, const StepArgs& a, const float* scores,
                              uint64_t stride, int n_chunks, bool vec4, hipStream_t st) {
  dim3 grid(n_chunks, d.S * d.G);
  if (vec4)
    hipLaunchKernelGGL(k_topk_filter<true>, grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  else
    hipLaunchKernelGGL(k_topk_filter<false>, grid, dim3(kScanThreads), 0, st, d, a, scores,
                       stride);
  return hipGetLastError();
}

}  // namespace hc
