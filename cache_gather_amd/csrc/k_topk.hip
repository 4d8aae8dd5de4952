// k_topk.hip — the one full-history pass of the exact top-K (gfx950).
//
// The DSA indexer keeps the 2,048 best history positions and the selection must
// be exact (page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
// Offloading", sections "Separate historical capacity from the current working
// set" and "Decision one: should the CPU store history and run the indexer?").
// Ranking is by the IEEE totalOrder key of the fp32 score, ties to the lower
// position.  The cut is found by radix selection on the 32-bit key; its first
// digit is the top 12 bits (4,096 bins).
//
// k_topk_scan reads every score once and classifies it against a cut window
// [b_lo, b_hi] of 12-bit bins predicted from the previous step's cut bin (one
// bin either side; the whole key range on a unit's first step): keys above the
// window go to `above` (only counted once `above` holds K), keys inside it go
// to `cand` with their key.  k_select then knows how many keys lie above the
// window and can count the window's bins from the candidates, which decides
// whether the K-th key fell inside the window.  If it did, the lists are exact
// (everything above the cut bin is selected; only the cut bin's candidates
// need the remaining 20 bits); if not, k_select rescans the scores itself.
// Scores change little between decode steps (the history is the same apart
// from one appended position), so the window almost always holds and a step
// reads the history once.
//
// A context's first step has no previous cut bin.  Rather than classify every
// key as a candidate (which leaves one k_select workgroup to rank the whole
// history: 1.4 ms at a million positions), k_cold_hist counts the keys of
// every 12-bit bin over many workgroups and k_cold_cut places the window on
// the bin holding the K-th key, so the first step's lists are as small as any
// other step's.
//
// Grid = (chunks of 2,048 or 4,096 positions) x (selection units: one per query row of
// each session and group), 256 threads; HBM-bound streaming read of 4 B per
// position.
#include "hc_internal.h"

namespace hc {

constexpr int kScanThreads = 256;

// Loads this thread's scores of the chunk: element j of the thread is position
// base + pos[j]; positions >= n are invalid.
template <bool VEC, int kPerThread>
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

// Inclusive prefix sum over the 256 threads of the block (thread order).
__device__ __forceinline__ int block_incl_scan256(int v, int* wtot) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  int off = 0;
  for (int i = 0; i < w; ++i) off += wtot[i];
  __syncthreads();
  return x + off;
}

// CHUNK scores per workgroup (2,048 or 4,096), CHUNK / 256 per thread.
template <bool VEC, int CHUNK>
__global__ __launch_bounds__(kScanThreads) void k_topk_scan(DevState d, StepArgs a,
                                                            const float* __restrict__ scores,
                                                            uint64_t stride) {
  __shared__ int wtot[kScanThreads / 64];
  __shared__ int off_above, off_cand;
  const int u = blockIdx.y;  // selection unit (s, g, q)
  const int64_t H = a.hist_len[u / (d.G * d.Q)];
  constexpr int kPerThread = CHUNK / kScanThreads;
  const int64_t base = (int64_t)blockIdx.x * CHUNK;
  if (base >= H) return;
  const int n = (int)(H - base < CHUNK ? H - base : CHUNK);
  const int tid = threadIdx.x;

  // predicted cut window from the previous step's cut bin (-1: none yet)
  uint32_t b_lo, b_hi;
  cut_window(d.cnt[u * kCntStride + kCntBin1], b_lo, b_hi);

  float x[kPerThread];
  int pos[kPerThread];
  load_chunk<VEC, kPerThread>(scores + (uint64_t)u * stride + base, n, x, pos);
  uint32_t key[kPerThread];
  int na = 0, nc = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    key[j] = order_key(x[j]);
    const uint32_t b = key[j] >> (32 - kBin1Bits);
    const bool ok = pos[j] < n;
    na += ok && b > b_hi;
    nc += ok && b >= b_lo && b <= b_hi;
  }
  // both counts fit 16 bits (at most 4,096 per block): scan them packed
  const int packed = (na << 16) | nc;
  const int pincl = block_incl_scan256(packed, wtot);
  if (tid == kScanThreads - 1) {
    // one atomic reserves both lists: above count in the low word, candidate
    // count in the high word (neither total exceeds 2^31, so no carry)
    static_assert(kCntCand == kCntAbove + 1 && kCntAbove % 2 == 0, "counter pair");
    const uint64_t add = ((uint64_t)(pincl & 0xFFFF) << 32) | (uint32_t)(pincl >> 16);
    const uint64_t old = atomicAdd(
        reinterpret_cast<unsigned long long*>(&d.cnt[u * kCntStride + kCntAbove]),
        (unsigned long long)add);
    off_above = (int)(uint32_t)old;
    off_cand = (int)(old >> 32);
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
    // a wrong prediction can overfill `above`; k_select then rescans, and the
    // guards keep the lists in bounds meanwhile
    if (b > b_hi) {
      if (ia < d.K) above[ia] = p;
      ++ia;
    } else if (b >= b_lo) {
      if (ic < d.hcap) cand[ic] = make_uint2(key[j], (uint32_t)p);
      ++ic;
    }
  }
}

constexpr int kColdChunk = 16384;   // positions per workgroup of the cold histogram
constexpr int kColdBatch = 16;      // loads in flight per thread

// The cold histogram of selection unit u lives in the first 16 KB of the
// unit's candidate list (zeroed by k_init; the scan overwrites it afterwards).
__device__ __forceinline__ uint32_t* cold_hist(const DevState& d, int u) {
  return reinterpret_cast<uint32_t*>(d.cand + (size_t)u * d.hcap);
}

__global__ __launch_bounds__(kScanThreads) void k_cold_hist(DevState d, StepArgs a,
                                                            const float* __restrict__ scores,
                                                            uint64_t stride) {
  __shared__ uint32_t h[kBins1];
  const int u = blockIdx.y, tid = threadIdx.x;
  const int64_t H = a.hist_len[u / (d.G * d.Q)];
  const int64_t base = (int64_t)blockIdx.x * kColdChunk;
  if (base >= H) return;
  const int n = (int)(H - base < kColdChunk ? H - base : kColdChunk);
  for (int b = tid; b < kBins1; b += kScanThreads) h[b] = 0;
  __syncthreads();
  const float* src = scores + (uint64_t)u * stride + base;
  for (int i0 = 0; i0 < n; i0 += kScanThreads * kColdBatch) {
    uint32_t bin[kColdBatch];
#pragma unroll
    for (int j = 0; j < kColdBatch; ++j) {
      const int i = i0 + j * kScanThreads + tid;
      bin[j] = i < n ? order_key(src[i]) >> (32 - kBin1Bits) : kBins1;
    }
#pragma unroll
    for (int j = 0; j < kColdBatch; ++j)
      if (bin[j] < (uint32_t)kBins1) atomicAdd(&h[bin[j]], 1u);
  }
  __syncthreads();
  uint32_t* g = cold_hist(d, u);
  for (int b = tid; b < kBins1; b += kScanThreads)
    if (h[b]) atomicAdd(&g[b], h[b]);
}

// One workgroup per selection unit: the bin where the count from the top
// reaches K becomes the unit's cut bin (H >= K, so it exists).
__global__ __launch_bounds__(kScanThreads) void k_cold_cut(DevState d) {
  __shared__ int wtot[kScanThreads / 64];
  constexpr int kPer = kBins1 / kScanThreads;   // 16 bins per thread, from the top
  const int u = blockIdx.x, tid = threadIdx.x;
  const uint32_t* g = cold_hist(d, u);
  int c[kPer];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    c[j] = (int)g[kBins1 - 1 - (tid * kPer + j)];
    sum += c[j];
  }
  const int incl = block_incl_scan256(sum, wtot);
  int cum = incl - sum;
  if (cum < d.K && incl >= d.K) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (cum < d.K && cum + c[j] >= d.K)
        d.cnt[u * kCntStride + kCntBin1] = kBins1 - 1 - (tid * kPer + j);
      cum += c[j];
    }
  }
}

hipError_t launch_cold_cut(const DevState& d, const StepArgs& a, const float* scores,
                           uint64_t stride, int64_t max_len, hipStream_t st) {
  const int units = d.S * d.G * d.Q;
  dim3 grid((unsigned)((max_len + kColdChunk - 1) / kColdChunk), units);
  hipLaunchKernelGGL(k_cold_hist, grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_cold_cut, dim3(units), dim3(kScanThreads), 0, st, d);
  return hipGetLastError();
}

hipError_t launch_topk_scan(const DevState& d, const StepArgs& a, const float* scores,
                            uint64_t stride, int64_t max_len, bool vec4, hipStream_t st) {
  // Short histories: more, smaller workgroups (the scan is latency-bound);
  // long ones: fewer, because every workgroup bumps its unit's list counters
  // (measured: 2,048-score chunks 4.95 vs 6.2 us at 50K positions x 20 units,
  // but 39 vs 25 us at 1M positions x 16 units).
  const bool small = max_len <= kScanSmallMax;
  const int chunk = small ? 2048 : 4096;
  dim3 grid((unsigned)((max_len + chunk - 1) / chunk), d.S * d.G * d.Q);
  if (vec4 && small)
    hipLaunchKernelGGL((k_topk_scan<true, 2048>), grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  else if (vec4)
    hipLaunchKernelGGL((k_topk_scan<true, 4096>), grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  else if (small)
    hipLaunchKernelGGL((k_topk_scan<false, 2048>), grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  else
    hipLaunchKernelGGL((k_topk_scan<false, 4096>), grid, dim3(kScanThreads), 0, st, d, a, scores, stride);
  return hipGetLastError();
}

}  // namespace hc
