// k_fetch.hip — copies this step's missing rows from pinned host RAM into the
// victim slots in HBM, for every layer of each selection group.
//
// On the page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading"
// (section "Decision three: let the GPU manage the hot cache directly") a miss
// reads the registered host-memory copy directly from the GPU; no CPU work sits
// between selection and transfer.  Issuing many small host-side copy
// submissions costs more than the bytes (section "Decision two: let the CPU
// manage the GPU hot cache first"), so here the GPU itself pulls the rows over
// PCIe with ordinary vector loads from the mapped pinned buffers (zero-copy).
//
// gfx950 mapping: one wave copies 8 rows at a time, i.e. 8 x 41 16-byte chunks
// spread over its 64 lanes; every lane issues all of its loads (up to 6 x 16 B)
// before its first store, so a wave keeps ~5 KB of PCIe reads in flight.
// Grid = (ceil(K / 32), S*L): blockIdx.y is the layer; workgroups past the
// unit's miss count exit at once.
#include "hc_internal.h"

namespace hc {

constexpr int kFetchThreads = 256;
constexpr int kRowsPerWave = 8;
constexpr int kRowsPerBlock = kRowsPerWave * (kFetchThreads / 64);
constexpr int kChunks = kRow / 16;  // 41
constexpr int kPerLane = (kRowsPerWave * kChunks + 63) / 64;  // 6

__global__ __launch_bounds__(kFetchThreads) void k_fetch(DevState d) {
  const int sl = blockIdx.y;
  const int s = sl / d.L, l = sl % d.L;
  const int u = s * d.G + l / d.R;
  const int m = d.cnt[u * kCnt + kCntMiss];
  const int row0 = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6) * kRowsPerWave;
  if (row0 >= m) return;
  const int nrows = m - row0 < kRowsPerWave ? m - row0 : kRowsPerWave;
  const int lane = threadIdx.x & 63;
  const int32_t* miss = d.miss_pos + (size_t)u * d.K + row0;
  const int32_t* vic = d.victim + (size_t)u * d.K + row0;
  const uint8_t* src = d.host[sl];
  uint8_t* dst = d.hot + (size_t)sl * d.C * kRow;

  u32x4 v[kPerLane];
#pragma unroll
  for (int it = 0; it < kPerLane; ++it) {
    const int c = lane + 64 * it;
    if (c < nrows * kChunks) {
      const int r = c / kChunks, ch = c - r * kChunks;
      const u32x4* p = reinterpret_cast<const u32x4*>(src + (size_t)miss[r] * kRow) + ch;
      v[it] = __builtin_nontemporal_load(p);
    }
  }
#pragma unroll
  for (int it = 0; it < kPerLane; ++it) {
    const int c = lane + 64 * it;
    if (c < nrows * kChunks) {
      const int r = c / kChunks, ch = c - r * kChunks;
      reinterpret_cast<u32x4*>(dst + (size_t)vic[r] * kRow)[ch] = v[it];
    }
  }
}

hipError_t launch_fetch(const DevState& d, hipStream_t st) {
  dim3 grid((d.K + kRowsPerBlock - 1) / kRowsPerBlock, d.S * d.L);
  hipLaunchKernelGGL(k_fetch, grid, dim3(kFetchThreads), 0, st, d);
  return hipGetLastError();
}

}  // namespace hc
