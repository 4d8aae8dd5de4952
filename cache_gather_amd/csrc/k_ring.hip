// k_ring.hip — recent ring of appended rows and its batched copyback (gfx950).
//
// Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading": in
// the data-flow figure of "Decision three" new KV goes to a GPU recent ring
// and then, by a batched copyback, to RAM history; section "GPU cache
// management has hazards too": the ring protects new rows that have not
// reached RAM yet; "Decision two" found that many small transfers cost more
// than their bytes and copied back in batches of 64 rows, and later work used
// compute copies and packing for small logs to cut DMA queue operations.
//
// Here one append launch writes the new row of every (session, layer) into
// its ring entry, and one copyback launch moves every pending row of every
// session and layer into the pinned host rows with GPU stores over PCIe (a
// compute copy: one launch instead of one DMA operation per layer).  A second
// tiny launch then publishes the new host row count of each session, so the
// count never runs ahead of the bytes.
//
// Rows are 656 B = 41 chunks of 16 B; one wave64 per row, 41 lanes active.
#include "hc_internal.h"

namespace hc {

constexpr int kChunks = kRow / 16;  // 41

__global__ __launch_bounds__(64) void k_append(DevState d, AppendArgs a,
                                               const uint8_t* __restrict__ rows) {
  const int sl = blockIdx.x;  // s * L + l
  const uint32_t e = a.entry[sl / d.L];
  if (e == kNoRing || threadIdx.x >= kChunks) return;
  const u32x4 v = *reinterpret_cast<const u32x4*>(rows + (size_t)sl * kRow + 16 * threadIdx.x);
  *reinterpret_cast<u32x4*>(d.ring + ((size_t)sl * d.ring_rows + e) * kRow + 16 * threadIdx.x) = v;
}

__global__ __launch_bounds__(64) void k_copyback(DevState d, CopybackArgs a) {
  const int sl = blockIdx.y;
  const int s = sl / d.L;
  const uint32_t p = a.lo[s] + blockIdx.x;
  if (p >= a.hi[s] || threadIdx.x >= kChunks) return;
  const u32x4 v = *reinterpret_cast<const u32x4*>(
      d.ring + ((size_t)sl * d.ring_rows + p % (uint32_t)d.ring_rows) * kRow + 16 * threadIdx.x);
  uint8_t* host = const_cast<uint8_t*>(d.host[sl]);
  *reinterpret_cast<u32x4*>(host + (size_t)p * kRow + 16 * threadIdx.x) = v;
}

__global__ __launch_bounds__(256) void k_commit(CopybackArgs a, int n_sessions,
                                                uint64_t* host_count) {
  for (int s = threadIdx.x; s < n_sessions; s += blockDim.x)
    if (a.hi[s] > a.lo[s]) host_count[s] = a.hi[s];
}

hipError_t launch_append(const DevState& d, const AppendArgs& a, const uint8_t* d_rows,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_append, dim3(d.S * d.L), dim3(64), 0, st, d, a, d_rows);
  return hipGetLastError();
}

hipError_t launch_copyback(const DevState& d, const CopybackArgs& a, uint64_t* host_count,
                           hipStream_t st) {
  if (a.max_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(k_copyback, dim3(a.max_rows, d.S * d.L), dim3(64), 0, st, d, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_commit, dim3(1), dim3(256), 0, st, a, d.S, host_count);
  return hipGetLastError();
}

}  // namespace hc
