// k_gather.hip — reads every selected row from its hot slot and writes the
// contiguous bf16 attention buffer [S][L][K][576].
//
// The hot gather emits a compact selection that attention consumes (page "From
// 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading", section
// "Decision three: let the GPU manage the hot cache directly", data-flow
// figure).  Row format (section "Separate historical capacity from the current
// working set"): 512 int8 latent values, 8 fp16 scales (one per 64 values),
// 64 bf16 RoPE values.  Output element j < 512 is the fp32 product
// int8 * scale, exact, rounded to bf16 (nearest, ties to even); the RoPE part
// is copied.  Rows filled by k_fetch are visible here through the kernel
// boundary, so no workgroup reads a slot another workgroup of the same launch
// writes (section "GPU cache management has hazards too").
//
// gfx950 mapping: a row is 40 work items — 32 latent chunks (16 B in, 32 B
// out) and 8 RoPE chunks (16 B in, 16 B out) — so 320 threads (5 wave64) do 8
// rows with every lane busy; lanes of a row read 656 contiguous bytes and
// write 1,152 contiguous bytes.  HBM-bound: 656 B read + 1,152 B written per
// selected row.  bf16 rounding uses v_cvt_pk_bf16_f32 (two values per op).
#include "hc_internal.h"

namespace hc {

constexpr int kRowsPerGatherBlock = 8;
constexpr int kItemsPerRow = 40;
constexpr int kGatherThreads = kRowsPerGatherBlock * kItemsPerRow;  // 320

__device__ __forceinline__ uint32_t bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Sign-extended int8 number k (0..3) of w, as float.
__device__ __forceinline__ float i8f(uint32_t w, int k) {
  return (float)((int32_t)(w << (24 - 8 * k)) >> 24);
}

__global__ __launch_bounds__(kGatherThreads) void k_gather(DevState d, uint16_t* __restrict__ out,
                                                           int64_t total_rows) {
  const int item = threadIdx.x % kItemsPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerGatherBlock + threadIdx.x / kItemsPerRow;
  if (row >= total_rows) return;
  const int64_t sl = row / d.K;
  const int i = (int)(row - sl * d.K);
  const int s = (int)(sl / d.L), l = (int)(sl - (int64_t)s * d.L);
  const int u = s * d.G + l / d.R;
  const int32_t slot = d.sel_slot[(size_t)u * d.K + i];
  const uint8_t* src = d.hot + ((size_t)sl * d.C + slot) * kRow;
  uint8_t* dst = reinterpret_cast<uint8_t*>(out) + (size_t)row * (kOut * 2);

  if (item < 32) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(src + 16 * item);
    const uint16_t sb = *reinterpret_cast<const uint16_t*>(src + HC_SCALE_OFFSET + 2 * (item >> 2));
    const float sc = (float)__builtin_bit_cast(_Float16, sb);
    u32x4 a, b;
    a.x = bf16x2(i8f(q.x, 0) * sc, i8f(q.x, 1) * sc);
    a.y = bf16x2(i8f(q.x, 2) * sc, i8f(q.x, 3) * sc);
    a.z = bf16x2(i8f(q.y, 0) * sc, i8f(q.y, 1) * sc);
    a.w = bf16x2(i8f(q.y, 2) * sc, i8f(q.y, 3) * sc);
    b.x = bf16x2(i8f(q.z, 0) * sc, i8f(q.z, 1) * sc);
    b.y = bf16x2(i8f(q.z, 2) * sc, i8f(q.z, 3) * sc);
    b.z = bf16x2(i8f(q.w, 0) * sc, i8f(q.w, 1) * sc);
    b.w = bf16x2(i8f(q.w, 2) * sc, i8f(q.w, 3) * sc);
    u32x4* o = reinterpret_cast<u32x4*>(dst + 32 * item);
    __builtin_nontemporal_store(a, o);
    __builtin_nontemporal_store(b, o + 1);
  } else {
    const int r = item - 32;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + HC_ROPE_OFFSET + 16 * r);
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + 2 * HC_LATENT_BYTES + 16 * r));
  }
}

hipError_t launch_gather(const DevState& d, uint16_t* d_out, hipStream_t st) {
  const int64_t total = (int64_t)d.S * d.L * d.K;
  const int64_t blocks = (total + kRowsPerGatherBlock - 1) / kRowsPerGatherBlock;
  hipLaunchKernelGGL(k_gather, dim3((uint32_t)blocks), dim3(kGatherThreads), 0, st, d, d_out,
                     total);
  return hipGetLastError();
}

}  // namespace hc
