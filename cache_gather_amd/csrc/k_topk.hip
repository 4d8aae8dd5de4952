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
// [b_lo, b_hi] of top-16-bit key prefixes predicted from the previous step's
// cut key (its prefix +- 8; the whole key range on a unit's first step, or
// the bin of a first-step histogram one bin either side): keys above the
// window and keys inside it are the unit's entries, kept with their key.  Each
// workgroup owns one segment of consecutive positions and writes the
// segment's entries in ascending position order to a region of its own
// (cand[su][segment * seg_len ...]) and its counts to seg[su][segment]
// (entries, how many of them lie above the window): no atomics and no
// ordering work is left for k_select, which reads the counts, knows how many
// keys lie above the window, and whether the K-th key fell inside it.  If it
// did, the entries are exact (everything above the cut bin is selected; only
// the cut bin's entries need the remaining 20 bits), and concatenated in
// segment order they are already in position order; if not, k_select rescans
// the scores itself.  Scores change little between decode steps (the history
// is the same apart from one appended position), so the window almost always
// holds and a step reads the history once.
//
// With one query row per round the scan also looks up each entry's slot, so
// that the select kernel reads it beside the entry instead of making about
// 3,000 dependent random reads from one workgroup (a workgroup serves about
// one cache line of a random gather per clock).
//
// A context's first step has no previous cut bin.  Rather than classify every
// key as an entry (which leaves one k_select workgroup to rank the whole
// history: 1.4 ms at a million positions), k_cold_hist counts the keys of
// every 12-bit bin over many workgroups and k_cold_cut places the window on
// the bin holding the K-th key, so the first step's lists are small too.
//
// Grid = (segments) x (selection units: one per query row of each session and
// group), 256 threads; a segment is `tiles` chunks of 2,048 positions (one
// chunk unless the history has more than kMaxSegs chunks); a streaming read of
// 4 B per position, plus one slot-map read per entry.
#include "hc_internal.h"

namespace hc {

constexpr int kScanThreads = 256;
constexpr int kScanChunk = 2048;   // positions per scan pass of a workgroup

// Loads this thread's scores of a chunk: four consecutive positions per group,
// group j of thread tid at chunk positions 4 * (tid + 256 j) + [0, 4), so that
// the order (j, thread, element) is the position order.  Invalid positions
// (>= n) read as 0 and are masked by the caller.
// The loads are non-temporal: a step reads its scores once, and a normal load
// would allocate them in the 256 MB Infinity Cache, displacing what the
// step's later kernels read again (the hot slots the gather reads, the maps
// and queues of the select kernel).
template <bool VEC, int kGroups>
__device__ __forceinline__ void load_chunk(const float* src, int n, float (&x)[4 * kGroups]) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kGroups; ++j) {
    const int q = tid + kScanThreads * j;
    if (VEC) {
      f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
      if (4 * q < n) v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + q);
      x[4 * j + 0] = v.x;
      x[4 * j + 1] = v.y;
      x[4 * j + 2] = v.z;
      x[4 * j + 3] = v.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        x[4 * j + c] = 4 * q + c < n ? __builtin_nontemporal_load(src + 4 * q + c) : 0.f;
    }
  }
}

// Inclusive prefix sums over the 256 threads of the block (thread order) of
// three values at once, with their block totals.
__device__ __forceinline__ void block_incl_scan256x3(int (&v)[3], int (&tot)[3], int (*wtot)[4]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x[3];
#pragma unroll
  for (int f = 0; f < 3; ++f) {
    x[f] = wave_incl_scan(v[f]);
    if (lane == 63) wtot[f][w] = x[f];
  }
  __syncthreads();
#pragma unroll
  for (int f = 0; f < 3; ++f) {
    int off = 0, t = 0;
#pragma unroll
    for (int i = 0; i < kScanThreads / 64; ++i) {
      off += i < w ? wtot[f][i] : 0;
      t += wtot[f][i];
    }
    v[f] = x[f] + off;
    tot[f] = t;
  }
  __syncthreads();
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

// CHUNK scores per pass (2,048: two groups of four per thread; 4,096 would be
// four); `tiles` chunks per workgroup (its segment).
// The workgroup is latency-bound: its first tile's scores are requested
// before anything else is known — their addresses need only the grid
// position, the score pointer and the stride (the loads are bounded by the
// row's stride, as the caller's array is [units][stride], and masked by the
// history length afterwards) — and the unit's counter line comes in the same
// round as a vector load (lane i holds word i mod 16).  m_gq = div_magic(G Q)
// gives the session without a division.  The compiler is held to eight waves
// per SIMD (it keeps fewer scalar registers, spilling some to vector lanes):
// without the bound the kernel's scalar registers allowed seven, so 1,792
// workgroups were resident at once instead of 2,048.
template <bool VEC, int CHUNK>
__global__ __launch_bounds__(kScanThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_topk_scan(DevState d, StepArgs a, const float* __restrict__ scores, uint64_t stride,
                 int tiles, uint32_t m_gq) {
  constexpr int kGroups = CHUNK / (4 * kScanThreads);   // 2 or 4
  static_assert(kGroups == 2 || kGroups == 4, "chunk of 2,048 or 4,096");
  __shared__ int wtot[3][kScanThreads / 64];
  const int su = blockIdx.y;  // selection unit (s, g, q)
  const int tid = threadIdx.x;
  const int64_t seg_len = (int64_t)CHUNK * tiles;
  const int64_t seg0 = (int64_t)blockIdx.x * seg_len;   // < max history <= stride
  const float* row = scores + (uint64_t)su * stride;
  float x[4 * kGroups];
  load_chunk<VEC, kGroups>(row + seg0, (int)min((int64_t)CHUNK, (int64_t)stride - seg0), x);
  static_assert(kCnt <= 16, "counters read from lanes 0-15");
  const int cword = d.cnt[(size_t)su * kCntStride + (tid & 15)];
  const int session = div_by(su, m_gq);
  const int64_t H = a.hist_len[session];
  if (seg0 >= H) return;

  // predicted cut window, in top-16-bit key units (none yet: every key)
  uint32_t b_lo, b_hi;
  cut_window(__builtin_amdgcn_readlane(cword, kCntWinLo), __builtin_amdgcn_readlane(cword, kCntWinHi),
             b_lo, b_hi);
  Ent* out = d.cand + (size_t)su * d.hcap + seg0;
  // one query row: each entry's slot, looked up here by the many scan
  // workgroups rather than one per unit later (the step's slot map is that of
  // the previous step until its select kernel has run)
  const bool lookup = d.Q == 1;
  const int32_t* pos2slot = d.pos2slot + (size_t)su * d.hcap;
  const uint32_t ring_lo = a.ring_lo[session];
  int run = 0, n_above = 0;   // entries of the segment so far, of which above the window
  for (int tile = 0; tile < tiles; ++tile) {
    const int64_t base = seg0 + (int64_t)tile * CHUNK;
    if (base >= H) break;
    const int n = (int)(H - base < CHUNK ? H - base : CHUNK);
    if (tile > 0) load_chunk<VEC, kGroups>(row + base, n, x);
    uint32_t key[4 * kGroups];
    uint32_t ent = 0;   // bit 4j + c: element c of group j is an entry
    int cj[4] = {0, 0, 0, 0}, na = 0;
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * j + c;
        key[e] = order_key(x[e]);
        const uint32_t b = key[e] >> 16;
        const bool ok = 4 * (tid + kScanThreads * j) + c < n;
        const bool up = ok && b > b_hi, in = ok && b >= b_lo && b <= b_hi;
        ent |= (uint32_t)(up || in) << e;
        cj[j] += up || in;
        na += up;
      }
    // the entries' slots, requested now so that the block scan below runs
    // while they are in flight
    int32_t sl[4 * kGroups];
#pragma unroll
    for (int e = 0; e < 4 * kGroups; ++e) {
      const int64_t p = base + 4 * (tid + kScanThreads * (e >> 2)) + (e & 3);
      sl[e] = lookup && ((ent >> e) & 1u) && (uint64_t)p < (uint64_t)ring_lo ? pos2slot[p] : -1;
    }
    // group totals are at most 1,024 per chunk: two groups per packed word
    int v[3] = {cj[0] | (cj[1] << 16), cj[2] | (cj[3] << 16), na};
    const int own[3] = {v[0], v[1], v[2]};
    int tot[3];
    block_incl_scan256x3(v, tot, wtot);
    const int gtot[4] = {tot[0] & 0xFFFF, tot[0] >> 16, tot[1] & 0xFFFF, tot[1] >> 16};
    const int gexc[4] = {(v[0] - own[0]) & 0xFFFF, (v[0] - own[0]) >> 16,
                         (v[1] - own[1]) & 0xFFFF, (v[1] - own[1]) >> 16};
    int gbase = run;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      int o = gbase + gexc[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 4 * j + c;
        if ((ent >> e) & 1u) {
          const int64_t p = base + 4 * (tid + kScanThreads * j) + c;
          out[o++] = Ent{key[e], (uint32_t)p, sl[e]};
        }
      }
      gbase += gtot[j];
    }
    run = gbase;
    n_above += tot[2];
  }
  if (tid == 0) d.seg[(size_t)su * d.max_segs + blockIdx.x] = make_int2(run, n_above);
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
      if (cum < d.K && cum + c[j] >= d.K) {
        // the bin holding the K-th key, one bin either side, in 16-bit units
        const int b = kBins1 - 1 - (tid * kPer + j);
        d.cnt[u * kCntStride + kCntWinLo] = b > 0 ? (b - 1) << 4 : 0;
        d.cnt[u * kCntStride + kCntWinHi] = b < kBins1 - 1 ? ((b + 2) << 4) - 1 : 65535;
      }
      cum += c[j];
    }
  }
}

hipError_t launch_cold_cut(const DevState& d, const StepArgs& a, const float* scores,
                           uint64_t stride, int64_t max_len, hipStream_t st, StageEv ev) {
  const int units = d.S * d.G * d.Q;
  dim3 grid((unsigned)((max_len + kColdChunk - 1) / kColdChunk), units);
  hipExtLaunchKernelGGL(k_cold_hist, grid, dim3(kScanThreads), 0, st, ev.start, nullptr, 0, d, a,
                        scores, stride);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipExtLaunchKernelGGL(k_cold_cut, dim3(units), dim3(kScanThreads), 0, st, nullptr, ev.stop, 0, d);
  return hipGetLastError();
}

// Segment length of a step whose longest history is max_len: one chunk of
// 2,048 positions, or several once there would be more segments than
// max_segs.
int64_t scan_seg_len(int64_t max_len, int max_segs) {
  const int64_t chunks = (max_len + kScanChunk - 1) / kScanChunk;
  const int64_t tiles = (chunks + max_segs - 1) / max_segs;
  return kScanChunk * (tiles < 1 ? 1 : tiles);
}

hipError_t launch_topk_scan(const DevState& d, const StepArgs& a, const float* scores,
                            uint64_t stride, int64_t max_len, bool vec4, hipStream_t st,
                            StageEv ev) {
  // 2,048 positions per workgroup: the scan is latency-bound, so more, smaller
  // workgroups (more of them resident per CU) finish sooner (the 16 x 1M scan:
  // 24.6 us against 28.5 us in 4,096-position workgroups)
  const int64_t seg_len = scan_seg_len(max_len, d.max_segs);
  const int tiles = (int)(seg_len / kScanChunk);
  dim3 grid((unsigned)((max_len + seg_len - 1) / seg_len), d.S * d.G * d.Q);
  const uint32_t m_gq = div_magic((uint32_t)(d.G * d.Q));
  if (vec4)
    hipExtLaunchKernelGGL((k_topk_scan<true, kScanChunk>), grid, dim3(kScanThreads), 0, st, ev.start,
                          ev.stop, 0, d, a, scores, stride, tiles, m_gq);
  else
    hipExtLaunchKernelGGL((k_topk_scan<false, kScanChunk>), grid, dim3(kScanThreads), 0, st, ev.start,
                          ev.stop, 0, d, a, scores, stride, tiles, m_gq);
  return hipGetLastError();
}

}  // namespace hc
