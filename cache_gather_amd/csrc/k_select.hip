// k_select.hip — exact top-K cut, hot-slot lookup, miss compaction and LRU
// victim selection for one unit (session, selection group) per workgroup.
//
// Method (page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
// Offloading"): the selection stays on the GPU, which checks its hot slots
// itself (section "Decision three: let the GPU manage the hot cache
// directly"); slots used in the current round are never replaced (section
// "GPU cache management has hazards too").  Replacement is LRU by last-use
// step with ties to the lowest slot; the i-th miss (ascending position) takes
// the i-th victim.
//
// Design on gfx950 (1,024 threads = 16 wave64, ~104 KB LDS, one unit each):
//  1. Radix-select the remaining 20 key bits (2 x 10-bit digits) over the
//     candidates of the cut bin; if more keys equal the cut key than are
//     needed, radix-select the position cut among them (lower positions win).
//  2. Gather the K winners into LDS and bitonic-sort them by position.
//  3. Lookup pos2slot; hits get last_use = t and are marked in an LDS bitmap of
//     touched slots; misses are compacted in ascending order by wave ballot +
//     mbcnt prefix.
//  4. LRU without any search: `order` holds all C slots sorted by
//     (last_use, slot).  Dropping the hit slots keeps it sorted, so the victims
//     are its first m entries.  The next order is the rest of the list followed
//     by this step's K touched slots (all now last_use = t) in slot order, read
//     out of the bitmap.  One stable partition of C entries per step.
//  5. Apply the m (miss, victim) pairs to pos2slot / slot2pos / last_use in
//     parallel (an evicted position is never one of this step's misses).
#include "hc_internal.h"

namespace hc {

constexpr int kSelThreads = 1024;
constexpr int kWaves = kSelThreads / 64;

struct SelShared {
  uint32_t hist[2048];
  int32_t sel[HC_MAX_TOPK];       // positions, then the slot of each selected row
  int32_t mpos[HC_MAX_TOPK];      // missing positions (ascending)
  int32_t midx[HC_MAX_TOPK];      // index in sel of miss k
  int32_t vic[HC_MAX_TOPK];       // victim slot of miss k
  uint32_t touched[HC_MAX_SLOTS / 32];
  int32_t wtot[kWaves];
  int32_t bcast[4];
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix over the block (thread order); `total` gets the block sum.
__device__ __forceinline__ int block_incl_scan(int v, int32_t* wtot, int& total) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wtot[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    off += i < w ? wtot[i] : 0;
    tot += wtot[i];
  }
  __syncthreads();
  total = tot;
  return x + off;
}

// Rank of this lane's flag among set flags of the block, in thread order, with
// the block count in `total` (wave ballot + mbcnt, then wave offsets).
__device__ __forceinline__ int block_flag_rank(bool f, int32_t* wtot, int& total) {
  const uint64_t bal = __ballot(f);
  const int w = threadIdx.x >> 6;
  const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                               __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
  if (lane_id() == 0) wtot[w] = __popcll(bal);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    off += i < w ? wtot[i] : 0;
    tot += wtot[i];
  }
  __syncthreads();
  total = tot;
  return off + below;
}

// Digit d (of nb bins, nb = 1024 or 2048) such that the count in bins above d
// is < r and the count in bins >= d is >= r; *gt = count in bins above d.
// If `from_top` is false the roles flip: bins below d, ascending.
__device__ void find_digit(const uint32_t* hist, int nb, int r, bool from_top, SelShared& sh,
                           int& digit, int& beyond) {
  const int per = nb / kSelThreads;  // 1 or 2 bins per thread
  if (threadIdx.x == 0) sh.bcast[0] = sh.bcast[1] = 0;  // ordered by the scan's barriers
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int b = from_top ? nb - 1 - (per * threadIdx.x + i) : per * threadIdx.x + i;
    sum += (int)hist[b];
  }
  int total;
  const int incl = block_incl_scan(sum, sh.wtot, total);
  const int excl = incl - sum;
  if (excl < r && r <= incl) {
    int cum = excl;
    for (int i = 0; i < per; ++i) {
      const int b = from_top ? nb - 1 - (per * threadIdx.x + i) : per * threadIdx.x + i;
      if (cum + (int)hist[b] >= r) {
        sh.bcast[0] = b;
        sh.bcast[1] = cum;
        break;
      }
      cum += (int)hist[b];
    }
  }
  __syncthreads();
  digit = sh.bcast[0];
  beyond = sh.bcast[1];
  __syncthreads();
}

__device__ __forceinline__ void clear_hist(SelShared& sh, int nb) {
  for (int b = threadIdx.x; b < nb; b += kSelThreads) sh.hist[b] = 0;
  __syncthreads();
}

// Bitonic sort (ascending) of the kSelThreads * E values in buf.  Value i
// lives in register i % E of thread i / E: compare-exchange partners closer
// than E are in the same thread, closer than 64 E in the same wave (cross-lane
// shuffle, no barrier); only strides of 64 E and more go through LDS.
__device__ __forceinline__ int32_t bitonic_pick(int32_t a, int32_t b, int i, int j, int k) {
  const bool lower = (i & j) == 0, asc = (i & k) == 0;
  return (lower == asc) ? min(a, b) : max(a, b);
}

template <int E>
__device__ void sort_positions(int32_t* buf) {
  constexpr int n = kSelThreads * E;
  const int tid = threadIdx.x;
  int32_t x[E];
#pragma unroll
  for (int e = 0; e < E; ++e) x[e] = buf[tid * E + e];
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64 * E) {
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) buf[tid * E + e] = x[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid * E + e;
          x[e] = bitonic_pick(x[e], buf[i ^ j], i, j, k);
        }
      } else if (j >= E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int i = tid * E + e;
          x[e] = bitonic_pick(x[e], __shfl_xor(x[e], j / E, 64), i, j, k);
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int p = e ^ j;
          if (p > e) {
            const bool asc = ((tid * E + e) & k) == 0;
            const int32_t lo = min(x[e], x[p]), hi = max(x[e], x[p]);
            x[e] = asc ? lo : hi;
            x[p] = asc ? hi : lo;
          }
        }
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < E; ++e) buf[tid * E + e] = x[e];
  __syncthreads();
}

// Miss count of the step, and a clean histogram and list counters for the
// next step's scan.
__device__ __forceinline__ void reset_scan_state(const DevState& d, int u, int m) {
  uint32_t* gh = d.hist + (size_t)u * kBins1;
  for (int b = threadIdx.x; b < kBins1; b += kSelThreads) gh[b] = 0;
  if (threadIdx.x == 0) {
    d.cnt[u * kCnt + kCntAbove] = 0;
    d.cnt[u * kCnt + kCntCand] = 0;
    d.cnt[u * kCnt + kCntMiss] = m;
  }
}

__global__ __launch_bounds__(kSelThreads) void k_select(DevState d, int32_t t,
                                                        int32_t* __restrict__ d_sel,
                                                        int32_t* __restrict__ d_trace) {
  __shared__ SelShared sh;
  const int u = blockIdx.x, tid = threadIdx.x;
  const int K = d.K, C = d.C;
  int32_t* cnt = d.cnt + u * kCnt;
  const int n_above = min(cnt[kCntAbove], K - 1);          // < K by construction
  const int n_cand = (int)min((int64_t)cnt[kCntCand], d.hcap);
  const uint32_t b1 = (uint32_t)cnt[kCntBin1];
  const uint2* cand = d.cand + (size_t)u * d.hcap;
  int r = K - n_above;  // winners still to take from the cut bin, >= 1

  // ---- 1. exact cut key T and position cut among keys equal to T ----------
  int d2, d3, skip;
  clear_hist(sh, 1024);
  for (int i = tid; i < n_cand; i += kSelThreads) atomicAdd(&sh.hist[(cand[i].x >> 10) & 1023], 1u);
  __syncthreads();
  find_digit(sh.hist, 1024, r, true, sh, d2, skip);
  r -= skip;
  clear_hist(sh, 1024);
  for (int i = tid; i < n_cand; i += kSelThreads) {
    const uint32_t k = cand[i].x;
    if (((k >> 10) & 1023) == (uint32_t)d2) atomicAdd(&sh.hist[k & 1023], 1u);
  }
  __syncthreads();
  find_digit(sh.hist, 1024, r, true, sh, d3, skip);
  r -= skip;
  const int n_eq = (int)sh.hist[d3];
  const uint32_t T = (b1 << 20) | ((uint32_t)d2 << 10) | (uint32_t)d3;
  int32_t pcut = 0x7FFFFFFF;  // take ties at T with position <= pcut
  if (r < n_eq) {
    // the r-th smallest position among keys == T: digits of 11, 10, 10 bits
    int e1, e2, e3, below;
    __syncthreads();
    clear_hist(sh, 2048);
    for (int i = tid; i < n_cand; i += kSelThreads) {
      const uint2 c = cand[i];
      if (c.x == T) atomicAdd(&sh.hist[c.y >> 20], 1u);
    }
    __syncthreads();
    find_digit(sh.hist, 2048, r, false, sh, e1, below);
    r -= below;
    clear_hist(sh, 1024);
    for (int i = tid; i < n_cand; i += kSelThreads) {
      const uint2 c = cand[i];
      if (c.x == T && (int)(c.y >> 20) == e1) atomicAdd(&sh.hist[(c.y >> 10) & 1023], 1u);
    }
    __syncthreads();
    find_digit(sh.hist, 1024, r, false, sh, e2, below);
    r -= below;
    clear_hist(sh, 1024);
    const uint32_t hi = ((uint32_t)e1 << 10) | (uint32_t)e2;
    for (int i = tid; i < n_cand; i += kSelThreads) {
      const uint2 c = cand[i];
      if (c.x == T && (c.y >> 10) == hi) atomicAdd(&sh.hist[c.y & 1023], 1u);
    }
    __syncthreads();
    find_digit(sh.hist, 1024, r, false, sh, e3, below);
    pcut = (int32_t)((hi << 10) | (uint32_t)e3);
  }

  // ---- 2. the K winners, sorted by position ------------------------------
  if (tid == 0) sh.bcast[2] = 0;
  __syncthreads();
  const int32_t* above = d.above + (size_t)u * K;
  for (int i = tid; i < n_above; i += kSelThreads) sh.sel[i] = above[i];
  for (int i = tid; i < n_cand; i += kSelThreads) {
    const uint2 c = cand[i];
    if (c.x > T || (c.x == T && (int32_t)c.y <= pcut)) {
      const int o = n_above + atomicAdd(&sh.bcast[2], 1);
      if (o < K) sh.sel[o] = (int32_t)c.y;  // exactly K - n_above winners by construction
    }
  }
  __syncthreads();
  if (sh.bcast[2] != K - n_above) {
    // Inconsistent scan state (cannot happen when the histogram was clean):
    // report an empty selection and touch nothing.
    for (int i = tid; i < K; i += kSelThreads) {
      d_sel[(size_t)u * K + i] = -1;
      d.sel_slot[(size_t)u * K + i] = 0;  // the gather then only reads slot 0
    }
    reset_scan_state(d, u, 0);
    return;
  }
  for (int i = K + tid; i < HC_MAX_TOPK; i += kSelThreads) sh.sel[i] = 0x7FFFFFFF;
  __syncthreads();
  if (K <= kSelThreads) sort_positions<1>(sh.sel);
  else if (K <= 2 * kSelThreads) sort_positions<2>(sh.sel);
  else sort_positions<4>(sh.sel);
  for (int i = tid; i < K; i += kSelThreads) d_sel[(size_t)u * K + i] = sh.sel[i];

  // ---- 3. lookup, hits, ascending miss compaction ------------------------
  const int nwords = (C + 31) >> 5;
  for (int w = tid; w < nwords; w += kSelThreads) sh.touched[w] = 0;
  int32_t* pos2slot = d.pos2slot + (size_t)u * d.hcap;
  int32_t* slot2pos = d.slot2pos + (size_t)u * C;
  int32_t* last_use = d.last_use + (size_t)u * C;
  constexpr int kLookRounds = HC_MAX_TOPK / kSelThreads;
  int32_t lp[kLookRounds], ls[kLookRounds];
#pragma unroll
  for (int r = 0; r < kLookRounds; ++r) {   // all map reads in flight together
    const int i = r * kSelThreads + tid;
    lp[r] = i < K ? sh.sel[i] : 0;
    ls[r] = i < K ? pos2slot[lp[r]] : 0;
  }
  __syncthreads();
  int m = 0;
#pragma unroll
  for (int r = 0; r < kLookRounds; ++r) {
    if (r * kSelThreads >= K) break;
    const int i = r * kSelThreads + tid;
    const bool valid = i < K;
    const bool miss = valid && ls[r] < 0;
    if (valid && !miss) {
      last_use[ls[r]] = t;
      atomicOr(&sh.touched[ls[r] >> 5], 1u << (ls[r] & 31));
    }
    if (valid) sh.sel[i] = ls[r];  // from here on sel[] holds slots (-1 = miss, filled below)
    int total;
    const int k = m + block_flag_rank(miss, sh.wtot, total);
    if (miss) {
      sh.mpos[k] = lp[r];
      sh.midx[k] = i;
    }
    m += total;
  }

  // ---- 4. LRU victims: first m untouched entries of the order list --------
  // Wave w of a round owns 2,048 consecutive entries, lane-interleaved so every
  // load is coalesced; ranks inside the wave come from ballots, and one block
  // scan of the 16 wave totals orders the waves.
  const int32_t* ocur = d.order + ((size_t)u * 2 + (t & 1)) * C;
  int32_t* onxt = d.order + ((size_t)u * 2 + ((t + 1) & 1)) * C;
  const int lane = lane_id(), wv = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  constexpr int kOrdPer = 32;
  int kept = 0;
  for (int j0 = 0; j0 < C; j0 += kSelThreads * kOrdPer) {
    const int wb = j0 + wv * 64 * kOrdPer;
    int32_t v[kOrdPer];
#pragma unroll
    for (int e = 0; e < kOrdPer; ++e) {
      const int j = wb + e * 64 + lane;
      v[e] = j < C ? ocur[j] : -1;
    }
    int wave_total = 0;
#pragma unroll
    for (int e = 0; e < kOrdPer; ++e) {
      const bool keep = v[e] >= 0 && !((sh.touched[v[e] >> 5] >> (v[e] & 31)) & 1u);
      if (!keep) v[e] = -1;
      wave_total += __popcll(__ballot(keep));
    }
    if (lane == 0) sh.wtot[wv] = wave_total;
    __syncthreads();
    int run = kept, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      run += i < wv ? sh.wtot[i] : 0;
      total += sh.wtot[i];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kOrdPer; ++e) {
      const uint64_t bal = __ballot(v[e] >= 0);
      if (v[e] >= 0) {
        const int k = run + __popcll(bal & lt_mask);
        if (k < m) sh.vic[k] = v[e];
        else onxt[k - m] = v[e];
      }
      run += __popcll(bal);
    }
    kept += total;
  }
  __syncthreads();
  for (int k = tid; k < m; k += kSelThreads) atomicOr(&sh.touched[sh.vic[k] >> 5], 1u << (sh.vic[k] & 31));
  __syncthreads();
  // this step's K slots, ascending, close the order list
  int base = C - K;
  for (int w0 = 0; w0 < nwords; w0 += kSelThreads) {
    const int w = w0 + tid;
    uint32_t bits = w < nwords ? sh.touched[w] : 0u;
    int total;
    const int incl = block_incl_scan(__popc(bits), sh.wtot, total);
    int o = base + incl - __popc(bits);
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      onxt[o++] = w * 32 + b;
    }
    base += total;
  }

  // ---- 5. apply (miss, victim) pairs --------------------------------------
  // A miss row is marked in sel_slot as -(slot + 1): the gather then reads it
  // from host RAM and writes it into that slot itself.
  if (tid == 0) sh.bcast[3] = 0;
  __syncthreads();
  int32_t* tr = d_trace ? d_trace + (size_t)u * HC_TRACE_INTS(K) : nullptr;
  int32_t* g_miss = d.miss_pos + (size_t)u * K;   // the gather's dense miss list
  int32_t* g_vic = d.victim + (size_t)u * K;
  int32_t* g_midx = d.miss_idx + (size_t)u * K;
  for (int k = tid; k < m; k += kSelThreads) {
    const int32_t v = sh.vic[k], p = sh.mpos[k];
    const int32_t old = slot2pos[v];
    if (old >= 0) {
      pos2slot[old] = -1;
      atomicAdd(&sh.bcast[3], 1);
    }
    pos2slot[p] = v;
    slot2pos[v] = p;
    last_use[v] = t;
    sh.sel[sh.midx[k]] = -(v + 1);
    g_miss[k] = p;
    g_vic[k] = v;
    g_midx[k] = sh.midx[k];
    if (tr) {
      tr[HC_TRACE_HEADER + K + k] = p;
      tr[HC_TRACE_HEADER + 2 * K + k] = v;
      tr[HC_TRACE_HEADER + 3 * K + k] = old;
    }
  }
  __syncthreads();
  int32_t* g_slot = d.sel_slot + (size_t)u * K;
  for (int i = tid; i < K; i += kSelThreads) {
    const int32_t enc = sh.sel[i];
    g_slot[i] = enc;
    if (tr) {
      tr[HC_TRACE_HEADER + i] = enc < 0 ? -enc - 1 : enc;
      if (i >= m) {
        tr[HC_TRACE_HEADER + K + i] = -1;
        tr[HC_TRACE_HEADER + 2 * K + i] = -1;
        tr[HC_TRACE_HEADER + 3 * K + i] = -1;
      }
    }
  }
  if (tr && tid == 0) {
    tr[0] = K - m;
    tr[1] = m;
    tr[2] = sh.bcast[3];
    tr[3] = 0;
  }

  reset_scan_state(d, u, m);
}

hipError_t launch_select(const DevState& d, int32_t t, int32_t* d_sel, int32_t* d_trace,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_select, dim3(d.S * d.G), dim3(kSelThreads), 0, st, d, t, d_sel, d_trace);
  return hipGetLastError();
}

}  // namespace hc
