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
//     candidates of the cut bin (kept in LDS when they fit); if more keys
//     equal the cut key than are needed, radix-select the position cut among
//     them (lower positions win).
//  2. Emit the K winners in ascending position order without a sort: count
//     them into at most 8,192 buckets of 2^s consecutive positions, place
//     each bucket at its prefix offset, and give each winner its rank inside
//     its bucket by comparing it with the bucket's other members (rarely more
//     than a few: 8 positions per bucket at 50K, 128 at a million).
//  3. Positions the recent ring holds (a suffix of the ascending selection)
//     are read from the ring and skip the cache.  For the rest, look up
//     pos2slot; hits get last_use = t and are marked in an LDS bitmap of
//     touched slots; misses are compacted in ascending order by wave ballot +
//     mbcnt prefix.
//  4. LRU without any search: a queue of (slot, step) entries in ascending
//     (step, slot) order, live while the slot's last use equals the entry's
//     step.  The victims are the first m live entries the step's hits do not
//     pin; the step's slots are appended in slot order; the queue is
//     compacted into its second buffer once every C / K steps or so.
//  5. Apply the m (miss, victim) pairs to pos2slot / slot2pos / last_use in
//     parallel (an evicted position is never one of this step's misses).
#include "hc_block.h"

namespace hc {

constexpr int kCandCache = 8192;               // cut-bin candidates kept in LDS (64 KB)
constexpr int kOrdBuckets = 8192;              // position buckets of the ordering phase

struct SelShared {
  uint32_t hist[kBins1];          // histograms of up to 4,096 bins
  int32_t sel[HC_MAX_TOPK];     // winners by ascending position, then the slot of each
  int32_t mpos[HC_MAX_TOPK];    // winners unordered (phase 2), then missing positions
  union {
    uint2 cand[kCandCache];       // phase 1: (key, position) of the cut bin
    struct {
      uint32_t start[kOrdBuckets];  // winners per bucket, then each bucket's offset
      int32_t member[HC_MAX_TOPK];  // winners grouped by bucket
    } ord;                        // phase 2
    struct {
      int32_t midx[HC_MAX_TOPK];  // index in sel of miss k
      int32_t vic[HC_MAX_TOPK];   // victim slot of miss k
      uint32_t touched[HC_MAX_SLOTS / 32];
    } lru;                        // phases 3-5
  } u;
  int32_t wtot[kWaves];
  int32_t bcast[4];
  int32_t wmax;
  int32_t n_ring;                 // selected rows the recent ring holds
};

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

// Miss count of the step, cleared list counters and the cut bin for the next
// step's scan.
__device__ __forceinline__ void reset_scan_state(const DevState& d, int u, int m, int cut_bin) {
  if (threadIdx.x == 0) {
    d.cnt[u * kCntStride + kCntAbove] = 0;
    d.cnt[u * kCntStride + kCntCand] = 0;
    d.cnt[u * kCntStride + kCntMiss] = m;
    d.cnt[u * kCntStride + kCntBin1] = cut_bin;  // centre of the next step's cut window
  }
}

// kTopkOnly (multi-query rounds): workgroup u is selection unit (s, g, q) and
// stops after writing its selection; k_round then runs steps 3-5 on the union
// of the group's selections.  Otherwise (one query) u is the unit (s, g).
template <bool kTopkOnly>
__global__ __launch_bounds__(kSelThreads) void k_select(DevState d, StepArgs a,
                                                        const float* __restrict__ scores,
                                                        uint64_t stride,
                                                        int32_t* __restrict__ d_sel,
                                                        int32_t* __restrict__ d_trace) {
  __shared__ SelShared sh;
  const int u = blockIdx.x, tid = threadIdx.x;
  const int session = u / (d.G * d.Q);
  const int K = d.K, C = d.C;
  const int32_t t = a.t;
  int32_t* cnt = d.cnt + u * kCntStride;
  int32_t* above_g = d.above + (size_t)u * K;
  uint2* gcand = d.cand + (size_t)u * d.hcap;

  // ---- 0. the cut bin b1: the 12-bit bin holding the K-th key ---------------
  uint32_t b_lo, b_hi;
  cut_window(cnt[kCntBin1], b_lo, b_hi);
  int n_above = cnt[kCntAbove];                      // keys above the window
  int n_cand = (int)min((int64_t)cnt[kCntCand], d.hcap);
  if (!(n_above < K && (int64_t)n_above + n_cand >= K)) {
    // The K-th key left the predicted window: rebuild both lists from the
    // scores — a 12-bit histogram for b1, then bins above b1 -> above, bin
    // b1 -> cand — and use the one-bin window [b1, b1].
    const int64_t H = a.hist_len[session];
    const float* src = scores + (uint64_t)u * stride;
    clear_hist(sh, kBins1);
    for (int64_t i = tid; i < H; i += kSelThreads)
      atomicAdd(&sh.hist[order_key(src[i]) >> (32 - kBin1Bits)], 1u);
    __syncthreads();
    int bt, gt;
    find_digit(sh.hist, kBins1, K, true, sh, bt, gt);
    if (tid == 0) sh.bcast[2] = sh.bcast[3] = 0;
    __syncthreads();
    const uint64_t lt = (lane_id() == 0) ? 0ull : (~0ull >> (64 - lane_id()));
    for (int64_t i0 = 0; i0 < H; i0 += kSelThreads) {
      const int64_t i = i0 + tid;
      uint32_t key = 0, b = 0;
      if (i < H) {
        key = order_key(src[i]);
        b = key >> (32 - kBin1Bits);
      }
      const bool up = i < H && b > (uint32_t)bt, eq = i < H && b == (uint32_t)bt;
      const uint64_t bu = __ballot(up), be = __ballot(eq);
      int ou = 0, oe = 0;
      if (lane_id() == 0) {
        if (bu) ou = atomicAdd(&sh.bcast[2], __popcll(bu));
        if (be) oe = atomicAdd(&sh.bcast[3], __popcll(be));
      }
      // every lane is active here, so the first active lane is lane 0
      ou = __builtin_amdgcn_readfirstlane(ou) + __popcll(bu & lt);
      oe = __builtin_amdgcn_readfirstlane(oe) + __popcll(be & lt);
      if (up && ou < K) above_g[ou] = (int32_t)i;
      if (eq && oe < d.hcap) gcand[oe] = make_uint2(key, (uint32_t)i);
    }
    __syncthreads();
    n_above = min(sh.bcast[2], K - 1);   // = gt < K
    n_cand = (int)min((int64_t)sh.bcast[3], d.hcap);
    b_lo = b_hi = (uint32_t)bt;
    __syncthreads();
  }
  // Copy the candidates into LDS when they fit, counting them per window bin;
  // the bin where the count from the top reaches K is b1.
  const bool cached = n_cand <= kCandCache;
  // Every pass below visits the candidates through each_cand, with the loop
  // written once for LDS and once for global memory: through one pointer that
  // may be either, the compiler emits generic loads that wait for every
  // outstanding load and LDS operation, one candidate at a time.
  auto each_cand = [&](auto&& f) {
    if (cached) {
#pragma unroll 4
      for (int i = tid; i < n_cand; i += kSelThreads) f(sh.u.cand[i]);
    } else {
      for (int i = tid; i < n_cand; i += kSelThreads) f(gcand[i]);
    }
  };
  clear_hist(sh, kBins1);
  if (cached) {
    // all of this thread's global reads in flight together
    constexpr int kCopy = kCandCache / kSelThreads;   // 8
    uint2 c[kCopy];
#pragma unroll
    for (int r = 0; r < kCopy; ++r) {
      const int i = r * kSelThreads + tid;
      c[r] = i < n_cand ? gcand[i] : uint2{0u, 0u};
    }
#pragma unroll
    for (int r = 0; r < kCopy; ++r) {
      const int i = r * kSelThreads + tid;
      if (i >= n_cand) continue;
      sh.u.cand[i] = c[r];
      atomicAdd(&sh.hist[(c[r].x >> (32 - kBin1Bits)) - b_lo], 1u);
    }
  } else {
    for (int i = tid; i < n_cand; i += kSelThreads)
      atomicAdd(&sh.hist[(gcand[i].x >> (32 - kBin1Bits)) - b_lo], 1u);
  }
  __syncthreads();
  int rel, beyond;
  find_digit(sh.hist, kBins1, K - n_above, true, sh, rel, beyond);
  const uint32_t b1 = b_lo + (uint32_t)rel;
  int r = K - n_above - beyond;  // winners still to take from bin b1, >= 1

  // ---- 1. exact cut key T and position cut among keys equal to T ----------
  int d2, d3, skip;
  clear_hist(sh, 1024);
  each_cand([&](const uint2 c) {
    if ((c.x >> 20) == b1) atomicAdd(&sh.hist[(c.x >> 10) & 1023], 1u);
  });
  __syncthreads();
  find_digit(sh.hist, 1024, r, true, sh, d2, skip);
  r -= skip;
  clear_hist(sh, 1024);
  each_cand([&](const uint2 c) {
    if ((c.x >> 10) == ((b1 << 10) | (uint32_t)d2)) atomicAdd(&sh.hist[c.x & 1023], 1u);
  });
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
    each_cand([&](const uint2 c) {
      if (c.x == T) atomicAdd(&sh.hist[c.y >> 20], 1u);
    });
    __syncthreads();
    find_digit(sh.hist, 2048, r, false, sh, e1, below);
    r -= below;
    clear_hist(sh, 1024);
    each_cand([&](const uint2 c) {
      if (c.x == T && (int)(c.y >> 20) == e1) atomicAdd(&sh.hist[(c.y >> 10) & 1023], 1u);
    });
    __syncthreads();
    find_digit(sh.hist, 1024, r, false, sh, e2, below);
    r -= below;
    clear_hist(sh, 1024);
    const uint32_t hi = ((uint32_t)e1 << 10) | (uint32_t)e2;
    each_cand([&](const uint2 c) {
      if (c.x == T && (c.y >> 10) == hi) atomicAdd(&sh.hist[c.y & 1023], 1u);
    });
    __syncthreads();
    find_digit(sh.hist, 1024, r, false, sh, e3, below);
    pcut = (int32_t)((hi << 10) | (uint32_t)e3);
  }

  // ---- 2. the K winners, in ascending position order ---------------------
  if (tid == 0) {
    sh.bcast[2] = 0;
    sh.wmax = 0;
    sh.n_ring = 0;
  }
  __syncthreads();
  int32_t pmax = 0;
  {
    // n_above < K: at most 4 per thread, all reads in flight together
    constexpr int kAbove = HC_MAX_TOPK / kSelThreads;
    int32_t ap[kAbove];
#pragma unroll
    for (int r = 0; r < kAbove; ++r) {
      const int i = r * kSelThreads + tid;
      ap[r] = i < n_above ? above_g[i] : 0;
    }
#pragma unroll
    for (int r = 0; r < kAbove; ++r) {
      const int i = r * kSelThreads + tid;
      if (i >= n_above) continue;
      sh.mpos[i] = ap[r];
      pmax = max(pmax, ap[r]);
    }
  }
  // candidates that win, compacted per wave: one LDS atomic per wave
  const uint64_t lt_mask = (lane_id() == 0) ? 0ull : (~0ull >> (64 - lane_id()));
  auto win_pass = [&](auto&& cand_at) {
    for (int i0 = 0; i0 < n_cand; i0 += kSelThreads) {
      const int i = i0 + tid;
      bool win = false;
      int32_t p = 0;
      if (i < n_cand) {
        const uint2 c = cand_at(i);
        p = (int32_t)c.y;
        win = c.x > T || (c.x == T && p <= pcut);
      }
      const uint64_t bal = __ballot(win);
      int base = 0;
      if (lane_id() == 0 && bal) base = atomicAdd(&sh.bcast[2], __popcll(bal));
      base = __builtin_amdgcn_readfirstlane(base);   // lane 0's: every lane is active
      if (win) {
        const int o = n_above + base + __popcll(bal & lt_mask);
        if (o < K) sh.mpos[o] = p;  // exactly K - n_above winners by construction
        pmax = max(pmax, p);
      }
    }
  };
  if (cached)
    win_pass([&](int i) { return sh.u.cand[i]; });
  else
    win_pass([&](int i) { return gcand[i]; });
  pmax = wave_max(pmax);
  if (lane_id() == 0) atomicMax(&sh.wmax, pmax);
  __syncthreads();
  if (sh.bcast[2] != K - n_above) {
    // Inconsistent scan state (cannot happen when the histogram was clean):
    // report an empty selection and touch nothing.
    for (int i = tid; i < K; i += kSelThreads) {
      d_sel[(size_t)u * K + i] = -1;
      d.sel_slot[(size_t)u * K + i] = 0;  // the gather then only reads slot 0
    }
    reset_scan_state(d, u, 0, (int)b1);
    return;
  }
  {
    // buckets of 2^shift positions, at most kOrdBuckets of them
    const int wmax = sh.wmax;
    int shift = 0;
    while ((wmax >> shift) >= kOrdBuckets) ++shift;
    const int nb = (wmax >> shift) + 1;
    constexpr int kRounds = HC_MAX_TOPK / kSelThreads;   // winners per thread
    constexpr int kBPer = kOrdBuckets / kSelThreads;     // buckets per thread
    for (int b = tid; b < nb; b += kSelThreads) sh.u.ord.start[b] = 0;
    __syncthreads();
    int32_t wp[kRounds];
    int arrival[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int i = r * kSelThreads + tid;
      wp[r] = i < K ? sh.mpos[i] : 0;
      arrival[r] = i < K ? (int)atomicAdd(&sh.u.ord.start[wp[r] >> shift], 1u) : 0;
    }
    __syncthreads();
    int cnt8[kBPer];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
      const int b = tid * kBPer + j;
      cnt8[j] = b < nb ? (int)sh.u.ord.start[b] : 0;
      sum += cnt8[j];
    }
    int total;
    int off = block_incl_scan(sum, sh.wtot, total) - sum;
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
      const int b = tid * kBPer + j;
      if (b < nb) sh.u.ord.start[b] = (uint32_t)off;
      off += cnt8[j];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int i = r * kSelThreads + tid;
      if (i < K) sh.u.ord.member[sh.u.ord.start[wp[r] >> shift] + arrival[r]] = wp[r];
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int i = r * kSelThreads + tid;
      if (i >= K) continue;
      const int b = wp[r] >> shift;
      const int lo = (int)sh.u.ord.start[b];
      const int hi = b + 1 < nb ? (int)sh.u.ord.start[b + 1] : K;
      int rank = 0;
      for (int q = lo; q < hi; ++q) rank += sh.u.ord.member[q] < wp[r];
      sh.sel[lo + rank] = wp[r];
    }
  }
  __syncthreads();
  for (int i = tid; i < K; i += kSelThreads) d_sel[(size_t)u * K + i] = sh.sel[i];
  if (kTopkOnly) {
    reset_scan_state(d, u, 0, (int)b1);
    return;
  }

  // ---- 3. lookup, hits, ascending miss compaction ------------------------
  const int nwords = (C + 31) >> 5;
  for (int w = tid; w < nwords; w += kSelThreads) sh.u.lru.touched[w] = 0;
  int32_t* pos2slot = d.pos2slot + (size_t)u * d.hcap;
  int32_t* slot2pos = d.slot2pos + (size_t)u * C;
  int32_t* last_use = d.last_use + (size_t)u * C;
  constexpr int kLookRounds = HC_MAX_TOPK / kSelThreads;
  const uint32_t ring_lo = a.ring_lo[session];
  int32_t lp[kLookRounds], ls[kLookRounds];
#pragma unroll
  for (int r = 0; r < kLookRounds; ++r) {   // all map reads in flight together
    const int i = r * kSelThreads + tid;
    lp[r] = i < K ? sh.sel[i] : 0;
    const bool in_ring = i < K && (uint32_t)lp[r] >= ring_lo;
    ls[r] = i < K && !in_ring ? pos2slot[lp[r]] : 0;
    // the first ring row of the ascending selection counts the suffix
    if (in_ring && (i == 0 || (uint32_t)sh.sel[i - 1] < ring_lo)) sh.n_ring = K - i;
  }
  __syncthreads();
  const int n_ring = sh.n_ring;
  const int first_ring = K - n_ring;
  int m = 0;
#pragma unroll
  for (int r = 0; r < kLookRounds; ++r) {
    if (r * kSelThreads >= K) break;
    const int i = r * kSelThreads + tid;
    const bool valid = i < K;
    const bool in_ring = valid && i >= first_ring;
    const bool miss = valid && !in_ring && ls[r] < 0;
    if (valid && !in_ring && !miss) {
      last_use[ls[r]] = t;
      atomicOr(&sh.u.lru.touched[ls[r] >> 5], 1u << (ls[r] & 31));
    }
    // from here on sel[] holds slots: C + ring entry for ring rows, -1 for a
    // miss (its victim is filled in below)
    if (valid) sh.sel[i] = in_ring ? d.C + (int32_t)((uint32_t)lp[r] % (uint32_t)d.ring_rows) : ls[r];
    int total;
    const int k = m + block_flag_rank(miss, sh.wtot, total);
    if (miss) {
      sh.mpos[k] = lp[r];
      sh.u.lru.midx[k] = i;
    }
    m += total;
  }

  // ---- 4. LRU victims: first m live, unpinned entries of the queue -------
  if (d.policy == HC_REPLACE_LRU)
    lru_victims(d, u, t, m, K - n_ring, sh.u.lru.touched, sh.u.lru.vic, sh.wtot, &sh.bcast[0]);
  else
    hand_victims(d, u, m, d.policy == HC_REPLACE_CLOCK, sh.u.lru.touched, sh.u.lru.vic, sh.wtot,
                 &sh.bcast[0]);

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
    const int32_t v = sh.u.lru.vic[k], p = sh.mpos[k];
    const int32_t old = slot2pos[v];
    if (old >= 0) {
      pos2slot[old] = -1;
      atomicAdd(&sh.bcast[3], 1);
    }
    pos2slot[p] = v;
    slot2pos[v] = p;
    last_use[v] = t;
    sh.sel[sh.u.lru.midx[k]] = -(v + 1);
    g_miss[k] = p;
    g_vic[k] = v;
    g_midx[k] = sh.u.lru.midx[k];
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
    tr[0] = K - m - n_ring;
    tr[1] = m;
    tr[2] = sh.bcast[3];
    tr[3] = n_ring;
  }

  reset_scan_state(d, u, m, (int)b1);
}

hipError_t launch_select(const DevState& d, const StepArgs& a, const float* scores,
                         uint64_t stride, int32_t* d_sel, int32_t* d_trace, hipStream_t st) {
  if (d.Q == 1)
    hipLaunchKernelGGL(k_select<false>, dim3(d.S * d.G), dim3(kSelThreads), 0, st, d, a, scores,
                       stride, d_sel, d_trace);
  else
    hipLaunchKernelGGL(k_select<true>, dim3(d.S * d.G * d.Q), dim3(kSelThreads), 0, st, d, a,
                       scores, stride, d_sel, d_trace);
  return hipGetLastError();
}

}  // namespace hc
