// k_select.hip — exact top-K cut, ordering, hot-slot lookup, miss compaction
// and LRU victim selection for one unit (session, selection group) per
// workgroup.
//
// Method (page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache
// Offloading"): the selection stays on the GPU, which checks its hot slots
// itself (section "Decision three: let the GPU manage the hot cache
// directly"); slots used in the current round are never replaced (section
// "GPU cache management has hazards too").  Replacement is LRU by last-use
// step with ties to the lowest slot; the i-th miss (ascending position) takes
// the i-th victim.
//
// Design on gfx950 (1,024 threads = 16 wave64, one unit each).  The kernel is
// a chain of dependent steps on one workgroup, and a dependent read of data
// another XCD's L2 wrote costs about 1.5 us, so the kernel is built around
// its few unavoidable round trips: every global read is issued as soon as
// its address is known, the LDS work runs while reads are in flight, and no
// global store is issued before the last read has been consumed (on this
// chip the vector memory counter also counts stores, so waiting for a read
// issued before a store waits for the store too).  Three rounds of reads:
//  1. the unit's counters and the score scan's segment counts;
//  2. the entries (keys above or inside the predicted cut window, with their
//     positions; one segment per scan workgroup, each in ascending position
//     order): a block scan of the counts places the segments, and each thread
//     loads a run of up to 8 consecutive entries into registers, so thread
//     order is position order — and, when the LRU queue may have to supply
//     victims, its first 4,096 entries from the head;
//  3. the slot-map entry of every entry's position, and the last use and
//     position held of every prefetched queue entry.
// Then, in LDS only: the radix cut over the window entries (the top 22 key
// bits in one histogram pass, window bin x next 10-bit digit; the entries
// sharing the cut's 22-bit prefix — usually a handful — rank themselves
// against each other, which also cuts exact ties by position, lower winning);
// one pass over the registers for winners, hits and misses, ranked together
// by one block scan; LRU victims without any search — never-used slots first
// (slots [fill, C), lowest first), then the first live (last use equal to the
// entry's stamp), unpinned entries of the queue of (slot, step) entries in
// ascending (step, slot) order, ranked by one block scan; and each slot the
// step used gets its place at the queue's tail in slot order from a block
// scan of per-word popcounts of the touched bitmap.  Finally every store:
// the selection, the hits' last-use stamps, the queue's new entries, the
// (miss, victim) pairs applied to pos2slot / slot2pos / last_use (an evicted
// position is never one of this step's misses), the gather's miss list and
// the trace.  The queue is compacted into its second buffer once every C / K
// steps or so.  Inconsistent state (corrupted counters or maps) is reported
// through the context's error words; every index stays in range.
#include "hc_block.h"

namespace hc {

constexpr int kRun = 8;                               // entries per thread and round
constexpr int kRoundEntries = kSelThreads * kRun;     // 8,192 entries per round
constexpr int kQWin = 4;                              // queue entries per thread, prefetched
constexpr int kSegPer = kMaxSegs / kSelThreads;       // segment counts per thread
constexpr int kRankMax = 256;                         // entries of the cut's 22-bit prefix ranked pairwise

struct SelShared {
  uint32_t hist[kBins1];                 // radix histograms; later the victims' evicted positions
  int32_t segoff[kMaxSegs];              // first entry of each segment
  uint32_t touched[HC_MAX_SLOTS / 32];   // slots the step's hits use (pinned)
  int32_t selpos[HC_MAX_TOPK];           // winners' positions, ascending
  int32_t selslot[HC_MAX_TOPK];          // their sources: slot, C + ring entry, -1 for a miss
  int32_t mpos[HC_MAX_TOPK];             // missing positions, ascending
  int32_t midx[HC_MAX_TOPK];             // winner index of miss k
  int32_t vic[HC_MAX_TOPK];              // victim slot of miss k
  uint2 near[kRankMax];                  // (key, position) of the entries sharing the cut's prefix
  int32_t wtot[kWaves];
  int32_t wtot2[kWaves];
  int32_t wdig[kWaves];                  // find_digit's wave totals
  int32_t bcast[8];
};

// Digit d (of nb bins, nb a multiple of 1,024 up to 4,096) such that the count
// in bins above d is < r and the count in bins >= d is >= r; `beyond` = count
// in bins above d.  If `from_top` is false the roles flip: bins below d,
// ascending.  Two barriers; its wave totals and answer have LDS words of their
// own, whose next writes are at least one barrier after every read.
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nb, int r, bool from_top, SelShared& sh,
                           int& digit, int& beyond) {
  const int per = nb / kSelThreads;
  const int lane = lane_id(), w = threadIdx.x >> 6;
  int sum = 0;
  for (int i = 0; i < per; ++i) {
    const int b = from_top ? nb - 1 - (per * threadIdx.x + i) : per * threadIdx.x + i;
    sum += (int)hist[b];
  }
  const int x = wave_incl_scan(sum);
  if (lane == 63) sh.wdig[w] = x;
  __syncthreads();
  int off = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) off += i < w ? sh.wdig[i] : 0;
  const int incl = x + off, excl = incl - sum;
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
}

__device__ __forceinline__ void clear_hist(SelShared& sh, int nb) {
  for (int b = threadIdx.x; b < nb; b += kSelThreads) sh.hist[b] = 0;
  __syncthreads();
}

// Inclusive prefix of v0 over the block (thread order) and the block totals of
// v0 and v1, with one pair of barriers.
__device__ __forceinline__ int block_scan_sum(int v0, int v1, SelShared& sh, int& tot0,
                                              int& tot1) {
  const int lane = lane_id(), w = threadIdx.x >> 6;
  const int x0 = wave_incl_scan(v0), x1 = wave_incl_scan(v1);
  if (lane == 63) {
    sh.wtot[w] = x0;
    sh.wtot2[w] = x1;
  }
  __syncthreads();
  int off = 0, t0 = 0, t1 = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    off += i < w ? sh.wtot[i] : 0;
    t0 += sh.wtot[i];
    t1 += sh.wtot2[i];
  }
  __syncthreads();
  tot0 = t0;
  tot1 = t1;
  return x0 + off;
}

// The K-th key left the predicted window: rebuild the unit's entries from its
// scores.  A 12-bit histogram of all H keys gives the cut bin bt; every key in
// a bin >= bt becomes an entry, in position order, at gcand[0 ..).  Returns
// the entry count; n_above = keys in bins above bt.
__device__ int rescan(const float* src, int64_t H, int K, Ent* gcand, SelShared& sh,
                      int& n_above, uint32_t& bt) {
  const int tid = threadIdx.x;
  clear_hist(sh, kBins1);
  for (int64_t i = tid; i < H; i += kSelThreads)
    atomicAdd(&sh.hist[order_key(src[i]) >> (32 - kBin1Bits)], 1u);
  __syncthreads();
  int b, gt;
  find_digit(sh.hist, kBins1, K, true, sh, b, gt);
  bt = (uint32_t)b;
  n_above = gt;
  int run = 0;
  for (int64_t base = 0; base < H; base += 4 * kSelThreads) {
    uint32_t key[4];
    int c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t p = base + 4 * tid + k;
      key[k] = p < H ? order_key(src[p]) : 0u;
      c += p < H && (key[k] >> (32 - kBin1Bits)) >= bt;
    }
    int total;
    int o = run + block_incl_scan(c, sh.wtot, total) - c;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t p = base + 4 * tid + k;
      if (p < H && (key[k] >> (32 - kBin1Bits)) >= bt) gcand[o++] = Ent{key[k], (uint32_t)p, -1};
    }
    run += total;
  }
  __syncthreads();   // the entries are read back by other threads
  return run;
}

// kTopkOnly (multi-query rounds): workgroup u is selection unit (s, g, q) and
// stops after writing its selection; k_round then runs steps 3-5 on the union
// of the group's selections.  Otherwise (one query) u is the unit (s, g).
template <bool kTopkOnly>
__global__ __launch_bounds__(kSelThreads) void k_select(DevState d, StepArgs a,
                                                        const float* __restrict__ scores,
                                                        uint64_t stride, int64_t seg_len,
                                                        int32_t* __restrict__ d_sel,
                                                        int32_t* __restrict__ d_trace) {
  __shared__ SelShared sh;
  constexpr bool kCache = !kTopkOnly;
  const int u = blockIdx.x, tid = threadIdx.x;
  const int session = u / (d.G * d.Q);
  const int K = d.K, C = d.C;
  const int32_t t = a.t;
  const int64_t H = a.hist_len[session];
  const uint32_t ring_lo = a.ring_lo[session];
  int32_t* cnt = d.cnt + (size_t)u * kCntStride;
  Ent* gcand = d.cand + (size_t)u * d.hcap;
  int32_t* pos2slot = d.pos2slot + (size_t)u * d.hcap;
  int32_t* slot2pos = d.slot2pos + (size_t)u * C;
  int32_t* last_use = d.last_use + (size_t)u * C;
  const bool lru = kCache && d.policy == HC_REPLACE_LRU;
  const int nwords = (C + 31) >> 5;

  // ==== reads, round 1: counters and segment counts =========================
  const int win_lo = cnt[kCntWinLo], win_hi = cnt[kCntWinHi];
  int qh = 0, qe = 0, qb = 0, fill = 0;
  if (kCache) {
    qh = cnt[kCntQHead];
    qe = cnt[kCntQTail];
    qb = cnt[kCntQBuf] & 1;
    fill = cnt[kCntFill];
  }
  const int nseg = (int)((H + seg_len - 1) / seg_len);   // <= max_segs, checked on the host
  int2 segc[kSegPer];
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int s = tid * kSegPer + k;
    segc[k] = s < nseg ? d.seg[(size_t)u * d.max_segs + s] : make_int2(0, 0);
  }
  for (int b = tid; b < kBins1; b += kSelThreads) sh.hist[b] = 0;
  if (kCache)
    for (int w = tid; w < nwords; w += kSelThreads) sh.touched[w] = 0;
  if (tid == 0) sh.bcast[7] = 0;   // evictions, counted at the stores
  fill = min(max(fill, 0), C);
  qe = min(max(qe, 0), d.qcap);
  qh = min(max(qh, 0), qe);
  // the queue supplies victims only once fewer than K never-used slots remain
  const bool q_pf = lru && fill + K > C && qe > qh;
  const int2* qbuf = d.oq + ((size_t)u * 2 + qb) * d.qcap;
  const int qj0 = (qh & ~(kQWin - 1)) + tid * kQWin;

  int sc[kSegPer];
  int se = 0, sa = 0;
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int s = tid * kSegPer + k;
    const int64_t room = H - (int64_t)s * seg_len < seg_len ? H - (int64_t)s * seg_len : seg_len;
    const int n = s < nseg ? (int)min((int64_t)max(segc[k].x, 0), room) : 0;
    sc[k] = n;
    se += n;
    sa += min(max(segc[k].y, 0), n);
  }
  int E, n_above;
  int o = block_scan_sum(se, sa, sh, E, n_above) - se;
#pragma unroll
  for (int k = 0; k < kSegPer; ++k) {
    const int s = tid * kSegPer + k;
    if (s < nseg) sh.segoff[s] = o;
    o += sc[k];
  }
  uint32_t b_lo, b_hi;   // the scan's cut window, top-16-bit key units
  cut_window(win_lo, win_hi, b_lo, b_hi);
  // Fast path: the K-th key lies inside the predicted window and at most
  // 8,192 entries lie above or inside it, so every entry fits in registers,
  // up to 8 per thread.  Otherwise the slow path makes every pass over the
  // entries in global memory: over the scan's segments if the window holds
  // the K-th key (ties, flat scores), else over a list rebuilt from the
  // scores (the cut jumped).
  const bool window_ok = n_above < K && E >= K;
  const bool fast = window_ok && E <= kRoundEntries;

  // ==== reads, round 2: the LRU queue's first window, the entries ===========
  int2 qent[kQWin];
  {
    int4 w0 = make_int4(-1, -1, -1, -1), w1 = w0;   // qcap % 4 == 0: both in bounds
    if (q_pf && qj0 < qe) w0 = *reinterpret_cast<const int4*>(qbuf + qj0);
    if (q_pf && qj0 + 2 < qe) w1 = *reinterpret_cast<const int4*>(qbuf + qj0 + 2);
    qent[0] = make_int2(w0.x, w0.y);
    qent[1] = make_int2(w0.z, w0.w);
    qent[2] = make_int2(w1.x, w1.y);
    qent[3] = make_int2(w1.z, w1.w);
  }
  // every thread reads segment offsets other threads wrote above (the fast
  // path's run placement, the slow path's entry lookup); the queue reads
  // issued just before stay in flight across the barrier
  __syncthreads();
  // this thread's run of R consecutive entries: thread order is position order
  uint32_t key[kRun];
  int32_t pos[kRun];
  int32_t slot[kRun];   // slot of each entry's position (the scan's lookup), -1: miss or ring
  int nv = 0;
  if (fast) {
    const int R = (E + kSelThreads - 1) / kSelThreads;
    const int j0 = tid * R;
    nv = max(0, min(R, E - j0));
    int lo = 0, hi = nseg;   // the last segment starting at or before j0
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sh.segoff[mid] <= j0) lo = mid;
      else hi = mid;
    }
    int sg = lo;
    int start = sh.segoff[sg];
    int next = sg + 1 < nseg ? sh.segoff[sg + 1] : 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      key[k] = 0u;
      pos[k] = -1;
      slot[k] = -1;
      if (k >= nv) continue;
      const int j = j0 + k;
      while (j >= next) {   // the run crosses into a later segment
        ++sg;
        start = next;
        next = sg + 1 < nseg ? sh.segoff[sg + 1] : 0x7FFFFFFF;
      }
      const Ent e = gcand[(int64_t)sg * seg_len + (j - start)];
      key[k] = e.key;
      pos[k] = (int32_t)e.pos;
      if (kCache) slot[k] = e.slot;
    }
  }

  // ==== reads, round 3: the prefetched queue entries' state ==================
  int qlu[kQWin], qsp[kQWin];
#pragma unroll
  for (int k = 0; k < kQWin; ++k) {
    const int j = qj0 + k;
    const bool ok = q_pf && j >= qh && j < qe && qent[k].x >= 0 && qent[k].x < C;
    qlu[k] = ok ? last_use[qent[k].x] : (int)0x80000000;
    qsp[k] = ok ? slot2pos[qent[k].x] : -1;
  }

  // ==== the cut key T and position cut (LDS) =================================
  // `each` visits every entry once as (key, position): from registers on the
  // fast path, from global memory on the slow path (entry j of the segments
  // found by a binary search over their first entries).
  int nrows = E;   // entries of the slow path
  int nsegs = nseg;
  if (!window_ok) {
    uint32_t bt;
    nrows = rescan(scores + (uint64_t)u * stride, H, K, gcand, sh, n_above, bt);
    b_lo = bt << 4;   // the rebuilt list's window: the 12-bit cut bin
    b_hi = (bt << 4) | 15;
    nsegs = 1;
    if (tid == 0) sh.segoff[0] = 0;
    for (int b = tid; b < kBins1; b += kSelThreads) sh.hist[b] = 0;
    __syncthreads();
  }
  auto entry = [&](int j) {   // slow path: entry j
    int lo = 0, hi = nsegs;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (sh.segoff[mid] <= j) lo = mid;
      else hi = mid;
    }
    return gcand[(int64_t)lo * seg_len + (j - sh.segoff[lo])];
  };
  auto each = [&](auto&& f) {
    if (fast) {
#pragma unroll
      for (int k = 0; k < kRun; ++k)
        if (k < nv) f(key[k], pos[k]);
    } else {
      for (int j = tid; j < nrows; j += kSelThreads) {
        const Ent e = entry(j);
        f(e.key, (int32_t)e.pos);
      }
    }
  };
  int r = K - n_above;   // winners still to take from the window, >= 1
  uint32_t lo16 = b_lo, hi16 = b_hi;
  int beyond;
  if (hi16 - lo16 + 1 > 64) {
    // a wide window (a unit's first step without a cut histogram): narrow it
    // to the 12-bit bin holding the K-th key first
    const uint32_t lo12 = lo16 >> 4;
    each([&](uint32_t kk, int32_t) {
      const uint32_t k16 = kk >> 16;
      if (k16 >= lo16 && k16 <= hi16) atomicAdd(&sh.hist[(kk >> 20) - lo12], 1u);
    });
    __syncthreads();
    int rel;
    find_digit(sh.hist, kBins1, r, true, sh, rel, beyond);
    r -= beyond;
    const uint32_t b12 = lo12 + (uint32_t)rel;
    lo16 = max(lo16, b12 << 4);
    hi16 = min(hi16, (b12 << 4) | 15u);
    clear_hist(sh, kBins1);
  }
  // the top 22 bits: window prefix x the next 6 bits in one histogram of at
  // most 64 x 64 bins
  const uint32_t w_lo22 = lo16 << 6, w_hi22 = (hi16 + 1) << 6;
  each([&](uint32_t kk, int32_t) {
    const uint32_t p22 = kk >> 10;
    if (p22 >= w_lo22 && p22 < w_hi22) atomicAdd(&sh.hist[p22 - w_lo22], 1u);
  });
  if (tid == 0) sh.bcast[2] = 0;   // entries of the cut prefix listed so far
  __syncthreads();
  int idx22;
  find_digit(sh.hist, kBins1, r, true, sh, idx22, beyond);
  r -= beyond;   // winners to take among the entries of the prefix, >= 1
  const uint32_t pre22 = w_lo22 + (uint32_t)idx22;
  const int n22 = (int)sh.hist[idx22];
  uint32_t T;
  int32_t pcut = 0x7FFFFFFF;   // take ties at T with position <= pcut
  if (n22 <= kRankMax) {
    // the prefix's entries (usually a handful) rank themselves by (key
    // descending, position ascending): the r-th is the last winner, whose key
    // and position are the cuts
    each([&](uint32_t kk, int32_t p) {
      if ((kk >> 10) == pre22) {
        const int i = atomicAdd(&sh.bcast[2], 1);
        if (i < kRankMax) sh.near[i] = make_uint2(kk, (uint32_t)p);
      }
    });
    __syncthreads();
    const int n = min(sh.bcast[2], kRankMax);
    for (int i = tid; i < n; i += kSelThreads) {
      const uint2 me = sh.near[i];
      int better = 0;
      for (int j = 0; j < n; ++j) {
        const uint2 o2 = sh.near[j];
        better += o2.x > me.x || (o2.x == me.x && o2.y < me.y);
      }
      if (better == r - 1) {
        sh.bcast[3] = (int)me.x;
        sh.bcast[4] = (int)me.y;
      }
    }
    __syncthreads();
    T = (uint32_t)sh.bcast[3];
    pcut = sh.bcast[4];
  } else {
    // many entries share the prefix (ties, flat scores): the last 10 key bits
    // by histogram, then, if the cut falls inside a run of equal keys, the
    // r-th smallest position among them (digits of 11, 10, 10 bits)
    clear_hist(sh, 1024);
    each([&](uint32_t kk, int32_t) {
      if ((kk >> 10) == pre22) atomicAdd(&sh.hist[kk & 1023], 1u);
    });
    __syncthreads();
    int d3;
    find_digit(sh.hist, 1024, r, true, sh, d3, beyond);
    r -= beyond;
    const int n_eq = (int)sh.hist[d3];
    T = (pre22 << 10) | (uint32_t)d3;
    if (r < n_eq) {
      int e1, e2, e3, below;
      __syncthreads();
      clear_hist(sh, 2048);
      each([&](uint32_t kk, int32_t p) {
        if (kk == T) atomicAdd(&sh.hist[(uint32_t)p >> 20], 1u);
      });
      __syncthreads();
      find_digit(sh.hist, 2048, r, false, sh, e1, below);
      r -= below;
      __syncthreads();
      clear_hist(sh, 1024);
      each([&](uint32_t kk, int32_t p) {
        if (kk == T && (int)((uint32_t)p >> 20) == e1)
          atomicAdd(&sh.hist[((uint32_t)p >> 10) & 1023], 1u);
      });
      __syncthreads();
      find_digit(sh.hist, 1024, r, false, sh, e2, below);
      r -= below;
      __syncthreads();
      clear_hist(sh, 1024);
      const uint32_t hi = ((uint32_t)e1 << 10) | (uint32_t)e2;
      each([&](uint32_t kk, int32_t p) {
        if (kk == T && ((uint32_t)p >> 10) == hi) atomicAdd(&sh.hist[(uint32_t)p & 1023], 1u);
      });
      __syncthreads();
      find_digit(sh.hist, 1024, r, false, sh, e3, below);
      pcut = (int32_t)((hi << 10) | (uint32_t)e3);
    }
  }

  // the next step's window: this cut's 16-bit prefix +- kWinHalf
  const int nlo = max((int)(T >> 16) - kWinHalf, 0), nhi = min((int)(T >> 16) + kWinHalf, 65535);

  // ==== winners in position order, hits, misses (LDS) ========================
  // one block scan ranks winners and misses (two 16-bit fields of one value)
  // and counts ring rows and corrupt slot-map entries (second value)
  int nwin = 0, m = 0, n_ring = 0, n_bad = 0;
  // Records winner wr (miss rank mr) with its source.
  auto record = [&](int wr, int mr, int32_t p, int32_t sl, bool ring, bool miss) {
    if (wr >= K) return;
    sh.selpos[wr] = p;
    if (!kCache) return;
    sh.selslot[wr] = ring ? C + (int32_t)((uint32_t)p % (uint32_t)d.ring_rows) : (miss ? -1 : sl);
    if (miss && mr < K) {
      sh.mpos[mr] = p;
      sh.midx[mr] = wr;
    }
    if (!ring && !miss) atomicOr(&sh.touched[sl >> 5], 1u << (sl & 31));
  };
  if (fast) {
    int cw = 0, cm = 0, cr = 0, cb = 0;
    uint32_t fw = 0, fm = 0, fr = 0;   // bit k: entry k wins / misses / is a ring row
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      const bool win = k < nv && (key[k] > T || (key[k] == T && pos[k] <= pcut));
      const bool ring = kCache && win && (uint32_t)pos[k] >= ring_lo;
      const bool corrupt = kCache && win && !ring && slot[k] >= C;   // a corrupt slot map entry
      const bool miss = kCache && win && !ring && (slot[k] < 0 || corrupt);
      fw |= (uint32_t)win << k;
      fm |= (uint32_t)miss << k;
      fr |= (uint32_t)ring << k;
      cw += win;
      cm += miss;
      cr += ring;
      cb += corrupt;
    }
    // winners <= 8,192, misses and ring rows <= K, corrupt entries <= 8,192:
    // 16-bit fields, no carry
    int tot, tot1;
    const int packed = cw | (cm << 16);
    const int ex = block_scan_sum(packed, cr | (cb << 16), sh, tot, tot1) - packed;
    int wr = ex & 0xFFFF, mr = ex >> 16;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      if (!((fw >> k) & 1u)) continue;
      const bool ring = (fr >> k) & 1u, miss = (fm >> k) & 1u;
      record(wr, mr, pos[k], slot[k], ring, miss);
      mr += miss;
      ++wr;
    }
    nwin = tot & 0xFFFF;
    m = tot >> 16;
    n_ring = tot1 & 0xFFFF;
    n_bad = tot1 >> 16;
  } else {
    // the rebuilt list in position order, 1,024 entries at a time; slots
    // looked up here
    for (int j0 = 0; j0 < nrows; j0 += kSelThreads) {
      const int j = j0 + tid;
      Ent e{0u, 0u, -1};
      if (j < nrows) e = entry(j);
      const int32_t p = (int32_t)e.pos;
      const bool win = j < nrows && (e.key > T || (e.key == T && p <= pcut));
      const bool ring = kCache && win && (uint32_t)p >= ring_lo;
      int32_t sl = -1;
      if (kCache && win && !ring && p >= 0 && p < H) sl = pos2slot[p];
      const bool corrupt = kCache && win && !ring && sl >= C;
      const bool miss = kCache && win && !ring && (sl < 0 || corrupt);
      int tot, tot1;
      const int packed = (int)win | ((int)miss << 16);
      const int ex = block_scan_sum(packed, (int)ring | ((int)corrupt << 16), sh, tot, tot1) - packed;
      if (win) record(nwin + (ex & 0xFFFF), m + (ex >> 16), p, sl, ring, miss);
      nwin += tot & 0xFFFF;
      m += tot >> 16;
      n_ring += tot1 & 0xFFFF;
      n_bad += tot1 >> 16;
    }
  }
#ifdef HC_TEST_HOOKS
  if (d.test_force) n_bad = 1;
#endif
  if (n_bad || nwin != K || m > K) {
    // inconsistent scan state or slot map: report it and touch nothing more;
    // the selection stays in range (the gather reads slot 0)
    if (tid == 0) report_error(d, kErrSelect);
    for (int i = tid; i < K; i += kSelThreads) {
      d_sel[(size_t)u * K + i] = -1;
      if (kCache) d.sel_slot[(size_t)u * K + i] = 0;
    }
    if (tid == 0) {
      if (kCache) cnt[kCntMiss] = 0;
      cnt[kCntWinLo] = cnt[kCntWinHi] = -1;   // the next step considers every key
    }
    return;
  }
  __syncthreads();   // the recorded winners are read by other threads below
  if (kTopkOnly) {
    for (int i = tid; i < K; i += kSelThreads) d_sel[(size_t)u * K + i] = sh.selpos[i];
    if (tid == 0) {
      cnt[kCntWinLo] = nlo;
      cnt[kCntWinHi] = nhi;
    }
    return;
  }

  // ==== victims (LDS; further queue reads only when the window falls short) ==
  int32_t* vold = reinterpret_cast<int32_t*>(sh.hist);   // position each victim held
  int32_t* vic = sh.vic;
  int n_new = 0;
  if (lru) {
    // never-used slots first, then the first live, unpinned queue entries
    n_new = min(m, C - fill);
    for (int k = tid; k < n_new; k += kSelThreads) {
      vic[k] = fill + k;
      vold[k] = -1;
    }
    const int need = m - n_new;
    if (tid == 0) sh.bcast[6] = qh - 1;   // queue index of the last victim
    if (need > 0) {
      // the prefetched window: entries [qh & ~3, + 4,096)
      auto pinned = [&](int v) { return (sh.touched[v >> 5] >> (v & 31)) & 1u; };
      bool f[kQWin];
      int c = 0;
#pragma unroll
      for (int k = 0; k < kQWin; ++k) {
        const int j = qj0 + k;
        f[k] = q_pf && j >= qh && j < qe && qent[k].x >= 0 && qent[k].x < C &&
               !pinned(qent[k].x) && qlu[k] == qent[k].y;
        c += f[k];
      }
      int total, dummy;
      int k0 = block_scan_sum(c, 0, sh, total, dummy) - c;
#pragma unroll
      for (int k = 0; k < kQWin; ++k) {
        if (!f[k]) continue;
        if (k0 < need) {
          vic[n_new + k0] = qent[k].x;
          vold[n_new + k0] = qsp[k];
          if (k0 == need - 1) sh.bcast[6] = qj0 + k;
        }
        ++k0;
      }
      int found = total;
      // further windows (rare: the 4,096 entries from the head hold fewer live
      // ones than the step needs)
      for (int jw = (qh & ~(kQWin - 1)) + kSelThreads * kQWin; found < need && jw < qe;
           jw += kSelThreads * kQWin) {
        const int jb = jw + tid * kQWin;
        int2 ent[kQWin];
        {
          int4 w0 = make_int4(-1, -1, -1, -1), w1 = w0;
          if (jb < qe) w0 = *reinterpret_cast<const int4*>(qbuf + jb);
          if (jb + 2 < qe) w1 = *reinterpret_cast<const int4*>(qbuf + jb + 2);
          ent[0] = make_int2(w0.x, w0.y);
          ent[1] = make_int2(w0.z, w0.w);
          ent[2] = make_int2(w1.x, w1.y);
          ent[3] = make_int2(w1.z, w1.w);
        }
        bool g[kQWin];
        int lu[kQWin], sp[kQWin];
#pragma unroll
        for (int k = 0; k < kQWin; ++k) {
          g[k] = jb + k < qe && ent[k].x >= 0 && ent[k].x < C && !pinned(ent[k].x);
          lu[k] = g[k] ? last_use[ent[k].x] : 0;
          sp[k] = g[k] ? slot2pos[ent[k].x] : -1;
        }
        int cc = 0;
#pragma unroll
        for (int k = 0; k < kQWin; ++k) {
          g[k] = g[k] && lu[k] == ent[k].y;
          cc += g[k];
        }
        int tot2;
        int q0 = found + block_scan_sum(cc, 0, sh, tot2, dummy) - cc;
#pragma unroll
        for (int k = 0; k < kQWin; ++k) {
          if (!g[k]) continue;
          if (q0 < need) {
            vic[n_new + q0] = ent[k].x;
            vold[n_new + q0] = sp[k];
            if (q0 == need - 1) sh.bcast[6] = jb + k;
          }
          ++q0;
        }
        found += tot2;
      }
      if (found < need) {
        // a corrupted queue: report it; keep every index in range
        if (tid == 0) report_error(d, kErrLru);
        for (int k = n_new + found + tid; k < m; k += kSelThreads) {
          vic[k] = 0;
          vold[k] = -1;
        }
      }
    }
  } else {
    hand_victims(d, u, m, d.policy == HC_REPLACE_CLOCK, sh.touched, vic, sh.wtot, &sh.bcast[6]);
    for (int k = tid; k < m; k += kSelThreads) vold[k] = slot2pos[vic[k]];
  }
  __syncthreads();

  // ==== stores ================================================================
  // The selection, each selected row's source for the gather (a miss row is
  // marked -(slot + 1): the gather reads it from host RAM and writes it into
  // that slot itself), the dense miss list with each victim's previous
  // position, and the trace.  The gather's bookkeeping workgroup of the unit
  // stamps the step's slots, applies the (miss, victim) pairs to the slot maps
  // and appends the step's slots to the LRU queue.
  int32_t* tr = d_trace ? d_trace + (size_t)u * HC_TRACE_INTS(K) : nullptr;
  int32_t* g_miss = d.miss_pos + (size_t)u * K;
  int32_t* g_vic = d.victim + (size_t)u * K;
  int32_t* g_midx = d.miss_idx + (size_t)u * K;
  int32_t* g_old = d.miss_old + (size_t)u * K;
  int n_evict = 0;
  for (int k = tid; k < m; k += kSelThreads) {
    const int32_t v = vic[k], p = sh.mpos[k];
    int32_t old = vold[k];
    if (old < 0 || old >= d.hcap) old = -1;
    n_evict += old >= 0;
    sh.selslot[sh.midx[k]] = -(v + 1);
    g_miss[k] = p;
    g_vic[k] = v;
    g_midx[k] = sh.midx[k];
    g_old[k] = old;
    if (tr) {
      tr[HC_TRACE_HEADER + K + k] = p;
      tr[HC_TRACE_HEADER + 2 * K + k] = v;
      tr[HC_TRACE_HEADER + 3 * K + k] = old;
    }
  }
  if (n_evict) atomicAdd(&sh.bcast[7], n_evict);
  __syncthreads();
  int32_t* g_slot = d.sel_slot + (size_t)u * K;
  for (int i = tid; i < K; i += kSelThreads) {
    d_sel[(size_t)u * K + i] = sh.selpos[i];
    const int32_t enc = sh.selslot[i];
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
  if (tid == 0) {
    if (tr) {
      tr[0] = K - m - n_ring;
      tr[1] = m;
      tr[2] = sh.bcast[7];
      tr[3] = n_ring;
    }
    if (lru) {
      cnt[kCntQHead] = sh.bcast[6] + 1;   // past the last victim; the gather appends at the tail
      cnt[kCntFill] = fill + n_new;
    }
    cnt[kCntMiss] = m;
    cnt[kCntWinLo] = nlo;   // the next step's cut window
    cnt[kCntWinHi] = nhi;
  }
}

hipError_t launch_select(const DevState& d, const StepArgs& a, const float* scores,
                         uint64_t stride, int64_t max_len, int32_t* d_sel, int32_t* d_trace,
                         hipStream_t st, StageEv ev) {
  const int64_t seg_len = scan_seg_len(max_len, d.max_segs);
  if (d.Q == 1)
    hipExtLaunchKernelGGL(k_select<false>, dim3(d.S * d.G), dim3(kSelThreads), 0, st, ev.start,
                          ev.stop, 0, d, a, scores, stride, seg_len, d_sel, d_trace);
  else
    hipExtLaunchKernelGGL(k_select<true>, dim3(d.S * d.G * d.Q), dim3(kSelThreads), 0, st,
                          ev.start, ev.stop, 0, d, a, scores, stride, seg_len, d_sel, d_trace);
  return hipGetLastError();
}

}  // namespace hc
