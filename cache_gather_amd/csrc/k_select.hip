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
// its address is known, without a branch between the loads of one round (a
// load behind a branch was issued only after the previous one returned), the
// LDS work runs while reads are in flight, and no global store is issued
// before the last read has been consumed (on this chip the vector memory
// counter also counts stores, so waiting for a read issued before a store
// waits for the store too).  Reads:
//  1. one round trip for the unit's counter line, each thread's segment count
//     and its 8 entry slots: the score scan wrote one segment of entries per
//     scan workgroup (keys above or inside the predicted cut window, their
//     positions and the slots holding them, in ascending position order),
//     and segment s belongs to 1,024 / nseg consecutive threads, so thread
//     order is position order (a segment with more entries than its threads
//     hold takes a second round for every segment count, and the entries
//     from global memory);
//  2. when the LRU queue may have to supply victims, its first 4,096 entries
//     from the head, and 3. the last use and position held of each.
// Then, in LDS only: the radix cut over the window entries (the top 22 key
// bits in one histogram, window bin x next 6 bits, built before the block
// totals are known; the entries sharing the cut's 22-bit prefix — usually a
// handful — rank themselves against each other, which also cuts exact ties
// by position, lower winning); one pass over the registers for winners, hits
// and misses, ranked together by one block scan; LRU victims without any
// search — never-used slots first (slots [fill, C), lowest first), then the
// first live (last use equal to the entry's stamp), unpinned entries of the
// queue of (slot, step) entries in ascending (step, slot) order, ranked by
// one block scan.  Finally every store: the selection, each selected row's
// source for the gather, the miss list with each victim's previous position,
// the trace and the counters.  The last-use stamps, the slot-map updates and
// the queue's new entries are left to the unit's bookkeeping workgroup in
// the gather launch.  Inconsistent state (corrupted counters or maps) is
// reported through the context's error words; every index stays in range.
#include "hc_block.h"

namespace hc {

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
// kRun: entries a thread holds in registers (4 for top-K up to 3,072, else
// 8): the per-entry code is unrolled, and on this kernel every instruction is
// fetched cold, so the smaller variant runs measurably faster.
// Workgroup c of kCountWGs marking unit u's LRU queue for a compaction (one
// query row), beside the select workgroups, when the step's slots might not
// fit after the tail: bit j of the unit's bitmap is set when entry j of
// [0, tail) is live (its slot's last use is the entry's step — every earlier
// step's stamps are in place, and this step's are the gather's).  The range
// starts at 0 rather than at the head, which the select workgroups move
// meanwhile: entries before any head value are dead or this step's victims,
// which the compaction drops as used by this step.  Workgroup 0 records the
// tail, the buffer and the step.  The queue itself is only read.
__device__ void queue_count(const DevState& d, int u, int c, int32_t t) {
  int32_t* cnt = d.cnt + (size_t)u * kCntStride;
  const int QC = d.qcap, C = d.C, tid = threadIdx.x;
  const int qe = min(max(cnt[kCntQTail], 0), QC);
  if (qe + d.K <= QC) return;   // the step's slots surely fit: nothing to prepare
  const int qb = cnt[kCntQBuf] & 1;
  const int len = ((qe + kCountWGs - 1) / kCountWGs + 63) / 64 * 64;
  const int lo = min(qe, c * len), hi = min(qe, lo + len);
  const int2* q = d.oq + ((size_t)u * 2 + qb) * QC;
  const int32_t* last_use = d.last_use + (size_t)u * C;
  uint32_t* bits = d.qlive + (size_t)u * d.qlive_words;
  const int lane = lane_id(), wv = tid >> 6;
  constexpr int kPer = 8;
  for (int j0 = lo; j0 < hi; j0 += kSelThreads * kPer) {
    int2 e[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = j0 + k * kSelThreads + wv * 64 + lane;
      e[k] = j < hi ? q[j] : make_int2(-1, -1);
    }
    int lu[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) lu[k] = e[k].x >= 0 && e[k].x < C ? last_use[e[k].x] : -1;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      // 64 consecutive entries per wave, starting at a multiple of 64
      const int jb = j0 + k * kSelThreads + wv * 64;
      const uint64_t live = __ballot(e[k].x >= 0 && e[k].x < C && e[k].y >= 0 && lu[k] == e[k].y);
      if (lane == 0 && jb < hi) {
        bits[jb >> 5] = (uint32_t)live;
        bits[(jb >> 5) + 1] = (uint32_t)(live >> 32);
      }
    }
  }
  if (c == 0 && tid == 0) {
    cnt[kCntCntTail] = qe;
    cnt[kCntCntBuf] = qb;
    cnt[kCntCntStep] = t;
  }
}

template <bool kTopkOnly, int kRun>
__global__ __launch_bounds__(kSelThreads) void k_select(DevState d, StepArgs a,
                                                        const float* __restrict__ scores,
                                                        uint64_t stride, int64_t seg_len,
                                                        int32_t* __restrict__ d_sel,
                                                        int32_t* __restrict__ d_trace) {
  __shared__ SelShared sh;
  constexpr bool kCache = !kTopkOnly;
  constexpr int kRoundEntries = kSelThreads * kRun;   // entries in registers at most
  // grid (G Q, S): the session is the grid row, so no division is needed;
  // grid layers z >= 1 (one query row, LRU): the queue-marking workgroups
  const int session = blockIdx.y;
  const int u = blockIdx.y * gridDim.x + blockIdx.x, tid = threadIdx.x;
  if (blockIdx.z > 0) {
    queue_count(d, u, (int)blockIdx.z - 1, a.t);
    return;
  }
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

  // ==== reads, round 1: counters, segment counts, entries ===================
  // With few segments (each gets at least 64 entry slots), segment s of the
  // scan's entries is held by spt = 1,024 / nseg consecutive threads, thread
  // c of them taking entry slots [kRun c, kRun (c + 1)) of it, so every
  // address is known at the start: the counter line, the thread's segment
  // count and its entry slots are read in one round trip, with clamped
  // in-range indices and no branch (slots past the segment's count are
  // ignored); thread order is position order.  With many segments, or when
  // a segment holds more entries than its threads, every segment count is
  // read and a second round gives each thread a run of consecutive entries.
  // lane i holds counter word i mod 16: a vector load (a scalar load of the
  // line would make the wait for the kernel's argument loads wait for it)
  static_assert(kCnt <= 16, "counters read from lanes 0-15");
  const int cword = cnt[tid & 15];
  // positions, segment lengths and entry indices are below 2^31: 32-bit math
  const uint32_t H32 = (uint32_t)H, len32 = (uint32_t)seg_len;
  const int nseg = (int)((H32 + len32 - 1) / len32);   // 1 .. max_segs, checked on the host
  const int spt = nseg <= kSelThreads ? kSelThreads / nseg : 0;
  const bool spec = spt * kRun >= 64;
  const int my_seg = spec ? min(tid / spt, nseg - 1) : 0;
  const bool has_seg = spec && tid < spt * nseg;
  const int c_lo = has_seg ? (tid - my_seg * spt) * kRun : 0;   // first entry slot of the thread
  const uint32_t s_base = (uint32_t)my_seg * len32;
  const uint32_t s_slots = min(len32, (uint32_t)d.hcap - s_base);   // >= 1: s_base < H <= hcap
  int2 segv = make_int2(0, 0);
  Ent ent[kRun];
  int2 segc[kSegPer];   // every segment count (kSegPer per thread), when read
  if (spec) {
    segv = d.seg[(size_t)u * d.max_segs + my_seg];
#pragma unroll
    for (int k = 0; k < kRun; ++k) ent[k] = gcand[s_base + min((uint32_t)(c_lo + k), s_slots - 1)];
  } else {
#pragma unroll
    for (int k = 0; k < kSegPer; ++k)
      segc[k] = d.seg[(size_t)u * d.max_segs + min(tid * kSegPer + k, nseg - 1)];
#pragma unroll
    for (int k = 0; k < kRun; ++k) ent[k] = Ent{0u, 0u, -1};
  }

  for (int b = tid; b < kBins1; b += kSelThreads) sh.hist[b] = 0;
  if (kCache)
    for (int w = tid; w < nwords; w += kSelThreads) sh.touched[w] = 0;
  if (tid == 0) {
    sh.bcast[2] = 0;   // entries of the cut prefix listed so far
    sh.bcast[5] = 0;   // a segment holds more entries than its threads
    sh.bcast[7] = 0;   // evictions, counted at the stores
  }
  __syncthreads();   // the round-1 reads stay in flight across it

  const int win_lo = __builtin_amdgcn_readlane(cword, kCntWinLo);
  const int win_hi = __builtin_amdgcn_readlane(cword, kCntWinHi);
  int qh = 0, qe = 0, qb = 0, fill = 0;
  if (kCache) {
    qh = __builtin_amdgcn_readlane(cword, kCntQHead);
    qe = __builtin_amdgcn_readlane(cword, kCntQTail);
    qb = __builtin_amdgcn_readlane(cword, kCntQBuf) & 1;
    fill = __builtin_amdgcn_readlane(cword, kCntFill);
  }
  fill = min(max(fill, 0), C);
  qe = min(max(qe, 0), d.qcap);
  qh = min(max(qh, 0), qe);
  // the queue supplies victims only once fewer than K never-used slots remain
  const bool q_pf = lru && fill + K > C && qe > qh;
  const int2* qbuf = d.oq + ((size_t)u * 2 + qb) * d.qcap;
  const int qj0 = (qh & ~(kQWin - 1)) + tid * kQWin;

  // ==== reads, round 2: the LRU queue's first window (when it may supply
  // victims); consumed after the cut ==========================================
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

  uint32_t b_lo, b_hi;   // the scan's cut window, top-16-bit key units
  cut_window(win_lo, win_hi, b_lo, b_hi);
  const int s_room = has_seg ? (int)min(len32, H32 - s_base) : 0;
  const int n_s = has_seg ? min(max(segv.x, 0), s_room) : 0;
  int nv = max(0, min(kRun, n_s - c_lo));   // this thread's entries
  uint32_t key[kRun];
  int32_t pos[kRun];
  int32_t slot[kRun];   // slot of each entry's position (the scan's lookup), -1: miss or ring
#pragma unroll
  for (int k = 0; k < kRun; ++k) {
    key[k] = ent[k].key;
    pos[k] = (int32_t)ent[k].pos;
    slot[k] = kCache ? ent[k].slot : -1;
  }
  // The fast path's first histogram, built before the totals are known: the
  // window's 22-bit prefixes (window prefix x the next 6 bits, at most 64 x 64
  // bins), or for a wide window (a unit's first step without a cut histogram)
  // its 12-bit bins, which narrow it first.
  const bool wide0 = b_hi - b_lo + 1 > 64;
  int E = 0, n_above = 0;
  bool layout_ok = false;
  if (spec) {
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      if (k >= nv) continue;
      const uint32_t kk = key[k];
      if (wide0) {
        const uint32_t k16 = kk >> 16;
        if (k16 >= b_lo && k16 <= b_hi) atomicAdd(&sh.hist[(kk >> 20) - (b_lo >> 4)], 1u);
      } else {
        const uint32_t p22 = kk >> 10;
        if (p22 >= (b_lo << 6) && p22 < ((b_hi + 1) << 6)) atomicAdd(&sh.hist[p22 - (b_lo << 6)], 1u);
      }
    }
    // block totals: entries and entries above the window (one lane per segment)
    const bool lead = has_seg && c_lo == 0;
    if (lead && n_s > spt * kRun) sh.bcast[5] = 1;
    const int ev = wave_incl_scan(lead ? n_s : 0);
    const int av = wave_incl_scan(lead ? min(max(segv.y, 0), n_s) : 0);
    if (lane_id() == 63) {
      sh.wtot[tid >> 6] = ev;
      sh.wtot2[tid >> 6] = av;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      E += sh.wtot[i];
      n_above += sh.wtot2[i];
    }
    layout_ok = sh.bcast[5] == 0;
  }
  if (!layout_ok) {
    // every segment count (a second read round after the speculative one),
    // their offsets and totals
    if (spec) {
#pragma unroll
      for (int k = 0; k < kSegPer; ++k)
        segc[k] = d.seg[(size_t)u * d.max_segs + min(tid * kSegPer + k, nseg - 1)];
    }
    int sc[kSegPer];
    int se = 0, sa = 0;
#pragma unroll
    for (int k = 0; k < kSegPer; ++k) {
      const int sg = tid * kSegPer + k;
      const int room = sg < nseg ? (int)min(len32, H32 - (uint32_t)sg * len32) : 0;
      const int n = min(max(segc[k].x, 0), room);
      sc[k] = n;
      se += n;
      sa += min(max(segc[k].y, 0), n);
    }
    if (spec) __syncthreads();   // the wave totals above are read before the scan rewrites them
    int o = block_scan_sum(se, sa, sh, E, n_above) - se;
#pragma unroll
    for (int k = 0; k < kSegPer; ++k) {
      const int sg = tid * kSegPer + k;
      if (sg < nseg) sh.segoff[sg] = o;
      o += sc[k];
    }
    __syncthreads();   // every thread reads the segment offsets
  }
  // Fast path: the K-th key lies inside the predicted window and the entries
  // are in registers — already, if every segment fit its threads' slots, or
  // else after a second round that gives each thread a run of consecutive
  // entries (at most kRoundEntries in all).  Otherwise the slow path makes
  // every pass over the entries in global memory: over the scan's segments
  // if the window holds the K-th key (ties, flat scores), else over a list
  // rebuilt from the scores (the cut jumped).
  const bool window_ok = n_above < K && E >= K;
  const bool hist0 = layout_ok && window_ok;   // the first histogram holds every entry
  bool fast = hist0;
  if (!layout_ok && window_ok && E <= kRoundEntries) {
    fast = true;
    const int R = (E + kSelThreads - 1) / kSelThreads;   // <= kRun
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
      if (k >= nv) continue;
      const int j = j0 + k;
      while (j >= next) {   // the run crosses into a later segment
        ++sg;
        start = next;
        next = sg + 1 < nseg ? sh.segoff[sg + 1] : 0x7FFFFFFF;
      }
      const Ent e = gcand[(uint32_t)sg * len32 + (uint32_t)(j - start)];
      key[k] = e.key;
      pos[k] = (int32_t)e.pos;
      if (kCache) slot[k] = e.slot;
    }
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
  } else if (!hist0) {
    clear_hist(sh, kBins1);   // the first histogram held the first slots of each segment only
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
    // a wide window: narrow it to the 12-bit bin holding the K-th key first
    const uint32_t lo12 = lo16 >> 4;
    if (!hist0) {
      each([&](uint32_t kk, int32_t) {
        const uint32_t k16 = kk >> 16;
        if (k16 >= lo16 && k16 <= hi16) atomicAdd(&sh.hist[(kk >> 20) - lo12], 1u);
      });
      __syncthreads();
    }
    int rel;
    find_digit(sh.hist, kBins1, r, true, sh, rel, beyond);
    r -= beyond;
    const uint32_t b12 = lo12 + (uint32_t)rel;
    lo16 = max(lo16, b12 << 4);
    hi16 = min(hi16, (b12 << 4) | 15u);
    clear_hist(sh, kBins1);
  }
  // the top 22 bits: window prefix x the next 6 bits in one histogram of at
  // most 64 x 64 bins (the fast path's, for a window that was not wide, is
  // already complete)
  const uint32_t w_lo22 = lo16 << 6, w_hi22 = (hi16 + 1) << 6;
  if (!hist0 || wide0) {
    each([&](uint32_t kk, int32_t) {
      const uint32_t p22 = kk >> 10;
      if (p22 >= w_lo22 && p22 < w_hi22) atomicAdd(&sh.hist[p22 - w_lo22], 1u);
    });
    __syncthreads();
  }
  // ==== reads, round 3: the prefetched queue entries' state (consumed by the
  // victims), issued once the queue window has arrived, so the reads overlap
  // the cut ==================================================================
  int qlu[kQWin], qsp[kQWin];
#pragma unroll
  for (int k = 0; k < kQWin; ++k) {
    qlu[k] = (int)0x80000000;
    qsp[k] = -1;
  }
  if (q_pf) {
#pragma unroll
    for (int k = 0; k < kQWin; ++k) {
      const int j = qj0 + k;
      if (j >= qh && j < qe && qent[k].x >= 0 && qent[k].x < C) {
        qlu[k] = last_use[qent[k].x];
        qsp[k] = slot2pos[qent[k].x];
      }
    }
  }

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
    // r-th smallest position among them (digits of 11, 10, 10 bits).  Every
    // thread has read n22 from the histogram before it is cleared.
    __syncthreads();
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
  // The ring holds positions [ring_lo, ring_lo + ring_rows), position p in
  // entry p mod ring_rows: entry ring_base + (p - ring_lo), wrapped once.
  const uint32_t rrows = d.ring_rows > 0 ? (uint32_t)d.ring_rows : 1u;
  const uint32_t ring_base = kCache && ring_lo != kNoRing ? ring_lo % rrows : 0u;
  auto ring_entry = [&](int32_t p) {
    uint32_t re = ring_base + ((uint32_t)p - ring_lo);
    re = re >= rrows ? re - rrows : re;
    return (int32_t)min(re, rrows - 1);   // in range whatever the inputs
  };
  // Records winner wr (miss rank mr) with its source.
  auto record = [&](int wr, int mr, int32_t p, int32_t sl, bool ring, bool miss) {
    if (wr >= K) return;
    sh.selpos[wr] = p;
    if (!kCache) return;
    sh.selslot[wr] = ring ? C + ring_entry(p) : (miss ? -1 : sl);
    if (miss && mr < K) {
      sh.mpos[mr] = p;
      sh.midx[mr] = wr;
    }
  };
  uint32_t fw = 0, fm = 0, fr = 0;   // fast path, bit k: entry k wins / misses / is a ring row
  int ex = 0;                        // fast path: winners (low 16 bits) and misses before this thread
  if (fast) {
    int cw = 0, cm = 0, cr = 0, cb = 0;
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
    ex = block_scan_sum(packed, cr | (cb << 16), sh, tot, tot1) - packed;
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
  // Direct stores: a top-K-only step, or a fast-path step whose victims are
  // all never-used slots (miss k takes slot fill + k: nothing to search,
  // nothing evicted), stores each thread's winners from its registers.
  if (fast && (kTopkOnly || (lru && m <= C - fill))) {
    int32_t* tr = kCache && d_trace ? d_trace + (size_t)u * HC_TRACE_INTS(K) : nullptr;
    int32_t* g_slot = d.sel_slot + (size_t)u * K;
    int32_t* g_miss = d.miss_pos + (size_t)u * K;
    int32_t* g_vic = d.victim + (size_t)u * K;
    int32_t* g_midx = d.miss_idx + (size_t)u * K;
    int32_t* g_old = d.miss_old + (size_t)u * K;
    int wr = ex & 0xFFFF, mr = ex >> 16;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      if (!((fw >> k) & 1u)) continue;
      const int32_t p = pos[k];
      d_sel[(size_t)u * K + wr] = p;
      if (kCache) {
        int32_t enc = slot[k];
        if ((fr >> k) & 1u) enc = C + ring_entry(p);
        if ((fm >> k) & 1u) {
          const int32_t v = fill + mr;
          enc = -(v + 1);
          g_miss[mr] = p;
          g_vic[mr] = v;
          g_midx[mr] = wr;
          g_old[mr] = -1;
          if (tr) {
            tr[HC_TRACE_HEADER + K + mr] = p;
            tr[HC_TRACE_HEADER + 2 * K + mr] = v;
            tr[HC_TRACE_HEADER + 3 * K + mr] = -1;
          }
          ++mr;
        }
        g_slot[wr] = enc;
        if (tr) {
          tr[HC_TRACE_HEADER + wr] = enc < 0 ? -enc - 1 : enc;
          if (wr >= m) {
            tr[HC_TRACE_HEADER + K + wr] = -1;
            tr[HC_TRACE_HEADER + 2 * K + wr] = -1;
            tr[HC_TRACE_HEADER + 3 * K + wr] = -1;
          }
        }
      }
      ++wr;
    }
    if (tid == 0) {
      if (kCache) {
        if (tr) {
          tr[0] = K - m - n_ring;
          tr[1] = m;
          tr[2] = 0;
          tr[3] = n_ring;
          tr[4] = tr[5] = tr[6] = tr[7] = 0;   // the gather's movement counts
        }
        cnt[kCntFill] = fill + m;
        cnt[kCntMiss] = m;
      }
      cnt[kCntWinLo] = nlo;   // the next step's cut window
      cnt[kCntWinHi] = nhi;
    }
    return;
  }
  if (fast) {
    int wr = ex & 0xFFFF, mr = ex >> 16;
#pragma unroll
    for (int k = 0; k < kRun; ++k) {
      if (!((fw >> k) & 1u)) continue;
      const bool ring = (fr >> k) & 1u, miss = (fm >> k) & 1u;
      record(wr, mr, pos[k], slot[k], ring, miss);
      mr += miss;
      ++wr;
    }
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
  // The slots this step's hits use are pinned: a bitmap of them, built only
  // when the queue or a hand supplies victims (never-used slots cannot be
  // pinned).
  if (!lru || m > C - fill) {
    for (int i = tid; i < K; i += kSelThreads) {
      const int32_t e = sh.selslot[i];   // a hit's slot, C + ring entry, or -1
      if (e >= 0 && e < C) atomicOr(&sh.touched[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
  }
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
      tr[4] = tr[5] = tr[6] = tr[7] = 0;   // the gather's movement counts
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
  // 4 entries per thread hold up to 4,096 entries: top-K plus the window's
  // other keys for K up to 3,072 in practice (a larger count takes the slow
  // path, exact as well)
  const bool small = d.K <= 3072;
  // grid (units per session, sessions)
  // with one query row and LRU, kCountWGs more workgroups per unit (grid
  // layers 1 ..) mark the queue's live entries when a compaction is due
  const unsigned layers = d.Q == 1 && d.policy == HC_REPLACE_LRU ? 1 + kCountWGs : 1;
  auto go = [&](auto kern) {
    hipExtLaunchKernelGGL(kern, dim3(d.G * d.Q, d.S, layers), dim3(kSelThreads), 0, st, ev.start,
                          ev.stop, 0, d, a, scores, stride, seg_len, d_sel, d_trace);
  };
  if (d.Q == 1) {
    if (small) go(k_select<false, 4>);
    else go(k_select<false, 8>);
  } else {
    if (small) go(k_select<true, 4>);
    else go(k_select<true, 8>);
  }
  return hipGetLastError();
}

}  // namespace hc
