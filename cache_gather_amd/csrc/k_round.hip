// k_round.hip — the cache round of a multi-query (MTP verification) step.
//
// Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
// section "GPU cache management has hazards too": verification processes
// several query rows, and several queries can select the same missing
// position.  The fixes the page keeps: a slot filled in the current round is
// a hit source only in the next round; duplicate misses in a round read host
// RAM directly; slots used by the current round are pinned.
//
// After k_select has written each query's top-K (ascending positions), one
// 1,024-thread workgroup per unit (session, group):
//  1. forms the ascending union of the group's Q selections window by window:
//     one bit per selected position in an LDS bitmap of 262,144 positions
//     (duplicates collapse), set bits read back in order, and each entry's
//     union index from per-word prefix counts — no sort and no search;
//  2. finds each union entry's first row (lowest query, by an LDS atomic
//     minimum): the row that fills a missing slot;
//  3. runs the single-query method on the union: lookup (ring rows skip the
//     cache), hits stamped and marked, LRU victims from the stamped queue,
//     and the (miss, victim) pairs applied;
//  4. gives every query row its source for the gather: the hit slot, the ring
//     entry, -(victim + 1) for the row that fills the slot, and
//     -(C + 1 + position) — read host RAM directly — for any other row of the
//     same missing position.
#include "hc_block.h"

namespace hc {

constexpr int kRoundMax = HC_MAX_ROUND_ROWS;        // Q * K <= 8,192
constexpr int kPer = kRoundMax / kSelThreads;       // entries per thread

struct RoundShared {
  int32_t a[kRoundMax];     // position-window bitmap, then the touched-slot bitmap
  int32_t b[kRoundMax];     // union index of each bitmap word, then union sources
  int32_t upos[kRoundMax];  // union positions, ascending
  int32_t vic[kRoundMax];   // first row of each union entry, then victim slot of miss k
  int32_t wtot[kWaves];
  int32_t n_evict;
  int32_t n_ring;
  int32_t wmin;
};

__global__ __launch_bounds__(kSelThreads) void k_round(DevState d, StepArgs a,
                                                       const int32_t* __restrict__ d_sel,
                                                       int32_t* __restrict__ d_trace) {
  __shared__ RoundShared sh;
  const int u = blockIdx.x, tid = threadIdx.x;
  const int K = d.K, C = d.C, Q = d.Q, QK = Q * K;
  const int32_t t = a.t;
  int32_t* g_slot = d.sel_slot + (size_t)u * QK;   // [Q][K] of this unit

  // ---- 0. the Q selections into LDS ----------------------------------------
  const int32_t* sel = d_sel + (size_t)u * QK;
  int32_t xe[kPer], je[kPer];   // this thread's entries e = k * 1024 + tid, their union index
  bool bad = false;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = k * kSelThreads + tid;
    xe[k] = e < QK ? sel[e] : 0x7FFFFFFF;
    je[k] = 0;
    bad |= xe[k] < 0;
  }
  if (tid == 0) sh.n_evict = sh.n_ring = 0;
  if (__syncthreads_or(bad)) {
    // a query's selection was abandoned (inconsistent scan state, already
    // reported): touch nothing, the gather reads slot 0
    for (int e = tid; e < QK; e += kSelThreads) g_slot[e] = 0;
    if (tid == 0) {
      d.cnt[(size_t)u * Q * kCntStride + kCntMiss] = 0;
      report_error(d, kErrRound);
    }
    return;
  }

  // ---- 1. the union, one position window at a time ------------------------
  // Each non-empty window of kWinBits positions: one bit per selected position
  // in an LDS bitmap (duplicates collapse), per-word prefix counts, set bits
  // read back in ascending order as union entries, and each entry's union
  // index = prefix of its word + set bits below it in the word.
  constexpr int kWinWords = kRoundMax;          // 8,192 words
  constexpr int kWinBits = kWinWords * 32;      // 262,144 positions
  constexpr int kWordsPer = kWinWords / kSelThreads;
  uint32_t* bm = reinterpret_cast<uint32_t*>(sh.a);
  int32_t* pre = sh.b;                          // word -> union index of its first bit
  int n = 0;
  int64_t wend = 0;
  for (;;) {
    // the next non-empty window starts at the window of the smallest entry >= wend
    int32_t lmin = 0x7FFFFFFF;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (xe[k] >= wend && xe[k] < lmin) lmin = xe[k];
    if (tid == 0) sh.wmin = 0x7FFFFFFF;
    __syncthreads();
    if (lmin != 0x7FFFFFFF) atomicMin(&sh.wmin, lmin);
    __syncthreads();
    const int32_t xmin = sh.wmin;
    if (xmin == 0x7FFFFFFF) break;
    const int32_t w0 = xmin & ~(kWinBits - 1);
    wend = (int64_t)w0 + kWinBits;
    for (int w = tid; w < kWinWords; w += kSelThreads) bm[w] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (xe[k] >= w0 && xe[k] < wend)
        atomicOr(&bm[(xe[k] - w0) >> 5], 1u << (xe[k] & 31));
    __syncthreads();
    uint32_t wd[kWordsPer];
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < kWordsPer; ++i) {
      wd[i] = bm[kWordsPer * tid + i];
      cnt += __popc(wd[i]);
    }
    int total;
    int o = n + block_incl_scan(cnt, sh.wtot, total) - cnt;
#pragma unroll
    for (int i = 0; i < kWordsPer; ++i) {
      const int w = kWordsPer * tid + i;
      pre[w] = o;
      uint32_t bits = wd[i];
      while (bits) {
        const int bit = __ffs(bits) - 1;
        bits &= bits - 1;
        sh.upos[o++] = w0 + w * 32 + bit;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (xe[k] >= w0 && xe[k] < wend) {
        const int w = (xe[k] - w0) >> 5, bit = xe[k] & 31;
        je[k] = pre[w] + __popc(bm[w] & ((1u << bit) - 1u));
      }
    n += total;
    __syncthreads();
  }

  // ---- 2. the first (lowest-query) row of every union entry -----------------
  int32_t* firstrow = sh.vic;                   // free until the LRU step
  for (int j = tid; j < n; j += kSelThreads) firstrow[j] = 0x7FFFFFFF;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = k * kSelThreads + tid;
    if (e < QK) atomicMin(&firstrow[je[k]], e);
  }
  __syncthreads();
  uint32_t first = 0;   // bit k: entry k is the lowest query's row of its position
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int e = k * kSelThreads + tid;
    if (e < QK && firstrow[je[k]] == e) first |= 1u << k;
  }
  __syncthreads();

  // ---- 3. lookup on the union ---------------------------------------------
  uint32_t* touched = reinterpret_cast<uint32_t*>(sh.a);
  const int nwords = (C + 31) >> 5;
  for (int w = tid; w < nwords; w += kSelThreads) touched[w] = 0;
  int32_t* pos2slot = d.pos2slot + (size_t)u * d.hcap;
  int32_t* slot2pos = d.slot2pos + (size_t)u * C;
  int32_t* last_use = d.last_use + (size_t)u * C;
  const uint32_t ring_lo = a.ring_lo[u / d.G];
  const int rounds = (n + kSelThreads - 1) / kSelThreads;   // union entries per thread
  int32_t lp[kPer], ls[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {   // all map reads in flight together
    const int j = k * kSelThreads + tid;
    lp[k] = j < n ? sh.upos[j] : 0;
    const bool in_ring = j < n && (uint32_t)lp[k] >= ring_lo;
    ls[k] = j < n && !in_ring ? pos2slot[lp[k]] : 0;
    // ring rows are a suffix of the ascending union
    if (in_ring && (j == 0 || (uint32_t)sh.upos[j - 1] < ring_lo)) sh.n_ring = n - j;
  }
  __syncthreads();
  const int n_ring = sh.n_ring;
  const int first_ring = n - n_ring;
  int my_miss = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int j = k * kSelThreads + tid;
    const bool valid = j < n;
    const bool in_ring = valid && j >= first_ring;
    const bool miss = valid && !in_ring && ls[k] < 0;
    if (valid && !in_ring && !miss) {
      last_use[ls[k]] = t;
      atomicOr(&touched[ls[k] >> 5], 1u << (ls[k] & 31));
    }
    // union sources: slot, C + ring entry, -1 for a miss (victim below)
    if (valid) sh.b[j] = in_ring ? C + (int32_t)((uint32_t)lp[k] % (uint32_t)d.ring_rows) : ls[k];
    my_miss += miss;
  }
  int m;
  block_incl_scan(my_miss, sh.wtot, m);

  // ---- 4. LRU victims ------------------------------------------------------
  if (d.policy == HC_REPLACE_LRU)
    lru_victims(d, u, t, m, n - n_ring, touched, sh.vic, sh.wtot, &sh.wmin);
  else
    hand_victims(d, u, m, d.policy == HC_REPLACE_CLOCK, touched, sh.vic, sh.wtot, &sh.wmin);

  // ---- 5. apply (miss, victim) pairs in ascending position order ----------
  int32_t* tr = d_trace ? d_trace + (size_t)u * HC_TRACE_INTS(QK) : nullptr;
  int32_t* g_miss = d.miss_pos + (size_t)u * QK;
  int32_t* g_vic = d.victim + (size_t)u * QK;
  int32_t* g_midx = d.miss_idx + (size_t)u * QK;
  int kbase = 0;
  for (int k = 0; k < rounds; ++k) {
    const int j = k * kSelThreads + tid;
    const bool miss = j < n && sh.b[j] == -1;
    int total;
    const int kk = kbase + block_flag_rank(miss, sh.wtot, total);
    if (miss) {
      const int32_t v = sh.vic[kk], p = sh.upos[j];
      const int32_t old = slot2pos[v];
      if (old >= 0) {
        pos2slot[old] = -1;
        atomicAdd(&sh.n_evict, 1);
      }
      pos2slot[p] = v;
      slot2pos[v] = p;
      last_use[v] = t;
      sh.b[j] = -(kk + 1);   // miss index; the victim is vic[kk]
      g_miss[kk] = p;
      g_vic[kk] = v;
      if (tr) {
        tr[HC_TRACE_HEADER + QK + kk] = p;
        tr[HC_TRACE_HEADER + 2 * QK + kk] = v;
        tr[HC_TRACE_HEADER + 3 * QK + kk] = old;
      }
    }
    kbase += total;
  }
  __syncthreads();

  // ---- 6. the source of every query row ------------------------------------
  // The first row of a missing position fills the victim slot (the gather's
  // miss workgroup writes that row); any other row of it reads host RAM.
#pragma unroll 1
  for (int k = 0; k < kPer; ++k) {
    const int e = k * kSelThreads + tid;
    if (e >= QK) continue;
    int32_t enc = sh.b[je[k]];
    if (enc < 0) {
      const int kk = -enc - 1;
      if ((first >> k) & 1u) {
        g_midx[kk] = e;
        enc = -(sh.vic[kk] + 1);
      } else {
        enc = -(C + 1 + sh.upos[je[k]]);
      }
    }
    g_slot[e] = enc;
  }
  if (tr) {
    for (int j = tid; j < QK; j += kSelThreads) {
      const int32_t enc = j < n ? sh.b[j] : -1;
      tr[HC_TRACE_HEADER + j] = j < n ? (enc < 0 ? sh.vic[-enc - 1] : enc) : -1;
      if (j >= m) {
        tr[HC_TRACE_HEADER + QK + j] = -1;
        tr[HC_TRACE_HEADER + 2 * QK + j] = -1;
        tr[HC_TRACE_HEADER + 3 * QK + j] = -1;
      }
    }
    if (tid == 0) {
      tr[0] = n - m - n_ring;
      tr[1] = m;
      tr[2] = sh.n_evict;
      tr[3] = n_ring;
      tr[4] = tr[5] = tr[6] = tr[7] = 0;   // the gather's movement counts
    }
  }
  if (tid == 0) d.cnt[(size_t)u * Q * kCntStride + kCntMiss] = m;
}

hipError_t launch_round(const DevState& d, const StepArgs& a, const int32_t* d_sel,
                        int32_t* d_trace, hipStream_t st, StageEv ev) {
  hipExtLaunchKernelGGL(k_round, dim3(d.S * d.G), dim3(kSelThreads), 0, st, ev.start, ev.stop, 0, d,
                        a, d_sel, d_trace);
  return hipGetLastError();
}

}  // namespace hc
