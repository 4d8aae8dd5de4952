// hc_block.h — prefix sums and ballot ranks over a 1,024-thread workgroup
// (16 wave64), shared by the selection kernels.
#pragma once

#include "hc_internal.h"

namespace hc {

constexpr int kSelThreads = 1024;
constexpr int kWaves = kSelThreads / 64;

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

// LRU victims of unit u at step t without any search.  The unit's order list
// (parity t & 1) holds all C slots in ascending (last_use, slot); `touched`
// (LDS bitmap) marks the slots this step's hits use.  Dropping them keeps the
// list sorted, so the m victims are its first m untouched entries (written to
// vic[0, m)); the next list (parity t + 1) is the remaining entries followed by
// the step's n_touched slots — hits and victims, all now last used at t — in
// slot order, read out of the bitmap after the victims are added to it.
// Wave w of a round owns 2,048 consecutive entries, lane-interleaved so every
// load is coalesced; ranks inside the wave come from ballots, and one block
// scan of the 16 wave totals orders the waves.
__device__ __forceinline__ void lru_victims(const DevState& d, int u, int32_t t, int m,
                                            int n_touched, uint32_t* touched, int32_t* vic,
                                            int32_t* wtot) {
  const int C = d.C, tid = threadIdx.x;
  const int nwords = (C + 31) >> 5;
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
      const bool keep = v[e] >= 0 && !((touched[v[e] >> 5] >> (v[e] & 31)) & 1u);
      if (!keep) v[e] = -1;
      wave_total += __popcll(__ballot(keep));
    }
    if (lane == 0) wtot[wv] = wave_total;
    __syncthreads();
    int run = kept, total = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      run += i < wv ? wtot[i] : 0;
      total += wtot[i];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kOrdPer; ++e) {
      const uint64_t bal = __ballot(v[e] >= 0);
      if (v[e] >= 0) {
        const int k = run + __popcll(bal & lt_mask);
        if (k < m) vic[k] = v[e];
        else onxt[k - m] = v[e];
      }
      run += __popcll(bal);
    }
    kept += total;
  }
  __syncthreads();
  for (int k = tid; k < m; k += kSelThreads) atomicOr(&touched[vic[k] >> 5], 1u << (vic[k] & 31));
  __syncthreads();
  int base = C - n_touched;
  for (int w0 = 0; w0 < nwords; w0 += kSelThreads) {
    const int w = w0 + tid;
    uint32_t bits = w < nwords ? touched[w] : 0u;
    int total;
    const int incl = block_incl_scan(__popc(bits), wtot, total);
    int o = base + incl - __popc(bits);
    while (bits) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      onxt[o++] = w * 32 + b;
    }
    base += total;
  }
}

// Hand-based victims of unit u at step t: circular (clock = false) or clock
// with reference bits (clock = true).  Sequentially the hand walks the slots
// from its position h, skipping slots used this step (`touched`); circular
// takes every slot it reaches, clock clears and skips slots whose reference
// bit is set and takes slots whose bit is clear.  In parallel: in circular
// order from h, let A be the unpinned slots with a clear bit (all unpinned
// slots for circular) and B those with a set bit.  The m victims are the first
// m of A in that order, and if A is shorter, the first m - |A| of B (the
// second revolution, after the first cleared every bit of B).  The hand stops
// just past the last victim.  Clock's new bits: set for pinned slots and
// victims (hits and fills), clear for every other slot the hand passed (all
// of B in the second case), unchanged beyond.  The circular order is cut into
// nwords + 1 pieces: the word holding h from h on, the following words, and
// that word's bits below h last.  `last` is LDS scratch of one int.
__device__ __forceinline__ void hand_victims(const DevState& d, int u, int m, bool clock,
                                             const uint32_t* touched, int32_t* vic,
                                             int32_t* wtot, int32_t* last) {
  const int C = d.C, tid = threadIdx.x;
  const int nwords = (C + 31) >> 5, npieces = nwords + 1;
  int32_t* hand = d.cnt + (size_t)u * d.Q * kCntStride + kCntHand;
  uint32_t* ref = d.refbits + (size_t)u * nwords;
  const int h = *hand, hw = h >> 5, hb = h & 31;
  const int per = (npieces + kSelThreads - 1) / kSelThreads;
  const int p0 = tid * per;
  constexpr int kMaxPer = (HC_MAX_SLOTS / 32 + 1 + kSelThreads - 1) / kSelThreads;  // 9
  uint32_t pa[kMaxPer], pb[kMaxPer], pm[kMaxPer];
  int pw[kMaxPer];
  int ca = 0, cb = 0;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int p = p0 + i;
    pa[i] = pb[i] = pm[i] = 0;
    pw[i] = 0;
    if (i >= per || p >= npieces) continue;
    const int w = p < nwords ? (hw + p) % nwords : hw;
    uint32_t mk = 0xFFFFFFFFu;
    if (w == nwords - 1 && (C & 31)) mk &= (1u << (C & 31)) - 1u;
    if (p == 0) mk &= ~((1u << hb) - 1u);
    if (p == nwords) mk &= (1u << hb) - 1u;
    const uint32_t avail = ~touched[w] & mk;
    const uint32_t r = clock ? ref[w] : 0u;
    pw[i] = w;
    pm[i] = mk;
    pa[i] = avail & ~r;
    pb[i] = avail & r;
    ca += __popc(pa[i]);
    cb += __popc(pb[i]);
  }
  int a_tot, b_tot = 0;
  const int a_ex = block_incl_scan(ca, wtot, a_tot) - ca;
  int b_ex = 0;
  if (clock) b_ex = block_incl_scan(cb, wtot, b_tot) - cb;
  const int mA = m < a_tot ? m : a_tot;   // victims of the first revolution
  const int mB = m - mA;                  // of the second (clock only)
  if (tid == 0) *last = -1;
  __syncthreads();
  uint32_t vbits[kMaxPer];
  int ra = a_ex, rb = b_ex;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    vbits[i] = 0;
    uint32_t bits = pa[i];
    while (bits && ra < mA) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      const int v = pw[i] * 32 + b;
      vic[ra] = v;
      vbits[i] |= 1u << b;
      if (ra == m - 1) *last = v;
      ++ra;
    }
    bits = pb[i];
    while (bits && rb < mB) {
      const int b = __ffs(bits) - 1;
      bits &= bits - 1;
      const int v = pw[i] * 32 + b;
      vic[mA + rb] = v;
      vbits[i] |= 1u << b;
      if (mA + rb == m - 1) *last = v;
      ++rb;
    }
  }
  __syncthreads();
  const int vl = *last;
  if (m > 0 && tid == 0) *hand = (vl + 1) % C;
  if (!clock) return;
  // new reference bits of this thread's pieces (the hand's word is split over
  // two pieces, so each piece changes only its own bits)
  const int cl = m > 0 ? (vl - h + C) % C : -1;   // circular position of the last victim
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    if (!pm[i]) continue;
    const uint32_t pinned = touched[pw[i]] & pm[i];
    uint32_t keep = 0;   // bits of B the hand did not pass
    if (m == 0) {
      keep = pb[i];
    } else if (mB == 0) {
      uint32_t bits = pb[i];
      while (bits) {
        const int b = __ffs(bits) - 1;
        bits &= bits - 1;
        if ((pw[i] * 32 + b - h + C) % C > cl) keep |= 1u << b;
      }
    }
    const uint32_t nb = pinned | vbits[i] | keep;
    atomicAnd(&ref[pw[i]], ~pm[i]);
    atomicOr(&ref[pw[i]], nb);
  }
}

}  // namespace hc
