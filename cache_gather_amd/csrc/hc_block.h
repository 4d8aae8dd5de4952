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
  const int x = wave_incl_scan(v);
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

// LRU victims of unit u at step t without any search.  Slots are filled in
// slot order while never-used ones remain: slots [fill, C) have never been
// used, they are the oldest (last use -1) and no hit touches them, so they come
// first, lowest slot first, and are not stored anywhere.  The used slots are
// ordered by the unit's queue of (slot, step) entries in ascending (step, slot)
// order between a head and a tail: each step appends the slots it used (hits
// and victims) at the tail in slot order, stamped with the step.  An entry is
// live while the slot's last_use still equals its stamp; a slot used again
// later has a newer entry, so the old one is dead without being touched.  The
// callers stamp the hits' last_use before this runs and the victims' after it.
// `touched` (LDS bitmap) marks the slots the step's hits use; the m victims
// (written to vic[0, m)) are the never-used slots from `fill` on, then the
// first live, untouched queue entries from the head, and everything before the
// last of those is dead afterwards, so the head moves past it.  A step reads
// about as many queue entries as it takes victims from the queue, instead of C.
// When the tail would pass the buffer's end (2C entries: once every C / K
// steps or so) the live entries are compacted into the other buffer, followed
// by the step's slots.  n_touched = hits + m; `scratch` is one int of LDS.
__device__ __forceinline__ void lru_victims(const DevState& d, int u, int32_t t, int m,
                                            int n_touched, uint32_t* touched, int32_t* vic,
                                            int32_t* wtot, int32_t* scratch) {
  const int C = d.C, QC = d.qcap, tid = threadIdx.x;
  constexpr int kPer = 4;   // queue entries per thread and window (two 16-byte loads)
  int32_t* cnt = d.cnt + (size_t)u * d.Q * kCntStride;
  // clamped, so that a corrupted counter line still keeps every access in range
  const int e = min(max(cnt[kCntQTail], 0), QC), h = min(max(cnt[kCntQHead], 0), e);
  const int b = cnt[kCntQBuf] & 1;
  const int2* q = d.oq + ((size_t)u * 2 + b) * QC;
  const int32_t* last = d.last_use + (size_t)u * C;
  auto pinned = [&](int v) { return (touched[v >> 5] >> (v & 31)) & 1u; };
  // entries jb .. jb + n - 1 (n a multiple of 2, jb even) of this thread
  auto load = [&](int jb, int n, int2* ent) {
    for (int x = 0; x < n; x += 2) {
      int4 w = make_int4(-1, -1, -1, -1);
      if (jb + x < e) w = *reinterpret_cast<const int4*>(q + jb + x);   // QC % 4 == 0
      ent[x] = make_int2(w.x, w.y);
      ent[x + 1] = make_int2(w.z, w.w);
    }
  };

  // never-used slots first, then the first live, untouched entries from the head
  if (tid == 0) *scratch = h - 1;   // queue index of the last victim taken from the queue
  const int fill = min(max(cnt[kCntFill], 0), C);
  const int n_new = m < C - fill ? m : C - fill;
  for (int k = tid; k < n_new; k += kSelThreads) vic[k] = fill + k;
  int found = n_new;
  for (int j0 = h & ~(kPer - 1); found < m && j0 < e; j0 += kSelThreads * kPer) {
    const int jb = j0 + tid * kPer;
    int2 ent[kPer];
    load(jb, kPer, ent);
    bool f[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = jb + k;
      f[k] = j >= h && j < e && ent[k].x >= 0 && ent[k].x < C && !pinned(ent[k].x);
    }
    int lu[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) lu[k] = f[k] ? last[ent[k].x] : 0;
    int c = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      f[k] = f[k] && lu[k] == ent[k].y;
      c += f[k];
    }
    int total;
    int k0 = found + block_incl_scan(c, wtot, total) - c;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (!f[k]) continue;
      if (k0 < m) {
        vic[k0] = ent[k].x;
        if (k0 == m - 1) *scratch = jb + k;
      }
      ++k0;
    }
    found += total;
  }
  // fewer than m candidates means a corrupted queue: report it, and keep every
  // index in range
  if (found < m && tid == 0) report_error(d, kErrLru);
  for (int k = found + tid; k < m; k += kSelThreads) vic[k] = 0;
  __syncthreads();
  const int hn = *scratch + 1;
  for (int k = tid; k < m; k += kSelThreads) atomicOr(&touched[vic[k] >> 5], 1u << (vic[k] & 31));
  __syncthreads();

  const bool fits = e + n_touched <= QC;
  int2* qw = const_cast<int2*>(fits ? q : d.oq + ((size_t)u * 2 + (b ^ 1)) * QC);
  int base = e;
  if (!fits) {
    // survivors: the live entries after the last victim that this step did
    // not use, in order, to the front of the other buffer.  Wave w of a
    // window owns 1,024 consecutive entries, lane-interleaved so that loads
    // and stores coalesce; ranks inside the wave come from ballots and one
    // block scan of the wave totals orders the waves.
    constexpr int kCPer = 16;
    const int lane = lane_id(), wv = tid >> 6;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int kept = 0;
    for (int j0 = hn; j0 < e; j0 += kSelThreads * kCPer) {
      const int wb = j0 + wv * 64 * kCPer;
      int2 ent[kCPer];
#pragma unroll
      for (int k = 0; k < kCPer; ++k) {
        const int j = wb + k * 64 + lane;
        ent[k] = j < e ? q[j] : make_int2(-1, -1);
      }
      bool f[kCPer];
#pragma unroll
      for (int k = 0; k < kCPer; ++k)
        f[k] = ent[k].x >= 0 && ent[k].x < C && !pinned(ent[k].x);
      int lu[kCPer];
#pragma unroll
      for (int k = 0; k < kCPer; ++k) lu[k] = f[k] ? last[ent[k].x] : 0;
      int wave_total = 0;
#pragma unroll
      for (int k = 0; k < kCPer; ++k) {
        f[k] = f[k] && lu[k] == ent[k].y;
        wave_total += __popcll(__ballot(f[k]));
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
      for (int k = 0; k < kCPer; ++k) {
        const uint64_t bal = __ballot(f[k]);
        if (f[k]) {
          const int o = run + __popcll(bal & lt_mask);
          if (o < QC) qw[o] = ent[k];
        }
        run += __popcll(bal);
      }
      kept += total;
    }
    base = kept;
  }
  // the step's slots in slot order at the tail
  const int nwords = (C + 31) >> 5;
  int o0 = base;
  for (int w0 = 0; w0 < nwords; w0 += kSelThreads) {
    const int w = w0 + tid;
    uint32_t bits = w < nwords ? touched[w] : 0u;
    int total;
    int o = o0 + block_incl_scan(__popc(bits), wtot, total) - __popc(bits);
    while (bits) {
      const int v = w * 32 + __ffs(bits) - 1;
      bits &= bits - 1;
      if (o < QC) qw[o] = make_int2(v, t);
      ++o;
    }
    o0 += total;
  }
  if (tid == 0) {
    cnt[kCntQHead] = fits ? hn : 0;
    cnt[kCntQTail] = o0 < QC ? o0 : QC;
    cnt[kCntQBuf] = fits ? b : (b ^ 1);
    cnt[kCntFill] = fill + n_new;
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
