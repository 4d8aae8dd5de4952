// k_gather.hip — the hot gather: every selected row, hit or miss, dequantised
// into the contiguous bf16 attention buffer [S][L][K][576].
//
// Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
// section "Decision three: let the GPU manage the hot cache directly" and its
// data-flow figure: a hit reads the hot slot in VRAM, a miss reads the
// registered host-memory copy, and the gather emits a compact selection for
// attention.  Section "GPU cache management has hazards too": a slot filled
// in a round is not read by another block of that round, and repeated misses
// read host RAM.
//
// One launch, three kinds of workgroup:
//   * the first workgroups walk the dense miss list (every layer
//     of every unit): each missing row is read from pinned host RAM over PCIe
//     (zero-copy), written into its victim slot, and dequantised from the same
//     registers — so its slot is only ever read in later steps, and all PCIe
//     reads are issued as soon as the launch starts;
//   * the remaining workgroups stream the hit rows out of the HBM slots, and
//     the rows of the recent ring out of the ring (rows that missed are
//     skipped; the miss workgroups write them).  In a multi-query round a
//     position several queries missed is filled by its first query's row; the
//     other queries' rows of it read host RAM directly (the page's rule for
//     duplicate misses), never the slot being filled;
//   * between them, with one query row per round, one bookkeeping workgroup
//     per unit: the select kernel only decides, and these write its decisions
//     into the unit's state (last-use stamps, slot maps, LRU queue) for the
//     next step while the rest of the launch streams rows.
// The PCIe transfer of the few missing rows thus overlaps the HBM stream of
// the many hits.
//
// Row format (section "Separate historical capacity from the current working
// set"): 512 int8 latent, 8 fp16 scales (one per 64 values), 64 bf16 RoPE.
// Output j < 512 is bf16_rne(int8 * scale) — the fp32 product is exact — and
// the RoPE values are copied.
//
// gfx950 mapping: a row is 40 work items — 32 latent chunks (16 B in, 32 B
// out) and 8 RoPE chunks (16 B in, 16 B out) — so 320 threads (5 wave64) hold
// 8 rows with every lane busy.  A hit workgroup takes two such passes, both
// rows' loads in flight before the first store (16 rows per workgroup:
// measured on MI355X with the caches flushed, 3-4% faster than one row per
// thread, and 4 rows slower again); a miss workgroup keeps one row per thread
// in flight (two slowed the PCIe reads).  Grid rows [0, miss_rows) are the
// miss workgroups, dispatched first; after the bookkeeping rows, grid row
// miss_rows + bk_rows + sl holds layer sl's hit rows, so no per-row index
// division is needed (with Q query rows, layer sl's query q).  HBM-bound:
// 656 B read (hit) or written (miss) + 1,152 B written per
// selected row; PCIe: 656 B per missing row.  bf16 rounding by
// v_cvt_pk_bf16_f32.
#include <algorithm>

#include "hc_internal.h"

namespace hc {

constexpr int kRowsPerPass = 8;
constexpr int kItemsPerRow = 40;
constexpr int kGatherThreads = kRowsPerPass * kItemsPerRow;  // 320
constexpr int kHitPasses = 2;                                  // rows per thread, hit workgroups
constexpr int kRowsPerRound = kRowsPerPass * kHitPasses;       // hit rows per workgroup: 16
constexpr int kMissRowsPerRound = kRowsPerPass;                // missing rows per workgroup round
// Workgroups reserved for the miss list.  Only about one per kMissRowsPerBlock
// missing rows is active (at least kMissBlocksMin): while the hit rows keep HBM
// busy, few CUs then wait on PCIe and the rest stream HBM (more miss
// workgroups slowed such steps, even steps the link bounds: a 78-layer step
// with 5K-55K missing rows among its 160K took 10% longer with one per 16),
// and a cold step still has enough reads in flight.  A launch with fewer than
// kFewHitRows other rows has no such stream to protect, and one workgroup per
// kMissRowsFewHits missing rows keeps more of them in flight (one layer,
// ~2,000 missing rows of 2,048: 45 -> 36 us).
constexpr int kMissBlocks = 256;
constexpr int kMissBlocksMin = 32;
constexpr int kMissRowsPerBlock = 64;
constexpr int kMissRowsFewHits = 16;
constexpr int kFewHitRows = 16384;

// Sign-extended int8 number k (0..3) of w, as float.
__device__ __forceinline__ float i8f(uint32_t w, int k) {
  return (float)((int32_t)(w << (24 - 8 * k)) >> 24);
}

// Where pass p of this thread reads its row, where it writes the output row,
// and (misses only) which slot it fills.
template <int kPasses>
struct RowJob {
  gbyte* src[kPasses];
  uint8_t* dst[kPasses];
  uint8_t* fill[kPasses];
};

// fp16 scale g (0..7) of a row's 16-B scale block, as float.
__device__ __forceinline__ float scale_of(const u32x4& blk, int g) {
  const uint32_t w = (g >> 1) == 0 ? blk.x : (g >> 1) == 1 ? blk.y : (g >> 1) == 2 ? blk.z : blk.w;
  const uint16_t h = (uint16_t)((g & 1) ? (w >> 16) : (w & 0xFFFF));
  return (float)__builtin_bit_cast(_Float16, h);
}

// Copies / dequantises this thread's item of up to kPasses rows; all loads are
// issued before the first store.  Latent lanes read their 16 latent bytes and
// the row's whole 16-B scale block (one address for all 32 lanes of a row, so
// it costs one request); RoPE lanes read 16 bytes each.
template <int kPasses>
__device__ __forceinline__ void run_rows(const RowJob<kPasses>& j, int item) {
  u32x4 v[kPasses], sblk[kPasses];
  const int off = item < 32 ? 16 * item : HC_ROPE_OFFSET + 16 * (item - 32);
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (!j.dst[p] && !j.fill[p]) continue;
    v[p] = gload<u32x4>(j.src[p] + off);
    if (item < 32) sblk[p] = gload<u32x4>(j.src[p] + HC_SCALE_OFFSET);
  }
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if (!j.dst[p] && !j.fill[p]) continue;
    if (j.fill[p]) {
      *reinterpret_cast<u32x4*>(j.fill[p] + off) = v[p];
      if (item == 0) *reinterpret_cast<u32x4*>(j.fill[p] + HC_SCALE_OFFSET) = sblk[p];
    }
    if (!j.dst[p]) continue;   // fill only: no gathered output
    if (item < 32) {
      const float sc = scale_of(sblk[p], item >> 2);
      const u32x4 q = v[p];
      u32x4 a, b;
      a.x = bf16x2_rne(i8f(q.x, 0) * sc, i8f(q.x, 1) * sc);
      a.y = bf16x2_rne(i8f(q.x, 2) * sc, i8f(q.x, 3) * sc);
      a.z = bf16x2_rne(i8f(q.y, 0) * sc, i8f(q.y, 1) * sc);
      a.w = bf16x2_rne(i8f(q.y, 2) * sc, i8f(q.y, 3) * sc);
      b.x = bf16x2_rne(i8f(q.z, 0) * sc, i8f(q.z, 1) * sc);
      b.y = bf16x2_rne(i8f(q.z, 2) * sc, i8f(q.z, 3) * sc);
      b.z = bf16x2_rne(i8f(q.w, 0) * sc, i8f(q.w, 1) * sc);
      b.w = bf16x2_rne(i8f(q.w, 2) * sc, i8f(q.w, 3) * sc);
      u32x4* o = reinterpret_cast<u32x4*>(j.dst[p] + 32 * item);
      __builtin_nontemporal_store(a, o);
      __builtin_nontemporal_store(b, o + 1);
    } else {
      __builtin_nontemporal_store(
          v[p], reinterpret_cast<u32x4*>(j.dst[p] + 2 * HC_LATENT_BYTES + 16 * (item - 32)));
    }
  }
}

__device__ __forceinline__ int layers_in_group(const DevState& d, int g) {
  const int n = d.L - g * d.R;
  return n < d.R ? n : d.R;
}

// Block-wide sum over the gather workgroup's 320 threads.
__device__ __forceinline__ int gather_block_sum(int v, int32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int tot = 0;
#pragma unroll
  for (int i = 0; i < kGatherThreads / 64; ++i) tot += wsum[i];
  __syncthreads();
  return tot;
}

// Inclusive prefix over the gather workgroup's threads (thread order).
__device__ __forceinline__ int gather_block_scan(int v, int32_t* wsum, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kGatherThreads / 64; ++i) {
    off += i < w ? wsum[i] : 0;
    tot += wsum[i];
  }
  __syncthreads();
  total = tot;
  return x + off;
}

// Bookkeeping of unit u after its select kernel (one query row per round),
// done beside the gather so that the select kernel's chain ends with its
// decisions: stamps the step's slots (hits and victims) with last use t,
// applies the (miss, victim) pairs to pos2slot / slot2pos (the evicted
// position leaves the map), and, for LRU, appends the step's slots to the
// unit's queue in slot order, stamped t.  Workgroup p of kBkSlices per unit;
// p = 0 stamps, maps and appends.  When this step's select launch marked the
// queue for a compaction (its slots might not fit after the tail), every slice
// p writes the survivors of its part of the queue — marked live then, and not
// used by this step — in order, to the other buffer at the place that the
// marks before the slice give, and fills the rest of its marked places with
// dead entries (-1, -1: entries this step used, which the queue's readers
// skip); p = 0 then appends after all of them.  Everything a slice reads to
// place its survivors was written by the select launch, so the slices never
// wait for one another.  Otherwise the queue
// is compacted, if it must be, by p = 0 alone.  Nothing else here is read by
// this launch's other workgroups; the next step's kernels come after the
// launch.  `touched` is LDS of ceil(C / 32) words.
__device__ __forceinline__ void bookkeeping(const DevState& d, int u, int p, int32_t t,
                                            uint32_t* touched, int32_t* wsum) {
  const int C = d.C, K = d.K, tid = threadIdx.x;
  const int nwords = (C + 31) >> 5;
  int32_t* cnt = d.cnt + (size_t)u * kCntStride;
  const bool lru = d.policy == HC_REPLACE_LRU;
  const bool counted = lru && cnt[kCntCntStep] == t;   // a compaction prepared for this step
  if (p > 0 && !counted) return;
  const int m = min(max(cnt[kCntMiss], 0), K);
  int32_t* pos2slot = d.pos2slot + (size_t)u * d.hcap;
  int32_t* slot2pos = d.slot2pos + (size_t)u * C;
  int32_t* last_use = d.last_use + (size_t)u * C;
  const int32_t* g_slot = d.sel_slot + (size_t)u * K;
  for (int w = tid; w < nwords; w += kGatherThreads) touched[w] = 0;
  __syncthreads();
  // hits: stamp (slice 0); hits and victims: mark.  Eight sources per thread
  // are loaded before any is used (a store between two loads keeps the
  // compiler from issuing the second before the first returns).
  constexpr int kSPer = 8;
  for (int i0 = 0; i0 < K; i0 += kGatherThreads * kSPer) {
    int32_t enc[kSPer];
#pragma unroll
    for (int k = 0; k < kSPer; ++k) {
      const int i = i0 + k * kGatherThreads + tid;
      enc[k] = i < K ? g_slot[i] : INT32_MIN;   // INT32_MIN: no slot
    }
#pragma unroll
    for (int k = 0; k < kSPer; ++k) {
      const int32_t e = enc[k];
      const int32_t v = e >= 0 ? (e < C ? e : -1) : (e >= -C ? -e - 1 : -1);
      if (v < 0) continue;   // a ring row, a host row, or past K
      if (e >= 0 && p == 0) last_use[v] = t;
      atomicOr(&touched[v >> 5], 1u << (v & 31));
    }
  }
  if (p == 0) {
    // (miss, victim) pairs
    const int32_t* g_miss = d.miss_pos + (size_t)u * K;
    const int32_t* g_vic = d.victim + (size_t)u * K;
    const int32_t* g_old = d.miss_old + (size_t)u * K;
    for (int k = tid; k < m; k += kGatherThreads) {
      const int32_t v = g_vic[k], pp = g_miss[k], old = g_old[k];
      if (v < 0 || v >= C || pp < 0 || pp >= d.hcap) continue;
      if (old >= 0 && old < d.hcap) pos2slot[old] = -1;
      pos2slot[pp] = v;
      slot2pos[v] = pp;
      last_use[v] = t;
    }
  }
  __syncthreads();
  if (!lru) return;

  const int QC = d.qcap;
  constexpr int kW = kGatherThreads / 64;
  const int lane = tid & 63, wv = tid >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  auto pinned = [&](int v) { return (touched[v >> 5] >> (v & 31)) & 1u; };
  // the step's slots: this thread's bitmap words, in slot order
  const int g = (nwords + kGatherThreads - 1) / kGatherThreads;   // words per thread
  int c = 0;
  for (int i = 0; i < g; ++i) {
    const int w = tid * g + i;
    if (w < nwords) c += __popc(touched[w]);
  }
  int2* qw;          // the buffer that receives the step's slots
  int base, head, buf;
  if (counted) {
    // the queue as the select launch marked it (none of these words changes
    // in this launch): entries [0, qe) of buffer qb; slice p starts at a
    // multiple of 64 entries, so it owns whole words of the marks
    const int qe = min(max(cnt[kCntCntTail], 0), QC);
    const int qb = cnt[kCntCntBuf] & 1;
    const int len = ((qe + kBkSlices - 1) / kBkSlices + 63) / 64 * 64;
    const int lo = min(qe, p * len), hi = min(qe, lo + len);
    const uint32_t* live = d.qlive + (size_t)u * d.qlive_words;
    // the marks before the slice (its first place), in it, and in all
    const int lo_w = lo >> 5, hi_w = lo < hi ? (hi + 31) >> 5 : lo_w, all_w = (qe + 31) >> 5;
    int b0 = 0, b1 = 0, b2 = 0;
    for (int w = tid; w < all_w; w += kGatherThreads) {
      const int n = __popc(live[w]);
      b0 += w < lo_w ? n : 0;
      b1 += w >= lo_w && w < hi_w ? n : 0;
      b2 += n;
    }
    const int off = gather_block_sum(b0, wsum);
    const int mine = gather_block_sum(b1, wsum);
    const int total = gather_block_sum(b2, wsum);
    const int2* q = d.oq + ((size_t)u * 2 + qb) * QC;
    int2* dst = d.oq + ((size_t)u * 2 + (qb ^ 1)) * QC + off;
    // wave w of a window owns 64 * kCPer consecutive entries, lane-interleaved;
    // ranks inside the wave come from ballots, the wave totals order the waves
    constexpr int kCPer = 8;
    int kept = 0;
    for (int j0 = lo; j0 < hi; j0 += kGatherThreads * kCPer) {
      const int wb = j0 + wv * 64 * kCPer;
      int2 ent[kCPer];
      uint32_t lw[kCPer];
#pragma unroll
      for (int k = 0; k < kCPer; ++k) {
        const int j = wb + k * 64 + lane;
        ent[k] = j < hi ? q[j] : make_int2(-1, -1);
        lw[k] = j < hi ? live[j >> 5] : 0u;
      }
      bool f[kCPer];
      int wave_total = 0;
#pragma unroll
      for (int k = 0; k < kCPer; ++k) {
        const int j = wb + k * 64 + lane;
        f[k] = ((lw[k] >> (j & 31)) & 1u) && ent[k].x >= 0 && ent[k].x < C && !pinned(ent[k].x);
        wave_total += __popcll(__ballot(f[k]));
      }
      if (lane == 0) wsum[wv] = wave_total;
      __syncthreads();
      int run = kept, wtotal = 0;
#pragma unroll
      for (int i = 0; i < kW; ++i) {
        run += i < wv ? wsum[i] : 0;
        wtotal += wsum[i];
      }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kCPer; ++k) {
        const uint64_t bal = __ballot(f[k]);
        if (f[k]) {
          const int o = run + __popcll(bal & lt_mask);
          if (o < mine) dst[o] = ent[k];
        }
        run += __popcll(bal);
      }
      kept += wtotal;
    }
    for (int i = min(kept, mine) + tid; i < mine; i += kGatherThreads) dst[i] = make_int2(-1, -1);
    if (p != 0) return;
    qw = d.oq + ((size_t)u * 2 + (qb ^ 1)) * QC;
    base = total;
    head = 0;
    buf = qb ^ 1;
  } else {
    const int qe = min(max(cnt[kCntQTail], 0), QC);
    const int hn = min(max(cnt[kCntQHead], 0), qe);
    const int qb = cnt[kCntQBuf] & 1;
    int2* q = d.oq + ((size_t)u * 2 + qb) * QC;
    const bool fits = qe + gather_block_sum(c, wsum) <= QC;
    qw = fits ? q : d.oq + ((size_t)u * 2 + (qb ^ 1)) * QC;
    base = qe;
    head = hn;
    buf = qb;
    if (!fits) {
      // (not reached when the scan launch prepared the compaction) survivors:
      // the live entries after the head that this step did not use, in
      // order, to the front of the other buffer, by this workgroup alone
      constexpr int kCPer = 8;
      int kept = 0;
      for (int j0 = hn; j0 < qe; j0 += kGatherThreads * kCPer) {
        const int wb = j0 + wv * 64 * kCPer;
        int2 ent[kCPer];
#pragma unroll
        for (int k = 0; k < kCPer; ++k) {
          const int j = wb + k * 64 + lane;
          ent[k] = j < qe ? q[j] : make_int2(-1, -1);
        }
        bool f[kCPer];
#pragma unroll
        for (int k = 0; k < kCPer; ++k) f[k] = ent[k].x >= 0 && ent[k].x < C && !pinned(ent[k].x);
        int lu[kCPer];
#pragma unroll
        for (int k = 0; k < kCPer; ++k) lu[k] = f[k] ? last_use[ent[k].x] : 0;
        int wave_total = 0;
#pragma unroll
        for (int k = 0; k < kCPer; ++k) {
          f[k] = f[k] && lu[k] == ent[k].y;
          wave_total += __popcll(__ballot(f[k]));
        }
        if (lane == 0) wsum[wv] = wave_total;
        __syncthreads();
        int run = kept, total = 0;
#pragma unroll
        for (int i = 0; i < kW; ++i) {
          run += i < wv ? wsum[i] : 0;
          total += wsum[i];
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
      head = 0;
      buf = qb ^ 1;
    }
  }
  // the step's slots at base, this thread's words after the words of the
  // threads before it
  int n_touched;
  int o = base + gather_block_scan(c, wsum, n_touched) - c;
  for (int i = 0; i < g; ++i) {
    const int w = tid * g + i;
    uint32_t bits = w < nwords ? touched[w] : 0u;
    while (bits) {
      const int v = w * 32 + __ffs(bits) - 1;
      bits &= bits - 1;
      if (o < QC) qw[o] = make_int2(v, t);
      ++o;
    }
  }
  if (tid == 0) {
    cnt[kCntQHead] = head;
    cnt[kCntQTail] = base + n_touched < QC ? base + n_touched : QC;
    cnt[kCntQBuf] = buf;
  }
}

__global__ __launch_bounds__(kGatherThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void k_gather(DevState d,
                                                           uint16_t* __restrict__ out,
                                                           int32_t t, int bk_rows,
                                                           int miss_rows, int few_hits_above,
                                                           uint32_t m_q, uint32_t m_l, uint32_t m_r,
                                                           int32_t* __restrict__ trace) {
  // dynamic LDS: [S*G + 1] miss rows (all layers) before unit u, or the
  // bookkeeping's touched-slot bitmap
  extern __shared__ int32_t pref[];
  __shared__ int32_t wsum[kGatherThreads / 64];
  const int item = threadIdx.x % kItemsPerRow;
  const int lrow = threadIdx.x / kItemsPerRow;
  uint8_t* const out_b = reinterpret_cast<uint8_t*>(out);
  const size_t out_row_bytes = (size_t)kOut * 2;

  if ((int)blockIdx.y >= miss_rows && (int)blockIdx.y < miss_rows + bk_rows) {
    // slice-major: every unit's slice 0 (which stamps, maps and appends) first
    const int b = (blockIdx.y - miss_rows) * gridDim.x + blockIdx.x, U = d.S * d.G;
    if (b < U * kBkSlices) bookkeeping(d, b % U, b / U, t, reinterpret_cast<uint32_t*>(pref), wsum);
    return;
  }
  const int row = (int)blockIdx.y < miss_rows ? (int)blockIdx.y : (int)blockIdx.y - bk_rows;
  if (row < miss_rows) {
    RowJob<1> j;
    const int mb = row * gridDim.x + blockIdx.x;  // miss workgroup number
    // ---- dense miss list: prefix of (misses x layers) over units --------
    const int U = d.S * d.G;
    int running = 0;
    for (int u0 = 0; u0 < U; u0 += kGatherThreads) {
      const int u = u0 + threadIdx.x;
      const int c = u < U ? d.cnt[(size_t)u * d.Q * kCntStride + kCntMiss] * layers_in_group(d, u % d.G)
                          : 0;
      // block inclusive scan of c
      const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
      const int x = wave_incl_scan(c);
      if (lane == 63) wsum[w] = x;
      __syncthreads();
      int off = running, tot = 0;
#pragma unroll
      for (int i = 0; i < kGatherThreads / 64; ++i) {
        off += i < w ? wsum[i] : 0;
        tot += wsum[i];
      }
      if (u < U) pref[u + 1] = off + x;
      running += tot;
      __syncthreads();
    }
    if (threadIdx.x == 0) pref[0] = 0;
    __syncthreads();
    const int M = pref[U];
    const int per = M > few_hits_above ? kMissRowsFewHits : kMissRowsPerBlock;
    int active = (M + per - 1) / per;
    active = active < kMissBlocksMin ? kMissBlocksMin : (active > kMissBlocks ? kMissBlocks : active);
    if (mb >= active) return;
    for (int base = mb * kMissRowsPerRound; base < M; base += active * kMissRowsPerRound) {
      const int q = base + lrow;
      if (q >= M) break;   // this thread's later rounds lie further beyond M
      int lo = 0, hi = U;  // largest u with pref[u] <= q
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= q) lo = mid;
        else hi = mid;
      }
      const int u = lo, g = u % d.G, s = u / d.G;
      const int nl = layers_in_group(d, g);
      const int r = q - pref[u], m = (pref[u + 1] - pref[u]) / nl;
      const int lig = r / m, k = r - lig * m;
      const int64_t sl = (int64_t)s * d.L + g * d.R + lig;
      const size_t QK = (size_t)d.Q * d.K;
      const size_t uk = (size_t)u * QK + k;
      j.src[0] = to_global(d.host[sl] + (size_t)d.miss_pos[uk] * kRow);
      j.fill[0] = d.hot + ((size_t)sl * d.C + d.victim[uk]) * kSlotStride;
      j.dst[0] = out ? out_b + ((size_t)sl * QK + d.miss_idx[uk]) * out_row_bytes : nullptr;
      run_rows(j, item);
      if (trace && item == 0) {   // the unit's movement counts (a trace was requested)
        int32_t* tu = trace + (size_t)u * HC_TRACE_INTS(QK);
        atomicAdd(&tu[4], 1);     // read from host RAM
        atomicAdd(&tu[6], 1);     // written into its victim slot
        if (out) atomicAdd(&tu[7], 1);
      }
    }
    return;
  }

  // ---- rows of (layer sl, query q), hr = row - miss_rows = sl * Q + q ---------
  const int hr = row - miss_rows;
  const int sl = div_by(hr, m_q), q = hr - sl * d.Q;   // uniform per workgroup; hr < 2^16
  const int s = div_by(sl, m_l), l = sl - s * d.L;
  const int32_t* slot = d.sel_slot + ((size_t)(s * d.G + div_by(l, m_r)) * d.Q + q) * d.K;
  const uint8_t* hot = d.hot + (size_t)sl * d.C * kSlotStride;
  uint8_t* orow = out_b + (size_t)hr * d.K * out_row_bytes;
  const int i0 = blockIdx.x * kRowsPerRound + lrow;
  RowJob<kHitPasses> j;
  int n_host = 0, n_hbm = 0;   // this thread's rows by source (item 0 of each row counts)
#pragma unroll
  for (int p = 0; p < kHitPasses; ++p) {
    const int i = i0 + p * kRowsPerPass;
    j.dst[p] = nullptr;
    j.fill[p] = nullptr;
    if (i >= d.K) continue;
    const int32_t enc = slot[i];
    if (enc < 0 && enc >= -d.C) continue;  // missed this step: written by a miss workgroup
    if (enc >= d.C)                        // a row of the recent ring (entry enc - C)
      j.src[p] = to_global(d.ring + ((size_t)sl * d.ring_rows + (enc - d.C)) * kRow);
    else if (enc >= 0)                     // a hit
      j.src[p] = to_global(hot + (size_t)enc * kSlotStride);
    else                                   // another query's row of a miss: host RAM
      j.src[p] = to_global(d.host[sl] + (size_t)(-(int64_t)enc - d.C - 1) * kRow);
    j.dst[p] = orow + (size_t)i * out_row_bytes;
    n_host += enc < -d.C;
    n_hbm += enc >= 0;
  }
  run_rows(j, item);
  if (trace) {
    // the unit's movement counts (a trace was requested): this workgroup's
    // rows by source, one atomic add per count
    if (threadIdx.x == 0) wsum[0] = wsum[1] = 0;
    __syncthreads();
    if (item == 0) {
      if (n_host) atomicAdd(&wsum[0], n_host);
      if (n_hbm) atomicAdd(&wsum[1], n_hbm);
    }
    __syncthreads();
    if (threadIdx.x == 0 && wsum[0] + wsum[1] > 0) {
      int32_t* tu = trace + (size_t)(s * d.G + div_by(l, m_r)) * HC_TRACE_INTS(d.Q * d.K);
      if (wsum[0]) atomicAdd(&tu[4], wsum[0]);
      if (wsum[1]) atomicAdd(&tu[5], wsum[1]);
      atomicAdd(&tu[7], wsum[0] + wsum[1]);
    }
  }
}

#ifdef HC_TEST_HOOKS
// Test build: writes a sentinel over every victim slot of every layer before
// the gather fills it, so that a read of a slot being filled in the same
// launch (a read before the fill) would carry the sentinel into the output.
__global__ __launch_bounds__(64) void k_poison(DevState d) {
  const int QK = d.Q * d.K;
  const int64_t n = (int64_t)d.S * d.G * QK * d.R;
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
    const int u = (int)(i / ((int64_t)QK * d.R));
    const int r = (int)(i - (int64_t)u * QK * d.R);
    const int k = r / d.R, lig = r - k * d.R;
    const int g = u % d.G, s = u / d.G;
    if (k >= d.cnt[(size_t)u * d.Q * kCntStride + kCntMiss] || lig >= layers_in_group(d, g)) continue;
    const int v = d.victim[(size_t)u * QK + k];
    if (v < 0 || v >= d.C) continue;
    uint8_t* slot = d.hot + ((size_t)(s * d.L + g * d.R + lig) * d.C + v) * kSlotStride;
    for (int j = threadIdx.x; j < kRow; j += blockDim.x) slot[j] = 0xA5;
  }
}

hipError_t launch_poison(const DevState& d, hipStream_t st) {
  hipLaunchKernelGGL(k_poison, dim3(4096), dim3(64), 0, st, d);
  return hipGetLastError();
}
#endif

hipError_t launch_gather(const DevState& d, uint16_t* d_out, int32_t t, int32_t* d_trace,
                         hipStream_t st, StageEv ev) {
  // grid rows [0, miss_rows): the miss workgroups, dispatched first (their
  // PCIe reads have the longest latency); then bk_rows rows holding
  // kBkSlices bookkeeping workgroups per unit (one query row per round;
  // k_round does its own); then row miss_rows + bk_rows + sl: the hit rows of
  // layer sl
  const int gx = (d.K + kRowsPerRound - 1) / kRowsPerRound;
  const int units = d.S * d.G;
  const int bk_rows = d.Q == 1 ? (units * kBkSlices + gx - 1) / gx : 0;
  const int miss_rows = (kMissBlocks + gx - 1) / gx;
  const size_t words = bk_rows ? (size_t)(d.C + 31) / 32 : 0;
  const size_t lds = std::max((size_t)units + 1, words) * sizeof(int32_t);
  // without an output buffer only the miss workgroups run (they fill slots)
  const int rows = bk_rows + (d_out ? d.S * d.L * d.Q + miss_rows : miss_rows);
  // more than this many missing rows leaves fewer than kFewHitRows other rows
  const int64_t rows_total = (int64_t)d.S * d.L * d.Q * d.K;
  const int few_hits_above = (int)(rows_total - kFewHitRows);
  // grid rows stay below 2^16, as div_by requires: S * L * Q <= 60,000 is checked at creation
  hipExtLaunchKernelGGL(k_gather, dim3(gx, rows), dim3(kGatherThreads), (uint32_t)lds, st, ev.start,
                        ev.stop, 0, d, d_out, t, bk_rows, miss_rows, few_hits_above,
                        div_magic((uint32_t)d.Q), div_magic((uint32_t)d.L), div_magic((uint32_t)d.R),
                        d_trace);
  return hipGetLastError();
}

}  // namespace hc
