// hc_internal.h — device-side layout shared by the host orchestration and the
// gfx950 kernels of the hot-cache decode step.  Not part of the public ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hc.h"

namespace hc {

constexpr int kRow = HC_ROW_BYTES;        // 656 B per Q8G64 row
constexpr int kSlotStride = kRow;         // bytes between hot slots in HBM (padding measured: no gain)
constexpr int kOut = HC_OUT_ELEMS;        // 576 bf16 per gathered row
constexpr int kBin1Bits = 12;             // first radix digit: key bits [20, 32)
constexpr int kBins1 = 1 << kBin1Bits;    // 4096 histogram bins per unit
constexpr int kMaxSessions = HC_MAX_SESSIONS;  // session lengths travel as kernel args
constexpr int kMaxUnits = HC_MAX_UNITS;   // S * G: the per-unit miss prefix lives in LDS
// Score-scan segments per selection unit and step, at most: a segment is one
// scan workgroup's run of positions, whose candidates it writes in order.
constexpr int kMaxSegs = 4096;
// Kinds of inconsistent device state a kernel can report (DevState::err).
enum { kErrSelect = 0, kErrLru = 1, kErrRound = 2, kErrKinds = 4 };

// Per-selection-unit counters (int32 each): unit su owns cnt[su * kCntStride ..
// + kCnt), a 256-byte line of its own.  kCntWinLo / kCntWinHi: the cut window
// of the unit's next score scan, in units of the key's top 16 bits (-1 before
// the first step: every key); kCntMiss and kCntHand (circular / clock hand)
// are kept at su = u * Q.  kCntQHead / kCntQTail / kCntQBuf: the LRU queue of
// the unit (at su = u * Q); kCntFill: slots the unit's LRU has filled so far
// (slots [fill, C) were never used).  kCntCntStep: the step whose select
// launch marked the LRU queue's live entries for a compaction (-1: none),
// carried out by that step's gather launch; kCntCntTail, kCntCntBuf: the
// queue's tail and buffer then (one query row; see kBkSlices).
enum {
  kCntMiss = 2, kCntWinLo = 3, kCntHand = 4,
  kCntQHead = 5, kCntQTail = 6, kCntQBuf = 7, kCntFill = 8, kCntWinHi = 9, kCnt = 10,
  kCntCntStep = 16, kCntCntTail = 17, kCntCntBuf = 18
};
// LRU queue compaction (one query row): when a step's slots might not fit
// after the tail, kCountWGs extra workgroups per unit of the select launch
// mark the queue's live entries in a bitmap, and kBkSlices workgroups per
// unit of the gather launch each write the survivors of one slice of the
// queue to their final places, found by counting the bitmap's bits before the
// slice, without waiting for one another.  Ranges are whole multiples of 64
// entries, so that each owns whole words of the bitmap.
constexpr int kCountWGs = 4;
constexpr int kBkSlices = 16;
// Half-width of the predicted cut window, in top-16-bit key units: the next
// step's window is the current cut key's 16-bit prefix +- kWinHalf (about
// +-0.06 around a cut near 2 or 3, several times the cut's movement between
// decode steps; a cut that leaves it costs a rescan of the scores).
constexpr int kWinHalf = 8;
constexpr int kCntStride = 64;
static_assert(kCntCntBuf < kCntStride, "the compaction's words fit the counter line");

// One entry of a unit's score scan: the totalOrder key of a score, its
// position, and (one query row) the slot holding that position at the scan,
// -1 for none or a ring row.  12 bytes: one load brings all three.
struct Ent {
  uint32_t key;
  uint32_t pos;
  int32_t slot;
};

// Device view of the caller's workspace.  Unit u = s * G + g; layer index
// sl = s * L + l.  All arrays are carved from one allocation (see hc_ctx.hip).
struct DevState {
  int32_t S, L, R, G, K, C;
  int32_t Q;           // query rows per round; selection unit su = u * Q + q
  int64_t hcap;
  int32_t* pos2slot;   // [U][hcap]  slot holding a position, -1 if none
  int32_t* slot2pos;   // [U][C]     position held by a slot, -1 if empty
  int32_t* last_use;   // [U][C]     step of the slot's last use, -1 if never
  int2* oq;            // [U][2][qcap] LRU queue of (slot, step) in ascending (step, slot)
                       //            over the used slots; an entry is live while
                       //            last_use[slot] == step
  int32_t qcap;        // entries per queue buffer: 2 C rounded up to a multiple of 4
  uint32_t* qlive;     // [U][qlive_words] LRU, one query row: bit j, entry j of the queue
                       //            live when the select launch marked it for a compaction
  int32_t qlive_words; // words per unit: 2 ceil(qcap / 64)
  int32_t* cnt;        // [U*Q][kCntStride] per selection unit; the round's miss count at su = u*Q
  Ent* cand;           // [U*Q][hcap] entries: the scores above or inside the cut
                       //            window, segment s of a step at s * seg_len,
                       //            ascending positions
  int2* seg;           // [U*Q][max_segs] (entries, of which above the window) per segment
  int32_t max_segs;    // segments per unit a step may use
  uint32_t* err;       // [kErrKinds] device-visible pinned host words: nonzero once a
                       //            kernel found an inconsistent state (kErr*)
  int32_t* sel_slot;   // [U*Q][K]   source of selected row i: slot, C + ring entry,
                       //            -(slot + 1) if it missed and this row fills the slot,
                       //            -(C + 1 + position) for a further row of that miss
  int32_t* miss_pos;   // [U][Q*K]   position of miss k (ascending), k < cnt[u*Q][kCntMiss]
  int32_t* victim;     // [U][Q*K]   slot that miss k fills
  int32_t* miss_idx;   // [U][Q*K]   output row (q * K + i) that miss k fills
  int32_t* miss_old;   // [U][Q*K]   position victim k held before this step, -1 if empty
                       //            (one query row: applied to the maps by the gather)
  const uint8_t* const* host;  // [S*L] device-visible pointers of the pinned host rows
  uint8_t* hot;        // [S*L][C][kSlotStride], a row in the first 656 B of its slot
  uint8_t* ring;       // [S*L][ring_rows][kRow] recent ring; position p at p % ring_rows
  int32_t ring_rows;   // 0: no ring
  int32_t policy;      // HC_REPLACE_LRU, HC_REPLACE_CIRCULAR or HC_REPLACE_CLOCK
  uint32_t* refbits;   // [U][ceil(C / 32)] clock reference bits
#ifdef HC_TEST_HOOKS
  int32_t test_force;  // test build only: the select kernels report an inconsistent state
#endif
};

struct StepArgs {
  int32_t t;                          // step number (last-use stamp)
  uint32_t hist_len[kMaxSessions];    // positions per session this step
  uint32_t ring_lo[kMaxSessions];     // positions >= ring_lo[s] are read from the ring
};

constexpr uint32_t kNoRing = 0xFFFFFFFFu;  // ring_lo / append slot of a session without one

// hc_append: ring entry written for each session (kNoRing: none).
struct AppendArgs {
  uint32_t entry[kMaxSessions];
};

// Copyback: session s copies positions [lo[s], hi[s]) (empty when equal).
struct CopybackArgs {
  uint32_t lo[kMaxSessions];
  uint32_t hi[kMaxSessions];
  uint32_t max_rows;                  // max_s hi[s] - lo[s]
};

// 16-byte vector usable with the nontemporal load/store builtins.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (nearest, ties to even), lo in the low half, as
// one packed conversion: converting them one at a time made the compiler pack
// each with a dummy and merge the halves with two more instructions.
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2v));
}

// Global-memory views of row pointers (hot slots, ring, pinned host rows
// mapped for the device).  Loads through them compile to global loads; through
// a pointer fetched from a table the compiler emits flat loads, which also
// count against the LDS counter and so hold up every later LDS wait.
typedef const __attribute__((address_space(1))) uint8_t gbyte;
__device__ __forceinline__ gbyte* to_global(const uint8_t* p) { return (gbyte*)p; }
template <class T>
__device__ __forceinline__ T gload(gbyte* p) {
  return *reinterpret_cast<const __attribute__((address_space(1))) T*>(p);
}

// Wave-level steps through DPP lane moves (register to register, no LDS round
// trip as __shfl's ds_bpermute takes).  DPP controls: quad_perm [1,0,3,2]
// 0xB1 and [2,3,0,1] 0x4E (partner lane ^1, ^2), row_shr:n 0x110 + n (lane
// - n within a row of 16), row_mirror 0x140 (lane 15 - l of the row),
// row_half_mirror 0x141 (lane 7 - l of each half row), row_bcast:15 0x142
// (lane 15 of each row to the next row), row_bcast:31 0x143 (lane 31 to rows
// 2 and 3).  Lanes whose move has no source are excluded by the conditions.
template <int kCtrl>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_mov_dpp(x, kCtrl, 0xf, 0xf, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, dpp_i<kCtrl>(__builtin_bit_cast(int, x)));
}

// Inclusive prefix sum over the 64 lanes of the wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  int t;
  t = dpp_i<0x111>(x); if (r >= 1) x += t;
  t = dpp_i<0x112>(x); if (r >= 2) x += t;
  t = dpp_i<0x114>(x); if (r >= 4) x += t;
  t = dpp_i<0x118>(x); if (r >= 8) x += t;
  t = dpp_i<0x142>(x); if (lane & 16) x += t;
  t = dpp_i<0x143>(x); if (lane >= 32) x += t;
  return x;
}

// Sum / maximum over each row of 16 lanes, left in every lane of the row.
// Each level combines a lane with the lane holding the other half of the
// partial (^1, ^2, the other quad of the half row, the other half row), the
// same pairs as a butterfly over lane ^1, ^2, ^4, ^8, so every lane gets the
// same bits.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x141>(x);
  x += dpp_f<0x140>(x);
  return x;
}
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return x;
}

// Maximum over the 64 lanes (all active), returned as a wave-uniform value.
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, dpp_i<0xB1>(x));
  x = max(x, dpp_i<0x4E>(x));
  x = max(x, dpp_i<0x141>(x));
  x = max(x, dpp_i<0x140>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// IEEE-754 totalOrder of a float as an unsigned integer key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}

// Cut window of a unit's score scan, [lo, hi] in top-16-bit key units: as
// stored, or every key when there is none yet (also for values out of range).
// The scan and the select kernel must agree on it exactly.
__device__ __forceinline__ void cut_window(int lo16, int hi16, uint32_t& lo, uint32_t& hi) {
  if (lo16 < 0 || hi16 < lo16 || hi16 > 65535) {
    lo = 0;
    hi = 65535;
  } else {
    lo = (uint32_t)lo16;
    hi = (uint32_t)hi16;
  }
}

// n / D for 0 <= n < 2^16 by a multiply: m = ceil(2^32 / D), 0 meaning D = 1.
// Exact because n * (m * D - 2^32) < 2^16 * D <= 2^32 for D <= 2^16.
__device__ __forceinline__ int div_by(int n, uint32_t m) {
  return m ? (int)__umulhi((uint32_t)n, m) : n;
}

__host__ __forceinline__ uint32_t div_magic(uint32_t D) {
  return D == 1 ? 0u : (uint32_t)(((1ull << 32) + D - 1) / D);
}

// Records an inconsistent device state of kind `kind` (kErr*); the host
// reports it at its next check of the context (HC_E_DEVICE).
__device__ __forceinline__ void report_error(const DevState& d, int kind) {
  d.err[kind] = 1u;
}

// Timing of a stage's kernels: `start` is attached to the stage's first
// dispatch and `stop` to its last (hipExtLaunchKernel records them when the
// kernel itself begins and ends, so no separate event sits between kernels);
// null events: an ordinary launch.
struct StageEv {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Launchers (each defined next to its kernel).  All return hipGetLastError().
hipError_t launch_init(const DevState& d, hipStream_t st);
// Positions per score-scan segment for a step whose longest history is max_len
// (the scan and the select kernel must use the same).
int64_t scan_seg_len(int64_t max_len, int max_segs);
hipError_t launch_topk_scan(const DevState& d, const StepArgs& a, const float* scores,
                            uint64_t stride, int64_t max_len, bool vec4, hipStream_t st,
                            StageEv ev = {});
// First step only (needs hcap >= kColdMinPositions): sets every selection
// unit's cut bin from a histogram of its scores.
constexpr int64_t kColdMinPositions = 2048;   // the histogram borrows 16 KB of `cand`
hipError_t launch_cold_cut(const DevState& d, const StepArgs& a, const float* scores,
                           uint64_t stride, int64_t max_len, hipStream_t st, StageEv ev = {});
// Q == 1: the fused per-unit selection + cache kernel.  Q > 1: the top-K part
// per selection unit, then launch_round per unit.
hipError_t launch_select(const DevState& d, const StepArgs& a, const float* scores,
                         uint64_t stride, int64_t max_len, int32_t* d_sel, int32_t* d_trace,
                         hipStream_t st, StageEv ev = {});
hipError_t launch_round(const DevState& d, const StepArgs& a, const int32_t* d_sel,
                        int32_t* d_trace, hipStream_t st, StageEv ev = {});
// d_out == nullptr: only the missing rows are fetched into their slots.  With
// one query row the launch also carries one bookkeeping workgroup per unit:
// last-use stamps, the (miss, victim) pairs applied to the slot maps, and the
// LRU queue's new entries for step t.  d_trace (or nullptr): the step's trace,
// whose movement counts (rows read from host RAM and from HBM, slot fills,
// output rows) the gather adds after the select has zeroed them.
hipError_t launch_gather(const DevState& d, uint16_t* d_out, int32_t t, int32_t* d_trace,
                         hipStream_t st, StageEv ev = {});
#ifdef HC_TEST_HOOKS
// Test build: a sentinel over every victim slot before the gather fills it.
hipError_t launch_poison(const DevState& d, hipStream_t st);
#endif
hipError_t launch_append(const DevState& d, const AppendArgs& a, const uint8_t* d_rows,
                         hipStream_t st);
// Attention over the last step's selection: rows from the gathered bf16
// buffer, or (from_slots) straight from the slots / ring / host RAM.
uint64_t attend_work_bytes(const DevState& d, int heads);
hipError_t launch_attend(const DevState& d, bool from_slots, const uint16_t* q, int heads,
                         float scale, const uint16_t* rows, void* work, float* out,
                         hipStream_t st);
// Copies the rows and then writes hi[s] into host_count[s] (device pointer of
// pinned host memory) for every session with rows to copy.
hipError_t launch_copyback(const DevState& d, const CopybackArgs& a, uint64_t* host_count,
                           hipStream_t st);

}  // namespace hc
