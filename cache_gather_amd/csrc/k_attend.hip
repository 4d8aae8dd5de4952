// k_attend.hip — MLA decode attention over the selected rows (gfx950 MFMA).
//
// Page "From 1M Total to 15+ × 1M Contexts: GLM-5.3 KV Cache Offloading",
// section "Decision three: let the GPU manage the hot cache directly" and its
// data-flow figure: the compact selection feeds GPU attention.  Absorbed MLA
// decode: for each head, z_i = scale * <q, row_i> over the 576 values of each
// selected row (512 latent + 64 RoPE), softmax over the K rows, and the output
// is the weighted sum of the rows' 512 latent values (fp32).
//
// Two sources of rows, one kernel:
//   * kFromBuffer: the bf16 rows the gather wrote ([S][L][Q][K][576]);
//   * kFromSlots: the rows straight from the hot slots, the recent ring, or
//     host RAM (a further query row of a miss), dequantised while they are
//     staged — the gather then only fills the missing slots and the bf16
//     buffer is never written.  The staged values are the same bf16 numbers
//     either way, so both sources give the same result bit for bit.
//
// Workgroup = (split of up to 1,024 rows of one (session, layer, query row),
// 64-head group): 8 wave64 in pairs.  Wave w serves head tile w % 4 (16 heads) and
// half w / 4: for Q.K^T the half of the 576 values it multiplies, for P.V the
// half of the 512 output values it accumulates — so a wave keeps 9 query
// fragments and 16 x 256 fp32 accumulators, and two waves fit on each SIMD.
// Per 64-row sub-chunk the rows are staged once in LDS, row-major (dequantised
// while staging for the slot source), and each wave runs
// v_mfma_f32_16x16x32_bf16: its half of Q.K^T in 9 k-steps x 4 row tiles; the
// pair adds its two partial scores through LDS (fp32 addition commutes, so
// both waves hold the same sums); online softmax in fp32 (each lane holds 4
// heads of one row per tile), in base-2 units: both waves of a pair test all
// 64 rows against each head's reference maximum (reducing over the 16 lanes
// of a head only when it must rise), and each computes the weights of its own
// 32 rows (half 0 rows 0-31, half 1 rows 32-63) and keeps their running sum
// per lane;
// P rounded to bf16 through LDS; P.V in 2 k-steps x 16 dim tiles, its B
// operand read from the row-major rows with the gfx950 transposing LDS load
// (ds_read_b64_tr_b16: within each 16-lane group, lane j receives value j % 4
// of what lane 4k + j / 4 addressed, so four lanes addressing four
// consecutive rows give every lane four consecutive rows of one column).
// LDS bank layout (64 banks of 4 bytes; measured with the LDS bank-conflict
// counter): rows are 1,184 B apart, at which the Q.K^T operand reads (16 rows,
// one 16-byte column) are conflict-free, where the 1,168-B stride served them
// in two passes.  A transposing load serves 32 lanes per pass, which must
// touch eight rows in distinct 32-byte bank blocks; at this stride rows with
// distinct residues mod 8 do.  So the k slots of a 32-row k-step are not in
// row order: slots 8g..8g+7 of lane group g hold rows 4g..4g+3 and
// 16+4g..16+4g+3 (the summation order of P.V is free, and P is stored in the
// same slot order).  The reference maximum of a head is raised only when a
// sub-chunk's maximum exceeds it by more than kLazy (weights at most
// 2^kLazy, far inside the bf16 and fp32 range), so after the first sub-chunk
// the 64 accumulators of a wave are seldom rescaled.  Each split writes
// (reference maximum, the two halves' sums, unnormalised output) per head; a
// second kernel merges the splits.
#include "hc_internal.h"

namespace hc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr int kAttThreads = 512;                  // 8 wave64
constexpr int kHeadsPerGroup = 64;                // 4 tiles of 16
constexpr int kMaxSplitRows = 1024;              // rows per workgroup, at most
constexpr int kResident = 256;                    // workgroups the chip runs at once (1 per CU)
constexpr int kSub = 64;                          // rows per LDS sub-chunk
constexpr int kRowLd = HC_OUT_ELEMS + 16;         // 592 bf16 = 1,184 B: padded row-major row
constexpr int kPLd = kSub + 8;
constexpr int kPartStride = 516;                  // floats per (head) partial: 512 + m + l0 + l1 + pad
static_assert(kPartStride % 4 == 0, "partials stay 16-byte aligned");
constexpr int kHalfK = HC_OUT_ELEMS / 32 / 2;     // 9 Q.K^T k-steps per half
constexpr int kDimTiles = 512 / 2 / 16;           // 16 P.V dim tiles per half
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedVmemRead = 0x020;
constexpr float kLazy = 8.f;                      // base-2 headroom of the reference maximum
constexpr float kLog2e = 1.4426950408889634f;

enum { kFromBuffer = 0, kFromSlots = 1 };

struct AttShared {
  alignas(16) __bf16 rows[kSub * kRowLd];         // 75,776 B
  alignas(16) f32x4 sx[8 * 4 * 64];               // 32,768 B: partial scores [wave][n][lane]
  alignas(16) __bf16 p[4 * 16 * kPLd];            //  9,216 B: weights [head tile][head][row]
  const uint8_t* src[kMaxSplitRows];              //  8,192 B: slot source of each row
};

__device__ __forceinline__ float i8f(uint32_t w, int k) {
  return (float)((int32_t)(w << (24 - 8 * k)) >> 24);
}

// Source row of selected row i of (sl, su): the gather's slot encoding.
__device__ __forceinline__ const uint8_t* slot_row(const DevState& d, int64_t sl, int32_t enc) {
  if (enc >= d.C) return d.ring + ((size_t)sl * d.ring_rows + (enc - d.C)) * kRow;
  if (enc >= 0) return d.hot + ((size_t)sl * d.C + enc) * kSlotStride;
  if (enc >= -d.C) return d.hot + ((size_t)sl * d.C + (-enc - 1)) * kSlotStride;  // filled
  return d.host[sl] + (size_t)(-(int64_t)enc - d.C - 1) * kRow;                     // host RAM
}

// 8 int8 latent values times an fp16 scale (low 16 bits of hs), as bf16.
__device__ __forceinline__ u32x4 dequant8(const uint2& qq, uint32_t hs) {
  const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(hs & 0xFFFFu));
  u32x4 w;
  w.x = bf16x2_rne(i8f(qq.x, 0) * sc, i8f(qq.x, 1) * sc);
  w.y = bf16x2_rne(i8f(qq.x, 2) * sc, i8f(qq.x, 3) * sc);
  w.z = bf16x2_rne(i8f(qq.y, 0) * sc, i8f(qq.y, 1) * sc);
  w.w = bf16x2_rne(i8f(qq.y, 2) * sc, i8f(qq.y, 3) * sc);
  return w;
}

// Four consecutive bf16 of LDS per lane, transposed across each 16-lane group.
__device__ __forceinline__ i16x4 lds_tr4(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
}

template <int SRC>
__global__ __launch_bounds__(kAttThreads) void k_attend(DevState d, const uint16_t* __restrict__ q,
                                                        int heads, float scale, int split_rows,
                                                        const uint16_t* __restrict__ rows_buf,
                                                        float* __restrict__ part) {
  __shared__ AttShared sh;
  const int split = blockIdx.x, hg = blockIdx.y, slq = blockIdx.z;  // slq = sl * Q + qi
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ht = wave & 3, half = wave >> 2;
  const int K = d.K, Q = d.Q;
  const int sl = slq / Q, qi = slq - sl * Q;
  const int s = sl / d.L, l = sl - s * d.L;
  const int32_t* enc_row = d.sel_slot + ((size_t)(s * d.G + l / d.R) * Q + qi) * K;
  const int r_begin = split * split_rows;
  const int r_end = min(K, r_begin + split_rows);
  // this lane's query fragments: head row lane % 16 of the tile, this half's k
  const int head0 = hg * kHeadsPerGroup + ht * 16;
  const uint16_t* qrow = q + ((size_t)slq * heads + head0 + (lane & 15)) * HC_OUT_ELEMS +
                         32 * kHalfK * half + 8 * (lane >> 4);
  bf16x8 qa[kHalfK];
#pragma unroll
  for (int ks = 0; ks < kHalfK; ++ks)
    qa[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * ks));

  f32x4 o[kDimTiles];
#pragma unroll
  for (int n = 0; n < kDimTiles; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  // per head i of this lane: the reference maximum (base 2, scaled), and the
  // running sum of this lane's weights (its row of each of the wave's own tiles)
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }
  const float scale2 = scale * kLog2e;

  // staging: thread tid handles row rr = tid / 8 of a sub-chunk and chunks
  // cc, cc + 8, ..., cc + 64 of 8 values (cc = tid % 8): 8 latent chunks, chunk
  // k in scale group k, and one RoPE chunk.  Eight consecutive lanes cover 128
  // contiguous bytes of a row.  Software pipeline: the raw loads of sub-chunk
  // j + 1 are issued during the matrix work of sub-chunk j.
  const int nsub = (r_end - r_begin + kSub - 1) / kSub;
  constexpr int kLat = 8;
  const int rr = tid >> 3, cc = tid & 7;
  if (SRC == kFromSlots) {
    for (int r = tid; r < r_end - r_begin; r += kAttThreads)
      sh.src[r] = slot_row(d, sl, enc_row[r_begin + r]);
    __syncthreads();
  }
  u32x4 bv[kLat + 1];                              // buffer source: 9 chunks of 16 B
  uint2 q8[kLat];                                  // slot source: 8 latent chunks of 8 B
  u32x4 rope, scb;                                 // slot source: RoPE chunk, scale block
  // Branch-free, so the loads can be interleaved with the matrix work: a row
  // past the split reads the split's last row instead, and staging stores
  // zeros for it.
  auto fetch = [&](int j) {
    const int r = min(r_begin + j * kSub + rr, r_end - 1);
    if (SRC == kFromBuffer) {
      // non-temporal: the buffer is read once, and normal loads would allocate
      // it in the Infinity Cache over the hot slots the next step reads again
      const uint16_t* base = rows_buf + ((size_t)slq * K + r) * HC_OUT_ELEMS + 8 * cc;
#pragma unroll
      for (int k = 0; k <= kLat; ++k)
        bv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 64 * k));
    } else {
      gbyte* src = to_global(sh.src[r - r_begin]);
#pragma unroll
      for (int k = 0; k < kLat; ++k) {
        const u32x2 w = gload<u32x2>(src + 8 * (cc + 8 * k));
        q8[k] = uint2{w.x, w.y};
      }
      rope = gload<u32x4>(src + HC_ROPE_OFFSET + 16 * cc);
      scb = gload<u32x4>(src + HC_SCALE_OFFSET);
    }
  };
  auto chunk = [&](int k) -> u32x4 {
    if (SRC == kFromBuffer) return bv[k];
    if (k == kLat) return rope;
    const uint32_t sw = (k >> 1) == 0 ? scb.x : (k >> 1) == 1 ? scb.y : (k >> 1) == 2 ? scb.z : scb.w;
    return dequant8(q8[k], (k & 1) ? (sw >> 16) : sw);
  };

  fetch(0);
  for (int j = 0; j < nsub; ++j) {
    const int nvalid = min(kSub, r_end - (r_begin + j * kSub));
    __syncthreads();   // the previous sub-chunk's matrix work is done with LDS
    if (nvalid == kSub) {
#pragma unroll
      for (int k = 0; k <= kLat; ++k)
        *reinterpret_cast<u32x4*>(&sh.rows[rr * kRowLd + 8 * (cc + 8 * k)]) = chunk(k);
    } else {   // the split's ragged last sub-chunk
      const bool vr = rr < nvalid;
#pragma unroll
      for (int k = 0; k <= kLat; ++k)
        *reinterpret_cast<u32x4*>(&sh.rows[rr * kRowLd + 8 * (cc + 8 * k)]) =
            vr ? chunk(k) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // the next sub-chunk's loads, in flight during this one's matrix work (the
    // last sub-chunk requests itself again rather than branch)
    fetch(min(j + 1, nsub - 1));

    // ---- this wave's half of S = Q K^T: 16 heads x 64 rows ----------------
    // slot t holds row tile t ^ (2 * half): the wave's own two tiles (those
    // it exponentiates) come first
    f32x4 sacc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) sacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kHalfK; ++ks) {
      const int kk = kHalfK * half + ks;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(
            &sh.rows[(16 * (n ^ (2 * half)) + (lane & 15)) * kRowLd + 32 * kk + 8 * (lane >> 4)]);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], b, sacc[n], 0, 0, 0);
      }
    }
    // schedule: six operand reads ahead of the matrix instructions, then one
    // read per matrix instruction, so the LDS latency is not waited out 18 times
    // The next sub-chunk's global loads go one per matrix instruction: issued
    // in a burst they held the address unit ahead of the operand reads.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 6, 0);
#pragma unroll
    for (int k = 0; k < 4 * kHalfK - 6; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      if (k < kLat + 2) __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 6, 0);
    // ---- the pair's two halves added through LDS ----------------------------
#pragma unroll
    for (int n = 0; n < 4; ++n) sh.sx[(wave * 4 + (n ^ (2 * half))) * 64 + lane] = sacc[n];
    __syncthreads();
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const f32x4 other = sh.sx[((wave ^ 4) * 4 + (n ^ (2 * half))) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[n][i] += other[i];
    }

    // ---- online softmax: in slot n a lane holds heads 4*(lane/16)+i of row
    // 16 * (n ^ (2 * half)) + lane%16
    // A head's maximum over the 64 rows is needed only when it exceeds the
    // reference by more than kLazy, and some lane's own maximum then does too:
    // the 16-lane reduction runs only in that (rare) branch.
    float mx[4];
    bool grow = false;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = -INFINITY;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bool ok = 16 * (n ^ (2 * half)) + (lane & 15) < nvalid;
        sacc[n][i] = ok ? sacc[n][i] * scale2 : -INFINITY;
        mx[i] = fmaxf(mx[i], sacc[n][i]);
      }
      grow |= mx[i] > m_run[i] + kLazy;
    }
    // both waves of the pair hold the same scores, so they take this branch
    // together and keep the same reference maxima
    if (__ballot(grow) != 0) {
      float factor[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float m_new = fmaxf(m_run[i], row16_max(mx[i]));
        factor[i] = m_run[i] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
        l_run[i] *= factor[i];
        m_run[i] = m_new;
      }
#pragma unroll
      for (int n = 0; n < kDimTiles; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[n][i] *= factor[i];
    }
    // P (bf16) of this wave's own 32 rows to LDS as [head][k slot]: row r of
    // a 32-row k-step sits in slot 8 * ((r % 16) / 4) + r % 4 + 4 * (r / 16)
    __bf16* pw = sh.p + ht * 16 * kPLd;
    const int kslot = 8 * ((lane & 15) >> 2) + (lane & 3);
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      const f32x4 z = sacc[nn];
      const int n = 2 * half + nn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pv = __builtin_amdgcn_exp2f(z[i] - m_run[i]);   // 0 for a masked row
        l_run[i] += pv;
        pw[(4 * (lane >> 4) + i) * kPLd + 32 * (n >> 1) + 4 * (n & 1) + kslot] = (__bf16)pv;
      }
    }
    __syncthreads();
    // ---- O[:, this half] += P V -------------------------------------------
    const int grp = lane >> 4, gl = lane & 15;
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&pw[gl * kPLd + 32 * ks + 8 * grp]);
      const __bf16* vb = &sh.rows[(32 * ks + 4 * grp + (gl >> 2)) * kRowLd + 256 * half + 4 * (gl & 3)];
#pragma unroll
      for (int n = 0; n < kDimTiles; ++n) {
        const i16x4 lo = lds_tr4(vb + 16 * n);
        const i16x4 hi = lds_tr4(vb + 16 * kRowLd + 16 * n);
        const i16x8 v8 = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, v8), o[n],
                                                      0, 0, 0);
      }
    }
    // schedule: the P fragment and four tiles' operands read ahead, then two
    // reads per matrix instruction
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 10, 0);
#pragma unroll
    for (int k = 0; k < kSub / 32 * kDimTiles - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
  }

  // ---- this split's partial: unnormalised output, reference maximum, and
  // the sums of the two halves' rows per head
  const int nsplit = gridDim.x;
  float* base = part + (((size_t)slq * gridDim.y + hg) * nsplit + split) * kHeadsPerGroup * kPartStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = ht * 16 + 4 * (lane >> 4) + i;
    float* ph = base + (size_t)h * kPartStride;
    const float lsum = row16_sum(l_run[i]);
#pragma unroll
    for (int n = 0; n < kDimTiles; ++n) ph[256 * half + 16 * n + (lane & 15)] = o[n][i];
    if ((lane & 15) == 0) {
      if (half == 0) ph[512] = m_run[i];
      ph[513 + half] = lsum;
    }
  }
}

// Merges the splits of four heads of one slq: out = sum_c 2^(m_c - M) O_c /
// sum_c 2^(m_c - M) (l0_c + l1_c), maxima in base-2 units.  128 threads per head, four output values each
// (16-byte loads and stores; a partial's 516-float stride keeps them aligned).
// NS > 0: exactly NS splits, whose loads all go out in one round; NS = 0: any
// number, maxima first.  Both add the splits in the same order.
constexpr int kMergeHeads = 4;
template <int NS>
__global__ __launch_bounds__(512) void k_attend_merge(const float* __restrict__ part, int heads,
                                                      int nsplit, float* __restrict__ out) {
  const int h = blockIdx.x * kMergeHeads + (threadIdx.x >> 7), slq = blockIdx.y;
  const int dd = 4 * (threadIdx.x & 127);
  const int hg = h / kHeadsPerGroup, hh = h - hg * kHeadsPerGroup;
  const int ngroups = heads / kHeadsPerGroup;
  const float* base = part + (((size_t)slq * ngroups + hg) * nsplit) * kHeadsPerGroup * kPartStride +
                      (size_t)hh * kPartStride;
  const size_t cstride = (size_t)kHeadsPerGroup * kPartStride;
  float M = -INFINITY;
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float mc, float lc, const float4& o) {
    const float w = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
    L += w * lc;
    acc.x += w * o.x;
    acc.y += w * o.y;
    acc.z += w * o.z;
    acc.w += w * o.w;
  };
  if (NS > 0) {
    float mc[NS > 0 ? NS : 1], lc[NS > 0 ? NS : 1];
    float4 oc[NS > 0 ? NS : 1];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      mc[c] = base[c * cstride + 512];
      lc[c] = base[c * cstride + 513] + base[c * cstride + 514];
      oc[c] = *reinterpret_cast<const float4*>(base + c * cstride + dd);
    }
#pragma unroll
    for (int c = 0; c < NS; ++c) M = fmaxf(M, mc[c]);
#pragma unroll
    for (int c = 0; c < NS; ++c) add(mc[c], lc[c], oc[c]);
  } else {
    for (int c = 0; c < nsplit; ++c) M = fmaxf(M, base[c * cstride + 512]);
    for (int c = 0; c < nsplit; ++c)
      add(base[c * cstride + 512], base[c * cstride + 513] + base[c * cstride + 514],
          *reinterpret_cast<const float4*>(base + c * cstride + dd));
  }
  *reinterpret_cast<float4*>(out + ((size_t)slq * heads + h) * 512 + dd) =
      make_float4(acc.x / L, acc.y / L, acc.z / L, acc.w / L);
}

// Splits of the K rows: as few as fill the chip in the fewest rounds.  The
// cost of a choice is (rounds of resident workgroups) x (sub-chunks per split
// + about one sub-chunk of fixed work per workgroup); ties go to fewer splits,
// which also means fewer partials to merge.
struct AttSplit {
  int nsplit, rows;
};

AttSplit attend_split(const DevState& d, int heads) {
  const int64_t units = (int64_t)d.S * d.L * d.Q * (heads / kHeadsPerGroup);
  AttSplit best{0, 0};
  double best_cost = 0.0;
  const int max_split = (d.K + kSub - 1) / kSub;
  for (int ns = (d.K + kMaxSplitRows - 1) / kMaxSplitRows; ns <= max_split; ++ns) {
    const int rows = ((d.K + ns - 1) / ns + kSub - 1) / kSub * kSub;
    const int n = (d.K + rows - 1) / rows;
    if (n != ns) continue;
    const int64_t rounds = (units * n + kResident - 1) / kResident;
    const double cost = (double)rounds * (rows / kSub + 1.2);
    if (best.nsplit == 0 || cost < best_cost - 1e-9) {
      best = AttSplit{n, rows};
      best_cost = cost;
    }
  }
  return best;
}

uint64_t attend_work_bytes(const DevState& d, int heads) {
  const uint64_t nsplit = attend_split(d, heads).nsplit;
  return (uint64_t)d.S * d.L * d.Q * (heads / kHeadsPerGroup) * nsplit * kHeadsPerGroup *
         kPartStride * sizeof(float);
}

hipError_t launch_attend(const DevState& d, bool from_slots, const uint16_t* q, int heads,
                         float scale, const uint16_t* rows, void* work, float* out,
                         hipStream_t st) {
  const AttSplit sp = attend_split(d, heads);
  dim3 grid(sp.nsplit, heads / kHeadsPerGroup, d.S * d.L * d.Q);
  float* part = static_cast<float*>(work);
  if (from_slots)
    hipLaunchKernelGGL(k_attend<kFromSlots>, grid, dim3(kAttThreads), 0, st, d, q, heads, scale,
                       sp.rows, rows, part);
  else
    hipLaunchKernelGGL(k_attend<kFromBuffer>, grid, dim3(kAttThreads), 0, st, d, q, heads, scale,
                       sp.rows, rows, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 mgrid(heads / kMergeHeads, d.S * d.L * d.Q);
  switch (sp.nsplit) {
    case 1: hipLaunchKernelGGL(k_attend_merge<1>, mgrid, dim3(512), 0, st, part, heads, 1, out); break;
    case 2: hipLaunchKernelGGL(k_attend_merge<2>, mgrid, dim3(512), 0, st, part, heads, 2, out); break;
    case 3: hipLaunchKernelGGL(k_attend_merge<3>, mgrid, dim3(512), 0, st, part, heads, 3, out); break;
    case 4: hipLaunchKernelGGL(k_attend_merge<4>, mgrid, dim3(512), 0, st, part, heads, 4, out); break;
    default:
      hipLaunchKernelGGL(k_attend_merge<0>, mgrid, dim3(512), 0, st, part, heads, sp.nsplit, out);
  }
  return hipGetLastError();
}

}  // namespace hc
