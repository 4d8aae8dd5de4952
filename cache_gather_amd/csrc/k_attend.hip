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
// Workgroup = (256-row split of one (session, layer, query row), 64-head
// group): 4 wave64, 16 heads each.  Per 64-row sub-chunk the rows are staged
// in LDS twice — row-major (the B operand of Q.K^T over 576 values) and the
// latent part transposed (the B operand of P.V) — and each wave runs
// v_mfma_f32_16x16x32_bf16: Q.K^T in 18 k-steps x 4 row tiles, online softmax
// in fp32 (each lane holds 4 heads of one row per tile), P rounded to bf16
// through LDS, P.V in 2 k-steps x 32 dim tiles accumulating 16 x 512 fp32 per
// wave.  Each split writes (max, sum, unnormalised output) per head; a second
// kernel merges the splits.
#include "hc_internal.h"

namespace hc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttThreads = 256;                  // 4 wave64
constexpr int kHeadsPerGroup = 64;                // 16 per wave
constexpr int kSplitRows = 256;                   // rows per workgroup
constexpr int kSub = 64;                          // rows per LDS sub-chunk
constexpr int kRowLd = HC_OUT_ELEMS + 8;          // 584 bf16: padded row-major row
constexpr int kVtLd = kSub + 8;                   // 72 bf16: padded transposed row
constexpr int kPLd = kSub + 8;
constexpr int kPartStride = 516;                  // floats per (head) partial: 512 + m + l + pad

enum { kFromBuffer = 0, kFromSlots = 1 };

struct AttShared {
  alignas(16) __bf16 rows[kSub * kRowLd];         // 74,752 B
  alignas(16) __bf16 vt[512 * kVtLd];             // 73,728 B
  alignas(16) __bf16 p[4 * 16 * kPLd];            //  9,216 B
};

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

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

// 8 int8 latent values times fp16 scale g of the row's scale block, as bf16.
__device__ __forceinline__ u32x4 dequant8(const uint2& qq, const u32x4& sblk, int g) {
  const uint32_t sw = (g >> 1) == 0 ? sblk.x : (g >> 1) == 1 ? sblk.y : (g >> 1) == 2 ? sblk.z : sblk.w;
  const uint16_t hs = (uint16_t)((g & 1) ? (sw >> 16) : (sw & 0xFFFFu));
  const float sc = (float)__builtin_bit_cast(_Float16, hs);
  u32x4 w;
  w.x = bf16x2_rne(i8f(qq.x, 0) * sc, i8f(qq.x, 1) * sc);
  w.y = bf16x2_rne(i8f(qq.x, 2) * sc, i8f(qq.x, 3) * sc);
  w.z = bf16x2_rne(i8f(qq.y, 0) * sc, i8f(qq.y, 1) * sc);
  w.w = bf16x2_rne(i8f(qq.y, 2) * sc, i8f(qq.y, 3) * sc);
  return w;
}

template <int SRC>
__global__ __launch_bounds__(kAttThreads) void k_attend(DevState d, const uint16_t* __restrict__ q,
                                                        int heads, float scale,
                                                        const uint16_t* __restrict__ rows_buf,
                                                        float* __restrict__ part) {
  __shared__ AttShared sh;
  const int split = blockIdx.x, hg = blockIdx.y, slq = blockIdx.z;  // slq = sl * Q + qi
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = d.K, Q = d.Q;
  const int sl = slq / Q, qi = slq - sl * Q;
  const int s = sl / d.L, l = sl - s * d.L;
  const int32_t* enc_row = d.sel_slot + ((size_t)(s * d.G + l / d.R) * Q + qi) * K;
  const int r_begin = split * kSplitRows;
  const int r_end = min(K, r_begin + kSplitRows);
  // this lane's query fragment base: head row lane % 16 of the wave's 16
  const int head0 = hg * kHeadsPerGroup + wave * 16;
  const uint16_t* qrow = q + ((size_t)slq * heads + head0 + (lane & 15)) * HC_OUT_ELEMS +
                         8 * (lane >> 4);

  f32x4 o[32];
#pragma unroll
  for (int n = 0; n < 32; ++n) o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }

  // the 18 query fragments of this lane (A operands of Q.K^T), kept in registers
  bf16x8 qa[HC_OUT_ELEMS / 32];
#pragma unroll
  for (int ks = 0; ks < HC_OUT_ELEMS / 32; ++ks)
    qa[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qrow + 32 * ks));

  // staging: thread tid always handles rows 2 * rp and 2 * rp + 1 of a
  // sub-chunk (rp = tid % 32) and chunks ch0, ch0 + 8, ..., ch0 + 64 of 8
  // values (ch0 = tid / 32): 8 latent chunks and one RoPE chunk per row.
  // Consecutive lanes take consecutive row pairs, so the transposed latent is
  // written as consecutive 32-bit words, free of bank conflicts.  Software
  // pipeline: the raw loads of sub-chunk j + 1 are issued before the matrix
  // work of sub-chunk j and only converted and stored after it.
  const int rp = tid & 31, ch0 = tid >> 5;
  const int ra = 2 * rp, rb = 2 * rp + 1;
  uint32_t* vt32 = reinterpret_cast<uint32_t*>(sh.vt);
  const int nsub = (r_end - r_begin + kSub - 1) / kSub;
  constexpr int kMaxSub = kSplitRows / kSub;       // 4
  constexpr int kLat = 8;                          // latent chunks per row and thread
  int32_t enca[kMaxSub], encb[kMaxSub];            // slot codes of this thread's rows
#pragma unroll
  for (int j = 0; j < kMaxSub; ++j) {
    enca[j] = encb[j] = 0;
    if (SRC == kFromSlots) {
      if (j < nsub && r_begin + j * kSub + ra < r_end) enca[j] = enc_row[r_begin + j * kSub + ra];
      if (j < nsub && r_begin + j * kSub + rb < r_end) encb[j] = enc_row[r_begin + j * kSub + rb];
    }
  }
  // raw data of the sub-chunk in flight
  u32x4 ba[kLat + 1], bb[kLat + 1];                // buffer source: 9 chunks of 16 B per row
  uint2 qa8[kLat], qb8[kLat];                      // slot source: 8 latent chunks of 8 B
  u32x4 ropea, ropeb, sca, scb;                    // slot source: RoPE chunk and scale block
  bool va = false, vb = false;
  auto fetch = [&](int j) {
    const int r0 = r_begin + j * kSub;
    va = r0 + ra < r_end;
    vb = r0 + rb < r_end;
    if (SRC == kFromBuffer) {
      const uint16_t* base = rows_buf + ((size_t)slq * K + r0) * HC_OUT_ELEMS + 8 * ch0;
#pragma unroll
      for (int k = 0; k <= kLat; ++k) {
        ba[k] = va ? *reinterpret_cast<const u32x4*>(base + (size_t)ra * HC_OUT_ELEMS + 64 * k)
                   : u32x4{0u, 0u, 0u, 0u};
        bb[k] = vb ? *reinterpret_cast<const u32x4*>(base + (size_t)rb * HC_OUT_ELEMS + 64 * k)
                   : u32x4{0u, 0u, 0u, 0u};
      }
    } else {
      const uint8_t* sa = va ? slot_row(d, sl, enca[j]) : nullptr;
      const uint8_t* sb = vb ? slot_row(d, sl, encb[j]) : nullptr;
#pragma unroll
      for (int k = 0; k < kLat; ++k) {
        qa8[k] = va ? *reinterpret_cast<const uint2*>(sa + 8 * (ch0 + 8 * k)) : uint2{0u, 0u};
        qb8[k] = vb ? *reinterpret_cast<const uint2*>(sb + 8 * (ch0 + 8 * k)) : uint2{0u, 0u};
      }
      ropea = va ? *reinterpret_cast<const u32x4*>(sa + HC_ROPE_OFFSET + 16 * ch0) : u32x4{0u, 0u, 0u, 0u};
      ropeb = vb ? *reinterpret_cast<const u32x4*>(sb + HC_ROPE_OFFSET + 16 * ch0) : u32x4{0u, 0u, 0u, 0u};
      sca = va ? *reinterpret_cast<const u32x4*>(sa + HC_SCALE_OFFSET) : u32x4{0u, 0u, 0u, 0u};
      scb = vb ? *reinterpret_cast<const u32x4*>(sb + HC_SCALE_OFFSET) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // chunk k (ch = ch0 + 8k) of this thread's two rows, as bf16
  auto chunk = [&](int k, u32x4& wa, u32x4& wb) {
    if (SRC == kFromBuffer) {
      wa = ba[k];
      wb = bb[k];
    } else if (k < kLat) {
      wa = dequant8(qa8[k], sca, k);   // latent chunk ch0 + 8k is in scale group k
      wb = dequant8(qb8[k], scb, k);
    } else {
      wa = ropea;
      wb = ropeb;
    }
  };

  fetch(0);
  for (int j = 0; j < nsub; ++j) {
    const int r0 = r_begin + j * kSub;
    const int nvalid = min(kSub, r_end - r0);
    __syncthreads();   // the previous sub-chunk's matrix work is done with LDS
#pragma unroll
    for (int k = 0; k <= kLat; ++k) {
      const int ch = ch0 + 8 * k;
      u32x4 wa, wb;
      chunk(k, wa, wb);
      *reinterpret_cast<u32x4*>(&sh.rows[ra * kRowLd + 8 * ch]) = wa;
      *reinterpret_cast<u32x4*>(&sh.rows[rb * kRowLd + 8 * ch]) = wb;
      if (k < kLat) {
        const uint32_t xa[4] = {wa.x, wa.y, wa.z, wa.w};
        const uint32_t xb[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t lo = (xa[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          const uint32_t hi = (xb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          vt32[(8 * ch + e) * (kVtLd / 2) + rp] = lo | (hi << 16);
        }
      }
    }
    __syncthreads();
    if (j + 1 < nsub) fetch(j + 1);   // in flight during this sub-chunk's matrix work

    // ---- S = Q K^T for this wave's 16 heads and the 64 rows ---------------
    f32x4 sacc[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) sacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < HC_OUT_ELEMS / 32; ++ks) {
      const bf16x8 a = qa[ks];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(
            &sh.rows[(16 * n + (lane & 15)) * kRowLd + 32 * ks + 8 * (lane >> 4)]);
        sacc[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, sacc[n], 0, 0, 0);
      }
    }
    // ---- online softmax: lane holds heads 4*(lane/16)+i of row 16n + lane%16
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mx[i] = -INFINITY;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bool ok = 16 * n + (lane & 15) < nvalid;
        sacc[n][i] = ok ? sacc[n][i] * scale : -INFINITY;
        mx[i] = fmaxf(mx[i], sacc[n][i]);
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) mx[i] = fmaxf(mx[i], __shfl_xor(mx[i], off, 64));
    }
    float factor[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float m_new = fmaxf(m_run[i], mx[i]);
      factor[i] = m_run[i] == -INFINITY ? 0.f : __expf(m_run[i] - m_new);
      float sum = 0.f;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const float pv = sacc[n][i] == -INFINITY ? 0.f : __expf(sacc[n][i] - m_new);
        sacc[n][i] = pv;
        sum += pv;
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) sum += __shfl_xor(sum, off, 64);
      l_run[i] = l_run[i] * factor[i] + sum;
      m_run[i] = m_new;
    }
#pragma unroll
    for (int n = 0; n < 32; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[n][i] *= factor[i];
    // P (bf16) to LDS as [head][row] for the A operand of P.V
    __bf16* pw = sh.p + wave * 16 * kPLd;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        pw[(4 * (lane >> 4) + i) * kPLd + 16 * n + (lane & 15)] = (__bf16)sacc[n][i];
    __syncthreads();
    // ---- O += P V ------------------------------------------------------------
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&pw[(lane & 15) * kPLd + 32 * ks + 8 * (lane >> 4)]);
#pragma unroll
      for (int n = 0; n < 32; ++n) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(
            &sh.vt[(16 * n + (lane & 15)) * kVtLd + 32 * ks + 8 * (lane >> 4)]);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, o[n], 0, 0, 0);
      }
    }
  }

  // ---- this split's partial: unnormalised output, max, sum per head --------
  const int nsplit = gridDim.x;
  float* base = part + (((size_t)slq * gridDim.y + hg) * nsplit + split) * kHeadsPerGroup * kPartStride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = wave * 16 + 4 * (lane >> 4) + i;
    float* ph = base + (size_t)h * kPartStride;
#pragma unroll
    for (int n = 0; n < 32; ++n) ph[16 * n + (lane & 15)] = o[n][i];
    if ((lane & 15) == 0) {
      ph[512] = m_run[i];
      ph[513] = l_run[i];
    }
  }
}

// Merges the splits of one (slq, head): out = sum_c e^(m_c - M) O_c / sum_c e^(m_c - M) l_c.
__global__ __launch_bounds__(512) void k_attend_merge(const float* __restrict__ part, int heads,
                                                      int nsplit, float* __restrict__ out) {
  const int h = blockIdx.x, slq = blockIdx.y, dd = threadIdx.x;
  const int hg = h / kHeadsPerGroup, hh = h - hg * kHeadsPerGroup;
  const int ngroups = heads / kHeadsPerGroup;
  const float* base = part + (((size_t)slq * ngroups + hg) * nsplit) * kHeadsPerGroup * kPartStride +
                      (size_t)hh * kPartStride;
  const size_t cstride = (size_t)kHeadsPerGroup * kPartStride;
  float M = -INFINITY;
  for (int c = 0; c < nsplit; ++c) M = fmaxf(M, base[c * cstride + 512]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < nsplit; ++c) {
    const float mc = base[c * cstride + 512];
    const float w = mc == -INFINITY ? 0.f : __expf(mc - M);
    L += w * base[c * cstride + 513];
    acc += w * base[c * cstride + dd];
  }
  out[((size_t)slq * heads + h) * 512 + dd] = acc / L;
}

uint64_t attend_work_bytes(const DevState& d, int heads) {
  const uint64_t nsplit = (d.K + kSplitRows - 1) / kSplitRows;
  return (uint64_t)d.S * d.L * d.Q * (heads / kHeadsPerGroup) * nsplit * kHeadsPerGroup *
         kPartStride * sizeof(float);
}

hipError_t launch_attend(const DevState& d, bool from_slots, const uint16_t* q, int heads,
                         float scale, const uint16_t* rows, void* work, float* out,
                         hipStream_t st) {
  const int nsplit = (d.K + kSplitRows - 1) / kSplitRows;
  dim3 grid(nsplit, heads / kHeadsPerGroup, d.S * d.L * d.Q);
  float* part = static_cast<float*>(work);
  if (from_slots)
    hipLaunchKernelGGL(k_attend<kFromSlots>, grid, dim3(kAttThreads), 0, st, d, q, heads, scale,
                       rows, part);
  else
    hipLaunchKernelGGL(k_attend<kFromBuffer>, grid, dim3(kAttThreads), 0, st, d, q, heads, scale,
                       rows, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attend_merge, dim3(heads, d.S * d.L * d.Q), dim3(512), 0, st, part, heads,
                     nsplit, out);
  return hipGetLastError();
}

}  // namespace hc
