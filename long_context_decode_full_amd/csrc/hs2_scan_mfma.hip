// Matrix-core scan of the Full Attention layer (records mode): the same work as the
// records mode of the VALU scan (online-softmax partials, a 2-byte bound record per
// position and a histogram of the candidate keys per split), with both contractions
// on v_mfma_f32_16x16x32_bf16.
//
// HySparse2 article, section 02 "KV Reuse": the full layer attends over the whole
// cache and its attention scores decide the positions the sparse layers reuse.
//
// Per wave step of 32 rows (two 16-row tiles), with lane = 16*grp + w16:
//   QK   D[row][head] = K[row][:] . Q[head][:]: A = K tile (lane: row w16, 16 bytes
//        at dims 32s + 8grp of each 32-dim slice s), B = Q^T (lane: head w16, same
//        dims; heads >= G are zero), four MFMAs per tile.  The accumulator lane
//        holds rows 4grp+v (v = 0..3) of head w16.
//   softmax per head: the 8 logits of a lane plus two permlane swaps give the step
//        maximum of head w16; the running maximum is raised only when a logit
//        exceeds it by 8 (log2 units).
//   record per row: log2 of the sum over the group's heads of 2^logit, reduced
//        over the 8 head lanes of each 16-lane row with DPP.
//   PV   O^T[dim][head] += V^T[dim][rows] . P[rows][head]: B = P, exactly the
//        lane's 8 probabilities (rows 4grp+v of both tiles), split into a bf16 high
//        part and a bf16 residual so the product keeps fp32 accuracy; A = V^T, read
//        from the wave's LDS copy of the V tile with ds_read_b64_tr_b16 (each lane
//        gets 4 rows of one dim per read).  Eight 16-dim blocks, two MFMAs each.
// The K loads feed the MFMA directly (each load instruction covers 16 rows x 64
// contiguous bytes); V rows are loaded whole (16 lanes per row) and stored to LDS.
// Loads run one step ahead through a two-buffer ring, with the non-temporal hint.
#include "hs2_rowops.h"

namespace hs2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2v_t;

constexpr int kStepRows = 32;
constexpr float kMSlack = 8.0f;
constexpr int kVRow = 272;                    // bytes per staged V row (256 + 16 pad)
constexpr int kVTile = kStepRows * kVRow;     // per wave
constexpr int kRecBytes = kMaxRecordSplit * 2;
constexpr int kHistBytes = kFastBins * 4;
constexpr int kMergeStride = kPartStride;     // floats per head in the wave merge area: m, z, -, -, o[128]
static_assert(8 * kMergeStride * 4 <= kVTile, "a wave's merge record fits its V tile");

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp32 -> one word of two bf16 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2v_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Max / sum over the 8 lanes w16 = 0..7 (and separately 8..15) of each 16-lane row.
__device__ __forceinline__ float max8(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppMirror8>(x));
  return x;
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppMirror8>(x);
  return x;
}

// Combine the 4 lanes w16, w16+16, w16+32, w16+48 (the four row groups) with the
// gfx950 permlane swaps.  The swap results are copied to scalars before any bit
// cast: a bit cast of a vector element reads element 0 here.
template <bool kMax>
__device__ __forceinline__ float reduce_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = s32[0], a1 = s32[1];
  x = kMax ? fmaxf(__uint_as_float(a0), __uint_as_float(a1)) : __uint_as_float(a0) + __uint_as_float(a1);
  const uint32_t w = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  const uint32_t c0 = s16[0], c1 = s16[1];
  return kMax ? fmaxf(__uint_as_float(c0), __uint_as_float(c1)) : __uint_as_float(c0) + __uint_as_float(c1);
}
__device__ __forceinline__ float max_groups(float x) { return reduce_groups<true>(x); }
__device__ __forceinline__ float sum_groups(float x) { return reduce_groups<false>(x); }

// One step's loads.  bf16: k[t][q] = 16 bytes of row (tile t, w16), v[i] = 16 bytes
// of row 4i + grp.  fp8: k[t][q] = 8 codes, v[i] = 16 codes of row 8i + lane/8, plus
// the per-row scales of the lane's 8 accumulator rows.
template <bool kFp8>
struct StepBuf;
template <>
struct StepBuf<false> {
  uint4 k[2][4];
  uint4 v[8];
};
template <>
struct StepBuf<true> {
  uint4 k[2][2];   // 16 codes: dim chunks kchunk_fp8(2h, grp), kchunk_fp8(2h + 1, grp)
  uint4 v[4];
  float ks[2][4], vs[2][4];
};

// fp8 keys: the 8-dim chunk of the row that MFMA slice q takes in row group grp.  A
// lane loads 16 contiguous codes (two chunks, slices 2h and 2h+1) and the 4 row groups
// cover 64 contiguous bytes per load; the queries are read in the same dim order, so
// the dot products are unchanged.  (bf16 keys: chunk 4q + grp.)
__device__ __forceinline__ int kchunk_fp8(int q, int grp) { return 8 * (q >> 1) + 2 * grp + (q & 1); }

// kVecScale (fp8, capacity a multiple of 4, so 16-byte aligned rows of scales): the 4
// scales of a lane's rows 4grp .. 4grp+3 of a tile in one 16-byte load.
template <bool kFp8, bool kVecScale = false>
__device__ __forceinline__ void load_step(StepBuf<kFp8>& s, const uint8_t* __restrict__ kb,
                                          const uint8_t* __restrict__ vb, const float* __restrict__ ksb,
                                          const float* __restrict__ vsb, int32_t base, int32_t last,
                                          int grp, int w16, int lane) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t row = (uint32_t)min(base + 16 * t + w16, last);
    if constexpr (kFp8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        s.k[t][h] = *reinterpret_cast<const uint4*>(kb + (uint64_t)row * 128 + 64 * h + 16 * grp);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s.k[t][q] = load_nt(reinterpret_cast<const uint4*>(kb + (uint64_t)row * 256 + 64 * q + 16 * grp));
    }
  }
  if constexpr (kFp8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = (uint32_t)min(base + 8 * i + (lane >> 3), last);
      s.v[i] = load_nt(reinterpret_cast<const uint4*>(vb + (uint64_t)row * 128 + 16 * (lane & 7)));
    }
    if constexpr (kVecScale) {
      // rows past `last` are masked; clamping the first row to a multiple of 4 at or
      // below `last` keeps all 4 inside the capacity (a multiple of 4)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t row = (uint32_t)min(base + 16 * t + 4 * grp, last & ~3);
        const float4 k4 = *reinterpret_cast<const float4*>(ksb + row);
        const float4 v4 = *reinterpret_cast<const float4*>(vsb + row);
        s.ks[t][0] = k4.x; s.ks[t][1] = k4.y; s.ks[t][2] = k4.z; s.ks[t][3] = k4.w;
        s.vs[t][0] = v4.x; s.vs[t][1] = v4.y; s.vs[t][2] = v4.z; s.vs[t][3] = v4.w;
      }
    } else {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const uint32_t row = (uint32_t)min(base + 16 * t + 4 * grp + v, last);
          s.ks[t][v] = ksb[row];
          s.vs[t][v] = vsb[row];
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t row = (uint32_t)min(base + 4 * i + grp, last);
      s.v[i] = load_nt(reinterpret_cast<const uint4*>(vb + (uint64_t)row * 256 + 16 * w16));
    }
  }
}

// One sparse-layer step's loads: the rows named by index-row entries e0 .. e0+31
// (srow: row per entry, -1 for a skipped entry, which loads row 0 and is masked).
// Ordinary loads: the next sparse layer gathers the same rows.
template <bool kFp8>
__device__ __forceinline__ void load_step_gather(StepBuf<kFp8>& s, const uint8_t* __restrict__ kb,
                                                 const uint8_t* __restrict__ vb, const float* __restrict__ ksb,
                                                 const float* __restrict__ vsb, const int32_t* srow, int e0,
                                                 int grp, int w16, int lane) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t row = (uint32_t)max(srow[e0 + 16 * t + w16], 0);
    if constexpr (kFp8) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        s.k[t][h] = *reinterpret_cast<const uint4*>(kb + (uint64_t)row * 128 + 64 * h + 16 * grp);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        s.k[t][q] = *reinterpret_cast<const uint4*>(kb + (uint64_t)row * 256 + 64 * q + 16 * grp);
    }
  }
  if constexpr (kFp8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t row = (uint32_t)max(srow[e0 + 8 * i + (lane >> 3)], 0);
      s.v[i] = *reinterpret_cast<const uint4*>(vb + (uint64_t)row * 128 + 16 * (lane & 7));
    }
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t row = (uint32_t)max(srow[e0 + 16 * t + 4 * grp + v], 0);
        s.ks[t][v] = ksb[row];
        s.vs[t][v] = vsb[row];
      }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t row = (uint32_t)max(srow[e0 + 4 * i + grp], 0);
      s.v[i] = *reinterpret_cast<const uint4*>(vb + (uint64_t)row * 256 + 16 * w16);
    }
  }
}

struct HeadState {
  f32x4_t o[8];   // o[b][v]: dim 16b + 4grp + v of head w16
  float m;        // running maximum of head w16 (log2 domain; equal in the 4 groups)
  float z;        // this lane's share of the softmax denominator
  float c;        // records: 2^(m - U) for a head of the group, else 0
};

// Reduce-scatter of 8 values over the 8 lanes w16 & 7 of a half-row: lane i ends with
// the sum over the 8 lanes of value i.  Each step keeps the half of the values named by
// one lane bit and adds the partner's copy of it (partners i^7, i^2, i^1: the bit
// differs, so the two keep complementary halves).
__device__ __forceinline__ float reduce_scatter8(const float (&x)[8], int w16) {
  const bool b2 = (w16 & 4) != 0, b1 = (w16 & 2) != 0, b0 = (w16 & 1) != 0;
  float y[4], z[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) y[j] = (b2 ? x[j + 4] : x[j]) + dpp<kDppMirror8>(b2 ? x[j] : x[j + 4]);
#pragma unroll
  for (int j = 0; j < 2; ++j) z[j] = (b1 ? y[j + 2] : y[j]) + dpp<kDppXor2>(b1 ? y[j] : y[j + 2]);
  return (b0 ? z[1] : z[0]) + dpp<kDppXor1>(b0 ? z[0] : z[1]);
}

// Max / sum over all 16 lanes w16 of each 16-lane row.
__device__ __forceinline__ float max16w(float x) {
  x = max8(x);
  return fmaxf(x, dpp<kDppRor8>(x));
}
__device__ __forceinline__ float sum16w(float x) {
  x = sum8(x);
  return x + dpp<kDppRor8>(x);
}

// Head layout of a step.  kHB head blocks of 16 (lane w16 holds head 16 hb + w16 of
// block hb); kWide: the bound record sums over all 16 lanes of a block (G > 8),
// otherwise over lanes 0..7 (G <= 8: the heads 8..15 of the tile are padding).
// kGather: a sparse-layer step; `base` is the step's first index-row entry and srow
// holds each entry's row (-1: skipped), so no records are formed.
// kBlk: a block-comparator step: instead of records, log2 of the sum of 2^logit over
// the step's 32 positions per head goes to blrow[(base / 32) * H + head], H the head
// slots of the layout (8, 16 or 32).
template <bool kFp8, bool kGather = false, int kHB = 1, bool kWide = false, bool kBlk = false>
__device__ __forceinline__ void process_step(const StepBuf<kFp8>& s, const bf16x8_t (&qf)[kHB][4], uint8_t* vt,
                                             int32_t base, int32_t w_begin, int32_t w_end, uint32_t cand_span,
                                             float scale_log2, int G, int grp, int w16, int lane,
                                             uint16_t* recs, uint32_t* shist, HeadState (&hs)[kHB], float& U,
                                             const int32_t* srow = nullptr, float* blrow = nullptr) {
  constexpr bool kRec = !kGather && !kBlk;   // bound records and their histogram
  // V tile -> LDS (row-major, padded rows)
  if constexpr (kFp8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 c = s.v[i];
      const uint4 lo = make_uint4(fp8x2_to_bf16x2(c.x, false), fp8x2_to_bf16x2(c.x, true),
                                  fp8x2_to_bf16x2(c.y, false), fp8x2_to_bf16x2(c.y, true));
      const uint4 hi = make_uint4(fp8x2_to_bf16x2(c.z, false), fp8x2_to_bf16x2(c.z, true),
                                  fp8x2_to_bf16x2(c.w, false), fp8x2_to_bf16x2(c.w, true));
      uint8_t* dst = vt + (8 * i + (lane >> 3)) * kVRow + 32 * (lane & 7);
      *reinterpret_cast<uint4*>(dst) = lo;
      *reinterpret_cast<uint4*>(dst + 16) = hi;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(vt + (4 * i + grp) * kVRow + 16 * w16) = s.v[i];
  }

  // QK (the key fragment of a tile and dim slice serves every head block)
  f32x4_t d[kHB][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) d[hb][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint4 kw;
      if constexpr (kFp8) {
        const uint4 c4 = s.k[t][q >> 1];
        const uint32_t c0 = (q & 1) ? c4.z : c4.x, c1 = (q & 1) ? c4.w : c4.y;
        kw = make_uint4(fp8x2_to_bf16x2(c0, false), fp8x2_to_bf16x2(c0, true), fp8x2_to_bf16x2(c1, false),
                        fp8x2_to_bf16x2(c1, true));
      } else {
        kw = s.k[t][q];
      }
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) d[hb][t] = mfma16(as_bf16x8(kw), qf[hb][q], d[hb][t]);
    }
  }
  float l[kHB][2][4];
  float mx[kHB];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) mx[hb] = kNegInf;
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int32_t row = base + 16 * t + 4 * grp + v;
      bool live;
      if constexpr (kGather) live = srow[row] >= 0;
      else live = row < w_end;
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) {
        float x = d[hb][t][v] * scale_log2;
        if constexpr (kFp8) x *= s.ks[t][v];
        l[hb][t][v] = live ? x : kNegInf;
        mx[hb] = fmaxf(mx[hb], l[hb][t][v]);
      }
    }

  // online softmax of head 16 hb + w16
  bool up[kHB];
  bool up_any = false;
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    mx[hb] = max_groups(mx[hb]);
    up[hb] = mx[hb] > hs[hb].m + kMSlack;
    up_any |= up[hb];
  }
  if (wave_any(up_any)) {
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const float mn = up[hb] ? mx[hb] : hs[hb].m;
      const float alpha = up[hb] ? fast_exp2(hs[hb].m - mn) : 1.0f;
#pragma unroll
      for (int b = 0; b < 8; ++b) hs[hb].o[b] *= alpha;
      hs[hb].z *= alpha;
      hs[hb].m = mn;
    }
    if constexpr (kRec) {
      // U: the largest running maximum of the group's heads (equal in every lane), and
      // the record scale of each head; they change only with a running maximum
      U = kNegInf;
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) U = fmaxf(U, 16 * hb + w16 < G ? hs[hb].m : kNegInf);
      U = kWide ? max16w(U) : max8(U);
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) hs[hb].c = 16 * hb + w16 < G ? fast_exp2(hs[hb].m - U) : 0.0f;
    }
  }
  bf16x8_t phi[kHB], plo[kHB];
  float rsum[2][4];                     // records: sum over this lane's head blocks of p 2^(m - U)
  float bsum[kHB];                      // block steps: this lane's sum of p per head block
  if constexpr (kRec) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) rsum[t][v] = 0.0f;
  }
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    float p[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[t][v] = l[hb][t][v] != kNegInf ? fast_exp2(l[hb][t][v] - hs[hb].m) : 0.0f;
        hs[hb].z += p[t][v];
        if constexpr (kRec) rsum[t][v] = fmaf(p[t][v], hs[hb].c, rsum[t][v]);
        if constexpr (kBlk) bsum[hb] = (t == 0 && v == 0) ? p[t][v] : bsum[hb] + p[t][v];
        // masked rows: the scale may come from a row past the end (4-row scale loads)
        if constexpr (kFp8) p[t][v] = l[hb][t][v] != kNegInf ? p[t][v] * s.vs[t][v] : 0.0f;
      }
    // P as bf16 high part + bf16 residual (B operand, k slot u <-> tile u/4, row 4grp + u%4)
    uint32_t hw[4], lw[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x0 = p[u >> 1][2 * (u & 1)];
      const float x1 = p[u >> 1][2 * (u & 1) + 1];
      hw[u] = pack_bf16(x0, x1);
      lw[u] = pack_bf16(x0 - __builtin_bit_cast(float, hw[u] << 16), x1 - __builtin_bit_cast(float, hw[u] & 0xFFFF0000u));
    }
    phi[hb] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
    plo[hb] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
  }

  // bound records: e = log2 sum over the group's heads of 2^l.  With p = 2^(l - m) of
  // each head (formed above for P.V), sum_h 2^l_h = 2^U sum_h p_h 2^(m_h - U).  The 8
  // row sums of a lane are reduce-scattered over the head lanes (the two half-rows
  // added first when the group spans 16 lanes), so lane w16 < 8 owns row w16 of its
  // row group: one logarithm, one record store and one histogram count per lane.  A
  // live row whose sum is below 2^-100 (terms lost to underflow could matter there)
  // makes the wave take the direct form, max then sum of 2^(l - max), for the step.
  if constexpr (kBlk) {
    // the step's share of each head's softmax sum, relative to the running maximum
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const float tot = sum_groups(bsum[hb]);
      const float lse = hs[hb].m + __builtin_amdgcn_logf(tot);   // -inf for an empty step
      if (grp == 0 && 16 * hb + w16 < G)
        blrow[(int64_t)(base / kStepRows) * ((kWide ? 16 : 8) * kHB) + 16 * hb + w16] = lse;
    }
  }
  if constexpr (kRec) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = rsum[i >> 2][i & 3];
      if constexpr (kWide) x[i] += dpp<kDppRor8>(x[i]);
    }
    const float sm = reduce_scatter8(x, w16);
    const int io = w16 & 7;   // own row: tile io >> 2, v = io & 3
    const int32_t row_o = base + 16 * (io >> 2) + 4 * grp + (io & 3);
    const bool writer = w16 < 8 && row_o < w_end;
    float e = U + __builtin_amdgcn_logf(sm);
    if (wave_any(writer && !(sm >= 0x1p-100f))) {
      // every lane takes part in the reductions; each keeps its own row's value
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float lm[kHB];
          float rmax = kNegInf;
#pragma unroll
          for (int hb = 0; hb < kHB; ++hb) {
            lm[hb] = 16 * hb + w16 < G ? l[hb][t][v] : kNegInf;
            rmax = fmaxf(rmax, lm[hb]);
          }
          rmax = kWide ? max16w(rmax) : max8(rmax);
          float ex = 0.0f;
#pragma unroll
          for (int hb = 0; hb < kHB; ++hb) ex += lm[hb] != kNegInf ? fast_exp2(lm[hb] - rmax) : 0.0f;
          const float sum = kWide ? sum16w(ex) : sum8(ex);
          const float ed = rmax + __builtin_amdgcn_logf(sum);
          e = io == 4 * t + v ? ed : e;
        }
    }
    if (writer) {
      const uint32_t rel = (uint32_t)(row_o - w_begin);
      const uint16_t rec = __builtin_bit_cast(uint16_t, (_Float16)e);
      recs[rel] = rec;
      if (rel < cand_span) atomicAdd(&shist[half_order_key(rec) >> kFastShift], 1u);
    }
  }

  // PV: A = V^T of dim block b, rows 4grp..4grp+3 of both tiles (transposed LDS reads)
  const uint8_t* tr0 = vt + (4 * grp + (w16 >> 2)) * kVRow + 8 * (w16 & 3);
  const uint8_t* tr1 = tr0 + 16 * kVRow;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(tr0 + 32 * b));
    const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(tr1 + 32 * b));
    const uint2 w0 = __builtin_bit_cast(uint2, x0);
    const uint2 w1 = __builtin_bit_cast(uint2, x1);
    const bf16x8_t av = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      hs[hb].o[b] = mfma16(av, phi[hb], hs[hb].o[b]);
      hs[hb].o[b] = mfma16(av, plo[hb], hs[hb].o[b]);
    }
  }
}

// kHB, kWide: head layout (see process_step); kThreads: 512 (8 waves) for up to 16
// heads, 256 (4 waves, one per SIMD, up to 512 registers a lane) for 32 heads.
// kBlk: the block comparator's scan (per-32-position block sums, no records).
template <bool kFp8, bool kVecScale, int kHB, bool kWide, int kThreads, bool kBlk = false>
__global__ __launch_bounds__(kThreads, 1) void scan_mfma_kernel(ScanArgs a) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kBH = kWide ? 16 : 8;   // heads per block with state (lanes w16 < kBH)
  __shared__ __attribute__((aligned(16))) uint8_t lds[kRecBytes + kHistBytes + kWaves * kVTile];
  uint16_t* srec = reinterpret_cast<uint16_t*>(lds);
  uint32_t* shist = reinterpret_cast<uint32_t*>(lds + kRecBytes);
  uint8_t* vt_all = lds + kRecBytes + kHistBytes;

  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int bj = blockIdx.z;
  const int b = bj / a.Lq;
  const int j = bj - b * a.Lq;
  const int64_t sel = (int64_t)bj * a.Hkv + g;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int w16 = lane & 15;
  uint8_t* vt = vt_all + wave * kVTile;

  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  int64_t n = ctx - a.Lq + j + 1;
  n = n < 0 ? 0 : n;
  const int64_t p_begin = (int64_t)split * a.split_len;
  int64_t p_end = p_begin + a.split_len;
  p_end = p_end < n ? p_end : n;
  // The waves share the split's 32-row steps through an LDS counter: a wave takes
  // the next step when it starts on one, so the workgroup reads K and V as two
  // contiguous streams and every wave ends within a step of the others.  (Waves are
  // not served equally: with a fixed share per wave, or two workgroups per CU, the
  // younger ones took up to 1.4x longer and set the kernel's end.)  Which wave sums
  // which step then varies from run to run, so the output can differ in the last
  // bits; a.fixed_steps gives wave w the steps w, w+8, ... instead (reproducible,
  // ~3% slower on the million-token scan).
  const int32_t w_begin = (int32_t)p_begin;   // rows < cap < 2^31
  const int32_t w_end = (int32_t)(p_end > p_begin ? p_end : p_begin);
  const int nsteps = (w_end - w_begin + kStepRows - 1) / kStepRows;
  __shared__ int step_next;

  // Q^T fragments: head 16 hb + w16, dims of chunk (4q + grp, or kchunk_fp8)
  bf16x8_t qf[kHB][4];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    const int h = 16 * hb + w16;
    const uint16_t* qh = a.q + ((int64_t)bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int chunk = kFp8 ? kchunk_fp8(q, grp) : 4 * q + grp;
      qf[hb][q] = as_bf16x8(h < a.G ? *reinterpret_cast<const uint4*>(qh + 8 * chunk) : make_uint4(0u, 0u, 0u, 0u));
    }
  }

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const int rowbytes = kFp8 ? 128 : 256;
  const uint8_t* kb = a.k + head_row0 * rowbytes;
  const uint8_t* vb = a.v + head_row0 * rowbytes;
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float* vsb = kFp8 ? a.v_scale + head_row0 : nullptr;

  // candidates are the positions before the forced window
  int64_t w0 = n - a.window;
  w0 = w0 < 0 ? 0 : w0;
  const uint32_t span = (uint32_t)(w_end - w_begin);
  uint32_t cand_span = w0 > p_begin ? (uint32_t)(w0 - p_begin) : 0u;
  cand_span = cand_span < span ? cand_span : span;

  if constexpr (!kBlk) {
    for (int i = tid; i < kFastBins; i += kThreads) shist[i] = 0u;
    if (split == 0) {   // the combine kernel sums every split's histogram into these words
      uint32_t* hm = a.hist_merged + sel * kSelWords + kSelHist1Off;
      for (int i = tid; i < kMergedWords; i += kThreads) hm[i] = 0u;
    }
  }
  if (tid == 0) step_next = kWaves;   // step w is wave w's first
  float* blrow = kBlk ? a.blse + sel * a.blse_stride * (kBH * kHB) : nullptr;
  __syncthreads();

  HeadState hs[kHB];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) hs[hb].o[bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    hs[hb].m = kNegInf;
    hs[hb].z = 0.0f;
    hs[hb].c = 0.0f;
  }
  float U = kNegInf;

  if (nsteps > 0) {
    const int32_t last = w_end - 1;
    // next step for this wave (wave-uniform); steps taken by a wave increase, so once
    // one is past the end every later one is too
    const bool fixed = a.fixed_steps != 0;
    int knext = wave + kWaves;
    auto take = [&]() -> int {
      int k = knext;
      knext += kWaves;
      if (!fixed && lane == 0)
        k = __hip_atomic_fetch_add(&step_next, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return __builtin_amdgcn_readfirstlane(k);
    };
    StepBuf<kFp8> s0, s1;
    int k0 = wave;
    load_step<kFp8, kVecScale>(s0, kb, vb, ksb, vsb, w_begin + k0 * kStepRows, last, grp, w16, lane);
    int k1 = take();
    load_step<kFp8, kVecScale>(s1, kb, vb, ksb, vsb, w_begin + k1 * kStepRows, last, grp, w16, lane);
    // two-buffer ring; every load is issued (rows past the end re-read `last`)
    while (k0 < nsteps) {
      process_step<kFp8, false, kHB, kWide, kBlk>(s0, qf, vt, w_begin + k0 * kStepRows, w_begin, w_end, cand_span,
                                                  a.scale_log2, a.G, grp, w16, lane, srec, shist, hs, U, nullptr,
                                                  blrow);
      k0 = take();
      load_step<kFp8, kVecScale>(s0, kb, vb, ksb, vsb, w_begin + k0 * kStepRows, last, grp, w16, lane);
      if (k1 >= nsteps) break;
      process_step<kFp8, false, kHB, kWide, kBlk>(s1, qf, vt, w_begin + k1 * kStepRows, w_begin, w_end, cand_span,
                                                  a.scale_log2, a.G, grp, w16, lane, srec, shist, hs, U, nullptr,
                                                  blrow);
      k1 = take();
      load_step<kFp8, kVecScale>(s1, kb, vb, ksb, vsb, w_begin + k1 * kStepRows, last, grp, w16, lane);
    }
  }

  // the split's records and key histogram, once every wave is done
  __syncthreads();
  if constexpr (!kBlk) {
    const int cnt = p_end > p_begin ? (int)(p_end - p_begin) : 0;
    uint16_t* grec = a.records + sel * a.logit_stride + p_begin;   // 512-byte aligned
    for (int i = tid; 2 * i + 1 < cnt; i += kThreads)
      reinterpret_cast<uint32_t*>(grec)[i] = reinterpret_cast<const uint32_t*>(srec)[i];
    if ((cnt & 1) && tid == 0) grec[cnt - 1] = srec[cnt - 1];
    uint32_t* ghist = reinterpret_cast<uint32_t*>(a.hist_part + (sel * a.n_split + split) * kFastBins);
    for (int i = tid; i < kFastBins / 2; i += kThreads)
      ghist[i] = (shist[2 * i] & 0xFFFFu) | (shist[2 * i + 1] << 16);   // counts < 2^16
  }

  // ---- merge, one head block at a time: the 4 row groups (shares of z), then the
  // waves through their LDS tiles (each wave's last reads of its tile are done)
  float* mrec = reinterpret_cast<float*>(vt);
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    if (hb > 0) __syncthreads();   // the previous block's merge reads are done
    const float zt = sum_groups(hs[hb].z);
    if (w16 < kBH) {
      float* mr = mrec + w16 * kMergeStride;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        *reinterpret_cast<float4*>(mr + 4 + 16 * bb + 4 * grp) =
            make_float4(hs[hb].o[bb][0], hs[hb].o[bb][1], hs[hb].o[bb][2], hs[hb].o[bb][3]);
      if (grp == 0) {
        mr[0] = hs[hb].m;
        mr[1] = zt;
      }
    }
    __syncthreads();
    // thread -> (head slot, 4 dims)
    for (int hl = tid >> 5; hl < kBH; hl += kThreads / 32) {
      const int h = 16 * hb + hl;
      const int dd = (tid & 31) * 4;
      float Mw = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        Mw = fmaxf(Mw, reinterpret_cast<const float*>(vt_all + w * kVTile)[hl * kMergeStride]);
      float Z = 0.0f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* mr = reinterpret_cast<const float*>(vt_all + w * kVTile) + hl * kMergeStride;
        const float mw = mr[0];
        const float fw = (mw == kNegInf) ? 0.0f : fast_exp2(mw - Mw);
        Z += fw * mr[1];
        const float4 ov = *reinterpret_cast<const float4*>(mr + 4 + dd);
        acc.x += fw * ov.x;
        acc.y += fw * ov.y;
        acc.z += fw * ov.z;
        acc.w += fw * ov.w;
      }
      if (h < a.G) {
        float* pp = a.part + ((sel * a.n_split + split) * a.G + h) * kPartStride;
        *reinterpret_cast<float4*>(pp + 4 + dd) = acc;
        if (dd == 0) {
          pp[0] = Mw;
          pp[1] = Z;
        }
      }
    }
  }
}

// ---- Sparse Attention layer (HySparse2 article, section 02 "KV Reuse": the sparse
// layers attend with their own queries over the rows of the shared cache that the
// full layer's index set names; section 03: window and global rows share one
// softmax).  One workgroup per (query token, KV head, split of the index row): its
// waves gather the entries 32 at a time with the step code of the scan (wave w takes
// steps w, w + waves, ...: a fixed share, so the output is bitwise reproducible) and
// merge through LDS.  With one split (out != nullptr) the workgroup writes the
// normalised output and no combine follows; with several it writes partials.
constexpr int kGMaxS = 4096;   // index row length bound (checked on the host)

template <bool kFp8, int kHB, bool kWide, int kThreads>
__global__ __launch_bounds__(kThreads, 1) void gather_mfma_kernel(ScanArgs a, float* __restrict__ out) {
  constexpr int kWaves = kThreads / 64;
  constexpr int kBH = kWide ? 16 : 8;
  __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kVTile + kGMaxS * 4];
  uint8_t* vt_all = lds;
  int32_t* srow = reinterpret_cast<int32_t*>(lds + kWaves * kVTile);

  const int split = blockIdx.x;   // entries [split * split_len, +split_len) of the index row
  const int g = blockIdx.y;
  const int bj = blockIdx.z;
  const int b = bj / a.Lq;
  const int j = bj - b * a.Lq;
  const int64_t sel = (int64_t)bj * a.Hkv + g;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int w16 = lane & 15;
  uint8_t* vt = vt_all + wave * kVTile;

  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  int64_t n = ctx - a.Lq + j + 1;
  n = n < 0 ? 0 : n;
  const int e_begin = split * a.split_len;
  const int e_count = max(0, min(a.split_len, a.S - e_begin));
  const int nsteps = (e_count + kStepRows - 1) / kStepRows;

  // this split's entries of the index row, those naming no visible row (or, for a
  // local cache, no row of it) turned into -1
  const int64_t lim = a.slot_rows ? a.cap : n;
  const int32_t* irow = a.idx + sel * a.S + e_begin;
  for (int e = tid; e < nsteps * kStepRows; e += kThreads) {
    const int32_t t = e < e_count ? irow[e] : -1;
    srow[e] = (t >= 0 && t < lim) ? t : -1;
  }
  bf16x8_t qf[kHB][4];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    const int h = 16 * hb + w16;
    const uint16_t* qh = a.q + ((int64_t)bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int chunk = kFp8 ? kchunk_fp8(q, grp) : 4 * q + grp;
      qf[hb][q] = as_bf16x8(h < a.G ? *reinterpret_cast<const uint4*>(qh + 8 * chunk) : make_uint4(0u, 0u, 0u, 0u));
    }
  }
  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const int rowbytes = kFp8 ? 128 : 256;
  const uint8_t* kb = a.k + head_row0 * rowbytes;
  const uint8_t* vb = a.v + head_row0 * rowbytes;
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float* vsb = kFp8 ? a.v_scale + head_row0 : nullptr;
  __syncthreads();

  HeadState hs[kHB];
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) hs[hb].o[bb] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    hs[hb].m = kNegInf;
    hs[hb].z = 0.0f;
    hs[hb].c = 0.0f;
  }
  float U = kNegInf;   // unused here: gather steps form no records

  if (wave < nsteps) {
    // two-buffer ring over steps wave, wave + kWaves, ...; loads past the last step re-read it
    const int klast = nsteps - 1;
    StepBuf<kFp8> s0, s1;
    int k0 = wave, k1 = wave + kWaves;
    load_step_gather<kFp8>(s0, kb, vb, ksb, vsb, srow, k0 * kStepRows, grp, w16, lane);
    load_step_gather<kFp8>(s1, kb, vb, ksb, vsb, srow, min(k1, klast) * kStepRows, grp, w16, lane);
    while (k0 < nsteps) {
      process_step<kFp8, true, kHB, kWide>(s0, qf, vt, k0 * kStepRows, 0, 0, 0u, a.scale_log2, a.G, grp, w16, lane,
                                           nullptr, nullptr, hs, U, srow);
      k0 += 2 * kWaves;
      load_step_gather<kFp8>(s0, kb, vb, ksb, vsb, srow, min(k0, klast) * kStepRows, grp, w16, lane);
      if (k1 >= nsteps) break;
      process_step<kFp8, true, kHB, kWide>(s1, qf, vt, k1 * kStepRows, 0, 0, 0u, a.scale_log2, a.G, grp, w16, lane,
                                           nullptr, nullptr, hs, U, srow);
      k1 += 2 * kWaves;
      load_step_gather<kFp8>(s1, kb, vb, ksb, vsb, srow, min(k1, klast) * kStepRows, grp, w16, lane);
    }
  }

  // merge, one head block at a time: the row groups, then the waves through LDS;
  // out = o / Z (0 when no entry is live)
  float* mrec = reinterpret_cast<float*>(vt);   // this wave's tile: its last reads are done
#pragma unroll
  for (int hb = 0; hb < kHB; ++hb) {
    if (hb > 0) __syncthreads();
    const float zt = sum_groups(hs[hb].z);
    if (w16 < kBH) {
      float* mr = mrec + w16 * kMergeStride;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb)
        *reinterpret_cast<float4*>(mr + 4 + 16 * bb + 4 * grp) =
            make_float4(hs[hb].o[bb][0], hs[hb].o[bb][1], hs[hb].o[bb][2], hs[hb].o[bb][3]);
      if (grp == 0) {
        mr[0] = hs[hb].m;
        mr[1] = zt;
      }
    }
    __syncthreads();
    for (int hl = tid >> 5; hl < kBH; hl += kThreads / 32) {
      const int h = 16 * hb + hl;
      const int dd = (tid & 31) * 4;
      float Mw = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w)
        Mw = fmaxf(Mw, reinterpret_cast<const float*>(vt_all + w * kVTile)[hl * kMergeStride]);
      float Z = 0.0f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* mr = reinterpret_cast<const float*>(vt_all + w * kVTile) + hl * kMergeStride;
        const float mw = mr[0];
        const float fw = (mw == kNegInf) ? 0.0f : fast_exp2(mw - Mw);
        Z += fw * mr[1];
        const float4 ov = *reinterpret_cast<const float4*>(mr + 4 + dd);
        acc.x += fw * ov.x;
        acc.y += fw * ov.y;
        acc.z += fw * ov.z;
        acc.w += fw * ov.w;
      }
      if (h < a.G) {
        if (out != nullptr) {   // the whole row in this workgroup: normalised output
          const float iz = Z > 0.0f ? 1.0f / Z : 0.0f;
          float* op = out + ((int64_t)bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim + dd;
          *reinterpret_cast<float4*>(op) = make_float4(acc.x * iz, acc.y * iz, acc.z * iz, acc.w * iz);
        } else {                // one split of the row: partials for the combine
          float* pp = a.part + ((sel * a.n_split + split) * a.G + h) * kPartStride;
          *reinterpret_cast<float4*>(pp + 4 + dd) = acc;
          if (dd == 0) {
            pp[0] = Mw;
            pp[1] = Z;
          }
        }
      }
    }
  }
}

}  // namespace

// Head layout by group size: G <= 8 (8-lane records, 8 waves), G <= 16 (16-lane
// records, 8 waves), G <= 32 (two head blocks, 4 waves with up to 512 registers).
template <bool kFp8, bool kVec>
static void launch_scan_g(const ScanArgs& a, dim3 grid, hipStream_t st, const KernelEvents* ev) {
  if (a.G <= 8)
    launch_on(ev, scan_mfma_kernel<kFp8, kVec, 1, false, 512>, grid, dim3(512), 0, st, a);
  else if (a.G <= 16)
    launch_on(ev, scan_mfma_kernel<kFp8, kVec, 1, true, 512>, grid, dim3(512), 0, st, a);
  else
    launch_on(ev, scan_mfma_kernel<kFp8, kVec, 2, true, 256>, grid, dim3(256), 0, st, a);
}

// the block comparator's scan, same head layouts (per-block sums in blse_heads_of(G) slots)
template <bool kFp8, bool kVec>
static void launch_scan_blocks_g(const ScanArgs& a, dim3 grid, hipStream_t st, const KernelEvents* ev) {
  if (a.G <= 8)
    launch_on(ev, scan_mfma_kernel<kFp8, kVec, 1, false, 512, true>, grid, dim3(512), 0, st, a);
  else if (a.G <= 16)
    launch_on(ev, scan_mfma_kernel<kFp8, kVec, 1, true, 512, true>, grid, dim3(512), 0, st, a);
  else
    launch_on(ev, scan_mfma_kernel<kFp8, kVec, 2, true, 256, true>, grid, dim3(256), 0, st, a);
}

hipError_t launch_scan_mfma_blocks(const ScanArgs& a, bool fp8, int B, hipStream_t st, const KernelEvents* ev) {
  if (a.G > kMaxHeads || a.blse == nullptr) return hipErrorInvalidValue;
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (fp8 && a.cap % 4 == 0)
    launch_scan_blocks_g<true, true>(a, grid, st, ev);
  else if (fp8)
    launch_scan_blocks_g<true, false>(a, grid, st, ev);
  else
    launch_scan_blocks_g<false, false>(a, grid, st, ev);
  return hipGetLastError();
}

hipError_t launch_scan_mfma(const ScanArgs& a, bool fp8, int B, hipStream_t st, const KernelEvents* ev) {
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (fp8 && a.cap % 4 == 0)
    launch_scan_g<true, true>(a, grid, st, ev);
  else if (fp8)
    launch_scan_g<true, false>(a, grid, st, ev);
  else
    launch_scan_g<false, false>(a, grid, st, ev);
  return hipGetLastError();
}

template <bool kFp8>
static void launch_gather_g(const ScanArgs& a, float* out, dim3 grid, hipStream_t st, const KernelEvents* ev) {
  if (a.G <= 8)
    launch_on(ev, gather_mfma_kernel<kFp8, 1, false, 512>, grid, dim3(512), 0, st, a, out);
  else if (a.G <= 16)
    launch_on(ev, gather_mfma_kernel<kFp8, 1, true, 512>, grid, dim3(512), 0, st, a, out);
  else
    launch_on(ev, gather_mfma_kernel<kFp8, 2, true, 256>, grid, dim3(256), 0, st, a, out);
}

hipError_t launch_gather_mfma(const ScanArgs& a, float* out, bool fp8, int B, hipStream_t st,
                              const KernelEvents* ev) {
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (fp8)
    launch_gather_g<true>(a, out, grid, st, ev);
  else
    launch_gather_g<false>(a, out, grid, st, ev);
  return hipGetLastError();
}

}  // namespace hs2
