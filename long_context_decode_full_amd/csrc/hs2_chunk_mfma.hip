// Matrix-core scan for a chunk of query tokens (q_len > 1): the Full Attention layer
// of a Hybrid Block for every token of an appended chunk, causal inside the chunk,
// with the record-path outputs of the decode scan (online-softmax partials per
// (token, head, split), a 2-byte bound record per (token, position) and a key
// histogram per (token, split)), or, in block mode, log2 of the sum of 2^logit over
// each aligned 64-position block per (token, head).
//
// HySparse2 article, section 02 "KV Reuse" (the full layer's own attention scores
// decide what the sparse layers reuse) and section 03 (selection per token: every
// query token of the chunk gets its own window and top-k).
//
// A workgroup owns one position split of one (sequence, KV head) and 256 query rows:
// 256 / kGp tokens of kGp head slots each (kGp = 8, 16 or 32: the group size rounded
// up; slots >= G are zero), so it reads every K/V row of its split once for all of
// them.  Per iteration of 64 positions the K and V tiles go through LDS (two stages:
// the next tiles are stored while the current ones are read; one barrier, at the end of
// the iteration, which also completes the stores of the stage the next one reads); fp8 K codes are widened to bf16
// as they are staged (V: see below).  Wave w owns 32 / kGp tokens as two query tiles of 16 rows, a
// token's heads spread over both tiles (head = (kGp / 2) tile + lane % (kGp / 2)).
// The scores are formed transposed, S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (A = K
// rows from the K
// tile, lane: position i, dims 32s + 8grp; B = Q^T from registers, lane: query row
// i, the same dims), so a lane's accumulators are 4 positions (4grp + v) of one query
// row (i) and the probabilities are already in the B-operand layout of the second
// product: O^T = V^T P^T with A = V^T read transposed from the V tile
// (ds_read_b64_tr_b16, rows 4grp..4grp+3 of two position tiles per lane) and B = the
// lane's own 8 probabilities of a 32-position block (P never goes through LDS).  The V
// tile is staged as fp16 (a bf16 value below 2^16 in magnitude exactly; an fp8 code
// times its row's scale with one rounding, <= 2^-12) and P is rounded to fp16, one MFMA
// per product (error <= 2^-12 relative per term); a split whose V has a tile outside
// that range (some |v| >= 2^16, or every |v| < 2^-6) starts again with P as a bf16 high
// part and a bf16 residual (two MFMAs, error ~2^-16; fp8: V as exact bf16 codes, the
// scale on P), the form HS2_FLAG_EXACT_PV always takes.  A block's P V is interleaved with the vector work of the next block (the
// matrix core and the VALU overlap only in part, so this mostly keeps both busy).
//   softmax per query row: the lane's 16 values per iteration, the running maximum
//     raised lazily by 8 (log2 units) with a max over the 4 row groups.
//   record per (token, position): log2 of the sum over the token's heads of 2^logit,
//     from the probabilities already formed: with U the largest running maximum of
//     the token's heads, e = U + log2 sum_h p_h 2^(m_h - U), the two tiles added
//     in-lane, then a DPP reduce-scatter over the token's kGp / 2 head lanes; sums
//     below 2^-100 (terms lost to underflow could matter there) take the exact form on
//     a wave-uniform branch.
#include "hs2_rowops.h"

#include <type_traits>

namespace hs2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2v_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kCThreads = 512;                 // 8 waves
constexpr int kCRows = 256;                    // query rows per workgroup
constexpr int kCPos = 64;                      // positions per iteration
constexpr float kCSlack = 8.0f;
constexpr int kVPre = 4;                       // V^T operands read ahead of the records (of 8)
constexpr float kMFloor = -1.0e30f;            // initial running maximum (below any logit)
// Staged rows are padded so that the fragment reads spread over the LDS banks: the K
// rows (16-byte reads, lane = row) by 16 bytes, the V rows (8-byte transposed reads,
// four lanes per row over four consecutive rows) by 32 bytes.
constexpr int kKRow = 272;                     // bytes per staged K row (256 + 16 pad)
constexpr int kVRow = 288;                     // bytes per staged V row (256 + 32 pad)
constexpr int kKTile = kCPos * kKRow;
constexpr int kVTile = kCPos * kVRow;
constexpr int kStage = kKTile + kVTile;        // K and V tiles of one iteration
constexpr int kHistWords = kFastBins / 2;      // two u16 counters per word
// fp8 caches: the per-position K and V scales of both stages, after the tiles
constexpr int kScaleBytes = 2 * 2 * kCPos * 4;

template <int kGp>
constexpr int tokens_per_wg() { return kCRows / kGp; }
template <int kGp, bool kBlockMode, bool kFp8>
constexpr int chunk_lds_bytes() {
  return 2 * kStage + (kFp8 ? kScaleBytes : 0) + (kBlockMode ? 0 : tokens_per_wg<kGp>() * kHistWords * 4);
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// the same product on fp16 operands (the bits of a and b are fp16 values)
__device__ __forceinline__ f32x4_t mfma16h(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                               0, 0);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2v_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
// two floats to fp16 (round to nearest even), packed
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f32x2v_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2_t));
}
// V tile range for the fp16 form, on the bf16 magnitude bits: every |v| below 2^16 (bf16
// values there are exact in fp16; inf and NaN are above) and some |v| at least 2^-6
// (fp16 subnormals then cost at most 2^-25 absolute, far below the 2^-12 relative
// rounding of P at that magnitude)
constexpr uint32_t kV16MaxBits = 0x4780u;   // 2^16
constexpr uint32_t kV16MinBits = 0x3C80u;   // 2^-6
// the same tests on fp16 bits (fp8 V, scaled and rounded to fp16 as staged)
constexpr uint32_t kF16InfBits = 0x7C00u;   // inf; NaN above
constexpr uint32_t kF16MinBits = 0x2400u;   // 2^-6
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Reductions over the lanes of one token's heads inside a 16-lane row: 4 lanes (each
// quad separately), 8 (lanes 0-7 and 8-15 separately) or all 16.
template <int kLanes>
__device__ __forceinline__ float head_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (kLanes >= 8) x += dpp<kDppMirror8>(x);
  if constexpr (kLanes == 16) x += dpp<kDppRor8>(x);
  return x;
}
template <int kLanes>
__device__ __forceinline__ float head_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (kLanes >= 8) x = fmaxf(x, dpp<kDppMirror8>(x));
  if constexpr (kLanes == 16) x = fmaxf(x, dpp<kDppRor8>(x));
  return x;
}

// Combine the 4 lanes i, i+16, i+32, i+48 (the four row groups, which hold other
// positions of the same query row) with the permlane swaps.  The swap results are
// copied to scalars before any bit cast (a bit cast of a vector element reads
// element 0 here).
template <bool kMax>
__device__ __forceinline__ float across_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = s32[0], a1 = s32[1];
  x = kMax ? fmaxf(__uint_as_float(a0), __uint_as_float(a1)) : __uint_as_float(a0) + __uint_as_float(a1);
  const uint32_t w = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
  const uint32_t c0 = s16[0], c1 = s16[1];
  return kMax ? fmaxf(__uint_as_float(c0), __uint_as_float(c1)) : __uint_as_float(c0) + __uint_as_float(c1);
}

// A token's kGp head slots are kGp / 2 lanes of the row (w16 % (kGp / 2)) in both query
// tiles of the wave: head = (kGp / 2) qt + w16 % (kGp / 2).  Sums and maxima over the
// token's heads therefore combine the two tiles in-lane and kGp / 2 lanes by DPP.
template <int kGp>
__device__ __forceinline__ void token_sums(const float (&x)[2], float (&out)[2]) {
  const float s = head_sum<kGp / 2>(x[0]) + head_sum<kGp / 2>(x[1]);
  out[0] = s;
  out[1] = s;
}
template <int kGp>
__device__ __forceinline__ void token_maxes(const float (&x)[2], float (&out)[2]) {
  const float s = fmaxf(head_max<kGp / 2>(x[0]), head_max<kGp / 2>(x[1]));
  out[0] = s;
  out[1] = s;
}

// Records of a 32-position block: every lane forms, for each of the block's 8
// positions it holds (index 4 tt + v: position tile tt of the block, position
// 4 grp + v of the tile), its two tiles' c p summed; these 8 values are then
// reduce-scattered over the token's kGp / 2 head lanes (each DPP step halves the
// values a lane keeps and adds its partner's other half), so that every lane ends with
// whole records:
//   8 head slots:  4 lanes, 2 records a lane: indices 2 (w16 & 3) + j (adjacent positions);
//   16 slots:      8 lanes, 1 record a lane: index w16 & 7;
//   32 slots:     16 lanes, 1 record per lane pair: index w16 >> 1 (lanes w16, w16 ^ 1 alike).
template <int kGp>
constexpr int kRecOut = kGp == 8 ? 2 : 1;
template <int kGp>
__device__ __forceinline__ int rec_index(int w16, int j) {
  return kGp == 8 ? 2 * (w16 & 3) + j : kGp == 16 ? (w16 & 7) : (w16 >> 1);
}
template <int kGp>
__device__ __forceinline__ bool rec_writer(int w16) {
  return kGp == 32 ? (w16 & 1) == 0 : true;
}
// keep x[j] or x[j + N] (by `upper`) plus the partner lane's other one
template <int CTRL, int N>
__device__ __forceinline__ void rs_step(const float* x, float* y, bool upper) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float keep = upper ? x[j + N] : x[j];
    const float send = upper ? x[j] : x[j + N];
    y[j] = keep + dpp<CTRL>(send);
  }
}
template <int kGp>
__device__ __forceinline__ void reduce_scatter(const float (&x)[8], int w16, float (&out)[kRecOut<kGp>]) {
  const bool b3 = (w16 & 8) != 0, b2 = (w16 & 4) != 0, b1 = (w16 & 2) != 0, b0 = (w16 & 1) != 0;
  float a4[4], a2[2], a1[1];
  if constexpr (kGp == 8) {
    rs_step<kDppXor2, 4>(x, a4, b1);
    rs_step<kDppXor1, 2>(a4, a2, b0);
    out[0] = a2[0];
    out[1] = a2[1];
  } else if constexpr (kGp == 16) {
    rs_step<kDppMirror8, 4>(x, a4, b2);   // partner 7 - i: bit 2 differs
    rs_step<kDppXor2, 2>(a4, a2, b1);
    rs_step<kDppXor1, 1>(a2, a1, b0);
    out[0] = a1[0];
  } else {
    rs_step<kDppRor8, 4>(x, a4, b3);
    rs_step<kDppMirror8, 2>(a4, a2, b2);
    rs_step<kDppXor2, 1>(a2, a1, b1);
    out[0] = a1[0] + dpp<kDppXor1>(a1[0]);
  }
}

// kBlockMode: false: records + key histograms; true: per-block sums.  kFp8: the cache
// holds E4M3FN codes with one fp32 scale per (position, KV head): the tiles are
// converted to bf16 (exactly) as they are staged, the scores take the K scale of their
// position, and the P^T operands of P V the V scale.
template <int kGp, bool kBlockMode, bool kFp8>
__global__ __launch_bounds__(kCThreads, 1) void chunk_mfma_kernel(ScanArgs a) {
  constexpr int kTPW = tokens_per_wg<kGp>();
  __shared__ __attribute__((aligned(16))) uint8_t lds[chunk_lds_bytes<kGp, kBlockMode, kFp8>()];
  // V staged as fp16 (bf16 values as they are, fp8 codes times their row's scale) unless
  // the caller asks for the two-part form; per stage and wave, bit 0: some staged value
  // out of the fp16 range (or not finite), bit 1: some |v| >= 2^-6
  constexpr bool kV16 = true;
  __shared__ uint32_t vflags[2][kCThreads / 64];
  uint32_t* shist = reinterpret_cast<uint32_t*>(lds + 2 * kStage + (kFp8 ? kScaleBytes : 0));
  // per-position scales of stage st: K (kv = 0) or V (kv = 1)
  auto stage_scales = [&](int st, int kv) { return reinterpret_cast<float*>(lds + 2 * kStage) + (2 * st + kv) * kCPos; };

  // blockIdx.x = split * token groups + group: the groups of one split are adjacent
  const int n_tgroups = (a.Lq + kTPW - 1) / kTPW;
  const int tgroup = blockIdx.x % n_tgroups;
  const int split = blockIdx.x / n_tgroups;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int w16 = lane & 15;

  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  const int tok0 = tgroup * kTPW;                   // first token of this workgroup
  const int ntok = min(kTPW, a.Lq - tok0);          // tokens present (may be <= 0)
  const int64_t p_begin = (int64_t)split * a.split_len;
  // the last present token sees the most positions
  int64_t n_last = ctx - a.Lq + (tok0 + ntok - 1) + 1;
  n_last = n_last < 0 ? 0 : n_last;
  int64_t p_end = p_begin + a.split_len;
  p_end = p_end < n_last ? p_end : n_last;
  if (ntok <= 0) return;
  // a split past every visible position of this group's tokens has nothing to write:
  // the combine folds, per token, only the splits below its visible length (split 0
  // always runs: it also clears the merged histograms)
  if (split > 0 && p_begin >= n_last) return;
  const int64_t sel_tok0 = ((int64_t)b * a.Lq + tok0) * a.Hkv + g;   // sel of token tok0; +Hkv per token

  constexpr bool want_rec = !kBlockMode;
  if constexpr (want_rec) {
    for (int i = tid; i < kTPW * kHistWords; i += kCThreads) shist[i] = 0u;
    if (split == 0) {
      for (int i = tid; i < ntok * kMergedWords; i += kCThreads) {
        const int t = i / kMergedWords;
        a.hist_merged[(sel_tok0 + (int64_t)t * a.Hkv) * kSelWords + kSelHist1Off + (i - t * kMergedWords)] = 0u;
      }
    }
  }

  // this lane's query row in tile qt: r = 32 wave + 16 qt + w16 = (token, head slot)
  int tokl[2], head[2];
  bool valid[2];       // a present token and a real head
  int32_t pj[2];       // last visible position of the token (positions < cap < 2^31)
  int32_t w0j[2];      // first window position (candidates are < w0j)
  bf16x8_t qf[2][4];   // Q^T fragments (B operand): dims 32s + 8grp of the lane's query row
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    tokl[qt] = (32 / kGp) * wave + w16 / (kGp / 2);   // the same in both tiles
    head[qt] = (kGp / 2) * qt + w16 % (kGp / 2);
    valid[qt] = tokl[qt] < ntok && head[qt] < a.G;
    const int64_t pp = ctx - a.Lq + tok0 + tokl[qt];
    pj[qt] = (int32_t)pp;
    const int64_t w0 = pp + 1 - a.window;
    w0j[qt] = (int32_t)(w0 < 0 ? 0 : w0);
    const uint16_t* qh = a.q + (((int64_t)b * a.Lq + tok0 + tokl[qt]) * a.Hq + (int64_t)g * a.G + head[qt]) * kHeadDim +
                         8 * grp;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[qt][s] = as_bf16x8(valid[qt] ? *reinterpret_cast<const uint4*>(qh + 32 * s) : make_uint4(0u, 0u, 0u, 0u));
  }

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  constexpr int kRowBytes = kFp8 ? 128 : 256;   // bytes of one cache row
  const uint8_t* kb = a.k + head_row0 * kRowBytes;
  const uint8_t* vb = a.v + head_row0 * kRowBytes;
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float* vsb = kFp8 ? a.v_scale + head_row0 : nullptr;

  f32x4_t o[2][8];     // O^T: dims 16 bb + 4 grp + v of the lane's query row
  float m[2], z[2];    // running maximum (log2 units, equal in the 4 row groups), this lane's share of Z
  float U[2], c[2];    // record scale: U = the token's largest running maximum, c = 2^(m - U) (0: no head)
  auto record_scale = [&]() {
    float mv[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) mv[qt] = valid[qt] ? m[qt] : kMFloor;
    token_maxes<kGp>(mv, U);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) c[qt] = valid[qt] ? fast_exp2(m[qt] - U[qt]) : 0.0f;
  };

  const int nit = p_end > p_begin ? (int)((p_end - p_begin + kCPos - 1) / kCPos) : 0;
  const int32_t last = (int32_t)(p_end - 1);
  // this thread's share of a tile load: bf16 rows (tid >> 4) + 32 r, 16 bytes at
  // (tid & 15); fp8 row (tid >> 3), 16 codes at (tid & 7), and with tid < 64 the K and V
  // scales of position tid.  (Named registers, not arrays: small arrays live across the
  // loop got placed in LDS / scratch by the compiler.)
  const bool f16v = kV16 && a.exact_pv == 0;   // workgroup-uniform
  const int lrow = kFp8 ? (tid >> 3) : (tid >> 4);
  const int lcol = kFp8 ? (tid & 7) * 16 : (tid & 15) * 16;
  uint4 kr0, kr1, vr0, vr1;
  float ksr = 0.0f, vsr = 0.0f, vsrow = 0.0f;   // vsrow: V scale of the row this thread stages (fp8)
  auto load_tiles = [&](int32_t base) {
    const uint32_t row0 = (uint32_t)min(base + lrow, last);
    kr0 = *reinterpret_cast<const uint4*>(kb + (uint64_t)row0 * kRowBytes + lcol);
    vr0 = *reinterpret_cast<const uint4*>(vb + (uint64_t)row0 * kRowBytes + lcol);
    if constexpr (kFp8) {
      vsrow = vsb[row0];
      if (tid < kCPos) {
        const uint32_t srow = (uint32_t)min(base + tid, last);
        ksr = ksb[srow];
        vsr = vsb[srow];
      }
    } else {
      const uint32_t row1 = (uint32_t)min(base + lrow + 32, last);
      kr1 = *reinterpret_cast<const uint4*>(kb + (uint64_t)row1 * 256 + lcol);
      vr1 = *reinterpret_cast<const uint4*>(vb + (uint64_t)row1 * 256 + lcol);
    }
  };
  // kHt true: bf16 V rows go to LDS as fp16, with the stage's range flags
  auto store_tiles = [&](int stg, auto kHt) {
    constexpr bool kH = decltype(kHt)::value;
    uint8_t* st = lds + stg * kStage;
    if constexpr (kFp8) {
      // 16 codes -> 16 bf16 (exact), bytes 2 lcol .. 2 lcol + 31 of the staged row
      auto widen = [](uint4 c, uint4& lo, uint4& hi) {
        lo = make_uint4(fp8x2_to_bf16x2(c.x, false), fp8x2_to_bf16x2(c.x, true), fp8x2_to_bf16x2(c.y, false),
                        fp8x2_to_bf16x2(c.y, true));
        hi = make_uint4(fp8x2_to_bf16x2(c.z, false), fp8x2_to_bf16x2(c.z, true), fp8x2_to_bf16x2(c.w, false),
                        fp8x2_to_bf16x2(c.w, true));
      };
      uint4 lo, hi;
      widen(kr0, lo, hi);
      *reinterpret_cast<uint4*>(st + lrow * kKRow + 2 * lcol) = lo;
      *reinterpret_cast<uint4*>(st + lrow * kKRow + 2 * lcol + 16) = hi;
      if constexpr (kH) {
        // V: 16 codes times the row's scale, rounded to fp16 (one rounding, <= 2^-12
        // relative); the range test on the fp16 magnitude bits (a value beyond fp16's
        // range became inf, a NaN code stays NaN: both at or above 0x7C00)
        u16x2_t mmax = {0, 0};
        auto scaled = [&](uint32_t c, uint32_t& h0, uint32_t& h1) {
          const f32x2_t a0 = fp8x2_to_f32(c, false), a1 = fp8x2_to_f32(c, true);
          h0 = pack_f16(a0[0] * vsrow, a0[1] * vsrow);
          h1 = pack_f16(a1[0] * vsrow, a1[1] * vsrow);
          mmax = __builtin_elementwise_max(mmax, __builtin_bit_cast(u16x2_t, h0 & 0x7FFF7FFFu));
          mmax = __builtin_elementwise_max(mmax, __builtin_bit_cast(u16x2_t, h1 & 0x7FFF7FFFu));
        };
        uint32_t h[8];
        scaled(vr0.x, h[0], h[1]);
        scaled(vr0.y, h[2], h[3]);
        scaled(vr0.z, h[4], h[5]);
        scaled(vr0.w, h[6], h[7]);
        *reinterpret_cast<uint4*>(st + kKTile + lrow * kVRow + 2 * lcol) = make_uint4(h[0], h[1], h[2], h[3]);
        *reinterpret_cast<uint4*>(st + kKTile + lrow * kVRow + 2 * lcol + 16) = make_uint4(h[4], h[5], h[6], h[7]);
        const uint32_t mm = max((uint32_t)mmax[0], (uint32_t)mmax[1]);
        const uint64_t ov = __builtin_amdgcn_ballot_w64(mm >= kF16InfBits);
        const uint64_t sm = __builtin_amdgcn_ballot_w64(mm >= kF16MinBits);
        if (lane == 0) vflags[stg][wave] = (ov != 0ull ? 1u : 0u) | (sm != 0ull ? 2u : 0u);
      } else {
        widen(vr0, lo, hi);
        *reinterpret_cast<uint4*>(st + kKTile + lrow * kVRow + 2 * lcol) = lo;
        *reinterpret_cast<uint4*>(st + kKTile + lrow * kVRow + 2 * lcol + 16) = hi;
      }
      if (tid < kCPos) {
        stage_scales(stg, 0)[tid] = ksr;
        stage_scales(stg, 1)[tid] = vsr;
      }
    } else {
      *reinterpret_cast<uint4*>(st + lrow * kKRow + lcol) = kr0;
      *reinterpret_cast<uint4*>(st + (lrow + 32) * kKRow + lcol) = kr1;
      if constexpr (kH) {
        // 8 bf16 -> 8 fp16 per store (exact inside the range the flags check); the
        // largest magnitude bits of each half-word lane
        u16x2_t mmax = {0, 0};
        auto widen = [&](uint4 w) {
          const uint32_t x[4] = {w.x, w.y, w.z, w.w};
          uint32_t h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            h[i] = pack_f16(__uint_as_float(x[i] << 16), __uint_as_float(x[i] & 0xFFFF0000u));
            mmax = __builtin_elementwise_max(mmax, __builtin_bit_cast(u16x2_t, x[i] & 0x7FFF7FFFu));
          }
          return make_uint4(h[0], h[1], h[2], h[3]);
        };
        *reinterpret_cast<uint4*>(st + kKTile + lrow * kVRow + lcol) = widen(vr0);
        *reinterpret_cast<uint4*>(st + kKTile + (lrow + 32) * kVRow + lcol) = widen(vr1);
        const uint32_t mm = max((uint32_t)mmax[0], (uint32_t)mmax[1]);
        const bool over = mm >= kV16MaxBits;
        const bool some = mm >= kV16MinBits;
        const uint64_t ov = __builtin_amdgcn_ballot_w64(over);
        const uint64_t sm = __builtin_amdgcn_ballot_w64(some);
        if (lane == 0) vflags[stg][wave] = (ov != 0ull ? 1u : 0u) | (sm != 0ull ? 2u : 0u);
      } else {
        *reinterpret_cast<uint4*>(st + kKTile + lrow * kVRow + lcol) = vr0;
        *reinterpret_cast<uint4*>(st + kKTile + (lrow + 32) * kVRow + lcol) = vr1;
      }
    }
  };
  // One pass over the split: P V with fp16 V and P (kHt true) or with the two-part
  // bf16 split of P.  The fp16 pass returns false, leaving at the first stage whose V
  // lies outside the fp16 range; the split then runs again in the two-part form (the
  // records it wrote are written again with the same values, the histograms restart).
  auto run_split = [&](auto kHt) -> bool {
    constexpr bool kH = decltype(kHt)::value;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
      for (int d = 0; d < 8; ++d) o[qt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m[qt] = kMFloor;   // finite, so exp2(l - m) needs no -inf test
      z[qt] = 0.0f;
    }
    if constexpr (want_rec) record_scale();
    if (nit > 0) {
      load_tiles((int32_t)p_begin);
      store_tiles(0, kHt);
      load_tiles((int32_t)p_begin + kCPos);
    }
    __syncthreads();   // stage 0 and the cleared histograms are ready
    const float sl2 = a.scale_log2;
    const int32_t first_pj = (int32_t)(ctx - a.Lq + tok0);   // the workgroup's first token sees least

    // K fragments of the first position tile, read one iteration ahead (the next stage
    // is visible once the barrier after its stores has passed)
    auto read_kf = [&](const uint8_t* ks, int pt, bf16x8_t (&kf)[4]) {
  #pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(ks + (pt * 16 + w16) * kKRow + 64 * s + 16 * grp));
    };
    bf16x8_t kpre[4];
    if (nit > 0) read_kf(lds, 0, kpre);
    for (int it = 0; it < nit; ++it) {
      const int32_t P0 = (int32_t)p_begin + it * kCPos;
      const uint8_t* ks = lds + (it & 1) * kStage;
      const uint8_t* vs = ks + kKTile;
      // the next iteration's tiles into the other stage (its last readers finished the
      // previous iteration before the barrier that ended it), then the loads after them
      store_tiles((it + 1) & 1, kHt);
      load_tiles(P0 + 2 * kCPos);
      // this stage is complete (its stores came before the barrier that ended the last
      // iteration); its first K fragments
      if (it > 0) read_kf(ks, 0, kpre);
      if constexpr (kH) {
        // this stage's V outside the fp16 range: the split is given up (every wave reads
        // the same flags here, right after the barrier, so all leave together)
        uint32_t f = 0u;
  #pragma unroll
        for (int w = 0; w < kCThreads / 64; ++w) f |= vflags[it & 1][w];
        if ((f & 1u) != 0u || (f & 2u) == 0u) return false;
      }

      // ---- S^T = K Q^T for 4 position tiles x 2 query tiles
      f32x4_t sacc[4][2];
      // the MFMA groups run at raised wave priority: when the two waves of a SIMD are
      // in different phases, the matrix core starts as soon as it is free and the
      // other wave's vector work fills the issue slots in between
      __builtin_amdgcn_s_setprio(1);
  #pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        bf16x8_t kf[4];
        if (pt == 0) {
  #pragma unroll
          for (int s = 0; s < 4; ++s) kf[s] = kpre[s];
        } else {
          read_kf(ks, pt, kf);
        }
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          f32x4_t d = {0.f, 0.f, 0.f, 0.f};
  #pragma unroll
          for (int s = 0; s < 4; ++s) d = mfma16(kf[s], qf[qt][s], d);
          sacc[pt][qt] = d;
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // raw scores; the log2-domain logit is scale_log2 * s (scale_log2 > 0), formed
      // inside the exp2 as fma(s, scale_log2, -m).  The causal mask only where some
      // position lies beyond the first token's last visible one (wave-uniform branch).
      // (fp8: the score of position i is scale_i * q.k_i, k_i the stored codes)
      float l[2][4][4];
  #pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        float4 ksc = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        if constexpr (kFp8) ksc = *reinterpret_cast<const float4*>(stage_scales(it & 1, 0) + pt * 16 + 4 * grp);
        const float kv4[4] = {ksc.x, ksc.y, ksc.z, ksc.w};
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt)
  #pragma unroll
          for (int v = 0; v < 4; ++v) l[qt][pt][v] = kFp8 ? sacc[pt][qt][v] * kv4[v] : sacc[pt][qt][v];
      }
      if (P0 + kCPos - 1 > first_pj) {
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt)
  #pragma unroll
          for (int pt = 0; pt < 4; ++pt)
  #pragma unroll
            for (int v = 0; v < 4; ++v)
              l[qt][pt][v] = P0 + pt * 16 + 4 * grp + v <= pj[qt] ? l[qt][pt][v] : kNegInf;
      }

      // ---- online softmax per query row: a lane test and one ballot per iteration; the
      // exact row maximum (over the 4 row groups) only on the rare raise
      {
        float x[2];
        bool up_any = false;
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          float mx = kNegInf;
  #pragma unroll
          for (int pt = 0; pt < 4; ++pt)
  #pragma unroll
            for (int v = 0; v < 4; ++v) mx = fmaxf(mx, l[qt][pt][v]);
          x[qt] = mx * sl2;
          up_any |= x[qt] > m[qt] + kCSlack;
        }
        if (wave_any(up_any)) {
  #pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const float mx = across_groups<true>(x[qt]);
            const bool up = mx > m[qt] + kCSlack;
            const float mn = up ? mx : m[qt];
            const float alpha = up ? fast_exp2(m[qt] - mn) : 1.0f;
  #pragma unroll
            for (int d = 0; d < 8; ++d) o[qt][d] *= alpha;
            z[qt] *= alpha;
            m[qt] = mn;
          }
          if constexpr (want_rec) record_scale();
        }
      }

      // ---- probabilities, records / block sums, P^T V^T per 32-position block.
      // The work of the two blocks is ordered so that each block's P V runs on the matrix
      // cores while this wave's vector work continues: block 0's probabilities, operands
      // and records first; then block 0's P V interleaved with block 1's probabilities,
      // operands and record sums; then block 1's P V interleaved with its record
      // reduction; block 1's records last.  (Each accumulator still takes the high part
      // and then the residual of its block, so the sums are those of a plain loop.)
      float bsum[2] = {0.f, 0.f};
      // A operands of a block's P V: V^T of dim block d, rows 4grp..4grp+3 of the block's
      // two tiles
      auto read_vt = [&](int kb2, int d) {
        const uint8_t* tr0 = vs + (32 * kb2 + 4 * grp + (w16 >> 2)) * kVRow + 8 * (w16 & 3) + 32 * d;
        const uint8_t* tr1 = tr0 + 16 * kVRow;
        const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)tr0);
        const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)tr1);
        const uint2 w0 = __builtin_bit_cast(uint2, x0);
        const uint2 w1 = __builtin_bit_cast(uint2, x1);
        return as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
      };
      // p[qt][tile of the block][v]
      auto probabilities = [&](int kb2, float (&p)[2][2][4]) {
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt)
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt)
  #pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float x = fast_exp2(__builtin_fmaf(l[qt][2 * kb2 + tt][v], sl2, -m[qt]));   // -inf -> 0
              p[qt][tt][v] = x;
              z[qt] += x;
              if constexpr (kBlockMode) bsum[qt] += x;
            }
      };
      // B operands: P^T of the block, k slot 8 grp + u <-> tile u / 4, position 4 grp + u % 4
      // (fp8: times the V scale of the position): fp16 (kH), or a bf16 high part and a bf16
      // residual
      auto operands = [&](auto kHt, int kb2, const float (&p)[2][2][4], bf16x8_t (&ph)[2], bf16x8_t (&pl)[2]) {
        constexpr bool kH = decltype(kHt)::value;
        float vsc[2][4] = {{1.0f, 1.0f, 1.0f, 1.0f}, {1.0f, 1.0f, 1.0f, 1.0f}};
        if constexpr (kFp8 && !kH) {   // fp16 form: the V scale is in the staged V
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const float4 s4 = *reinterpret_cast<const float4*>(stage_scales(it & 1, 1) + (2 * kb2 + tt) * 16 + 4 * grp);
            vsc[tt][0] = s4.x;
            vsc[tt][1] = s4.y;
            vsc[tt][2] = s4.z;
            vsc[tt][3] = s4.w;
          }
        }
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          uint32_t hw[4], lw[4];
  #pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float x0 = p[qt][u >> 1][2 * (u & 1)] * ((kFp8 && !kH) ? vsc[u >> 1][2 * (u & 1)] : 1.0f);
            const float x1 = p[qt][u >> 1][2 * (u & 1) + 1] * ((kFp8 && !kH) ? vsc[u >> 1][2 * (u & 1) + 1] : 1.0f);
            if constexpr (kH) {
              hw[u] = pack_f16(x0, x1);
              lw[u] = 0u;
            } else {
              hw[u] = pack_bf16(x0, x1);
              lw[u] = pack_bf16(x0 - __uint_as_float(hw[u] << 16), x1 - __uint_as_float(hw[u] & 0xFFFF0000u));
            }
          }
          ph[qt] = as_bf16x8(make_uint4(hw[0], hw[1], hw[2], hw[3]));
          pl[qt] = as_bf16x8(make_uint4(lw[0], lw[1], lw[2], lw[3]));
        }
      };
      auto pv = [&](auto kHt, int kb2, const bf16x8_t (&avp)[kVPre], const bf16x8_t (&ph)[2], const bf16x8_t (&pl)[2]) {
        constexpr bool kH = decltype(kHt)::value;
  #pragma unroll
        for (int d = 0; d < 8; ++d) {
          const bf16x8_t av = d < kVPre ? avp[d < kVPre ? d : 0] : read_vt(kb2, d);
  #pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            if constexpr (kH) {
              o[qt][d] = mfma16h(av, ph[qt], o[qt][d]);
            } else {
              o[qt][d] = mfma16(av, ph[qt], o[qt][d]);
              o[qt][d] = mfma16(av, pl[qt], o[qt][d]);
            }
          }
        }
      };
      // Records of a block's 32 positions: per (token, position) the sum over the token's
      // heads of c p (both tiles in-lane: rec_sums; then the head lanes: rec_reduce), then
      // the exact form where a sum underflowed (rec_write); a token's rows share tokl, pj
      // and w0j.
      constexpr int kOut = kRecOut<kGp>;
      struct RecState {
        int32_t pos[kOut];
        bool live[kOut], tiny[kOut];
        float e[kOut];
        bool any_tiny;
      };
      auto rec_sums = [&](const float (&p)[2][2][4], float (&x)[8]) {
  #pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = p[0][i >> 2][i & 3] * c[0] + p[1][i >> 2][i & 3] * c[1];
      };
      auto rec_reduce = [&](int kb2, const float (&x)[8], RecState& r) {
        float sum[kOut];
        reduce_scatter<kGp>(x, w16, sum);
        r.any_tiny = false;
  #pragma unroll
        for (int j = 0; j < kOut; ++j) {
          const int idx = rec_index<kGp>(w16, j);
          r.pos[j] = P0 + (2 * kb2 + (idx >> 2)) * 16 + 4 * grp + (idx & 3);
          r.live[j] = rec_writer<kGp>(w16) && r.pos[j] <= pj[0] && tokl[0] < ntok;
          r.tiny[j] = r.live[j] && !(sum[j] >= 0x1p-100f);
          r.any_tiny |= r.tiny[j];
          r.e[j] = U[0] + __builtin_amdgcn_logf(sum[j]);
        }
      };
      auto rec_write = [&](int kb2, RecState& r) {
        const int tl = tokl[0];
        if (wave_any(r.any_tiny)) {
          // exact: max and sum of 2^(l - max) over the token's heads, for every value of
          // the lane (all-reduce: every lane takes part in the DPP reductions)
          float ex_own[kOut];
  #pragma unroll
          for (int j = 0; j < kOut; ++j) ex_own[j] = 0.0f;
  #pragma unroll
          for (int tt = 0; tt < 2; ++tt)
  #pragma unroll
            for (int v = 0; v < 4; ++v) {
              float lv[2], rmax[2], ex[2], sums[2];
  #pragma unroll
              for (int qt = 0; qt < 2; ++qt) lv[qt] = valid[qt] ? l[qt][2 * kb2 + tt][v] * sl2 : kNegInf;
              token_maxes<kGp>(lv, rmax);
  #pragma unroll
              for (int qt = 0; qt < 2; ++qt) {
                rmax[qt] = fmaxf(rmax[qt], kMFloor);   // finite: exp2 of -inf is 0
                ex[qt] = fast_exp2(lv[qt] - rmax[qt]);
              }
              token_sums<kGp>(ex, sums);
              const float val = rmax[0] + __builtin_amdgcn_logf(sums[0]);
  #pragma unroll
              for (int j = 0; j < kOut; ++j) ex_own[j] = rec_index<kGp>(w16, j) == 4 * tt + v ? val : ex_own[j];
            }
  #pragma unroll
          for (int j = 0; j < kOut; ++j) r.e[j] = r.tiny[j] ? ex_own[j] : r.e[j];
        }
        uint16_t rec[kOut];
  #pragma unroll
        for (int j = 0; j < kOut; ++j) rec[j] = __builtin_bit_cast(uint16_t, (_Float16)r.e[j]);
        uint16_t* rrow = a.records + (sel_tok0 + (int64_t)tl * a.Hkv) * a.logit_stride;
        if constexpr (kOut == 2) {
          // adjacent positions (pos[0] is even): one 4-byte store where both are visible
          // (live[1] implies live[0])
          if (r.live[1])
            *reinterpret_cast<uint32_t*>(rrow + r.pos[0]) = (uint32_t)rec[0] | ((uint32_t)rec[1] << 16);
          else if (r.live[0])
            rrow[r.pos[0]] = rec[0];
        } else {
          if (r.live[0]) rrow[r.pos[0]] = rec[0];
        }
  #pragma unroll
        for (int j = 0; j < kOut; ++j) {
          if (r.live[j] && r.pos[j] < w0j[0]) {
            const uint32_t bin = half_order_key(rec[j]) >> kFastShift;
            atomicAdd(&shist[tl * kHistWords + (bin >> 1)], (bin & 1) ? 65536u : 1u);
          }
        }
      };
      // one matrix-core instruction, then three vector instructions, once per MFMA of a
      // block's P V (16 fp16 or 32 bf16): the scheduler's order inside the current region
      auto interleave_pv = [&](auto kHt) {
        constexpr int kN = decltype(kHt)::value ? 16 : 32;
  #pragma unroll
        for (int i = 0; i < kN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
        }
      };

      // the two blocks, with P V in fp16 (kHt true) or in the two-part bf16 form
      auto blocks = [&](auto kHt) {
        // block 0: V^T operands read ahead (their LDS latency passes under the vector
        // work), probabilities, operands, records
        bf16x8_t avp0[kVPre];
    #pragma unroll
        for (int d = 0; d < kVPre; ++d) avp0[d] = read_vt(0, d);
        bf16x8_t ph0[2], pl0[2];
        RecState r0{}, r1{};
        {
          float p0[2][2][4];
          probabilities(0, p0);
          operands(kHt, 0, p0, ph0, pl0);
          if constexpr (want_rec) {
            float x0[8];
            rec_sums(p0, x0);
            rec_reduce(0, x0, r0);
          }
        }
        if constexpr (want_rec) rec_write(0, r0);
        // block 0's P V with block 1's probabilities, operands and record sums
        bf16x8_t avp1[kVPre];
    #pragma unroll
        for (int d = 0; d < kVPre; ++d) avp1[d] = read_vt(1, d);
        bf16x8_t ph1[2], pl1[2];
        float x1[8];
        {
          float p1[2][2][4];
          pv(kHt, 0, avp0, ph0, pl0);
          probabilities(1, p1);
          operands(kHt, 1, p1, ph1, pl1);
          if constexpr (want_rec) rec_sums(p1, x1);
          interleave_pv(kHt);
        }
        // block 1's P V with its record reduction
        pv(kHt, 1, avp1, ph1, pl1);
        if constexpr (want_rec) rec_reduce(1, x1, r1);
        interleave_pv(kHt);
        if constexpr (want_rec) rec_write(1, r1);
      };
      blocks(kHt);
      if constexpr (kBlockMode) {
        // log2 of the sum of 2^logit over this 64-position block, per (token, head)
  #pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float sum = across_groups<false>(bsum[qt]);
          const float lse = m[qt] + __builtin_amdgcn_logf(sum);   // -inf for an empty block
          if (grp == 0 && valid[qt])
            a.blse[((sel_tok0 + (int64_t)tokl[qt] * a.Hkv) * a.blse_stride + P0 / kCPos) * kGp + head[qt]] = lse;
        }
      }
      __syncthreads();   // every wave is done with this stage; the next one is stored
    }
    return true;
  };
  bool done = false;
  if constexpr (kV16) {
    if (f16v) {
      done = run_split(std::true_type{});
      if (!done) {
        __syncthreads();   // every wave has left the fp16 pass
        if constexpr (want_rec)
          for (int i = tid; i < kTPW * kHistWords; i += kCThreads) shist[i] = 0u;
      }
    }
  }
  if (!done) run_split(std::false_type{});

  // ---- partials per (token, head): O^T dims 16 d + 4 grp .. +3 of the lane's query row
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const float zz = across_groups<false>(z[qt]);
    if (valid[qt]) {
      float* pp = a.part + (((sel_tok0 + (int64_t)tokl[qt] * a.Hkv) * a.n_split + split) * a.G + head[qt]) *
                               kPartStride;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        *reinterpret_cast<float4*>(pp + 4 + 16 * d + 4 * grp) =
            make_float4(o[qt][d][0], o[qt][d][1], o[qt][d][2], o[qt][d][3]);
      if (grp == 0) {
        pp[0] = m[qt] == kMFloor ? kNegInf : m[qt];   // no visible position: -inf
        pp[1] = zz;
      }
    }
  }
  // ---- per-token key histograms of this split
  if constexpr (want_rec) {
    __syncthreads();
    for (int i = tid; i < ntok * kHistWords; i += kCThreads) {
      const int t = i / kHistWords;
      const int w = i - t * kHistWords;
      reinterpret_cast<uint32_t*>(a.hist_part + ((sel_tok0 + (int64_t)t * a.Hkv) * a.n_split + split) * kFastBins)[w] =
          shist[i];
    }
  }
}

template <int kGp>
dim3 chunk_grid(const ScanArgs& a, int B) {
  return dim3(a.n_split * ((a.Lq + tokens_per_wg<kGp>() - 1) / tokens_per_wg<kGp>()), a.Hkv, B);
}
template <bool kFp8>
hipError_t launch_chunk_t(const ScanArgs& a, int B, hipStream_t st, const KernelEvents* ev) {
  if (a.blse != nullptr) {   // block mode: per-block sums in kGp head slots
    if (a.G <= 8)
      launch_on(ev, chunk_mfma_kernel<8, true, kFp8>, chunk_grid<8>(a, B), dim3(kCThreads), 0, st, a);
    else if (a.G <= 16)
      launch_on(ev, chunk_mfma_kernel<16, true, kFp8>, chunk_grid<16>(a, B), dim3(kCThreads), 0, st, a);
    else if (a.G <= 32)
      launch_on(ev, chunk_mfma_kernel<32, true, kFp8>, chunk_grid<32>(a, B), dim3(kCThreads), 0, st, a);
    else
      return hipErrorInvalidValue;
  } else if (a.G <= 8) {
    launch_on(ev, chunk_mfma_kernel<8, false, kFp8>, chunk_grid<8>(a, B), dim3(kCThreads), 0, st, a);
  } else if (a.G <= 16) {
    launch_on(ev, chunk_mfma_kernel<16, false, kFp8>, chunk_grid<16>(a, B), dim3(kCThreads), 0, st, a);
  } else if (a.G <= 32) {
    launch_on(ev, chunk_mfma_kernel<32, false, kFp8>, chunk_grid<32>(a, B), dim3(kCThreads), 0, st, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

// Token and block mode for G <= 32.
hipError_t launch_chunk_mfma(const ScanArgs& a, int B, bool fp8, hipStream_t st, const KernelEvents* ev) {
  return fp8 ? launch_chunk_t<true>(a, B, st, ev) : launch_chunk_t<false>(a, B, st, ev);
}

}  // namespace hs2
