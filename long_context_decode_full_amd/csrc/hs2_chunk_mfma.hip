// Matrix-core scan for a chunk of query tokens (q_len > 1): the Full Attention layer
// of a Hybrid Block for every token of an appended chunk, causal inside the chunk,
// with the record-path outputs of the decode scan (online-softmax partials per
// (token, head, split), a 2-byte bound record per (token, position) and a key
// histogram per (token, split)).
//
// HySparse2 article, section 02 "KV Reuse" (the full layer's own attention scores
// decide what the sparse layers reuse) and section 03 (selection per token: every
// query token of the chunk gets its own window and top-k).
//
// A workgroup owns one position split of one (sequence, KV head) and 32 query tokens
// (16 tiles of 16 query rows = 2 tokens x 8 head slots; slots >= G are zero), so it
// reads every K/V row of its split once for 256 query rows.  Per iteration of 64
// positions the K and V tiles go through LDS (shared by the 8 waves); wave w owns
// query tiles 2w, 2w+1.  With lane = 16*grp + i:
//   S = Q K^T on v_mfma_f32_16x16x32_bf16: A = Q (lane: query row i, dims 32s + 8grp),
//     B = K^T (lane: position i, the same dims) read from the K tile; the
//     accumulator lane holds query rows 4grp+v (v = 0..3) at position i, so the 4
//     rows of a lane are 4 heads of one token.
//   softmax per query row: maxima over the 16 lanes of a row group (DPP), lazy
//     raise by 8 (log2 units) as in the decode scan.
//   record per (token, position): log2 of the sum over the token's heads of
//     2^logit, from the probabilities already formed for P.V: with U the largest
//     running maximum of the token's heads, e = U + log2 sum_h p_h 2^(m_h - U)
//     (4 heads in the lane, 4 in the partner row group via a permlane16 swap);
//     sums below 2^-100 (terms lost to underflow could matter there) take the
//     exact form on a wave-uniform branch.
//   O = P V: P (bf16 high part + bf16 residual) is staged per wave in LDS position-
//     major and read back as the A operand with ds_read_b64_tr_b16; B = V read from
//     the V tile with the same transposed read.
#include "hs2_rowops.h"

namespace hs2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2v_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kCThreads = 512;                 // 8 waves
constexpr int kCWaves = kCThreads / 64;
constexpr int kCTokens = 32;                   // query tokens per workgroup
constexpr int kCPos = 64;                      // positions per iteration
constexpr float kCSlack = 8.0f;
constexpr float kMFloor = -1.0e30f;            // initial running maximum (below any logit)
constexpr int kKRow = 272;                     // bytes per staged K/V row (256 + 16 pad)
constexpr int kKTile = kCPos * kKRow;
constexpr int kPRow = 72;                      // bytes per staged P row: 32 query rows bf16 + pad
constexpr int kPHalf = 32 * kPRow;             // 32 positions
constexpr int kPWave = 2 * kPHalf;             // high part + residual
constexpr int kHistWords = kFastBins / 2;      // two u16 counters per word
constexpr int kCLds = 2 * kKTile + kCWaves * kPWave + kCTokens * kHistWords * 4;

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2v_t x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}
__device__ __forceinline__ bf16x8_t tr_pair(const uint8_t* p0, const uint8_t* p1) {
  const s16x4_t x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p0);
  const s16x4_t x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p1);
  const uint2 w0 = __builtin_bit_cast(uint2, x0);
  const uint2 w1 = __builtin_bit_cast(uint2, x1);
  return as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
}
// Max / sum over the 16 lanes of a row group.
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppMirror8>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  return x;
}
// Partner row group (grp ^ 1): permlane16 swap.  Results are copied to scalars
// before any bit cast (a bit cast of a vector element reads element 0 here).
__device__ __forceinline__ float partner(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const uint32_t a0 = s[0], a1 = s[1];
  // lanes of even row groups receive the odd group's value in a1, odd ones in a0
  return __uint_as_float((__lane_id() & 16) ? a0 : a1);
}

// U per query tile and c per accumulator row, after the running maxima m changed.
__device__ __forceinline__ void update_record_scale(const float (&m)[2][4], int hbase, int G,
                                                    float (&U)[2], float (&c)[2][4]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    float u = kMFloor;
#pragma unroll
    for (int v = 0; v < 4; ++v) u = hbase + v < G ? fmaxf(u, m[qt][v]) : u;
    u = fmaxf(u, partner(u));
    U[qt] = u;
#pragma unroll
    for (int v = 0; v < 4; ++v) c[qt][v] = hbase + v < G ? fast_exp2(m[qt][v] - u) : 0.0f;
  }
}
// log2 of the sum over the token's valid heads of 2^l (this lane's 4 + the partner's 4),
// with the per-position maximum as reference.
__device__ __forceinline__ float exact_record(const float (&lv)[4], int hbase, int G) {
  float lm[4];
  float r = kNegInf;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    lm[v] = hbase + v < G ? lv[v] : kNegInf;
    r = fmaxf(r, lm[v]);
  }
  r = fmaxf(fmaxf(r, partner(r)), kMFloor);   // finite: exp2 of -inf is 0
  float sum = 0.0f;
#pragma unroll
  for (int v = 0; v < 4; ++v) sum += fast_exp2(lm[v] - r);
  sum += partner(sum);
  return r + __builtin_amdgcn_logf(sum);
}

template <bool kBlockMode>   // false: records + key histograms; true: per-block sums
__global__ __launch_bounds__(kCThreads, 1) void chunk_mfma_kernel(ScanArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kCLds];
  uint8_t* ktile = lds;
  uint8_t* vtile = lds + kKTile;
  uint8_t* pst_all = lds + 2 * kKTile;
  uint32_t* shist = reinterpret_cast<uint32_t*>(lds + 2 * kKTile + kCWaves * kPWave);

  // blockIdx.x = split * token groups + group: the groups of 32 tokens of one split are
  // adjacent.  (Placing the two groups of a 64-token chunk on one XCD, 8 workgroups
  // apart, was measured slower: the pair then contends for the same L2 lines at once.)
  const int n_tgroups = (a.Lq + kCTokens - 1) / kCTokens;
  const int tgroup = blockIdx.x % n_tgroups;
  const int split = blockIdx.x / n_tgroups;
  const int g = blockIdx.y;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int li = lane & 15;
  uint8_t* pst = pst_all + wave * kPWave;

  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  const int tok0 = tgroup * kCTokens;               // first token of this workgroup
  const int ntok = min(kCTokens, a.Lq - tok0);      // tokens present (may be <= 0)
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

  constexpr bool want_rec = !kBlockMode;   // token selection: records + histograms
  constexpr bool want_blk = kBlockMode;    // block comparator: per-block sums
  // histograms of this workgroup's tokens; split 0 also clears the merged ones
  for (int i = tid; i < kCTokens * kHistWords; i += kCThreads) shist[i] = 0u;
  if (want_rec && split == 0) {
    for (int i = tid; i < ntok * kFastBins; i += kCThreads) {
      const int t = i / kFastBins;
      a.hist_merged[(sel_tok0 + (int64_t)t * a.Hkv) * kSelWords + kSelHist1Off + (i - t * kFastBins)] = 0u;
    }
  }

  // Q fragments (A operand): query tile Qt = 2*wave + qt, row li -> token 2Qt + li/8,
  // head li%8; dims 32s + 8grp
  bf16x8_t qf[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int tl = 2 * (2 * wave + qt) + (li >> 3);   // token within the workgroup
    const int h = li & 7;
    const bool ok = tl < ntok && h < a.G;
    const uint16_t* qh = a.q + (((int64_t)b * a.Lq + tok0 + tl) * a.Hq + (int64_t)g * a.G + h) * kHeadDim + 8 * grp;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qf[qt][s] = as_bf16x8(ok ? *reinterpret_cast<const uint4*>(qh + 32 * s) : make_uint4(0u, 0u, 0u, 0u));
  }
  // per accumulator row (qt, v): token, head, visibility limits
  int tokl[2];        // token of the lane's rows in tile qt (within the workgroup)
  int32_t pj[2];      // last visible position of that token (positions < cap < 2^31)
  int32_t w0j[2];     // first window position (candidates are < w0j)
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    tokl[qt] = 2 * (2 * wave + qt) + (grp >> 1);
    const int64_t pp = ctx - a.Lq + tok0 + tokl[qt];
    pj[qt] = (int32_t)pp;
    int64_t w0 = pp + 1 - a.window;
    w0j[qt] = (int32_t)(w0 < 0 ? 0 : w0);
  }

  // record scale: U = the largest running maximum over the token's heads, c_v =
  // 2^(m_v - U) for this lane's 4 heads (0 for head slots >= G)
  const int hbase = 4 * (grp & 1);   // heads of this lane's accumulator rows: hbase .. hbase+3
  float U[2], c[2][4];

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const uint8_t* kb = a.k + head_row0 * 256;
  const uint8_t* vb = a.v + head_row0 * 256;

  f32x4_t o[2][8];
  float m[2][4], z[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
#pragma unroll
    for (int d = 0; d < 8; ++d) o[qt][d] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      m[qt][v] = kMFloor;   // finite, so exp2(l - m) needs no -inf test
      z[qt][v] = 0.0f;
    }
  }
  update_record_scale(m, hbase, a.G, U, c);
  __syncthreads();

  const int nit = p_end > p_begin ? (int)((p_end - p_begin + kCPos - 1) / kCPos) : 0;
  const int32_t last = (int32_t)(p_end - 1);
  // this thread's share of a tile load: rows (tid >> 4) + 32r, 16 bytes at (tid & 15)
  const int lrow = tid >> 4, lcol = (tid & 15) * 16;
  // (named registers, not arrays: small arrays live across the loop got placed in
  // LDS / scratch by the compiler)
  uint4 kr0, kr1, vr0, vr1;
  auto load_tiles = [&](int32_t base) {
    const uint32_t row0 = (uint32_t)min(base + lrow, last);
    const uint32_t row1 = (uint32_t)min(base + lrow + 32, last);
    kr0 = *reinterpret_cast<const uint4*>(kb + (uint64_t)row0 * 256 + lcol);
    kr1 = *reinterpret_cast<const uint4*>(kb + (uint64_t)row1 * 256 + lcol);
    vr0 = *reinterpret_cast<const uint4*>(vb + (uint64_t)row0 * 256 + lcol);
    vr1 = *reinterpret_cast<const uint4*>(vb + (uint64_t)row1 * 256 + lcol);
  };
  if (nit > 0) load_tiles((int32_t)p_begin);
  for (int it = 0; it < nit; ++it) {
    const int32_t P0 = (int32_t)p_begin + it * kCPos;
    __syncthreads();   // every wave is done with the previous tiles
    *reinterpret_cast<uint4*>(ktile + lrow * kKRow + lcol) = kr0;
    *reinterpret_cast<uint4*>(ktile + (lrow + 32) * kKRow + lcol) = kr1;
    *reinterpret_cast<uint4*>(vtile + lrow * kKRow + lcol) = vr0;
    *reinterpret_cast<uint4*>(vtile + (lrow + 32) * kKRow + lcol) = vr1;
    __syncthreads();
    // next tiles: in flight during this iteration's compute (the last iteration
    // re-reads clamped rows; no branch, so the loads are not sunk into one)
    load_tiles(P0 + kCPos);

    // ---- S = Q K^T for 2 query tiles x 4 position tiles
    f32x4_t sacc[2][4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      bf16x8_t kf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(ktile + (pt * 16 + li) * kKRow + 64 * s + 16 * grp));
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) d = mfma16(qf[qt][s], kf[s], d);
        sacc[qt][pt] = d;
      }
    }
    // raw scores q.k; the log2-domain logit is l = scale_log2 * s (scale_log2 > 0, so
    // maxima can be taken on s), formed inside the exp2 as fma(s, scale_log2, -m).  The
    // causal mask of each row's token only where some position lies beyond the first
    // token's (wave-uniform branch)
    const float sl2 = a.scale_log2;
    float l[2][4][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int v = 0; v < 4; ++v) l[qt][pt][v] = sacc[qt][pt][v];
    if ((int64_t)P0 + kCPos - 1 > ctx - a.Lq + tok0) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const bool vis = P0 + pt * 16 + li <= pj[qt];
#pragma unroll
          for (int v = 0; v < 4; ++v) l[qt][pt][v] = vis ? l[qt][pt][v] : kNegInf;
        }
    }

    // ---- online softmax per query row.  The running maximum m only needs raising
    // when some logit exceeds m + 8: a per-lane test and one ballot per step; the
    // exact row maximum (DPP over the row group) only on that rare path.
    {
      float x[2][4];
      bool up_any = false;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[qt][v] = fmaxf(fmaxf(l[qt][0][v], l[qt][1][v]), fmaxf(l[qt][2][v], l[qt][3][v])) * sl2;
          up_any |= x[qt][v] > m[qt][v] + kCSlack;
        }
      if (wave_any(up_any)) {
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float mx = max16(x[qt][v]);
            const bool up = mx > m[qt][v] + kCSlack;
            const float mn = up ? mx : m[qt][v];
            const float alpha = up ? fast_exp2(m[qt][v] - mn) : 1.0f;
#pragma unroll
            for (int d = 0; d < 8; ++d) o[qt][d][v] *= alpha;
            z[qt][v] *= alpha;
            m[qt][v] = mn;
          }
        update_record_scale(m, hbase, a.G, U, c);
      }
    }

    // ---- P V, one half of the positions at a time
    float bsum[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // this block's sums
    uint32_t tinybits = 0;   // bit 2qt + hf: this lane's record sum fell below 2^-100 (this half)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // P of position tiles 2hf, 2hf+1 -> LDS [position][query row], high part and residual
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float rs[2];   // this lane's 4 heads' share of the record sums of tiles 2hf, 2hf+1
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int pt = 2 * hf + pp;
          float p[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            p[v] = fast_exp2(__builtin_fmaf(l[qt][pt][v], sl2, -m[qt][v]));   // m finite: -inf gives 0
            z[qt][v] += p[v];
            if constexpr (want_blk) bsum[qt][v] += p[v];
          }
          if constexpr (want_rec) rs[pp] = p[0] * c[qt][0] + p[1] * c[qt][1] + p[2] * c[qt][2] + p[3] * c[qt][3];
          const uint32_t h01 = pack_bf16(p[0], p[1]);
          const uint32_t h23 = pack_bf16(p[2], p[3]);
          const uint32_t r01 = pack_bf16(p[0] - __uint_as_float(h01 << 16), p[1] - __uint_as_float(h01 & 0xFFFF0000u));
          const uint32_t r23 = pack_bf16(p[2] - __uint_as_float(h23 << 16), p[3] - __uint_as_float(h23 & 0xFFFF0000u));
          uint8_t* dst = pst + (pp * 16 + li) * kPRow + 2 * (qt * 16 + 4 * grp);
          *reinterpret_cast<uint2*>(dst) = make_uint2(h01, h23);
          *reinterpret_cast<uint2*>(dst + kPHalf) = make_uint2(r01, r23);
        }
        if constexpr (want_rec) {
          // Records e = U + log2 sum_h p_h 2^(m_h - U) over the token's 8 heads (4 in this
          // lane, 4 in the partner row group).  Even row groups finish tile 2hf, odd ones
          // tile 2hf+1: each lane sends its partner the share of the tile the partner
          // finishes, so one swap serves both tiles and every lane writes one record.  A
          // sum below 2^-100 (terms lost to underflow could matter there) is not counted
          // here and is redone exactly below.
          const int own = grp & 1;
          const float sum = (own ? rs[1] : rs[0]) + partner(own ? rs[0] : rs[1]);
          const int32_t pos = P0 + (2 * hf + own) * 16 + li;
          const int tl = tokl[qt];
          const bool live = pos <= pj[qt] && tl < ntok;
          const bool tiny = live && sum < 0x1p-100f;
          tinybits |= tiny ? (1u << (2 * qt + hf)) : 0u;
          const float e = U[qt] + __builtin_amdgcn_logf(sum);
          if (live) {
            const uint16_t rec = __builtin_bit_cast(uint16_t, (_Float16)e);
            a.records[(sel_tok0 + (int64_t)tl * a.Hkv) * a.logit_stride + pos] = rec;
            if (!tiny && pos < w0j[qt]) {
              const uint32_t bin = half_order_key(rec) >> kFastShift;
              atomicAdd(&shist[tl * kHistWords + (bin >> 1)], (bin & 1) ? 65536u : 1u);
            }
          }
        }
      }
      if constexpr (want_rec) {
        // exact records of this half where the sum underflowed (rare: logits 100 log2
        // units below the running maxima); every lane takes part in exact_record's swaps
        if (wave_any(tinybits != 0u)) {
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const uint32_t bit = 1u << (2 * qt + hf);
            if (!wave_any((tinybits & bit) != 0u)) continue;
            float l0[4], l1[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              l0[v] = l[qt][2 * hf][v] * sl2;
              l1[v] = l[qt][2 * hf + 1][v] * sl2;
            }
            const float ex0 = exact_record(l0, hbase, a.G);
            const float ex1 = exact_record(l1, hbase, a.G);
            const int own = grp & 1;
            if (tinybits & bit) {   // implies a visible position of a present token
              const int32_t pos = P0 + (2 * hf + own) * 16 + li;
              const int tl = tokl[qt];
              const uint16_t rec = __builtin_bit_cast(uint16_t, (_Float16)(own ? ex1 : ex0));
              a.records[(sel_tok0 + (int64_t)tl * a.Hkv) * a.logit_stride + pos] = rec;
              if (pos < w0j[qt]) {
                const uint32_t bin = half_order_key(rec) >> kFastShift;
                atomicAdd(&shist[tl * kHistWords + (bin >> 1)], (bin & 1) ? 65536u : 1u);
              }
            }
          }
          tinybits = 0u;
        }
      }
      // A operands: P[query row li][positions 8grp .. 8grp+7] of this half
      bf16x8_t ph[2], pl[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const uint8_t* p0 = pst + (8 * grp + (li >> 2)) * kPRow + 2 * (qt * 16 + 4 * (li & 3));
        const uint8_t* p1 = p0 + 4 * kPRow;
        ph[qt] = tr_pair(p0, p1);
        pl[qt] = tr_pair(p0 + kPHalf, p1 + kPHalf);
      }
      // B operands: V[positions 32hf + 8grp .. +7][dims 16d + li]
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint8_t* v0 = vtile + (32 * hf + 8 * grp + (li >> 2)) * kKRow + 2 * (16 * d + 4 * (li & 3));
        const bf16x8_t vf = tr_pair(v0, v0 + 4 * kKRow);
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          o[qt][d] = mfma16(ph[qt], vf, o[qt][d]);
          o[qt][d] = mfma16(pl[qt], vf, o[qt][d]);
        }
      }
    }
    if constexpr (want_blk) {
      // log2 of the sum of 2^logit over this 64-position block, per (token, head)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float lse[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float x = bsum[qt][v];
          x += dpp<kDppXor1>(x);
          x += dpp<kDppXor2>(x);
          x += dpp<kDppMirror8>(x);
          x += dpp<kDppRor8>(x);
          lse[v] = m[qt][v] + __builtin_amdgcn_logf(x);   // -inf for an empty block
        }
        const int tl = tokl[qt];
        if (li == 0 && tl < ntok) {
          float* dst = a.blse + ((sel_tok0 + (int64_t)tl * a.Hkv) * a.blse_stride + P0 / kCPos) * 8 + 4 * (grp & 1);
          *reinterpret_cast<float4*>(dst) = make_float4(lse[0], lse[1], lse[2], lse[3]);
        }
      }
    }
  }

  // ---- partials per (token, head): rows 4grp+v of tile qt
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int tl = tokl[qt];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float zz = z[qt][v];
      zz += dpp<kDppXor1>(zz);
      zz += dpp<kDppXor2>(zz);
      zz += dpp<kDppMirror8>(zz);
      zz += dpp<kDppRor8>(zz);
      const int h = 4 * (grp & 1) + v;
      if (tl < ntok && h < a.G) {
        float* pp = a.part + (((sel_tok0 + (int64_t)tl * a.Hkv) * a.n_split + split) * a.G + h) * kPartStride;
#pragma unroll
        for (int d = 0; d < 8; ++d) pp[4 + 16 * d + li] = o[qt][d][v];
        if (li == 0) {
          pp[0] = m[qt][v] == kMFloor ? kNegInf : m[qt][v];   // no visible position: -inf
          pp[1] = zz;
        }
      }
    }
  }
  // ---- per-token key histograms of this split
  if (!want_rec) return;
  __syncthreads();
  for (int i = tid; i < ntok * kHistWords; i += kCThreads) {
    const int t = i / kHistWords;
    const int w = i - t * kHistWords;
    reinterpret_cast<uint32_t*>(a.hist_part + ((sel_tok0 + (int64_t)t * a.Hkv) * a.n_split + split) * kFastBins)[w] =
        shist[i];
  }
}

}  // namespace

hipError_t launch_chunk_mfma(const ScanArgs& a, int B, hipStream_t st) {
  dim3 grid(a.n_split * ((a.Lq + kCTokens - 1) / kCTokens), a.Hkv, B);
  if (a.blse != nullptr)
    hipLaunchKernelGGL((chunk_mfma_kernel<true>), grid, dim3(kCThreads), 0, st, a);
  else
    hipLaunchKernelGGL((chunk_mfma_kernel<false>), grid, dim3(kCThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs2
