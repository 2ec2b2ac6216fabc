// Token selection from bound records (the default path of hs2_full_attn_select).
//
// HySparse2 article, section 03: keep the 128 most recent tokens plus the 1,024
// tokens outside that window with the highest score; section 02: the score comes
// from the full layer's own attention.  Score of position t for KV group g:
//   s(t) = sum over the group's heads h of exp2(l_h(t) - M_h) / Z_h.
//
// The scan leaves, per position, e(t) = log2 sum_h 2^l_h(t) rounded to binary16,
// and a histogram of those values over the positions outside the window.  With
// w_h = 2^-M_h / Z_h (global statistics from the combine step),
//   2^(e - u) * min_h w_h  <=  s(t)  <=  2^(e + u) * max_h w_h
// where u is the binary16 spacing at e.  The lower edge e* of the histogram bin
// holding the k-th largest e gives at least k positions with s >= 2^(e* - u*) min w,
// so the k-th largest s is at least that; a position can be selected only if its
// upper bound reaches it.
//   candidate_kernel: finds e* from the merged histogram, keeps the positions whose
//                     upper bound reaches the threshold (in position order per
//                     chunk) and re-scores them exactly by re-reading their keys
//                     with the scan's own arithmetic (row_logit), so s is
//                     bit-identical to the value the scan's logits would give.
//                     From 256 rows on (chunks of query tokens) the stage runs as two
//                     kernels instead, cand_filter_kernel and cand_rescore_kernel, that
//                     take the exact k-th largest record in place of its bin's edges.
//   final_kernel:     exact top-k of the candidates by (s desc, position asc): a
//                     radix digit on the fp32 bit pattern of s (s >= 0 orders like
//                     its bits) finds the bin of the k-th score, the entries of that
//                     bin are ranked pairwise by a unique (s, position) key, and one
//                     block-wide scan emits the chosen positions ascending, followed
//                     by the window.  Oversized candidate sets or bins fall back to
//                     two more digits with ties taken in position order.
#include "hs2_rowops.h"

#include <type_traits>

namespace hs2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kThreads = 256;
constexpr float kBoundSlack = 2e-3f;   // log2 units: fp32 rounding of e and of the exact s

struct RowGeom {
  int64_t n;    // visible positions
  int64_t w0;   // candidates are [0, w0); window is [w0, n)
};

__device__ __forceinline__ RowGeom row_geom(const FastSelArgs& a, int64_t sel) {
  const int64_t bj = sel / a.Hkv;
  const int64_t b = bj / a.Lq;
  const int64_t j = bj - b * a.Lq;
  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  int64_t n = ctx - a.Lq + j + 1;
  n = n < 0 ? 0 : n;
  int64_t w0 = n - a.window;
  w0 = w0 < 0 ? 0 : w0;
  return {n, w0};
}

__device__ __forceinline__ uint32_t* sel_block(const FastSelArgs& a, int64_t sel) {
  return a.selblk + sel * kSelWords;
}

__device__ __forceinline__ void load_mz(const FastSelArgs& a, int64_t sel, float (&Mh)[8], float (&iz)[8]) {
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    Mh[h] = a.mz[(sel * kMaxHeads + h) * 2 + 0];
    iz[h] = a.mz[(sel * kMaxHeads + h) * 2 + 1];
  }
}

// Largest bin B of the histogram h[0, nb) with (entries in bins >= B) >= need, and
// the count strictly above B; if fewer than `need` entries exist, B = 0 and `above`
// is the total.  Block-wide over NT threads, thread t holding bins [t*PER, t*PER+PER):
// a DPP prefix sum per wave plus one cross-wave step through LDS.
template <int NT, int PER>
__device__ void block_threshold(const uint32_t* h, int nb, uint32_t need, uint32_t& bin,
                                uint32_t& above) {
  __shared__ uint32_t wtot[NT / 64];
  __shared__ uint32_t res[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t loc[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int bi = tid * PER + i;
    loc[i] = bi < nb ? h[bi] : 0u;
    tot += loc[i];
  }
  const uint32_t p = wave_prefix_incl(tot);
  const uint32_t wt = (uint32_t)__builtin_amdgcn_readlane((int)p, 63);
  if (lane == 0) wtot[wave] = wt;
  if (tid == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  __syncthreads();
  uint32_t higher = wt - p;   // bins held by the later lanes of this wave
  uint32_t all = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint32_t v = wtot[w];
    all += v;
    higher += w > wave ? v : 0u;
  }
  if (tid == 0 && all < need) res[1] = all;
  if (higher < need && higher + tot >= need) {
    uint32_t cum = higher;
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (cum + loc[i] >= need) {
        res[0] = (uint32_t)(tid * PER + i);
        res[1] = cum;
        break;
      }
      cum += loc[i];
    }
  }
  __syncthreads();
  bin = res[0];
  above = res[1];
  __syncthreads();   // res and wtot are reused by the next call
}

// Unique 64-bit order key of a candidate: larger score first, then lower position.
__device__ __forceinline__ uint64_t cand_key(uint32_t sbits, int32_t pos) {
  return ((uint64_t)sbits << 32) | (uint32_t)(0x7FFFFFFF - pos);
}
__device__ __forceinline__ int32_t key_pos(uint64_t key) {
  return 0x7FFFFFFF - (int32_t)(uint32_t)key;
}

// Records t0 .. t0 + R - 1 of a row as R/2 packed words; slots at or past `limit` (the
// row's record slots, or the candidate range) read as zero.  Records past w0 are stale
// (a row's scan writes only its visible positions); the tests mask them off.
template <int R>
__device__ __forceinline__ void load_records(uint32_t (&words)[R / 2], const uint16_t* __restrict__ rrow,
                                             int64_t t0, int64_t w0) {
  if (t0 + R <= w0) {
#pragma unroll
    for (int v = 0; v < R / 8; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(rrow + t0 + 8 * v);
      words[4 * v + 0] = x.x; words[4 * v + 1] = x.y; words[4 * v + 2] = x.z; words[4 * v + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < R / 2; ++i) {
      const int64_t t = t0 + 2 * i;
      const uint32_t lo = t < w0 ? (uint32_t)rrow[t] : 0u;
      const uint32_t hi = t + 1 < w0 ? (uint32_t)rrow[t + 1] : 0u;
      words[i] = lo | (hi << 16);
    }
  }
}

// Records that pass a test which does not decrease with the record's value (e + u(e)
// >= thr, e - u(e) > thr: both hold from some order key on): the first passing key by a
// binary search on the test itself, then, as binary16 codes, one interval of
// non-negative codes [plo, +inf] and, when that key falls below +0, one interval of
// negative codes [0x8000, 0xFFFF - kmin].  NaN codes (above +inf) never pass.
struct CodeRange {
  uint32_t plo, pspan, nspan;
  bool none, neg;
};
template <class Pass>
__device__ __forceinline__ CodeRange code_range(Pass pass) {
  uint32_t lo = 0u, hi = 0x10000u;   // the first passing key lies in [lo, hi] (0x10000: none)
  while (lo < hi) {
    const uint32_t mid = (lo + hi) >> 1;
    if (pass(half_bits_of_key(mid))) hi = mid; else lo = mid + 1;
  }
  constexpr uint32_t kPInf = 0x7C00u;
  CodeRange c;
  c.plo = lo >= 0x8000u ? lo - 0x8000u : 0u;
  c.none = lo > 0xFC00u;   // not even +inf passes
  c.pspan = c.plo <= kPInf ? kPInf - c.plo : 0u;
  c.neg = lo < 0x8000u;
  c.nspan = c.neg ? 0x7FFFu - lo : 0u;
  return c;
}
// Bit i set where record i of the R (packed two per word) lies in the range.
template <int R, typename mask_t>
__device__ __forceinline__ mask_t range_mask(const uint32_t (&words)[R / 2], const CodeRange& c) {
  mask_t m = 0;
  if (!c.none) {   // workgroup-uniform
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const uint32_t rb = (words[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      m |= rb - c.plo <= c.pspan ? ((mask_t)1 << i) : (mask_t)0;
    }
    if (c.neg) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const uint32_t rb = (words[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
        m |= rb - 0x8000u <= c.nspan ? ((mask_t)1 << i) : (mask_t)0;
      }
    }
  }
  return m;
}
// The first `nv` of R bits (positions before w0).
template <int R, typename mask_t>
__device__ __forceinline__ mask_t valid_mask(int64_t nv) {
  if (nv >= R) return ~(mask_t)0 >> (8 * sizeof(mask_t) - R);
  return nv <= 0 ? (mask_t)0 : (mask_t)((((mask_t)1) << nv) - 1);
}

// Exact re-score with more than 8 query heads per KV head (up to 32), on the matrix
// cores: tiles of 16 list entries, S = K Q^T with A = the entries' key rows (lane:
// entry w16 of the tile, dims 32 s + 8 grp) and B = Q^T of each 16-head block, so lane
// (head w16, grp) gets the logits of entries 4 grp + v; the group sum adds the two
// blocks, then the 16 head lanes (DPP).  Wave w of 4 takes tiles w, w + 4, ...; the key
// loads of kRsTiles tiles are issued together.  pos_of(i): entry i's position;
// write(i, s): store its score.
constexpr int kRsTiles = 4;
struct WideQuery {
  bf16x8_t qf[2][4];   // Q^T of heads 16 hb + w16 (zero past G), dims 32 s + 8 grp
  float M[2], iz[2];   // their (M, 1/Z)
};
__device__ __forceinline__ void load_wide_query(const FastSelArgs& a, int64_t sel, int64_t bj, int g, int r,
                                                int rgrp, WideQuery& wq) {
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const int h = 16 * hb + r;
    const bool in = h < a.G;
    const uint16_t* qh = a.q + (bj * a.Hq + (int64_t)g * a.G + (in ? h : 0)) * kHeadDim;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const uint4 x = *reinterpret_cast<const uint4*>(qh + 32 * sl + 8 * rgrp);
      wq.qf[hb][sl] = __builtin_bit_cast(bf16x8_t, in ? x : make_uint4(0u, 0u, 0u, 0u));
    }
    wq.M[hb] = in ? a.mz[(sel * kMaxHeads + h) * 2] : 0.0f;
    wq.iz[hb] = in ? a.mz[(sel * kMaxHeads + h) * 2 + 1] : 0.0f;
  }
}
template <bool kFp8, class PosOf, class Write>
__device__ __forceinline__ void rescore_wide(int nu, int wave, int r, int rgrp, const WideQuery& wq,
                                             const uint8_t* __restrict__ kb, const float* __restrict__ ksb,
                                             float scale_log2, int G, PosOf pos_of, Write write) {
  const int ntiles = (nu + 15) >> 4;
  for (int t0 = wave; t0 < ntiles; t0 += 4 * kRsTiles) {
    bf16x8_t kf[kRsTiles][4];
    float ks4[kRsTiles][4];
#pragma unroll
    for (int u = 0; u < kRsTiles; ++u) {
      const int t = min(t0 + 4 * u, ntiles - 1);   // past the end: a valid tile, dropped
      const int i = 16 * t + r;
      const uint32_t pos = pos_of(i < nu ? i : 16 * t);
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if constexpr (kFp8) {
          const uint2 c = *reinterpret_cast<const uint2*>(kb + (uint64_t)pos * 128 + 32 * sl + 8 * rgrp);
          kf[u][sl] = __builtin_bit_cast(bf16x8_t, make_uint4(fp8x2_to_bf16x2(c.x, false), fp8x2_to_bf16x2(c.x, true),
                                                              fp8x2_to_bf16x2(c.y, false), fp8x2_to_bf16x2(c.y, true)));
        } else {
          kf[u][sl] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(kb + (uint64_t)pos * 256 + 64 * sl + 16 * rgrp));
        }
      }
      if constexpr (kFp8) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int iv = 16 * t + 4 * rgrp + v;
          ks4[u][v] = ksb[pos_of(iv < nu ? iv : 16 * t)];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRsTiles; ++u) {
      const int t = t0 + 4 * u;
      if (t < ntiles) {   // wave-uniform
        float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          f32x4_t d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int sl = 0; sl < 4; ++sl) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[u][sl], wq.qf[hb][sl], d, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float l = d[v] * scale_log2;
            if constexpr (kFp8) l *= ks4[u][v];
            x[v] += 16 * hb + r < G ? fast_exp2(l - wq.M[hb]) * wq.iz[hb] : 0.0f;
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          x[v] += dpp<kDppXor1>(x[v]);
          x[v] += dpp<kDppXor2>(x[v]);
          x[v] += dpp<kDppMirror8>(x[v]);
          x[v] += dpp<kDppRor8>(x[v]);
        }
        const int iv = 16 * t + 4 * rgrp + r;   // lanes r < 4 write entry 4 grp + r
        if (r < 4 && iv < nu) write(iv, r == 0 ? x[0] : r == 1 ? x[1] : r == 2 ? x[2] : x[3]);
      }
    }
  }
}

// ------------------------------------------------------------------ candidates + exact re-score
// Work unit: one (row, chunk of chunk_len positions); workgroup w of a row takes its
// chunks w, w + cand_wgs, ... (blockIdx.x = row * cand_wgs + w; the grid is sized so
// that rows of a long context do not leave most workgroups of short rows empty).
// The threshold bin of the k-th record gives two tests per position (records are
// bounds, see above):
//   candidate: its upper bound reaches the lower bound of the k-th score;
//   certain:   its lower bound exceeds the upper bound of the k-th score (built from
//              the bin's upper edge), so it is selected whatever the exact scores are.
// Certain positions get an infinite score key without re-scoring; only the uncertain
// candidates re-read their key rows.  Keys stay in position order per chunk.
// kMB: more than 8 query heads per KV head; the exact scores are summed over blocks of
// 8 heads (one query load per block), per candidate in LDS.
template <bool kFp8, int R, bool kMB>   // R = records per thread = chunk_len / 256 (8..64)
__global__ __launch_bounds__(kThreads) void candidate_kernel(FastSelArgs a) {
  const int64_t sel = blockIdx.x / (uint32_t)a.cand_wgs;
  const int wg = (int)(blockIdx.x % (uint32_t)a.cand_wgs);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int clen = R * kThreads;
  const uint16_t* rrow = a.records + sel * a.rec_stride;
  // The first chunk's records do not wait for the row's length: the loads cover the
  // row's record slots and the tests below mask the positions at or past w0.
  uint32_t words[R / 2];
  load_records<R>(words, rrow, (int64_t)wg * clen + (int64_t)tid * R, a.rec_stride);
  const RowGeom rg = row_geom(a, sel);
  if (rg.w0 <= a.topk || a.topk == 0) return;
  // chunks at or past the first window position hold no candidate
  if ((int64_t)wg * clen >= rg.w0) return;

  __shared__ uint16_t cpos[clen];    // chunk-relative positions of the candidates
  __shared__ uint16_t ulist[clen];   // indices into cpos of the uncertain ones
  __shared__ uint32_t total_s;
  __shared__ uint32_t wscan[kThreads / 64];
  float Mh[8], iz[8];
  load_mz(a, sel, Mh, iz);
  const int64_t bj = sel / a.Hkv;
  const int g = (int)(sel - bj * a.Hkv);
  const int b = (int)(bj / a.Lq);
  const int r = lane & 15;
  const int rgrp = lane >> 4;
  const int hown = head_of(r);
  // the queries are loaded early: their latency overlaps the threshold and the filter
  uint32_t qp[8][4];   // up to 8 heads: the scan's row layout (VALU re-score)
  WideQuery wq;        // more heads: the matrix-core re-score's fragments
  if constexpr (!kMB)
    load_query(a.q + (bj * a.Hq + (int64_t)g * a.G) * kHeadDim, a.G, r, qp);
  else
    load_wide_query(a, sel, bj, g, r, rgrp, wq);
  // With R <= 32 the next chunk's records are loaded while the current chunk re-scores
  // (a row's workgroup takes its chunks in turn when rows are many).
  constexpr bool kPrefetch = R <= 32;

  // threshold: bin of the k-th largest record key in the merged histogram
  uint32_t tb, above;
  block_threshold<kThreads, kFastBins / kThreads>(sel_block(a, sel) + kSelHist1Off, kFastBins,
                                                  (uint32_t)a.topk, tb, above);
  const uint32_t ebits = half_bits_of_key(tb << kFastShift);                  // smallest record in the bin
  const uint32_t ebits_hi = half_bits_of_key(((tb + 1) << kFastShift) - 1);   // largest
  float lwmin = __builtin_huge_valf(), lwmax = -__builtin_huge_valf();
  if constexpr (kMB) {
    for (int h = 0; h < a.G; ++h) {
      const float lw = __builtin_amdgcn_logf(a.mz[(sel * kMaxHeads + h) * 2 + 1]) - a.mz[(sel * kMaxHeads + h) * 2];
      lwmin = fminf(lwmin, lw);
      lwmax = fmaxf(lwmax, lw);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h < a.G) {
        const float lw = __builtin_amdgcn_logf(iz[h]) - Mh[h];   // log2 w_h
        lwmin = fminf(lwmin, lw);
        lwmax = fmaxf(lwmax, lw);
      }
    }
  }
  // candidate  <=>  e + u(e) + log2 max w  >=  e* - u(e*) + log2 min w  (with slack)
  const float thr = half_bits_to_float(ebits) - half_ulp(ebits) - (lwmax - lwmin) - 2.0f * kBoundSlack;
  // certain    <=>  e - u(e) + log2 min w  >   e_hi + u(e_hi) + log2 max w  (with slack)
  const float thr_in = half_bits_to_float(ebits_hi) + half_ulp(ebits_hi) + (lwmax - lwmin) + 2.0f * kBoundSlack;
  // The certain test pays off where candidates are dense: rows whose candidate range
  // is short next to top-k (row-uniform); long rows have a few per workgroup.
  const bool use_cert = rg.w0 < (int64_t)a.topk * 64;
  const CodeRange cand_r = code_range([&](uint32_t h) { return half_bits_to_float(h) + half_ulp(h) >= thr; });
  const CodeRange cert_r = code_range([&](uint32_t h) { return half_bits_to_float(h) - half_ulp(h) > thr_in; });

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const uint8_t* kb = a.k + head_row0 * (kFp8 ? 128 : 256);
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float Mown = Mh[hown];
  const float izown = iz[hown];

  for (int chunk = wg; (int64_t)chunk * clen < rg.w0; chunk += a.cand_wgs) {
    const int64_t c0 = (int64_t)chunk * clen;
    // Each thread owns R consecutive positions (one batch of 16-byte loads); a
    // block-wide exclusive scan of the per-thread counts keeps position order.
    const int64_t t0 = c0 + (int64_t)tid * R;
    if (!kPrefetch && chunk != wg) load_records<R>(words, rrow, t0, a.rec_stride);
    // positions at or past w0 (their records read as zero) are not candidates
    const uint64_t hitmask = range_mask<R, uint64_t>(words, cand_r) & valid_mask<R, uint64_t>(rg.w0 - t0);
    const uint64_t certmask = use_cert ? hitmask & range_mask<R, uint64_t>(words, cert_r) : 0ull;
    const uint64_t uncmask = hitmask & ~certmask;
    if constexpr (kPrefetch) {   // this chunk's records are consumed: load the next chunk's
      const int64_t cn = c0 + (int64_t)a.cand_wgs * clen;
      if (cn < rg.w0) load_records<R>(words, rrow, cn + (int64_t)tid * R, a.rec_stride);
    }
    // block exclusive scan of (hits, uncertain hits), packed in one word (each < 2^16)
    const uint32_t mine = (uint32_t)__builtin_popcountll(hitmask) | ((uint32_t)__builtin_popcountll(uncmask) << 16);
    const uint32_t x = wave_prefix_incl(mine);
    __syncthreads();   // the previous chunk is done with wscan, cpos and ulist
    if (lane == 63) wscan[wave] = x;
    __syncthreads();
    uint32_t before = x - mine;
    for (int w = 0; w < wave; ++w) before += wscan[w];
    if (tid == kThreads - 1) total_s = before + mine;
    const int64_t slot0 = (sel * a.n_chunks + chunk) * (int64_t)clen;
    uint32_t ih = before & 0xFFFFu, iu = before >> 16;
    uint64_t hm = (uint64_t)hitmask;
    while (hm) {
      const int i = __builtin_ctzll(hm);
      hm &= hm - 1;
      cpos[ih] = (uint16_t)(t0 + i - c0);
      if ((uncmask >> i) & 1ull)
        ulist[iu++] = (uint16_t)ih;
      else
        a.cand_keys[slot0 + ih] = cand_key(0x7F800000u, (int32_t)(t0 + i));   // certainly selected
      ++ih;
    }
    __syncthreads();
    const int cnt = (int)(total_s & 0xFFFFu);   // candidates
    const int unc = (int)(total_s >> 16);       // of which uncertain
    if (tid == 0) a.cand_count[sel * a.n_chunks + chunk] = cnt;

    // exact re-score: 4 rows per wave step, the scan's lane layout and arithmetic.
    // Batches of kRescoreBatch wave steps: all their key loads are issued before the
    // first row is scored, so a long candidate list does not wait on one load per step.
    constexpr int kRescoreBatch = 4;
    if constexpr (!kMB) {
      for (int i0 = wave * 4; i0 < unc; i0 += 16 * kRescoreBatch) {
        RowData d[kRescoreBatch];
        int32_t tpos[kRescoreBatch];
        int tidx[kRescoreBatch];
#pragma unroll
        for (int u = 0; u < kRescoreBatch; ++u) {
          const int i = i0 + 16 * u + rgrp;
          // past the end: re-read the batch's first row (valid), the result is dropped
          tidx[u] = ulist[i < unc ? i : i0];
          tpos[u] = (int32_t)(c0 + cpos[tidx[u]]);
          load_key<kFp8>(kb, ksb, (uint32_t)tpos[u], r, d[u]);
        }
#pragma unroll
        for (int u = 0; u < kRescoreBatch; ++u) {
          const int i = i0 + 16 * u + rgrp;
          const float l = row_logit<kFp8>(qp, d[u], a.scale_log2);
          const float part = ((r & 1) == 0 && hown < a.G) ? fast_exp2(l - Mown) * izown : 0.0f;
          const float s = rowgroup_sum16(part);
          if (i < unc && r == 0) a.cand_keys[slot0 + tidx[u]] = cand_key(__float_as_uint(s), tpos[u]);
        }
      }
    } else {
      rescore_wide<kFp8>(unc, wave, r, rgrp, wq, kb, ksb, a.scale_log2, a.G,
                         [&](int i) { return (uint32_t)(c0 + cpos[ulist[i]]); },
                         [&](int i, float sv) {
                           const int ti = ulist[i];
                           a.cand_keys[slot0 + ti] = cand_key(__float_as_uint(sv), (int32_t)(c0 + cpos[ti]));
                         });
    }
  }
}

// ------------------------------------------------------------------ two-step candidates
// The same tests with the exact k-th largest record E_k in place of its histogram bin's
// edges: the k-th largest score lies between 2^(E_k - u) min w and 2^(E_k + u) max w
// (u = u(E_k)), so
//   candidate:  e + u(e) + log2 max w  >=  E_k - u + log2 min w
//   certain:    e - u(e) + log2 min w  >   E_k + u + log2 max w.
// E_k is known only once every record of the row has been seen, hence two kernels
// over the same (row, chunk) work units:
//   cand_filter_kernel:  keeps the positions that reach the bin-edge test (a superset,
//                        since x - u(x) does not decrease with x), writes them with their
//                        records, and counts the records inside the threshold bin by
//                        their low key bits (kFastSubBins counters per row);
//   cand_rescore_kernel: finds E_k from those counts, applies the two tests to the list
//                        and re-scores the uncertain candidates.
// The filter's list sits in the upper half of each chunk's key slots (32-bit entries:
// record bits << 16 | chunk-relative position); keys are written from the bottom, and
// a block of kRsBlk entries is read in full before its keys are written, so a key never
// lands on an entry that is still to be read (key j < base + kRsBlk ends at byte
// 8 (base + kRsBlk) <= 4 clen + 4 (base + kRsBlk), the start of the next block).
constexpr int kRsBlk = 1024;   // list entries per re-score block
constexpr int kRsPer = kRsBlk / kThreads;
constexpr int kRsBatch = 8;    // wave steps (4 rows each) whose key loads are issued together
static_assert(kFastSubBins == 64, "one lane per sub-bin");
static_assert(kMinCandChunkLen % kRsBlk == 0, "blocks tile a chunk");

__device__ __forceinline__ void log_weight_range(const FastSelArgs& a, int64_t sel, float& lwmin, float& lwmax) {
  lwmin = __builtin_huge_valf();
  lwmax = -__builtin_huge_valf();
  for (int h = 0; h < a.G; ++h) {
    const float lw = __builtin_amdgcn_logf(a.mz[(sel * kMaxHeads + h) * 2 + 1]) - a.mz[(sel * kMaxHeads + h) * 2];
    lwmin = fminf(lwmin, lw);
    lwmax = fmaxf(lwmax, lw);
  }
}

template <int R>   // records per thread: chunk_len / 256
__global__ __launch_bounds__(kThreads) void cand_filter_kernel(FastSelArgs a) {
  const int64_t sel = blockIdx.x / (uint32_t)a.cand_wgs;
  const int wg = (int)(blockIdx.x % (uint32_t)a.cand_wgs);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int clen = R * kThreads;
  const uint16_t* rrow = a.records + sel * a.rec_stride;
  uint32_t words[R / 2];   // issued before the row's length is known (see candidate_kernel)
  load_records<R>(words, rrow, (int64_t)wg * clen + (int64_t)tid * R, a.rec_stride);
  const RowGeom rg = row_geom(a, sel);
  if (rg.w0 <= a.topk || a.topk == 0) return;
  if ((int64_t)wg * clen >= rg.w0) return;

  __shared__ uint32_t sub[kFastSubBins];
  __shared__ uint32_t wscan[kThreads / 64];
  __shared__ uint32_t srec[kThreads][R / 2 + 1];   // this thread's records, for its hits
  if (tid < kFastSubBins) sub[tid] = 0u;
  uint32_t* blk = sel_block(a, sel);
  uint32_t tb, above;
  block_threshold<kThreads, kFastBins / kThreads>(blk + kSelHist1Off, kFastBins, (uint32_t)a.topk, tb, above);
  if (wg == 0 && tid == 0) {
    blk[kStFastBin] = tb;
    blk[kStFastAbove] = above;
  }
  float lwmin, lwmax;
  log_weight_range(a, sel, lwmin, lwmax);
  const uint32_t ebits = half_bits_of_key(tb << kFastShift);   // smallest record in the bin
  const float thr = half_bits_to_float(ebits) - half_ulp(ebits) - (lwmax - lwmin) - 2.0f * kBoundSlack;
  const CodeRange cr = code_range([&](uint32_t h) { return half_bits_to_float(h) + half_ulp(h) >= thr; });
  typedef typename std::conditional<(R > 32), uint64_t, uint32_t>::type mask_t;

  for (int chunk = wg; (int64_t)chunk * clen < rg.w0; chunk += a.cand_wgs) {
    const int64_t c0 = (int64_t)chunk * clen;
    const int64_t t0 = c0 + (int64_t)tid * R;
    // positions at or past w0 (their records read as zero) are not candidates
    const mask_t hitmask = range_mask<R, mask_t>(words, cr) & valid_mask<R, mask_t>(rg.w0 - t0);
    if (hitmask != 0) {
#pragma unroll
      for (int i = 0; i < R / 2; ++i) srec[tid][i] = words[i];
    }
    const int64_t cn = c0 + (int64_t)a.cand_wgs * clen;   // this workgroup's next chunk
    if (cn < rg.w0) load_records<R>(words, rrow, cn + (int64_t)tid * R, a.rec_stride);
    const uint32_t mine = (uint32_t)__builtin_popcountll((uint64_t)hitmask);
    const uint32_t x = wave_prefix_incl(mine);
    __syncthreads();   // the previous chunk is done with wscan
    if (lane == 63) wscan[wave] = x;
    __syncthreads();
    uint32_t ih = x - mine, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      total += wscan[w];
      ih += w < wave ? wscan[w] : 0u;
    }
    uint32_t* ent = reinterpret_cast<uint32_t*>(a.cand_keys + (sel * a.n_chunks + chunk) * (int64_t)clen) + clen;
    uint64_t hm = (uint64_t)hitmask;
    while (hm) {
      const int i = __builtin_ctzll(hm);
      hm &= hm - 1;
      const uint32_t rb = (srec[tid][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      ent[ih++] = (rb << 16) | (uint32_t)(tid * R + i);
      const uint32_t key = half_order_key(rb);
      if ((key >> kFastShift) == tb) atomicAdd(&sub[key & (kFastSubBins - 1)], 1u);
    }
    if (tid == 0) a.cand_count[sel * a.n_chunks + chunk] = (int32_t)total;
  }
  __syncthreads();
  if (tid < kFastSubBins) {
    const uint32_t c = sub[tid];
    if (c != 0u) atomicAdd(blk + kSelSubOff + tid, c);
  }
}

template <bool kFp8, bool kMB>
__global__ __launch_bounds__(kThreads) void cand_rescore_kernel(FastSelArgs a) {
  const int64_t sel = blockIdx.x / (uint32_t)a.cand_wgs;
  const int wg = (int)(blockIdx.x % (uint32_t)a.cand_wgs);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const RowGeom rg = row_geom(a, sel);
  if (rg.w0 <= a.topk || a.topk == 0) return;
  const int clen = a.chunk_len;
  if ((int64_t)wg * clen >= rg.w0) return;

  __shared__ uint32_t ulist[kRsBlk];   // uncertain: key slot << 16 | chunk-relative position
  __shared__ uint32_t wscan[kThreads / 64];
  const int64_t bj = sel / a.Hkv;
  const int g = (int)(sel - bj * a.Hkv);
  const int b = (int)(bj / a.Lq);
  const int r = lane & 15;
  const int rgrp = lane >> 4;
  const int hown = head_of(r);
  uint32_t qp[8][4];   // VALU re-score (up to 8 heads): the scan's row layout
  float Mown = 0.0f, izown = 0.0f;
  WideQuery wq;        // matrix-core re-score (more heads)
  if constexpr (!kMB) {
    load_query(a.q + (bj * a.Hq + (int64_t)g * a.G) * kHeadDim, a.G, r, qp);
    Mown = hown < a.G ? a.mz[(sel * kMaxHeads + hown) * 2] : 0.0f;
    izown = hown < a.G ? a.mz[(sel * kMaxHeads + hown) * 2 + 1] : 0.0f;
  } else {
    load_wide_query(a, sel, bj, g, r, rgrp, wq);
  }

  // E_k: the sub-bins of the threshold bin from the top, one per lane
  const uint32_t* blk = sel_block(a, sel);
  const uint32_t tb = blk[kStFastBin];
  const uint32_t need = (uint32_t)a.topk - blk[kStFastAbove];   // >= 1: the bin holds the k-th
  const uint32_t cum = wave_prefix_incl(blk[kSelSubOff + (kFastSubBins - 1 - lane)]);
  const uint64_t reach = __builtin_amdgcn_ballot_w64(cum >= need);
  uint32_t e_lo, e_hi;   // binary16 bits bracketing E_k (equal once the counts are known)
  if (reach != 0ull) {
    e_lo = e_hi = half_bits_of_key((tb << kFastShift) | (uint32_t)(kFastSubBins - 1 - __builtin_ctzll(reach)));
  } else {   // counts short of `need` cannot happen; the bin's edges remain valid bounds
    e_lo = half_bits_of_key(tb << kFastShift);
    e_hi = half_bits_of_key(((tb + 1) << kFastShift) - 1);
  }
  float lwmin, lwmax;
  log_weight_range(a, sel, lwmin, lwmax);
  const float thr = half_bits_to_float(e_lo) - half_ulp(e_lo) - (lwmax - lwmin) - 2.0f * kBoundSlack;
  const float thr_in = half_bits_to_float(e_hi) + half_ulp(e_hi) + (lwmax - lwmin) + 2.0f * kBoundSlack;

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const uint8_t* kb = a.k + head_row0 * (kFp8 ? 128 : 256);
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;

  for (int chunk = wg; (int64_t)chunk * clen < rg.w0; chunk += a.cand_wgs) {
    const int64_t c0 = (int64_t)chunk * clen;
    const int64_t slot0 = (sel * a.n_chunks + chunk) * (int64_t)clen;
    const uint32_t* ent = reinterpret_cast<const uint32_t*>(a.cand_keys + slot0) + clen;
    const uint32_t cnt = (uint32_t)a.cand_count[sel * a.n_chunks + chunk];
    uint32_t outn = 0;
    for (uint32_t base = 0; base < cnt; base += kRsBlk) {
      // thread t classifies entries base + kRsPer t + i (position order is kept)
      const uint32_t f0 = base + kRsPer * tid;
      uint32_t ev[kRsPer];
      if (f0 + kRsPer <= cnt) {
        const uint4 v4 = *reinterpret_cast<const uint4*>(ent + f0);
        ev[0] = v4.x; ev[1] = v4.y; ev[2] = v4.z; ev[3] = v4.w;
      } else {
#pragma unroll
        for (int i = 0; i < kRsPer; ++i) ev[i] = f0 + i < cnt ? ent[f0 + i] : 0u;
      }
      uint32_t cm = 0u, um = 0u;
#pragma unroll
      for (int i = 0; i < kRsPer; ++i) {
        const uint32_t rb = ev[i] >> 16;
        const float e = half_bits_to_float(rb), u = half_ulp(rb);
        const bool c = f0 + i < cnt && e + u >= thr;
        cm |= (uint32_t)c << i;
        um |= (uint32_t)(c && !(e - u > thr_in)) << i;
      }
      const uint32_t mine = (uint32_t)__builtin_popcount(cm) | ((uint32_t)__builtin_popcount(um) << 16);
      const uint32_t x = wave_prefix_incl(mine);
      __syncthreads();   // the previous block is done with ulist and wscan
      if (lane == 63) wscan[wave] = x;
      __syncthreads();   // every entry of this block has been read
      uint32_t before = x - mine, total = 0;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        total += wscan[w];
        before += w < wave ? wscan[w] : 0u;
      }
      uint32_t ic = outn + (before & 0xFFFFu), iu = before >> 16;
#pragma unroll
      for (int i = 0; i < kRsPer; ++i) {
        if ((cm >> i) & 1u) {
          const uint32_t pos = ev[i] & 0xFFFFu;
          if ((um >> i) & 1u)
            ulist[iu++] = (ic << 16) | pos;
          else
            a.cand_keys[slot0 + ic] = cand_key(0x7F800000u, (int32_t)(c0 + pos));   // certainly selected
          ++ic;
        }
      }
      __syncthreads();
      const int nu = (int)(total >> 16);
      // exact re-score: 4 rows per wave step, the scan's lane layout and arithmetic;
      // the key loads of kRsBatch steps are issued before the first row is scored
      if constexpr (!kMB) {
        for (int i0 = wave * 4; i0 < nu; i0 += 16 * kRsBatch) {
          RowData d[kRsBatch];
          uint32_t ue[kRsBatch];
#pragma unroll
          for (int u = 0; u < kRsBatch; ++u) {
            const int i = i0 + 16 * u + rgrp;
            ue[u] = ulist[i < nu ? i : i0];   // past the end: a valid row, result dropped
            load_key<kFp8>(kb, ksb, (uint32_t)(c0 + (ue[u] & 0xFFFFu)), r, d[u]);
          }
#pragma unroll
          for (int u = 0; u < kRsBatch; ++u) {
            if (i0 + 16 * u < nu) {
              const int i = i0 + 16 * u + rgrp;
              const float l = row_logit<kFp8>(qp, d[u], a.scale_log2);
              const float part = ((r & 1) == 0 && hown < a.G) ? fast_exp2(l - Mown) * izown : 0.0f;
              const float s = rowgroup_sum16(part);
              if (i < nu && r == 0)
                a.cand_keys[slot0 + (ue[u] >> 16)] = cand_key(__float_as_uint(s), (int32_t)(c0 + (ue[u] & 0xFFFFu)));
            }
          }
        }
      } else {
        rescore_wide<kFp8>(nu, wave, r, rgrp, wq, kb, ksb, a.scale_log2, a.G,
                           [&](int i) { return (uint32_t)(c0 + (ulist[i] & 0xFFFFu)); },
                           [&](int i, float sv) {
                             const uint32_t e = ulist[i];
                             a.cand_keys[slot0 + (e >> 16)] = cand_key(__float_as_uint(sv), (int32_t)(c0 + (e & 0xFFFFu)));
                           });
      }
      outn += total & 0xFFFFu;
    }
    if (tid == 0) a.cand_count[sel * a.n_chunks + chunk] = (int32_t)outn;
  }
}

// ------------------------------------------------------------------ exact top-k + output
constexpr int kFinThreads = 1024;
constexpr int kFinStage = 12288;  // candidates staged in LDS (larger sets read global memory)
constexpr int kFinBnd = 1024;     // threshold-bin entries ranked pairwise
constexpr int kDigitBins = 4096;  // first radix digit: score bits 30..19
constexpr int kFinChunkLds = kDigitBins / 2;   // chunks whose counts the general path keeps in lh


// One workgroup per selection.  Stages the candidates (position order) in LDS,
// finds the bin of the k-th largest score with one 4096-bin digit, ranks the
// entries of that bin pairwise by their unique keys to get the k-th key exactly,
// and writes the chosen positions ascending with one block-wide scan, then the
// window.  Candidate sets beyond the LDS stage or threshold bins beyond kFinBnd
// entries take two more radix digits and resolve equal scores in position order.
template <int kFinThreads, int kFinStage, int kFinBnd, int kMaxCh>
__global__ __launch_bounds__(kFinThreads) void final_kernel(FastSelArgs a) {
  constexpr int kFinWaves = kFinThreads / 64;
  // the per-chunk tie pass takes two chunks per thread, for up to kFinChunkLds chunks
  static_assert((kMaxCh < kFinChunkLds ? kMaxCh : kFinChunkLds) <= 2 * kFinThreads, "tie pass covers the chunks");
  const int64_t sel = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int clen = a.chunk_len;
  const int32_t* cc = a.cand_count + sel * a.n_chunks;
  const int64_t lbase = sel * a.n_chunks * (int64_t)clen;
  // Up to 64 chunks a row: every wave reads the 64 counts and, speculatively, the first
  // 64 keys of its chunks wave, wave + kFinWaves, ... (the slots exist whether or not
  // they hold candidates), before the row's length is known; what lies past the row's
  // candidate chunks is dropped below.
  constexpr int kU = 64 / kFinWaves;
  const bool one_round = a.n_chunks <= kFinWaves * kU;
  uint32_t cnt_s = 0u;
  uint64_t kv[kU];
  if (one_round) {
    cnt_s = lane < a.n_chunks ? (uint32_t)cc[lane] : 0u;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = wave + u * kFinWaves;
      kv[u] = c < a.n_chunks ? a.cand_keys[lbase + (int64_t)c * clen + lane] : 0ull;
    }
  }
  const RowGeom rg = row_geom(a, sel);
  const int n = (int)rg.n;
  const int w0 = (int)rg.w0;
  int32_t* out = a.idx + sel * a.S;

  __shared__ uint32_t pref[kMaxCh + 1];
  __shared__ uint32_t lh[kDigitBins];
  __shared__ uint64_t st_key[kFinStage];
  __shared__ uint64_t bkey[kFinBnd];
  __shared__ uint32_t wsum[kFinWaves][2];
  __shared__ uint32_t carry[2];
  __shared__ uint32_t nbnd;
  __shared__ uint64_t kth;

  int kk;
  if (w0 <= a.topk || a.topk == 0) {
    kk = a.topk == 0 ? 0 : w0;
    for (int i = tid; i < kk; i += kFinThreads) out[i] = i;
  } else {
    for (int i = tid; i < kDigitBins; i += kFinThreads) lh[i] = 0u;
    if (tid == 0) {
      nbnd = 0u;
      kth = ~0ull;
    }
    const int nch = (w0 + clen - 1) / clen;
    uint32_t m = 0;
    bool staged;
    if (one_round) {   // nch <= n_chunks <= 64
      const uint32_t cnt = lane < nch ? cnt_s : 0u;
      const uint32_t incl = wave_prefix_incl(cnt);
      m = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      if (wave == 0) {
        if (lane < nch) pref[lane] = incl - cnt;
        if (lane == 0) pref[nch] = m;
      }
      staged = m <= (uint32_t)kFinStage;
      if (staged) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int c = wave + u * kFinWaves;   // wave-uniform
          const uint32_t off = (uint32_t)__builtin_amdgcn_readlane((int)(incl - cnt), c & 63);
          const uint32_t cn = c < nch ? (uint32_t)__builtin_amdgcn_readlane((int)cnt, c & 63) : 0u;
          if ((uint32_t)lane < cn) st_key[off + lane] = kv[u];
          const uint64_t* src = a.cand_keys + lbase + (int64_t)c * clen;
          for (uint32_t j = 64 + lane; j < cn; j += 64) st_key[off + j] = src[j];
        }
      }
      __syncthreads();
    } else {
      for (int cb = 0; cb < nch; cb += 64) {
        const int c = cb + lane;
        const uint32_t cnt = c < nch ? (uint32_t)cc[c] : 0u;
        const uint32_t incl = wave_prefix_incl(cnt);
        if (wave == 0 && c < nch) pref[c] = m + incl - cnt;
        m += (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      }
      if (tid == 0) pref[nch] = m;
      __syncthreads();
      staged = m <= (uint32_t)kFinStage;
      if (staged) {
        for (int c = wave; c < nch; c += kFinWaves) {
          const uint32_t off = pref[c], cn = pref[c + 1] - off;
          const uint64_t* src = a.cand_keys + lbase + (int64_t)c * clen;
          for (uint32_t j = lane; j < cn; j += 64) st_key[off + j] = src[j];
        }
        __syncthreads();
      }
    }
    const uint32_t need0 = (uint32_t)a.topk < m ? (uint32_t)a.topk : m;
    // flat candidate index -> slot in the per-chunk lists (unstaged sets)
    auto slot_of = [&](uint32_t fi) -> int64_t {
      int lo = 0, hi = nch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= fi) lo = mid; else hi = mid - 1;
      }
      return lbase + (int64_t)lo * clen + (fi - pref[lo]);
    };
    auto key_of = [&](uint32_t fi) -> uint64_t {
      return staged ? st_key[fi] : a.cand_keys[slot_of(fi)];
    };
    auto score_bits = [&](uint32_t fi) -> uint32_t { return (uint32_t)(key_of(fi) >> 32); };
    auto position = [&](uint32_t fi) -> int32_t { return key_pos(key_of(fi)); };

    // digit 1: bin b1 of the need0-th largest score
    for (uint32_t fi = tid; fi < m; fi += kFinThreads) atomicAdd(&lh[score_bits(fi) >> 19], 1u);
    __syncthreads();
    uint32_t b1, above1;
    block_threshold<kFinThreads, kDigitBins / kFinThreads>(lh, kDigitBins, need0, b1, above1);
    const uint32_t need1 = need0 - above1;   // >= 1: the bin holds the need0-th entry
    const uint32_t nb1 = lh[b1];
    const bool fastk = staged && nb1 <= (uint32_t)kFinBnd;
    if (fastk) {
      // the bin's entries (any order: their keys are unique)
      for (uint32_t base = 0; base < m; base += kFinThreads) {
        const uint32_t fi = base + tid;
        uint64_t key = 0;
        bool hit = false;
        if (fi < m) {
          key = st_key[fi];
          hit = (uint32_t)(key >> 51) == b1;
        }
        const uint64_t hm = __builtin_amdgcn_ballot_w64(hit);
        if (hm != 0ull) {
          uint32_t wbase = 0;
          if (lane == 0) wbase = atomicAdd(&nbnd, (uint32_t)__builtin_popcountll(hm));
          wbase = (uint32_t)__builtin_amdgcn_readfirstlane((int)wbase);
          if (hit) bkey[wbase + lanes_below(hm)] = key;
        }
      }
      __syncthreads();
      // rank of entry e = number of bin entries with a larger key; rank need1-1 is
      // the k-th.  Lanes hold the comparands, waves take the entries, a ballot counts.
      {
        constexpr int kJ = kFinBnd / 64;
        const uint32_t nj = (nb1 + 63) / 64;
        uint64_t kf[kJ];
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const uint32_t f = (uint32_t)(lane + 64 * j);
          kf[j] = ((uint32_t)j < nj && f < nb1) ? bkey[f] : 0ull;   // keys are > 0
        }
        for (uint32_t e = wave; e < nb1; e += kFinWaves) {
          const uint64_t ke = bkey[e];
          uint32_t rank = 0;
#pragma unroll
          for (int j = 0; j < kJ; ++j)
            if ((uint32_t)j < nj) rank += (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(kf[j] > ke));
          if (rank == need1 - 1 && lane == 0) kth = ke;
        }
      }
      __syncthreads();
      // chosen = key >= kth: each thread takes a run of consecutive candidates
      const uint64_t kt = kth;
      const uint32_t run = (m + kFinThreads - 1) / kFinThreads;
      const uint32_t f0 = tid * run;
      uint32_t mine = 0;
      for (uint32_t i = 0; i < run; ++i) {
        const uint32_t fi = f0 + i;
        mine += (fi < m && st_key[fi] >= kt) ? 1u : 0u;
      }
      const uint32_t incl = wave_prefix_incl(mine);
      if (lane == 63) wsum[wave][0] = incl;
      __syncthreads();
      uint32_t opos = incl - mine, total = 0;
#pragma unroll
      for (int w = 0; w < kFinWaves; ++w) {
        const uint32_t v = wsum[w][0];
        total += v;
        opos += w < wave ? v : 0u;
      }
      for (uint32_t i = 0; i < run; ++i) {
        const uint32_t fi = f0 + i;
        if (fi < m) {
          const uint64_t key = st_key[fi];
          if (key >= kt) {
            if (opos < need0) out[opos] = key_pos(key);
            ++opos;
          }
        }
      }
      kk = (int)(total < need0 ? total : need0);
    } else {
      // general path: two more digits give the exact k-th score value vk; equal
      // scores are taken in position order by the ordered pass.  A candidate set
      // beyond the LDS stage is read straight from the per-chunk lists (wave w takes
      // chunks w, w + kFinWaves, ...: coalesced loads, no flat-index lookups) when its
      // chunk counts fit the histogram's LDS.
      const bool bychunk = !staged && nch <= kFinChunkLds;
      uint32_t prefix = b1, need = need1;
      const int shifts[2] = {7, 0};
      const int widths[2] = {12, 7};
      for (int d = 0; d < 2; ++d) {
        const int sh = shifts[d];
        const uint32_t nb = 1u << widths[d];
        const int shp = d == 0 ? 19 : 7;
        __syncthreads();   // the previous digit's threshold has read lh
        for (uint32_t i = tid; i < nb; i += kFinThreads) lh[i] = 0u;
        __syncthreads();
        if (bychunk) {
          for (int c = wave; c < nch; c += kFinWaves) {
            const uint32_t cn = pref[c + 1] - pref[c];
            const uint64_t* src = a.cand_keys + lbase + (int64_t)c * clen;
            for (uint32_t j = lane; j < cn; j += 64) {
              const uint32_t u = (uint32_t)(src[j] >> 32);
              if ((u >> shp) == prefix) atomicAdd(&lh[(u >> sh) & (nb - 1)], 1u);
            }
          }
        } else {
          for (uint32_t fi = tid; fi < m; fi += kFinThreads) {
            const uint32_t u = score_bits(fi);
            if ((u >> shp) == prefix) atomicAdd(&lh[(u >> sh) & (nb - 1)], 1u);
          }
        }
        __syncthreads();
        uint32_t bd, ab;
        block_threshold<kFinThreads, kDigitBins / kFinThreads>(lh, (int)nb, need, bd, ab);
        need -= ab;
        prefix = (prefix << widths[d]) | bd;
      }
      const uint32_t vk = prefix;   // bits of the k-th largest score
      if (bychunk) {
        // per chunk: keys above vk (cgt) and equal to vk (ctie), in the histogram's LDS
        uint32_t* cgt = lh;
        uint32_t* ctie = lh + kFinChunkLds;
        __syncthreads();
        for (int c = wave; c < nch; c += kFinWaves) {
          const uint32_t cn = pref[c + 1] - pref[c];
          const uint64_t* src = a.cand_keys + lbase + (int64_t)c * clen;
          uint32_t gt = 0, tie = 0;
          for (uint32_t j = lane; j < cn; j += 64) {
            const uint32_t u = (uint32_t)(src[j] >> 32);
            gt += u > vk ? 1u : 0u;
            tie += u == vk ? 1u : 0u;
          }
          gt = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl(gt), 63);
          tie = (uint32_t)__builtin_amdgcn_readlane((int)wave_prefix_incl(tie), 63);
          if (lane == 0) {
            cgt[c] = gt;
            ctie[c] = tie;
          }
        }
        __syncthreads();
        // ties before each chunk (exclusive prefix, in place), then each chunk's chosen
        // count = its keys above vk + the ties it supplies before `need` is reached, and
        // the output offset of each chunk (exclusive prefix of the chosen counts)
        {
          const uint32_t a0 = 2 * tid < nch ? ctie[2 * tid] : 0u;
          const uint32_t a1 = 2 * tid + 1 < nch ? ctie[2 * tid + 1] : 0u;
          const uint32_t incl = wave_prefix_incl(a0 + a1);
          if (lane == 63) wsum[wave][0] = incl;
          __syncthreads();
          uint32_t off = 0;
          for (int w = 0; w < wave; ++w) off += wsum[w][0];
          const uint32_t ex = off + incl - (a0 + a1);
          if (2 * tid < nch) {
            const uint32_t t0 = ex;
            const uint32_t take0 = need > t0 ? min(need - t0, a0) : 0u;
            cgt[2 * tid] += take0;
            ctie[2 * tid] = t0;
          }
          if (2 * tid + 1 < nch) {
            const uint32_t t1 = ex + a0;
            const uint32_t take1 = need > t1 ? min(need - t1, a1) : 0u;
            cgt[2 * tid + 1] += take1;
            ctie[2 * tid + 1] = t1;
          }
        }
        __syncthreads();
        uint32_t chosen_total;
        {
          const uint32_t a0 = 2 * tid < nch ? cgt[2 * tid] : 0u;
          const uint32_t a1 = 2 * tid + 1 < nch ? cgt[2 * tid + 1] : 0u;
          const uint32_t incl = wave_prefix_incl(a0 + a1);
          if (lane == 63) wsum[wave][1] = incl;
          __syncthreads();
          uint32_t off = 0, all = 0;
          for (int w = 0; w < kFinWaves; ++w) {
            all += wsum[w][1];
            off += w < wave ? wsum[w][1] : 0u;
          }
          chosen_total = all;
          const uint32_t ex = off + incl - (a0 + a1);
          __syncthreads();   // every thread has read its counts
          if (2 * tid < nch) cgt[2 * tid] = ex;
          if (2 * tid + 1 < nch) cgt[2 * tid + 1] = ex + a0;
        }
        __syncthreads();
        // ordered write: keys above vk, and ties while their rank (in position order) is
        // below `need`, at the chunk's output offset
        for (int c = wave; c < nch; c += kFinWaves) {
          const uint32_t cn = pref[c + 1] - pref[c];
          const uint64_t* src = a.cand_keys + lbase + (int64_t)c * clen;
          uint32_t opos = cgt[c], trank = ctie[c];
          for (uint32_t j0 = 0; j0 < cn; j0 += 64) {
            const uint32_t j = j0 + lane;
            const bool in = j < cn;
            const uint64_t key = in ? src[j] : 0ull;
            const uint32_t u = (uint32_t)(key >> 32);
            const bool tie = in && u == vk;
            const uint64_t tmask = __builtin_amdgcn_ballot_w64(tie);
            const bool chosen = in && (u > vk || (tie && trank + lanes_below(tmask) < need));
            const uint64_t cmask = __builtin_amdgcn_ballot_w64(chosen);
            const uint32_t o = opos + lanes_below(cmask);
            if (chosen && o < need0) out[o] = key_pos(key);
            opos += (uint32_t)__builtin_popcountll(cmask);
            trank += (uint32_t)__builtin_popcountll(tmask);
          }
        }
        kk = (int)min(need0, chosen_total);
      } else {
      if (tid == 0) {
        carry[0] = 0u;   // chosen so far
        carry[1] = 0u;   // ties so far
      }
      __syncthreads();
      for (uint32_t base = 0; base < m; base += kFinThreads) {
        const uint32_t fi = base + tid;
        const bool in = fi < m;
        const uint32_t u = in ? score_bits(fi) : 0u;
        const bool tie = in && u == vk;
        const uint64_t tmask = __builtin_amdgcn_ballot_w64(tie);
        if (lane == 0) wsum[wave][0] = __builtin_popcountll(tmask);
        __syncthreads();
        uint32_t tie_rank = carry[1] + lanes_below(tmask);
        for (int w = 0; w < wave; ++w) tie_rank += wsum[w][0];
        const bool chosen = in && (u > vk || (tie && tie_rank < need));
        const uint64_t cmask = __builtin_amdgcn_ballot_w64(chosen);
        if (lane == 0) wsum[wave][1] = __builtin_popcountll(cmask);
        __syncthreads();
        uint32_t opos = carry[0] + lanes_below(cmask);
        for (int w = 0; w < wave; ++w) opos += wsum[w][1];
        if (chosen && opos < need0) out[opos] = position(fi);
        __syncthreads();
        if (tid == 0) {
          uint32_t tc = 0, cs = 0;
          for (int w = 0; w < kFinWaves; ++w) {
            tc += wsum[w][0];
            cs += wsum[w][1];
          }
          carry[0] += cs;
          carry[1] += tc;
        }
        __syncthreads();
      }
      kk = (int)min(need0, carry[0]);
      }
    }
  }
  const int nwin = n - w0;
  for (int i = tid; i < nwin; i += kFinThreads) out[kk + i] = w0 + i;
  for (int i = kk + nwin + tid; i < a.S; i += kFinThreads) out[i] = -1;
}

}  // namespace

template <bool kFp8>
void launch_two_step(const FastSelArgs& a, hipStream_t st) {
  const dim3 grid((uint32_t)((uint64_t)a.cand_wgs * (uint64_t)a.n_sel));
  switch (a.chunk_len / kThreads) {
    case 8: hipLaunchKernelGGL((cand_filter_kernel<8>), grid, dim3(kThreads), 0, st, a); break;
    case 16: hipLaunchKernelGGL((cand_filter_kernel<16>), grid, dim3(kThreads), 0, st, a); break;
    case 32: hipLaunchKernelGGL((cand_filter_kernel<32>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((cand_filter_kernel<64>), grid, dim3(kThreads), 0, st, a); break;
  }
  if (a.G > 8)
    hipLaunchKernelGGL((cand_rescore_kernel<kFp8, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((cand_rescore_kernel<kFp8, false>), grid, dim3(kThreads), 0, st, a);
}

template <bool kFp8>
void launch_candidates_r(const FastSelArgs& a, hipStream_t st) {
  const dim3 grid((uint32_t)((uint64_t)a.cand_wgs * (uint64_t)a.n_sel));
  if (a.G > 8) {
    switch (a.chunk_len / kThreads) {
      case 8: hipLaunchKernelGGL((candidate_kernel<kFp8, 8, true>), grid, dim3(kThreads), 0, st, a); break;
      case 16: hipLaunchKernelGGL((candidate_kernel<kFp8, 16, true>), grid, dim3(kThreads), 0, st, a); break;
      case 32: hipLaunchKernelGGL((candidate_kernel<kFp8, 32, true>), grid, dim3(kThreads), 0, st, a); break;
      default: hipLaunchKernelGGL((candidate_kernel<kFp8, 64, true>), grid, dim3(kThreads), 0, st, a); break;
    }
    return;
  }
  switch (a.chunk_len / kThreads) {
    case 8: hipLaunchKernelGGL((candidate_kernel<kFp8, 8, false>), grid, dim3(kThreads), 0, st, a); break;
    case 16: hipLaunchKernelGGL((candidate_kernel<kFp8, 16, false>), grid, dim3(kThreads), 0, st, a); break;
    case 32: hipLaunchKernelGGL((candidate_kernel<kFp8, 32, false>), grid, dim3(kThreads), 0, st, a); break;
    default: hipLaunchKernelGGL((candidate_kernel<kFp8, 64, false>), grid, dim3(kThreads), 0, st, a); break;
  }
}

hipError_t launch_fast_candidates(const FastSelArgs& a, bool fp8, hipStream_t st) {
  if (a.n_sel >= kTwoStepMinRows) {
    if (fp8)
      launch_two_step<true>(a, st);
    else
      launch_two_step<false>(a, st);
  } else if (fp8) {
    launch_candidates_r<true>(a, st);
  } else {
    launch_candidates_r<false>(a, st);
  }
  return hipGetLastError();
}

hipError_t launch_fast_final(const FastSelArgs& a, hipStream_t st) {
  // Many rows (query chunks): half-size workgroups with a 4,096-key stage (~60 KB of
  // LDS: two workgroups per CU) for rows of up to 1,024 candidate chunks; larger sets
  // take the global-memory path of the same kernel.  Few rows: the 1,024-thread form.
  if (a.n_sel >= kTwoStepMinRows && a.n_chunks <= 1024) {
    hipLaunchKernelGGL((final_kernel<512, 4096, 1024, 1024>), dim3(a.n_sel), dim3(512), 0, st, a);
  } else {
    hipLaunchKernelGGL((final_kernel<kFinThreads, kFinStage, kFinBnd, kMaxFastChunks>), dim3(a.n_sel),
                       dim3(kFinThreads), 0, st, a);
  }
  return hipGetLastError();
}

namespace {
// Group-summed probabilities s of every visible position of a row for more than 8
// query heads per KV head (the logits path holds 8 head slots): the candidate stage's
// matrix-core re-score applied to each position once the row's (M, 1/Z) are known.
// Work unit: kProbsChunk positions of one row (blockIdx.x = row * chunks + chunk).
constexpr int kProbsChunk = 2048;
template <bool kFp8>
__global__ __launch_bounds__(kThreads) void probs_wide_kernel(FastSelArgs a, float* probs, int64_t probs_stride,
                                                                int chunks) {
  const int64_t sel = blockIdx.x / (uint32_t)chunks;
  const int64_t p0 = (int64_t)(blockIdx.x % (uint32_t)chunks) * kProbsChunk;
  const RowGeom rg = row_geom(a, sel);
  if (p0 >= rg.n) return;
  const int nu = (int)min((int64_t)kProbsChunk, rg.n - p0);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t bj = sel / a.Hkv;
  const int g = (int)(sel - bj * a.Hkv);
  const int b = (int)(bj / a.Lq);
  const int r = lane & 15;
  const int rgrp = lane >> 4;
  WideQuery wq;
  load_wide_query(a, sel, bj, g, r, rgrp, wq);
  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const uint8_t* kb = a.k + head_row0 * (kFp8 ? 128 : 256);
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  float* prow = probs + sel * probs_stride + p0;
  rescore_wide<kFp8>(nu, wave, r, rgrp, wq, kb, ksb, a.scale_log2, a.G,
                     [&](int i) { return (uint32_t)(p0 + i); }, [&](int i, float sv) { prow[i] = sv; });
}
}  // namespace

hipError_t launch_probs_wide(const FastSelArgs& a, float* probs, int64_t probs_stride, bool fp8, hipStream_t st) {
  if (a.G <= kSlots || a.G > kMaxHeads) return hipErrorInvalidValue;
  const int64_t chunks = (a.ctx_max + kProbsChunk - 1) / kProbsChunk;
  if ((uint64_t)a.n_sel * (uint64_t)chunks > 0x7FFFFFFFull) return hipErrorInvalidValue;   // grid x
  const dim3 grid((uint32_t)((uint64_t)a.n_sel * (uint64_t)chunks));
  if (fp8)
    hipLaunchKernelGGL(probs_wide_kernel<true>, grid, dim3(kThreads), 0, st, a, probs, probs_stride, (int)chunks);
  else
    hipLaunchKernelGGL(probs_wide_kernel<false>, grid, dim3(kThreads), 0, st, a, probs, probs_stride, (int)chunks);
  return hipGetLastError();
}

}  // namespace hs2
