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
//   final_kernel:     exact top-k of the candidates by (s desc, position asc): a
//                     three-digit radix select on the fp32 bit pattern of s (s >= 0
//                     orders like its bits), then an ordered pass that emits the
//                     chosen positions ascending (ties taken in position order),
//                     followed by the window.
#include "hs2_rowops.h"

namespace hs2 {
namespace {

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
    Mh[h] = a.mz[(sel * 8 + h) * 2 + 0];
    iz[h] = a.mz[(sel * 8 + h) * 2 + 1];
  }
}

// Largest bin B with (entries in bins >= B) >= need; also the count strictly above.
// Block-wide over kThreads threads (wave suffix scans + one cross-wave step).  If
// fewer than `need` entries exist, B = 0 and `above` is the total.
template <int NB>
__device__ void threshold_bin(const uint32_t* h, uint32_t need, uint32_t& bin, uint32_t& above) {
  constexpr int PER = NB / kThreads;
  __shared__ uint32_t wtot[kThreads / 64];
  __shared__ uint32_t res[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t loc[PER];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(h + tid * PER + i);
    loc[i] = v.x; loc[i + 1] = v.y; loc[i + 2] = v.z; loc[i + 3] = v.w;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) tot += loc[i];
  uint32_t x = tot;   // inclusive suffix sum within the wave
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off, 64);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) wtot[wave] = x;
  if (tid == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  __syncthreads();
  uint32_t higher = x - tot;
  for (int w = wave + 1; w < kThreads / 64; ++w) higher += wtot[w];
  if (tid == 0) {
    uint32_t all = 0;
    for (int w = 0; w < kThreads / 64; ++w) all += wtot[w];
    if (all < need) res[1] = all;
  }
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
  __syncthreads();
}

constexpr int kRecPerThread = kCandChunkLen / kThreads;   // 64

// ------------------------------------------------------------------ candidates + exact re-score
template <bool kFp8>
__global__ __launch_bounds__(kThreads) void candidate_kernel(FastSelArgs a) {
  const int chunk = blockIdx.x;
  const int64_t sel = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const RowGeom rg = row_geom(a, sel);
  if (rg.w0 <= a.topk || a.topk == 0) return;
  const int64_t c0 = (int64_t)chunk * kCandChunkLen;
  if (c0 >= rg.w0) {
    if (tid == 0) a.cand_count[sel * a.n_chunks + chunk] = 0;
    return;
  }

  __shared__ int32_t cpos[kCandChunkLen];
  __shared__ int32_t total_s;
  float Mh[8], iz[8];
  load_mz(a, sel, Mh, iz);
  const int64_t bj = sel / a.Hkv;
  const int g = (int)(sel - bj * a.Hkv);
  const int b = (int)(bj / a.Lq);
  const int r = lane & 15;
  const int rgrp = lane >> 4;
  const int hown = head_of(r);
  uint32_t qp[8][4];   // issued early: its latency overlaps the threshold and the filter
  load_query(a.q + (bj * a.Hq + (int64_t)g * a.G) * kHeadDim, a.G, r, qp);

  const uint16_t* rrow = a.records + sel * a.rec_stride;
  // Each thread owns kRecPerThread consecutive positions (128 bytes of records, one
  // batch of 16-byte loads); a block-wide exclusive scan of the per-thread hit counts
  // places the candidates in LDS in position order.
  const int64_t t0 = c0 + (int64_t)tid * kRecPerThread;
  uint32_t words[kRecPerThread / 2];
  if (t0 + kRecPerThread <= rg.w0) {
#pragma unroll
    for (int v = 0; v < kRecPerThread / 8; ++v) {
      const uint4 x = *reinterpret_cast<const uint4*>(rrow + t0 + 8 * v);
      words[4 * v + 0] = x.x; words[4 * v + 1] = x.y; words[4 * v + 2] = x.z; words[4 * v + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kRecPerThread / 2; ++i) {
      const int64_t t = t0 + 2 * i;
      const uint32_t lo = t < rg.w0 ? (uint32_t)rrow[t] : 0u;
      const uint32_t hi = t + 1 < rg.w0 ? (uint32_t)rrow[t + 1] : 0u;
      words[i] = lo | (hi << 16);
    }
  }
  // threshold: bin of the k-th largest record key in the merged histogram
  uint32_t tb, above;
  threshold_bin<kFastBins>(sel_block(a, sel) + kSelHist1Off, (uint32_t)a.topk, tb, above);
  const uint32_t ebits = half_bits_of_key(tb << kFastShift);   // smallest record in the bin
  float lwmin = __builtin_huge_valf(), lwmax = -__builtin_huge_valf();
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    if (h < a.G) {
      const float lw = __builtin_amdgcn_logf(iz[h]) - Mh[h];   // log2 w_h
      lwmin = fminf(lwmin, lw);
      lwmax = fmaxf(lwmax, lw);
    }
  }
  // candidate  <=>  e + u(e) + log2 max w  >=  e* - u(e*) + log2 min w  (with slack)
  const float thr = half_bits_to_float(ebits) - half_ulp(ebits) - (lwmax - lwmin) - 2.0f * kBoundSlack;

  uint64_t hitmask = 0ull;
#pragma unroll
  for (int i = 0; i < kRecPerThread; ++i) {
    const uint32_t rb = (words[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
    const bool hit = t0 + i < rg.w0 && half_bits_to_float(rb) + half_ulp(rb) >= thr;
    hitmask |= (uint64_t)hit << i;
  }
  const uint32_t nhit = (uint32_t)__builtin_popcountll(hitmask);
  // block exclusive scan of nhit
  __shared__ uint32_t wscan[kThreads / 64];
  uint32_t x = nhit;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wscan[wave] = x;
  __syncthreads();
  uint32_t before = x - nhit;
  for (int w = 0; w < wave; ++w) before += wscan[w];
  if (tid == kThreads - 1) total_s = (int)(before + nhit);
  uint64_t hm = hitmask;
  while (hm) {
    const int i = __builtin_ctzll(hm);
    hm &= hm - 1;
    cpos[before++] = (int32_t)(t0 + i);
  }
  __syncthreads();
  const int cnt = total_s;
  const int64_t slot0 = (sel * a.n_chunks + chunk) * (int64_t)kCandChunkLen;
  if (tid == 0) a.cand_count[sel * a.n_chunks + chunk] = cnt;
  if (cnt == 0) return;

  // exact re-score: 4 rows per wave step, the scan's lane layout and arithmetic
  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const uint8_t* kb = a.k + head_row0 * (kFp8 ? 128 : 256);
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float Mown = Mh[hown];
  const float izown = iz[hown];
  for (int i0 = wave * 4; i0 < cnt; i0 += 16) {
    const int i = i0 + rgrp;
    const bool valid = i < cnt;
    const int32_t t = cpos[valid ? i : i0];
    RowData d;
    load_key<kFp8>(kb, ksb, (uint32_t)t, r, d);
    const float l = row_logit<kFp8>(qp, d, a.scale_log2);
    float part = ((r & 1) == 0 && hown < a.G) ? fast_exp2(l - Mown) * izown : 0.0f;
    const float s = rowgroup_sum16(part);
    if (valid && r == 0) {
      a.cand_pos[slot0 + i] = t;
      a.cand_s[slot0 + i] = s;
    }
  }
}

// ------------------------------------------------------------------ exact top-k + output
constexpr int kFinThreads = 1024;
constexpr int kFinStage = 6144;   // candidates staged in LDS (larger sets read global memory)
constexpr int kFinBnd = 1024;     // threshold-bin entries ranked by brute force

// Largest bin B of an LDS histogram with (entries in bins >= B) >= need, and the
// count strictly above B.  Block-wide over kFinThreads threads (nb <= 4 per thread).
__device__ void block_threshold(const uint32_t* lh, uint32_t nb, uint32_t need, uint32_t& bin,
                                uint32_t& above) {
  __shared__ uint32_t wtot[kFinThreads / 64];
  __shared__ uint32_t res[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t per = nb / kFinThreads > 0 ? nb / kFinThreads : 1;
  uint32_t loc[4];
  uint32_t tot = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t bidx = tid * per + q;
    loc[q] = (q < (int)per && bidx < nb) ? lh[bidx] : 0u;
    tot += loc[q];
  }
  uint32_t x = tot;   // inclusive suffix sum within the wave
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off, 64);
    if (lane + off < 64) x += y;
  }
  if (lane == 0) wtot[wave] = x;
  if (tid == 0) {
    res[0] = 0u;
    res[1] = 0u;
  }
  __syncthreads();
  uint32_t higher = x - tot;
  for (int w = wave + 1; w < kFinThreads / 64; ++w) higher += wtot[w];
  if (higher < need && higher + tot >= need) {
    uint32_t cum = higher;
    for (int q = (int)per - 1; q >= 0; --q) {
      if (cum + loc[q] >= need) {
        res[0] = tid * per + q;
        res[1] = cum;
        break;
      }
      cum += loc[q];
    }
  }
  __syncthreads();
  bin = res[0];
  above = res[1];
  __syncthreads();
}

__global__ __launch_bounds__(kFinThreads) void final_kernel(FastSelArgs a) {
  const int64_t sel = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const RowGeom rg = row_geom(a, sel);
  const int n = (int)rg.n;
  const int w0 = (int)rg.w0;
  int32_t* out = a.idx + sel * a.S;

  __shared__ uint32_t pref[kMaxFastChunks + 1];
  __shared__ uint32_t lh[kFastBins];
  __shared__ int32_t st_pos[kFinStage];
  __shared__ uint32_t st_s[kFinStage];
  __shared__ uint8_t flag[kFinStage];
  __shared__ uint32_t blist[kFinBnd];
  __shared__ uint32_t bnd_s[kFinBnd];
  __shared__ int32_t bnd_p[kFinBnd];
  __shared__ uint32_t nbnd;
  __shared__ uint32_t wsum[kFinThreads / 64][2];
  __shared__ uint32_t carry[2];

  int kk;
  if (w0 <= a.topk || a.topk == 0) {
    kk = a.topk == 0 ? 0 : w0;
    for (int i = tid; i < kk; i += kFinThreads) out[i] = i;
  } else {
    kk = a.topk;
    const int nch = (w0 + kCandChunkLen - 1) / kCandChunkLen;
    const int32_t* cc = a.cand_count + sel * a.n_chunks;
    // exclusive prefix of the per-chunk counts (serial per 1024 chunks, then fix-up)
    for (int base = 0; base < nch; base += kFinThreads) {
      const int c = base + tid;
      const uint32_t v = c < nch ? (uint32_t)cc[c] : 0u;
      // wave-level inclusive scan
      uint32_t x = v;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane == 63) wsum[wave][0] = x;
      __syncthreads();
      uint32_t wpre = base == 0 ? 0u : pref[base];
      for (int w = 0; w < wave; ++w) wpre += wsum[w][0];
      if (c < nch) pref[c] = wpre + x - v;
      __syncthreads();
      if (tid == 0) {
        uint32_t t = base == 0 ? 0u : pref[base];
        for (int w = 0; w < kFinThreads / 64; ++w) t += wsum[w][0];
        pref[min(base + kFinThreads, nch)] = t;
      }
      __syncthreads();
    }
    const uint32_t m = pref[nch];
    const int64_t lbase = sel * a.n_chunks * (int64_t)kCandChunkLen;
    // flat index -> candidate slot (binary search over the chunk prefix)
    auto slot_of = [&](uint32_t fi) -> int64_t {
      int lo = 0, hi = nch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= fi) lo = mid; else hi = mid - 1;
      }
      return lbase + (int64_t)lo * kCandChunkLen + (fi - pref[lo]);
    };
    const uint32_t need0 = (uint32_t)kk < m ? (uint32_t)kk : m;
    // stage the candidates in LDS (position order) when they fit; the passes below
    // then read LDS instead of chasing per-chunk lists in global memory
    const bool staged = m <= (uint32_t)kFinStage;
    if (staged) {
      for (uint32_t fi = tid; fi < m; fi += kFinThreads) {
        const int64_t slot = slot_of(fi);
        st_pos[fi] = a.cand_pos[slot];
        st_s[fi] = __float_as_uint(a.cand_s[slot]);
      }
      __syncthreads();
    }
    auto score_bits = [&](uint32_t fi) -> uint32_t {
      return staged ? st_s[fi] : __float_as_uint(a.cand_s[slot_of(fi)]);
    };
    auto position = [&](uint32_t fi) -> int32_t {
      return staged ? st_pos[fi] : a.cand_pos[slot_of(fi)];
    };

    // Radix digit 1 (score bits 30..19) finds the bin B holding the k-th largest
    // score.  If that bin is small and the candidates are staged, its entries are
    // ranked exactly by brute force (score desc, position asc); otherwise two more
    // digits give the exact k-th value and ties are taken in position order.
    for (uint32_t i = tid; i < (uint32_t)kFastBins; i += kFinThreads) lh[i] = 0u;
    if (tid == 0) {
      carry[0] = 0u;
      carry[1] = 0u;
      nbnd = 0u;
    }
    __syncthreads();
    for (uint32_t fi = tid; fi < m; fi += kFinThreads) atomicAdd(&lh[score_bits(fi) >> 19], 1u);
    __syncthreads();
    uint32_t b1, above1;
    block_threshold(lh, kFastBins, need0, b1, above1);
    const uint32_t need1 = need0 - above1;
    bool brute = false;
    if (staged) {
      // entries of bin b1, compacted in position order by ballot prefix sums
      for (uint32_t base = 0; base < m; base += kFinThreads) {
        const uint32_t fi = base + tid;
        const bool in = fi < m;
        if (in) flag[fi] = 0u;
        const bool hit = in && (st_s[fi] >> 19) == b1;
        const uint64_t hmask = __builtin_amdgcn_ballot_w64(hit);
        if (lane == 0) wsum[wave][0] = __builtin_popcountll(hmask);
        __syncthreads();
        uint32_t slot = nbnd + __builtin_popcountll(hmask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        for (int w = 0; w < wave; ++w) slot += wsum[w][0];
        if (hit && slot < (uint32_t)kFinBnd) blist[slot] = fi;
        __syncthreads();
        if (tid == 0) {
          uint32_t t = nbnd;
          for (int w = 0; w < kFinThreads / 64; ++w) t += wsum[w][0];
          nbnd = t;
        }
        __syncthreads();
      }
      brute = nbnd <= (uint32_t)kFinBnd;
    }
    uint32_t vk = 0u, need = need1;
    if (brute) {
      const uint32_t nb = nbnd;
      for (uint32_t e = tid; e < nb; e += kFinThreads) {
        bnd_s[e] = st_s[blist[e]];
        bnd_p[e] = st_pos[blist[e]];
      }
      __syncthreads();
      for (uint32_t e = tid; e < nb; e += kFinThreads) {
        const uint32_t se = bnd_s[e];
        const int32_t pe = bnd_p[e];
        uint32_t rank = 0;
        for (uint32_t f = 0; f < nb; ++f) {   // broadcast LDS reads, independent iterations
          const uint32_t sf = bnd_s[f];
          const int32_t pf = bnd_p[f];
          rank += (sf > se || (sf == se && pf < pe)) ? 1u : 0u;
        }
        flag[blist[e]] = rank < need1 ? 1u : 0u;
      }
      __syncthreads();
    } else {
      uint32_t prefix = b1;
      const int shifts[2] = {7, 0};
      const int widths[2] = {12, 7};
      for (int d = 0; d < 2; ++d) {
        const int sh = shifts[d];
        const uint32_t nb = 1u << widths[d];
        const int shp = d == 0 ? 19 : 7;
        for (uint32_t i = tid; i < nb; i += kFinThreads) lh[i] = 0u;
        __syncthreads();
        for (uint32_t fi = tid; fi < m; fi += kFinThreads) {
          const uint32_t u = score_bits(fi);
          if ((u >> shp) == prefix) atomicAdd(&lh[(u >> sh) & (nb - 1)], 1u);
        }
        __syncthreads();
        uint32_t bd, ab;
        block_threshold(lh, nb, need, bd, ab);
        need -= ab;
        prefix = (prefix << widths[d]) | bd;
      }
      vk = prefix;   // bits of the k-th largest score
    }
    // ordered output of the chosen candidates
    if (tid == 0) {
      carry[0] = 0u;   // chosen so far
      carry[1] = 0u;   // ties so far (general path)
    }
    __syncthreads();
    for (uint32_t base = 0; base < m; base += kFinThreads) {
      const uint32_t fi = base + tid;
      const bool in = fi < m;
      const uint32_t u = in ? score_bits(fi) : 0u;
      const bool tie = !brute && in && u == vk;
      const uint64_t tmask = __builtin_amdgcn_ballot_w64(tie);
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (lane == 0) wsum[wave][0] = __builtin_popcountll(tmask);
      __syncthreads();
      uint32_t tie_rank = carry[1] + __builtin_popcountll(tmask & below);
      for (int w = 0; w < wave; ++w) tie_rank += wsum[w][0];
      const bool chosen = in && (brute ? ((u >> 19) > b1 || flag[fi] != 0u)
                                       : (u > vk || (tie && tie_rank < need)));
      const uint64_t cmask = __builtin_amdgcn_ballot_w64(chosen);
      __syncthreads();
      if (lane == 0) wsum[wave][1] = __builtin_popcountll(cmask);
      __syncthreads();
      uint32_t opos = carry[0] + __builtin_popcountll(cmask & below);
      for (int w = 0; w < wave; ++w) opos += wsum[w][1];
      if (chosen && opos < (uint32_t)kk) out[opos] = position(fi);
      __syncthreads();
      if (tid == 0) {
        uint32_t tc = 0, cs = 0;
        for (int w = 0; w < kFinThreads / 64; ++w) {
          tc += wsum[w][0];
          cs += wsum[w][1];
        }
        carry[0] += cs;
        carry[1] += tc;
      }
      __syncthreads();
    }
    kk = (int)min((uint32_t)kk, carry[0]);
  }
  const int nwin = n - w0;
  for (int i = tid; i < nwin; i += kFinThreads) out[kk + i] = w0 + i;
  for (int i = kk + nwin + tid; i < a.S; i += kFinThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_fast_candidates(const FastSelArgs& a, bool fp8, hipStream_t st) {
  if (fp8)
    hipLaunchKernelGGL(candidate_kernel<true>, dim3(a.n_chunks, a.n_sel), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(candidate_kernel<false>, dim3(a.n_chunks, a.n_sel), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fast_final(const FastSelArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(final_kernel, dim3(a.n_sel), dim3(kFinThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs2
