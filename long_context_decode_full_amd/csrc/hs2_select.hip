// Token selection of the Full Attention layer (HySparse2 article, section 03:
// keep the 128 most recent tokens and the 1,024 highest-scoring tokens outside
// that window; section 02: the scores are the full layer's own attention).
//
// Score of position t for KV head g: s[t] = sum over the group's query heads h of
// exp2(l_h[t] - M_h) / Z_h, from the logits and the softmax statistics the scan
// and combine kernels produced.  Selection is an exact top-k with ties to the
// lower position, done as a radix select on the fp32 bit pattern of s (s >= 0,
// so the unsigned bit pattern orders like the value):
//   pass 1 (groupsum_kernel): compute s, store it, LDS histogram of bits 30..20
//   pass 2/3 (refine_kernel): histograms of bits 19..8 and 7..0 inside the
//          threshold bin, only while that bin holds more than kBoundaryCap entries
//   collect_kernel: strict winners and the threshold-bin entries, wave-aggregated
//          atomic appends
//   finalize_kernel: one workgroup per row sorts the threshold-bin entries by
//          (score desc, position asc) in LDS, takes what is missing, sorts the
//          selected positions and appends the window.
// The last workgroup of each histogram pass (atomic ticket) computes the
// threshold bin for the row, so no separate launch is needed for it.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr int kThreads = 256;

struct RowGeom {
  int64_t n;    // visible positions
  int64_t w0;   // candidates are [0, w0); window is [w0, n)
};

__device__ __forceinline__ uint32_t* sel_state(const SelectArgs& a, int64_t sel) {
  return a.selblk + sel * kSelWords;
}

__device__ __forceinline__ RowGeom row_geom(const SelectArgs& a, int64_t sel) {
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

// Block-wide: is this the last workgroup of the pass for row `sel`?
__device__ bool last_block(uint32_t* counter, int nblocks) {
  __shared__ int is_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = atomicAdd(counter, 1u);
    is_last = (prev == (uint32_t)(nblocks - 1));
  }
  __syncthreads();
  return is_last != 0;
}

// Merge an LDS histogram into the global one (non-empty bins only).
template <int NB>
__device__ void merge_hist(const uint32_t* lh, uint32_t* gh) {
  for (int i = threadIdx.x; i < NB; i += kThreads) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(gh + i, c);
  }
}

// Threshold bin of a global histogram: largest bin B with (count of bins >= B) >= need.
// Returns B, the count strictly above B and the count in B (block-wide, 256 threads).
template <int NB>
__device__ void find_threshold(const uint32_t* gh, uint32_t need, uint32_t& bin, uint32_t& above,
                               uint32_t& inbin) {
  constexpr int PER = NB / kThreads > 0 ? NB / kThreads : 1;
  __shared__ uint32_t tsum[kThreads];
  __shared__ uint32_t res[3];
  const int tid = threadIdx.x;
  uint32_t loc[PER];
  uint32_t total = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int b = tid * PER + i;
    loc[i] = b < NB ? atomic_load_relaxed(gh + b) : 0u;
    total += loc[i];
  }
  tsum[tid] = total;
  __syncthreads();
  // inclusive suffix sums over threads (Hillis-Steele)
  for (int off = 1; off < kThreads; off <<= 1) {
    const uint32_t v = (tid + off < kThreads) ? tsum[tid + off] : 0u;
    __syncthreads();
    tsum[tid] += v;
    __syncthreads();
  }
  uint32_t cum = (tid + 1 < kThreads) ? tsum[tid + 1] : 0u;  // count in higher threads
  if (cum < need && cum + total >= need) {
#pragma unroll
    for (int i = PER - 1; i >= 0; --i) {
      if (cum + loc[i] >= need) {
        res[0] = (uint32_t)(tid * PER + i);
        res[1] = cum;
        res[2] = loc[i];
        break;
      }
      cum += loc[i];
    }
  }
  __syncthreads();
  bin = res[0];
  above = res[1];
  inbin = res[2];
  __syncthreads();
}

// ------------------------------------------------------------------ pass 1
__global__ __launch_bounds__(kThreads) void groupsum_kernel(SelectArgs a) {
  // blockIdx.x = row * n_chunks + chunk (rows can exceed the 65,535 of grid y)
  const int chunk = (int)(blockIdx.x % (uint32_t)a.n_chunks);
  const int64_t sel = blockIdx.x / (uint32_t)a.n_chunks;
  const int tid = threadIdx.x;
  const RowGeom rg = row_geom(a, sel);

  __shared__ uint32_t lh[kHist1Bins];
  if (a.with_hist)
    for (int i = tid; i < kHist1Bins; i += kThreads) lh[i] = 0u;

  float Mh[8], iz[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    Mh[h] = a.mz[(sel * kMaxHeads + h) * 2 + 0];
    iz[h] = a.mz[(sel * kMaxHeads + h) * 2 + 1];
  }
  __syncthreads();

  const float* lrow = a.logits + sel * a.logit_stride * 8;
  float* srow = a.s + sel * a.s_stride;
  const int64_t c0 = (int64_t)chunk * a.chunk_len;
  int64_t c1 = c0 + a.chunk_len;
  c1 = c1 < rg.n ? c1 : rg.n;
  for (int64_t t = c0 + tid; t < c1; t += kThreads) {
    const float4 l0 = *reinterpret_cast<const float4*>(lrow + t * 8);
    const float4 l1 = *reinterpret_cast<const float4*>(lrow + t * 8 + 4);
    const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
    float s = 0.0f;
#pragma unroll
    for (int h = 0; h < 8; ++h)
      if (h < a.G) s = __builtin_fmaf(fast_exp2(lv[h] - Mh[h]), iz[h], s);
    srow[t] = s;
    if (a.with_hist && t < rg.w0) atomicAdd(&lh[(__float_as_uint(s) >> 20) & (kHist1Bins - 1)], 1u);
  }
  if (!a.with_hist) return;
  __syncthreads();
  merge_hist<kHist1Bins>(lh, sel_state(a, sel) + kSelHist1Off);
  if (!last_block(sel_state(a, sel) + kSelCounterOff + 0, a.n_chunks)) return;

  // Last workgroup of the row: decide how the row continues.
  uint32_t* st = sel_state(a, sel);
  const uint32_t ncand = (uint32_t)rg.w0;
  if (ncand <= (uint32_t)a.topk || a.topk == 0) {
    // every candidate (or none, when topk is 0) is selected: no threshold needed
    if (tid == 0) {
      st[kStTakeAll] = 1u;
      st[kStKK] = a.topk == 0 ? 0u : ncand;
      st[kStResolved] = 1u;
    }
    return;
  }
  uint32_t bin, above, inbin;
  find_threshold<kHist1Bins>(st + kSelHist1Off, (uint32_t)a.topk, bin, above, inbin);
  const bool resolved = inbin <= (uint32_t)kBoundaryCap;
  if (!resolved)
    for (int i = tid; i < kHist2Bins; i += kThreads) a.hist2[sel * kHist2Bins + i] = 0u;
  if (tid == 0) {
    st[kStTakeAll] = 0u;
    st[kStKK] = (uint32_t)a.topk;
    st[kStPrefix] = bin;
    st[kStPrefixLen] = 11u;
    st[kStAbove] = above;
    st[kStInBin] = inbin;
    st[kStResolved] = resolved ? 1u : 0u;
    st[kStWinCount] = 0u;
    st[kStBndCount] = 0u;
  }
}

// ------------------------------------------------------------------ passes 2 and 3
template <int PASS>
__global__ __launch_bounds__(kThreads) void refine_kernel(SelectArgs a) {
  constexpr int NB = PASS == 2 ? kHist2Bins : kHist3Bins;
  constexpr int DIGIT = PASS == 2 ? 12 : 8;
  // blockIdx.x = row * n_chunks + chunk (rows can exceed the 65,535 of grid y)
  const int chunk = (int)(blockIdx.x % (uint32_t)a.n_chunks);
  const int64_t sel = blockIdx.x / (uint32_t)a.n_chunks;
  const int tid = threadIdx.x;
  uint32_t* st = sel_state(a, sel);
  if (st[kStResolved]) return;   // uniform across the row's workgroups
  const RowGeom rg = row_geom(a, sel);
  const uint32_t prefix = st[kStPrefix];
  const uint32_t plen = st[kStPrefixLen];
  const uint32_t shift_prev = 31u - plen;
  const uint32_t shift = shift_prev - DIGIT;

  __shared__ uint32_t lh[NB];
  for (int i = tid; i < NB; i += kThreads) lh[i] = 0u;
  __syncthreads();
  const float* srow = a.s + sel * a.s_stride;
  const int64_t c0 = (int64_t)chunk * a.chunk_len;
  int64_t c1 = c0 + a.chunk_len;
  c1 = c1 < rg.w0 ? c1 : rg.w0;
  for (int64_t t = c0 + tid; t < c1; t += kThreads) {
    const uint32_t u = __float_as_uint(srow[t]);
    if ((u >> shift_prev) == prefix) atomicAdd(&lh[(u >> shift) & (NB - 1)], 1u);
  }
  __syncthreads();
  uint32_t* gh = (PASS == 2 ? a.hist2 + sel * kHist2Bins : a.hist3 + sel * kHist3Bins);
  merge_hist<NB>(lh, gh);
  if (!last_block(st + kSelCounterOff + (PASS - 1), a.n_chunks)) return;

  const uint32_t above0 = st[kStAbove];
  const uint32_t need = st[kStKK] - above0;
  uint32_t bin, above, inbin;
  find_threshold<NB>(gh, need, bin, above, inbin);
  const bool resolved = inbin <= (uint32_t)kBoundaryCap || PASS == 3;
  if (!resolved && PASS == 2)
    for (int i = tid; i < kHist3Bins; i += kThreads) a.hist3[sel * kHist3Bins + i] = 0u;
  if (tid == 0) {
    st[kStPrefix] = (prefix << DIGIT) | bin;
    st[kStPrefixLen] = plen + DIGIT;
    st[kStAbove] = above0 + above;
    st[kStInBin] = inbin;
    st[kStResolved] = resolved ? 1u : 0u;
  }
}

// ------------------------------------------------------------------ collect
__device__ __forceinline__ uint32_t wave_append(bool pred, uint32_t* counter) {
  const uint64_t mask = __builtin_amdgcn_ballot_w64(pred);
  if (mask == 0) return 0u;
  const int lane = threadIdx.x & 63;
  const int leader = __builtin_ctzll(mask);
  uint32_t base = 0;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__builtin_popcountll(mask));
  base = __shfl(base, leader, 64);
  const uint64_t below = mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
  return base + (uint32_t)__builtin_popcountll(below);
}

__global__ __launch_bounds__(kThreads) void collect_kernel(SelectArgs a) {
  // blockIdx.x = row * n_chunks + chunk (rows can exceed the 65,535 of grid y)
  const int chunk = (int)(blockIdx.x % (uint32_t)a.n_chunks);
  const int64_t sel = blockIdx.x / (uint32_t)a.n_chunks;
  const int tid = threadIdx.x;
  uint32_t* st = sel_state(a, sel);
  if (st[kStTakeAll]) return;
  const RowGeom rg = row_geom(a, sel);
  const uint32_t prefix = st[kStPrefix];
  const uint32_t shift = 31u - st[kStPrefixLen];
  const float* srow = a.s + sel * a.s_stride;
  int32_t* win = a.winners + sel * a.topk;
  uint2* bnd = a.boundary + sel * kBoundaryCap;
  const int64_t c0 = (int64_t)chunk * a.chunk_len;
  int64_t c1 = c0 + a.chunk_len;
  c1 = c1 < rg.w0 ? c1 : rg.w0;
  // every lane of a wave runs the same trip count (ballots need the full wave)
  for (int64_t base = c0; base < c1; base += kThreads) {
    const int64_t t = base + tid;
    const bool in = t < c1;
    const uint32_t u = in ? __float_as_uint(srow[t]) : 0u;
    const uint32_t key = u >> shift;
    const bool is_win = in && key > prefix;
    const bool is_bnd = in && key == prefix;
    const uint32_t wslot = wave_append(is_win, st + kStWinCount);
    const uint32_t bslot = wave_append(is_bnd, st + kStBndCount);
    if (is_win && wslot < (uint32_t)a.topk) win[wslot] = (int32_t)t;
    if (is_bnd && bslot < (uint32_t)kBoundaryCap) bnd[bslot] = make_uint2(u, (uint32_t)t);
  }
}

// ------------------------------------------------------------------ finalize
template <typename T>
__device__ void bitonic_sort_desc(T* v, int npow2) {
  for (int k = 2; k <= npow2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < npow2; i += blockDim.x) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const T x = v[i], y = v[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            v[i] = y;
            v[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

constexpr int kFinThreads = 512;

__global__ __launch_bounds__(kFinThreads) void finalize_kernel(SelectArgs a) {
  const int64_t sel = blockIdx.x;
  const int tid = threadIdx.x;
  const RowGeom rg = row_geom(a, sel);
  const uint32_t* st = sel_state(a, sel);
  int32_t* out = a.idx + sel * a.S;

  __shared__ uint64_t keys[kBoundaryCap];
  __shared__ int32_t top[4096];
  __shared__ int32_t scan_take;

  const int n = (int)rg.n;
  const int w0 = (int)rg.w0;
  int kk;
  if (st[kStTakeAll]) {
    kk = (int)st[kStKK];
    for (int i = tid; i < kk; i += kFinThreads) top[i] = i;
    __syncthreads();
  } else {
    kk = (int)st[kStKK];
    const int above = (int)st[kStAbove];
    const int need = kk - above;
    const int32_t* win = a.winners + sel * a.topk;
    for (int i = tid; i < above; i += kFinThreads) top[i] = win[i];
    const uint32_t bcount = st[kStBndCount];
    if (bcount <= (uint32_t)kBoundaryCap) {
      const int m = (int)bcount;
      const int np = pow2_at_least(m > 1 ? m : 1);
      const uint2* bnd = a.boundary + sel * kBoundaryCap;
      for (int i = tid; i < np; i += kFinThreads) {
        if (i < m) {
          const uint2 e = bnd[i];
          keys[i] = ((uint64_t)e.x << 32) | (uint64_t)(0xFFFFFFFFu - e.y);
        } else {
          keys[i] = 0ull;
        }
      }
      __syncthreads();
      bitonic_sort_desc(keys, np);
      for (int i = tid; i < need; i += kFinThreads)
        top[above + i] = (int32_t)(0xFFFFFFFFu - (uint32_t)(keys[i] & 0xFFFFFFFFull));
      __syncthreads();
    } else {
      // More exactly-equal scores than the boundary buffer holds: every entry of the
      // threshold bin has the same score, so take them in position order.
      const uint32_t vk = st[kStPrefix];
      const float* srow = a.s + sel * a.s_stride;
      __shared__ int32_t wave_cnt[kFinThreads / 64];
      if (tid == 0) scan_take = 0;
      __syncthreads();
      for (int base = 0; base < w0; base += kFinThreads) {
        const int t = base + tid;
        const bool hit = t < w0 && __float_as_uint(srow[t]) == vk;
        const uint64_t mask = __builtin_amdgcn_ballot_w64(hit);
        const int lane = tid & 63, wv = tid >> 6;
        if (lane == 0) wave_cnt[wv] = __builtin_popcountll(mask);
        __syncthreads();
        int before = scan_take;
        for (int w = 0; w < wv; ++w) before += wave_cnt[w];
        const uint64_t below = mask & ((lane == 0) ? 0ull : (~0ull >> (64 - lane)));
        const int rank = before + __builtin_popcountll(below);
        if (hit && rank < need) top[above + rank] = t;
        __syncthreads();
        if (tid == 0) {
          int tot = scan_take;
          for (int w = 0; w < kFinThreads / 64; ++w) tot += wave_cnt[w];
          scan_take = tot;
        }
        __syncthreads();
        if (scan_take >= need) break;
      }
    }
  }
  // ascending order of the selected global positions
  {
    const int np = pow2_at_least(kk > 1 ? kk : 1);
    for (int i = tid + kk; i < np; i += kFinThreads) top[i] = -1;   // sorts last in descending order
    __syncthreads();
    bitonic_sort_desc(top, np);
    // top[0..kk) is descending; write ascending
    for (int i = tid; i < kk; i += kFinThreads) out[i] = top[kk - 1 - i];
  }
  const int nwin = n - w0;
  for (int i = tid; i < nwin; i += kFinThreads) out[kk + i] = w0 + i;
  for (int i = kk + nwin + tid; i < a.S; i += kFinThreads) out[i] = -1;
}

// ------------------------------------------------------------------ block comparator
// First-generation HySparse selected whole blocks (article sections 01 and 03).
// Block score = sum of s over the block's visible positions; the n_blocks best
// blocks (ties to the lower block) are expanded to their visible positions.
constexpr int kBlkThreads = 1024;

// Block masses from the scans' block sums: per aligned block of blse_gran positions and
// head h, L_h = log2 sum 2^logit, so the block's share of head h's softmax is
// 2^(L_h - M_h) / Z_h; a block's mass adds those of its block sums and heads h < G in
// that order (sums ascending, heads ascending).  H = blse_heads_of(G) head slots.
template <int H>
__device__ __forceinline__ void load_head_stats(const SelectArgs& a, int64_t sel, float (&Mh)[H], float (&iz)[H]) {
#pragma unroll
  for (int h = 0; h < H; ++h) {
    Mh[h] = a.mz[(sel * kMaxHeads + h) * 2 + 0];
    iz[h] = a.mz[(sel * kMaxHeads + h) * 2 + 1];
  }
}
template <int H>
__device__ __forceinline__ void load_block_sum(const float* brow, int sb, float4 (&l)[H / 4]) {
#pragma unroll
  for (int j = 0; j < H / 4; ++j) l[j] = *reinterpret_cast<const float4*>(brow + (int64_t)sb * H + 4 * j);
}
template <int H>
__device__ __forceinline__ float add_block_sum(float acc, const float4 (&l)[H / 4], const float (&Mh)[H],
                                               const float (&iz)[H], int G) {
#pragma unroll
  for (int j = 0; j < H / 4; ++j) {
    const float lv[4] = {l[j].x, l[j].y, l[j].z, l[j].w};
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (4 * j + c < G) acc += fast_exp2(lv[c] - Mh[4 * j + c]) * iz[4 * j + c];
  }
  return acc;
}

template <int H>   // block-sum head slots (blse_heads_of(G))
__global__ __launch_bounds__(kBlkThreads) void block_select_kernel(SelectArgs a) {
  const int64_t sel = blockIdx.x;
  const int tid = threadIdx.x;
  const RowGeom rg = row_geom(a, sel);
  const int n = (int)rg.n;
  const int bs = a.block_size;
  const int nb = (n + bs - 1) / bs;
  const float* srow = a.s + sel * a.s_stride;
  int32_t* out = a.idx + sel * a.S;

  __shared__ float mass[kMaxBlocksLds];
  __shared__ int32_t chosen[4096];
  __shared__ float red_v[kBlkThreads / 64];
  __shared__ int32_t red_i[kBlkThreads / 64];
  __shared__ int32_t cnt[4097];

  if (a.blse != nullptr) {
    // the scans' block sums (bs is a multiple of blse_gran)
    float Mh[H], iz[H];
    load_head_stats<H>(a, sel, Mh, iz);
    const int gran = a.blse_gran;
    const int sub = bs / gran;
    const int nsub = (n + gran - 1) / gran;   // block sums holding visible positions
    const float* brow = a.blse + sel * a.blse_stride * H;
    for (int blk = tid; blk < nb; blk += kBlkThreads) {
      float acc = 0.0f;
      for (int u = 0; u < sub; ++u) {
        const int sb = blk * sub + u;
        if (sb >= nsub) break;
        float4 l[H / 4];
        load_block_sum<H>(brow, sb, l);
        acc = add_block_sum<H>(acc, l, Mh, iz, a.G);
      }
      mass[blk] = acc;
    }
  } else {
    for (int blk = tid; blk < nb; blk += kBlkThreads) {
      const int t0 = blk * bs;
      const int t1 = (t0 + bs < n) ? t0 + bs : n;
      float acc = 0.0f;
      for (int t = t0; t < t1; ++t) acc += srow[t];
      mass[blk] = acc;
    }
  }
  __syncthreads();
  const int take = a.n_blocks < nb ? a.n_blocks : nb;
  for (int round = 0; round < take; ++round) {
    float bv = -1.0f;
    int bi = 0x7FFFFFFF;
    for (int blk = tid; blk < nb; blk += kBlkThreads) {
      const float v = mass[blk];
      if (v > bv || (v == bv && blk < bi)) { bv = v; bi = blk; }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if ((tid & 63) == 0) { red_v[tid >> 6] = bv; red_i[tid >> 6] = bi; }
    __syncthreads();
    if (tid == 0) {
      float v = red_v[0];
      int ii = red_i[0];
      for (int w = 1; w < kBlkThreads / 64; ++w)
        if (red_v[w] > v || (red_v[w] == v && red_i[w] < ii)) { v = red_v[w]; ii = red_i[w]; }
      chosen[round] = ii;
      mass[ii] = -2.0f;   // below every score, never chosen again
    }
    __syncthreads();
  }
  // ascending block order
  const int np = pow2_at_least(take > 1 ? take : 1);
  for (int i = tid + take; i < np; i += kBlkThreads) chosen[i] = -1;
  __syncthreads();
  bitonic_sort_desc(chosen, np);
  // chosen[0..take) descending -> expand ascending
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < take; ++i) {
      const int blk = chosen[take - 1 - i];
      const int t0 = blk * bs;
      const int t1 = (t0 + bs < n) ? t0 + bs : n;
      cnt[i] = acc;
      acc += t1 - t0;
    }
    cnt[take] = acc;
  }
  __syncthreads();
  for (int i = tid; i < take; i += kBlkThreads) {
    const int blk = chosen[take - 1 - i];
    const int t0 = blk * bs;
    const int t1 = (t0 + bs < n) ? t0 + bs : n;
    for (int t = t0; t < t1; ++t) out[cnt[i] + (t - t0)] = t;
  }
  for (int i = cnt[take] + tid; i < a.S; i += kBlkThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_groupsum(const SelectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(groupsum_kernel, dim3((uint32_t)((uint64_t)a.n_chunks * (uint64_t)a.n_sel)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_refine(const SelectArgs& a, int pass, hipStream_t st) {
  if (pass == 2)
    hipLaunchKernelGGL(refine_kernel<2>, dim3((uint32_t)((uint64_t)a.n_chunks * (uint64_t)a.n_sel)), dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL(refine_kernel<3>, dim3((uint32_t)((uint64_t)a.n_chunks * (uint64_t)a.n_sel)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_collect(const SelectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(collect_kernel, dim3((uint32_t)((uint64_t)a.n_chunks * (uint64_t)a.n_sel)), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const SelectArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(finalize_kernel, dim3(a.n_sel), dim3(kFinThreads), 0, st, a);
  return hipGetLastError();
}

namespace {

// ------------------------------------------------------------------ block comparator on block sums
// The same selection from the scans' block sums in two launches that spread a long row
// over many workgroups:
//   block_mass_kernel: workgroup w of a row takes blocks [kBmBlocks w, kBmBlocks (w+1)),
//                      forms their masses (the sum above, same order) and keeps its
//                      n_blocks best (mass desc, block asc) as candidates;
//   block_pick_kernel: one wave per row: the n_blocks best of the row's candidates (a
//                      merge of the workgroups' sorted lists on a unique key), then the
//                      chosen blocks ascending, expanded to their visible positions.
// The row's best n_blocks are among the union of every workgroup's best n_blocks.
constexpr int kBmThreads = 256;
constexpr int kBmBlocks = kBlockMassBlocks;        // blocks per mass workgroup
constexpr int kPickLists = kMaxBlockMassWgs / 64;   // mass workgroups' lists a lane merges

// Unique order key of a candidate: larger mass first (masses are >= 0, so their bits
// order like the values), then the lower block; 0 marks no candidate.
__device__ __forceinline__ uint64_t block_key(float mass, int32_t blk) {
  return ((uint64_t)__float_as_uint(mass) << 32) | (uint32_t)(0x7FFFFFFF - blk);
}

// Maximum over the 64 lanes (all active): DPP steps inside each 16-lane row, then the
// permlane swaps across the four rows (VALU only, no LDS round trip).  The swap
// results are copied to scalars before use.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, dpp_u<kDppXor1>(x));
  x = max(x, dpp_u<kDppXor2>(x));
  x = max(x, dpp_u<kDppMirror8>(x));
  x = max(x, dpp_u<kDppRor8>(x));
  const auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  const uint32_t a0 = s32[0], a1 = s32[1];
  x = max(a0, a1);
  const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const uint32_t c0 = s16[0], c1 = s16[1];
  return max(c0, c1);
}
// 64-bit maximum as two 32-bit ones: the high words, then the low words of the lanes
// that hold the largest high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  const uint32_t hi = (uint32_t)(x >> 32), lo = (uint32_t)x;
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

template <int H>   // block-sum head slots (blse_heads_of(G))
__global__ __launch_bounds__(kBmThreads) void block_mass_kernel(SelectArgs a) {
  const int64_t sel = blockIdx.x / (uint32_t)a.bm_wgs;
  const int wg = (int)(blockIdx.x % (uint32_t)a.bm_wgs);
  const int tid = threadIdx.x;
  const RowGeom rg = row_geom(a, sel);
  const int n = (int)rg.n;
  const int bs = a.block_size;
  const int nb = (n + bs - 1) / bs;
  const int b0 = wg * kBmBlocks;
  uint64_t* outc = a.bcand + (sel * a.bm_wgs + wg) * a.n_blocks;
  __shared__ float mass[kBmBlocks];
  if (b0 < nb) {
    float Mh[H], iz[H];
    load_head_stats<H>(a, sel, Mh, iz);
    const int gran = a.blse_gran;
    const int sub = bs / gran;
    const int nsub = (n + gran - 1) / gran;
    const float* brow = a.blse + sel * a.blse_stride * H;
    for (int i = tid; i < kBmBlocks; i += kBmThreads) {
      const int blk = b0 + i;
      float acc = -1.0f;   // no block
      if (blk < nb) {
        acc = 0.0f;
        // the first kSubPre sums of the block (8 float4 loads) issued together, then
        // every sum added in order
        constexpr int kSubPre = 32 / H;
        float4 pre[kSubPre][H / 4];
#pragma unroll
        for (int u = 0; u < kSubPre; ++u) {
          const int sb = blk * sub + u;
          if (u < sub && sb < nsub) load_block_sum<H>(brow, sb, pre[u]);
        }
        for (int u = 0; u < sub; ++u) {
          const int sb = blk * sub + u;
          if (sb >= nsub) break;
          float4 l[H / 4];
          if (u < kSubPre) {
#pragma unroll
            for (int j = 0; j < H / 4; ++j) l[j] = pre[u < kSubPre ? u : 0][j];
          } else {
            load_block_sum<H>(brow, sb, l);
          }
          acc = add_block_sum<H>(acc, l, Mh, iz, a.G);
        }
      }
      mass[i] = acc;
    }
  }
  __syncthreads();
  if (tid >= 64) return;
  // wave 0: the workgroup's n_blocks best, 4 blocks a lane
  const int lane = tid;
  uint64_t key[kBmBlocks / 64];
#pragma unroll
  for (int j = 0; j < kBmBlocks / 64; ++j) {
    const int i = lane + 64 * j;
    key[j] = (b0 < nb && mass[i] >= 0.0f) ? block_key(mass[i], b0 + i) : 0ull;
  }
  for (int r = 0; r < a.n_blocks; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int j = 0; j < kBmBlocks / 64; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    if (lane == 0) outc[r] = best;
#pragma unroll
    for (int j = 0; j < kBmBlocks / 64; ++j) key[j] = key[j] == best ? 0ull : key[j];
  }
}

__global__ __launch_bounds__(64) void block_pick_kernel(SelectArgs a) {
  const int64_t sel = blockIdx.x;
  const int lane = threadIdx.x;
  const RowGeom rg = row_geom(a, sel);
  const int n = (int)rg.n;
  const int bs = a.block_size;
  const int nb = (n + bs - 1) / bs;
  const int take = a.n_blocks < nb ? a.n_blocks : nb;
  int32_t* out = a.idx + sel * a.S;
  // Each mass workgroup's list is in descending key order: a k-way merge.  Lane l keeps
  // the heads of lists l, l + 64, ... (at most kPickLists) and each round the wave takes
  // the largest head; keys are unique, so exactly one list advances.
  const int nl = a.bm_wgs, ll = a.n_blocks;
  const uint64_t* cand = a.bcand + sel * (int64_t)nl * ll;
  __shared__ uint64_t lists[kMaxBlockPick];
  // the lists into LDS, 16 loads a lane in flight per batch (one memory latency each
  // batch instead of one per key)
  constexpr int kBatch = 16;
  const int nk = nl * ll;
  for (int base = 0; base < nk; base += 64 * kBatch) {
    uint64_t t[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + 64 * u + lane;
      t[u] = i < nk ? cand[i] : 0ull;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int i = base + 64 * u + lane;
      if (i < nk) lists[i] = t[u];
    }
  }
  __syncthreads();
  int ptr[kPickLists];
  uint64_t head[kPickLists];
#pragma unroll
  for (int u = 0; u < kPickLists; ++u) {
    const int li = lane + 64 * u;
    ptr[u] = 0;
    head[u] = li < nl ? lists[li * ll] : 0ull;
  }
  __shared__ int32_t chosen[64];
  for (int r = 0; r < take; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int u = 0; u < kPickLists; ++u) best = head[u] > best ? head[u] : best;
    best = wave_max_u64(best);
    if (lane == 0) chosen[r] = 0x7FFFFFFF - (int32_t)(uint32_t)best;
#pragma unroll
    for (int u = 0; u < kPickLists; ++u) {
      if (head[u] == best) {   // the list the round took from (best > 0)
        const int li = lane + 64 * u;
        ++ptr[u];
        head[u] = ptr[u] < ll ? lists[li * ll + ptr[u]] : 0ull;
      }
    }
  }
  __syncthreads();
  // ascending block order: lane r < take holds chosen block r and its rank
  int myblk = lane < take ? chosen[lane] : 0x7FFFFFFF;
  int rank = 0;
  for (int i = 0; i < take; ++i) rank += chosen[i] < myblk ? 1 : 0;
  int len = 0;
  if (lane < take) {
    const int t0 = myblk * bs;
    len = ((t0 + bs < n) ? t0 + bs : n) - t0;
  }
  __shared__ int32_t sorted_blk[64], sorted_len[64];
  if (lane < take) {
    sorted_blk[rank] = myblk;
    sorted_len[rank] = len;
  }
  __syncthreads();
  int off = 0;
  for (int i = 0; i < take; ++i) {
    const int blk = sorted_blk[i], ln = sorted_len[i];
    for (int t = lane; t < ln; t += 64) out[off + t] = blk * bs + t;
    off += ln;
  }
  for (int i = off + lane; i < a.S; i += 64) out[i] = -1;
}

}  // namespace

template <int H>
static void launch_block_select_h(const SelectArgs& a, hipStream_t st) {
  if (a.blse != nullptr && a.bcand != nullptr) {
    hipLaunchKernelGGL(block_mass_kernel<H>, dim3((uint32_t)((uint64_t)a.n_sel * a.bm_wgs)), dim3(kBmThreads), 0, st, a);
    hipLaunchKernelGGL(block_pick_kernel, dim3(a.n_sel), dim3(64), 0, st, a);
  } else {
    hipLaunchKernelGGL(block_select_kernel<H>, dim3(a.n_sel), dim3(kBlkThreads), 0, st, a);
  }
}

hipError_t launch_block_select(const SelectArgs& a, hipStream_t st) {
  // per-position scores (logits path) or block sums in blse_heads_of(G) head slots
  const int H = a.blse != nullptr ? blse_heads_of(a.G) : 8;
  if (H == 8)
    launch_block_select_h<8>(a, st);
  else if (H == 16)
    launch_block_select_h<16>(a, st);
  else
    launch_block_select_h<32>(a, st);
  return hipGetLastError();
}

}  // namespace hs2
