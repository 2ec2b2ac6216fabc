// Split-K attention scan for one KV group of G <= 8 query heads, and the split combine.
//
// Dense modes: the Full Attention layer of a Hybrid Block (HySparse2 article,
// section 02 "KV Reuse": the full layer computes its own output over the shared
// cache and, from its attention scores, the positions the sparse layers reuse).
// Besides the online-softmax partials it leaves per-position information for the
// selection, which needs the global softmax statistics and so runs afterwards:
//   records mode: a 2-byte bound record per position (row_record) and a histogram
//     of the record keys of the split's selection candidates, both kept in LDS for
//     the whole split and written when the split is done (writes interleaved with
//     the HBM read stream cost far more than their byte count);
//   logits mode: all 8 head logits per position (32 bytes), for callers that ask
//     for every position's group-summed probability, and the block comparator.
// Sparse mode: a Sparse Attention layer gathering the rows named by the index set
// (section 02: same KV cache, same index set; section 03: window and global
// tokens share one softmax).
//
// Work decomposition (wave64, 4 waves per workgroup):
//   grid = (split, KV head g, b*Lq + j); a workgroup owns `split_len` consecutive
//   positions, each wave a contiguous quarter, walked 4 rows per step.
//   Inside a wave, lane = 16*rg + r: the 16 lanes of row group rg share one row and
//   lane r holds dims [8r, 8r+8) (one 16-byte load of bf16, 8 bytes of fp8), so a
//   step reads 4 whole rows (1 KiB of K and 1 KiB of V in bf16) with coalesced
//   loads.  Loads run kPrefetch steps ahead through a register ring, so a wave keeps
//   several KiB in flight while it computes.
//   QK: each lane forms 8 partial dot products (one per head slot) with
//   v_dot2_f32_bf16; a 4-step DPP butterfly (row_ror:8, row_half_mirror,
//   quad_perm x2 halving, then quad_perm x1 adding) reduce-scatters them so each
//   lane ends with the full logit of head P(r) (lanes r and r^1 share a head).  The
//   reverse DPP all-gather gives every lane the 8 probabilities of its row for the
//   P.V update into its 8 x 8 fp32 accumulators.
//   Each row group runs its own online softmax (no cross-group traffic in the
//   loop); the running max is only raised when a logit exceeds it by 8 (log2
//   units), so rescales are rare.  Streams are merged at the end of the split:
//   shuffles across the 4 row groups, LDS across the 4 waves.
#include "hs2_rowops.h"
#include "hs2_swa.h"

namespace hs2 {
namespace {

constexpr float kSlack = 8.0f;
constexpr int kThreads = 256;
constexpr int kPrefetch = 4;

enum ScanMode { kDenseLogits = 0, kDenseRecords = 1, kSparseGather = 2 };

// LDS of one workgroup: logit or record staging during the scan, reused for the
// cross-wave merge afterwards.
template <int kMode>
struct ScanLds {
  static constexpr int kStage = kMode == kDenseRecords ? kMaxRecordSplit * 2 + kFastBins * 4
                              : kMode == kDenseLogits ? 4 * 4 * 4 * 8 * 4 : 0;
  static constexpr int kMerge = (4 * 8 * kHeadDim + 2 * 4 * 8) * 4;
  static constexpr int kBytes = kStage > kMerge ? kStage : kMerge;
};

// Online-softmax state of one lane plus its 8 x 8 output accumulators.
struct LaneState {
  float o[8][8];
  float m, z;
};

// One row for this lane's row group: logits of the 8 heads (returned: the logit of
// head `hown`, log2 domain), online-softmax update and P.V accumulation.
template <bool kFp8>
__device__ __forceinline__ float process_row(const uint32_t (&qp)[8][4], const RowData& cur,
                                             bool cur_valid, float scale_log2, LaneState& ls) {
  float l = row_logit<kFp8>(qp, cur, scale_log2);
  l = cur_valid ? l : kNegInf;

  const bool up = l > ls.m + kSlack;
  if (wave_any(up)) {
    const float mn = up ? l : ls.m;
    const float alpha = up ? fast_exp2(ls.m - mn) : 1.0f;
    float al[8];
    gather8(alpha, al);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) ls.o[i][e] *= al[i];
    ls.z *= alpha;
    ls.m = mn;
  }
  const float p = cur_valid ? fast_exp2(l - ls.m) : 0.0f;
  ls.z += p;
  float pv[8];
  gather8(kFp8 ? p * cur.vs : p, pv);
  if (kFp8) {
#pragma unroll
    for (int u2 = 0; u2 < 2; ++u2) {
      const f32x2_t lo = fp8x2_to_f32(cur.v[u2], false);
      const f32x2_t hi = fp8x2_to_f32(cur.v[u2], true);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ls.o[i][4 * u2 + 0] = __builtin_fmaf(pv[i], lo.x, ls.o[i][4 * u2 + 0]);
        ls.o[i][4 * u2 + 1] = __builtin_fmaf(pv[i], lo.y, ls.o[i][4 * u2 + 1]);
        ls.o[i][4 * u2 + 2] = __builtin_fmaf(pv[i], hi.x, ls.o[i][4 * u2 + 2]);
        ls.o[i][4 * u2 + 3] = __builtin_fmaf(pv[i], hi.y, ls.o[i][4 * u2 + 3]);
      }
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float v0 = bf16_lo(cur.v[w]);
      const float v1 = bf16_hi(cur.v[w]);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ls.o[i][2 * w] = __builtin_fmaf(pv[i], v0, ls.o[i][2 * w]);
        ls.o[i][2 * w + 1] = __builtin_fmaf(pv[i], v1, ls.o[i][2 * w + 1]);
      }
    }
  }
  return l;
}

// Online-softmax fold of the split partials of one (selection, head) for the 4
// output dims 4dq .. 4dq+3: running maximum, denominator and weighted sum.
__device__ __forceinline__ void fold_splits(const float* base, int64_t split_stride, int n_split, int dq,
                                            float& m_loc, float& z_loc, float4& o) {
  m_loc = kNegInf;
  z_loc = 0.0f;
  o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < n_split; s0 += 4) {
    float ms[4], zs[4];
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = min(s0 + u, n_split - 1);
      const float* ps = base + (int64_t)s * split_stride;
      ms[u] = s0 + u < n_split ? ps[0] : kNegInf;
      zs[u] = ps[1];
      v[u] = *reinterpret_cast<const float4*>(ps + 4 + 4 * dq);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (ms[u] == kNegInf) continue;
      const float mn = fmaxf(m_loc, ms[u]);
      const float fo = fast_exp2(m_loc - mn);
      const float fn = fast_exp2(ms[u] - mn);
      z_loc = z_loc * fo + zs[u] * fn;
      o.x = o.x * fo + v[u].x * fn;
      o.y = o.y * fo + v[u].y * fn;
      o.z = o.z * fo + v[u].z * fn;
      o.w = o.w * fo + v[u].w * fn;
      m_loc = mn;
    }
  }
}

template <int kMode, bool kFp8>
__global__ __launch_bounds__(kThreads, 3) void scan_kernel(ScanArgs a) {
  constexpr bool kSparse = kMode == kSparseGather;
  __shared__ __attribute__((aligned(16))) uint8_t lds_raw[ScanLds<kMode>::kBytes];
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int bj = blockIdx.z;
  const int b = bj / a.Lq;
  const int j = bj - b * a.Lq;
  const int64_t sel = (int64_t)bj * a.Hkv + g;
  const int tid = threadIdx.x;
  // wave-uniform: keeps the wave's ranges in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int rg = lane >> 4;
  const int r = lane & 15;
  const int hown = head_of(r);

  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  int64_t n = ctx - a.Lq + j + 1;
  n = n < 0 ? 0 : n;

  const int64_t p_begin = (int64_t)split * a.split_len;
  const int64_t p_limit = kSparse ? (int64_t)a.S : n;
  int64_t p_end = p_begin + a.split_len;
  p_end = p_end < p_limit ? p_end : p_limit;
  const int wave_len = a.split_len >> 2;
  const int64_t w_begin = p_begin + (int64_t)wave * wave_len;
  int64_t w_end = w_begin + wave_len;
  w_end = w_end < p_end ? w_end : p_end;
  const int nsteps = w_end > w_begin ? (int)((w_end - w_begin + 3) >> 2) : 0;

  uint32_t qp[8][4];
  load_query(a.q + ((int64_t)bj * a.Hq + (int64_t)g * a.G) * kHeadDim, a.G, r, qp);

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const int rowbytes = kFp8 ? 128 : 256;
  const uint8_t* kb = a.k + head_row0 * rowbytes;
  const uint8_t* vb = a.v + head_row0 * rowbytes;
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float* vsb = kFp8 ? a.v_scale + head_row0 : nullptr;

  LaneState ls;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) ls.o[i][e] = 0.0f;
  ls.m = kNegInf;
  ls.z = 0.0f;

  // Rows are < cap < 2^31, so 32-bit row numbers suffice.
  const int32_t wb = (int32_t)w_begin;
  const int32_t we = (int32_t)w_end;
  // sparse mode: entries name visible positions (< n), or local-cache rows (< cap)
  const int32_t n32 = (kSparse && a.slot_rows) ? (int32_t)a.cap : (int32_t)n;

  // The step loops are straight-line per step: every prefetch load is issued (steps
  // past the end re-read a valid row and are masked) and no load or store sits under
  // a branch, so the waitcnt pass keeps kPrefetch steps of loads in flight.
  if (!kSparse) {
    const uint32_t span = we > wb ? (uint32_t)(we - wb) : 0u;
    const uint32_t last = span > 0 ? span - 1 : 0u;
    const int nsteps_pad = (nsteps + kPrefetch - 1) / kPrefetch * kPrefetch;
    float* mylog = reinterpret_cast<float*>(lds_raw) + wave * (kPrefetch * 4 * 8);
    uint16_t* srec = reinterpret_cast<uint16_t*>(lds_raw);
    uint16_t* myrec = srec + wave * wave_len;
    uint32_t* shist = reinterpret_cast<uint32_t*>(lds_raw + kMaxRecordSplit * 2);
    float* lrow = a.logits + sel * a.logit_stride * 8;
    // candidates are the positions before the forced window
    int64_t w0 = n - a.window;
    w0 = w0 < 0 ? 0 : w0;
    uint32_t cand_span = w0 > wb ? (uint32_t)(w0 - wb) : 0u;
    cand_span = cand_span < span ? cand_span : span;
    if (kMode == kDenseRecords) {
      for (int i = tid; i < kFastBins; i += kThreads) shist[i] = 0u;
      if (split == 0) {   // the combine kernel sums every split's histogram into these words
        uint32_t* hm = a.hist_merged + sel * kSelWords + kSelHist1Off;
        for (int i = tid; i < kMergedWords; i += kThreads) hm[i] = 0u;
      }
      __syncthreads();
    }
    RowData buf[kPrefetch];
    if (nsteps > 0) {
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u)
        load_row<kFp8, true>(kb, vb, ksb, vsb, (uint32_t)wb + min((uint32_t)(u * 4 + rg), last), r, buf[u]);
    }
    for (int base = 0; base < nsteps_pad; base += kPrefetch) {
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        // consume ring slot u, then refill it kPrefetch steps ahead (no register copy)
        const uint32_t rel = (uint32_t)((base + u) * 4 + rg);
        const float l = process_row<kFp8>(qp, buf[u], rel < span, a.scale_log2, ls);
        load_row<kFp8, true>(kb, vb, ksb, vsb, (uint32_t)wb + min(rel + 4 * kPrefetch, last), r, buf[u]);
        if (kMode == kDenseLogits) {
          if ((r & 1) == 0) mylog[(u * 4 + rg) * 8 + hown] = l;
        } else {
          const uint16_t rec = row_record(l, r, hown, a.G);
          if (r == 0) {
            myrec[rel] = rec;
            if (rel < cand_span) atomicAdd(&shist[half_order_key(rec) >> kFastShift], 1u);
          }
        }
      }
      if (kMode == kDenseLogits) {
        // one ring turn of logits (16 rows x 8 heads): lane -> row base*4 + lane/4,
        // heads 2*(lane%4) .. +1; 512 contiguous bytes per wave
        const uint32_t rel = (uint32_t)(base * 4 + (lane >> 2));
        const uint64_t row = rel < span ? (uint64_t)(uint32_t)wb + rel : (uint64_t)a.logit_stride - 1;
        const float2 x = *reinterpret_cast<const float2*>(mylog + lane * 2);
        *reinterpret_cast<float2*>(lrow + row * 8 + 2 * (lane & 3)) = x;
      }
    }
    if (kMode == kDenseRecords) {
      // the split's records and key histogram leave once every wave is done
      __syncthreads();
      const int cnt = p_end > p_begin ? (int)(p_end - p_begin) : 0;
      uint16_t* grec = a.records + sel * a.logit_stride + p_begin;   // 512-byte aligned
      for (int i = tid; 2 * i + 1 < cnt; i += kThreads)
        reinterpret_cast<uint32_t*>(grec)[i] = reinterpret_cast<const uint32_t*>(srec)[i];
      if ((cnt & 1) && tid == 0) grec[cnt - 1] = srec[cnt - 1];
      uint32_t* ghist = reinterpret_cast<uint32_t*>(a.hist_part + (sel * a.n_split + split) * kFastBins);
      for (int i = tid; i < kFastBins / 2; i += kThreads)
        ghist[i] = (shist[2 * i] & 0xFFFFu) | (shist[2 * i + 1] << 16);   // counts < 2^16
    }
  } else {
    // Sparse mode: index entries first (one batch per ring of kPrefetch steps), then
    // the gathered rows, so no row load waits behind an index load.
    const int32_t* irow = a.idx + sel * a.S;
    for (int base = 0; base < nsteps; base += kPrefetch) {
      int32_t trow[kPrefetch];
      bool tval[kPrefetch];
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        const int32_t pos = wb + (base + u) * 4 + rg;
        tval[u] = pos < we;
        trow[u] = tval[u] ? irow[pos] : -1;
      }
      RowData buf[kPrefetch];
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        tval[u] = tval[u] && trow[u] >= 0 && trow[u] < n32;
        load_row<kFp8>(kb, vb, ksb, vsb, tval[u] ? (uint32_t)trow[u] : 0u, r, buf[u]);
      }
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u)
        (void)process_row<kFp8>(qp, buf[u], tval[u], a.scale_log2, ls);
    }
  }
  float (&o)[8][8] = ls.o;
  const float m = ls.m;
  const float z = ls.z;

  // ---- merge the 4 row-group streams of this wave (same r = same head)
  float M = m;
  M = fmaxf(M, shfl_xor(M, 16));
  M = fmaxf(M, shfl_xor(M, 32));
  const float f = (m == kNegInf) ? 0.0f : fast_exp2(m - M);
  float zz = z * f;
  zz += shfl_xor(zz, 16);
  zz += shfl_xor(zz, 32);
  float fg[8];
  gather8(f, fg);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[i][e] * fg[i];
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      o[i][e] = x;
    }

  float(*lds_o)[8][kHeadDim] = reinterpret_cast<float(*)[8][kHeadDim]>(lds_raw);
  float(*lds_m)[8] = reinterpret_cast<float(*)[8]>(lds_raw + 4 * 8 * kHeadDim * 4);
  float(*lds_z)[8] = reinterpret_cast<float(*)[8]>(lds_raw + (4 * 8 * kHeadDim + 4 * 8) * 4);
  __syncthreads();   // every wave is done with its staging area
  if (rg == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int head = i ^ hown;
#pragma unroll
      for (int e = 0; e < 8; ++e) lds_o[wave][head][8 * r + e] = o[i][e];
    }
    if ((r & 1) == 0) {
      lds_m[wave][hown] = M;
      lds_z[wave][hown] = zz;
    }
  }
  __syncthreads();

  // ---- merge the 4 waves: thread -> (head, 4 dims)
  {
    const int h = tid >> 5;
    const int d = (tid & 31) * 4;
    float Mw = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mw = fmaxf(Mw, lds_m[w][h]);
    float Z = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = lds_m[w][h];
      const float fw = (mw == kNegInf) ? 0.0f : fast_exp2(mw - Mw);
      Z += fw * lds_z[w][h];
      acc.x += fw * lds_o[w][h][d + 0];
      acc.y += fw * lds_o[w][h][d + 1];
      acc.z += fw * lds_o[w][h][d + 2];
      acc.w += fw * lds_o[w][h][d + 3];
    }
    if (h < a.G) {
      float* pp = a.part + ((sel * a.n_split + split) * a.G + h) * kPartStride;
      *reinterpret_cast<float4*>(pp + 4 + d) = acc;
      if (d == 0) {
        pp[0] = Mw;
        pp[1] = Z;
      }
    }
  }

}

// Splits of selection row `sel` that hold visible positions (all of them for the
// sparse gather, whose splits run over index entries).
__device__ __forceinline__ int live_splits(const CombineArgs& a, int64_t sel) {
  if (a.ctx_len == nullptr) return a.n_split;
  const int64_t bj = sel / a.Hkv;
  const int64_t b = bj / a.Lq;
  const int64_t j = bj - b * a.Lq;
  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  int64_t n = ctx - a.Lq + j + 1;
  n = n < 0 ? 0 : n;
  const int64_t live = (n + a.split_len - 1) / a.split_len;
  return (int)(live < a.n_split ? live : a.n_split);
}

// One workgroup per (selection row, head, 32-dim chunk) merges the split partials
// into the normalised output and records the row's softmax statistics (M, 1/Z),
// which the selection kernels need to turn logits into probabilities.  It merges the
// split partials of one (selection, head) for 32 output dims: every
// thread takes whole splits (one pass of loads), folds them with the online-softmax
// rule, and the block merges the 256 states (wave DPP reductions + LDS).  Workgroups
// with blockIdx.y >= 4 instead sum kHistMergeSplits per-split key histograms
// (records mode) into the selection's merged histogram.
__device__ __forceinline__ void combine_block(const CombineArgs& a, int bx, int by) {
  const int sh = bx;
  const int sel = sh / a.G;
  const int h = sh - sel * a.G;
  const int chunk = by + (a.hist_only ? kHeadDim / 32 : 0);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  if (chunk >= kHeadDim / 32) {
    if (a.hist_part == nullptr) return;
    const int mg = (chunk - kHeadDim / 32) * a.G + h;
    const int s0 = mg * kHistMergeSplits;
    const int live = live_splits(a, sel);
    if (s0 >= live) return;
    __shared__ __attribute__((aligned(16))) uint32_t hred[4][kFastBins];
    // wave w: splits s0 + 4w .. s0 + 4w + 3; lane l: bins [16 l, 16 l + 16)
    const uint16_t* hp = a.hist_part + (int64_t)sel * a.n_split * kFastBins + lane * 16;
    uint4 wv[4][2];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + wave * 4 + u;
      if (s < live) {
        wv[u][0] = *reinterpret_cast<const uint4*>(hp + (int64_t)s * kFastBins);
        wv[u][1] = *reinterpret_cast<const uint4*>(hp + (int64_t)s * kFastBins + 8);
      } else {
        wv[u][0] = make_uint4(0u, 0u, 0u, 0u);
        wv[u][1] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    uint32_t acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0u;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t w4[4] = {wv[u][q].x, wv[u][q].y, wv[u][q].z, wv[u][q].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          acc[q * 8 + 2 * c] += w4[c] & 0xFFFFu;
          acc[q * 8 + 2 * c + 1] += w4[c] >> 16;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<uint4*>(&hred[wave][lane * 16 + i]) = make_uint4(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    __syncthreads();
    uint32_t* ho = a.hist_out + (int64_t)sel * kSelWords + kSelHist1Off;
    for (int bin = tid; bin < kFastBins; bin += 256) {
      const uint32_t t = hred[0][bin] + hred[1][bin] + hred[2][bin] + hred[3][bin];
      if (t != 0u) atomicAdd(ho + bin, t);
    }
    return;
  }
  const int64_t split_stride = (int64_t)a.G * kPartStride;
  const float* base = a.part + ((int64_t)sel * a.n_split * a.G + h) * kPartStride;

  // per-thread online merge of its splits
  float m_loc = kNegInf, z_loc = 0.0f;
  float o[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = 0.0f;
  const int live = live_splits(a, sel);
  for (int s = tid; s < live; s += 256) {
    const float* ps = base + (int64_t)s * split_stride;
    const float ms = ps[0];
    const float zs = ps[1];
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const float4*>(ps + 4 + chunk * 32 + 4 * i);
    if (ms == kNegInf) continue;   // split without visible rows: z = 0, o = 0
    const float mn = fmaxf(m_loc, ms);
    const float fo = fast_exp2(m_loc - mn);   // 0 while m_loc = -inf
    const float fn = fast_exp2(ms - mn);
    z_loc = z_loc * fo + zs * fn;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      o[4 * i + 0] = o[4 * i + 0] * fo + v[i].x * fn;
      o[4 * i + 1] = o[4 * i + 1] * fo + v[i].y * fn;
      o[4 * i + 2] = o[4 * i + 2] * fo + v[i].z * fn;
      o[4 * i + 3] = o[4 * i + 3] * fo + v[i].w * fn;
    }
    m_loc = mn;
  }

  __shared__ float wmax[4];
  __shared__ float red[16][33];
  const float wm = wave_max(m_loc);
  if (lane == 0) wmax[wave] = wm;
  __syncthreads();
  const float M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float f = m_loc == kNegInf ? 0.0f : fast_exp2(m_loc - M);
  // sums over each row of 16 lanes, then over the 16 rows of the block
  const float zr = rowgroup_sum16(z_loc * f);
#pragma unroll
  for (int i = 0; i < 32; ++i) o[i] = rowgroup_sum16(o[i] * f);
  if ((lane & 15) == 0) {
    const int row = wave * 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 32; ++i) red[row][i] = o[i];
    red[row][32] = zr;
  }
  __syncthreads();
  if (tid < 32) {
    float t = 0.0f, Z = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      t += red[r][tid];
      Z += red[r][32];
    }
    const int bj = sel / a.Hkv;
    const int g = sel - bj * a.Hkv;
    a.out[((int64_t)bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim + chunk * 32 + tid] =
        Z > 0.0f ? t / Z : 0.0f;
    if (a.mz != nullptr && chunk == 0 && tid == 0) {
      a.mz[((int64_t)sel * kMaxHeads + h) * 2 + 0] = M;
      a.mz[((int64_t)sel * kMaxHeads + h) * 2 + 1] = Z > 0.0f ? 1.0f / Z : 0.0f;
    }
  }
  if (a.sel_zero != nullptr && h == 0 && chunk == 0) {
    uint32_t* zp = a.sel_zero + (int64_t)sel * a.sel_zero_words;
    for (int w = tid; w < a.sel_zero_words; w += 256) zp[w] = 0u;
  }
}

// Few splits (sparse layers), or many rows (query chunks: a row folds only its live
// splits, ~30 on average there): one thread per (row, head, 4 dims) folds every split
// itself, four splits of loads in flight; no cross-thread reduction.
constexpr int kSmallSplits = 32;
constexpr int64_t kSmallPairs = 8192;   // (row, head) pairs from which rows give the parallelism
__device__ __forceinline__ void combine_small_block(const CombineArgs& a, int64_t bx) {
  const int tid = threadIdx.x;
  const int64_t pair = bx * 8 + (tid >> 5);   // sel * G + h
  const int dq = tid & 31;
  if (pair >= (int64_t)a.n_sel * a.G) return;
  const int sel = (int)(pair / a.G);
  const int h = (int)(pair - (int64_t)sel * a.G);
  float m_loc, z_loc;
  float4 o;
  fold_splits(a.part + ((int64_t)sel * a.n_split * a.G + h) * kPartStride, (int64_t)a.G * kPartStride,
              live_splits(a, sel), dq, m_loc, z_loc, o);
  const float iz = z_loc > 0.0f ? 1.0f / z_loc : 0.0f;
  const int bj = sel / a.Hkv;
  const int g = sel - bj * a.Hkv;
  *reinterpret_cast<float4*>(a.out + ((int64_t)bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim + 4 * dq) =
      make_float4(o.x * iz, o.y * iz, o.z * iz, o.w * iz);
  if (a.mz != nullptr && dq == 0) {
    a.mz[((int64_t)sel * kMaxHeads + h) * 2 + 0] = m_loc;
    a.mz[((int64_t)sel * kMaxHeads + h) * 2 + 1] = iz;
  }
  if (a.sel_zero != nullptr && h == 0) {
    uint32_t* zp = a.sel_zero + (int64_t)sel * a.sel_zero_words;
    for (int w = dq; w < a.sel_zero_words; w += 32) zp[w] = 0u;
  }
}

__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) { combine_block(a, blockIdx.x, blockIdx.y); }
__global__ __launch_bounds__(256) void combine_small_kernel(CombineArgs a) { combine_small_block(a, blockIdx.x); }
// Both folds of a many-row call in one launch: blocks [0, n_small) fold the output
// partials (combine_small_block), the rest merge the key histograms (combine_block with
// h.hist_only), hist_x of them per histogram group; the two halves run side by side.
__global__ __launch_bounds__(256) void combine_pair_kernel(CombineArgs a, CombineArgs h, uint32_t n_small,
                                                           uint32_t hist_x) {
  const uint32_t b = blockIdx.x;
  if (b < n_small) {
    combine_small_block(a, b);
  } else {
    const uint32_t k = b - n_small;
    combine_block(h, (int)(k % hist_x), (int)(k / hist_x));
  }
}

// ---- Sparse Attention layer at decode sizes (HySparse2 article, section 02 "KV
// Reuse": each sparse layer attends with its own queries over the rows the full
// layer's index set names; section 03: window and global rows share one softmax).
// One workgroup of 16 waves per (query token, query head, 128/kDs output dims)
// gathers every index entry of its KV head and writes its dims of the normalised
// output: no partials, no combine launch.  The kDs workgroups of a head compute the
// same logits and softmax (same operands, same order) and differ only in the V dims
// they read, which cuts the bytes one workgroup pulls (K 256 B + V 256/kDs B per
// bf16 row).  Its 64 row groups of 16 lanes take entries gi, gi + 64, ... (lane r
// holds dims [8r, 8r+8) of the key and of the query, and 8/kDs of its workgroup's V
// dims); each group runs its own online softmax and the groups merge in a fixed order
// (the 4 of a wave by lane exchanges, then the waves through LDS), so the output is
// bitwise reproducible.  blockIdx.x = row + rows *
// (head + G * dim part) (workgroups go to the XCDs round-robin) keeps the workgroups
// of one (token, KV head) on 8 / gcd(rows, 8) XCDs, one from 8 rows on, whose L2 then
// serves the repeated row reads.  A workgroup reads about S * (256 + 256/kDs) bytes
// itself, at ~80 GB/s per workgroup, so this form suits calls with few rows: the host
// takes it for fewer than 64 rows, with the most dim parts that keep every workgroup
// resident at once (one per CU).
constexpr int kHeadThreads = 1024;
constexpr int kHeadGroups = kHeadThreads / 16;
constexpr int kHeadWaves = kHeadThreads / 64;
// rows per group in flight: 2 (1,024 threads) measured fastest; 4 or 8 rows, 512 or 256
// threads, or a second batch in flight were 2-50% slower on the million-token decode
constexpr int kHeadBatch = 2;

// N bytes at p (N = 2, 4, 8, 16; p aligned to N) as little-endian words
template <int N>
__device__ __forceinline__ void load_bytes(const uint8_t* p, uint32_t (&w)[(N + 3) / 4]) {
  if constexpr (N == 16) {
    const uint4 x = *reinterpret_cast<const uint4*>(p);
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (N == 8) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    w[0] = x.x; w[1] = x.y;
  } else if constexpr (N == 4) {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  }
}

template <bool kFp8, int kDs, bool kSwa>
__global__ __launch_bounds__(kHeadThreads) void sparse_head_kernel(ScanArgs a, int64_t n_sel, float* __restrict__ out,
                                                                   SwaBranch sw) {
  constexpr int kDw = kHeadDim / kDs;        // output dims of the workgroup
  constexpr int kDl = kDw / 16;              // V dims of a lane
  constexpr int kVB = kDl * (kFp8 ? 1 : 2);  // V bytes of a lane per row
  constexpr int kVWords = (kVB + 3) / 4;
  __shared__ int32_t sidx[kMaxHeadPathS];
  __shared__ float smz[kHeadWaves][2];
  __shared__ __attribute__((aligned(16))) float so[kHeadWaves][kDw];

  const int64_t wg = blockIdx.x;
  const int64_t sel = wg % n_sel;
  const int64_t hd = wg / n_sel;
  const int h = (int)(hd % a.G);   // head of the KV group
  const int ds = (int)(hd / a.G);  // dim part, < kDs
  const int64_t bj = sel / a.Hkv;
  const int g = (int)(sel - bj * a.Hkv);
  const int64_t b = bj / a.Lq;
  const int j = (int)(bj - b * a.Lq);
  const int tid = threadIdx.x;
  const int r = tid & 15;
  const int gi = tid >> 4;

  int64_t ctx = a.ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > a.ctx_max ? a.ctx_max : ctx);
  int64_t n = ctx - a.Lq + j + 1;
  n = n < 0 ? 0 : n;
  // entries name visible positions (< n), or local-cache rows (< cap)
  const int64_t lim = a.slot_rows ? a.cap : n;
  const int32_t* irow = a.idx + sel * a.S;
  for (int e = tid; e < a.S; e += kHeadThreads) {
    const int32_t t = irow[e];
    sidx[e] = (t >= 0 && t < lim) ? t : -1;
  }
  const int64_t qrow = (bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim;
  const uint4 qv = *reinterpret_cast<const uint4*>(a.q + qrow + 8 * r);
  const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w};
  const int rowbytes = kFp8 ? 128 : 256;
  const int wave = tid >> 6;
  __syncthreads();

  // One attention over the rows sidx[0, S) names in a cache of `cap` rows per (sequence,
  // KV head); returns, for threads tid < kDw, output dim kDw * ds + tid normalised.
  auto attend = [&](const uint8_t* kc, const uint8_t* vc, const float* ksc, const float* vsc, int64_t cap,
                    int S) -> float {
  const int64_t head_row0 = (b * a.Hkv + g) * cap;
  const uint8_t* kb = kc + head_row0 * rowbytes;
  const uint8_t* vb = vc + head_row0 * rowbytes + (kDw * ds + kDl * r) * (kFp8 ? 1 : 2);
  const float* ksb = kFp8 ? ksc + head_row0 : nullptr;
  const float* vsb = kFp8 ? vsc + head_row0 : nullptr;

  struct Row {
    uint32_t k[kFp8 ? 2 : 4];
    uint32_t v[kVWords];
    float ks, vs;
  };
  float m = kNegInf, z = 0.0f;
  float o[kDl];
#pragma unroll
  for (int i = 0; i < kDl; ++i) o[i] = 0.0f;
  auto load_batch = [&](int e0, int32_t (&t)[kHeadBatch], Row (&d)[kHeadBatch]) {
#pragma unroll
    for (int u = 0; u < kHeadBatch; ++u) {
      const int e = e0 + u * kHeadGroups;
      t[u] = e < S ? sidx[e] : -1;
      const uint32_t row = t[u] >= 0 ? (uint32_t)t[u] : 0u;
      load_bytes<kFp8 ? 8 : 16>(kb + (uint64_t)row * rowbytes + (kFp8 ? 8 : 16) * r, d[u].k);
      load_bytes<kVB>(vb + (uint64_t)row * rowbytes, d[u].v);
      if constexpr (kFp8) {
        d[u].ks = ksb[row];
        d[u].vs = vsb[row];
      }
    }
  };
  auto use_batch = [&](const int32_t (&t)[kHeadBatch], const Row (&d)[kHeadBatch]) {
#pragma unroll
    for (int u = 0; u < kHeadBatch; ++u) {
      if (t[u] < 0) continue;   // the 16 lanes of a group agree
      uint32_t kw[4];
      if constexpr (kFp8) {
        kw[0] = fp8x2_to_bf16x2(d[u].k[0], false);
        kw[1] = fp8x2_to_bf16x2(d[u].k[0], true);
        kw[2] = fp8x2_to_bf16x2(d[u].k[1], false);
        kw[3] = fp8x2_to_bf16x2(d[u].k[1], true);
      } else {
        kw[0] = d[u].k[0]; kw[1] = d[u].k[1]; kw[2] = d[u].k[2]; kw[3] = d[u].k[3];
      }
      float s = dot2_bf16(qw[0], kw[0], 0.0f);
      s = dot2_bf16(qw[1], kw[1], s);
      s = dot2_bf16(qw[2], kw[2], s);
      s = dot2_bf16(qw[3], kw[3], s);
      s = rowgroup_sum16(s);
      float l = s * a.scale_log2;
      if constexpr (kFp8) l *= d[u].ks;
      if (l > m + kSlack) {   // raise the running maximum (rare)
        const float alpha = fast_exp2(m - l);
#pragma unroll
        for (int i = 0; i < kDl; ++i) o[i] *= alpha;
        z *= alpha;
        m = l;
      }
      const float p = fast_exp2(l - m);
      z += p;
      float pv = p;
      if constexpr (kFp8) pv *= d[u].vs;
      float vf[kDl];
      if constexpr (kFp8) {
#pragma unroll
        for (int c = 0; c < kDl / 2; ++c) {
          const f32x2_t x = fp8x2_to_f32(d[u].v[c >> 1], (c & 1) != 0);
          vf[2 * c] = x[0];
          vf[2 * c + 1] = x[1];
        }
      } else {
#pragma unroll
        for (int c = 0; c < kDl / 2; ++c) {
          vf[2 * c] = bf16_lo(d[u].v[c]);
          vf[2 * c + 1] = bf16_hi(d[u].v[c]);
        }
      }
#pragma unroll
      for (int i = 0; i < kDl; ++i) o[i] = __builtin_fmaf(pv, vf[i], o[i]);
    }
  };
  for (int e0 = gi; e0 < S; e0 += kHeadGroups * kHeadBatch) {
    int32_t t[kHeadBatch];
    Row d[kHeadBatch];
    load_batch(e0, t, d);
    use_batch(t, d);
  }

  // merge (fixed order): the 4 groups of a wave (lanes r, r+16, r+32, r+48 hold the
  // same dims) by lane exchanges, then the 16 waves through LDS
  float M = fmaxf(m, shfl_xor(m, 16));
  M = fmaxf(M, shfl_xor(M, 32));
  const float f = m == kNegInf ? 0.0f : fast_exp2(m - M);
  float zz = z * f;
  zz += shfl_xor(zz, 16);
  zz += shfl_xor(zz, 32);
#pragma unroll
  for (int i = 0; i < kDl; ++i) {
    float x = o[i] * f;
    x += shfl_xor(x, 16);
    x += shfl_xor(x, 32);
    o[i] = x;
  }
  if ((tid & 63) < 16) {
    if (r == 0) {
      smz[wave][0] = M;
      smz[wave][1] = zz;
    }
#pragma unroll
    for (int i = 0; i < kDl; ++i) so[wave][kDl * r + i] = o[i];
  }
  __syncthreads();
  float res = 0.0f;
  if (tid < kDw) {
    float Mw = kNegInf;
    for (int q = 0; q < kHeadWaves; ++q) Mw = fmaxf(Mw, smz[q][0]);
    float Z = 0.0f, acc = 0.0f;
    if (Mw != kNegInf) {
      for (int q = 0; q < kHeadWaves; ++q) {
        const float mq = smz[q][0];
        const float fq = mq == kNegInf ? 0.0f : fast_exp2(mq - Mw);
        Z = __builtin_fmaf(fq, smz[q][1], Z);
        acc = __builtin_fmaf(fq, so[q][tid], acc);
      }
    }
    res = Z > 0.0f ? acc / Z : 0.0f;
  }
  return res;
  };

  float res = attend(a.k, a.v, a.k_scale, a.v_scale, a.cap, a.S);
  if constexpr (kSwa) {
    // the first-generation comparator's sliding-window branch: the sw.W most recent
    // visible positions, rows p % sw.R of the layer's own ring, its own softmax; the
    // two normalised outputs are added
    __syncthreads();   // every wave is done with sidx, smz and so
    const int64_t cnt = n < sw.W ? n : sw.W;
    for (int e = tid; e < sw.W; e += kHeadThreads) sidx[e] = e < cnt ? (int32_t)((n - cnt + e) % sw.R) : -1;
    __syncthreads();
    const float loc = attend(sw.k, sw.v, sw.k_scale, sw.v_scale, sw.R, sw.W);
    res = res + loc;
  }
  if (tid < kDw) out[qrow + kDw * ds + tid] = res;
}

template <bool kFp8, bool kSwa>
void launch_head_ds(const ScanArgs& a, int64_t n_sel, float* out, int ds, unsigned wgs, const SwaBranch& sw,
                    hipStream_t st, const KernelEvents* ev) {
  if (ds == 4)
    launch_on(ev, sparse_head_kernel<kFp8, 4, kSwa>, dim3(wgs), dim3(kHeadThreads), 0, st, a, n_sel, out, sw);
  else if (ds == 2)
    launch_on(ev, sparse_head_kernel<kFp8, 2, kSwa>, dim3(wgs), dim3(kHeadThreads), 0, st, a, n_sel, out, sw);
  else
    launch_on(ev, sparse_head_kernel<kFp8, 1, kSwa>, dim3(wgs), dim3(kHeadThreads), 0, st, a, n_sel, out, sw);
}

}  // namespace

static hipError_t launch_head(const ScanArgs& a, int64_t n_sel, float* out, bool fp8, const SwaBranch* sw,
                              hipStream_t st, const KernelEvents* ev) {
  if (a.S > kMaxHeadPathS || n_sel < 1 || a.G < 1 || a.G > kMaxHeads) return hipErrorInvalidValue;
  if (sw != nullptr && (sw->W < 1 || sw->W > kMaxHeadPathS || sw->R < sw->W)) return hipErrorInvalidValue;
  // dim parts: as many as keep every workgroup resident at once (one per CU)
  constexpr int64_t kResident = 256;
  const int64_t heads = n_sel * a.G;
  const int ds = heads * 4 <= kResident ? 4 : heads * 2 <= kResident ? 2 : 1;
  const int64_t wgs = heads * ds;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  const SwaBranch none{};
  if (sw != nullptr) {
    if (fp8)
      launch_head_ds<true, true>(a, n_sel, out, ds, (unsigned)wgs, *sw, st, ev);
    else
      launch_head_ds<false, true>(a, n_sel, out, ds, (unsigned)wgs, *sw, st, ev);
  } else if (fp8) {
    launch_head_ds<true, false>(a, n_sel, out, ds, (unsigned)wgs, none, st, ev);
  } else {
    launch_head_ds<false, false>(a, n_sel, out, ds, (unsigned)wgs, none, st, ev);
  }
  return hipGetLastError();
}

hipError_t launch_sparse_head(const ScanArgs& a, int64_t n_sel, float* out, bool fp8, hipStream_t st,
                              const KernelEvents* ev) {
  return launch_head(a, n_sel, out, fp8, nullptr, st, ev);
}

hipError_t launch_sparse_head_swa(const ScanArgs& a, int64_t n_sel, float* out, bool fp8, const SwaBranch& sw,
                                  hipStream_t st) {
  return launch_head(a, n_sel, out, fp8, &sw, st, nullptr);
}

hipError_t launch_scan_dense(const ScanArgs& a, bool fp8, bool records, int B, hipStream_t st,
                             const KernelEvents* ev) {
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (records) {
    if (fp8)
      launch_on(ev, scan_kernel<kDenseRecords, true>, grid, dim3(kThreads), 0, st, a);
    else
      launch_on(ev, scan_kernel<kDenseRecords, false>, grid, dim3(kThreads), 0, st, a);
  } else {
    if (fp8)
      launch_on(ev, scan_kernel<kDenseLogits, true>, grid, dim3(kThreads), 0, st, a);
    else
      launch_on(ev, scan_kernel<kDenseLogits, false>, grid, dim3(kThreads), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_scan_sparse(const ScanArgs& a, bool fp8, int B, hipStream_t st, const KernelEvents* ev) {
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (fp8)
    launch_on(ev, scan_kernel<kSparseGather, true>, grid, dim3(kThreads), 0, st, a);
  else
    launch_on(ev, scan_kernel<kSparseGather, false>, grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int n_groups = (a.n_split + kHistMergeSplits - 1) / kHistMergeSplits;
  const int extra = a.hist_part != nullptr ? (n_groups + a.G - 1) / a.G : 0;
  if (a.n_split <= kSmallSplits || (int64_t)a.n_sel * a.G >= kSmallPairs) {
    const int64_t pairs = (int64_t)a.n_sel * a.G;
    const int64_t n_small = (pairs + 7) / 8;
    if (extra > 0) {   // and the histogram merge, in the same launch
      CombineArgs h = a;
      h.hist_only = 1;
      const int64_t hist_x = (int64_t)a.n_sel * a.G;
      const int64_t total = n_small + hist_x * extra;
      if (total > 0x7FFFFFFF) return hipErrorInvalidValue;
      hipLaunchKernelGGL(combine_pair_kernel, dim3((unsigned)total), dim3(256), 0, st, a, h, (uint32_t)n_small,
                         (uint32_t)hist_x);
    } else {
      hipLaunchKernelGGL(combine_small_kernel, dim3((unsigned)n_small), dim3(256), 0, st, a);
    }
    return hipGetLastError();
  }
  dim3 grid(a.n_sel * a.G, kHeadDim / 32 + extra);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs2
