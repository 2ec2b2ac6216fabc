// Split-K attention scan for one KV group of G <= 8 query heads, and the split combine.
//
// Dense mode: the Full Attention layer of a Hybrid Block (HySparse2 article,
// section 02 "KV Reuse": the full layer computes its own output over the shared
// cache and, from its attention scores, the positions the sparse layers reuse).
// Besides the online-softmax partials it stores every position's logits so the
// selection kernels can form normalised probabilities once the global softmax
// statistics are known.
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
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr float kSlack = 8.0f;
constexpr int kThreads = 256;
constexpr int kPrefetch = 4;

// LDS of one workgroup: per-wave logit staging during the scan, reused for the
// cross-wave merge afterwards.
#ifndef HS2_LOGIT_STORE
#define HS2_LOGIT_STORE(ptr, val) (*reinterpret_cast<float2*>(ptr) = (val))
#endif

union ScanLds {
  float logit[4][kPrefetch * 4 * 8];
  struct {
    float o[4][8][kHeadDim];
    float m[4][8];
    float z[4][8];
  } merge;
};

// Head whose logit lane r (0..15 inside its row group) holds after the butterfly;
// register slot i of lane r holds head i ^ head_of(r).  head_of is the linear map
// with head_of(8) = 4, head_of(7) = 2, head_of(2) = 1, head_of(1) = 0, which makes
// every butterfly partner hold the matching head in the matching slot.
__device__ __forceinline__ int head_of(int r) {
  const int a = (r >> 3) & 1;
  const int r1 = r ^ (a * 8);
  const int b = (r1 >> 2) & 1;
  const int r2 = r1 ^ (b * 7);
  const int c = (r2 >> 1) & 1;
  return (4 * a) ^ (2 * b) ^ c;
}

// All-gather inside the 16-lane row group: out[i] = probability of head i ^ head_of(r).
__device__ __forceinline__ void gather8(float x, float (&out)[8]) {
  out[0] = x;
  out[1] = dpp<kDppXor2>(out[0]);
  out[2] = dpp<kDppMirror8>(out[0]);
  out[3] = dpp<kDppMirror8>(out[1]);
  out[4] = dpp<kDppRor8>(out[0]);
  out[5] = dpp<kDppRor8>(out[1]);
  out[6] = dpp<kDppRor8>(out[2]);
  out[7] = dpp<kDppRor8>(out[3]);
}

struct RowData {
  uint32_t k[4];   // bf16: 4 pairs of the lane's 8 dims; fp8: k[0..1] hold 8 codes
  uint32_t v[4];
  float ks, vs;    // fp8 per-token scales
};

template <bool kFp8>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb,
                                         const float* __restrict__ ksb, const float* __restrict__ vsb,
                                         uint32_t t, int r, RowData& d) {
  if (kFp8) {
    const uint2 kw = *reinterpret_cast<const uint2*>(kb + (uint64_t)t * 128 + 8 * r);
    const uint2 vw = *reinterpret_cast<const uint2*>(vb + (uint64_t)t * 128 + 8 * r);
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = 0u; d.k[3] = 0u;
    d.v[0] = vw.x; d.v[1] = vw.y; d.v[2] = 0u; d.v[3] = 0u;
    d.ks = ksb[t];
    d.vs = vsb[t];
  } else {
    const uint4 kw = *reinterpret_cast<const uint4*>(kb + (uint64_t)t * 256 + 16 * r);
    const uint4 vw = *reinterpret_cast<const uint4*>(vb + (uint64_t)t * 256 + 16 * r);
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = kw.z; d.k[3] = kw.w;
    d.v[0] = vw.x; d.v[1] = vw.y; d.v[2] = vw.z; d.v[3] = vw.w;
    d.ks = 1.0f;
    d.vs = 1.0f;
  }
}

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
  uint32_t kw[4];
  if (kFp8) {
    kw[0] = fp8x2_to_bf16x2(cur.k[0], false);
    kw[1] = fp8x2_to_bf16x2(cur.k[0], true);
    kw[2] = fp8x2_to_bf16x2(cur.k[1], false);
    kw[3] = fp8x2_to_bf16x2(cur.k[1], true);
  } else {
    kw[0] = cur.k[0]; kw[1] = cur.k[1]; kw[2] = cur.k[2]; kw[3] = cur.k[3];
  }
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float s = dot2_bf16(qp[i][0], kw[0], 0.0f);
    s = dot2_bf16(qp[i][1], kw[1], s);
    s = dot2_bf16(qp[i][2], kw[2], s);
    acc[i] = dot2_bf16(qp[i][3], kw[3], s);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] += dpp<kDppRor8>(acc[i + 4]);
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i] += dpp<kDppMirror8>(acc[i + 2]);
  acc[0] += dpp<kDppXor2>(acc[1]);
  acc[0] += dpp<kDppXor1>(acc[0]);

  float l = acc[0] * scale_log2;
  if (kFp8) l *= cur.ks;
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

template <bool kSparse, bool kFp8>
__global__ __launch_bounds__(kThreads, 3) void scan_kernel(ScanArgs a) {
  __shared__ ScanLds lds_u;
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int bj = blockIdx.z;
  const int b = bj / a.Lq;
  const int j = bj - b * a.Lq;
  const int64_t sel = (int64_t)bj * a.Hkv + g;
  const int tid = threadIdx.x;
  // wave-uniform: keeps the wave's ranges and buffer descriptors in SGPRs
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

  // Query slice: slot i holds dims [8r, 8r+8) of head i ^ hown (zero beyond the group).
  uint32_t qp[8][4];
  const uint16_t* qrow = a.q + ((int64_t)bj * a.Hq + (int64_t)g * a.G) * kHeadDim;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int head = i ^ hown;
    if (head < a.G) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + head * kHeadDim + 8 * r);
      qp[i][0] = x.x; qp[i][1] = x.y; qp[i][2] = x.z; qp[i][3] = x.w;
    } else {
      qp[i][0] = qp[i][1] = qp[i][2] = qp[i][3] = 0u;
    }
  }

  const int64_t head_row0 = (int64_t)(b * a.Hkv + g) * a.cap;
  const int rowbytes = kFp8 ? 128 : 256;
  const uint8_t* kb = a.k + head_row0 * rowbytes;
  const uint8_t* vb = a.v + head_row0 * rowbytes;
  const float* ksb = kFp8 ? a.k_scale + head_row0 : nullptr;
  const float* vsb = kFp8 ? a.v_scale + head_row0 : nullptr;
  const int32_t* irow = kSparse ? a.idx + sel * a.S : nullptr;
  float* lrow = kSparse ? nullptr : a.logits + sel * a.logit_stride * 8;

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
  const int32_t n32 = (int32_t)n;

  // Both loops below are straight-line per step: every prefetch load is issued
  // (steps past the end read a harmless row and are masked), and there are no
  // loads or stores under branches, so the waitcnt pass keeps kPrefetch steps of
  // loads in flight.
  if (!kSparse) {
    // Logits of one ring turn (kPrefetch steps x 4 rows x 8 heads) are staged in LDS
    // and written with one 8-byte store per lane: 512 contiguous bytes per wave.
    float* mylog = lds_u.logit[wave];
    const uint32_t span = we > wb ? (uint32_t)(we - wb) : 0u;
    // rows past the wave's range re-read its last row (in bounds) and are masked
    const uint32_t last = span > 0 ? span - 1 : 0u;
    const int nsteps_pad = (nsteps + kPrefetch - 1) / kPrefetch * kPrefetch;
    RowData buf[kPrefetch];
    if (nsteps > 0) {
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u)
        load_row<kFp8>(kb, vb, ksb, vsb, (uint32_t)wb + min((uint32_t)(u * 4 + rg), last), r, buf[u]);
    }
    for (int base = 0; base < nsteps_pad; base += kPrefetch) {
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        // consume ring slot u, then refill it kPrefetch steps ahead (no register copy)
        const uint32_t rel = (uint32_t)((base + u) * 4 + rg);
        const float l = process_row<kFp8>(qp, buf[u], rel < span, a.scale_log2, ls);
        load_row<kFp8>(kb, vb, ksb, vsb, (uint32_t)wb + min(rel + 4 * kPrefetch, last), r, buf[u]);
        if ((r & 1) == 0) mylog[(u * 4 + rg) * 8 + hown] = l;
      }
      // lane -> row base*4 + lane/4, heads 2*(lane%4) .. +1
      const uint32_t rel = (uint32_t)(base * 4 + (lane >> 2));
      const uint64_t row = rel < span ? (uint64_t)(uint32_t)wb + rel : (uint64_t)a.logit_stride - 1;
      const float2 x = *reinterpret_cast<const float2*>(mylog + lane * 2);
      HS2_LOGIT_STORE(lrow + row * 8 + 2 * (lane & 3), x);
    }
  } else {
    // Sparse mode: index entries first (one batch per ring of kPrefetch steps), then
    // the gathered rows, so no row load waits behind an index load.
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

  float (&lds_o)[4][8][kHeadDim] = lds_u.merge.o;
  float (&lds_m)[4][8] = lds_u.merge.m;
  float (&lds_z)[4][8] = lds_u.merge.z;
  __syncthreads();   // every wave is done with its logit staging area
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

// One workgroup per (selection row, head, 32-dim chunk): merges the split partials
// into the normalised output and records the row's softmax statistics (M, 1/Z),
// which the selection kernels need to turn logits into probabilities.
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  const int sh = blockIdx.x;
  const int sel = sh / a.G;
  const int h = sh - sel * a.G;
  const int chunk = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t split_stride = (int64_t)a.G * kPartStride;
  const float* base = a.part + ((int64_t)sel * a.n_split * a.G + h) * kPartStride;

  __shared__ float w_lds[2048];
  __shared__ float red[256];
  __shared__ float acc_lds[8][32];

  float mx = kNegInf;
  for (int s = tid; s < a.n_split; s += 256) mx = fmaxf(mx, base[s * split_stride]);
  red[tid] = mx;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] = fmaxf(red[tid], red[tid + o]);
    __syncthreads();
  }
  const float M = red[0];
  __syncthreads();

  float zs = 0.0f;
  for (int s = tid; s < a.n_split; s += 256) {
    const float ms = base[s * split_stride];
    const float w = (ms == kNegInf) ? 0.0f : fast_exp2(ms - M);
    w_lds[s] = w;
    zs += w * base[s * split_stride + 1];
  }
  red[tid] = zs;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) red[tid] += red[tid + o];
    __syncthreads();
  }
  const float Z = red[0];

  const int dl = tid & 31;
  const int sg = tid >> 5;
  const int d = chunk * 32 + dl;
  float acc = 0.0f;
  for (int s = sg; s < a.n_split; s += 8) acc += w_lds[s] * base[s * split_stride + 4 + d];
  acc_lds[sg][dl] = acc;
  __syncthreads();
  if (tid < 32) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) t += acc_lds[i][tid];
    const int bj = sel / a.Hkv;
    const int g = sel - bj * a.Hkv;
    a.out[((int64_t)bj * a.Hq + (int64_t)g * a.G + h) * kHeadDim + chunk * 32 + tid] =
        Z > 0.0f ? t / Z : 0.0f;
  }
  if (a.mz != nullptr && chunk == 0 && tid == 0) {
    a.mz[((int64_t)sel * 8 + h) * 2 + 0] = M;
    a.mz[((int64_t)sel * 8 + h) * 2 + 1] = Z > 0.0f ? 1.0f / Z : 0.0f;
  }
  if (a.sel_zero != nullptr && h == 0 && chunk == 0) {
    uint32_t* zp = a.sel_zero + (int64_t)sel * a.sel_zero_words;
    for (int w = tid; w < a.sel_zero_words; w += 256) zp[w] = 0u;
  }
}

}  // namespace

hipError_t launch_scan_dense(const ScanArgs& a, bool fp8, int B, hipStream_t st) {
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (fp8)
    hipLaunchKernelGGL((scan_kernel<false, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((scan_kernel<false, false>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scan_sparse(const ScanArgs& a, bool fp8, int B, hipStream_t st) {
  dim3 grid(a.n_split, a.Hkv, B * a.Lq);
  if (fp8)
    hipLaunchKernelGGL((scan_kernel<true, true>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((scan_kernel<true, false>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  dim3 grid(a.n_sel * a.G, kHeadDim / 32);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs2
