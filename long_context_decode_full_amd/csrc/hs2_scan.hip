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
//   positions, each wave a contiguous quarter, walked 8 rows per step.
//   Inside a wave, lane = 8*tg + r: the 8 lanes of token group tg share one row,
//   lane r holds 16 of its 128 dims (two 16-byte loads of bf16, one of fp8), so a
//   step reads 8 whole rows = 2 KiB (bf16) with 128-bit coalesced loads.
//   QK: each lane forms 8 partial dot products (one per head slot) with
//   v_dot2_f32_bf16, then a 3-step DPP butterfly (row_half_mirror, quad_perm x2,
//   quad_perm x1) reduce-scatters them so lane r ends with the full logit of head
//   code(r).  A matching DPP all-gather hands every lane the 8 probabilities of
//   its row for the P.V update into its 8x16 fp32 accumulators.
//   Each token group runs its own online softmax (no cross-group traffic in the
//   loop); the running max is only raised when a logit exceeds it by 8 (log2
//   units), so rescales are rare.  Streams are merged at the end of the split:
//   DPP/shuffles across token groups, LDS across the 4 waves.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {
namespace {

constexpr float kSlack = 8.0f;
constexpr int kThreads = 256;

// Head held in register slot i of lane r is (i ^ code(r)); the butterfly below
// leaves lane r with the complete sum for head code(r).
__device__ __forceinline__ int lane_code(int r) { return r ^ ((r >> 2) * 3); }

// Element e (0..15) of lane r's slice of a 128-dim row.
template <bool kFp8>
__device__ __forceinline__ int elem_dim(int r, int e) {
  if (kFp8) return 16 * r + e;
  return 64 * (e >> 3) + 8 * r + (e & 7);
}

// All-gather within the 8-lane group: out[i] = value of the lane holding head i ^ code(r).
__device__ __forceinline__ void gather8(float x, float (&out)[8]) {
  out[0] = x;
  out[1] = dpp<kDppXor1>(out[0]);
  out[2] = dpp<kDppXor2>(out[0]);
  out[3] = dpp<kDppXor2>(out[1]);
  out[4] = dpp<kDppMirror8>(out[0]);
  out[5] = dpp<kDppMirror8>(out[1]);
  out[6] = dpp<kDppMirror8>(out[2]);
  out[7] = dpp<kDppMirror8>(out[3]);
}

struct RowData {
  uint32_t k[8];   // bf16 pairs of the lane's 16 dims (fp8 codes decoded to bf16)
  uint32_t v[8];   // raw words: bf16 pairs, or fp8 codes in v[0..3]
  float ks, vs;    // fp8 scales
};

template <bool kFp8>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb,
                                         const float* __restrict__ ksb, const float* __restrict__ vsb,
                                         int64_t t, int r, RowData& d) {
  if (kFp8) {
    const uint4 kw = *reinterpret_cast<const uint4*>(kb + t * 128 + 16 * r);
    const uint4 vw = *reinterpret_cast<const uint4*>(vb + t * 128 + 16 * r);
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = kw.z; d.k[3] = kw.w;
    d.v[0] = vw.x; d.v[1] = vw.y; d.v[2] = vw.z; d.v[3] = vw.w;
    d.ks = ksb[t];
    d.vs = vsb[t];
  } else {
    const uint8_t* kr = kb + t * 256;
    const uint8_t* vr = vb + t * 256;
    const uint4 k0 = *reinterpret_cast<const uint4*>(kr + 16 * r);
    const uint4 k1 = *reinterpret_cast<const uint4*>(kr + 128 + 16 * r);
    const uint4 v0 = *reinterpret_cast<const uint4*>(vr + 16 * r);
    const uint4 v1 = *reinterpret_cast<const uint4*>(vr + 128 + 16 * r);
    d.k[0] = k0.x; d.k[1] = k0.y; d.k[2] = k0.z; d.k[3] = k0.w;
    d.k[4] = k1.x; d.k[5] = k1.y; d.k[6] = k1.z; d.k[7] = k1.w;
    d.v[0] = v0.x; d.v[1] = v0.y; d.v[2] = v0.z; d.v[3] = v0.w;
    d.v[4] = v1.x; d.v[5] = v1.y; d.v[6] = v1.z; d.v[7] = v1.w;
    d.ks = 1.0f;
    d.vs = 1.0f;
  }
}

template <bool kSparse, bool kFp8>
__global__ __launch_bounds__(kThreads, 2) void scan_kernel(ScanArgs a) {
  const int split = blockIdx.x;
  const int g = blockIdx.y;
  const int bj = blockIdx.z;
  const int b = bj / a.Lq;
  const int j = bj - b * a.Lq;
  const int64_t sel = (int64_t)bj * a.Hkv + g;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int tg = lane >> 3;
  const int r = lane & 7;
  const int code = lane_code(r);

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
  const int nsteps = w_end > w_begin ? (int)((w_end - w_begin + 7) >> 3) : 0;

  // Query slice: slot i holds head i ^ code (zero for slots beyond the group).
  uint32_t qp[8][8];
  const uint16_t* qrow = a.q + ((int64_t)bj * a.Hq + (int64_t)g * a.G) * kHeadDim;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int head = i ^ code;
    if (head < a.G) {
      const uint16_t* qh = qrow + head * kHeadDim;
      const uint4 x0 = *reinterpret_cast<const uint4*>(qh + (kFp8 ? 16 * r : 8 * r));
      const uint4 x1 = *reinterpret_cast<const uint4*>(qh + (kFp8 ? 16 * r + 8 : 64 + 8 * r));
      qp[i][0] = x0.x; qp[i][1] = x0.y; qp[i][2] = x0.z; qp[i][3] = x0.w;
      qp[i][4] = x1.x; qp[i][5] = x1.y; qp[i][6] = x1.z; qp[i][7] = x1.w;
    } else {
#pragma unroll
      for (int w = 0; w < 8; ++w) qp[i][w] = 0u;
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

  float o[8][16];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;
  float m = kNegInf;
  float z = 0.0f;

  auto row_of = [&](int st, bool& valid) -> int64_t {
    const int64_t pos = w_begin + (int64_t)st * 8 + tg;
    valid = pos < w_end;
    if (kSparse) {
      const int ti = valid ? irow[pos] : -1;
      valid = valid && ti >= 0 && (int64_t)ti < n;
      return valid ? (int64_t)ti : 0;
    }
    return valid ? pos : w_begin;
  };

  RowData cur, nxt;
  bool cur_valid = false, nxt_valid = false;
  int64_t cur_t = 0, nxt_t = 0;
  if (nsteps > 0) {
    cur_t = row_of(0, cur_valid);
    load_row<kFp8>(kb, vb, ksb, vsb, cur_t, r, cur);
  }

  for (int st = 0; st < nsteps; ++st) {
    if (st + 1 < nsteps) {
      nxt_t = row_of(st + 1, nxt_valid);
      load_row<kFp8>(kb, vb, ksb, vsb, nxt_t, r, nxt);
    }

    // ---- logits: 8 partial dot products, then DPP reduce-scatter over the 8 lanes
    uint32_t kw[8];
    if (kFp8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        kw[2 * u] = fp8x2_to_bf16x2(cur.k[u], false);
        kw[2 * u + 1] = fp8x2_to_bf16x2(cur.k[u], true);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 8; ++w) kw[w] = cur.k[w];
    }
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < 8; ++w) s = dot2_bf16(qp[i][w], kw[w], s);
      acc[i] = s;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += dpp<kDppMirror8>(acc[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] += dpp<kDppXor2>(acc[i + 2]);
    acc[0] += dpp<kDppXor1>(acc[1]);

    float l = acc[0] * a.scale_log2;
    if (kFp8) l *= cur.ks;
    l = cur_valid ? l : kNegInf;
    if (!kSparse && cur_valid) lrow[cur_t * 8 + code] = l;

    // ---- online softmax of this token group's stream for head `code`
    const bool up = l > m + kSlack;
    if (wave_any(up)) {
      const float mn = up ? l : m;
      const float alpha = up ? fast_exp2(m - mn) : 1.0f;
      float al[8];
      gather8(alpha, al);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[i][e] *= al[i];
      z *= alpha;
      m = mn;
    }
    const float p = cur_valid ? fast_exp2(l - m) : 0.0f;
    z += p;
    float pv[8];
    gather8(kFp8 ? p * cur.vs : p, pv);

    // ---- P.V into the lane's 8 x 16 accumulators
    if (kFp8) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f32x2_t lo = fp8x2_to_f32(cur.v[u], false);
        const f32x2_t hi = fp8x2_to_f32(cur.v[u], true);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i][4 * u + 0] = __builtin_fmaf(pv[i], lo.x, o[i][4 * u + 0]);
          o[i][4 * u + 1] = __builtin_fmaf(pv[i], lo.y, o[i][4 * u + 1]);
          o[i][4 * u + 2] = __builtin_fmaf(pv[i], hi.x, o[i][4 * u + 2]);
          o[i][4 * u + 3] = __builtin_fmaf(pv[i], hi.y, o[i][4 * u + 3]);
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const float v0 = bf16_lo(cur.v[w]);
        const float v1 = bf16_hi(cur.v[w]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          o[i][2 * w] = __builtin_fmaf(pv[i], v0, o[i][2 * w]);
          o[i][2 * w + 1] = __builtin_fmaf(pv[i], v1, o[i][2 * w + 1]);
        }
      }
    }

    cur = nxt;
    cur_valid = nxt_valid;
    cur_t = nxt_t;
  }

  // ---- merge the 8 token-group streams of this wave (same head = same r)
  float M = m;
  M = fmaxf(M, dpp<kDppRor8>(M));
  M = fmaxf(M, shfl_xor(M, 16));
  M = fmaxf(M, shfl_xor(M, 32));
  const float f = (m == kNegInf) ? 0.0f : fast_exp2(m - M);
  float zz = z * f;
  zz += dpp<kDppRor8>(zz);
  zz += shfl_xor(zz, 16);
  zz += shfl_xor(zz, 32);
  float fg[8];
  gather8(f, fg);
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float x = o[i][e] * fg[i];
      x += dpp<kDppRor8>(x);
      x += shfl_xor(x, 16);
      x += shfl_xor(x, 32);
      o[i][e] = x;
    }

  __shared__ float lds_o[4][8][kHeadDim];
  __shared__ float lds_m[4][8];
  __shared__ float lds_z[4][8];
  if (tg == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int head = i ^ code;
#pragma unroll
      for (int e = 0; e < 16; ++e) lds_o[wave][head][elem_dim<kFp8>(r, e)] = o[i][e];
    }
    lds_m[wave][code] = M;
    lds_z[wave][code] = zz;
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
