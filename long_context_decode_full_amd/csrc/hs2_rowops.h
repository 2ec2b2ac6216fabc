// Per-row building blocks shared by the attention scan and the exact re-scoring of
// selection candidates.  Both must produce bit-identical logits for a row, so both
// use these functions with the same lane layout:
//   wave64 = 4 row groups of 16 lanes; lane r of a row group holds dims [8r, 8r+8)
//   of its row (one 16-byte load of bf16, 8 bytes of fp8) and, in register slot i,
//   the matching query slice of head i ^ head_of(r).
#pragma once

#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {

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

// All-gather inside the 16-lane row group: out[i] = value of head i ^ head_of(r).
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

// Reductions over the 8 distinct heads of a row group (lanes r and r^1 hold the
// same head, and {xor 2, half-mirror, ror 8} moves between all 8 of them).
__device__ __forceinline__ float rowgroup_max8(float x) {
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppMirror8>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  return x;
}
__device__ __forceinline__ uint32_t rowgroup_or8(uint32_t x) {
  x |= dpp_u<kDppXor2>(x);
  x |= dpp_u<kDppMirror8>(x);
  x |= dpp_u<kDppRor8>(x);
  return x;
}
__device__ __forceinline__ float rowgroup_sum16(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppMirror8>(x);
  x += dpp<kDppRor8>(x);
  return x;
}

struct RowData {
  uint32_t k[4];   // bf16: 4 pairs of the lane's 8 dims; fp8: k[0..1] hold 8 codes
  uint32_t v[4];
  float ks, vs;    // fp8 per-token scales
};

// kStream: the rows are read once (the dense scan), so they take the non-temporal
// hint; the 16 lanes of a row cover whole cache lines.  Scales stay ordinary loads
// (4 bytes per row: a line serves 32 rows).
template <bool kFp8, bool kStream = false>
__device__ __forceinline__ void load_row(const uint8_t* __restrict__ kb, const uint8_t* __restrict__ vb,
                                         const float* __restrict__ ksb, const float* __restrict__ vsb,
                                         uint32_t t, int r, RowData& d) {
  if (kFp8) {
    const uint2* kp = reinterpret_cast<const uint2*>(kb + (uint64_t)t * 128 + 8 * r);
    const uint2* vp = reinterpret_cast<const uint2*>(vb + (uint64_t)t * 128 + 8 * r);
    const uint2 kw = kStream ? load_nt(kp) : *kp;
    const uint2 vw = kStream ? load_nt(vp) : *vp;
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = 0u; d.k[3] = 0u;
    d.v[0] = vw.x; d.v[1] = vw.y; d.v[2] = 0u; d.v[3] = 0u;
    d.ks = ksb[t];
    d.vs = vsb[t];
  } else {
    const uint4* kp = reinterpret_cast<const uint4*>(kb + (uint64_t)t * 256 + 16 * r);
    const uint4* vp = reinterpret_cast<const uint4*>(vb + (uint64_t)t * 256 + 16 * r);
    const uint4 kw = kStream ? load_nt(kp) : *kp;
    const uint4 vw = kStream ? load_nt(vp) : *vp;
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = kw.z; d.k[3] = kw.w;
    d.v[0] = vw.x; d.v[1] = vw.y; d.v[2] = vw.z; d.v[3] = vw.w;
    d.ks = 1.0f;
    d.vs = 1.0f;
  }
}

// K part only (candidate re-scoring).
template <bool kFp8>
__device__ __forceinline__ void load_key(const uint8_t* __restrict__ kb, const float* __restrict__ ksb,
                                         uint32_t t, int r, RowData& d) {
  if (kFp8) {
    const uint2 kw = *reinterpret_cast<const uint2*>(kb + (uint64_t)t * 128 + 8 * r);
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = 0u; d.k[3] = 0u;
    d.ks = ksb[t];
  } else {
    const uint4 kw = *reinterpret_cast<const uint4*>(kb + (uint64_t)t * 256 + 16 * r);
    d.k[0] = kw.x; d.k[1] = kw.y; d.k[2] = kw.z; d.k[3] = kw.w;
    d.ks = 1.0f;
  }
}

// Query slice of lane r: slot i holds dims [8r, 8r+8) of head i ^ head_of(r) of the
// KV group starting at qgroup (zero beyond the group's G heads).
__device__ __forceinline__ void load_query(const uint16_t* qgroup, int G, int r, uint32_t (&qp)[8][4]) {
  const int hown = head_of(r);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // branch-free: a slot past the group reads head 0 (in bounds) and keeps zeros
    const int head = i ^ hown;
    const bool in = head < G;
    const uint4 x = *reinterpret_cast<const uint4*>(qgroup + (in ? head : 0) * kHeadDim + 8 * r);
    qp[i][0] = in ? x.x : 0u; qp[i][1] = in ? x.y : 0u; qp[i][2] = in ? x.z : 0u; qp[i][3] = in ? x.w : 0u;
  }
}

// Logit (log2 domain: sm_scale * log2(e) * q.k, times the key's fp8 scale) of head
// head_of(r) for the row whose key slice this lane holds: 8 partial dot products with
// v_dot2_f32_bf16 (bf16 x bf16 products are exact), then a DPP butterfly that
// halves the slots three times (row_ror:8, row_half_mirror, quad_perm) and adds
// the last pair (quad_perm).
template <bool kFp8>
__device__ __forceinline__ float row_logit(const uint32_t (&qp)[8][4], const RowData& cur, float scale_log2) {
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
  return l;
}

// Bound record of one row (2 bytes): e = log2(sum over the group's real heads h of
// 2^l_h), rounded to IEEE binary16.  With per-head weights w_h = 2^-M_h / Z_h the
// row's group-summed probability s = sum_h w_h 2^l_h lies within
// [min_h w_h, max_h w_h] * 2^e, so e bounds s once the global statistics are known.
// Every lane of the row group computes it; `l` is this lane's (masked) logit.
__device__ __forceinline__ uint16_t row_record(float l, int r, int hown, int G) {
  const float lm = hown < G ? l : kNegInf;
  const float rmax = rowgroup_max8(lm);
  const float ex = ((r & 1) == 0 && lm != kNegInf) ? fast_exp2(lm - rmax) : 0.0f;
  const float sum = rowgroup_sum16(ex);
  const float e = rmax + __builtin_amdgcn_logf(sum);   // v_log_f32: log2; sum >= 1 for valid rows
  return __builtin_bit_cast(uint16_t, (_Float16)e);
}

// Order-preserving 16-bit key of a binary16 bit pattern.
__device__ __forceinline__ uint32_t half_order_key(uint32_t bits) {
  return (bits & 0x8000u) ? (~bits & 0xFFFFu) : (bits | 0x8000u);
}
__device__ __forceinline__ uint32_t half_bits_of_key(uint32_t key) {
  return (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
}
__device__ __forceinline__ float half_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}
// Spacing of binary16 values at `bits` (finite values): 2^(E-25), 2^-24 for subnormals.
__device__ __forceinline__ float half_ulp(uint32_t bits) {
  const int e5 = (int)((bits >> 10) & 31u);
  return e5 == 0 ? 0x1p-24f : __builtin_ldexpf(1.0f, e5 - 25);
}

}  // namespace hs2
