// KV Bridging projection on the matrix cores: the K/V caches of the Cross-Decoder's
// Full Attention layers built from one Self-Decoder hidden state.
//
// HySparse2 article, section 02 "two-level KV sharing" (KV Bridging: each target Full
// layer has its own K and V projections of the source hidden state) and section 04
// (prefill ends once the Self-Decoder and these projections have run).
//
// One launch computes Y = X W^T for every target layer at once (W holds W_k,l and
// W_v,l of each layer one after the other, so X is read once for all of them), then
// rounds every (token, KV head) row of 128 features to bf16, or quantises it to OCP
// E4M3FN with one fp32 scale (max|row| / 448; the division and the rounding in fp32),
// and stores it at cache row (seq[t], KV head, pos[t]) of its layer.
//
// Tiling: a workgroup of 4 waves owns 128 tokens x 256 features (two heads); wave
// (wm, wn) owns 64 tokens x the 128 features of one head, so the quantisation of a
// row never leaves the wave.  Per iteration of 64 hidden dims the X and W tiles go
// through LDS (rows padded to 144 bytes: 16-byte reads of 8 (or 16) consecutive rows
// hit distinct banks), double-buffered, with the next tiles loaded into registers
// while the matrix cores work on the current ones.  Products on
// v_mfma_f32_16x16x32_bf16: A = X rows (lane: token i, dims 8grp..), B = W rows.
// The W rows of a head are stored in LDS permuted (LDS row 16j + i holds feature
// 8i + j), so B tile j, lane i is feature 8i + j and the accumulators of a lane for
// one token are the 8 consecutive features 8i .. 8i + 7: each lane stores 16 bytes
// (bf16) or 8 bytes (fp8) of a cache row directly, and a row's maximum is a max over
// 8 registers and the 16 lanes of its DPP row.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2v_t;

constexpr int kBThreads = 256;                    // 4 waves
constexpr int kBM = 128;                          // tokens per workgroup
constexpr int kBN = 256;                          // features per workgroup (two heads)
constexpr int kBK = 64;                           // hidden dims per iteration
constexpr int kRow = kBK * 2 + 16;                // bytes per staged row (128 + pad)
constexpr int kStage = (kBM + kBN) * kRow;        // one X tile + one W tile
constexpr int kBridgeLds = 2 * kStage;            // double-buffered: 110,592 bytes
constexpr int kAChunks = kBM * kBK / 8 / kBThreads;   // 16-byte loads per thread: 4
constexpr int kBChunks = kBN * kBK / 8 / kBThreads;   // 8
constexpr int kGroupM = 8;                        // token tiles per tile group
constexpr float kE4M3Max = 448.0f;

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2v_t x = {lo, hi};   // round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Maximum over the 16 lanes of a DPP row.
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppMirror8>(x));
  return fmaxf(x, dpp<kDppRor8>(x));
}

// fp32 -> E4M3FN codes of two values into bytes 0-1 (hi = false) or 2-3 of `old`:
// round to nearest even; the inputs are clamped to +-448 first (saturation).
__device__ __forceinline__ uint32_t cvt_fp8x2(float a, float b, uint32_t old, bool hi) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}

// Workgroup -> (token tile, feature tile).  Workgroups are dealt to the 8 XCDs in
// turn; each XCD takes a contiguous run of tiles in grouped order (kGroupM token
// tiles per feature tile before the next feature tile), so the workgroups resident
// on one XCD share X and W tiles in its L2.
__device__ __forceinline__ void tile_of(const BridgeArgs& a, int& mt, int& nt) {
  const int n_total = a.m_tiles * a.n_tiles;
  int id = blockIdx.x;
  if ((n_total & 7) == 0) id = (id & 7) * (n_total >> 3) + (id >> 3);
  const int per_group = kGroupM * a.n_tiles;
  const int group = id / per_group;
  const int first = group * kGroupM;
  const int gsize = min(a.m_tiles - first, kGroupM);
  const int in_group = id - group * per_group;
  mt = first + in_group % gsize;
  nt = in_group / gsize;
}

template <bool kFp8>
__global__ __launch_bounds__(kBThreads, 1) void bridge_kernel(BridgeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kBridgeLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1;
  const int wn = wave >> 1;
  int mt, nt;
  tile_of(a, mt, nt);
  const int m0 = mt * kBM;
  const int n0 = nt * kBN;
  const int nk = a.Hd / kBK;

  // global -> LDS assignment: 8 threads per 128-byte row slice, 32 rows per pass
  const int lrow = tid >> 3;
  const int lchunk = tid & 7;
  const u32x4_t* xa[kAChunks];
  const u32x4_t* wb[kBChunks];
  int aoff[kAChunks], boff[kBChunks];
#pragma unroll
  for (int j = 0; j < kAChunks; ++j) {
    const int r = lrow + 32 * j;
    const int t = min(m0 + r, a.T - 1);          // rows past T load row T-1 (not stored)
    xa[j] = reinterpret_cast<const u32x4_t*>(a.x + (size_t)t * a.Hd) + lchunk;
    aoff[j] = r * kRow + lchunk * 16;
  }
#pragma unroll
  for (int j = 0; j < kBChunks; ++j) {
    const int r = lrow + 32 * j;                 // feature row of the tile, 0..255
    wb[j] = reinterpret_cast<const u32x4_t*>(a.w + (size_t)(n0 + r) * a.Hd) + lchunk;
    const int h = r >> 7, f = r & 127;
    boff[j] = (kBM + h * 128 + ((f & 7) << 4) + (f >> 3)) * kRow + lchunk * 16;
  }

  u32x4_t ra[kAChunks], rb[kBChunks];
#define HS2_BRIDGE_GLOAD(kb)                                                  \
  do {                                                                        \
    const int o_ = (kb) * (kBK / 8);                                          \
    _Pragma("unroll") for (int j = 0; j < kAChunks; ++j) ra[j] = xa[j][o_];   \
    _Pragma("unroll") for (int j = 0; j < kBChunks; ++j) rb[j] = wb[j][o_];   \
  } while (0)
#define HS2_BRIDGE_LSTORE(stage)                                              \
  do {                                                                        \
    uint8_t* s_ = lds + (stage) * kStage;                                     \
    _Pragma("unroll") for (int j = 0; j < kAChunks; ++j)                      \
      *reinterpret_cast<u32x4_t*>(s_ + aoff[j]) = ra[j];                        \
    _Pragma("unroll") for (int j = 0; j < kBChunks; ++j)                      \
      *reinterpret_cast<u32x4_t*>(s_ + boff[j]) = rb[j];                        \
  } while (0)

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int a_rd = (wm * 64 + (lane & 15)) * kRow + (lane >> 4) * 16;
  const int b_rd = (kBM + wn * 128 + (lane & 15)) * kRow + (lane >> 4) * 16;

  HS2_BRIDGE_GLOAD(0);
  HS2_BRIDGE_LSTORE(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const bool more = kb + 1 < nk;
    if (more) HS2_BRIDGE_GLOAD(kb + 1);
    const uint8_t* s = lds + (kb & 1) * kStage;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t af[4], bfr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(s + a_rd + i * 16 * kRow + ks * 64);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(s + b_rd + j * 16 * kRow + ks * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
    if (more) HS2_BRIDGE_LSTORE((kb + 1) & 1);
    __syncthreads();
  }

#undef HS2_BRIDGE_GLOAD
#undef HS2_BRIDGE_LSTORE
  // epilogue: wave's head = feature block (n0 + 128 wn) / 128 -> (layer, K|V, KV head)
  const int head = (n0 >> 7) + wn;
  const int layer = head / (2 * a.Hkv);
  const int is_v = (head / a.Hkv) & 1;
  const int g = head % a.Hkv;
  uint8_t* cache = static_cast<uint8_t*>(is_v ? a.vc[layer] : a.kc[layer]);
  float* scales = is_v ? a.vs[layer] : a.ks[layer];
  const int li = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      const int t = row < a.T ? row : 0;
      const int sq = a.seq[t];
      const int ps = a.pos[t];
      const bool ok = row < a.T && sq >= 0 && sq < a.B && ps >= 0 && (int64_t)ps < a.cap;
      const size_t crow = ok ? ((size_t)sq * a.Hkv + g) * (size_t)a.cap + (size_t)ps : 0;
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = acc[i][j][r];
      if constexpr (kFp8) {
        float m = fabsf(v[0]);
#pragma unroll
        for (int j = 1; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
        m = max16(m);
        const float sc = m > 0.f ? m / kE4M3Max : 1.0f;
        uint32_t w0 = cvt_fp8x2(v[0] / sc, v[1] / sc, 0u, false);
        w0 = cvt_fp8x2(v[2] / sc, v[3] / sc, w0, true);
        uint32_t w1 = cvt_fp8x2(v[4] / sc, v[5] / sc, 0u, false);
        w1 = cvt_fp8x2(v[6] / sc, v[7] / sc, w1, true);
        if (ok) {
          *reinterpret_cast<uint2*>(cache + crow * 128 + li * 8) = make_uint2(w0, w1);
          if (li == 0) scales[crow] = sc;
        }
      } else {
        const uint4 o = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]),
                                   pack_bf16(v[4], v[5]), pack_bf16(v[6], v[7]));
        if (ok) *reinterpret_cast<uint4*>(cache + crow * 256 + li * 16) = o;
      }
    }
  }
}

}  // namespace

hipError_t launch_bridge(const BridgeArgs& a, bool fp8, hipStream_t st) {
  const dim3 grid((unsigned)(a.m_tiles * a.n_tiles));
  if (fp8)
    hipLaunchKernelGGL((bridge_kernel<true>), grid, dim3(kBThreads), 0, st, a);
  else
    hipLaunchKernelGGL((bridge_kernel<false>), grid, dim3(kBThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace hs2
