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
// Tiling: a workgroup owns kBM tokens x 256 features (two heads); wave (wm, wn) owns
// 64 tokens x the 128 features of one head, so the quantisation of a row never
// leaves the wave.  The hidden dims go through a ring of kStages LDS stages of kBK
// dims, filled by direct global -> LDS loads (global_load_lds_dwordx4: a wave
// instruction writes 64 lanes x 16 bytes into 1 KiB of LDS, no registers in
// between), so the loads of step kb + kStages - 1 are in flight while step kb
// computes.  Inside a staged row the 16-byte chunks are XOR-swizzled (chunk_swz) so
// that the fragment reads run without LDS bank conflicts.  Products on
// v_mfma_f32_16x16x32_bf16: A = X rows (lane: token i, dims 8grp..), B = W rows.  The
// W rows of a head are staged permuted (staged row 16j + i holds feature 8i + j), so B
// tile j, lane i is feature 8i + j and the accumulators of a lane for one token are
// the 8 consecutive features 8i .. 8i + 7: each lane stores 16 bytes (bf16) or 8
// bytes (fp8) of a cache row directly, and a row's maximum is a max over 8 registers
// and the 16 lanes of its DPP row.
//
// Bound: with the loads removed the loop runs at ~0.8 of the bf16 matrix-core peak;
// with them, the tile loads set the pace (each X tile is re-read by every feature
// tile and each W tile by every token tile, ~1/5 of those reads miss the XCD's L2,
// and a CU keeps only so many lines in flight), which is why the largest tile that
// the registers allow (256 x 256) is used for prefill-size calls.
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2v_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void global_cvoid_t;

// Tile configuration: kBM tokens x 256 features per workgroup, kStages LDS stages of
// kBK hidden dims.
template <int BM, int STAGES, int BK>
struct BridgeCfg {
  static constexpr int kBM = BM;
  static constexpr int kStages = STAGES;
  static constexpr int kBK = BK;
  static constexpr int kWavesM = BM / 64;                  // waves along the tokens
  static constexpr int kWaves = kWavesM * 2;               // x 2 heads
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRowBytes = BK * 2;                 // staged row, unpadded
  static constexpr int kRowChunks = kRowBytes / 16;        // 16-byte chunks per staged row
  static constexpr int kBlockRows = 1024 / kRowBytes;      // staged rows per direct load
  static constexpr int kStageRows = BM + 256;
  static constexpr int kStage = kStageRows * kRowBytes;
  static constexpr int kLds = STAGES * kStage;
  static constexpr int kOcc = (kLds * 2 <= 160 * 1024) ? 2 : 1;   // workgroups per CU
  static constexpr int kBlocks = kStageRows / kBlockRows;  // 1 KiB row blocks per stage
  static constexpr int kLoads = kBlocks / kWaves;          // direct loads per wave per stage
  static_assert(kBlocks % kWaves == 0, "row blocks must split evenly over the waves");
};
// Prefill-size calls: 256 x 256 tiles (8 waves, one workgroup per CU), two stages of 64
// dims (whole 128-byte rows per load).  Small calls (decode appends, short chunks):
// 128 x 256 tiles, two workgroups per CU, three stages of 32 dims.
using BridgeLarge = BridgeCfg<256, 2, 64>;
using BridgeSmall = BridgeCfg<128, 3, 32>;
constexpr int kLargeMinTokens = 4096;
constexpr int kBN = 256;                          // features per workgroup (two heads)
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

// Swizzle of the 16-byte chunks of a staged row (a function of the row mod 16): the
// fragment reads (16 consecutive rows x 4 chunks per instruction) run without LDS
// bank conflicts on gfx950 with chunk c of row r at c ^ ((r >> 1) & 3) in 64-byte
// rows and at c ^ (r & 7) in 128-byte rows (measured with the LDS bank-conflict
// counter; unswizzled rows, 16-byte padding and other XOR patterns conflict).
template <int kRowChunks>
__device__ __forceinline__ int chunk_swz(int r) {
  if constexpr (kRowChunks == 4) return (r >> 1) & 3;
  else return r & 7;
}

// Wait until at most N direct loads of this wave are outstanding, then meet the other
// waves: after it, the stages those loads filled are complete for every wave, and
// every wave has finished reading the stage about to be refilled.  One asm block so
// that no LDS access is moved across either instruction.
template <int N>
__device__ __forceinline__ void wait_loads_and_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
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

template <bool kFp8, class C>
__global__ __launch_bounds__(C::kThreads, C::kOcc) void bridge_kernel(BridgeArgs a) {
  constexpr int kBM = C::kBM, kStages = C::kStages, kBK = C::kBK, kWavesM = C::kWavesM;
  constexpr int kWaves = C::kWaves, kRowBytes = C::kRowBytes, kRowChunks = C::kRowChunks;
  constexpr int kBlockRows = C::kBlockRows, kStage = C::kStage, kLoads = C::kLoads;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[C::kLds];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave % kWavesM;
  const int wn = wave / kWavesM;
  int mt, nt;
  tile_of(a, mt, nt);
  const int m0 = mt * kBM;
  const int n0 = nt * kBN;
  const int nk = a.Hd / kBK;

  // direct loads: wave `wave` fills row blocks wave, wave + kWaves, ... of every
  // stage; lane l writes staged row 16 * block + l / 4, physical chunk l % 4, which
  // holds logical chunk (l % 4) ^ f(row) of the source row
  const uint16_t* src[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int r = (wave + kWaves * i) * kBlockRows + lane / kRowChunks;   // staged row
    const int c = (lane % kRowChunks) ^ chunk_swz<kRowChunks>(r);
    const uint16_t* row;
    if (r < kBM) {
      row = a.x + (size_t)min(m0 + r, a.T - 1) * a.Hd;       // rows past T: row T-1
    } else {
      const int rho = r - kBM;                               // 0..255
      const int h = rho >> 7, q = rho & 127;
      const int f = ((q & 15) << 3) + (q >> 4);              // feature held by row q
      row = a.w + (size_t)(n0 + h * 128 + f) * a.Hd;
    }
    src[i] = row + c * 8;
  }

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int li = lane & 15;
  const int grp = lane >> 4;
  const int swz = chunk_swz<kRowChunks>(li);                             // f depends on row mod 16
  const int a_rd = (wm * 64 + li) * kRowBytes;
  const int b_rd = (kBM + wn * 128 + li) * kRowBytes;

#define HS2_BRIDGE_ISSUE(kb, stage)                                                       \
  do {                                                                                    \
    uint8_t* d_ = lds + (stage) * kStage;                                                 \
    _Pragma("unroll") for (int i = 0; i < kLoads; ++i)                                    \
      __builtin_amdgcn_global_load_lds((global_cvoid_t*)(src[i] + (kb) * kBK),            \
                                       (lds_void_t*)(d_ + (wave + kWaves * i) * 1024), 16, 0, 0); \
  } while (0)

#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) HS2_BRIDGE_ISSUE(s, s);
  for (int kb = 0; kb < nk; ++kb) {
    const int rem = nk - 1 - kb;          // steps issued after this one
    if (rem >= kStages - 2) wait_loads_and_barrier<kLoads * (kStages - 2)>();
    else if (kStages > 3 && rem == 1) wait_loads_and_barrier<kLoads>();
    else wait_loads_and_barrier<0>();
    if (kb + kStages - 1 < nk) HS2_BRIDGE_ISSUE(kb + kStages - 1, (kb + kStages - 1) % kStages);
    const uint8_t* s = lds + (kb % kStages) * kStage;
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      const int cofs = ((4 * ks + grp) ^ swz) * 16;
      bf16x8_t af[4], bfr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(s + a_rd + cofs + i * 16 * kRowBytes);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(s + b_rd + cofs + j * 16 * kRowBytes);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = mfma16(af[i], bfr[j], acc[i][j]);
    }
  }
#undef HS2_BRIDGE_ISSUE

  // epilogue: wave's head = feature block (n0 + 128 wn) / 128 -> (layer, K|V, KV head)
  const int head = (n0 >> 7) + wn;
  const int layer = head / (2 * a.Hkv);
  const int is_v = (head / a.Hkv) & 1;
  const int g = head % a.Hkv;
  uint8_t* cache = static_cast<uint8_t*>(is_v ? a.vc[layer] : a.kc[layer]);
  float* scales = is_v ? a.vs[layer] : a.ks[layer];
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

// Decode-size projection (a few tokens): the tile kernel would stream W through LDS
// for 128-token tiles that are almost all padding.  Here a workgroup owns kSlices
// slices of 16 features and 16 tokens; its waves are (slice, part of the hidden dims)
// pairs, each reading its W rows straight into registers (kGemvUnroll steps of 16
// bytes per lane in flight).  The parts meet in LDS (summed in part order).  bf16
// rows need nothing across features, so a workgroup takes one slice (4 waves, 8
// workgroups per 128-feature row: enough workgroups to keep the W stream going);
// an fp8 row's scale is the maximum over its 128 features, so a workgroup takes a
// whole row (8 slices x 2 parts), the slice maxima meeting in LDS.  W is read once
// per 16 tokens.
constexpr int kGemvTokens = 16;
constexpr int kGemvUnroll = 8;

template <bool kFp8>
struct GemvShape {
  static constexpr int kSlices = kFp8 ? 8 : 1;
  static constexpr int kParts = kFp8 ? 2 : 4;
  static constexpr int kThreads = 64 * kSlices * kParts;
};

template <bool kFp8>
__global__ __launch_bounds__(GemvShape<kFp8>::kThreads) void bridge_gemv_kernel(BridgeArgs a) {
  constexpr int kSlices = GemvShape<kFp8>::kSlices;
  constexpr int kParts = GemvShape<kFp8>::kParts;
  const int m0 = blockIdx.y * kGemvTokens;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int fs = wave % kSlices;   // feature slice
  const int kp = wave / kSlices;   // part of the hidden dims
  const int li = lane & 15;
  const int grp = lane >> 4;
  const int feat0 = (blockIdx.x * kSlices + fs) * 16;   // first feature of the slice
  // part kp takes 32-dim steps [s0, s1) of the Hd / 32
  const int n_steps = a.Hd / 32;
  const int s0 = kp * n_steps / kParts;
  const int s1 = (kp + 1) * n_steps / kParts;
  // A = X rows (lane: token m0 + li, clamped; rows past T are dropped at the store),
  // B = W rows (lane: feature feat0 + li); both take dims 8 grp .. 8 grp + 7 of a step
  const int tok = min(m0 + li, a.T - 1);
  const uint16_t* xr = a.x + (size_t)tok * a.Hd + 8 * grp;
  const uint16_t* wr = a.w + ((size_t)feat0 + li) * a.Hd + 8 * grp;
  f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  int st = s0;
  for (; st + kGemvUnroll <= s1; st += kGemvUnroll) {
    bf16x8_t xa[kGemvUnroll], wb[kGemvUnroll];
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      wb[u] = *reinterpret_cast<const bf16x8_t*>(wr + (size_t)(st + u) * 32);
      xa[u] = *reinterpret_cast<const bf16x8_t*>(xr + (size_t)(st + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) acc = mfma16(xa[u], wb[u], acc);
  }
  for (; st < s1; ++st) {
    const bf16x8_t wb = *reinterpret_cast<const bf16x8_t*>(wr + (size_t)st * 32);
    const bf16x8_t xa = *reinterpret_cast<const bf16x8_t*>(xr + (size_t)st * 32);
    acc = mfma16(xa, wb, acc);
  }

  // lane (li, grp) holds y[token m0 + 4 grp + r][feature feat0 + li], r = 0..3
  __shared__ float red[kParts - 1][kSlices][4][64];
  __shared__ float rmax[kSlices][kGemvTokens];
  if (kp > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[kp - 1][fs][r][lane] = acc[r];
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll
    for (int q = 0; q < kParts - 1; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += red[q][fs][r][lane];
    if constexpr (kFp8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m = max16(fabsf(acc[r]));
        if (li == 0) rmax[fs][4 * grp + r] = m;
      }
    }
  }
  if constexpr (kFp8) __syncthreads();
  if (kp != 0) return;
  const int head = feat0 >> 7;   // (layer, K|V, KV head) feature block
  const int layer = head / (2 * a.Hkv);
  const int is_v = (head / a.Hkv) & 1;
  const int g = head % a.Hkv;
  uint8_t* cache = static_cast<uint8_t*>(is_v ? a.vc[layer] : a.kc[layer]);
  float* scales = is_v ? a.vs[layer] : a.ks[layer];
  const int f = (feat0 & 127) + li;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = m0 + 4 * grp + r;
    const int t = row < a.T ? row : 0;
    const int sq = a.seq[t];
    const int ps = a.pos[t];
    const bool ok = row < a.T && sq >= 0 && sq < a.B && ps >= 0 && (int64_t)ps < a.cap;
    if (!ok) continue;
    const size_t crow = ((size_t)sq * a.Hkv + g) * (size_t)a.cap + (size_t)ps;
    if constexpr (kFp8) {
      float m = rmax[0][4 * grp + r];
#pragma unroll
      for (int k = 1; k < kSlices; ++k) m = fmaxf(m, rmax[k][4 * grp + r]);
      const float sc = m > 0.f ? m / kE4M3Max : 1.0f;
      cache[crow * 128 + f] = (uint8_t)(cvt_fp8x2(acc[r] / sc, 0.0f, 0u, false) & 0xFFu);
      if (f == 0) scales[crow] = sc;
    } else {
      reinterpret_cast<uint16_t*>(cache)[crow * 128 + f] = (uint16_t)(pack_bf16(acc[r], 0.0f) & 0xFFFFu);
    }
  }
}

}  // namespace

int bridge_tile_tokens(int n_tokens) {
  return n_tokens >= kLargeMinTokens ? BridgeLarge::kBM : BridgeSmall::kBM;
}

hipError_t launch_bridge(const BridgeArgs& a, bool fp8, hipStream_t st) {
  if (a.gemv) {
    const unsigned n_slices = (unsigned)(2 * a.n_layers * a.Hkv * (128 / 16));
    const unsigned m_blocks = (unsigned)((a.T + kGemvTokens - 1) / kGemvTokens);
    if (fp8)
      hipLaunchKernelGGL((bridge_gemv_kernel<true>), dim3(n_slices / GemvShape<true>::kSlices, m_blocks),
                         dim3(GemvShape<true>::kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bridge_gemv_kernel<false>), dim3(n_slices / GemvShape<false>::kSlices, m_blocks),
                         dim3(GemvShape<false>::kThreads), 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(a.m_tiles * a.n_tiles));
  if (bridge_tile_tokens(a.T) == BridgeLarge::kBM) {
    if (fp8)
      hipLaunchKernelGGL((bridge_kernel<true, BridgeLarge>), grid, dim3(BridgeLarge::kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bridge_kernel<false, BridgeLarge>), grid, dim3(BridgeLarge::kThreads), 0, st, a);
  } else {
    if (fp8)
      hipLaunchKernelGGL((bridge_kernel<true, BridgeSmall>), grid, dim3(BridgeSmall::kThreads), 0, st, a);
    else
      hipLaunchKernelGGL((bridge_kernel<false, BridgeSmall>), grid, dim3(BridgeSmall::kThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace hs2

// ---------------------------------------------------------------- decode step helper
namespace hs2 {
namespace {

// One new token per sequence: its cache position is the current context length, after
// which the context grows by one (HySparse2 article, section 02: the Cross-Decoder's
// caches grow by the bridged K/V of each generated token).  A sequence whose cache is
// full (or whose length is invalid) gets position -1, which the bridge skips, and
// keeps its length.
// limit: the largest length a sequence may reach (the attention calls' max_ctx_len)
__global__ void advance_kernel(int32_t* ctx_len, int32_t* seq, int32_t* pos, int B, int64_t limit) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int32_t c = ctx_len[b];
  seq[b] = b;
  if (c >= 0 && (int64_t)c < limit) {
    pos[b] = c;
    ctx_len[b] = c + 1;
  } else {
    pos[b] = -1;
  }
}

}  // namespace

hipError_t launch_advance(int32_t* ctx_len, int32_t* seq, int32_t* pos, int B, int64_t limit,
                          hipStream_t st) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 255) / 256), dim3(256), 0, st, ctx_len, seq, pos, B, limit);
  return hipGetLastError();
}

}  // namespace hs2
