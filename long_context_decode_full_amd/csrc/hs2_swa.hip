// First-generation HySparse sparse layer (comparator): the separate sliding-window
// branch over the layer's own local KV.
//
// HySparse2 article, section 03: in the first-generation HySparse the recent tokens were
// reached by an independent SWA branch whose cache came from the sparse layer's own
// hidden state; HySparse2 folds that local access into the one sparse computation over
// the shared cache.  The local cache is a ring of R rows: position p sits at row p % R,
// so a query token that sees positions [0, n) reads the rows of [max(0, n - W), n).
#include "hs2_device.h"
#include "hs2_internal.h"

namespace hs2 {
namespace {

// One selection row (b, j, g) per workgroup: the local-cache rows of its window, -1 past
// the end (fewer than W visible positions).
__global__ void swa_rows_kernel(const int32_t* __restrict__ ctx_len, int32_t* __restrict__ idx, int Lq,
                                int Hkv, int W, int R, int64_t ctx_max) {
  const int64_t row = blockIdx.x;
  const int64_t bj = row / Hkv;
  const int b = (int)(bj / Lq);
  const int j = (int)(bj - (int64_t)b * Lq);
  int64_t ctx = ctx_len[b];
  ctx = ctx < 0 ? 0 : (ctx > ctx_max ? ctx_max : ctx);
  int64_t n = ctx - Lq + j + 1;
  n = n < 0 ? 0 : n;
  const int64_t cnt = n < W ? n : W;
  const int64_t p0 = n - cnt;
  for (int e = threadIdx.x; e < W; e += blockDim.x)
    idx[row * W + e] = e < cnt ? (int32_t)((p0 + e) % R) : -1;
}

__global__ void add_kernel(float4* __restrict__ out, const float4* __restrict__ add, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) {
    const float4 a = out[i], c = add[i];
    out[i] = make_float4(a.x + c.x, a.y + c.y, a.z + c.z, a.w + c.w);
  }
}

}  // namespace

hipError_t launch_swa_rows(const int32_t* ctx_len, int32_t* idx, int64_t n_sel, int Lq, int Hkv, int W,
                           int R, int64_t ctx_max, hipStream_t st) {
  hipLaunchKernelGGL(swa_rows_kernel, dim3((unsigned)n_sel), dim3(128), 0, st, ctx_len, idx, Lq, Hkv, W, R,
                     ctx_max);
  return hipGetLastError();
}

hipError_t launch_add(float* out, const float* add, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(out), reinterpret_cast<const float4*>(add), n4);
  return hipGetLastError();
}

}  // namespace hs2
