// The first-generation comparator's sliding-window branch, folded into the decode
// sparse layer (one launch per layer).
//
// HySparse2 article, section 03: the first-generation HySparse reached the recent tokens
// through an independent SWA branch over a local KV cache built from the sparse layer's
// own hidden state.  Its output is added to the block-selected branch's (separate
// softmaxes).
#pragma once

#include "hs2_internal.h"

namespace hs2 {

struct SwaBranch {
  const uint8_t* k;         // [B, Hkv, R, D] the layer's own ring (bf16 bits or e4m3fn codes)
  const uint8_t* v;
  const float* k_scale;     // [B, Hkv, R] (fp8 only)
  const float* v_scale;
  int32_t W;                // window: the W most recent visible positions
  int32_t R;                // ring rows: position p at row p % R (R >= W + q_len - 1)
};

// sparse_head_kernel over the shared cache's index rows (as launch_sparse_head), then
// over the window rows of the ring, writing the sum of the two normalised outputs.
// a.S <= kMaxHeadPathS, 1 <= sw.W <= kMaxHeadPathS, sw.R >= sw.W.
hipError_t launch_sparse_head_swa(const ScanArgs& a, int64_t n_sel, float* out, bool fp8, const SwaBranch& sw,
                                  hipStream_t st);

}  // namespace hs2
