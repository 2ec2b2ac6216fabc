// Host-only stand-ins for the kernel launchers of libhs2.so, for a CPU build of the
// C-ABI host layer (hs2_api.cpp) under AddressSanitizer / UndefinedBehaviorSanitizer.
// Nothing here touches a GPU.  Each stand-in checks, on the host, that every
// workspace-derived array the kernel would touch lies inside the workspace the test
// announced (hs2_stub_set_workspace), using the extents the kernels index, and counts
// the launches.  A violation is recorded and reported by hs2_stub_errors().
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "hs2_internal.h"
#include "hs2_swa.h"

namespace {
uintptr_t g_ws_lo = 0, g_ws_hi = 0;
int g_launches = 0, g_errors = 0;
char g_first[256] = {0};

void fail(const char* what) {
  if (g_errors++ == 0) std::snprintf(g_first, sizeof g_first, "%s", what);
}

// [p, p + bytes) inside the workspace (null pointers and empty extents pass)
void in_ws(const void* p, uint64_t bytes, const char* what) {
  if (p == nullptr || bytes == 0 || g_ws_hi == 0) return;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if (a < g_ws_lo || a + bytes > g_ws_hi || a + bytes < a) fail(what);
}
}  // namespace

extern "C" __attribute__((visibility("default"))) void hs2_stub_set_workspace(const void* p, uint64_t bytes) {
  g_ws_lo = reinterpret_cast<uintptr_t>(p);
  g_ws_hi = g_ws_lo + bytes;
  g_launches = 0;
  g_errors = 0;
  g_first[0] = 0;
}
extern "C" __attribute__((visibility("default"))) int hs2_stub_launches() { return g_launches; }
extern "C" __attribute__((visibility("default"))) int hs2_stub_errors() { return g_errors; }
extern "C" __attribute__((visibility("default"))) const char* hs2_stub_first_error() { return g_first; }

namespace hs2 {

static uint64_t sel_rows(const ScanArgs& a, int B) { return (uint64_t)B * a.Lq * a.Hkv; }

static void check_scan(const ScanArgs& a, int B, bool records) {
  if (a.n_split < 1 || a.split_len < 1) fail("scan: empty split geometry");
  if ((int64_t)a.n_split * a.split_len < a.ctx_max) fail("scan: splits do not cover the context");
  const uint64_t n = sel_rows(a, B);
  in_ws(a.part, n * a.n_split * a.G * kPartStride * 4ull, "scan: partials");
  if (records) {
    in_ws(a.records, n * (uint64_t)a.logit_stride * 2ull, "scan: records");
    in_ws(a.hist_part, n * a.n_split * (uint64_t)kFastBins * 2ull, "scan: split histograms");
    in_ws(a.hist_merged, n * (uint64_t)kSelWords * 4ull, "scan: merged histograms");
  }
  if (a.blse != nullptr) in_ws(a.blse, n * (uint64_t)a.blse_stride * 8ull * 4ull, "scan: block sums");
  ++g_launches;
}

int bridge_tile_tokens(int n_tokens) { return n_tokens >= 4096 ? 256 : 128; }

// the no-allocation entry point's scratch: a fake device address; the test announces
// [kStubScratch, kStubScratch + kNoallocScratchBytes) as the workspace
constexpr uintptr_t kStubScratch = uintptr_t(0x7D0000000000);
hipError_t noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(kStubScratch);
  return hipSuccess;
}

hipError_t launch_bridge(const BridgeArgs& a, bool, hipStream_t) {
  if (a.T < 1) fail("bridge: launched with no token");
  for (int l = 0; l < a.n_layers; ++l)
    if (a.kc[l] == nullptr || a.vc[l] == nullptr) fail("bridge: null layer cache");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_advance(int32_t*, int32_t* seq, int32_t* pos, int B, int64_t limit, hipStream_t) {
  in_ws(seq, (uint64_t)B * 4ull, "advance: seq");
  in_ws(pos, (uint64_t)B * 4ull, "advance: pos");
  if (limit < 1) fail("advance: limit");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_swa_rows(const int32_t*, int32_t* idx, int64_t n_sel, int, int, int W, int R, int64_t,
                           hipStream_t) {
  in_ws(idx, (uint64_t)n_sel * W * 4ull, "swa: local index rows");
  if (R < W) fail("swa: ring shorter than the window");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_add(float* out, const float* add, int64_t n, hipStream_t) {
  in_ws(add, (uint64_t)n * 4ull, "add: local branch output");
  if (n % 4 != 0) fail("add: length not a multiple of 4");
  (void)out;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fast_candidates(const FastSelArgs& a, bool, hipStream_t) {
  const uint64_t n = (uint64_t)a.n_sel;
  in_ws(a.records, n * (uint64_t)a.rec_stride * 2ull, "candidates: records");
  in_ws(a.mz, n * kMaxHeads * 2ull * 4ull, "candidates: (M, 1/Z)");
  in_ws(a.selblk, n * (uint64_t)kSelWords * 4ull, "candidates: histograms");
  in_ws(a.cand_keys, n * a.n_chunks * (uint64_t)a.chunk_len * 8ull, "candidates: keys");
  in_ws(a.cand_count, n * (uint64_t)a.n_chunks * 4ull, "candidates: counts");
  if ((int64_t)a.n_chunks * a.chunk_len < a.ctx_max) fail("candidates: chunks do not cover");
  if (a.cand_wgs < 1 || a.cand_wgs > a.n_chunks) fail("candidates: workgroups per row");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_probs_wide(const FastSelArgs& a, float* probs, int64_t probs_stride, bool, hipStream_t) {
  in_ws(a.mz, (uint64_t)a.n_sel * kMaxHeads * 2ull * 4ull, "probs: (M, 1/Z)");
  if (probs == nullptr || probs_stride < a.ctx_max) fail("probs: rows");
  if (a.G <= kSlots || a.G > kMaxHeads) fail("probs: group size");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_fast_final(const FastSelArgs& a, hipStream_t) {
  in_ws(a.cand_keys, (uint64_t)a.n_sel * a.n_chunks * (uint64_t)a.chunk_len * 8ull, "final: keys");
  if (a.n_chunks > kMaxFastChunks) fail("final: chunk count beyond its LDS");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_scan_dense(const ScanArgs& a, bool, bool records, int B, hipStream_t, const KernelEvents*) {
  check_scan(a, B, records);
  if (!records) in_ws(a.logits, sel_rows(a, B) * (uint64_t)a.logit_stride * 8ull * 4ull, "scan: logits");
  return hipSuccess;
}
hipError_t launch_scan_mfma(const ScanArgs& a, bool, int B, hipStream_t, const KernelEvents*) {
  if (a.split_len > kMaxRecordSplit) fail("mfma scan: split beyond its LDS records");
  check_scan(a, B, true);
  return hipSuccess;
}
hipError_t launch_scan_mfma_blocks(const ScanArgs& a, bool, int B, hipStream_t, const KernelEvents*) {
  if (a.split_len > kMaxRecordSplit) fail("block scan: split beyond the scan's LDS");
  if (a.G > kSlots || a.blse == nullptr) fail("block scan: head slots or no block sums");
  if (a.blse != nullptr && (int64_t)a.blse_stride * 32 < a.ctx_max) fail("block scan: block sums do not cover the context");
  check_scan(a, B, false);
  return hipSuccess;
}
hipError_t launch_gather_mfma(const ScanArgs& a, float* out, bool, int B, hipStream_t, const KernelEvents*) {
  if (out == nullptr) in_ws(a.part, sel_rows(a, B) * a.n_split * a.G * kPartStride * 4ull, "gather: partials");
  if ((int64_t)a.n_split * a.split_len < a.S) fail("gather: splits do not cover the index row");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_chunk_mfma(const ScanArgs& a, int B, bool fp8, hipStream_t, const KernelEvents*) {
  if (a.G > kMaxHeads || (a.blse != nullptr && a.G > kSlots)) fail("chunk kernel: head slots");
  if (fp8 && (a.k_scale == nullptr || a.v_scale == nullptr)) fail("chunk kernel: fp8 scales");
  check_scan(a, B, a.blse == nullptr);
  return hipSuccess;
}
hipError_t launch_scan_sparse(const ScanArgs& a, bool, int B, hipStream_t, const KernelEvents*) {
  in_ws(a.part, sel_rows(a, B) * a.n_split * a.G * kPartStride * 4ull, "sparse: partials");
  if ((int64_t)a.n_split * a.split_len < a.S) fail("sparse: splits do not cover the index row");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_sparse_head(const ScanArgs& a, int64_t n_sel, float* out, bool, hipStream_t, const KernelEvents*) {
  if (a.S > kMaxHeadPathS) fail("sparse head: index row beyond its LDS");
  if (n_sel < 1 || out == nullptr) fail("sparse head: rows or output");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_sparse_head_swa(const ScanArgs& a, int64_t n_sel, float* out, bool fp8, const SwaBranch& sw,
                                  hipStream_t) {
  if (a.S > kMaxHeadPathS || sw.W > kMaxHeadPathS) fail("sparse head + window: index rows beyond their LDS");
  if (n_sel < 1 || out == nullptr) fail("sparse head + window: rows or output");
  if (sw.W < 1 || sw.R < sw.W) fail("sparse head + window: ring shorter than the window");
  if (sw.k == nullptr || sw.v == nullptr || (fp8 && (sw.k_scale == nullptr || sw.v_scale == nullptr)))
    fail("sparse head + window: local cache");
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_combine(const CombineArgs& a, hipStream_t) {
  const uint64_t n = (uint64_t)a.n_sel;
  in_ws(a.part, n * a.n_split * a.G * kPartStride * 4ull, "combine: partials");
  in_ws(a.mz, n * kMaxHeads * 2ull * 4ull, "combine: (M, 1/Z)");
  in_ws(a.sel_zero, n * (uint64_t)a.sel_zero_words * 4ull, "combine: control blocks");
  in_ws(a.hist_part, n * a.n_split * (uint64_t)kFastBins * 2ull, "combine: split histograms");
  if (a.hist_part != nullptr) in_ws(a.hist_out, n * (uint64_t)kSelWords * 4ull, "combine: merged histograms");
  ++g_launches;
  return hipSuccess;
}
static void check_select(const SelectArgs& a) {
  const uint64_t n = (uint64_t)a.n_sel;
  in_ws(a.logits, n * (uint64_t)a.logit_stride * 8ull * 4ull, "select: logits");
  in_ws(a.mz, n * kMaxHeads * 2ull * 4ull, "select: (M, 1/Z)");
  in_ws(a.selblk, n * (uint64_t)kSelWords * 4ull, "select: control blocks");
  in_ws(a.hist2, n * (uint64_t)kHist2Bins * 4ull, "select: histogram 2");
  in_ws(a.hist3, n * (uint64_t)kHist3Bins * 4ull, "select: histogram 3");
  in_ws(a.winners, n * (uint64_t)(a.topk > 0 ? a.topk : 1) * 4ull, "select: winners");
  in_ws(a.boundary, n * (uint64_t)kBoundaryCap * 8ull, "select: boundary");
  if (a.blse != nullptr) in_ws(a.blse, n * (uint64_t)a.blse_stride * 8ull * 4ull, "select: block sums");
  ++g_launches;
}
hipError_t launch_groupsum(const SelectArgs& a, hipStream_t) {
  check_select(a);
  // s goes to the workspace unless the caller passed probs (s_stride = capacity then)
  if (a.s_stride == a.logit_stride) in_ws(a.s, (uint64_t)a.n_sel * a.s_stride * 4ull, "groupsum: s");
  return hipSuccess;
}
hipError_t launch_refine(const SelectArgs& a, int, hipStream_t) { check_select(a); return hipSuccess; }
hipError_t launch_collect(const SelectArgs& a, hipStream_t) { check_select(a); return hipSuccess; }
hipError_t launch_finalize(const SelectArgs& a, hipStream_t) { check_select(a); return hipSuccess; }
hipError_t launch_block_select(const SelectArgs& a, hipStream_t) {
  if (a.blse != nullptr && (a.blse_gran < 1 || a.block_size % a.blse_gran != 0)) fail("block select: block-sum granularity");
  if (a.bcand != nullptr) {
    in_ws(a.bcand, (uint64_t)a.n_sel * a.bm_wgs * a.n_blocks * 8ull, "block select: candidate keys");
    if (a.n_blocks > 64 || a.bm_wgs > kMaxBlockMassWgs || (int64_t)a.bm_wgs * a.n_blocks > kMaxBlockPick)
      fail("block select: pick wave capacity");
    if ((int64_t)a.bm_wgs * kBlockMassBlocks * a.block_size < a.ctx_max) fail("block select: mass workgroups do not cover the row");
  }
  check_select(a);
  return hipSuccess;
}

}  // namespace hs2
