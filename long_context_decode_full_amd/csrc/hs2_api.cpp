// C-ABI host layer: descriptor validation, workspace layout, launch sequences.
// Contract of every entry point: include/hs2.h.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "hs2.h"
#include "hs2_internal.h"
#include "hs2_swa.h"

#define HS2_API extern "C" __attribute__((visibility("default")))

namespace hs2 {
namespace {

constexpr size_t kAlign = 256;
constexpr int kScanTargetWorkgroups = 768;   // 3 per CU (3 waves/SIMD) on 256 CUs
constexpr int kMfmaTargetWorkgroups = 256;   // matrix-core scan: 1 per CU (8 waves)
constexpr int64_t kFusedSparseRows = 256;    // sparse layer: one workgroup per row from here
constexpr int64_t kHeadPathRows = 64;        // ... and one workgroup per query head below this
constexpr int kCandTargetWorkgroups = 4096;  // candidate stage: workgroups over all rows
constexpr int kCandTwoStepPerRow = 2;         // the two-kernel form (many rows): workgroups per row
constexpr double kMaxLogitsBytes = 16.0 * (1 << 30);   // logits-path workspace budget
constexpr int kMaxSplits = 2048;             // combine kernel keeps one weight per split in LDS
constexpr int kChunkMaxSplit = 4096;         // positions per chunk-kernel split (at most)
constexpr int kSparseSplitLen = 64;          // index entries per sparse workgroup (fewest)
constexpr int kSparseTargetWorkgroups = 320;  // ... unless the rows would launch more than this
constexpr int kSelectChunk = kSelectChunkLen;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Layout {
  int64_t n_sel = 0;
  int64_t logit_stride = 0;
  int32_t G = 0, S = 0;
  int32_t split_len = 0, n_split = 0;
  int32_t split_len_sp = 0, n_split_sp = 0;
  int32_t chunk_len = 0, n_chunks = 0;
  int32_t rec_split_len = 0, rec_n_split = 0;   // scan geometry of the record path
  int32_t n_cchunks = 0;                        // record path: candidate chunks per row
  int32_t cand_chunk_len = 0;                   // positions per candidate chunk
  bool fast_ok = false;                         // record path usable for this descriptor
  bool logits_ok = false;                       // logits path (probs, block mode) fits its budget
  size_t off_records = 0;
  size_t off_blse = 0;                          // block mode: per-block sums
  int64_t blse_stride = 0;
  int32_t blse_gran = 0;                        // positions per block sum
  size_t off_bcand = 0;                         // block mode: mass workgroups' candidate keys
  int32_t bm_wgs = 0;                           // ... workgroups a row (0: one-kernel selection)
  size_t off_cand_keys = 0, off_cand_count = 0, off_hist_part = 0;
  size_t off_logits = 0, off_part = 0, off_mz = 0, off_s = 0, off_selblk = 0, off_hist2 = 0,
         off_hist3 = 0, off_winners = 0, off_boundary = 0, total = 0;
};

hs2_status validate_desc(const hs2_attn_desc* d) {
  if (d == nullptr) return HS2_ERR_INVALID_ARG;
  if (d->batch < 1 || d->q_len < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1)
    return HS2_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return HS2_ERR_INVALID_ARG;
  if (d->kv_dtype != HS2_KV_BF16 && d->kv_dtype != HS2_KV_FP8_E4M3FN) return HS2_ERR_INVALID_ARG;
  if (d->kv_capacity < 1 || d->max_ctx_len < d->q_len || d->max_ctx_len > d->kv_capacity)
    return HS2_ERR_INVALID_ARG;
  if (!(d->sm_scale > 0.0f) || !std::isfinite(d->sm_scale)) return HS2_ERR_INVALID_ARG;
  // options: known flag bits, not both sparse routes, non-negative sizes
  if ((d->flags & ~HS2_FLAGS_ALL) != 0u) return HS2_ERR_INVALID_ARG;
  const uint32_t sparse_paths = d->flags & (HS2_FLAG_SPARSE_FUSED | HS2_FLAG_SPARSE_SPLIT | HS2_FLAG_SPARSE_HEAD);
  if ((sparse_paths & (sparse_paths - 1u)) != 0u) return HS2_ERR_INVALID_ARG;   // at most one
  if (d->split_len < 0 || d->sparse_split_len < 0 || d->cand_workgroups < 0) return HS2_ERR_INVALID_ARG;
  if (d->select_mode == HS2_SELECT_TOKEN) {
    if (d->window < 0 || d->topk < 0 || (int64_t)d->window + d->topk < 1) return HS2_ERR_INVALID_ARG;
    if ((int64_t)d->window + d->topk > 4096) return HS2_ERR_UNSUPPORTED;
  } else if (d->select_mode == HS2_SELECT_BLOCK) {
    if (d->block_size < 1 || d->n_blocks < 1) return HS2_ERR_INVALID_ARG;
    if ((int64_t)d->block_size * d->n_blocks > 4096) return HS2_ERR_UNSUPPORTED;
    if (ceil_div(d->max_ctx_len, d->block_size) > kMaxBlocksLds) return HS2_ERR_UNSUPPORTED;
  } else {
    return HS2_ERR_INVALID_ARG;
  }
  if (d->head_dim != kHeadDim) return HS2_ERR_UNSUPPORTED;
  // up to 32 query heads per KV head (MQA at Hq = 32); beyond 8 the record path and the
  // block sums only (no logits path), see wide_group() and full_path_supported()
  if (d->n_q_heads / d->n_kv_heads > kMaxHeads) return HS2_ERR_UNSUPPORTED;
  if (d->kv_capacity >= (int64_t(1) << 31)) return HS2_ERR_UNSUPPORTED;
  if ((int64_t)d->batch * d->q_len > 65535) return HS2_ERR_UNSUPPORTED;
  if (d->n_kv_heads > 65535) return HS2_ERR_UNSUPPORTED;
  // selection rows index flattened grids of (row, chunk) workgroups
  if ((int64_t)d->batch * d->q_len * d->n_kv_heads > 65535ll * 1024) return HS2_ERR_UNSUPPORTED;
  return HS2_OK;
}

bool has_flag(const hs2_attn_desc* d, uint32_t f) { return (d->flags & f) != 0u; }

// Token selection for a chunk of query tokens (q_len > 1, bf16 or fp8 cache) runs the
// matrix-core chunk kernel, which reads each KV row once for 256 query rows (32 tokens
// of up to 8 heads, 16 of up to 16, 8 of up to 32).
// HS2_FLAG_CHUNK_PER_TOKEN runs the decode scan once per token instead (comparison).
bool chunk_path(const hs2_attn_desc* d) {
  return d->q_len > 1 && d->select_mode == HS2_SELECT_TOKEN && !has_flag(d, HS2_FLAG_CHUNK_PER_TOKEN);
}
// More than 8 query heads per KV head: the matrix-core scans with 16-head blocks, the
// matrix-core gather and block-wise re-scoring; the logits path (probs) keeps 8 head
// slots and is not used.
bool wide_group(const hs2_attn_desc* d) { return d->n_q_heads / d->n_kv_heads > kSlots; }
// The block comparator for a chunk (block sizes that are multiples of 64) takes its
// block masses from the same kernel's per-block sums instead of per-position logits.
bool chunk_block_path(const hs2_attn_desc* d) {
  return d->q_len > 1 && d->select_mode == HS2_SELECT_BLOCK && d->block_size % 64 == 0 &&
         !has_flag(d, HS2_FLAG_CHUNK_PER_TOKEN);
}
// The block comparator otherwise (decode, per-token chunks): per-32-position
// block sums from the decode scan, in the scan's head layout (up to 32 query heads per
// KV head).  HS2_FLAG_FORCE_LOGITS or HS2_FLAG_SCAN_VALU keep it on the logits path.
bool scan_block_path(const hs2_attn_desc* d) {
  return d->select_mode == HS2_SELECT_BLOCK && !chunk_block_path(d) && d->block_size % 32 == 0 &&
         !has_flag(d, HS2_FLAG_FORCE_LOGITS) && !has_flag(d, HS2_FLAG_SCAN_VALU);
}

// logits_area: reserve the logits path's per-position scores whenever that path fits
// its budget (the workspace callers size with hs2_workspace_size), or only when this
// call takes that path (the no-allocation entry point, which knows its call).
Layout make_layout(const hs2_attn_desc* d, bool logits_area = true) {
  Layout L;
  L.n_sel = (int64_t)d->batch * d->q_len * d->n_kv_heads;
  L.G = d->n_q_heads / d->n_kv_heads;
  L.S = d->select_mode == HS2_SELECT_TOKEN ? d->window + d->topk : d->block_size * d->n_blocks;
  // one spare row per selection receives the scan's masked logit stores
  L.logit_stride = ceil_div(d->max_ctx_len + 1, 64) * 64;

  // Dense scan: enough splits to give ~2 workgroups per CU in one residency round.
  const int64_t rows = L.n_sel * d->max_ctx_len;
  int64_t split = ceil_div(ceil_div(rows, kScanTargetWorkgroups), 256) * 256;
  split = d->split_len > 0 ? (int64_t)d->split_len : std::min<int64_t>(split, 1 << 30);
  split = ceil_div(split, 256) * 256;
  if (split < 256) split = 256;
  while (ceil_div(d->max_ctx_len, split) > kMaxSplits) split *= 2;
  L.split_len = (int32_t)split;
  L.n_split = (int32_t)ceil_div(d->max_ctx_len, split);

  // Record path: a split's records stay in LDS until it is done, which bounds the split.
  // The matrix-core scan holds 1 workgroup per CU: one residency round of 256.  The
  // chunk kernel (one workgroup per CU, 32 query tokens each) takes 1/16 of the
  // longest context per split, between 1,024 and 4,096 positions: ragged batches
  // then spread over many rounds of workgroups (16,384-position splits left a third
  // of the CUs idle in the last round; splits past a sequence's end cost nothing).
  int64_t rsplit;
  if (chunk_path(d) || chunk_block_path(d)) {
    rsplit = ceil_div(ceil_div(d->max_ctx_len, 16), 256) * 256;
    rsplit = std::min<int64_t>(std::max<int64_t>(rsplit, 1024), kChunkMaxSplit);
    while (ceil_div(d->max_ctx_len, rsplit) > kMaxSplits && rsplit < kMaxRecordSplit) rsplit *= 2;
  } else {
    const int64_t rec_target = has_flag(d, HS2_FLAG_SCAN_VALU) ? kScanTargetWorkgroups : kMfmaTargetWorkgroups;
    rsplit = ceil_div(ceil_div(rows, rec_target), 256) * 256;
  }
  rsplit = d->split_len > 0 ? (int64_t)d->split_len : std::min<int64_t>(rsplit, 1 << 30);
  rsplit = ceil_div(rsplit, 256) * 256;
  if (rsplit < 256) rsplit = 256;
  if (rsplit > kMaxRecordSplit) rsplit = kMaxRecordSplit;
  L.rec_split_len = (int32_t)rsplit;
  L.rec_n_split = (int32_t)ceil_div(d->max_ctx_len, rsplit);
  // candidate workgroups: ~64 per row, 2048..16384 positions each (a power of two)
  int64_t clen = kMinCandChunkLen;
  while (clen < kCandChunkLen && clen * 64 < d->max_ctx_len) clen *= 2;
  L.cand_chunk_len = (int32_t)clen;
  L.n_cchunks = (int32_t)ceil_div(d->max_ctx_len, clen);
  L.fast_ok = d->select_mode == HS2_SELECT_TOKEN && L.n_cchunks <= kMaxFastChunks &&
              L.rec_n_split <= kMaxSplits;

  // index entries per sparse workgroup: 64, doubled (up to 256) while the rows would
  // launch more than ~320 workgroups (many rows: fewer, longer chains measured faster)
  int64_t sp = kSparseSplitLen;
  while (sp < 256 && L.n_sel * ceil_div(L.S, sp) > kSparseTargetWorkgroups) sp *= 2;
  if (d->sparse_split_len > 0) sp = d->sparse_split_len;
  sp = std::max<int64_t>(ceil_div(sp, 32) * 32, 32);
  while (ceil_div(L.S, sp) > kMaxSplits) sp *= 2;
  L.split_len_sp = (int32_t)sp;
  L.n_split_sp = (int32_t)ceil_div(L.S, sp);

  L.chunk_len = kSelectChunk;
  L.n_chunks = (int32_t)ceil_div(d->max_ctx_len, kSelectChunk);

  const int64_t n = L.n_sel;
  // (the matrix-core split gather of wide groups takes 128-entry splits)
  const int64_t nsplit_max = std::max({(int64_t)L.n_split, (int64_t)L.n_split_sp, (int64_t)L.rec_n_split,
                                       ceil_div(L.S, 128)});
  // The logits path keeps 36 bytes per (selection row, position); beyond kMaxLogitsBytes
  // (chunk configurations with long contexts) it is not offered and not reserved.
  L.logits_ok = (double)n * (double)L.logit_stride * 36.0 <= (double)kMaxLogitsBytes;
  size_t off = 0;
  L.off_part = off;   off = align_up(off + (size_t)n * nsplit_max * L.G * kPartStride * sizeof(float));
  L.off_mz = off;     off = align_up(off + (size_t)n * kMaxHeads * 2 * sizeof(float));
  L.off_selblk = off; off = align_up(off + (size_t)n * kSelWords * sizeof(uint32_t));
  if (L.logits_ok && logits_area) {
    L.off_logits = off; off = align_up(off + (size_t)n * L.logit_stride * 8 * sizeof(float));
    L.off_records = L.off_logits;   // the record path's 2-byte records share that area
    L.off_s = off;      off = align_up(off + (size_t)n * L.logit_stride * sizeof(float));
    L.off_hist2 = off;  off = align_up(off + (size_t)n * kHist2Bins * sizeof(uint32_t));
    L.off_hist3 = off;  off = align_up(off + (size_t)n * kHist3Bins * sizeof(uint32_t));
    L.off_winners = off; off = align_up(off + (size_t)n * std::max(d->topk, 1) * sizeof(int32_t));
    L.off_boundary = off; off = align_up(off + (size_t)n * kBoundaryCap * sizeof(uint2));
  } else {
    L.off_records = off; off = align_up(off + (size_t)n * L.logit_stride * sizeof(uint16_t));
  }
  if (chunk_block_path(d) || scan_block_path(d)) {
    L.blse_gran = chunk_block_path(d) ? 64 : 32;
    L.blse_stride = ceil_div(d->max_ctx_len, L.blse_gran);
    L.off_blse = off; off = align_up(off + (size_t)n * L.blse_stride * blse_heads_of(L.G) * sizeof(float));
    // block selection over many workgroups a row (up to 64 blocks kept)
    const int64_t wgs = ceil_div(ceil_div(d->max_ctx_len, d->block_size), kBlockMassBlocks);
    if (d->n_blocks <= 64 && wgs <= kMaxBlockMassWgs && wgs * d->n_blocks <= kMaxBlockPick) {
      L.bm_wgs = (int32_t)wgs;
      L.off_bcand = off; off = align_up(off + (size_t)n * wgs * d->n_blocks * sizeof(uint64_t));
    }
  }
  if (L.fast_ok) {
    const size_t slots = (size_t)n * L.n_cchunks * L.cand_chunk_len;
    L.off_cand_keys = off; off = align_up(off + slots * sizeof(uint64_t));
    L.off_cand_count = off; off = align_up(off + (size_t)n * L.n_cchunks * sizeof(int32_t));
    L.off_hist_part = off; off = align_up(off + (size_t)n * L.rec_n_split * kFastBins * sizeof(uint16_t));
  }
  L.total = off;
  return L;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The events of a timed call (hs2_*_timed), bound to its dominant kernel's launch.
struct TimedLaunch {
  KernelEvents kev{};
  const KernelEvents* ptr = nullptr;
  explicit TimedLaunch(const hs2_kernel_events* ev) {
    if (ev != nullptr) {
      kev = KernelEvents{ev->begin, ev->end};
      ptr = &kev;
    }
  }
};

}  // namespace
}  // namespace hs2

using namespace hs2;

HS2_API hs2_status hs2_validate(const hs2_attn_desc* desc, size_t workspace_bytes) {
  const hs2_status s = validate_desc(desc);
  if (s != HS2_OK) return s;
  return workspace_bytes < make_layout(desc).total ? HS2_ERR_WORKSPACE : HS2_OK;
}

#ifndef HS2_BUILD_ID
#define HS2_BUILD_ID "unknown"
#endif
HS2_API const char* hs2_build_id(void) { return HS2_BUILD_ID; }

HS2_API hs2_status hs2_workspace_size(const hs2_attn_desc* desc, size_t* bytes) {
  const hs2_status s = validate_desc(desc);
  if (s != HS2_OK) return s;
  if (bytes == nullptr) return HS2_ERR_INVALID_ARG;
  *bytes = make_layout(desc).total;
  return HS2_OK;
}

HS2_API const char* hs2_status_string(hs2_status status) {
  switch (status) {
    case HS2_OK: return "ok";
    case HS2_ERR_INVALID_ARG: return "invalid argument";
    case HS2_ERR_UNSUPPORTED: return "unsupported configuration";
    case HS2_ERR_WORKSPACE: return "workspace too small";
    case HS2_ERR_ALIGNMENT: return "misaligned pointer";
    case HS2_ERR_LAUNCH: return "kernel launch failed";
    case HS2_ERR_SCRATCH_LIMIT: return "call needs more than the library's no-allocation scratch";
  }
  return "unknown status";
}

static hs2_status check_common(const hs2_attn_desc* d, const void* q, const void* k, const void* v,
                               const float* ks, const float* vs, const int32_t* ctx_len,
                               const void* out, const void* idx, void* ws, size_t ws_bytes,
                               Layout* L) {
  hs2_status s = validate_desc(d);
  if (s != HS2_OK) return s;
  if (!q || !k || !v || !ctx_len || !out || !idx || !ws) return HS2_ERR_INVALID_ARG;
  if (d->kv_dtype == HS2_KV_FP8_E4M3FN && (!ks || !vs)) return HS2_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(idx, 16) || !aligned(ws, 16) || !aligned(ctx_len, 4))
    return HS2_ERR_ALIGNMENT;
  if (d->kv_dtype == HS2_KV_FP8_E4M3FN && (!aligned(ks, 4) || !aligned(vs, 4)))
    return HS2_ERR_ALIGNMENT;
  *L = make_layout(d);
  if (ws_bytes < L->total) return HS2_ERR_WORKSPACE;
  return HS2_OK;
}

// Which selection path hs2_full_attn_select takes, and whether it has one for this call.
// More than 8 query heads per KV head: no logits path; probs, when asked for, come from
// an exact re-score of every visible position after the selection (launch_probs_wide).
static bool use_record_path(const hs2_attn_desc* d, const Layout& L, const float* probs) {
  return L.fast_ok && (probs == nullptr || wide_group(d)) && (wide_group(d) || !has_flag(d, HS2_FLAG_FORCE_LOGITS));
}
// Block comparator on the scans' block sums (needs no per-position scores).
static bool block_sums_path(const hs2_attn_desc* d, const float* probs) {
  return (probs == nullptr || wide_group(d)) && (chunk_block_path(d) || scan_block_path(d));
}
// probs for G > 8: s of every visible position from the row's (M, 1/Z), after the selection
static hipError_t probs_pass(const hs2_attn_desc* d, const Layout& L, const ScanArgs& sa, const float* mz,
                             float* probs, hipStream_t stream) {
  FastSelArgs fa{};
  fa.mz = mz;
  fa.ctx_len = sa.ctx_len;
  fa.ctx_max = d->max_ctx_len;
  fa.q = sa.q;
  fa.k = sa.k;
  fa.k_scale = sa.k_scale;
  fa.cap = d->kv_capacity;
  fa.scale_log2 = sa.scale_log2;
  fa.n_sel = (int32_t)L.n_sel;
  fa.Lq = d->q_len;
  fa.Hq = d->n_q_heads;
  fa.Hkv = d->n_kv_heads;
  fa.G = L.G;
  fa.window = d->window;
  fa.topk = d->topk;
  fa.S = L.S;
  return launch_probs_wide(fa, probs, d->kv_capacity, d->kv_dtype == HS2_KV_FP8_E4M3FN, stream);
}
static hs2_status full_path_supported(const hs2_attn_desc* d, const Layout& L, const float* probs) {
  const bool fast = use_record_path(d, L, probs);
  const bool bsums = block_sums_path(d, probs);
  if (!fast && !bsums && !L.logits_ok) return HS2_ERR_UNSUPPORTED;
  if (!fast && !bsums && wide_group(d)) return HS2_ERR_UNSUPPORTED;   // the logits path has 8 head slots
  return HS2_OK;
}

static ScanArgs scan_args(const hs2_attn_desc* d, const Layout& L, const void* q, const void* k,
                          const void* v, const float* ks, const float* vs, const int32_t* ctx_len,
                          uint8_t* ws) {
  ScanArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint8_t*>(k);
  a.v = static_cast<const uint8_t*>(v);
  a.k_scale = ks;
  a.v_scale = vs;
  a.ctx_len = ctx_len;
  a.part = reinterpret_cast<float*>(ws + L.off_part);
  a.cap = d->kv_capacity;
  a.ctx_max = d->max_ctx_len;
  a.logit_stride = L.logit_stride;
  a.Lq = d->q_len;
  a.Hq = d->n_q_heads;
  a.Hkv = d->n_kv_heads;
  a.G = L.G;
  a.S = L.S;
  a.scale_log2 = d->sm_scale * 1.44269504088896340736f;
  a.fixed_steps = has_flag(d, HS2_FLAG_DETERMINISTIC) ? 1 : 0;
  a.exact_pv = has_flag(d, HS2_FLAG_EXACT_PV) ? 1 : 0;
  return a;
}

// Block comparator on block sums: the chunk kernel's (64 positions) or the decode
// scan's (32 positions) per-block log-sum-exp per head, the split combine, then the
// block selection on those sums.  No per-position score is written or re-read.
hs2_status block_sums_select(const hs2_attn_desc* desc, const Layout& L, ScanArgs sa,
                             const int32_t* ctx_len, float* out, int32_t* idx, float* probs, uint8_t* ws,
                             hipStream_t stream, const hs2_kernel_events* ev) {
  sa.records = nullptr;
  sa.hist_part = nullptr;
  sa.hist_merged = nullptr;
  sa.blse = reinterpret_cast<float*>(ws + L.off_blse);
  sa.blse_stride = L.blse_stride;
  sa.window = 0;
  sa.n_split = L.rec_n_split;
  sa.split_len = L.rec_split_len;
  const TimedLaunch tl(ev);
  const hipError_t e = chunk_block_path(desc)
                           ? launch_chunk_mfma(sa, desc->batch, desc->kv_dtype == HS2_KV_FP8_E4M3FN, stream, tl.ptr)
                           : launch_scan_mfma_blocks(sa, desc->kv_dtype == HS2_KV_FP8_E4M3FN, desc->batch, stream,
                                                     tl.ptr);
  if (e != hipSuccess) return HS2_ERR_LAUNCH;

  CombineArgs ca{};
  ca.part = sa.part;
  ca.out = out;
  ca.mz = reinterpret_cast<float*>(ws + L.off_mz);
  ca.hist_out = reinterpret_cast<uint32_t*>(ws + L.off_selblk);
  ca.n_sel = (int32_t)L.n_sel;
  ca.Hkv = desc->n_kv_heads;
  ca.G = L.G;
  ca.Hq = desc->n_q_heads;
  ca.n_split = sa.n_split;
  ca.ctx_len = sa.ctx_len;   // fold only the splits below each row's visible length
  ca.ctx_max = sa.ctx_max;
  ca.Lq = sa.Lq;
  ca.split_len = sa.split_len;
  if (launch_combine(ca, stream) != hipSuccess) return HS2_ERR_LAUNCH;

  SelectArgs sl{};
  sl.mz = ca.mz;
  sl.ctx_len = ctx_len;
  sl.ctx_max = desc->max_ctx_len;
  sl.idx = idx;
  sl.n_sel = (int32_t)L.n_sel;
  sl.Lq = desc->q_len;
  sl.Hkv = desc->n_kv_heads;
  sl.G = L.G;
  sl.window = desc->window;
  sl.topk = desc->topk;
  sl.S = L.S;
  sl.block_size = desc->block_size;
  sl.n_blocks = desc->n_blocks;
  sl.blse = sa.blse;
  sl.blse_stride = L.blse_stride;
  sl.blse_gran = L.blse_gran;
  sl.bcand = L.bm_wgs > 0 ? reinterpret_cast<uint64_t*>(ws + L.off_bcand) : nullptr;
  sl.bm_wgs = L.bm_wgs;
  if (launch_block_select(sl, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  if (probs != nullptr && probs_pass(desc, L, sa, ca.mz, probs, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  return HS2_OK;
}

// The launches of hs2_full_attn_select for a checked call, in workspace layout L.
static hs2_status full_select_launch(const hs2_attn_desc* desc, const Layout& L, const void* q,
                                     const void* k, const void* v, const float* k_scale,
                                     const float* v_scale, const int32_t* ctx_len, float* out,
                                     int32_t* idx, float* probs, uint8_t* ws, hipStream_t stream,
                                     const hs2_kernel_events* ev);

HS2_API hs2_status hs2_full_attn_select_timed(const hs2_attn_desc* desc, const void* q, const void* k,
                                              const void* v, const float* k_scale, const float* v_scale,
                                              const int32_t* ctx_len, float* out, int32_t* idx,
                                              float* probs, void* workspace, size_t workspace_bytes,
                                              hipStream_t stream, const hs2_kernel_events* ev) {
  Layout L;
  hs2_status s = check_common(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, workspace,
                              workspace_bytes, &L);
  if (s != HS2_OK) return s;
  if (probs != nullptr && !aligned(probs, 4)) return HS2_ERR_ALIGNMENT;
  s = full_path_supported(desc, L, probs);
  if (s != HS2_OK) return s;
  return full_select_launch(desc, L, q, k, v, k_scale, v_scale, ctx_len, out, idx, probs,
                            static_cast<uint8_t*>(workspace), stream, ev);
}

static hs2_status full_select_launch(const hs2_attn_desc* desc, const Layout& L, const void* q,
                                     const void* k, const void* v, const float* k_scale,
                                     const float* v_scale, const int32_t* ctx_len, float* out,
                                     int32_t* idx, float* probs, uint8_t* ws, hipStream_t stream,
                                     const hs2_kernel_events* ev) {
  const bool fp8 = desc->kv_dtype == HS2_KV_FP8_E4M3FN;
  // Record path (default for token selection): compact bound records, exact
  // re-scoring of the candidates.  Logits path: every position's logits, needed
  // when the caller wants all probabilities (probs) or for the block comparator.
  const bool fast = use_record_path(desc, L, probs);
  ScanArgs sa = scan_args(desc, L, q, k, v, k_scale, v_scale, ctx_len, ws);
  if (block_sums_path(desc, probs)) return block_sums_select(desc, L, sa, ctx_len, out, idx, probs, ws, stream, ev);
  sa.logits = reinterpret_cast<float*>(ws + L.off_logits);
  sa.records = reinterpret_cast<uint16_t*>(ws + L.off_records);
  sa.hist_part = reinterpret_cast<uint16_t*>(ws + L.off_hist_part);
  sa.hist_merged = reinterpret_cast<uint32_t*>(ws + L.off_selblk);
  sa.window = desc->window;
  sa.n_split = fast ? L.rec_n_split : L.n_split;
  sa.split_len = fast ? L.rec_split_len : L.split_len;

  // record path: matrix-core scan (HS2_FLAG_SCAN_VALU selects the VALU scan instead)
  const bool mfma = fast && (wide_group(desc) || !has_flag(desc, HS2_FLAG_SCAN_VALU));
  const TimedLaunch tl(ev);
  const hipError_t e = (fast && chunk_path(desc)) ? launch_chunk_mfma(sa, desc->batch, fp8, stream, tl.ptr)
                 : mfma                     ? launch_scan_mfma(sa, fp8, desc->batch, stream, tl.ptr)
                                            : launch_scan_dense(sa, fp8, fast, desc->batch, stream, tl.ptr);
  if (e != hipSuccess) return HS2_ERR_LAUNCH;

  CombineArgs ca{};
  ca.part = sa.part;
  ca.out = out;
  ca.mz = reinterpret_cast<float*>(ws + L.off_mz);
  // the logits path clears the selection control blocks here; on the record path
  // the scan has cleared the merged key histograms that the combine sums into
  ca.sel_zero = fast ? nullptr : reinterpret_cast<uint32_t*>(ws + L.off_selblk);
  ca.sel_zero_words = kSelWords;
  ca.hist_part = fast ? sa.hist_part : nullptr;
  ca.hist_out = reinterpret_cast<uint32_t*>(ws + L.off_selblk);
  ca.n_sel = (int32_t)L.n_sel;
  ca.Hkv = desc->n_kv_heads;
  ca.G = L.G;
  ca.Hq = desc->n_q_heads;
  ca.n_split = sa.n_split;
  ca.ctx_len = sa.ctx_len;   // fold only the splits below each row's visible length
  ca.ctx_max = sa.ctx_max;
  ca.Lq = sa.Lq;
  ca.split_len = sa.split_len;
  if (launch_combine(ca, stream) != hipSuccess) return HS2_ERR_LAUNCH;

  if (fast) {
    FastSelArgs fa{};
    fa.records = sa.records;
    fa.rec_stride = L.logit_stride;
    fa.mz = ca.mz;
    fa.ctx_len = ctx_len;
    fa.ctx_max = desc->max_ctx_len;
    fa.selblk = ca.hist_out;
    fa.cand_keys = reinterpret_cast<uint64_t*>(ws + L.off_cand_keys);
    fa.cand_count = reinterpret_cast<int32_t*>(ws + L.off_cand_count);
    fa.idx = idx;
    fa.q = static_cast<const uint16_t*>(q);
    fa.k = static_cast<const uint8_t*>(k);
    fa.k_scale = k_scale;
    fa.cap = desc->kv_capacity;
    fa.scale_log2 = sa.scale_log2;
    fa.n_chunks = L.n_cchunks;
    fa.chunk_len = L.cand_chunk_len;
    // workgroups per row: all chunks of a row while rows are few (decode), fewer once
    // there are many rows, so short rows do not launch mostly empty workgroups
    const int64_t per_row = desc->cand_workgroups > 0 ? ceil_div(desc->cand_workgroups, L.n_sel)
                            : L.n_sel >= kTwoStepMinRows ? kCandTwoStepPerRow
                                                         : ceil_div(kCandTargetWorkgroups, L.n_sel);
    fa.cand_wgs = (int32_t)std::max<int64_t>(1, std::min<int64_t>(L.n_cchunks, per_row));
    fa.n_sel = (int32_t)L.n_sel;
    fa.Lq = desc->q_len;
    fa.Hq = desc->n_q_heads;
    fa.Hkv = desc->n_kv_heads;
    fa.G = L.G;
    fa.window = desc->window;
    fa.topk = desc->topk;
    fa.S = L.S;
    if (launch_fast_candidates(fa, fp8, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (launch_fast_final(fa, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (probs != nullptr && probs_pass(desc, L, sa, ca.mz, probs, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    return HS2_OK;
  }

  SelectArgs sl{};
  sl.logits = sa.logits;
  sl.mz = ca.mz;
  sl.s = probs != nullptr ? probs : reinterpret_cast<float*>(ws + L.off_s);
  sl.s_stride = probs != nullptr ? desc->kv_capacity : L.logit_stride;
  sl.logit_stride = L.logit_stride;
  sl.ctx_len = ctx_len;
  sl.ctx_max = desc->max_ctx_len;
  sl.selblk = ca.sel_zero;
  sl.hist2 = reinterpret_cast<uint32_t*>(ws + L.off_hist2);
  sl.hist3 = reinterpret_cast<uint32_t*>(ws + L.off_hist3);
  sl.winners = reinterpret_cast<int32_t*>(ws + L.off_winners);
  sl.boundary = reinterpret_cast<uint2*>(ws + L.off_boundary);
  sl.idx = idx;
  sl.n_sel = (int32_t)L.n_sel;
  sl.Lq = desc->q_len;
  sl.Hkv = desc->n_kv_heads;
  sl.G = L.G;
  sl.window = desc->window;
  sl.topk = desc->topk;
  sl.S = L.S;
  sl.block_size = desc->block_size;
  sl.n_blocks = desc->n_blocks;
  sl.chunk_len = L.chunk_len;
  sl.n_chunks = L.n_chunks;

  if (desc->select_mode == HS2_SELECT_TOKEN) {
    sl.with_hist = 1;
    if (launch_groupsum(sl, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (launch_refine(sl, 2, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (launch_refine(sl, 3, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (launch_collect(sl, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (launch_finalize(sl, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  } else {
    sl.with_hist = 0;
    if (launch_groupsum(sl, stream) != hipSuccess) return HS2_ERR_LAUNCH;
    if (launch_block_select(sl, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  }
  return HS2_OK;
}

HS2_API hs2_status hs2_full_attn_select(const hs2_attn_desc* desc, const void* q, const void* k,
                                        const void* v, const float* k_scale, const float* v_scale,
                                        const int32_t* ctx_len, float* out, int32_t* idx,
                                        float* probs, void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  return hs2_full_attn_select_timed(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, probs,
                                    workspace, workspace_bytes, stream, nullptr);
}

// Same launches over the library's own scratch (one static device array per GPU): no
// workspace argument, nothing allocated.  The layout reserves only what this call's
// path uses, so the record path at a million positions fits the array.
HS2_API hs2_status hs2_full_attn_select_noalloc(const hs2_attn_desc* desc, const void* q, const void* k,
                                                const void* v, const float* k_scale, const float* v_scale,
                                                const int32_t* ctx_len, float* out, int32_t* idx,
                                                float* probs, hipStream_t stream) {
  hs2_status s = validate_desc(desc);
  if (s != HS2_OK) return s;
  Layout L;
  // every pointer check of the workspace entry point (the workspace itself aside)
  static uint8_t stand_in[16] __attribute__((aligned(16)));
  s = check_common(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, stand_in, SIZE_MAX, &L);
  if (s != HS2_OK) return s;
  if (probs != nullptr && !aligned(probs, 4)) return HS2_ERR_ALIGNMENT;
  L = make_layout(desc, false);
  if (!use_record_path(desc, L, probs) && !block_sums_path(desc, probs))
    L = make_layout(desc, true);   // the logits path's scores are needed
  s = full_path_supported(desc, L, probs);
  if (s != HS2_OK) return s;
  if (L.total > kNoallocScratchBytes) return HS2_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (noalloc_scratch(&ws) != hipSuccess || ws == nullptr) return HS2_ERR_LAUNCH;
  return full_select_launch(desc, L, q, k, v, k_scale, v_scale, ctx_len, out, idx, probs,
                            static_cast<uint8_t*>(ws), stream, nullptr);
}

// slot_rows: index entries are rows of a local cache (any row < cap), not positions.
static hs2_status sparse_impl(const hs2_attn_desc* desc, const void* q, const void* k, const void* v,
                              const float* k_scale, const float* v_scale, const int32_t* ctx_len,
                              const int32_t* idx, float* out, void* workspace, size_t workspace_bytes,
                              hipStream_t stream, int slot_rows, const hs2_kernel_events* ev) {
  Layout L;
  hs2_status s = check_common(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, workspace,
                              workspace_bytes, &L);
  if (s != HS2_OK) return s;
  const bool fp8 = desc->kv_dtype == HS2_KV_FP8_E4M3FN;
  uint8_t* ws = static_cast<uint8_t*>(workspace);

  ScanArgs sa = scan_args(desc, L, q, k, v, k_scale, v_scale, ctx_len, ws);
  sa.idx = idx;
  sa.slot_rows = slot_rows;
  sa.n_split = L.n_split_sp;
  sa.split_len = L.split_len_sp;

  // With a row per CU or more (query chunks), one matrix-core workgroup per (query
  // token, KV head) gathers the whole index row and writes the output: 2.1x faster on
  // the 64-token chunks.  With fewer rows (decode) its 4-5 dependent steps per wave
  // are latency-bound.  Below kHeadPathRows rows one workgroup per (query token,
  // query head) gathers its KV head's whole index row and writes the output in one
  // launch; in between, the split VALU gather + combine.
  // HS2_FLAG_SPARSE_FUSED / _SPLIT / _HEAD force a path.
  // More than 8 heads per KV head on the split path: the matrix-core gather over
  // splits of one step per wave (256 entries with 8 waves, 128 with the 4-wave 32-head
  // layout) writing partials, then the combine.
  const int64_t rows = (int64_t)desc->batch * desc->q_len * desc->n_kv_heads;
  static_assert(kMaxHeadPathS >= 4096, "validate_desc admits index rows of up to 4,096 entries");
  const bool forced = has_flag(desc, HS2_FLAG_SPARSE_FUSED) || has_flag(desc, HS2_FLAG_SPARSE_SPLIT) ||
                      has_flag(desc, HS2_FLAG_SPARSE_HEAD);
  const bool fused = has_flag(desc, HS2_FLAG_SPARSE_FUSED) || (!forced && rows >= kFusedSparseRows);
  const bool head = has_flag(desc, HS2_FLAG_SPARSE_HEAD) || (!forced && rows < kHeadPathRows);
  const TimedLaunch tl(ev);
  if (head) {
    const hipError_t e = launch_sparse_head(sa, rows, out, fp8, stream, tl.ptr);
    return e == hipSuccess ? HS2_OK : HS2_ERR_LAUNCH;
  }
  if (fused) {
    sa.n_split = 1;
    sa.split_len = L.S;
    const hipError_t e = launch_gather_mfma(sa, out, fp8, desc->batch, stream, tl.ptr);
    return e == hipSuccess ? HS2_OK : HS2_ERR_LAUNCH;
  }
  hipError_t e;
  if (wide_group(desc)) {
    sa.split_len = L.G > 16 ? 128 : 256;
    sa.n_split = (int32_t)ceil_div(L.S, sa.split_len);
    e = launch_gather_mfma(sa, nullptr, fp8, desc->batch, stream, tl.ptr);
  } else {
    e = launch_scan_sparse(sa, fp8, desc->batch, stream, tl.ptr);
  }
  if (e != hipSuccess) return HS2_ERR_LAUNCH;

  CombineArgs ca{};
  ca.part = sa.part;
  ca.out = out;
  ca.n_sel = (int32_t)L.n_sel;
  ca.Hkv = desc->n_kv_heads;
  ca.G = L.G;
  ca.Hq = desc->n_q_heads;
  ca.n_split = sa.n_split;
  if (launch_combine(ca, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  return HS2_OK;
}

HS2_API hs2_status hs2_sparse_attn_timed(const hs2_attn_desc* desc, const void* q, const void* k,
                                         const void* v, const float* k_scale, const float* v_scale,
                                         const int32_t* ctx_len, const int32_t* idx, float* out,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                                         const hs2_kernel_events* ev) {
  return sparse_impl(desc, q, k, v, k_scale, v_scale, ctx_len, idx, out, workspace, workspace_bytes,
                     stream, 0, ev);
}

HS2_API hs2_status hs2_sparse_attn(const hs2_attn_desc* desc, const void* q, const void* k,
                                   const void* v, const float* k_scale, const float* v_scale,
                                   const int32_t* ctx_len, const int32_t* idx, float* out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sparse_impl(desc, q, k, v, k_scale, v_scale, ctx_len, idx, out, workspace, workspace_bytes,
                     stream, 0, nullptr);
}

// Every check of hs2_kv_bridge; fills the launch arguments.  *empty: nothing to launch.
static hs2_status bridge_prepare(const hs2_bridge_desc* d, const void* x, const void* w,
                                 const int32_t* seq, const int32_t* pos, void* const* k_caches,
                                 void* const* v_caches, float* const* k_scales,
                                 float* const* v_scales, BridgeArgs* out, bool* empty) {
  if (d == nullptr) return HS2_ERR_INVALID_ARG;
  if (d->n_tokens < 0 || d->hidden < 1 || d->n_layers < 1 || d->n_kv_heads < 1 ||
      d->batch < 1 || d->kv_capacity < 1)
    return HS2_ERR_INVALID_ARG;
  if (d->gemv_max_tokens < -1 || d->gemv_max_tokens > 1024 || d->reserved != 0) return HS2_ERR_INVALID_ARG;
  if (d->kv_dtype != HS2_KV_BF16 && d->kv_dtype != HS2_KV_FP8_E4M3FN) return HS2_ERR_INVALID_ARG;
  if (d->head_dim != kHeadDim || d->hidden % 64 != 0 || d->hidden > 65536 ||
      d->n_layers > kMaxBridgeLayers || d->n_kv_heads > 65535 ||
      d->kv_capacity >= (int64_t(1) << 31))
    return HS2_ERR_UNSUPPORTED;
  const bool fp8 = d->kv_dtype == HS2_KV_FP8_E4M3FN;
  if (!x || !w || !seq || !pos || !k_caches || !v_caches) return HS2_ERR_INVALID_ARG;
  if (fp8 && (!k_scales || !v_scales)) return HS2_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(seq, 4) || !aligned(pos, 4))
    return HS2_ERR_ALIGNMENT;
  BridgeArgs a{};
  for (int l = 0; l < d->n_layers; ++l) {
    if (!k_caches[l] || !v_caches[l]) return HS2_ERR_INVALID_ARG;
    if (!aligned(k_caches[l], 16) || !aligned(v_caches[l], 16)) return HS2_ERR_ALIGNMENT;
    a.kc[l] = k_caches[l];
    a.vc[l] = v_caches[l];
    if (fp8) {
      if (!k_scales[l] || !v_scales[l]) return HS2_ERR_INVALID_ARG;
      if (!aligned(k_scales[l], 4) || !aligned(v_scales[l], 4)) return HS2_ERR_ALIGNMENT;
      a.ks[l] = k_scales[l];
      a.vs[l] = v_scales[l];
    }
  }
  // features: n_layers x {K, V} x n_kv_heads x 128, in tiles of 256 (two heads)
  const int64_t n_feat = (int64_t)d->n_layers * 2 * d->n_kv_heads * kHeadDim;
  const int64_t n_tiles = n_feat / 256;
  const int64_t m_tiles = ceil_div(d->n_tokens, bridge_tile_tokens(d->n_tokens));
  if (m_tiles * n_tiles > INT32_MAX) return HS2_ERR_UNSUPPORTED;
  a.x = static_cast<const uint16_t*>(x);
  a.w = static_cast<const uint16_t*>(w);
  a.seq = seq;
  a.pos = pos;
  a.cap = d->kv_capacity;
  a.T = d->n_tokens;
  a.Hd = d->hidden;
  a.Hkv = d->n_kv_heads;
  a.B = d->batch;
  a.n_layers = d->n_layers;
  a.m_tiles = (int32_t)m_tiles;
  a.n_tiles = (int32_t)n_tiles;
  // few tokens (decode): the W-streaming path; gemv_max_tokens moves the switch
  const int gemv_max = d->gemv_max_tokens == 0 ? kBridgeGemvMaxTokens : d->gemv_max_tokens;   // -1: never
  a.gemv = d->n_tokens <= gemv_max ? 1 : 0;
  *out = a;
  *empty = d->n_tokens == 0;
  return HS2_OK;
}

HS2_API hs2_status hs2_kv_bridge(const hs2_bridge_desc* d, const void* x, const void* w,
                                 const int32_t* seq, const int32_t* pos,
                                 void* const* k_caches, void* const* v_caches,
                                 float* const* k_scales, float* const* v_scales,
                                 hipStream_t stream) {
  BridgeArgs a{};
  bool empty = false;
  const hs2_status s = bridge_prepare(d, x, w, seq, pos, k_caches, v_caches, k_scales, v_scales,
                                      &a, &empty);
  if (s != HS2_OK || empty) return s;
  const bool fp8 = d->kv_dtype == HS2_KV_FP8_E4M3FN;
  if (launch_bridge(a, fp8, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  return HS2_OK;
}

// ---------------------------------------------------------------- decode step
namespace {

struct DecodeWs {
  size_t attn = 0, off_seq = 0, off_pos = 0, total = 0;
};

hs2_status decode_layout(const hs2_decode_plan* p, DecodeWs* w) {
  if (p == nullptr) return HS2_ERR_INVALID_ARG;
  const hs2_status s = validate_desc(&p->attn);
  if (s != HS2_OK) return s;
  if (p->attn.q_len != 1) return HS2_ERR_INVALID_ARG;
  if (p->n_blocks < 1 || p->n_sparse < 0 || p->hidden < 1) return HS2_ERR_INVALID_ARG;
  if (p->n_blocks > kMaxBridgeLayers || p->n_sparse > kMaxDecodeSparse) return HS2_ERR_UNSUPPORTED;
  w->attn = make_layout(&p->attn).total;
  w->off_seq = align_up(w->attn);
  w->off_pos = align_up(w->off_seq + (size_t)p->attn.batch * sizeof(int32_t));
  w->total = align_up(w->off_pos + (size_t)p->attn.batch * sizeof(int32_t));
  return HS2_OK;
}

}  // namespace

HS2_API hs2_status hs2_decode_workspace_size(const hs2_decode_plan* plan, size_t* bytes) {
  DecodeWs w;
  const hs2_status s = decode_layout(plan, &w);
  if (s != HS2_OK) return s;
  if (bytes == nullptr) return HS2_ERR_INVALID_ARG;
  *bytes = w.total;
  return HS2_OK;
}

HS2_API hs2_status hs2_decode_step(const hs2_decode_plan* plan, const void* x, const void* w,
                                   const void* const* q_full, const void* const* q_sparse,
                                   void* const* k_caches, void* const* v_caches,
                                   float* const* k_scales, float* const* v_scales,
                                   int32_t* ctx_len, float* const* out_full,
                                   int32_t* const* idx, float* const* out_sparse,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  DecodeWs wl;
  hs2_status s = decode_layout(plan, &wl);
  if (s != HS2_OK) return s;
  const hs2_attn_desc* d = &plan->attn;
  const int nb = plan->n_blocks, ns = plan->n_sparse;
  const bool fp8 = d->kv_dtype == HS2_KV_FP8_E4M3FN;
  if (!q_full || !k_caches || !v_caches || !ctx_len || !out_full || !idx || !workspace)
    return HS2_ERR_INVALID_ARG;
  if (ns > 0 && (!q_sparse || !out_sparse)) return HS2_ERR_INVALID_ARG;
  if (fp8 && (!k_scales || !v_scales)) return HS2_ERR_INVALID_ARG;
  if (!aligned(workspace, 16)) return HS2_ERR_ALIGNMENT;
  if (workspace_bytes < wl.total) return HS2_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* seq = reinterpret_cast<int32_t*>(ws + wl.off_seq);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + wl.off_pos);

  // every check of every call below, before anything is enqueued
  hs2_bridge_desc bd{};
  bd.n_tokens = d->batch;
  bd.hidden = plan->hidden;
  bd.n_layers = nb;
  bd.n_kv_heads = d->n_kv_heads;
  bd.head_dim = d->head_dim;
  bd.kv_dtype = d->kv_dtype;
  bd.batch = d->batch;
  bd.kv_capacity = d->kv_capacity;
  BridgeArgs ba{};
  bool empty = false;
  s = bridge_prepare(&bd, x, w, seq, pos, k_caches, v_caches, k_scales, v_scales, &ba, &empty);
  if (s != HS2_OK) return s;
  for (int l = 0; l < nb; ++l) {
    const float* ks = fp8 ? k_scales[l] : nullptr;
    const float* vs = fp8 ? v_scales[l] : nullptr;
    Layout L;
    s = check_common(d, q_full[l], k_caches[l], v_caches[l], ks, vs, ctx_len, out_full[l], idx[l],
                     workspace, wl.attn, &L);
    if (s != HS2_OK) return s;
    s = full_path_supported(d, L, nullptr);
    if (s != HS2_OK) return s;
    for (int j = 0; j < ns; ++j) {
      s = check_common(d, q_sparse[l * ns + j], k_caches[l], v_caches[l], ks, vs, ctx_len,
                       out_sparse[l * ns + j], idx[l], workspace, wl.attn, &L);
      if (s != HS2_OK) return s;
    }
  }

  // 1. positions of the new tokens; contexts grow by one
  if (launch_advance(ctx_len, seq, pos, d->batch, d->max_ctx_len, stream) != hipSuccess)
    return HS2_ERR_LAUNCH;
  // 2. KV Bridging: the new tokens' K/V rows into every block's cache
  if (launch_bridge(ba, fp8, stream) != hipSuccess) return HS2_ERR_LAUNCH;
  // 3. every Hybrid Block: the full layer selects, its sparse layers reuse the selection
  for (int l = 0; l < nb; ++l) {
    const float* ks = fp8 ? k_scales[l] : nullptr;
    const float* vs = fp8 ? v_scales[l] : nullptr;
    s = hs2_full_attn_select(d, q_full[l], k_caches[l], v_caches[l], ks, vs, ctx_len, out_full[l],
                             idx[l], nullptr, workspace, wl.attn, stream);
    if (s != HS2_OK) return s;
    for (int j = 0; j < ns; ++j) {
      s = hs2_sparse_attn(d, q_sparse[l * ns + j], k_caches[l], v_caches[l], ks, vs, ctx_len,
                          idx[l], out_sparse[l * ns + j], workspace, wl.attn, stream);
      if (s != HS2_OK) return s;
    }
  }
  return HS2_OK;
}

// ---------------------------------------------------------------- first-generation sparse layer
namespace {

struct SwaWs {
  hs2_attn_desc local{};
  size_t attn = 0, off_idx = 0, off_out = 0, total = 0;
};

hs2_status swa_layout(const hs2_attn_desc* d, int32_t W, int32_t R, SwaWs* w) {
  const hs2_status s = validate_desc(d);
  if (s != HS2_OK) return s;
  if (W < 1 || R < 1) return HS2_ERR_INVALID_ARG;
  if (W > 4096 || (int64_t)R < (int64_t)W + d->q_len - 1) return HS2_ERR_UNSUPPORTED;
  // the local branch: the same heads and queries over a cache of R rows, index rows of W
  w->local = *d;
  w->local.kv_capacity = R;
  w->local.max_ctx_len = R;
  w->local.window = W;
  w->local.topk = 0;
  w->local.select_mode = HS2_SELECT_TOKEN;
  const hs2_status sl = validate_desc(&w->local);
  if (sl != HS2_OK) return sl;
  const size_t a = make_layout(d).total, b = make_layout(&w->local).total;
  const int64_t n_sel = (int64_t)d->batch * d->q_len * d->n_kv_heads;
  w->attn = std::max(a, b);
  w->off_idx = align_up(w->attn);
  w->off_out = align_up(w->off_idx + (size_t)n_sel * W * sizeof(int32_t));
  w->total = align_up(w->off_out + (size_t)d->batch * d->q_len * d->n_q_heads * kHeadDim * sizeof(float));
  return HS2_OK;
}

}  // namespace

HS2_API hs2_status hs2_sparse_attn_swa_workspace_size(const hs2_attn_desc* desc, int32_t local_window,
                                                      int32_t local_rows, size_t* bytes) {
  SwaWs w;
  const hs2_status s = swa_layout(desc, local_window, local_rows, &w);
  if (s != HS2_OK) return s;
  if (bytes == nullptr) return HS2_ERR_INVALID_ARG;
  *bytes = w.total;
  return HS2_OK;
}

HS2_API hs2_status hs2_sparse_attn_swa(const hs2_attn_desc* desc, const void* q, const void* k,
                                       const void* v, const float* k_scale, const float* v_scale,
                                       const int32_t* ctx_len, const int32_t* idx, const void* k_local,
                                       const void* v_local, const float* kl_scale, const float* vl_scale,
                                       int32_t local_window, int32_t local_rows, float* out,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  SwaWs w;
  hs2_status s = swa_layout(desc, local_window, local_rows, &w);
  if (s != HS2_OK) return s;
  if (!workspace) return HS2_ERR_INVALID_ARG;
  if (!aligned(workspace, 16)) return HS2_ERR_ALIGNMENT;
  if (workspace_bytes < w.total) return HS2_ERR_WORKSPACE;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  int32_t* idx_local = reinterpret_cast<int32_t*>(ws + w.off_idx);
  float* out_local = reinterpret_cast<float*>(ws + w.off_out);
  // every check of both branches before anything is enqueued
  Layout Ls, L;   // the shared branch's layout, the local one's
  s = check_common(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, workspace, w.attn, &Ls);
  if (s != HS2_OK) return s;
  s = check_common(&w.local, q, k_local, v_local, kl_scale, vl_scale, ctx_len, out_local, idx_local,
                   workspace, w.attn, &L);
  if (s != HS2_OK) return s;

  const int64_t n_sel = (int64_t)desc->batch * desc->q_len * desc->n_kv_heads;
  // Decode sizes (the one-launch sparse layer, no route forced): both branches in one
  // launch, the window rows derived in the kernel, the outputs added there.  The same
  // arithmetic as the three-step form below with HS2_FLAG_SPARSE_HEAD.
  const bool forced = has_flag(desc, HS2_FLAG_SPARSE_FUSED) || has_flag(desc, HS2_FLAG_SPARSE_SPLIT) ||
                      has_flag(desc, HS2_FLAG_SPARSE_HEAD);
  if (!forced && n_sel < kHeadPathRows && local_window <= kMaxHeadPathS) {
    ScanArgs sa = scan_args(desc, Ls, q, k, v, k_scale, v_scale, ctx_len, ws);
    sa.idx = idx;
    SwaBranch sw{};
    sw.k = static_cast<const uint8_t*>(k_local);
    sw.v = static_cast<const uint8_t*>(v_local);
    sw.k_scale = kl_scale;
    sw.v_scale = vl_scale;
    sw.W = local_window;
    sw.R = local_rows;
    const bool fp8 = desc->kv_dtype == HS2_KV_FP8_E4M3FN;
    return launch_sparse_head_swa(sa, n_sel, out, fp8, sw, stream) == hipSuccess ? HS2_OK : HS2_ERR_LAUNCH;
  }
  // 1. the block-selected rows of the shared cache
  s = sparse_impl(desc, q, k, v, k_scale, v_scale, ctx_len, idx, out, workspace, w.attn, stream, 0, nullptr);
  if (s != HS2_OK) return s;
  // 2. the separate sliding-window branch over the layer's own local cache
  if (launch_swa_rows(ctx_len, idx_local, n_sel, desc->q_len, desc->n_kv_heads, local_window, local_rows,
                      desc->max_ctx_len, stream) != hipSuccess)
    return HS2_ERR_LAUNCH;
  s = sparse_impl(&w.local, q, k_local, v_local, kl_scale, vl_scale, ctx_len, idx_local, out_local,
                  workspace, w.attn, stream, 1, nullptr);
  if (s != HS2_OK) return s;
  // 3. the two branches' outputs summed
  if (launch_add(out, out_local, (int64_t)desc->batch * desc->q_len * desc->n_q_heads * kHeadDim,
                 stream) != hipSuccess)
    return HS2_ERR_LAUNCH;
  return HS2_OK;
}
