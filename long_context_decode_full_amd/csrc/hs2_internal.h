// Internal interface between the C-ABI host layer (hs2_api.cpp) and the HIP
// kernels.  Host-visible argument structs plus one launcher per kernel; every
// launcher enqueues on the given stream and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hs2 {

constexpr int kHeadDim = 128;
constexpr int kSlots = 8;             // head slots per KV group handled by one wave
constexpr int kMaxHeads = 32;         // query heads per KV head (G) at most; per-row (M, 1/Z)
                                      // statistics keep kMaxHeads slots
// Head slots of the block comparator's per-block sums: the group size rounded up to 8,
// 16 or 32 (the head layouts of the scans and of the chunk kernel).
constexpr int blse_heads_of(int G) { return G <= 8 ? 8 : G <= 16 ? 16 : 32; }
constexpr int kPartStride = 132;      // floats per (split, head) partial: m, z, pad, pad, o[128]
constexpr int kHist1Bins = 2048;      // score bits 30..20
constexpr int kHist2Bins = 4096;      // score bits 19..8
constexpr int kHist3Bins = 256;       // score bits 7..0
constexpr int kBoundaryCap = 4096;    // boundary-bin entries resolved by one sort
constexpr int kStateWords = 16;       // u32 per selection state
// Record-based selection (default token-mode path).
constexpr int kSelectChunkLen = 4096; // positions per workgroup in the selection passes
constexpr int kFastBins = 1024;       // histogram of the record keys (top 10 of 16 bits)
constexpr int kFastShift = 6;
constexpr int kHistMergeSplits = 16;  // per-split histograms summed by one combine workgroup
constexpr int kCandChunkLen = 16384;  // record path: most positions per candidate workgroup
constexpr int kMinCandChunkLen = 2048;  // fewest (a power of two in between is chosen per call)
constexpr int kTwoStepMinRows = 256;  // record path: rows from which candidates take two kernels
constexpr int kMaxFastChunks = 8192;  // positions per row <= kMaxFastChunks * kCandChunkLen
// Per-selection control block (u32 words): [0,16) state, [16,20) pass tickets,
// [32, 32+2048) first histogram.  The logits path clears it in the combine kernel.
// The record path keeps the merged key histogram at [32, 32+kFastBins) and, after it,
// the kFastSubBins-way histogram of the keys inside the threshold bin; its scan clears
// those kMergedWords words.
constexpr int kSelCounterOff = 16;
constexpr int kSelHist1Off = 32;
constexpr int kSelWords = kSelHist1Off + (kFastBins > kHist1Bins ? kFastBins : kHist1Bins);
constexpr int kFastSubBins = 1 << kFastShift;  // key values per histogram bin
constexpr int kSelSubOff = kSelHist1Off + kFastBins;
constexpr int kMergedWords = kFastBins + kFastSubBins;
static_assert(kSelSubOff + kFastSubBins <= kSelWords, "control block too small");
constexpr int kMaxBlocksLds = 16384;  // block mode: blocks per row held in LDS
constexpr int kBlockMassBlocks = 256; // block mode on block sums: blocks per mass workgroup
constexpr int kMaxBlockPick = 4096;   // ... candidate keys per row held by the pick wave
constexpr int kMaxBlockMassWgs = 256; // ... and mass workgroups per row (4 lists a lane)
constexpr int kMaxRecordSplit = 16384; // records mode: positions per scan workgroup (LDS bound)

// Per-selection state words (u32).
enum StateWord {
  kStTakeAll = 0,    // 1: candidates <= topk, every candidate is selected
  kStResolved = 1,   // 1: boundary bin small enough (or all bits fixed)
  kStPrefix = 2,     // fixed high bits of the threshold key
  kStPrefixLen = 3,  // number of fixed bits below the sign bit (11, 23, 31)
  kStAbove = 4,      // candidates whose key prefix is strictly greater
  kStInBin = 5,      // candidates in the threshold bin
  kStWinCount = 6,   // collect: winners appended
  kStBndCount = 7,   // collect: boundary entries appended (may exceed the cap)
  kStKK = 8,         // number of global positions to select
  kStFastBin = 10,   // record path: histogram bin of the k-th largest record key
  kStFastAbove = 11, // record path: records in the bins above it
};

struct ScanArgs {
  const uint16_t* q;        // [B, Lq, Hq, D] bf16 bits
  const uint8_t* k;         // [B, Hkv, cap, D] bf16 bits or e4m3fn codes
  const uint8_t* v;
  const float* k_scale;     // [B, Hkv, cap] (fp8 only)
  const float* v_scale;
  const int32_t* ctx_len;   // [B]
  const int32_t* idx;       // sparse mode: [n_sel, S]
  float* logits;            // logits mode: [n_sel, logit_stride, 8] log2-domain logits
  uint16_t* records;        // records mode: [n_sel, logit_stride] binary16 bound records
  uint16_t* hist_part;      // records mode: [n_sel, n_split, kFastBins] key histograms
  uint32_t* hist_merged;    // records mode: merged histograms at + sel*kSelWords + kSelHist1Off,
                            // cleared by split 0 of each selection
  float* blse;              // block mode: [n_sel, blse_stride, 8] log2 of the sum of 2^logit
                            // over each aligned block of positions, per head (64 positions
                            // from the chunk kernel, 32 from the decode scan)
  int64_t blse_stride;
  int32_t window;           // records mode: positions >= ctx - window are not candidates
  float* part;              // [n_sel, n_split, G, kPartStride]
  int64_t cap;              // rows per (sequence, KV head)
  int64_t ctx_max;          // ctx_len[] is clamped to [0, ctx_max] (ctx_max <= cap)
  int64_t logit_stride;
  int32_t Lq, Hq, Hkv, G;
  int32_t S;                // sparse mode: index row length
  int32_t n_split;
  int32_t split_len;        // positions per split (dense: tokens, sparse: idx entries)
  float scale_log2;         // sm_scale * log2(e)
  int32_t fixed_steps;      // matrix-core scan: 1 = fixed step share per wave (bitwise
                            // reproducible), 0 = waves take steps from a shared counter
  int32_t slot_rows;        // sparse mode: 1 = index entries are rows of a local cache, taken
                            // when 0 <= entry < cap (no visibility limit); 0 = positions < n
  int32_t exact_pv;         // chunk kernel, bf16 caches: 1 = P V always with the two-part bf16
                            // split of P; 0 = fp16 V and P where the tile's V fits fp16
};

struct CombineArgs {
  const float* part;        // [n_sel, n_split, G, kPartStride]
  float* out;               // [B, Lq, Hq, D]
  float* mz;                // [n_sel, kMaxHeads, 2] (M, 1/Z) or nullptr
  uint32_t* sel_zero;       // selection words to clear per selection, or nullptr
  int32_t sel_zero_words;   // words per selection in sel_zero
  const uint16_t* hist_part;  // records mode: per-split key histograms to merge, or nullptr
  uint32_t* hist_out;       // merged histogram of selection `sel` at hist_out + sel*kSelWords
                            // + kSelHist1Off (atomic sums into words the scan cleared)
  int32_t hist_only;        // launch-internal: blockIdx.y indexes histogram groups only
  int32_t n_sel, Hkv, G, Hq, n_split;
  // context scans: a row folds only the splits that hold its visible positions
  // (ceil(n / split_len)); the others may be unwritten.  nullptr: every split.
  const int32_t* ctx_len;
  int64_t ctx_max;
  int32_t Lq, split_len;
};

struct SelectArgs {
  const float* logits;      // [n_sel, logit_stride, 8]
  const float* mz;          // [n_sel, kMaxHeads, 2]
  float* s;                 // [n_sel, s_stride] group-summed probabilities
  int64_t s_stride;
  int64_t logit_stride;
  const int32_t* ctx_len;
  int64_t ctx_max;          // ctx_len[] is clamped to [0, ctx_max]
  uint32_t* selblk;         // [n_sel, kSelWords] control blocks
  uint32_t* hist2;          // [n_sel, kHist2Bins]
  uint32_t* hist3;          // [n_sel, kHist3Bins]
  int32_t* winners;         // [n_sel, topk]
  uint2* boundary;          // [n_sel, kBoundaryCap] (score bits, position)
  int32_t* idx;             // [n_sel, S]
  int32_t n_sel, Lq, Hkv, G;
  int32_t window, topk, S;
  int32_t block_size, n_blocks;
  int32_t chunk_len;        // positions per workgroup in the streaming passes
  int32_t n_chunks;
  int32_t with_hist;        // token mode: build the first histogram
  const float* blse;        // block mode from the scans' block sums, else nullptr
  int64_t blse_stride;
  int32_t blse_gran;        // positions per block sum (32 or 64; divides block_size)
  uint64_t* bcand;          // block sums, many blocks: [n_sel, bm_wgs, n_blocks] candidate
                            // keys of the mass workgroups (see block_mass_kernel), or nullptr
  int32_t bm_wgs;           // mass workgroups per row (kBlockMassBlocks blocks each)
};

struct FastSelArgs {
  const uint16_t* records;  // [n_sel, rec_stride] binary16 bound records
  int64_t rec_stride;
  const float* mz;          // [n_sel, kMaxHeads, 2] (M, 1/Z)
  const int32_t* ctx_len;
  int64_t ctx_max;
  uint32_t* selblk;         // [n_sel, kSelWords]
  uint64_t* cand_keys;      // [n_sel, n_chunks, chunk_len] candidate keys: fp32 bits of the
                            // exact score (+inf when certainly selected) << 32 | (2^31-1-position)
  int32_t* cand_count;      // [n_sel, n_chunks]
  int32_t* idx;             // [n_sel, S]
  const uint16_t* q;        // full-layer queries (exact re-score)
  const uint8_t* k;
  const float* k_scale;
  int64_t cap;
  float scale_log2;
  int32_t n_chunks;
  int32_t chunk_len;        // positions per candidate chunk (power of two, 2048..16384)
  int32_t cand_wgs;         // candidate workgroups per row (each takes every cand_wgs-th chunk)
  int32_t n_sel, Lq, Hq, Hkv, G;
  int32_t window, topk, S;
};

// KV Bridging projection: Y = X W^T for one source hidden state and every target
// layer of the call, rounded (bf16) or quantised (E4M3FN + per-row scale) and
// written to cache row (seq[t], KV head, pos[t]) of the target layer.
constexpr int kMaxBridgeLayers = 16;
constexpr int kMaxDecodeSparse = 8;     // sparse layers per Hybrid Block in one decode step
struct BridgeArgs {
  const uint16_t* x;        // [T, Hd] bf16
  const uint16_t* w;        // [L * 2 * Hkv * 128, Hd] bf16 (W_k,l then W_v,l per layer)
  const int32_t* seq;       // [T]
  const int32_t* pos;       // [T]
  void* kc[kMaxBridgeLayers];   // [B, Hkv, cap, 128] per target layer
  void* vc[kMaxBridgeLayers];
  float* ks[kMaxBridgeLayers];  // [B, Hkv, cap] (fp8 caches)
  float* vs[kMaxBridgeLayers];
  int64_t cap;
  int32_t T, Hd, Hkv, B, n_layers;
  int32_t m_tiles, n_tiles;     // token tiles x feature tiles of the launch
  int32_t gemv;                 // 1: decode-size path (one workgroup per 128 features x 16 tokens)
};
constexpr int kBridgeGemvMaxTokens = 16;   // default largest T of the decode-size path
int bridge_tile_tokens(int n_tokens);   // tokens per workgroup tile launch_bridge uses
hipError_t launch_bridge(const BridgeArgs& a, bool fp8, hipStream_t st);
// decode step: pos[b] = ctx_len[b] and ctx_len[b] += 1 (pos -1 and no change once the
// length has reached `limit`, the attention calls' max_ctx_len)
hipError_t launch_advance(int32_t* ctx_len, int32_t* seq, int32_t* pos, int B, int64_t limit,
                          hipStream_t st);

// first-generation sparse layer: local-cache rows of every selection row's window, and
// out += add (n floats, a multiple of 4)
hipError_t launch_swa_rows(const int32_t* ctx_len, int32_t* idx, int64_t n_sel, int Lq, int Hkv, int W,
                           int R, int64_t ctx_max, hipStream_t st);
hipError_t launch_add(float* out, const float* add, int64_t n, hipStream_t st);

// hs2_full_attn_select_noalloc: the device address of the calling thread's current
// GPU's copy of the library's scratch array (taken once per device, then cached)
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// Events bound to one kernel launch (the timed entry points): the launch takes them
// through hipExtLaunchKernelGGL, so they carry that kernel's own start and end times
// (no dispatch or completion latency in between).  Either may be null.
struct KernelEvents {
  hipEvent_t begin;
  hipEvent_t end;
};

hipError_t launch_fast_candidates(const FastSelArgs& a, bool fp8, hipStream_t st);
hipError_t launch_fast_final(const FastSelArgs& a, hipStream_t st);
// probs (s of every visible position) for G > 8: the exact re-score of every position
// (uses q, k, k_scale, mz, ctx_len, ctx_max, cap, scale_log2, n_sel, Lq, Hq, Hkv, G)
hipError_t launch_probs_wide(const FastSelArgs& a, float* probs, int64_t probs_stride, bool fp8, hipStream_t st);
hipError_t launch_scan_dense(const ScanArgs& a, bool fp8, bool records, int B, hipStream_t st,
                             const KernelEvents* ev = nullptr);
hipError_t launch_scan_mfma(const ScanArgs& a, bool fp8, int B, hipStream_t st, const KernelEvents* ev = nullptr);
// The decode scan in block-comparator mode: per-32-position block sums into a.blse (G <= 8).
hipError_t launch_scan_mfma_blocks(const ScanArgs& a, bool fp8, int B, hipStream_t st,
                                   const KernelEvents* ev = nullptr);
// sparse layer on the matrix cores, one workgroup per (query token, KV head, split of
// a.split_len index entries); out != nullptr (one split): normalised output, else
// partials in a.part for launch_combine (S <= 4096)
hipError_t launch_gather_mfma(const ScanArgs& a, float* out, bool fp8, int B, hipStream_t st,
                              const KernelEvents* ev = nullptr);
// query chunks (q_len > 1) on the matrix cores, bf16 or fp8 caches (chunk_mfma_kernel)
hipError_t launch_chunk_mfma(const ScanArgs& a, int B, bool fp8, hipStream_t st, const KernelEvents* ev = nullptr);
hipError_t launch_scan_sparse(const ScanArgs& a, bool fp8, int B, hipStream_t st, const KernelEvents* ev = nullptr);
// sparse layer, one 1024-thread workgroup per (query token, query head) over the
// whole index row (a.S <= kMaxHeadPathS), normalised output straight to `out`
// (n_sel = B * Lq * Hkv rows; no workspace)
constexpr int kMaxHeadPathS = 4096;
hipError_t launch_sparse_head(const ScanArgs& a, int64_t n_sel, float* out, bool fp8, hipStream_t st,
                              const KernelEvents* ev = nullptr);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
hipError_t launch_groupsum(const SelectArgs& a, hipStream_t st);
hipError_t launch_refine(const SelectArgs& a, int pass, hipStream_t st);
hipError_t launch_collect(const SelectArgs& a, hipStream_t st);
hipError_t launch_finalize(const SelectArgs& a, hipStream_t st);
hipError_t launch_block_select(const SelectArgs& a, hipStream_t st);

}  // namespace hs2
