/*
 * hs2.h -- C ABI of the HySparse2 Hybrid-Block decode library for MI355X (gfx950).
 *
 * What it computes (HySparse2 article, Xiaomi MiMo, reprinted by IT Home; the
 * AIHOT.vn translation numbers its sections 01-05):
 *   section 02, "KV Reuse": a Hybrid Block is one Full Attention layer followed
 *     by several Sparse Attention layers.  While the full layer computes its own
 *     output it picks important positions from its attention scores, and the
 *     sparse layers reuse its KV cache and its index set.
 *   section 03: selection is per token (not per block).  The 128 most recent
 *     tokens are always kept, plus 1,024 global tokens from outside that window,
 *     and both go through one sparse attention computation over the shared cache.
 * The article does not say how scores become a selection.  This library takes,
 * per KV head, the softmax probabilities of the full layer (normalised over
 * every visible position) summed over the query heads of that KV head's GQA
 * group, and keeps the top-k of them with ties going to the lower position.
 *
 * Conventions shared by every call
 *   - Pointers named q, k, v, k_scale, v_scale, ctx_len, idx, out, probs and
 *     workspace are DEVICE pointers; `desc` and `bytes` are HOST pointers.
 *   - The caller allocates and owns every buffer, including the workspace.  The
 *     library allocates nothing, never synchronises, and keeps no pointer after
 *     a call returns.  Work is enqueued on `stream`; buffers must stay valid
 *     until the stream has executed it.
 *   - Every argument is checked on the host before anything is enqueued.  A
 *     failed check returns its status and enqueues nothing.  A launch failure
 *     returns HS2_ERR_LAUNCH.  Nothing is printed and nothing aborts.
 *   - The library keeps no state between calls (no globals, no environment
 *     reads): everything a call does follows from its arguments, so it is
 *     reentrant; concurrent calls on different streams need distinct
 *     workspaces and outputs.
 *
 * Layouts (row-major; B batch, Lq query tokens per sequence, Hq query heads,
 * Hkv KV heads, G = Hq / Hkv, D = head_dim = 128, cap = kv_capacity,
 * S = window + topk in token mode or block_size * n_blocks in block mode):
 *   q        [B, Lq, Hq, D]    bfloat16                               16-B aligned
 *   k, v     [B, Hkv, cap, D]  bfloat16, or OCP E4M3FN bytes          16-B aligned
 *   k_scale, v_scale [B, Hkv, cap] float32, one per token (E4M3FN only; NULL for bf16)
 *   ctx_len  [B] int32: visible positions of sequence b, INCLUDING its Lq query
 *            tokens, which occupy positions ctx_len[b]-Lq .. ctx_len[b]-1.  Query
 *            token j sees positions [0, ctx_len[b]-Lq+j] (causal inside the chunk).
 *            Values are clamped to [0, max_ctx_len] on the device (max_ctx_len is
 *            the descriptor's host-side bound; values above it are a caller error).
 *   out      [B, Lq, Hq, D]    float32                                16-B aligned
 *   idx      [B, Lq, Hkv, S]   int32, ascending positions, -1 padding at the end
 *   probs    [B, Lq, Hkv, cap] float32 group-summed probabilities (optional)
 */
#ifndef HS2_H
#define HS2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hs2_status {
  HS2_OK = 0,
  HS2_ERR_INVALID_ARG = 1,   /* null pointer, bad size or inconsistent descriptor    */
  HS2_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim != 128, G > 32 ..)*/
  HS2_ERR_WORKSPACE = 3,     /* workspace_bytes smaller than hs2_workspace_size()      */
  HS2_ERR_ALIGNMENT = 4,     /* a device pointer is not aligned as required            */
  HS2_ERR_LAUNCH = 5,        /* the HIP runtime refused a launch                        */
  HS2_ERR_SCRATCH_LIMIT = 6  /* hs2_full_attn_select_noalloc: the call needs more scratch
                                than HS2_NOALLOC_SCRATCH_BYTES                          */
} hs2_status;

enum { HS2_KV_BF16 = 0, HS2_KV_FP8_E4M3FN = 1 };
enum { HS2_SELECT_TOKEN = 0, HS2_SELECT_BLOCK = 1 };

typedef struct hs2_attn_desc {
  int32_t batch;          /* B >= 1                                                    */
  int32_t q_len;          /* Lq >= 1: 1 at decode, e.g. 64 for an appended chunk       */
  int32_t n_q_heads;      /* Hq                                                         */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 and G = Hq / Hkv <= 32                   */
  int32_t head_dim;       /* must be 128                                                */
  int32_t kv_dtype;       /* HS2_KV_BF16 or HS2_KV_FP8_E4M3FN                            */
  int64_t kv_capacity;    /* cap: rows allocated per (sequence, KV head)                */
  int64_t max_ctx_len;    /* host-side upper bound of ctx_len[]; Lq <= max_ctx_len <= cap */
  int32_t window;         /* forced recent window, 128 in the article (>= 0)            */
  int32_t topk;           /* global tokens outside the window, 1,024 in the article     */
  int32_t select_mode;    /* HS2_SELECT_TOKEN, or HS2_SELECT_BLOCK (comparator)          */
  int32_t block_size;     /* block mode only: positions per block (64)                   */
  int32_t n_blocks;       /* block mode only: blocks kept (18)                           */
  float sm_scale;         /* softmax scale, normally 1/sqrt(head_dim); must be > 0       */
  /* Options.  A zero-initialised tail gives the defaults; every value below changes
   * only how the work is split or which kernels run, never what is computed (up to
   * fp32 summation order in `out`; idx is the same).  All are part of the descriptor,
   * so hs2_workspace_size and the calls always agree on the workspace layout. */
  uint32_t flags;         /* HS2_FLAG_* bits                                             */
  int32_t split_len;      /* positions per context-scan workgroup: 0 = automatic, else
                             rounded up to a multiple of 256 (kernel limits applied)      */
  int32_t sparse_split_len; /* index entries per sparse-gather workgroup: 0 = automatic,
                             else rounded up to a multiple of 32                          */
  int32_t cand_workgroups;  /* candidate-stage workgroups over all selection rows:
                             0 = automatic (4096; from 256 rows on, 2 per row), else at
                             least one per row                                            */
} hs2_attn_desc;

/* hs2_attn_desc.flags */
enum {
  /* Fixed step shares in the context scan.  By default the waves of a scan workgroup
   * take steps from a shared counter, so the order in which a head's probabilities are
   * summed into `out` varies between runs and `out` of hs2_full_attn_select can differ
   * in the last fp32 bits (idx never does).  With this flag `out` is bitwise
   * reproducible; the scan is ~3% slower. */
  HS2_FLAG_DETERMINISTIC = 1u << 0,
  /* Selection on the logits path (every logit kept; token mode: exact radix select,
   * block mode: block sums of the per-position s) even when probs is NULL.  For
   * comparing the selection paths (up to 8 query heads per KV head).  Without it, block
   * mode sums the blocks inside the context scan. */
  HS2_FLAG_FORCE_LOGITS = 1u << 1,
  /* The record path's context scan on the VALU kernel (dot2 + DPP) instead of the
   * matrix cores (block mode: the logits path).  For comparing the two scans. */
  HS2_FLAG_SCAN_VALU = 1u << 2,
  /* Query chunks (q_len > 1) run the decode scan once per query token instead of the
   * matrix-core chunk kernel. */
  HS2_FLAG_CHUNK_PER_TOKEN = 1u << 3,
  /* Sparse layers (rows = batch * q_len * n_kv_heads): one workgroup per (token, KV
   * head) gathering the whole index row (SPARSE_FUSED, the default from 256 rows); the
   * split gather + combine (SPARSE_SPLIT, the default from 64 rows); one workgroup per
   * (token, query head) gathering its KV head's whole index row, no combine launch
   * (SPARSE_HEAD, the default below 64 rows).  Setting more than one is
   * HS2_ERR_INVALID_ARG. */
  HS2_FLAG_SPARSE_FUSED = 1u << 4,
  HS2_FLAG_SPARSE_SPLIT = 1u << 5,
  HS2_FLAG_SPARSE_HEAD = 1u << 6,
  /* Query chunks on the matrix-core chunk kernel: P V with P split into a bf16 high
   * part and a bf16 residual (two MFMAs, error ~2^-16 relative per product), the form
   * the decode scan always uses.  By default a chunk stages V as fp16 (bf16 values
   * exactly within fp16's range; fp8 codes times their row's scale, rounded once) and
   * rounds P to fp16 (one MFMA, error <= 2^-12 relative per product); a split whose V
   * lies outside that range takes the two-part form anyway.  idx never depends on this
   * flag. */
  HS2_FLAG_EXACT_PV = 1u << 7
};
#define HS2_FLAGS_ALL 0xFFu

/* Host only, touches no GPU: checks a descriptor and that `workspace_bytes` covers
 * hs2_workspace_size(desc) (HS2_ERR_WORKSPACE otherwise; pass SIZE_MAX to check the
 * descriptor alone).  Limits: head_dim == 128,
 * 1 <= G <= 32; with G > 8 (up to MQA at 32 query heads) probs come from an exact
 * re-score of every visible position after the selection, and hs2_full_attn_select
 * returns HS2_ERR_UNSUPPORTED where only the logits path (8 head slots) would serve the
 * call (block mode with HS2_FLAG_FORCE_LOGITS, HS2_FLAG_SCAN_VALU or a block_size that
 * is not a multiple of 32), window + topk <= 4096
 * (token mode), block_size in [1, 4096] and
 * block_size * n_blocks <= 4096 (block mode), 1 <= q_len <= max_ctx_len <= cap,
 * cap < 2^31, batch * q_len <= 65535, n_kv_heads <= 65535 and
 * batch * q_len * n_kv_heads (selection rows) <= 65535 * 1024; beyond these limits
 * HS2_ERR_UNSUPPORTED; unknown flag bits or negative tuning values are
 * HS2_ERR_INVALID_ARG. */
hs2_status hs2_validate(const hs2_attn_desc* desc, size_t workspace_bytes);

/* Host only: bytes of device workspace that hs2_full_attn_select and
 * hs2_sparse_attn need for this descriptor (the larger of the two).  Requesting probs,
 * or block mode, keeps 36 bytes of scores per (selection row, position); when that
 * exceeds 16 GiB (long contexts times many query tokens) those calls return
 * HS2_ERR_UNSUPPORTED and the size leaves that space out. */
hs2_status hs2_workspace_size(const hs2_attn_desc* desc, size_t* bytes);

/* The Full Attention layer of a Hybrid Block plus its selection (section 02
 * "KV Reuse"; section 03 window + global tokens).  For every sequence b, query
 * token j and query head h (KV head g = h / G):
 *   out[b,j,h]  = softmax_t(sm_scale * q[b,j,h] . K[b,g,t]) . V[b,g,t]  over visible t
 *   s[b,j,g,t]  = sum over the G heads of group g of their softmax probability at t
 *   idx[b,j,g]  = token mode: the `window` most recent visible positions plus the
 *                 `topk` positions outside the window with the largest s (ties to the
 *                 lower position; all of them if fewer), ascending, -1 padded.
 *                 block mode: the n_blocks aligned blocks with the largest sum of s over
 *                 their visible positions (ties to the lower block), expanded to visible
 *                 positions, ascending, -1 padded.  No forced window.
 * probs may be NULL; otherwise s is written there (positions >= the visible count of a
 * row are left untouched).  q/k/v/out/idx/workspace must be 16-byte aligned, probs
 * 4-byte aligned.  With ctx_len[b]-Lq+j+1 <= 0 the row's out is 0 and idx is all -1. */
hs2_status hs2_full_attn_select(const hs2_attn_desc* desc,
                                const void* q, const void* k, const void* v,
                                const float* k_scale, const float* v_scale,
                                const int32_t* ctx_len,
                                float* out, int32_t* idx, float* probs,
                                void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* One Sparse Attention layer of the Hybrid Block (section 02 "KV Reuse": same KV
 * cache, same index set; section 03: one softmax over window and global tokens).
 *   out[b,j,h] = softmax over t in idx[b,j,g] of (sm_scale * q[b,j,h] . K[b,g,t]) . V[b,g,t]
 * Entries of idx that are negative or not below the row's visible count are skipped.
 * A row with no valid entry gets out = 0.  Same alignment rules as above. */
hs2_status hs2_sparse_attn(const hs2_attn_desc* desc,
                           const void* q, const void* k, const void* v,
                           const float* k_scale, const float* v_scale,
                           const int32_t* ctx_len, const int32_t* idx,
                           float* out,
                           void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Static English text for a status; never NULL. */
const char* hs2_status_string(hs2_status status);

/* ------------------------------------------------------------ first-generation sparse layer
 * Comparator, not part of HySparse2: the sparse layer of the first-generation HySparse
 * (HySparse2 article, section 01: block-level selection by a few Full layers; section
 * 03: the recent tokens came from an independent sliding-window branch with its own
 * local KV cache built from the sparse layer's own hidden state, which HySparse2 folds
 * into the one sparse computation).  out = attention of q over the shared-cache rows
 * named by idx (as hs2_sparse_attn; normally a block-mode selection), PLUS attention of
 * q over the layer's own local K/V of the token's window: the positions
 * [max(0, n - local_window), n) of a query token that sees n positions, held in a ring
 * k_local / v_local [batch, n_kv_heads, local_rows, 128] at row p % local_rows (with
 * kl_scale / vl_scale [batch, n_kv_heads, local_rows] for fp8).  Two softmaxes; the
 * outputs are added (the article gives no gate).  local_rows >= local_window + q_len - 1
 * (so every query token of a chunk finds its whole window), local_window <= 4096.  The
 * workspace (hs2_sparse_attn_swa_workspace_size) holds the branches' scratch.  Errors
 * as hs2_sparse_attn, all returned before anything is enqueued. */
hs2_status hs2_sparse_attn_swa_workspace_size(const hs2_attn_desc* desc, int32_t local_window,
                                              int32_t local_rows, size_t* bytes);
hs2_status hs2_sparse_attn_swa(const hs2_attn_desc* desc, const void* q, const void* k,
                               const void* v, const float* k_scale, const float* v_scale,
                               const int32_t* ctx_len, const int32_t* idx, const void* k_local,
                               const void* v_local, const float* kl_scale, const float* vl_scale,
                               int32_t local_window, int32_t local_rows, float* out,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ KV Bridging
 * HySparse2 article, section 02 "two-level KV sharing" (KV Bridging: every Full
 * Attention layer of the Cross-Decoder builds its own KV cache from the input hidden
 * state of the corresponding Self-Decoder Full Attention layer, with its own K and V
 * projections) and section 04 (prefill ends once the Self-Decoder and these
 * projections have run: they finish every cache the Cross-Decoder reads).
 *
 * One call projects T rows of ONE source hidden state into the caches of n_layers
 * target layers (the Self-Decoder has a single Full Attention layer, so one source
 * feeds every target):
 *   K_l = X W_k,l^T and V_l = X W_v,l^T  (no bias, norm or rotary; fp32 accumulation)
 * and writes, for every token t and KV head g, the 128 features of head g to cache
 * row (seq[t], g, pos[t]) of layer l:
 *   bf16 caches: rounded to nearest even;
 *   fp8 caches:  OCP E4M3FN codes with one fp32 scale per (token, KV head) row,
 *                scale = max|row| / 448 (1.0 for an all-zero row),
 *                code = nearest E4M3FN value of row / scale (ties to even, at most
 *                +-448), both fp32 operations; the row reads back as code x scale,
 *                the format hs2_full_attn_select / hs2_sparse_attn read.
 *
 *   x         [T, hidden] bf16, row-major, finite values
 *   w         [n_layers, 2, n_kv_heads * 128, hidden] bf16: W_k,l then W_v,l of each
 *             layer, output-feature major (a linear layer's weight); rows
 *             g*128 .. g*128+127 of a block give KV head g
 *   seq, pos  [T] int32: destination sequence and cache position of token t; a token
 *             with seq outside [0, batch) or pos outside [0, kv_capacity) is skipped.
 *             Destinations must be distinct (two tokens writing one row race).
 *   k_caches, v_caches   HOST arrays of n_layers DEVICE pointers, each to one layer's
 *             cache [batch, n_kv_heads, kv_capacity, 128] (bf16, or E4M3FN bytes)
 *   k_scales, v_scales   HOST arrays of n_layers device pointers to the layers'
 *             [batch, n_kv_heads, kv_capacity] fp32 scales (fp8), or NULL (bf16)
 * Only the destination rows (and their scales) are written; every other byte of the
 * caches is left as it was.  x, w and the caches must be 16-byte aligned, seq, pos
 * and the scales 4-byte aligned.  The call is asynchronous on `stream`, allocates
 * nothing, keeps no pointer after it returns and needs no workspace.  Errors
 * (HS2_ERR_INVALID_ARG: a NULL pointer or layer pointer, a bad size;
 * HS2_ERR_UNSUPPORTED: head_dim != 128, hidden not a multiple of 64, more than 16
 * layers, too large a grid; HS2_ERR_ALIGNMENT; HS2_ERR_INVALID_ARG for a
 * gemv_max_tokens outside -1 .. 1024 or reserved != 0) are returned before anything is
 * enqueued; n_tokens == 0 enqueues nothing and returns HS2_OK. */
typedef struct hs2_bridge_desc {
  int32_t n_tokens;       /* T >= 0 rows of the source hidden state                      */
  int32_t hidden;         /* hidden size: a multiple of 64, at most 65536                */
  int32_t n_layers;       /* target Full layers fed by this source: 1 .. 16              */
  int32_t n_kv_heads;     /* KV heads per layer (1 for MQA)                              */
  int32_t head_dim;       /* must be 128                                                 */
  int32_t kv_dtype;       /* HS2_KV_BF16 or HS2_KV_FP8_E4M3FN                             */
  int32_t batch;          /* sequences per cache, >= 1                                    */
  int64_t kv_capacity;    /* rows per (sequence, KV head), 1 .. 2^31 - 1                  */
  /* Option (zero = default): calls of at most this many tokens take the decode-size
   * kernel (W rows streamed into registers) instead of the tile GEMM.  0 = 16 tokens,
   * -1 = never, else 1 .. 1024.  Same results either way (fp32 sums of the same
   * products in another order). */
  int32_t gemv_max_tokens;
  int32_t reserved;       /* 0                                                           */
} hs2_bridge_desc;

hs2_status hs2_kv_bridge(const hs2_bridge_desc* desc, const void* x, const void* w,
                         const int32_t* seq, const int32_t* pos,
                         void* const* k_caches, void* const* v_caches,
                         float* const* k_scales, float* const* v_scales,
                         hipStream_t stream);

/* ------------------------------------------------------------------ decode step
 * One generated token for each of `batch` sequences through the Cross-Decoder's
 * attention: HySparse2 article, section 02 (KV Bridging builds each target Full
 * layer's cache from the Self-Decoder hidden state; KV Reuse: in every Hybrid Block the
 * Full layer selects positions from its own attention scores and the Sparse layers
 * reuse its cache and selection) and section 04 (generation keeps the full network).
 * In stream order:
 *   1. pos[b] = ctx_len[b] and ctx_len[b] += 1, except that a sequence whose length
 *      has reached attn.max_ctx_len (the bound every attention call reads up to; at
 *      most the capacity) keeps its length and appends nothing -- its attention then
 *      runs over the same max_ctx_len positions again;
 *   2. hs2_kv_bridge of the batch's new source rows x [batch, hidden] into the caches
 *      of every block (block l = target layer l of w), at (b, pos[b]);
 *   3. for each block l: hs2_full_attn_select(q_full[l]) into out_full[l], idx[l],
 *      then hs2_sparse_attn(q_sparse[l * n_sparse + j], idx[l]) into
 *      out_sparse[l * n_sparse + j] for j < n_sparse.
 * `attn` describes every block's attention: q_len must be 1 and max_ctx_len bounds
 * the lengths the step may reach (grids are sized for it, so the step can be
 * captured once into a HIP graph and replayed while the contexts grow).  q_full,
 * q_sparse, k/v_caches, k/v_scales, out_full, idx and out_sparse are HOST arrays of
 * device pointers (n_blocks, or n_blocks * n_sparse, entries); layouts and
 * alignment as in the calls above.  The step allocates nothing, never synchronises,
 * and enqueues only kernels (no memset or copy nodes), so it can be captured.  Every
 * check of every call it makes is done before anything is enqueued; the workspace
 * (hs2_decode_workspace_size) holds the attention workspace plus the new tokens'
 * positions. */
typedef struct hs2_decode_plan {
  hs2_attn_desc attn;     /* per-block attention; q_len == 1                           */
  int32_t n_blocks;       /* Hybrid Blocks = bridge target layers: 1 .. 16              */
  int32_t n_sparse;       /* Sparse layers per block: 0 .. 8 (3 in the article)         */
  int32_t hidden;         /* hidden size of the bridge source rows                      */
  int32_t reserved;       /* 0                                                          */
} hs2_decode_plan;

hs2_status hs2_decode_workspace_size(const hs2_decode_plan* plan, size_t* bytes);
hs2_status hs2_decode_step(const hs2_decode_plan* plan, const void* x, const void* w,
                           const void* const* q_full, const void* const* q_sparse,
                           void* const* k_caches, void* const* v_caches,
                           float* const* k_scales, float* const* v_scales,
                           int32_t* ctx_len, float* const* out_full, int32_t* const* idx,
                           float* const* out_sparse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* ------------------------------------------------------------------ no allocation
 * For callers that cannot allocate device memory or pass a workspace: code under HIP
 * graph capture, serving loops and harnesses that forbid allocation.  Computes exactly
 * what hs2_full_attn_select computes, with the same kernels, but its scratch is one
 * static device array of HS2_NOALLOC_SCRATCH_BYTES held by the library on each GPU it
 * runs on (until the process ends); the caller passes only inputs and outputs.  The
 * scratch needed is the call's own path only (no logits area on the record path):
 * the million-token decode needs ~47 MiB; a call needing more returns
 * HS2_ERR_SCRATCH_LIMIT before anything is enqueued (as does every argument check of
 * hs2_full_attn_select).  The device is the calling thread's current HIP device, which
 * must own `stream`.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (concurrent streams, several host threads) race.  The array
 * keeps the last call's contents, which no later call reads before writing.  Calls
 * no hipMalloc, hipFree or allocating library routine. */
#define HS2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
hs2_status hs2_full_attn_select_noalloc(const hs2_attn_desc* desc,
                                        const void* q, const void* k, const void* v,
                                        const float* k_scale, const float* v_scale,
                                        const int32_t* ctx_len,
                                        float* out, int32_t* idx, float* probs,
                                        hipStream_t stream);

/* ------------------------------------------------------------------ kernel timing
 * Benchmark support without library state: the caller creates two HIP events
 * (hipEventCreate) and passes them; the call launches its dominant kernel -- the
 * context scan of hs2_full_attn_select, the gather of hs2_sparse_attn -- with
 * hipExtLaunchKernel, which sets `begin` to that kernel's start and `end` to its end,
 * so hipEventElapsedTime(begin, end) is the kernel's own duration (the dispatch and
 * completion latency around it excluded).  Either event may be NULL.  Otherwise
 * identical to the untimed calls (which are these with events == NULL).  The caller
 * owns and destroys the events. */
typedef struct hs2_kernel_events {
  hipEvent_t begin;
  hipEvent_t end;
} hs2_kernel_events;

hs2_status hs2_full_attn_select_timed(const hs2_attn_desc* desc,
                                      const void* q, const void* k, const void* v,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* ctx_len,
                                      float* out, int32_t* idx, float* probs,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream, const hs2_kernel_events* events);
hs2_status hs2_sparse_attn_timed(const hs2_attn_desc* desc,
                                 const void* q, const void* k, const void* v,
                                 const float* k_scale, const float* v_scale,
                                 const int32_t* ctx_len, const int32_t* idx,
                                 float* out,
                                 void* workspace, size_t workspace_bytes,
                                 hipStream_t stream, const hs2_kernel_events* events);

/* Static text naming the sources the library was built from (a hash of the kernel,
 * host and header files); never NULL.  Lets a caller detect a stale binary. */
const char* hs2_build_id(void);

#ifdef __cplusplus
}
#endif
#endif /* HS2_H */
