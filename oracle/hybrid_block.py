"""Float64 reference for one HySparse2 Hybrid Block at decode time (test infrastructure only).

Sources (the article is the authority on what is computed):
  "HySparse2" for MiMo-V3, Xiaomi MiMo article reprinted by IT Home (Chinese,
  Aioga page titled "小米公开 MiMo-V3 核心架构 HySparse2") and its AIHOT.vn
  translation, whose headings number the sections 01-05:
    section 02 -- KV Reuse: a Hybrid Block is one Full Attention layer followed
                  by Sparse Attention layers; the full layer picks important
                  positions from its own attention scores while computing its
                  output, and the sparse layers reuse its KV cache and index set.
    section 03 -- token-level (not block-level) selection; the 128 most recent
                  tokens are always selected, plus 1,024 global tokens from
                  outside that window; local and global tokens go through one
                  sparse attention computation over the shared KV cache.
    section 01 / 03 -- the first-generation HySparse selected whole blocks.

Readings where the article is silent (each is listed in the design doc):
  R1 score -> selection: post-softmax probabilities over all visible
     positions (window included in the normaliser), summed over the query
     heads of each KV head's group; exact top-k, ties to the lower index.
  R2 one index set per (sequence, query token, KV head).
  R3 the window includes the current token: window = [n-128, n-1].
  R4 fewer than 1,024 candidates outside the window: take them all.
  R5 query head h reads KV head h // G (contiguous GQA groups).
  R6 no soft-cap, sink, positional bias or rotary inside the path; scale 1/sqrt(D).
  R7 sparse layers: one softmax over window + selected tokens.
  R8 query token j of a Lq-token chunk sits at position ctx_len - Lq + j and
     sees positions [0, that position] (causal inside the chunk).
  R9 idx rows are ascending with -1 padding at the end.
  R10 fp8 caches: OCP E4M3FN codes; the dequantised value is code value x the
     token's fp32 scale, evaluated exactly (float64).
  R11 block baseline: aligned blocks of 64 positions, block score = sum of the
     group-summed probabilities of its visible positions, best 18 blocks (ties
     to the lower block), no forced window.
"""
from __future__ import annotations

import numpy as np


# --------------------------------------------------------------------------- number formats
def bf16_to_f64(bits) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64: the 16 bits are the high half of an IEEE binary32."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one OCP 8-bit float E4M3FN code (OCP OFP8 specification):
    1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 is
    subnormal (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3fn_table() -> np.ndarray:
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3FN = e4m3fn_table()


def dequant_fp8(codes, scales) -> np.ndarray:
    """Reading R10: value(code) * scale of its token, exactly (no intermediate rounding)."""
    codes = np.asarray(codes, dtype=np.uint8)
    return _E4M3FN[codes] * np.asarray(scales, dtype=np.float64)[..., None]


def kv_rows(inp: dict, b: int, g: int, n: int):
    """Rows [0, n) of the shared K and V caches of sequence b, KV head g, as float64."""
    if inp["k"].dtype == np.uint8:
        K = dequant_fp8(inp["k"][b, g, :n], inp["k_scale"][b, g, :n])
        V = dequant_fp8(inp["v"][b, g, :n], inp["v_scale"][b, g, :n])
    else:
        K = bf16_to_f64(inp["k"][b, g, :n])
        V = bf16_to_f64(inp["v"][b, g, :n])
    return K, V


# --------------------------------------------------------------------------- the method
def full_attention(q, K, V, sm_scale):
    """Dense attention of the G query heads of one KV group over all n visible rows
    (section 02: the Full Attention layer computes its own output).

    q [G, D], K [n, D], V [n, D] -> (out [G, D], P [G, n]) where
    l[h, t] = sm_scale * q[h] . K[t],  P[h, :] = softmax(l[h, :]),  out[h] = sum_t P[h, t] V[t].
    """
    G = q.shape[0]
    n = K.shape[0]
    if n == 0:
        return np.zeros((G, q.shape[1])), np.zeros((G, 0))
    logits = sm_scale * (q @ K.T)
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    P = e / e.sum(axis=1, keepdims=True)
    return P @ V, P


def group_scores(P):
    """Reading R1: the score of position t for a KV group is the sum over the group's
    query heads of their softmax probabilities at t.  P [G, n] -> s [n]."""
    return P.sum(axis=0)


def select_tokens(s, window: int, topk: int):
    """Section 03: keep the `window` most recent positions (R3: the current token is
    the most recent), plus the `topk` highest-scoring positions outside the window,
    ties to the lower index (R1), all of them if there are fewer (R4).

    s [n] float -> idx [window + topk] int64, ascending, -1 padded (R9).
    """
    n = len(s)
    w0 = max(0, n - window)
    win = np.arange(w0, n)
    cand = np.arange(0, w0)
    kk = min(topk, len(cand))
    # np.lexsort sorts by the last key first: primary -s (descending s), then t ascending.
    order = np.lexsort((cand, -np.asarray(s)[cand]))
    top = cand[order[:kk]]
    chosen = np.sort(np.concatenate([top, win]))
    out = np.full(window + topk, -1, dtype=np.int64)
    out[: len(chosen)] = chosen
    return out


def sparse_attention(q, K, V, idx, sm_scale):
    """Section 02 / 03: a sparse layer attends, with its own queries, over the rows of
    the shared cache named by the full layer's index set; window and global rows share
    one softmax (R7).  q [G, D], K/V [n, D] (rows 0..n-1), idx [S] with -1 pads."""
    I = np.asarray(idx)
    I = I[I >= 0]
    out, _ = full_attention(q, K[I], V[I], sm_scale)
    return out


def block_select(s, block: int, n_blocks: int):
    """First-generation block-level selection used as the comparator (sections 01 and 03
    name it; reading R11 fixes the rule).  s [n] -> idx [block * n_blocks], ascending
    positions of the chosen blocks that are visible (t < n), -1 padded."""
    n = len(s)
    nb = (n + block - 1) // block
    mass = np.array([np.sum(s[b * block: min((b + 1) * block, n)]) for b in range(nb)])
    order = np.lexsort((np.arange(nb), -mass))
    chosen = np.sort(order[: min(n_blocks, nb)])
    toks = [np.arange(b * block, min((b + 1) * block, n)) for b in chosen]
    toks = np.concatenate(toks) if toks else np.zeros(0, dtype=np.int64)
    out = np.full(block * n_blocks, -1, dtype=np.int64)
    out[: len(toks)] = toks
    return out


# --------------------------------------------------------------------------- one Hybrid Block
def hybrid_block_token(inp: dict, b: int, j: int, window=128, topk=1024, mode="token",
                       block=64, n_blocks=18, want_scores=True, groups=None, ctx_max=None,
                       kv_cache=None):
    """Everything the Hybrid Block computes for query token j of sequence b, per KV group g:
    full-layer output, group scores, index set, and each sparse layer's output.
    `groups` restricts the work to some KV groups (others are left zero / -1).
    `ctx_max`: the caller's bound on the context length (default: the capacity); a
    larger ctx_len counts as ctx_max.  `kv_cache`: optional dict g -> (K, V) of float64
    rows [0, m) of sequence b (as kv_rows returns them, m >= the visible count), so that
    several tokens of one sequence share one conversion."""
    q_full = bf16_to_f64(inp["q_full"][b, j])            # [Hq, D]
    qs = [bf16_to_f64(q[b, j]) for q in inp["q_sparse"]]
    Hq = q_full.shape[0]
    Hkv = inp["k"].shape[1]
    G = Hq // Hkv
    Lq = inp["q_full"].shape[1]
    sm = inp["sm_scale"]
    cap = inp["k"].shape[2]
    ctx = min(max(int(inp["ctx_len"][b]), 0), cap if ctx_max is None else min(int(ctx_max), cap))
    n = max(0, ctx - Lq + j + 1)                           # R8
    S = block * n_blocks if mode == "block" else window + topk
    out_full = np.zeros((Hq, q_full.shape[1]))
    out_sp = [np.zeros_like(out_full) for _ in qs]
    idx_all = np.full((Hkv, S), -1, dtype=np.int64)
    s_all = []
    for g in (range(Hkv) if groups is None else groups):
        heads = slice(g * G, (g + 1) * G)                  # R5
        if kv_cache is not None:
            K, V = kv_cache[g][0][:n], kv_cache[g][1][:n]
        else:
            K, V = kv_rows(inp, b, g, n)
        o, P = full_attention(q_full[heads], K, V, sm)
        out_full[heads] = o
        s = group_scores(P)
        idx = block_select(s, block, n_blocks) if mode == "block" else select_tokens(s, window, topk)
        idx_all[g] = idx
        if want_scores:
            s_all.append(s)
        for li, q in enumerate(qs):
            out_sp[li][heads] = sparse_attention(q[heads], K, V, idx, sm)
    return dict(out_full=out_full, idx=idx_all, s=s_all, out_sparse=out_sp, n=n)


def hybrid_block(inp: dict, tokens=None, **kw):
    """Run hybrid_block_token over `tokens` (list of (b, j)); default every token."""
    B, Lq = inp["q_full"].shape[:2]
    if tokens is None:
        tokens = [(b, j) for b in range(B) for j in range(Lq)]
    return {(b, j): hybrid_block_token(inp, b, j, **kw) for (b, j) in tokens}


def ctx_tokens(inp: dict) -> int:
    return int(np.sum(inp["ctx_len"]))

