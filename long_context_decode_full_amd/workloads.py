"""Seeded synthetic inputs for one HySparse2 Hybrid Block (full layer + sparse layers).

This module builds inputs only: query vectors, a shared K/V cache (bf16 bit
patterns, or OCP e4m3fn bytes with one fp32 scale per token), per-sequence
context lengths and planted "needle" keys.  It holds none of the attention,
probability or selection arithmetic; the CPU oracle and the HIP library both
consume what it produces.

The workloads stand in for the long-context suites the HySparse2 article
(Xiaomi MiMo, reprinted by IT Home, section 05 "lower cost, faster, better
long-text") evaluates on; no suite item is reproduced.  Planted keys aligned
with the query play the part of retrieval needles; lengths of 32k, 256k and
1M mirror the article's ablation ceiling, evaluation ceiling and cost analysis.

Layouts (row-major):
  q        [B, Lq, Hq, D]   bf16 bits (uint16)
  k, v     [B, Hkv, cap, D] bf16 bits (uint16)  or e4m3fn codes (uint8)
  k_scale, v_scale [B, Hkv, cap] float32 (fp8 caches only)
  ctx_len  [B] int32; the Lq query tokens of a sequence sit at the end of it
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
E4M3FN_NAN = np.uint8(0x7F)
E4M3FN_MAX = 448.0


@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    q_len: int
    n_q_heads: int
    n_kv_heads: int
    ctx_lens: Optional[List[int]] = None     # explicit lengths, or None for a log-uniform draw
    ctx_log_uniform: Optional[tuple] = None  # (lo, hi) for floor(exp(U(ln lo, ln hi)))
    head_dim: int = 128
    kv_dtype: str = "bf16"                   # "bf16" | "fp8"
    n_needles: int = 0                       # per (sequence, KV head)
    needle_cos: float = 0.6
    needle_scale: float = 1.0                # multiplies the needle row (1.0 = unit-variance norm)
    drift_sigma: float = 0.0                 # per-dim random walk step for keys
    drift_block: int = 4096
    n_sparse_layers: int = 3
    capacity: Optional[int] = None           # rows per (b, kv head); default max ctx
    poison_tail: bool = False                # fill rows >= ctx_len with NaN
    identical_keys: bool = False             # every key row of a (b, g) equal
    zero_q: bool = False                     # all query vectors zero
    unaligned_queries: bool = False          # full-layer queries drawn after the needles, unrelated to them
    seed: int = 0

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


def standard_workloads():
    """The five configurations (tiny decode, batched decode, fp8 long decode,
    million-token decode, the ragged 64-token chunk), the MQA variants of the
    million-token decode and of the chunk (one KV head for all 32 query heads; the
    chunk variant draws the same context lengths as the chunk configuration) and the
    chunk with fp8 caches (same lengths)."""
    return {
        "tiny": Workload("tiny decode", 1, 1, 16, 2, ctx_lens=[4096], n_needles=8, seed=1001),
        "batched": Workload("batched decode", 8, 1, 32, 4, ctx_lens=[32768] * 8, n_needles=64,
                            seed=1002),
        "fp8_256k": Workload("long-context fp8 decode", 1, 1, 32, 4, ctx_lens=[262144],
                             kv_dtype="fp8", n_needles=256, seed=1003),
        "million": Workload("million-token decode", 1, 1, 32, 4, ctx_lens=[1048576],
                            n_needles=1024, drift_sigma=0.01, drift_block=4096, seed=1004),
        "chunk": Workload("ragged 64-token chunk", 16, 64, 32, 4, ctx_log_uniform=(8192, 524288),
                          n_needles=64, seed=1005),
        "mqa_million": Workload("MQA million-token decode", 1, 1, 32, 1, ctx_lens=[1048576],
                                n_needles=1024, drift_sigma=0.01, drift_block=4096, seed=1006),
        "mqa_chunk": Workload("MQA ragged 64-token chunk", 16, 64, 32, 1, ctx_log_uniform=(8192, 524288),
                              n_needles=64, seed=1005),
        "fp8_chunk": Workload("ragged 64-token chunk, fp8 caches", 16, 64, 32, 4,
                              ctx_log_uniform=(8192, 524288), kv_dtype="fp8", n_needles=64, seed=1005),
    }


# --------------------------------------------------------------------------- encoders
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_e4m3fn_rows(x: np.ndarray):
    """Per-row symmetric quantisation: scale = max|row| / 448, code = RNE(x / scale)
    saturated to +-448.  Returns (codes uint8 [rows, D], scales float32 [rows])."""
    import torch  # the OCP e4m3fn encoder of torch's CPU cast; encoding is input preparation
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)
    scale[scale == 0] = np.float32(1.0)
    y = np.clip(x / scale[..., None], -E4M3FN_MAX, E4M3FN_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return codes, scale


# --------------------------------------------------------------------------- generator
def _ctx_lens(w: Workload, rng: np.random.Generator) -> List[int]:
    if w.ctx_lens is not None:
        assert len(w.ctx_lens) == w.batch
        return [int(c) for c in w.ctx_lens]
    lo, hi = w.ctx_log_uniform
    u = rng.uniform(math.log(lo), math.log(hi), size=w.batch)
    return [int(min(hi, max(lo, math.floor(math.exp(x))))) for x in u]


def make_inputs(w: Workload, threads: int = 8) -> dict:
    """Build every input of one Hybrid Block decode step for workload `w`.

    Streams (numpy PCG64, SeedSequence(w.seed) spawned per purpose and per
    (sequence, KV head)): keys, values, full-layer q, sparse-layer q, needle
    positions, needle directions, key drift, lengths.
    """
    B, Lq, Hq, Hkv, D = w.batch, w.q_len, w.n_q_heads, w.n_kv_heads, w.head_dim
    assert Hq % Hkv == 0
    G = Hq // Hkv
    root = np.random.SeedSequence(w.seed)
    s_k, s_v, s_qf, s_qs, s_np, s_nd, s_dr, s_len = root.spawn(8)
    ctx = _ctx_lens(w, np.random.default_rng(s_len))
    cap = int(w.capacity) if w.capacity is not None else max(ctx)
    assert cap >= max(ctx) and min(ctx) >= Lq

    def qgen(seed):
        rng = np.random.default_rng(seed)
        x = rng.standard_normal((B, Lq, Hq, D), dtype=np.float32)
        if w.zero_q:
            x[:] = 0
        return f32_to_bf16_bits(x)

    q_full = qgen(s_qf)
    q_sparse = [qgen(s) for s in s_qs.spawn(w.n_sparse_layers)]

    fp8 = w.kv_dtype == "fp8"
    kdt = np.uint8 if fp8 else np.uint16
    k = np.zeros((B, Hkv, cap, D), dtype=kdt)
    v = np.zeros((B, Hkv, cap, D), dtype=kdt)
    k_scale = np.ones((B, Hkv, cap), dtype=np.float32) if fp8 else None
    v_scale = np.ones((B, Hkv, cap), dtype=np.float32) if fp8 else None

    kseeds = s_k.spawn(B * Hkv)
    vseeds = s_v.spawn(B * Hkv)
    npos_seeds = s_np.spawn(B * Hkv)
    ndir_seeds = s_nd.spawn(B * Hkv)
    drift_seeds = s_dr.spawn(Hkv)
    qf32 = bf16_bits_to_f32(q_full).astype(np.float64)

    def drift_rows(g, n):
        if w.drift_sigma <= 0:
            return None
        nblk = (n + w.drift_block - 1) // w.drift_block
        steps = np.random.default_rng(drift_seeds[g]).normal(0.0, w.drift_sigma, size=(nblk, D))
        steps[0] = 0.0                       # D_0 = 0, D_i = D_{i-1} + N(0, sigma^2)
        walk = np.cumsum(steps, axis=0)
        return walk

    def fill(task):
        which, b, g = task
        n = ctx[b]
        i = b * Hkv + g
        rng = np.random.default_rng(kseeds[i] if which == "k" else vseeds[i])
        x = rng.standard_normal((n, D), dtype=np.float32)
        if which == "k":
            if w.identical_keys:
                x[:] = x[0]
            walk = drift_rows(g, n)
            if walk is not None:
                x += walk[np.arange(n) // w.drift_block].astype(np.float32)
            if w.n_needles > 0:
                m = min(w.n_needles, n)
                pos = np.random.default_rng(npos_seeds[i]).choice(n, size=m, replace=False)
                drng = np.random.default_rng(ndir_seeds[i])
                u = qf32[b, :, g * G:(g + 1) * G, :].sum(axis=(0, 1))
                un = np.linalg.norm(u)
                u = u / un if un > 0 else np.eye(D)[0]
                for p in pos:
                    r = drng.standard_normal(D)
                    r -= r.dot(u) * u
                    r /= np.linalg.norm(r)
                    c = w.needle_cos
                    x[p] = (w.needle_scale * math.sqrt(D) * (c * u + math.sqrt(1 - c * c) * r)).astype(np.float32)
        dst = k if which == "k" else v
        if fp8:
            codes, sc = quantize_e4m3fn_rows(x)
            dst[b, g, :n] = codes
            (k_scale if which == "k" else v_scale)[b, g, :n] = sc
            if w.poison_tail and n < cap:
                dst[b, g, n:] = E4M3FN_NAN
                (k_scale if which == "k" else v_scale)[b, g, n:] = np.nan
        else:
            dst[b, g, :n] = f32_to_bf16_bits(x)
            if w.poison_tail and n < cap:
                dst[b, g, n:] = BF16_NAN

    tasks = [(which, b, g) for which in ("k", "v") for b in range(B) for g in range(Hkv)]
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(fill, tasks))

    if w.unaligned_queries:
        # the keys (and needles) stay as built; the full layer's queries are fresh draws,
        # so no planted key stands out and the selection boundary falls among many
        # similar scores
        q_full = qgen(np.random.SeedSequence([w.seed, 7919]))
    return dict(workload=w, q_full=q_full, q_sparse=q_sparse, k=k, v=v, k_scale=k_scale,
                v_scale=v_scale, ctx_len=np.asarray(ctx, dtype=np.int32), capacity=cap,
                sm_scale=1.0 / math.sqrt(D))


# --------------------------------------------------------------------------- KV Bridging inputs
@dataclasses.dataclass
class BridgeWorkload:
    """One KV Bridging call: T source hidden-state rows projected into the K/V caches
    of n_layers target Full layers (HySparse2 article, section 02 "KV Bridging";
    section 04: prefill ends after the Self-Decoder and these projections)."""
    name: str
    n_tokens: int                    # T rows of the source hidden state
    hidden: int                      # Hd (the article gives no hidden size)
    n_layers: int                    # target Full layers fed by this source
    n_kv_heads: int
    batch: int                       # sequences held by each cache
    capacity: int                    # rows per (sequence, KV head)
    kv_dtype: str = "fp8"            # "bf16" | "fp8"
    head_dim: int = 128
    placement: str = "prefill"       # "prefill" | "decode" | "ragged"
    start: int = 0                   # prefill: position of the first token
    outlier_channels: int = 4        # hidden channels with a larger spread
    outlier_scale: float = 8.0
    bad_rows: int = 0                # tokens given an out-of-range destination
    seed: int = 0


def bridge_workloads():
    """KV Bridging cases.  The hidden size (2048) and the number of target layers (6)
    are not on the pages: 6 is (49 - 25) / (1 + 3), the Cross-Decoder's 24 layers in
    Hybrid Blocks of one Full and three Sparse layers; 2048 is a stand-in hidden size."""
    return {
        "bridge_prefill": BridgeWorkload("prefill chunk of a 1M-token context", 16384, 2048, 6, 4,
                                         batch=1, capacity=1048576, start=1048576 - 16384, seed=2001),
        "bridge_prefill_bf16": BridgeWorkload("prefill chunk, bf16 caches", 16384, 2048, 6, 4, batch=1,
                                              capacity=1048576, kv_dtype="bf16",
                                              start=1048576 - 16384, seed=2002),
        "bridge_mqa": BridgeWorkload("MQA prefill chunk", 16384, 2048, 6, 1, batch=1, capacity=1048576,
                                     start=1048576 - 16384, seed=2003),
        "bridge_decode": BridgeWorkload("batched decode append", 16, 2048, 6, 4, batch=16,
                                        capacity=32768, placement="decode", seed=2004),
        "bridge_ragged": BridgeWorkload("ragged chunk append", 1000, 512, 2, 2, batch=5, capacity=4096,
                                        placement="ragged", bad_rows=7, seed=2005),
    }


def make_bridge_inputs(w: BridgeWorkload) -> dict:
    """Source hidden state, projection weights and destinations of one bridging call.

      x        [T, Hd] bf16 bits: N(0, 1) entries, `outlier_channels` channels scaled up
      weight   [L, 2, Hkv * D, Hd] bf16 bits: N(0, 1 / Hd) (W_k then W_v per layer,
               output-feature major)
      seq, pos [T] int32 destinations; "prefill" puts the tokens of sequence 0 at
               start, start + 1, ...; "decode" gives sequence t one token at a random
               position; "ragged" splits the tokens into `batch` runs of random
               lengths at random starts; `bad_rows` tokens get an out-of-range
               sequence or position.
    """
    T, Hd, L, Hkv, D = w.n_tokens, w.hidden, w.n_layers, w.n_kv_heads, w.head_dim
    root = np.random.SeedSequence(w.seed)
    s_x, s_w, s_o, s_d, s_b = root.spawn(5)
    x = np.random.default_rng(s_x).standard_normal((T, Hd), dtype=np.float32)
    if w.outlier_channels > 0:
        ch = np.random.default_rng(s_o).choice(Hd, size=min(w.outlier_channels, Hd), replace=False)
        x[:, ch] *= np.float32(w.outlier_scale)
    wt = np.random.default_rng(s_w).standard_normal((L, 2, Hkv * D, Hd), dtype=np.float32)
    wt *= np.float32(1.0 / math.sqrt(Hd))
    rng = np.random.default_rng(s_d)
    if w.placement == "prefill":
        assert w.start + T <= w.capacity
        seq = np.zeros(T, dtype=np.int32)
        pos = (w.start + np.arange(T)).astype(np.int32)
    elif w.placement == "decode":
        assert T == w.batch
        seq = np.arange(T, dtype=np.int32)
        pos = rng.integers(0, w.capacity, size=T).astype(np.int32)
    elif w.placement == "ragged":
        cuts = np.sort(rng.choice(np.arange(1, T), size=w.batch - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [T]]))
        seq = np.repeat(np.arange(w.batch), lens).astype(np.int32)
        pos = np.concatenate([rng.integers(0, w.capacity - n + 1) + np.arange(n) for n in lens]).astype(np.int32)
    else:
        raise ValueError(w.placement)
    if w.bad_rows > 0:
        rb = np.random.default_rng(s_b)
        bad = rb.choice(T, size=min(w.bad_rows, T), replace=False)
        choices = [(-1, None), (w.batch, None), (None, -1), (None, w.capacity), (None, -(2 ** 31))]
        for i, t in enumerate(bad):
            sb, pb = choices[i % len(choices)]
            if sb is not None:
                seq[t] = sb
            if pb is not None:
                pos[t] = pb
    return dict(workload=w, x=f32_to_bf16_bits(x), weight=f32_to_bf16_bits(wt), seq=seq, pos=pos)


def bridge_cache_sentinel(kv_dtype: str):
    """Initial cache contents for bridging tests: NaN codes and NaN scales, so that a
    row written by mistake or left unwritten shows."""
    return (E4M3FN_NAN, np.float32(np.nan)) if kv_dtype == "fp8" else (BF16_NAN, None)


def make_decode_steps(w: Workload, n_blocks: int, steps: int, hidden: int, seed: int,
                      outlier_channels: int = 4, outlier_scale: float = 8.0) -> dict:
    """Per-step inputs of a multi-step decode over n_blocks Hybrid Blocks that all start
    from the caches of make_inputs(w): the bridge weights of every block and, for each
    step, the new tokens' source rows and every layer's queries.

      w_bits     [n_blocks, 2, Hkv * 128, hidden] bf16 bits, N(0, 1 / hidden)
      x[t]       [B, hidden] bf16 bits, N(0, 1) with `outlier_channels` channels scaled
      q_full[t]  n_blocks arrays [B, 1, Hq, 128] bf16 bits, N(0, 1)
      q_sparse[t] n_blocks * n_sparse arrays (block-major), N(0, 1)
    """
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    ns = w.n_sparse_layers
    root = np.random.SeedSequence(seed)
    s_w, s_x, s_q, s_o = root.spawn(4)
    wt = np.random.default_rng(s_w).standard_normal((n_blocks, 2, Hkv * D, hidden), dtype=np.float32)
    wt *= np.float32(1.0 / math.sqrt(hidden))
    ch = np.random.default_rng(s_o).choice(hidden, size=min(outlier_channels, hidden), replace=False)
    rx = np.random.default_rng(s_x)
    rq = np.random.default_rng(s_q)
    xs, qf, qs = [], [], []
    for _ in range(steps):
        x = rx.standard_normal((B, hidden), dtype=np.float32)
        x[:, ch] *= np.float32(outlier_scale)
        xs.append(f32_to_bf16_bits(x))
        qf.append([f32_to_bf16_bits(rq.standard_normal((B, 1, Hq, D), dtype=np.float32))
                   for _ in range(n_blocks)])
        qs.append([f32_to_bf16_bits(rq.standard_normal((B, 1, Hq, D), dtype=np.float32))
                   for _ in range(n_blocks * ns)])
    return dict(w_bits=f32_to_bf16_bits(wt), x=xs, q_full=qf, q_sparse=qs)


def make_local_rings(w: Workload, rows: int, seed: int) -> list:
    """The first-generation comparator's local caches: for each sparse layer a ring of
    `rows` K/V rows per (sequence, KV head) standing for the layer's own K/V of its
    most recent positions (position p at row p % rows).  N(0, 1) rows, stored like the
    shared cache (bf16 bits, or e4m3fn codes with per-row scales).  Returns a list of
    dicts with k, v (and k_scale, v_scale for fp8)."""
    B, Hkv, D = w.batch, w.n_kv_heads, w.head_dim
    out = []
    for s in np.random.SeedSequence(seed).spawn(w.n_sparse_layers):
        rk, rv = (np.random.default_rng(x) for x in s.spawn(2))
        xk = rk.standard_normal((B, Hkv, rows, D), dtype=np.float32)
        xv = rv.standard_normal((B, Hkv, rows, D), dtype=np.float32)
        if w.kv_dtype == "fp8":
            ck, sk = quantize_e4m3fn_rows(xk.reshape(-1, D))
            cv, sv = quantize_e4m3fn_rows(xv.reshape(-1, D))
            out.append(dict(k=ck.reshape(B, Hkv, rows, D), v=cv.reshape(B, Hkv, rows, D),
                            k_scale=sk.reshape(B, Hkv, rows), v_scale=sv.reshape(B, Hkv, rows)))
        else:
            out.append(dict(k=f32_to_bf16_bits(xk), v=f32_to_bf16_bits(xv), k_scale=None, v_scale=None))
    return out
