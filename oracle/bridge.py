"""Float64 reference for the KV Bridging projection (test infrastructure only).

Source (the authority on what is computed): the HySparse2 article for MiMo-V3
(Xiaomi MiMo, reprinted by IT Home, AIHOT.vn translation with sections 01-05):
  section 02 "two-level KV sharing", KV Bridging -- every Full Attention layer of
      the Cross-Decoder builds its own KV cache from the input hidden state of the
      corresponding Full Attention layer of the Self-Decoder; each target layer
      keeps its own K and V projections, so one source hidden state can build
      different K/V for different targets.
  section 04 "prefill ends half-way" -- prefill runs the Self-Decoder, which holds
      a single Full Attention layer, plus the bridging projections; that finishes
      the KV caches of the Cross-Decoder.

Readings where the article is silent (each is listed in the design doc):
  B1 one source hidden state X [T, Hd] feeds every target layer of the call (the
     Self-Decoder has one Full Attention layer, section 04).
  B2 the projections are plain linear maps without bias, norm or rotary:
     K_l = X W_k,l^T and V_l = X W_v,l^T with W stored [Hkv * D, Hd] (output
     feature major); column block g*D .. g*D + D - 1 is KV head g.
  B3 the K/V rows of token t go to cache row (seq[t], g, pos[t]) of every KV head
     g of every target layer; a token with seq outside [0, B) or pos outside
     [0, cap) is skipped, and every other cache row keeps its contents.
  B4 bf16 caches hold the projection rounded to nearest-even bfloat16.  fp8
     caches hold OCP E4M3FN codes with one fp32 scale per (token, KV head) row:
     scale = max|row| / 448 (1 when the row is all zero), code = the nearest
     E4M3FN value of row / scale, ties to the even code, saturated at +-448; the
     row reads back as code value x scale, which is how the decode path reads an
     fp8 cache.
  B5 rounding decisions are taken in fp32, the accumulation precision of the
     projection: the float64 projection is rounded to fp32 first, and max, the
     scale and the division are fp32 operations (correctly rounded), as a fused
     kernel evaluates them.

Parity status: every function here is pinned in tests/test_oracle_bridge_pins.py
(format definitions against torch's independent casts and hand-made tie and
saturation cases, the projection against brute-force loops, the scatter against
a per-element brute force); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .hybrid_block import bf16_to_f64, e4m3fn_table

E4M3FN_MAX = 448.0

_E4M3 = e4m3fn_table()
# non-negative finite E4M3FN values in increasing order with their codes (0x00 .. 0x7E)
_POS_CODES = np.arange(0x00, 0x7F, dtype=np.int64)
_POS_VALS = _E4M3[_POS_CODES]
assert np.all(np.diff(_POS_VALS) > 0)


# --------------------------------------------------------------------------- rounding to formats
def bf16_rne(x32) -> np.ndarray:
    """fp32 -> bfloat16 bits, round to nearest, ties to even (IEEE 754 roundTiesToEven
    applied to the 8-bit significand of bfloat16).  The two candidates are the
    fp32 value truncated to its top 16 bits and the next bfloat16 away from zero;
    the nearer one wins, a tie goes to the candidate whose last kept bit is 0.
    NaN -> 0x7FC0.  Values that round past the largest bfloat16 become infinity."""
    x = np.ascontiguousarray(x32, dtype=np.float32)
    u = x.view(np.uint32).astype(np.int64)
    sign = u & 0x80000000
    mag = u & 0x7FFFFFFF
    lo = mag & 0x7FFF0000                       # truncation (toward zero)
    rem = mag - lo                              # the 16 dropped bits
    up = (rem > 0x8000) | ((rem == 0x8000) & (((lo >> 16) & 1) == 1))
    res = (lo + np.where(up, 0x10000, 0)) | sign
    res = np.where(np.isnan(x), 0x7FC0, res)
    return (res >> 16).astype(np.uint16)


def e4m3fn_encode(x32) -> np.ndarray:
    """fp32 -> OCP E4M3FN code: the nearest finite E4M3FN value, ties to the code with
    an even last mantissa bit, magnitudes beyond 448 saturate to +-448 (codes 0x7E /
    0xFE); the sign is kept, also for zero; NaN -> 0x7F.  Comparisons are exact:
    a value below the midpoint (a + b) / 2 of its two neighbours rounds down."""
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    j = np.clip(np.searchsorted(_POS_VALS, a, side="right") - 1, 0, len(_POS_VALS) - 1)
    lo_v = _POS_VALS[j]
    hi_j = np.minimum(j + 1, len(_POS_VALS) - 1)
    hi_v = _POS_VALS[hi_j]
    mid2 = lo_v + hi_v                          # twice the midpoint, exact in float64
    lo_c = _POS_CODES[j]
    hi_c = _POS_CODES[hi_j]
    pick_hi = (2.0 * a > mid2) | ((2.0 * a == mid2) & ((lo_c & 1) == 1))
    code = np.where(pick_hi, hi_c, lo_c)
    code = np.where(a >= E4M3FN_MAX, 0x7E, code)   # saturation
    code = code | np.where(neg, 0x80, 0)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows(y32) -> tuple:
    """Reading B4/B5: per-row E4M3FN quantisation of fp32 rows [..., D].
    Returns (codes uint8 [..., D], scales float32 [...])."""
    y = np.asarray(y32, dtype=np.float32)
    amax = np.abs(y).max(axis=-1)
    scale = (amax / np.float32(E4M3FN_MAX)).astype(np.float32)      # fp32 division
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    q = (y / scale[..., None]).astype(np.float32)                     # fp32 division
    return e4m3fn_encode(q), scale


# --------------------------------------------------------------------------- the projection
def project(x_bits, w_bits) -> np.ndarray:
    """Reading B2: Y = X W^T for bf16 X [T, Hd] and bf16 W [N, Hd], exact products and
    float64 sums (a plain matmul of the decoded values)."""
    X = bf16_to_f64(x_bits)
    W = bf16_to_f64(w_bits)
    return X @ W.T


def kv_bridge(x_bits, w_bits, seq, pos, caches: dict) -> dict:
    """KV Bridging for n_layers target layers from one source hidden state (B1-B5).

    x_bits  [T, Hd] uint16 bf16 bits of the source hidden state
    w_bits  [L, 2, Hkv * D, Hd] uint16 bf16 bits: W_k,l then W_v,l of target layer l
    seq, pos [T] int: destination sequence and cache position of each token
    caches  {"k": [L, B, Hkv, cap, D], "v": same, and for fp8 "k_scale"/"v_scale":
             [L, B, Hkv, cap] float32}; uint16 arrays are bf16 caches, uint8 fp8 ones.
    Returns new arrays (the inputs are not modified)."""
    out = {key: np.array(val, copy=True) for key, val in caches.items() if val is not None}
    L, two, N, Hd = w_bits.shape
    assert two == 2
    Lc, B, Hkv, cap, D = out["k"].shape
    assert Lc == L and N == Hkv * D
    fp8 = out["k"].dtype == np.uint8
    seq = np.asarray(seq, dtype=np.int64)
    pos = np.asarray(pos, dtype=np.int64)
    keep = (seq >= 0) & (seq < B) & (pos >= 0) & (pos < cap)
    rows = np.nonzero(keep)[0]
    if rows.size == 0:
        return out
    Y = project(x_bits[rows], w_bits.reshape(L * 2 * N, Hd))          # [T', L*2*N]
    Y32 = Y.astype(np.float32).reshape(rows.size, L, 2, Hkv, D)        # B5: fp32 first
    for l in range(L):
        for which, name in ((0, "k"), (1, "v")):
            y = Y32[:, l, which]                                       # [T', Hkv, D]
            if fp8:
                codes, scales = quantize_rows(y)
                out[name][l, seq[rows], :, pos[rows]] = codes
                out[name + "_scale"][l, seq[rows], :, pos[rows]] = scales
            else:
                out[name][l, seq[rows], :, pos[rows]] = bf16_rne(y)
    return out
