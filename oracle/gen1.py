"""Float64 reference for the first-generation HySparse sparse layer (test infrastructure
only): the comparator in which the recent tokens come from a separate sliding-window
branch over the layer's own local KV rather than from the shared cache.

Source: the HySparse2 article for MiMo-V3 (Xiaomi MiMo, reprinted by IT Home, AIHOT.vn
translation with sections 01-05):
  section 01 -- the first-generation HySparse: a few Full Attention layers hand their
      KV cache and selected positions to later Sparse Attention layers; its selection
      is block-level.
  section 03 -- in it, local information was reached by an independent SWA branch with
      its own local KV cache built from the sparse layer's own hidden state; HySparse2
      merges that local access into the one sparse computation over the shared cache.

Readings where the article is silent (listed in the design doc):
  G1 the SWA branch attends, with the sparse layer's queries, over the layer's own K/V
     of the W most recent positions [max(0, n - W), n) of the query token (W = 128,
     HySparse2's forced window, so that both methods see the same local span).
  G2 the two branches keep separate softmaxes (independent computations) and their
     outputs are added; the article gives no gate, so none is applied.
  G3 the local cache is a ring of R rows (R >= W + q_len - 1): position p sits at row
     p % R; the shared branch attends over the block-level selection (reading R11).

Parity status: pinned in tests/test_oracle_pins.py (ring rows against a linear
layout, the branch against torch's float64 scaled_dot_product_attention, the sum
against each branch alone); not "parity unpinned".
"""
from __future__ import annotations

import numpy as np

from .hybrid_block import bf16_to_f64, dequant_fp8, full_attention, sparse_attention


def local_rows(n: int, W: int, R: int) -> np.ndarray:
    """Reading G1/G3: ring rows of the positions [max(0, n - W), n), oldest first."""
    return np.arange(max(0, n - W), n, dtype=np.int64) % R


def local_kv(inp_local: dict, b: int, g: int):
    """The layer's local ring of sequence b, KV head g, as float64 [R, D]."""
    k, v = inp_local["k"], inp_local["v"]
    if k.dtype == np.uint8:
        return (dequant_fp8(k[b, g], inp_local["k_scale"][b, g]),
                dequant_fp8(v[b, g], inp_local["v_scale"][b, g]))
    return bf16_to_f64(k[b, g]), bf16_to_f64(v[b, g])


def swa_branch(q, K_local, V_local, n: int, W: int, sm_scale):
    """The separate sliding-window branch: q [G, D] over the ring rows of the window."""
    rows = local_rows(n, W, K_local.shape[0])
    out, _ = full_attention(q, K_local[rows], V_local[rows], sm_scale)
    return out


def gen1_sparse_layer(q, K, V, idx, K_local, V_local, n: int, W: int, sm_scale):
    """Readings G1-G3: block-selected rows of the shared cache (one softmax) plus the
    sliding-window branch over the local ring (its own softmax), outputs added."""
    return sparse_attention(q, K, V, idx, sm_scale) + swa_branch(q, K_local, V_local, n, W, sm_scale)
