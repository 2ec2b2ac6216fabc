"""GPU parity of the first-generation comparator (hs2_sparse_attn_swa through the C ABI):
block-level selection by the full layer, then sparse layers that add a separate
sliding-window branch over their own local rings, against the float64 oracle
(oracle/gen1.py) fed the same index sets; the block selection itself against the
oracle's block rule (tests/parity.py)."""
import numpy as np
import pytest
import torch

import oracle
from long_context_decode_full_amd import workloads as wl
from long_context_decode_full_amd.runner import HybridBlockDevice
from tests.parity import assert_out_close, check_block_row

pytestmark = pytest.mark.gpu

W = 128
CASES = {
    # decode; sequence 1 sees fewer positions than the window
    "decode_bf16": (wl.Workload("gen1 decode", 2, 1, 16, 2, ctx_lens=[3000, 100], n_needles=8, seed=5001), 128),
    "decode_fp8": (wl.Workload("gen1 decode fp8", 2, 1, 16, 2, ctx_lens=[4096, 2000], kv_dtype="fp8",
                               n_needles=8, seed=5002), 128),
    # query chunks: every token of the chunk finds its whole window in a ring of >= W + Lq - 1 rows
    "chunk_bf16": (wl.Workload("gen1 chunk", 2, 16, 16, 2, ctx_lens=[5000, 900], n_needles=8, seed=5003), 160),
    "chunk_g8": (wl.Workload("gen1 chunk G8", 1, 8, 32, 4, ctx_lens=[7000], n_needles=8, seed=5004), 135),
    # 256 selection rows: the one-launch matrix-core gather for both branches
    "chunk_256_rows": (wl.Workload("gen1 chunk 256 rows", 4, 16, 32, 4, ctx_lens=[3000, 2000, 1000, 4000],
                                   n_needles=8, seed=5005), 143),
}


@pytest.mark.parametrize("name", list(CASES))
def test_gen1_sparse_layers(name):
    w, R = CASES[name]
    print(f"\n[gen1] {name}: B={w.batch} Lq={w.q_len} Hq={w.n_q_heads}/Hkv={w.n_kv_heads} "
          f"ctx={w.ctx_lens} {w.kv_dtype} ring={R}", flush=True)
    inp = wl.make_inputs(w)
    rings = wl.make_local_rings(w, R, seed=w.seed + 100)
    dev = HybridBlockDevice(inp, mode="gen1", local_rings=rings, local_window=W)
    dev.step()
    got = dev.results()
    G = w.n_q_heads // w.n_kv_heads
    sm = inp["sm_scale"]
    worst = 0.0
    for b in range(w.batch):
        for j in range(w.q_len):
            n = int(inp["ctx_len"][b]) - w.q_len + j + 1
            ref = oracle.hybrid_block_token(inp, b, j, mode="block")
            for g in range(w.n_kv_heads):
                check_block_row(got["idx"][b, j, g], ref["idx"][g], ref["s"][g], n, 64, 18)
                K, V = oracle.kv_rows(inp, b, g, n)
                heads = slice(g * G, (g + 1) * G)
                for layer in range(w.n_sparse_layers):
                    Kl, Vl = oracle.local_kv(rings[layer], b, g)
                    q = oracle.bf16_to_f64(inp["q_sparse"][layer][b, j, heads])
                    want = oracle.gen1_sparse_layer(q, K, V, got["idx"][b, j, g], Kl, Vl, n, W, sm)
                    worst = max(worst, assert_out_close(got["out_sparse"][layer][b, j, heads], want,
                                                        what=f"{name} layer {layer} [{b},{j},{g}]"))
    print(f"[gen1] {name}: worst row relative error {worst:.2e}", flush=True)


@pytest.mark.parametrize("name", ["decode_bf16", "decode_fp8"])
def test_gen1_decode_one_launch_equals_three_steps(name):
    """At decode sizes both branches run in one launch (the window rows formed in the
    kernel, the two normalised outputs added there); the result equals the three-step
    form that HS2_FLAG_SPARSE_HEAD keeps (shared gather, window rows, local gather, sum)
    bit for bit, since both take the same arithmetic in the same order."""
    from long_context_decode_full_amd import HS2_FLAG_SPARSE_HEAD
    w, R = CASES[name]
    print(f"\n[gen1] {name}: one launch against three steps", flush=True)
    inp = wl.make_inputs(w)
    rings = wl.make_local_rings(w, R, seed=w.seed + 100)
    outs = []
    for flags in (0, HS2_FLAG_SPARSE_HEAD):
        dev = HybridBlockDevice(inp, mode="gen1", local_rings=rings, local_window=W, flags=flags)
        dev.step()
        outs.append(dev.results())
    a, b = outs
    assert np.array_equal(a["idx"], b["idx"])
    for layer in range(w.n_sparse_layers):
        assert np.array_equal(a["out_sparse"][layer], b["out_sparse"][layer]), f"layer {layer}"
