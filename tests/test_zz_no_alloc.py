"""GPU test of hs2_full_attn_select_noalloc (the entry point for callers that cannot
allocate): through the C ABI, two calls in a row -- the second with a smaller input --
against hs2_full_attn_select with a caller-owned workspace, on the same inputs and the
deterministic scan, so the outputs must be bitwise equal; the first call is also
checked against the float64 oracle on a sample (the parity bar of tests/parity.py)."""
import numpy as np
import pytest
import torch

import oracle
from long_context_decode_full_amd import (HS2_FLAG_DETERMINISTIC, HS2_OK, hs2_full_attn_select_noalloc)
from long_context_decode_full_amd import workloads as wl
from long_context_decode_full_amd.runner import HybridBlockDevice
from parity import assert_out_close, check_idx_row

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


CALLS = [
    # the larger call first: 3 sequences of a batched decode, bf16
    (wl.Workload("noalloc large", 3, 1, 32, 4, ctx_lens=[150000, 40000, 90001], n_needles=32, seed=5101),
     dict(with_probs=False)),
    # then a smaller one: fp8, fewer heads, a short context, and every probability
    (wl.Workload("noalloc small", 2, 1, 16, 2, ctx_lens=[7000, 900], n_needles=8, kv_dtype="fp8", seed=5102),
     dict(with_probs=True)),
]


def _noalloc(dev):
    out = torch.full_like(dev.out_full, float("nan"))
    idx = torch.full_like(dev.idx, -7)
    probs = None if dev.probs is None else torch.full_like(dev.probs, -1.0)
    st = hs2_full_attn_select_noalloc(dev.desc, dev.q_full, dev.k, dev.v, dev.k_scale, dev.v_scale,
                                      dev.ctx_len, out, idx, probs)
    assert st == HS2_OK, st
    torch.cuda.synchronize()
    return out.cpu().numpy(), idx.cpu().numpy(), None if probs is None else probs.cpu().numpy()


def test_noalloc_equals_the_workspace_entry_point():
    for i, (w, kw) in enumerate(CALLS):
        print(f"\n[gpu case] noalloc call {i}: {w.name} B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
              f"ctx={w.ctx_lens} kv={w.kv_dtype} probs={kw['with_probs']} seed={w.seed}", flush=True)
        inp = wl.make_inputs(w)
        dev = HybridBlockDevice(inp, flags=HS2_FLAG_DETERMINISTIC, **kw)
        dev.workspace.fill_(0xFF)
        dev.full()
        ref = dev.results()
        out, idx, probs = _noalloc(dev)
        assert np.array_equal(idx, ref["idx"]), "index sets differ from the workspace call"
        assert np.array_equal(out.view(np.uint32), ref["out_full"].view(np.uint32)), "outputs differ"
        if probs is not None:
            n = inp["ctx_len"]
            for b in range(w.batch):
                assert np.array_equal(probs[b, 0, :, :n[b]].view(np.uint32),
                                      ref["probs"][b, 0, :, :n[b]].view(np.uint32))
        # and the oracle, on the first sequence
        r = oracle.hybrid_block_token(inp, 0, 0)
        assert_out_close(out[0, 0], r["out_full"])
        for g in range(w.n_kv_heads):
            check_idx_row(idx[0, 0, g], r["idx"][g], r["s"][g], r["n"], 128, 1024)
        print(f"[gpu case] noalloc call {i}: bitwise equal to hs2_full_attn_select, oracle sample ok",
              flush=True)
