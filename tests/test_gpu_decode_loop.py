"""GPU tests of the multi-step decode (hs2_decode_step through the C ABI): every step
appends each sequence's new token to every Hybrid Block's cache through KV Bridging,
then runs every block's full layer and sparse layers (HySparse2 article, section 02).

- A step captured once into a HIP graph and replayed, with new inputs copied into
  its slots and synchronisations between the replays, gives bitwise the same
  contexts, caches and outputs as the same steps run eagerly (deterministic scan
  mode), after every step.
- Every appended K/V row matches the KV Bridging oracle (interval rule of
  tests/bridge_check.py); the last step's outputs and index sets match the
  Hybrid-Block oracle on the caches as they then are (rules of tests/parity.py).
- A sequence whose cache is full keeps its length and its rows; so does one that has
  reached the plan's max_ctx_len below the capacity (the rows past it stay untouched).
"""
import numpy as np
import pytest
import torch

import oracle
from long_context_decode_full_amd import HS2_FLAG_DETERMINISTIC
from long_context_decode_full_amd import workloads as wl
from long_context_decode_full_amd.runner import DecodeLoopDevice
from tests import bridge_check as bc
from tests.parity import assert_out_close, check_idx_row

pytestmark = pytest.mark.gpu


def _appended_rows(dev, ctx_before, ctx_after):
    """Cache rows written by the last step: codes [B, L, 2, Hkv, D] (+ scales), for the
    sequences that advanced."""
    torch.cuda.synchronize()
    bs = [b for b in range(len(ctx_before)) if ctx_after[b] == ctx_before[b] + 1]
    codes, scales = [], []
    for b in bs:
        p = int(ctx_before[b])
        codes.append(np.stack([np.stack([c[l][b, :, p].cpu().numpy() for c in (dev.k, dev.v)])
                               for l in range(dev.nb)]))
        if dev.fp8:
            scales.append(np.stack([np.stack([c[l][b, :, p].cpu().numpy() for c in (dev.ks, dev.vs)])
                                    for l in range(dev.nb)]))
    out = dict(codes=np.asarray(codes))
    if dev.fp8:
        out["scales"] = np.asarray(scales)
    else:
        out["codes"] = out["codes"].view(np.uint16)
    return bs, out


def _check_bridge_rows(dev, dec, t, bs, got):
    if not bs:
        return
    Y, E = bc.reference(dec["x"][t], dec["w_bits"], np.asarray(bs))
    if dev.fp8:
        bc.check_fp8(got["codes"], got["scales"], Y, E)
    else:
        bc.check_bf16(got["codes"], Y, E)


def _check_attention(dev, dec, t):
    st = dev.state()
    for l in range(dev.nb):
        qf = dec["q_full"][t][l]
        qs = dec["q_sparse"][t][l * dev.ns:(l + 1) * dev.ns]
        inp = dev.block_inputs(l, qf, qs)
        ref = oracle.hybrid_block(inp)
        G = dev.Hq // dev.Hkv
        for (b, j), r in ref.items():
            assert_out_close(st["out_full"][l][b, j], r["out_full"], what=f"block {l} out_full[{b}]")
            for g in range(dev.Hkv):
                check_idx_row(st["idx"][l][b, j, g], r["idx"][g], r["s"][g], r["n"], 128, 1024)
                if np.array_equal(st["idx"][l][b, j, g], r["idx"][g]):
                    heads = slice(g * G, (g + 1) * G)
                    for s in range(dev.ns):
                        assert_out_close(st["out_sparse"][l * dev.ns + s][b, j, heads],
                                         r["out_sparse"][s][heads], what=f"block {l} sparse {s}[{b},{g}]")


def _same_state(a, b, dev_a, dev_b):
    assert np.array_equal(a["ctx_len"], b["ctx_len"])
    for x, y in zip(a["out_full"] + a["out_sparse"], b["out_full"] + b["out_sparse"]):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
    for x, y in zip(a["idx"], b["idx"]):
        assert np.array_equal(x, y)
    for l in range(dev_a.nb):
        assert torch.equal(dev_a.k[l], dev_b.k[l]) and torch.equal(dev_a.v[l], dev_b.v[l])
        if dev_a.fp8:
            assert torch.equal(dev_a.ks[l], dev_b.ks[l]) and torch.equal(dev_a.vs[l], dev_b.vs[l])


CASES = {
    "bf16": dict(kv="bf16", ctx=[3000, 5000], cap=5008, steps=4),
    # MQA: 32 query heads on one KV head (wide-group scan and gather)
    "mqa": dict(kv="bf16", ctx=[4000, 2500], cap=4010, steps=3, hq=32, hkv=1),
    "fp8": dict(kv="fp8", ctx=[2500, 4100], cap=4110, steps=3),
    # sequence 1 starts with a full cache: it keeps its length, appends nothing
    "full_cache": dict(kv="bf16", ctx=[1200, 1500], cap=1500, steps=3),
    # the plan bounds lengths at 1502 < capacity 1600: sequence 1 grows twice, then stays
    "length_bound": dict(kv="bf16", ctx=[1200, 1500], cap=1600, steps=4, max_ctx=1502),
}


@pytest.mark.parametrize("name", list(CASES))
def test_decode_loop_graph_eager_and_oracle(name):
    c = CASES[name]
    hq, hkv = c.get("hq", 16), c.get("hkv", 2)
    limit = c.get("max_ctx", c["cap"])
    w = wl.Workload(f"decode loop {name}", 2, 1, hq, hkv, ctx_lens=c["ctx"], capacity=c["cap"],
                    kv_dtype=c["kv"], n_needles=8, poison_tail=limit < c["cap"], seed=3001)
    print(f"\n[decode loop] {name}: B=2 Hq{hq}/Hkv{hkv} ctx={c['ctx']} cap={c['cap']} {c['kv']} "
          f"blocks=2 hidden=256 steps={c['steps']}", flush=True)
    inp = wl.make_inputs(w)
    dec = wl.make_decode_steps(w, n_blocks=2, steps=c["steps"], hidden=256, seed=3002)
    eager = DecodeLoopDevice(inp, 2, dec["w_bits"], max_ctx_len=limit, flags=HS2_FLAG_DETERMINISTIC)
    graph = DecodeLoopDevice(inp, 2, dec["w_bits"], max_ctx_len=limit, flags=HS2_FLAG_DETERMINISTIC)
    g = None
    ctx = inp["ctx_len"].copy()
    for t in range(c["steps"]):
        eager.set_inputs(dec["x"][t], dec["q_full"][t], dec["q_sparse"][t])
        eager.step()
        graph.set_inputs(dec["x"][t], dec["q_full"][t], dec["q_sparse"][t])
        if g is None:
            g = graph.capture()
        g.replay()
        torch.cuda.synchronize()
        se, sg = eager.state(), graph.state()
        _same_state(se, sg, eager, graph)
        expect = np.where(ctx < limit, ctx + 1, ctx)
        assert np.array_equal(sg["ctx_len"], expect), (sg["ctx_len"], expect)
        bs, rows = _appended_rows(graph, ctx, sg["ctx_len"])
        _check_bridge_rows(graph, dec, t, bs, rows)
        ctx = sg["ctx_len"].copy()
        print(f"[decode loop]   step {t}: ctx {ctx.tolist()}, graph == eager", flush=True)
    _check_attention(graph, dec, c["steps"] - 1)
    if name == "full_cache":
        assert int(ctx[1]) == c["cap"]
        # the full sequence's rows are the initial ones
        k0 = inp["k"][1]
        assert np.array_equal(graph.k[0][1].cpu().numpy().view(np.uint16), k0)
    if name == "length_bound":
        assert int(ctx[1]) == limit
        # rows at and past the bound are never written (they still hold the NaN poison)
        for l in range(2):
            for cache in (graph.k[l], graph.v[l]):
                tail = cache[1, :, limit:].cpu().numpy().view(np.uint16)
                assert np.all(tail == inp["k"][1, :, limit:]) and np.all(tail == wl.BF16_NAN)


def test_decode_step_at_the_million_token_context():
    """One hs2_decode_step at full size: a million-token context (32 query heads on 4 KV
    heads, bf16) grows by one token through KV Bridging (hidden 2048), then the block's
    full layer selects over 1,048,577 positions and its 3 sparse layers reuse the
    selection; the appended rows against the bridge oracle and every output and index
    set against the Hybrid-Block oracle, as in the small cases."""
    import dataclasses
    base = wl.standard_workloads()["million"]
    w = dataclasses.replace(base, capacity=base.ctx_lens[0] + 8)
    print(f"\n[decode loop] million: B=1 Hq32/Hkv4 ctx={w.ctx_lens} cap={w.capacity} bf16 blocks=1 "
          f"hidden=2048 steps=1", flush=True)
    inp = wl.make_inputs(w, threads=16)
    dec = wl.make_decode_steps(w, n_blocks=1, steps=1, hidden=2048, seed=3010)
    dev = DecodeLoopDevice(inp, 1, dec["w_bits"])
    del inp
    ctx = dev.ctx_len.cpu().numpy().copy()
    dev.set_inputs(dec["x"][0], dec["q_full"][0], dec["q_sparse"][0])
    dev.step()
    st = dev.state()
    assert np.array_equal(st["ctx_len"], ctx + 1)
    bs, rows = _appended_rows(dev, ctx, st["ctx_len"])
    _check_bridge_rows(dev, dec, 0, bs, rows)
    _check_attention(dev, dec, 0)
    print("[decode loop]   million step: bridge rows and attention match the oracles", flush=True)
