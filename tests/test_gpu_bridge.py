"""GPU parity of the KV Bridging kernel (hs2_kv_bridge through the C ABI) against the
float64 oracle (oracle/bridge.py), with the interval rule of tests/bridge_check.py:
every written code must lie between the decisions at Y - E and Y + E (the kernel's
fp32 summation bound), codes whose interval holds one value must match exactly, and
every row that is not a destination must keep its bytes.

Small cases compare whole caches; the full-size prefill chunk (16,384 tokens,
hidden 2048, 6 target layers, in the launch configuration bench.py times) checks a
sample of tokens against the oracle and, for every token, that its destination rows
were written while the rows around the chunk were not.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from long_context_decode_full_amd import workloads as wl
from long_context_decode_full_amd.runner import BridgeDevice
from tests import bridge_check as bc

pytestmark = pytest.mark.gpu

MAX_DIFFER = 0.005          # codes differing from the oracle's own decision (all ambiguous)


def _announce(name, w):
    print(f"[bridge] {name}: T={w.n_tokens} Hd={w.hidden} L={w.n_layers} Hkv={w.n_kv_heads} "
          f"B={w.batch} cap={w.capacity} {w.kv_dtype} {w.placement}", flush=True)


def _valid(inp):
    w = inp["workload"]
    s, p = inp["seq"], inp["pos"]
    return (s >= 0) & (s < w.batch) & (p >= 0) & (p < w.capacity)


def _check_rows(inp, got, tokens):
    w = inp["workload"]
    Y, E = bc.reference(inp["x"], inp["weight"], tokens)
    if w.kv_dtype == "fp8":
        amb, differ = bc.check_fp8(got["codes"], got["scales"], Y, E)
    else:
        amb, differ = bc.check_bf16(got["codes"], Y, E)
    n = got["codes"].size
    print(f"[bridge]   {len(tokens)} tokens: ambiguous {amb / n:.4f}, differ {differ / n:.5f}", flush=True)
    assert differ <= MAX_DIFFER * n
    return amb, differ


def _full_compare(inp, dev):
    """Whole caches: destination rows by the interval rule, all other rows unchanged."""
    w = inp["workload"]
    got = dev.caches()
    fill, sfill = wl.bridge_cache_sentinel(w.kv_dtype)
    shape = (w.n_layers, w.batch, w.n_kv_heads, w.capacity, w.head_dim)
    start = dict(k=np.full(shape, fill), v=np.full(shape, fill))
    if w.kv_dtype == "fp8":
        start["k_scale"] = np.full(shape[:4], sfill, np.float32)
        start["v_scale"] = np.full(shape[:4], sfill, np.float32)
    ok = _valid(inp)
    dest = np.zeros((w.batch, w.capacity), dtype=bool)
    dest[inp["seq"][ok], inp["pos"][ok]] = True
    for name in got:
        a, b = got[name], start[name].astype(got[name].dtype)
        keep = ~dest[None, :, None, :]
        if a.ndim == 5:
            keep = keep[..., None]
        keep = np.broadcast_to(keep, a.shape)
        same = (a == b) | (np.isnan(a) & np.isnan(b)) if a.dtype == np.float32 else (a == b)
        assert same[keep].all(), f"{name}: a row that is not a destination changed"
    tokens = np.nonzero(ok)[0]
    if tokens.size:
        rows = dev.rows(tokens)
        _check_rows(inp, rows, tokens)
    return tokens.size


def _run(w, **over):
    inp = wl.make_bridge_inputs(w)
    for k, v in over.items():
        inp[k] = v(inp) if callable(v) else v
    fill, sfill = wl.bridge_cache_sentinel(w.kv_dtype)
    dev = BridgeDevice(inp, fill=fill, scale_fill=float("nan") if sfill is None else float(sfill))
    dev.run()
    torch.cuda.synchronize()
    return inp, dev


SMALL = {
    "ragged_fp8": wl.bridge_workloads()["bridge_ragged"],
    "ragged_bf16": dataclasses.replace(wl.bridge_workloads()["bridge_ragged"], kv_dtype="bf16"),
    "mqa_ragged": wl.BridgeWorkload("MQA ragged", 300, 256, 3, 1, batch=2, capacity=1024,
                                    placement="ragged", bad_rows=3, seed=2101),
    "one_token_one_step": wl.BridgeWorkload("single token, hidden 64", 1, 64, 1, 1, batch=1, capacity=8,
                                            placement="decode", seed=2102),
    "tile_plus_one_hidden_4096": wl.BridgeWorkload("129 tokens, hidden 4096", 129, 4096, 1, 2, batch=1,
                                                   capacity=129, seed=2103),
    "many_layers_bf16": wl.BridgeWorkload("16 layers", 200, 128, 16, 1, batch=3, capacity=300,
                                          kv_dtype="bf16", placement="ragged", seed=2104),
    # both sides of the switch from 128- to 256-token tiles (4,096 tokens), ragged tails
    "below_large_tiles": wl.BridgeWorkload("4095 tokens", 4095, 512, 2, 2, batch=3, capacity=8192,
                                           placement="ragged", bad_rows=9, seed=2107),
    "large_tiles_ragged_fp8": wl.BridgeWorkload("4097 tokens", 4097, 512, 2, 2, batch=3, capacity=8192,
                                                placement="ragged", bad_rows=9, seed=2108),
    "large_tiles_ragged_bf16": wl.BridgeWorkload("4097 tokens, bf16", 4097, 256, 1, 1, batch=2,
                                                 capacity=8192, kv_dtype="bf16", placement="ragged",
                                                 bad_rows=5, seed=2109),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_bridge_small_whole_caches(name):
    w = SMALL[name]
    _announce(name, w)
    inp, dev = _run(w)
    assert _full_compare(inp, dev) == int(_valid(inp).sum())


# The decode-size path (one workgroup per 128 features x 16 tokens, W read straight
# into registers) takes calls of at most 16 tokens; the descriptor's gemv_max_tokens
# moves the switch, so each path is also run on the other's sizes.
GEMV = {
    # hidden 64: one 32-dim step per half (remainder loop only)
    "gemv_hidden_64_bf16": (wl.BridgeWorkload("5 tokens, hidden 64", 5, 64, 2, 1, batch=2, capacity=16,
                                              kv_dtype="bf16", placement="ragged", seed=2110), None),
    # hidden 576: 9 steps per half (one unrolled batch of 8 + one)
    "gemv_hidden_576_fp8": (wl.BridgeWorkload("9 tokens, hidden 576", 9, 576, 3, 2, batch=4, capacity=64,
                                              placement="ragged", bad_rows=2, seed=2111), None),
    "gemv_mqa_fp8": (wl.BridgeWorkload("16 tokens, one KV head", 16, 2048, 4, 1, batch=16, capacity=40,
                                       placement="decode", seed=2112), None),
    # three token blocks, the last one ragged
    "gemv_forced_40_tokens_fp8": (wl.BridgeWorkload("40 tokens on the decode-size path", 40, 1024, 2, 4,
                                                    batch=3, capacity=128, placement="ragged", bad_rows=3,
                                                    seed=2113), 64),
    "gemv_forced_40_tokens_bf16": (wl.BridgeWorkload("40 tokens on the decode-size path, bf16", 40, 512, 2, 2,
                                                     batch=3, capacity=128, kv_dtype="bf16",
                                                     placement="ragged", bad_rows=3, seed=2114), 64),
    # the tile path on a decode-size call
    "tile_forced_16_tokens_fp8": (wl.BridgeWorkload("16 tokens on the tile path", 16, 2048, 2, 4, batch=16,
                                                    capacity=40, placement="decode", seed=2115), -1),
}


@pytest.mark.parametrize("name", list(GEMV))
def test_bridge_decode_size_paths(name):
    w, switch = GEMV[name]
    _announce(name, w)
    inp, dev = _run(w, gemv_max_tokens=switch or 0)
    assert _full_compare(inp, dev) == int(_valid(inp).sum())


def test_bridge_every_destination_invalid_writes_nothing():
    w = wl.BridgeWorkload("all invalid", 50, 128, 2, 2, batch=2, capacity=64, placement="ragged",
                          bad_rows=50, seed=2105)
    _announce("all_invalid", w)
    inp, dev = _run(w)
    assert not _valid(inp).any()
    assert _full_compare(inp, dev) == 0


@pytest.mark.parametrize("n_tokens", [256, 12])
def test_bridge_zero_and_large_rows(n_tokens):
    """All-zero hidden rows give all-zero K/V rows (scale 1, codes 0); rows scaled by
    2^12 keep the same codes with scales 2^12 larger (the maximum still maps to 448).
    256 tokens take the tile kernel, 12 the decode-size kernel."""
    w = wl.BridgeWorkload("zero and large", n_tokens, 512, 2, 2, batch=1, capacity=256, seed=2106)
    _announce(f"zero_and_large_{n_tokens}", w)
    k = min(16, n_tokens // 3)
    base = wl.make_bridge_inputs(w)
    x = base["x"].copy()
    x[:k] = 0                                           # zero rows
    big = x[k:2 * k].view(np.uint16).astype(np.uint32) + (12 << 7)   # exponent + 12
    x[k:2 * k] = big.astype(np.uint16)
    inp, dev = _run(w, x=x)
    _full_compare(inp, dev)
    rows = dev.rows(np.arange(2 * k))
    assert np.all(rows["scales"][:k] == 1.0) and not rows["codes"][:k].any()
    # the same tokens unscaled, in a second call
    inp2, dev2 = _run(w)
    r2 = dev2.rows(np.arange(k, 2 * k))
    assert np.array_equal(rows["codes"][k:2 * k], r2["codes"])
    assert np.array_equal(rows["scales"][k:2 * k], r2["scales"] * np.float32(4096.0))


def test_bridge_decode_append():
    w = wl.bridge_workloads()["bridge_decode"]
    _announce("bridge_decode", w)
    inp, dev = _run(w)
    tokens = np.arange(w.n_tokens)
    _check_rows(inp, dev.rows(tokens), tokens)
    # the rows next to each destination are untouched
    torch.cuda.synchronize()
    for l in range(w.n_layers):
        for c in (dev.k[l], dev.v[l]):
            for t in tokens:
                s, p = int(inp["seq"][t]), int(inp["pos"][t])
                for q in (p - 1, p + 1):
                    if 0 <= q < w.capacity:
                        assert bool((c[s, :, q] == 0x7F).all())


@pytest.mark.parametrize("name", ["bridge_prefill", "bridge_prefill_bf16", "bridge_mqa"])
def test_bridge_prefill_chunk_full_size(name):
    w = wl.bridge_workloads()[name]
    _announce(name, w)
    inp, dev = _run(w)
    T = w.n_tokens
    rng = np.random.default_rng(77)
    sample = np.unique(np.concatenate([[0, 1, 127, 128, 129, T // 2, T - 129, T - 128, T - 1],
                                       rng.choice(T, 183, replace=False)]))
    _check_rows(inp, dev.rows(sample), sample)
    # every destination row written, the rows before and after the chunk not
    lo, hi = w.start, w.start + T
    for l in range(w.n_layers):
        for c in (dev.k[l], dev.v[l]):
            chunk = c[0, :, lo:hi]
            if w.kv_dtype == "fp8":
                assert not bool((chunk == 0x7F).any()), "unwritten or NaN code in the chunk"
            else:
                assert not bool(torch.isnan(chunk.view(torch.bfloat16)).any())
            sent = 0x7F if w.kv_dtype == "fp8" else 0x7FC0
            if lo > 0:
                assert bool((c[0, :, lo - 1] == sent).all())
            if hi < w.capacity:
                assert bool((c[0, :, hi] == sent).all())
        if w.kv_dtype == "fp8":
            for s in (dev.ks[l], dev.vs[l]):
                sc = s[0, :, lo:hi]
                assert bool(torch.isfinite(sc).all() and (sc > 0).all())
                assert bool(torch.isnan(s[0, :, lo - 1]).all())
