"""Pins for the KV Bridging oracle (oracle/bridge.py): each test ties it to
something other than itself -- torch's own bfloat16 and float8_e4m3fn casts (an
independent implementation of the same rounding), hand-made ties and saturation
cases from the format definitions, brute-force loops on tiny inputs, and
closed forms of the per-row quantisation.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
from oracle import bridge as kb


def _f32(x):
    return np.asarray(x, dtype=np.float32)


# ----------------------------------------------------------------------------- bf16 rounding
def test_bf16_rne_matches_torch_cast_on_random_values():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(kb.bf16_rne(x), ref)


def test_bf16_rne_ties_go_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 (even) and 1 + 2^-7 (odd): rounds to 1.0;
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even): rounds up
    x = _f32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20])
    got = kb.bf16_rne(x)
    assert list(got) == [0x3F80, 0x3F82, 0xBF80, 0x3F81]


# ----------------------------------------------------------------------------- e4m3fn encoding
def test_e4m3fn_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.e4m3fn_table()[codes].astype(np.float32)
    assert np.array_equal(kb.e4m3fn_encode(vals), codes)


def test_e4m3fn_encode_ties_and_neighbours_of_every_midpoint():
    tab = oracle.e4m3fn_table()
    pos = [(c, tab[c]) for c in range(0x00, 0x7F)]
    for (ca, a), (cb, b) in zip(pos[:-1], pos[1:]):
        mid = np.float32((a + b) / 2)
        assert float(mid) == (a + b) / 2            # midpoints are exact in fp32
        even = ca if ca % 2 == 0 else cb
        assert kb.e4m3fn_encode(mid) == even, (a, b)
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1000))
        assert kb.e4m3fn_encode(below) == ca and kb.e4m3fn_encode(above) == cb
        assert kb.e4m3fn_encode(-above) == (cb | 0x80)


def test_e4m3fn_encode_saturates_and_special_values():
    x = _f32([448.0, 460.0, 464.0, 1e30, np.inf, -500.0, -np.inf, 0.0, -0.0, np.nan,
              2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11])
    got = kb.e4m3fn_encode(x)
    # 2^-9 is the smallest subnormal (code 1); 2^-10 ties between 0 and it -> 0 (even);
    # 3 * 2^-10 ties between codes 1 and 2 -> 2 (even); 2^-11 rounds to 0
    assert list(got) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x00, 0x80, 0x7F,
                         0x01, 0x00, 0x02, 0x00]


def test_e4m3fn_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(12)
    mag = np.exp(rng.uniform(math.log(2.0 ** -12), math.log(448.0), 300000))
    x = (mag * np.where(rng.random(mag.size) < 0.5, -1, 1)).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(kb.e4m3fn_encode(x), ref)


# ----------------------------------------------------------------------------- per-row quantisation
def test_quantize_rows_closed_forms():
    rng = np.random.default_rng(13)
    y = rng.standard_normal((50, 128)).astype(np.float32)
    y[3] = 0.0
    y[4, 17] = -9.5                                  # a negative maximum magnitude
    codes, scales = kb.quantize_rows(y)
    amax = np.abs(y).max(axis=1)
    for r in range(50):
        if r == 3:
            assert scales[r] == 1.0 and not codes[r].any()
            continue
        # scale is the correctly rounded fp32 quotient amax / 448
        assert scales[r] == np.float32(np.float64(amax[r]) / 448.0)
        j = int(np.argmax(np.abs(y[r])))
        assert codes[r, j] == (0xFE if y[r, j] < 0 else 0x7E)    # the maximum maps to +-448
        # every code is the nearest E4M3FN value of y / scale: error at most half a spacing
        deq = oracle.e4m3fn_table()[codes[r]] * float(scales[r])
        q = y[r].astype(np.float64) / float(scales[r])
        tab = oracle.e4m3fn_table()[codes[r]]
        e = np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6)))
        half = 2.0 ** (e - 3) / 2                     # half the spacing at that binade
        assert np.all(np.abs(tab - q) <= half * (1 + 1e-6) + 1e-12)
        assert np.allclose(deq, y[r], rtol=1 / 16, atol=float(scales[r]) * 2.0 ** -9)


def test_quantize_rows_is_scale_invariant_by_powers_of_two():
    rng = np.random.default_rng(14)
    y = rng.standard_normal((20, 128)).astype(np.float32)
    c1, s1 = kb.quantize_rows(y)
    c2, s2 = kb.quantize_rows(y * np.float32(64.0))
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * np.float32(64.0))


# ----------------------------------------------------------------------------- projection
def test_project_brute_force_tiny():
    rng = np.random.default_rng(15)
    x = rng.integers(0, 2 ** 16, size=(3, 5), dtype=np.uint16) & np.uint16(0xBFFF)
    w = rng.integers(0, 2 ** 16, size=(4, 5), dtype=np.uint16) & np.uint16(0xBFFF)

    def val(b):
        return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]

    y = kb.project(x, w)
    for t in range(3):
        for n in range(4):
            ref = math.fsum(val(x[t, i]) * val(w[n, i]) for i in range(5))
            assert y[t, n] == pytest.approx(ref, rel=1e-15, abs=1e-300)


def test_project_one_hot_rows_pick_weight_columns():
    rng = np.random.default_rng(16)
    w = torch.from_numpy(rng.standard_normal((6, 8)).astype(np.float32)).to(torch.bfloat16)
    w = w.view(torch.int16).numpy().view(np.uint16)
    x = np.zeros((8, 8), dtype=np.uint16)
    x[np.arange(8), np.arange(8)] = 0x3F80           # bf16 1.0
    y = kb.project(x, w)
    assert np.array_equal(y, oracle.bf16_to_f64(w).T)   # row i of X picks column i of W^T


# ----------------------------------------------------------------------------- the whole bridge
def _tiny_case(fp8, seed=17, L=2, B=3, Hkv=2, D=128, cap=9, Hd=16, T=5):
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((T, Hd)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy((rng.standard_normal((L, 2, Hkv * D, Hd)) / 4).astype(np.float32)).to(torch.bfloat16)
    x = x.view(torch.int16).numpy().view(np.uint16)
    w = w.view(torch.int16).numpy().view(np.uint16)
    seq = np.array([0, 2, 2, 5, 1], dtype=np.int32)[:T]      # seq 5 is out of range: skipped
    pos = np.array([4, 0, 8, 1, 9], dtype=np.int32)[:T]      # pos 9 == cap: skipped
    if fp8:
        caches = dict(k=np.full((L, B, Hkv, cap, D), 0x7F, np.uint8), v=np.full((L, B, Hkv, cap, D), 0x7F, np.uint8),
                      k_scale=np.full((L, B, Hkv, cap), -3.0, np.float32),
                      v_scale=np.full((L, B, Hkv, cap), -3.0, np.float32))
    else:
        caches = dict(k=np.full((L, B, Hkv, cap, D), 0x7FC0, np.uint16),
                      v=np.full((L, B, Hkv, cap, D), 0x7FC0, np.uint16))
    return x, w, seq, pos, caches


@pytest.mark.parametrize("fp8", [False, True], ids=["bf16", "fp8"])
def test_kv_bridge_matches_per_element_brute_force(fp8):
    x, w, seq, pos, caches = _tiny_case(fp8)
    out = kb.kv_bridge(x, w, seq, pos, caches)
    L, _, N, Hd = w.shape
    _, B, Hkv, cap, D = caches["k"].shape

    def val(b):
        return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]

    written = set()
    for t in range(len(seq)):
        b, p = int(seq[t]), int(pos[t])
        if not (0 <= b < B and 0 <= p < cap):
            continue
        written.add((b, p))
        for l in range(L):
            for which, name in ((0, "k"), (1, "v")):
                for g in range(Hkv):
                    row = np.array([math.fsum(val(x[t, i]) * val(w[l, which, g * D + d, i]) for i in range(Hd))
                                    for d in range(D)], dtype=np.float32)
                    rt = torch.from_numpy(row)
                    if fp8:
                        amax = float(np.abs(row).max())
                        s = np.float32(amax / 448.0) if amax > 0 else np.float32(1.0)
                        codes = (rt / torch.tensor(s)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
                        assert out[name + "_scale"][l, b, g, p] == s
                        assert np.array_equal(out[name][l, b, g, p], codes)
                    else:
                        ref = rt.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                        assert np.array_equal(out[name][l, b, g, p], ref)
    # every other row is untouched
    for name in out:
        for b in range(B):
            for p in range(cap):
                if (b, p) not in written:
                    assert np.array_equal(out[name][:, b, :, p], caches[name][:, b, :, p])


def test_kv_bridge_layers_and_heads_use_their_own_weights():
    # swapping W_k and W_v, or two layers, swaps the written rows: no transposed operand
    x, w, seq, pos, caches = _tiny_case(False, seed=18)
    base = kb.kv_bridge(x, w, seq, pos, caches)
    sw = kb.kv_bridge(x, w[:, ::-1].copy(), seq, pos, caches)
    assert np.array_equal(sw["k"], base["v"]) and np.array_equal(sw["v"], base["k"])
    sl = kb.kv_bridge(x, w[::-1].copy(), seq, pos, caches)
    assert np.array_equal(sl["k"][0], base["k"][1])
    wh = w.reshape(2, 2, 2, 128, -1)[:, :, ::-1].reshape(w.shape).copy()   # swap KV heads
    shh = kb.kv_bridge(x, wh, seq, pos, caches)
    assert np.array_equal(shh["k"][:, :, 0], base["k"][:, :, 1])
