"""CPU checks of the KV Bridging parity rule (tests/bridge_check.py): an fp32
emulation of the kernel (a different summation order, the same fp32 decisions)
passes, and planted mistakes in such an emulation fail."""
import numpy as np
import pytest
import torch

from oracle import bridge as ob
from long_context_decode_full_amd import workloads as wl
from tests import bridge_check as bc


def _case(kv_dtype="fp8", T=96, Hd=512, L=2, Hkv=2, seed=7):
    w = wl.BridgeWorkload("rule", T, Hd, L, Hkv, batch=1, capacity=T, kv_dtype=kv_dtype, seed=seed)
    return wl.make_bridge_inputs(w)


def _emulate(inp, tokens):
    """fp32 projection in the kernel's order: blocks of 32 products summed in fp32,
    the blocks accumulated one after another in fp32."""
    x = torch.from_numpy(inp["x"][tokens].view(np.int16)).view(torch.bfloat16).float().numpy()
    w = inp["weight"]
    L, two, N, Hd = w.shape
    W = torch.from_numpy(w.reshape(-1, Hd).view(np.int16)).view(torch.bfloat16).float().numpy()
    y = np.zeros((len(tokens), W.shape[0]), dtype=np.float32)
    for b in range(0, Hd, 32):
        y = (y + (x[:, b:b + 32] @ W[:, b:b + 32].T).astype(np.float32)).astype(np.float32)
    return y.reshape(len(tokens), L, two, N // 128, 128)


def test_fp32_emulation_passes_fp8_and_bf16():
    inp = _case()
    tok = np.arange(96)
    Y, E = bc.reference(inp["x"], inp["weight"], tok)
    y = _emulate(inp, tok)
    codes, scales = ob.quantize_rows(y)
    amb, differ = bc.check_fp8(codes, scales, Y, E)
    assert amb < 0.02 * codes.size and differ <= amb
    amb, differ = bc.check_bf16(ob.bf16_rne(y), Y, E)
    assert amb < 0.15 * y.size and differ <= amb


def test_planted_code_error_fails():
    inp = _case(seed=8)
    tok = np.arange(96)
    Y, E = bc.reference(inp["x"], inp["weight"], tok)
    codes, scales = ob.quantize_rows(_emulate(inp, tok))
    bad = codes.copy()
    bad[5, 1, 0, 1, 77] ^= 0x02                       # one code two steps off
    with pytest.raises(AssertionError):
        bc.check_fp8(bad, scales, Y, E)


def test_planted_scale_error_fails():
    inp = _case(seed=9)
    tok = np.arange(96)
    Y, E = bc.reference(inp["x"], inp["weight"], tok)
    codes, scales = ob.quantize_rows(_emulate(inp, tok))
    bad = scales.copy()
    bad[3, 0, 1, 0] *= np.float32(1.01)
    with pytest.raises(AssertionError):
        bc.check_fp8(codes, bad, Y, E)


def test_swapped_heads_and_dropped_term_fail():
    inp = _case("bf16", seed=10)
    tok = np.arange(96)
    Y, E = bc.reference(inp["x"], inp["weight"], tok)
    y = _emulate(inp, tok)
    sw = y[:, :, :, ::-1].copy()                      # KV heads swapped
    with pytest.raises(AssertionError):
        bc.check_bf16(ob.bf16_rne(sw), Y, E)
    x = inp["x"].copy()
    x[:, -64:] = 0                                    # the last 64 hidden dims dropped
    y2 = _emulate(dict(inp, x=x), tok)
    with pytest.raises(AssertionError):
        bc.check_bf16(ob.bf16_rne(y2), Y, E)
