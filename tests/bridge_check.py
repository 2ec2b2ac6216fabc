"""Parity rule for the KV Bridging kernel against the oracle (oracle/bridge.py).

The kernel accumulates the projection in fp32 (bf16 x bf16 products are exact in
fp32); the oracle sums in float64.  The kernel's sum is Hd / 32 matrix-core steps,
each adding a block of 32 exact products to the fp32 accumulator: with the block
summed in fp32 or wider (at most 31 roundings) and one rounding per accumulation,
the textbook bound for recursive summation gives
|y - Y| <= (Hd / 32 + 31) u sum|x_i w_i| + O(u^2), u = 2^-24, which E rounds up
(factor Hd / 32 + 32).  Every rounding decision
that follows is monotone in y (round to bf16; max; scale = max / 448; y / scale;
round to E4M3FN), so the codes the kernel may produce are exactly those between the
decisions taken at Y - E and at Y + E.  Where that interval holds one code -- all
but a few elements -- the kernel must match the oracle exactly; elsewhere either
neighbour is correct and the element is counted as ambiguous.  Both sides take the
decisions in fp32 (reading B5): the oracle's own codes come from
quantize_rows / bf16_rne of fp32(Y).
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import bridge as ob

_U = 2.0 ** -24


def _down(x):
    """float64 -> the largest fp32 value <= x."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f).astype(np.float32)


def _up(x):
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f).astype(np.float32)


def reference(x_bits, w_bits, tokens):
    """Float64 projection Y and error radius E of the given tokens, shaped
    [n, L, 2, Hkv, D] from w_bits [L, 2, Hkv * D, Hd]."""
    L, two, N, Hd = w_bits.shape
    X = oracle.bf16_to_f64(x_bits[np.asarray(tokens)])
    W = oracle.bf16_to_f64(w_bits.reshape(L * two * N, Hd))
    Y = ob.project(x_bits[np.asarray(tokens)], w_bits.reshape(L * two * N, Hd))
    A = np.abs(X) @ np.abs(W).T
    E = A * ((Hd // 32 + 32) * _U)
    shape = (len(tokens), L, two, N // 128, 128)
    return Y.reshape(shape), E.reshape(shape)


def check_bf16(codes, Y, E):
    """codes: uint16 bf16 bits, same shape as Y.  Returns (n_ambiguous, n_differ)."""
    got = oracle.bf16_to_f64(codes)
    lo = oracle.bf16_to_f64(ob.bf16_rne(_down(Y - E)))
    hi = oracle.bf16_to_f64(ob.bf16_rne(_up(Y + E)))
    bad = ~((lo <= got) & (got <= hi))
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"bf16 code outside the admissible interval at {tuple(i)}: "
                             f"got {got[tuple(i)]!r}, interval [{lo[tuple(i)]!r}, {hi[tuple(i)]!r}], "
                             f"Y {Y[tuple(i)]!r}; {int(bad.sum())} such elements")
    own = ob.bf16_rne(Y.astype(np.float32))
    return int((lo != hi).sum()), int((own != codes).sum())


def _e4m3(codes):
    return oracle.e4m3fn_table()[np.asarray(codes, dtype=np.uint8)]


def check_fp8(codes, scales, Y, E):
    """codes uint8 [..., D], scales float32 [...].  Checks the scale of every row
    against the admissible interval, then every code given the kernel's own scale.
    Returns (n_ambiguous, n_differ) over codes."""
    absY = np.abs(Y)
    amax_lo = np.maximum(absY - E, 0.0).max(axis=-1)
    amax_hi = (absY + E).max(axis=-1)
    s_lo = np.where(amax_lo > 0, _down(_down(amax_lo) / np.float32(448.0)), np.float32(0.0))
    s_hi = np.where(amax_hi > 0, _up(_up(amax_hi) / np.float32(448.0)), np.float32(1.0))
    zero_possible = amax_lo == 0
    ok = ((s_lo <= scales) & (scales <= s_hi)) | (zero_possible & (scales == np.float32(1.0)))
    ok &= np.isfinite(scales) & (scales > 0)
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError(f"fp8 scale outside the admissible interval at {i}: got {scales[i]!r}, "
                             f"interval [{s_lo[i]!r}, {s_hi[i]!r}]; {int((~ok).sum())} such rows")
    s = scales.astype(np.float32)[..., None]
    q_lo = _down(_down(Y - E).astype(np.float64) / s.astype(np.float64))
    q_hi = _up(_up(Y + E).astype(np.float64) / s.astype(np.float64))
    lo = _e4m3(ob.e4m3fn_encode(q_lo))
    hi = _e4m3(ob.e4m3fn_encode(q_hi))
    got = _e4m3(codes)
    bad = ~((lo <= got) & (got <= hi)) | np.isnan(got)
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"fp8 code outside the admissible interval at {i}: got {got[i]!r} "
                             f"(code {int(codes[i]):#04x}), interval [{lo[i]!r}, {hi[i]!r}], "
                             f"Y/scale {Y[i] / float(s[i[:-1]][0])!r}; {int(bad.sum())} such elements")
    own_codes, own_scales = ob.quantize_rows(Y.astype(np.float32))
    differ = (_e4m3(own_codes) != got)
    return int((lo != hi).sum()), int(differ.sum())
