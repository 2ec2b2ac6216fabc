"""Comparison rules between the HIP path and the CPU oracle (test infrastructure).

Outputs (float32 from the GPU vs float64 oracle): per row (b, j, h) the max abs
difference over the 128 dims divided by the row's max |reference| must not exceed
2e-3 (fp32 accumulate); a row whose reference is all zero must be all zero.

Index sets: the GPU row and the oracle row must hold the same number of valid
positions, be ascending without duplicates and -1 padded, contain the forced
window, and may differ only by positions whose oracle score lies within 1e-6
(relative) of the oracle's k-th largest candidate score.  Block rows: same
count, and differing blocks must have oracle block masses within 1e-6 relative
of the n_blocks-th mass.

The selection is an integer decision taken from floating-point scores, so the
comparison takes it in the kernel's precision: the oracle's float64 scores are
rounded to float32 and values below the smallest normal float32 are flushed to
zero (the kernel's exp2 does not produce subnormals) before the k-th value and
the band are evaluated.  Probabilities that small (e.g. 1e-72 next to a
dominant key) are all zero in float32, and then the lower-position tie rule
decides on both sides -- and is checked: when the rows differ, the GPU's choice
must be the top-k by (score desc, position asc) for SOME scores within the band
of the kernel-precision ones.  Each candidate gets the interval
[s32 (1 - band), s32 (1 + band)] (lower end 0 for scores at the edge of the
float32 range, which the kernel may flush), and no unselected candidate may
beat a selected one for every choice in the intervals: an unselected u beats a
selected t if lo(u) > hi(t), or lo(u) == hi(t) (a degenerate interval, i.e. an
exact zero on both sides) and u < t.  So among candidates whose score is 0 in
float32, the GPU must pick the lowest positions.
"""
import numpy as np

F32_TINY = float(np.finfo(np.float32).tiny)


def kernel_precision(s):
    """float64 scores as the kernel represents them: float32, subnormals flushed."""
    s32 = np.asarray(s, dtype=np.float64).astype(np.float32).astype(np.float64)
    s32[np.abs(s32) < F32_TINY] = 0.0
    return s32


OUT_TOL = 2e-3
TIE_BAND = 1e-6


def out_row_errors(gpu, ref):
    """Relative error per row over the last axis."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max(axis=-1)
    num = np.abs(gpu - ref).max(axis=-1)
    zero_row_err = np.where(num > 0, np.inf, 0.0)
    return np.where(den > 0, num / np.where(den > 0, den, 1), zero_row_err)


def assert_out_close(gpu, ref, tol=OUT_TOL, what="out"):
    err = out_row_errors(gpu, ref)
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    assert worst <= tol, f"{what}: worst row relative error {worst:.3e} > {tol:.1e}"
    return worst


def order_violation(sel_mask, s32, band=TIE_BAND):
    """First (t, u) with candidate t selected, u not, and u ahead of t in (score desc,
    position asc) order for every score within the band of s32 (see the module
    docstring), or None.  sel_mask: boolean per candidate position; s32:
    kernel-precision scores of the candidates."""
    sel = np.nonzero(sel_mask)[0]
    unsel = np.nonzero(~sel_mask)[0]
    if len(sel) == 0 or len(unsel) == 0:
        return None
    edge = F32_TINY * (1.0 + 4.0 * band)
    h = s32[sel] * (1.0 + band)
    su = s32[unsel]
    l = np.where(su <= edge, 0.0, su * (1.0 - band))
    a, b = h.min(), l.max()
    if a > b:
        return None
    if a < b:
        return int(sel[np.argmin(h)]), int(unsel[np.argmax(l)])
    # a == b: only exact equalities (zeros) remain; positions decide
    t_last = sel[h == a].max()
    u_first = unsel[l == b].min()
    if u_first < t_last:
        return int(t_last), int(u_first)
    return None


def check_idx_row(gpu_row, ref_row, s, n, window, topk, band=TIE_BAND):
    """Returns the number of positions swapped inside the tie band (asserts otherwise)."""
    gpu_row = np.asarray(gpu_row)
    ref_row = np.asarray(ref_row)
    gv = gpu_row[gpu_row >= 0]
    rv = ref_row[ref_row >= 0]
    assert len(gv) == len(rv), f"count {len(gv)} != {len(rv)}"
    assert np.all(gpu_row[len(gv):] == -1), "padding is not -1"
    assert np.all(np.diff(gv) > 0), "not strictly ascending"
    assert gv.max(initial=-1) < n, "position beyond the visible range"
    w0 = max(0, n - window)
    assert set(range(w0, n)) <= set(gv.tolist()), "forced window missing"
    diff = set(gv.tolist()) ^ set(rv.tolist())
    kk = min(topk, w0)
    if kk == w0:
        assert not diff, "all candidates are selected, no swap is allowed"
        return 0
    s32 = kernel_precision(np.asarray(s)[:w0])
    if not diff and np.count_nonzero(s32 > 0) >= kk:
        # same set as the oracle, whose float64 order is consistent with every band
        return 0
    vk = np.sort(s32)[::-1][kk - 1]
    edge = F32_TINY * (1.0 + 4.0 * band)
    for t in diff:
        assert t < w0, f"window position {t} differs"
        near = abs(s32[t] - vk) <= band * vk or (vk == 0.0 and s32[t] <= edge)
        assert near, f"swap at {t}: score {s[t]!r} vs k-th {vk!r}"
    sel_mask = np.zeros(w0, dtype=bool)
    sel_mask[gv[gv < w0]] = True
    bad = order_violation(sel_mask, s32, band)
    assert bad is None, (f"tie order: position {bad[0]} selected over {bad[1]} "
                         f"(scores {s32[bad[0]]!r}, {s32[bad[1]]!r}, k-th {vk!r})")
    return len(diff) // 2


def check_block_row(gpu_row, ref_row, s, n, block, n_blocks, band=TIE_BAND):
    gpu_row = np.asarray(gpu_row)
    ref_row = np.asarray(ref_row)
    gv = gpu_row[gpu_row >= 0]
    rv = ref_row[ref_row >= 0]
    assert np.all(gpu_row[len(gv):] == -1)
    assert np.all(np.diff(gv) > 0)
    gb = sorted(set((gv // block).tolist()))
    rb = sorted(set((rv // block).tolist()))
    assert len(gb) == len(rb)
    for b in gb:   # every chosen block is expanded to all its visible positions
        assert set(range(b * block, min((b + 1) * block, n))) <= set(gv.tolist())
    diff = set(gb) ^ set(rb)
    if not diff:
        return 0
    nb = (n + block - 1) // block
    s32 = kernel_precision(s)
    mass = np.array([np.sum(s32[b * block: min((b + 1) * block, n)]) for b in range(nb)])
    mk = np.sort(mass)[::-1][min(n_blocks, nb) - 1]
    for b in diff:
        assert abs(mass[b] - mk) <= band * mk, f"block swap {b}: {mass[b]!r} vs {mk!r}"
    return len(diff) // 2
