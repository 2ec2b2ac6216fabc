"""Guard bands: every output of a Hybrid Block step (out, idx, probs, each sparse
layer's out) and the workspace sit inside larger device buffers whose margins hold a
sentinel pattern; after the step the margins must be untouched, and the outputs must
equal those of a run on ordinary buffers.  Catches a kernel writing past the end (or
before the start) of what the C ABI gives it, on every selection and sparse-layer
path.  Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

from long_context_decode_full_amd import (HS2_FLAG_SPARSE_FUSED, HS2_FLAG_SPARSE_HEAD,
                                          HS2_FLAG_SPARSE_SPLIT)
from long_context_decode_full_amd import workloads as wl

pytestmark = pytest.mark.gpu

GUARD = 4096                      # elements (bytes for the workspace) on each side
F32_SENTINEL = 0x7FA5A5A5         # a NaN payload no kernel produces
I32_SENTINEL = 0x5A5A5A5A
U8_SENTINEL = 0xA5


@pytest.fixture(autouse=True)
def _gpu_only():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _guarded(t: torch.Tensor):
    """A buffer of t's dtype with GUARD elements on each side, filled with the sentinel,
    and the view of t's shape inside it (its contents copied from t)."""
    n = t.numel()
    buf = torch.empty(n + 2 * GUARD, dtype=t.dtype, device=t.device)
    if t.dtype == torch.uint8:
        buf.fill_(U8_SENTINEL)
    else:
        buf.view(torch.int32).fill_(F32_SENTINEL if t.dtype == torch.float32 else I32_SENTINEL)
    view = buf[GUARD:GUARD + n].view(t.shape)
    view.copy_(t)
    return buf, view


def _margins_intact(buf: torch.Tensor, what: str):
    if buf.dtype == torch.uint8:
        lo, hi, want = buf[:GUARD], buf[-GUARD:], U8_SENTINEL
    else:
        bits = buf.view(torch.int32)
        lo, hi = bits[:GUARD], bits[-GUARD:]
        want = F32_SENTINEL if buf.dtype == torch.float32 else I32_SENTINEL
        want = np.array([want], dtype=np.uint32).view(np.int32)[0]
    lo, hi = lo.cpu().numpy(), hi.cpu().numpy()
    bad_lo, bad_hi = np.flatnonzero(lo != want), np.flatnonzero(hi != want)
    assert bad_lo.size == 0, f"{what}: {bad_lo.size} elements written before the buffer (first at -{GUARD - bad_lo[-1]})"
    assert bad_hi.size == 0, f"{what}: {bad_hi.size} elements written past the end (first at +{bad_hi[0]})"


CASES = {
    "decode-head": (wl.Workload("guard decode", 2, 1, 16, 2, ctx_lens=[3000, 700], n_needles=4, seed=4100),
                    dict()),
    "decode-split": (wl.Workload("guard decode", 2, 1, 16, 2, ctx_lens=[3000, 700], n_needles=4, seed=4100),
                     dict(flags=HS2_FLAG_SPARSE_SPLIT)),
    "decode-fused": (wl.Workload("guard decode", 2, 1, 16, 2, ctx_lens=[3000, 700], n_needles=4, seed=4100),
                     dict(flags=HS2_FLAG_SPARSE_FUSED)),
    "fp8-probs": (wl.Workload("guard fp8", 2, 1, 32, 4, ctx_lens=[4100, 900], n_needles=4, kv_dtype="fp8",
                              seed=4110), dict(with_probs=True)),
    "mqa-probs": (wl.Workload("guard mqa", 1, 1, 32, 1, ctx_lens=[5000], n_needles=4, seed=4120),
                  dict(with_probs=True)),
    "chunk": (wl.Workload("guard chunk", 2, 64, 32, 4, ctx_lens=[64, 3000], n_needles=4, seed=4130), dict()),
    "chunk-head": (wl.Workload("guard chunk", 2, 64, 32, 4, ctx_lens=[64, 3000], n_needles=4, seed=4130),
                   dict(flags=HS2_FLAG_SPARSE_HEAD)),
    "block-decode": (wl.Workload("guard block", 2, 1, 32, 4, ctx_lens=[9000, 2000], n_needles=4, seed=4140),
                     dict(mode="block")),
    "block-chunk": (wl.Workload("guard block chunk", 2, 64, 32, 4, ctx_lens=[64, 5000], n_needles=4,
                                seed=4150), dict(mode="block")),
}


@pytest.mark.parametrize("name", list(CASES))
def test_outputs_stay_inside_their_buffers(name):
    from long_context_decode_full_amd.runner import HybridBlockDevice
    w, kw = CASES[name]
    print(f"\n[gpu case] guard-{name}: B={w.batch} Lq={w.q_len} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
          f"ctx={w.ctx_lens} kv={w.kv_dtype} seed={w.seed} {kw}", flush=True)
    inp = wl.make_inputs(w)

    plain = HybridBlockDevice(inp, **kw)
    plain.step()
    want = plain.results()

    dev = HybridBlockDevice(inp, **kw)
    bufs = {}
    bufs["out_full"], dev.out_full = _guarded(dev.out_full)
    bufs["idx"], dev.idx = _guarded(dev.idx)
    if dev.probs is not None:
        bufs["probs"], dev.probs = _guarded(dev.probs)
    for layer in range(len(dev.out_sparse)):
        bufs[f"out_sparse{layer}"], dev.out_sparse[layer] = _guarded(dev.out_sparse[layer])
    bufs["workspace"], ws = _guarded(dev.workspace[:dev.ws_bytes])
    dev.workspace = ws
    dev.step()
    got = dev.results()

    for what, buf in bufs.items():
        _margins_intact(buf, what)
    assert np.array_equal(got["idx"], want["idx"])
    np.testing.assert_allclose(got["out_full"], want["out_full"], rtol=1e-5, atol=1e-6)
    for layer in range(len(want["out_sparse"])):
        # the sparse layers are bitwise reproducible for equal index sets
        assert np.array_equal(got["out_sparse"][layer], want["out_sparse"][layer]), f"sparse layer {layer}"
    if want["probs"] is not None:
        ok = want["probs"] >= 0
        np.testing.assert_allclose(got["probs"][ok], want["probs"][ok], rtol=1e-5, atol=1e-12)
