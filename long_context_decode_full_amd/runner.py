"""Device-side plumbing for one Hybrid Block: torch allocates and uploads the buffers,
the C ABI of libhs2.so does all of the computation.

HybridBlockDevice owns the device copies of one set of inputs (as built by
workloads.make_inputs), the outputs and the workspace, and runs
hs2_full_attn_select followed by one hs2_sparse_attn per sparse layer, all on
one stream (HySparse2 article, section 02 "KV Reuse": every sparse layer reuses
the full layer's KV cache and index set).
"""
from __future__ import annotations

import numpy as np
import torch

from . import (HS2_KV_BF16, HS2_KV_FP8_E4M3FN, HS2_OK, HS2_SELECT_BLOCK, HS2_SELECT_TOKEN,
               Hs2Error, hs2_full_attn_select, hs2_kv_bridge, hs2_sparse_attn, hs2_workspace_size,
               make_bridge_desc, make_desc)


def _dev(a: np.ndarray, device):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class HybridBlockDevice:
    def __init__(self, inp: dict, device="cuda", window=128, topk=1024, mode="token",
                 block_size=64, n_blocks=18, with_probs=False, max_ctx_len=None):
        self.device = torch.device(device)
        q = inp["q_full"]
        B, Lq, Hq, D = q.shape
        Hkv = inp["k"].shape[1]
        cap = inp["k"].shape[2]
        fp8 = inp["k"].dtype == np.uint8
        mctx = int(max_ctx_len if max_ctx_len is not None else max(int(inp["ctx_len"].max()), Lq))
        self.desc = make_desc(B, Lq, Hq, Hkv, cap, mctx, head_dim=D,
                              kv_dtype=HS2_KV_FP8_E4M3FN if fp8 else HS2_KV_BF16,
                              window=window, topk=topk,
                              select_mode=HS2_SELECT_BLOCK if mode == "block" else HS2_SELECT_TOKEN,
                              block_size=block_size, n_blocks=n_blocks, sm_scale=inp["sm_scale"])
        self.S = block_size * n_blocks if mode == "block" else window + topk
        dv = self.device
        self.q_full = _dev(q, dv)
        self.q_sparse = [_dev(x, dv) for x in inp["q_sparse"]]
        self.k = _dev(inp["k"], dv)
        self.v = _dev(inp["v"], dv)
        self.k_scale = _dev(inp["k_scale"], dv) if fp8 else None
        self.v_scale = _dev(inp["v_scale"], dv) if fp8 else None
        self.ctx_len = _dev(inp["ctx_len"].astype(np.int32), dv)
        self.out_full = torch.zeros((B, Lq, Hq, D), dtype=torch.float32, device=dv)
        self.idx = torch.full((B, Lq, Hkv, self.S), -7, dtype=torch.int32, device=dv)
        self.probs = (torch.full((B, Lq, Hkv, cap), -1.0, dtype=torch.float32, device=dv)
                      if with_probs else None)
        self.out_sparse = [torch.zeros_like(self.out_full) for _ in self.q_sparse]
        self.alloc_workspace()

    def alloc_workspace(self):
        st, nbytes = hs2_workspace_size(self.desc)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_workspace_size")
        self.ws_bytes = nbytes
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)

    def full(self, stream=None):
        st = hs2_full_attn_select(self.desc, self.q_full, self.k, self.v, self.k_scale,
                                  self.v_scale, self.ctx_len, self.out_full, self.idx, self.probs,
                                  self.workspace, self.ws_bytes, stream)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_full_attn_select")

    def sparse(self, layer: int, idx=None, stream=None):
        st = hs2_sparse_attn(self.desc, self.q_sparse[layer], self.k, self.v, self.k_scale,
                             self.v_scale, self.ctx_len, self.idx if idx is None else idx,
                             self.out_sparse[layer], self.workspace, self.ws_bytes, stream)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_sparse_attn")

    def step(self, stream=None):
        self.full(stream)
        for layer in range(len(self.q_sparse)):
            self.sparse(layer, stream=stream)

    def results(self) -> dict:
        torch.cuda.synchronize(self.device)
        return dict(out_full=self.out_full.cpu().numpy(), idx=self.idx.cpu().numpy(),
                    probs=None if self.probs is None else self.probs.cpu().numpy(),
                    out_sparse=[o.cpu().numpy() for o in self.out_sparse])


class BridgeDevice:
    """Device buffers of one KV Bridging call (HySparse2 article, section 02 "KV
    Bridging"): the source hidden state, the projection weights of every target layer,
    the destinations, and one K and one V cache (plus scales for fp8) per target layer.
    The caches start filled with `fill` codes (and `scale_fill` scales)."""

    def __init__(self, inp: dict, device="cuda", fill=None, scale_fill=float("nan")):
        w = inp["workload"]
        self.device = torch.device(device)
        self.fp8 = w.kv_dtype == "fp8"
        self.L, self.Hkv, self.B, self.cap, self.D = w.n_layers, w.n_kv_heads, w.batch, w.capacity, w.head_dim
        self.T, self.Hd = w.n_tokens, w.hidden
        self.desc = make_bridge_desc(self.T, self.Hd, self.L, self.Hkv, self.B, self.cap, head_dim=self.D,
                                     kv_dtype=HS2_KV_FP8_E4M3FN if self.fp8 else HS2_KV_BF16)
        dv = self.device
        self.x = _dev(inp["x"], dv)
        self.w = _dev(inp["weight"], dv)
        self.seq = _dev(inp["seq"].astype(np.int32), dv)
        self.pos = _dev(inp["pos"].astype(np.int32), dv)
        shape = (self.B, self.Hkv, self.cap, self.D)
        if self.fp8:
            code = 0x7F if fill is None else int(fill)
            self.k = [torch.full(shape, code, dtype=torch.uint8, device=dv) for _ in range(self.L)]
            self.v = [torch.full(shape, code, dtype=torch.uint8, device=dv) for _ in range(self.L)]
            self.ks = [torch.full(shape[:3], scale_fill, dtype=torch.float32, device=dv) for _ in range(self.L)]
            self.vs = [torch.full(shape[:3], scale_fill, dtype=torch.float32, device=dv) for _ in range(self.L)]
        else:
            code = 0x7FC0 if fill is None else int(fill)
            code = code - 0x10000 if code >= 0x8000 else code
            self.k = [torch.full(shape, code, dtype=torch.int16, device=dv) for _ in range(self.L)]
            self.v = [torch.full(shape, code, dtype=torch.int16, device=dv) for _ in range(self.L)]
            self.ks = self.vs = None

    def run(self, stream=None):
        st = hs2_kv_bridge(self.desc, self.x, self.w, self.seq, self.pos, self.k, self.v,
                           self.ks, self.vs, stream)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_kv_bridge")

    def rows(self, tokens) -> dict:
        """Cache rows of the given tokens (which must have valid destinations):
        codes [n, L, 2, Hkv, D] (uint8 or uint16 bits) and, for fp8, scales [n, L, 2, Hkv]."""
        torch.cuda.synchronize(self.device)
        t = torch.as_tensor(np.asarray(tokens, dtype=np.int64), device=self.device)
        s = self.seq.long()[t]
        p = self.pos.long()[t]
        codes = torch.stack([torch.stack([c[l][s, :, p] for c in (self.k, self.v)], 1)
                             for l in range(self.L)], 1)
        out = dict(codes=codes.cpu().numpy())
        if not self.fp8:
            out["codes"] = out["codes"].view(np.uint16)
        else:
            out["scales"] = torch.stack([torch.stack([c[l][s, :, p] for c in (self.ks, self.vs)], 1)
                                         for l in range(self.L)], 1).cpu().numpy()
        return out

    def caches(self) -> dict:
        """Whole caches on the host, stacked over layers: k, v [L, B, Hkv, cap, D] (and
        k_scale, v_scale [L, B, Hkv, cap] for fp8); for small cases only."""
        torch.cuda.synchronize(self.device)
        k = torch.stack(self.k).cpu().numpy()
        v = torch.stack(self.v).cpu().numpy()
        if not self.fp8:
            return dict(k=k.view(np.uint16), v=v.view(np.uint16))
        return dict(k=k, v=v, k_scale=torch.stack(self.ks).cpu().numpy(),
                    v_scale=torch.stack(self.vs).cpu().numpy())
