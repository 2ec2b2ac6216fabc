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
               Hs2Error, hs2_full_attn_select, hs2_sparse_attn, hs2_workspace_size, make_desc)


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
