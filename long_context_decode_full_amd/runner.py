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
               Hs2Error, hs2_decode_step, hs2_decode_workspace_size, hs2_full_attn_select_timed,
               hs2_kv_bridge, hs2_sparse_attn_timed, hs2_sparse_attn_swa,
               hs2_sparse_attn_swa_workspace_size, hs2_workspace_size, make_bridge_desc,
               make_decode_plan, make_desc)


def _dev(a: np.ndarray, device):
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class HybridBlockDevice:
    def __init__(self, inp: dict, device="cuda", window=128, topk=1024, mode="token",
                 block_size=64, n_blocks=18, with_probs=False, max_ctx_len=None, local_rings=None,
                 local_window=128, flags=0, split_len=0, sparse_split_len=0):
        self.device = torch.device(device)
        q = inp["q_full"]
        B, Lq, Hq, D = q.shape
        Hkv = inp["k"].shape[1]
        cap = inp["k"].shape[2]
        fp8 = inp["k"].dtype == np.uint8
        mctx = int(max_ctx_len if max_ctx_len is not None else max(int(inp["ctx_len"].max()), Lq))
        # "gen1": the first-generation comparator -- block selection, and sparse layers
        # with a separate sliding-window branch over their own local rings
        blockish = mode in ("block", "gen1")
        self.desc = make_desc(B, Lq, Hq, Hkv, cap, mctx, head_dim=D,
                              kv_dtype=HS2_KV_FP8_E4M3FN if fp8 else HS2_KV_BF16,
                              window=window, topk=topk,
                              select_mode=HS2_SELECT_BLOCK if blockish else HS2_SELECT_TOKEN,
                              block_size=block_size, n_blocks=n_blocks, sm_scale=inp["sm_scale"],
                              flags=flags, split_len=split_len, sparse_split_len=sparse_split_len)
        self.S = block_size * n_blocks if blockish else window + topk
        self.gen1 = mode == "gen1"
        self.local_window = local_window
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
        if self.gen1:
            assert local_rings is not None and len(local_rings) == len(self.q_sparse)
            self.local = [dict(k=_dev(r["k"], dv), v=_dev(r["v"], dv),
                               k_scale=_dev(r["k_scale"], dv) if fp8 else None,
                               v_scale=_dev(r["v_scale"], dv) if fp8 else None) for r in local_rings]
            self.local_rows = int(local_rings[0]["k"].shape[2])
        self.alloc_workspace()

    def alloc_workspace(self):
        st, nbytes = hs2_workspace_size(self.desc)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_workspace_size")
        if self.gen1:
            st, n2 = hs2_sparse_attn_swa_workspace_size(self.desc, self.local_window, self.local_rows)
            if st != HS2_OK:
                raise Hs2Error(st, "hs2_sparse_attn_swa_workspace_size")
            nbytes = max(nbytes, n2)
        self.ws_bytes = nbytes
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)

    def full(self, stream=None, events=None):
        """events: optional (begin, end) HIP events recorded around the context scan."""
        st = hs2_full_attn_select_timed(self.desc, self.q_full, self.k, self.v, self.k_scale,
                                        self.v_scale, self.ctx_len, self.out_full, self.idx, self.probs,
                                        self.workspace, self.ws_bytes, stream, events)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_full_attn_select")

    def sparse(self, layer: int, idx=None, stream=None, events=None):
        if self.gen1:
            lr = self.local[layer]
            st = hs2_sparse_attn_swa(self.desc, self.q_sparse[layer], self.k, self.v, self.k_scale,
                                     self.v_scale, self.ctx_len, self.idx if idx is None else idx,
                                     lr["k"], lr["v"], lr["k_scale"], lr["v_scale"], self.local_window,
                                     self.local_rows, self.out_sparse[layer], self.workspace,
                                     self.ws_bytes, stream)
            if st != HS2_OK:
                raise Hs2Error(st, "hs2_sparse_attn_swa")
            return
        st = hs2_sparse_attn_timed(self.desc, self.q_sparse[layer], self.k, self.v, self.k_scale,
                                   self.v_scale, self.ctx_len, self.idx if idx is None else idx,
                                   self.out_sparse[layer], self.workspace, self.ws_bytes, stream, events)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_sparse_attn")

    def step(self, stream=None, scan_events=None, gather_events=None):
        """One Hybrid Block: the full layer, then every sparse layer.  scan_events /
        gather_events: optional (begin, end) HIP events around the context scan / the
        first sparse layer's gather."""
        self.full(stream, scan_events)
        for layer in range(len(self.q_sparse)):
            self.sparse(layer, stream=stream, events=gather_events if layer == 0 else None)

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

    def __init__(self, inp: dict, device="cuda", fill=None, scale_fill=float("nan"), gemv_max_tokens=0):
        w = inp["workload"]
        self.device = torch.device(device)
        self.fp8 = w.kv_dtype == "fp8"
        self.L, self.Hkv, self.B, self.cap, self.D = w.n_layers, w.n_kv_heads, w.batch, w.capacity, w.head_dim
        self.T, self.Hd = w.n_tokens, w.hidden
        self.desc = make_bridge_desc(self.T, self.Hd, self.L, self.Hkv, self.B, self.cap, head_dim=self.D,
                                     kv_dtype=HS2_KV_FP8_E4M3FN if self.fp8 else HS2_KV_BF16,
                                     gemv_max_tokens=gemv_max_tokens)
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


class DecodeLoopDevice:
    """Device state of a multi-step decode through the Cross-Decoder's attention
    (HySparse2 article, section 02: KV Bridging appends each new token's K/V to every
    Full layer's cache; each Hybrid Block's full layer selects, its sparse layers
    reuse the selection).  n_blocks Hybrid Blocks, each with its own cache, all
    starting from the caches of `inp` (as built by workloads.make_inputs); the bridge
    weights `w_bits` [n_blocks, 2, Hkv*128, hidden]; per step the new tokens' source
    rows and every layer's queries are copied into fixed input slots, so one step can
    be captured in a HIP graph and replayed (hs2_decode_step enqueues only kernels)."""

    def __init__(self, inp: dict, n_blocks: int, w_bits: np.ndarray, device="cuda",
                 max_ctx_len=None, window=128, topk=1024, flags=0):
        self.device = dv = torch.device(device)
        B, Lq, Hq, D = inp["q_full"].shape
        assert Lq == 1, "decode: one query token per sequence"
        Hkv, cap = inp["k"].shape[1], inp["k"].shape[2]
        self.fp8 = inp["k"].dtype == np.uint8
        self.B, self.Hq, self.Hkv, self.cap, self.D = B, Hq, Hkv, cap, D
        self.nb, self.ns = n_blocks, len(inp["q_sparse"])
        self.hidden = w_bits.shape[-1]
        mctx = int(max_ctx_len if max_ctx_len is not None else cap)
        self.desc = make_desc(B, 1, Hq, Hkv, cap, mctx, head_dim=D,
                              kv_dtype=HS2_KV_FP8_E4M3FN if self.fp8 else HS2_KV_BF16,
                              window=window, topk=topk, sm_scale=inp["sm_scale"], flags=flags)
        self.plan = make_decode_plan(self.desc, n_blocks, self.ns, self.hidden)
        k0, v0 = _dev(inp["k"], dv), _dev(inp["v"], dv)
        self.k = [k0.clone() for _ in range(n_blocks)]
        self.v = [v0.clone() for _ in range(n_blocks)]
        if self.fp8:
            ks0, vs0 = _dev(inp["k_scale"], dv), _dev(inp["v_scale"], dv)
            self.ks = [ks0.clone() for _ in range(n_blocks)]
            self.vs = [vs0.clone() for _ in range(n_blocks)]
        else:
            self.ks = self.vs = None
        del k0, v0
        self.ctx_len = _dev(inp["ctx_len"].astype(np.int32), dv)
        self.w = _dev(w_bits, dv)
        self.x = torch.zeros((B, self.hidden), dtype=torch.int16, device=dv)
        self.q_full = [torch.zeros((B, 1, Hq, D), dtype=torch.int16, device=dv) for _ in range(n_blocks)]
        self.q_sparse = [torch.zeros((B, 1, Hq, D), dtype=torch.int16, device=dv)
                         for _ in range(n_blocks * self.ns)]
        self.out_full = [torch.zeros((B, 1, Hq, D), dtype=torch.float32, device=dv) for _ in range(n_blocks)]
        self.idx = [torch.full((B, 1, Hkv, window + topk), -7, dtype=torch.int32, device=dv)
                    for _ in range(n_blocks)]
        self.out_sparse = [torch.zeros((B, 1, Hq, D), dtype=torch.float32, device=dv)
                           for _ in range(n_blocks * self.ns)]
        st, nbytes = hs2_decode_workspace_size(self.plan)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_decode_workspace_size")
        self.ws_bytes = nbytes
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dv)

    def set_inputs(self, x_bits, q_full_bits, q_sparse_bits):
        """x_bits [B, hidden]; q_full_bits: n_blocks arrays [B, 1, Hq, D]; q_sparse_bits:
        n_blocks * n_sparse arrays (block-major) -- copied into the input slots."""
        self.x.copy_(torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)))
        for dst, src in zip(self.q_full, q_full_bits):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.int16)))
        for dst, src in zip(self.q_sparse, q_sparse_bits):
            dst.copy_(torch.from_numpy(np.ascontiguousarray(src).view(np.int16)))

    def step(self, stream=None):
        st = hs2_decode_step(self.plan, self.x, self.w, self.q_full, self.q_sparse, self.k, self.v,
                             self.ks, self.vs, self.ctx_len, self.out_full, self.idx, self.out_sparse,
                             self.workspace, self.ws_bytes, stream)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_decode_step")

    def full_layer(self, l: int, events=None, stream=None):
        """Block l's full layer alone (hs2_full_attn_select on the block's cache, query
        slot, outputs and the step's workspace), with optional (begin, end) events around
        its context scan -- for timing the scan outside a captured step."""
        ks = self.ks[l] if self.fp8 else None
        vs = self.vs[l] if self.fp8 else None
        st = hs2_full_attn_select_timed(self.desc, self.q_full[l], self.k[l], self.v[l], ks, vs,
                                        self.ctx_len, self.out_full[l], self.idx[l], None,
                                        self.workspace, self.ws_bytes, stream, events)
        if st != HS2_OK:
            raise Hs2Error(st, "hs2_full_attn_select")

    def capture(self):
        """One step captured into a HIP graph (torch.cuda.CUDAGraph); nothing runs until
        replay().  The graph reads the input slots and the device-side ctx_len."""
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize(self.device)
        with torch.cuda.graph(g):
            self.step()
        torch.cuda.synchronize(self.device)
        return g

    def state(self) -> dict:
        torch.cuda.synchronize(self.device)
        out = dict(ctx_len=self.ctx_len.cpu().numpy(),
                   out_full=[o.cpu().numpy() for o in self.out_full],
                   idx=[i.cpu().numpy() for i in self.idx],
                   out_sparse=[o.cpu().numpy() for o in self.out_sparse])
        return out

    def block_inputs(self, l: int, q_full_bits, q_sparse_bits) -> dict:
        """Block l's caches as they are now, with the given queries, in the layout of
        workloads.make_inputs (for the oracle)."""
        torch.cuda.synchronize(self.device)
        kt = np.uint8 if self.fp8 else np.uint16
        d = dict(q_full=np.asarray(q_full_bits), q_sparse=[np.asarray(q) for q in q_sparse_bits],
                 k=self.k[l].cpu().numpy().view(kt), v=self.v[l].cpu().numpy().view(kt),
                 k_scale=self.ks[l].cpu().numpy() if self.fp8 else None,
                 v_scale=self.vs[l].cpu().numpy() if self.fp8 else None,
                 ctx_len=self.ctx_len.cpu().numpy(), capacity=self.cap,
                 sm_scale=float(self.desc.sm_scale))
        return d
