"""HySparse2 Hybrid-Block decode for MI355X (gfx950): Python binding of libhs2.so.

The binding only marshals arguments (descriptor struct, device pointers, stream)
into the C ABI declared in include/hs2.h; every step of the computation runs in
the HIP kernels of libhs2.so.  There is no fallback: if the library is missing,
every call raises.

Pointer arguments accept a torch tensor (its data_ptr() is passed), a plain
integer address, or None (NULL).  `stream` accepts a torch.cuda.Stream, a raw
hipStream_t integer, or None for torch's current stream.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "HS2_OK", "HS2_ERR_INVALID_ARG", "HS2_ERR_UNSUPPORTED", "HS2_ERR_WORKSPACE",
    "HS2_ERR_ALIGNMENT", "HS2_ERR_LAUNCH", "HS2_KV_BF16", "HS2_KV_FP8_E4M3FN",
    "HS2_SELECT_TOKEN", "HS2_SELECT_BLOCK", "Hs2AttnDesc", "Hs2Error", "make_desc",
    "hs2_validate", "hs2_workspace_size", "hs2_full_attn_select", "hs2_sparse_attn",
    "hs2_status_string", "hs2_full_attn_select_timed", "hs2_sparse_attn_timed", "Hs2KernelEvents",
    "hs2_build_id", "HS2_FLAG_DETERMINISTIC", "HS2_FLAG_FORCE_LOGITS", "HS2_FLAG_SCAN_VALU",
    "HS2_FLAG_CHUNK_PER_TOKEN", "HS2_FLAG_SPARSE_FUSED", "HS2_FLAG_SPARSE_SPLIT", "HS2_FLAG_SPARSE_HEAD", "HS2_FLAG_EXACT_PV",
    "HS2_FLAGS_ALL",
    "library_path", "load_library", "Hs2BridgeDesc", "make_bridge_desc",
    "hs2_kv_bridge", "Hs2DecodePlan", "make_decode_plan", "hs2_decode_workspace_size",
    "hs2_decode_step", "hs2_sparse_attn_swa_workspace_size", "hs2_sparse_attn_swa",
    "EXPORTED_SYMBOLS", "SIZE_MAX", "hs2_full_attn_select_noalloc", "HS2_ERR_SCRATCH_LIMIT",
    "HS2_NOALLOC_SCRATCH_BYTES",
]

HS2_OK = 0
HS2_ERR_INVALID_ARG = 1
HS2_ERR_UNSUPPORTED = 2
HS2_ERR_WORKSPACE = 3
HS2_ERR_ALIGNMENT = 4
HS2_ERR_LAUNCH = 5
HS2_ERR_SCRATCH_LIMIT = 6
HS2_NOALLOC_SCRATCH_BYTES = 64 << 20
HS2_KV_BF16 = 0
HS2_KV_FP8_E4M3FN = 1
HS2_SELECT_TOKEN = 0
HS2_SELECT_BLOCK = 1
# hs2_attn_desc.flags
HS2_FLAG_DETERMINISTIC = 1 << 0
HS2_FLAG_FORCE_LOGITS = 1 << 1
HS2_FLAG_SCAN_VALU = 1 << 2
HS2_FLAG_CHUNK_PER_TOKEN = 1 << 3
HS2_FLAG_SPARSE_FUSED = 1 << 4
HS2_FLAG_SPARSE_SPLIT = 1 << 5
HS2_FLAG_SPARSE_HEAD = 1 << 6
HS2_FLAG_EXACT_PV = 1 << 7
HS2_FLAGS_ALL = 0xFF
SIZE_MAX = (1 << 64) - 1

EXPORTED_SYMBOLS = ("hs2_validate", "hs2_workspace_size", "hs2_full_attn_select",
                    "hs2_sparse_attn", "hs2_status_string", "hs2_full_attn_select_timed",
                    "hs2_sparse_attn_timed", "hs2_build_id", "hs2_kv_bridge",
                    "hs2_decode_workspace_size", "hs2_decode_step",
                    "hs2_sparse_attn_swa_workspace_size", "hs2_sparse_attn_swa",
                    "hs2_full_attn_select_noalloc")


class Hs2AttnDesc(ctypes.Structure):
    """Mirror of hs2_attn_desc (include/hs2.h)."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int64),
        ("max_ctx_len", ctypes.c_int64),
        ("window", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("select_mode", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("split_len", ctypes.c_int32),
        ("sparse_split_len", ctypes.c_int32),
        ("cand_workgroups", ctypes.c_int32),
    ]


class Hs2BridgeDesc(ctypes.Structure):
    """Mirror of hs2_bridge_desc (include/hs2.h)."""
    _fields_ = [
        ("n_tokens", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("n_layers", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int64),
        ("gemv_max_tokens", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def make_bridge_desc(n_tokens, hidden, n_layers, n_kv_heads, batch, kv_capacity, head_dim=128,
                     kv_dtype=HS2_KV_FP8_E4M3FN, gemv_max_tokens=0) -> Hs2BridgeDesc:
    return Hs2BridgeDesc(int(n_tokens), int(hidden), int(n_layers), int(n_kv_heads), int(head_dim),
                         int(kv_dtype), int(batch), int(kv_capacity), int(gemv_max_tokens), 0)


class Hs2KernelEvents(ctypes.Structure):
    """Mirror of hs2_kernel_events (include/hs2.h): two caller-owned hipEvent_t."""
    _fields_ = [("begin", ctypes.c_void_p), ("end", ctypes.c_void_p)]


class Hs2DecodePlan(ctypes.Structure):
    """Mirror of hs2_decode_plan (include/hs2.h)."""
    _fields_ = [
        ("attn", Hs2AttnDesc),
        ("n_blocks", ctypes.c_int32),
        ("n_sparse", ctypes.c_int32),
        ("hidden", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


def make_decode_plan(attn: Hs2AttnDesc, n_blocks, n_sparse, hidden) -> Hs2DecodePlan:
    return Hs2DecodePlan(attn, int(n_blocks), int(n_sparse), int(hidden), 0)


class Hs2Error(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = status
        super().__init__(f"{where}: {hs2_status_string(status)} (status {status})")


def make_desc(batch, q_len, n_q_heads, n_kv_heads, kv_capacity, max_ctx_len, head_dim=128,
              kv_dtype=HS2_KV_BF16, window=128, topk=1024, select_mode=HS2_SELECT_TOKEN,
              block_size=64, n_blocks=18, sm_scale=None, flags=0, split_len=0, sparse_split_len=0,
              cand_workgroups=0) -> Hs2AttnDesc:
    return Hs2AttnDesc(int(batch), int(q_len), int(n_q_heads), int(n_kv_heads), int(head_dim),
                       int(kv_dtype), int(kv_capacity), int(max_ctx_len), int(window), int(topk),
                       int(select_mode), int(block_size), int(n_blocks),
                       float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(head_dim)),
                       int(flags), int(split_len), int(sparse_split_len), int(cand_workgroups))


# --------------------------------------------------------------------------- loading
_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhs2.so")


def load_library(path=None):
    """Load libhs2.so (built in-tree by build.py), or the library at `path` (a host-only
    build for sanitizer tests) if none is loaded yet.  Raises if it is absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    D = ctypes.POINTER(Hs2AttnDesc)
    E = ctypes.POINTER(Hs2KernelEvents)
    lib.hs2_validate.argtypes = [D, ctypes.c_size_t]
    lib.hs2_validate.restype = ctypes.c_int
    lib.hs2_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.hs2_workspace_size.restype = ctypes.c_int
    lib.hs2_full_attn_select.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hs2_full_attn_select.restype = ctypes.c_int
    lib.hs2_sparse_attn.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.hs2_sparse_attn.restype = ctypes.c_int
    lib.hs2_full_attn_select_timed.argtypes = [D, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, E]
    lib.hs2_full_attn_select_timed.restype = ctypes.c_int
    lib.hs2_sparse_attn_timed.argtypes = [D, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, E]
    lib.hs2_sparse_attn_timed.restype = ctypes.c_int
    lib.hs2_full_attn_select_noalloc.argtypes = [D, P, P, P, P, P, P, P, P, P, P]
    lib.hs2_full_attn_select_noalloc.restype = ctypes.c_int
    lib.hs2_build_id.argtypes = []
    lib.hs2_build_id.restype = ctypes.c_char_p
    lib.hs2_kv_bridge.argtypes = [ctypes.POINTER(Hs2BridgeDesc), P, P, P, P, P, P, P, P, P]
    lib.hs2_kv_bridge.restype = ctypes.c_int
    lib.hs2_decode_workspace_size.argtypes = [ctypes.POINTER(Hs2DecodePlan), ctypes.POINTER(ctypes.c_size_t)]
    lib.hs2_decode_workspace_size.restype = ctypes.c_int
    lib.hs2_decode_step.argtypes = [ctypes.POINTER(Hs2DecodePlan), P, P, P, P, P, P, P, P, P, P, P, P,
                                    P, ctypes.c_size_t, P]
    lib.hs2_decode_step.restype = ctypes.c_int
    lib.hs2_sparse_attn_swa_workspace_size.argtypes = [D, ctypes.c_int32, ctypes.c_int32,
                                                       ctypes.POINTER(ctypes.c_size_t)]
    lib.hs2_sparse_attn_swa_workspace_size.restype = ctypes.c_int
    lib.hs2_sparse_attn_swa.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32,
                                        P, P, ctypes.c_size_t, P]
    lib.hs2_sparse_attn_swa.restype = ctypes.c_int
    lib.hs2_status_string.argtypes = [ctypes.c_int]
    lib.hs2_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


# --------------------------------------------------------------------------- C ABI
def hs2_validate(desc: Hs2AttnDesc, workspace_bytes: int = SIZE_MAX) -> int:
    """Checks the descriptor and that workspace_bytes covers its workspace (the default
    SIZE_MAX checks the descriptor alone)."""
    return load_library().hs2_validate(ctypes.byref(desc), int(workspace_bytes))


def hs2_workspace_size(desc: Hs2AttnDesc):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = load_library().hs2_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    return st, n.value


def hs2_full_attn_select(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, probs,
                         workspace, workspace_bytes, stream=None) -> int:
    return load_library().hs2_full_attn_select(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
        _ptr(ctx_len), _ptr(out), _ptr(idx), _ptr(probs), _ptr(workspace),
        int(workspace_bytes), _stream(stream))


def hs2_sparse_attn(desc, q, k, v, k_scale, v_scale, ctx_len, idx, out, workspace,
                    workspace_bytes, stream=None) -> int:
    return load_library().hs2_sparse_attn(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
        _ptr(ctx_len), _ptr(idx), _ptr(out), _ptr(workspace), int(workspace_bytes),
        _stream(stream))


def hs2_full_attn_select_noalloc(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, probs,
                                 stream=None) -> int:
    """hs2_full_attn_select over the library's own scratch: no workspace argument."""
    return load_library().hs2_full_attn_select_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
        _ptr(ctx_len), _ptr(out), _ptr(idx), _ptr(probs), _stream(stream))


def _events(events):
    """(begin, end) hipEvent_t handles (ints, or objects with a `cuda_event` handle such
    as a recorded torch.cuda.Event) -> Hs2KernelEvents, or None."""
    if events is None:
        return None
    b, e = (x if isinstance(x, int) else x.cuda_event for x in events)
    return Hs2KernelEvents(b, e)


def hs2_full_attn_select_timed(desc, q, k, v, k_scale, v_scale, ctx_len, out, idx, probs,
                               workspace, workspace_bytes, stream=None, events=None) -> int:
    """hs2_full_attn_select recording events = (begin, end) around its context scan."""
    ev = _events(events)
    return load_library().hs2_full_attn_select_timed(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
        _ptr(ctx_len), _ptr(out), _ptr(idx), _ptr(probs), _ptr(workspace),
        int(workspace_bytes), _stream(stream), ctypes.byref(ev) if ev is not None else None)


def hs2_sparse_attn_timed(desc, q, k, v, k_scale, v_scale, ctx_len, idx, out, workspace,
                          workspace_bytes, stream=None, events=None) -> int:
    """hs2_sparse_attn recording events = (begin, end) around its gather kernel."""
    ev = _events(events)
    return load_library().hs2_sparse_attn_timed(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale),
        _ptr(ctx_len), _ptr(idx), _ptr(out), _ptr(workspace), int(workspace_bytes),
        _stream(stream), ctypes.byref(ev) if ev is not None else None)


def _ptr_array(xs):
    """A host array of device pointers (void* const*), or None for NULL."""
    if xs is None:
        return None
    arr = (ctypes.c_void_p * max(1, len(xs)))(*[_ptr(x) for x in xs])
    return arr


def hs2_kv_bridge(desc, x, w, seq, pos, k_caches, v_caches, k_scales=None, v_scales=None,
                  stream=None) -> int:
    """k_caches / v_caches (and k_scales / v_scales for fp8): one tensor or device
    address per target layer, passed to the library as host arrays of pointers."""
    ka, va = _ptr_array(k_caches), _ptr_array(v_caches)
    ksa, vsa = _ptr_array(k_scales), _ptr_array(v_scales)
    return load_library().hs2_kv_bridge(
        ctypes.byref(desc), _ptr(x), _ptr(w), _ptr(seq), _ptr(pos),
        ctypes.cast(ka, ctypes.c_void_p) if ka is not None else None,
        ctypes.cast(va, ctypes.c_void_p) if va is not None else None,
        ctypes.cast(ksa, ctypes.c_void_p) if ksa is not None else None,
        ctypes.cast(vsa, ctypes.c_void_p) if vsa is not None else None,
        _stream(stream))


def hs2_decode_workspace_size(plan):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = load_library().hs2_decode_workspace_size(ctypes.byref(plan), ctypes.byref(n))
    return st, n.value


def hs2_decode_step(plan, x, w, q_full, q_sparse, k_caches, v_caches, k_scales, v_scales,
                    ctx_len, out_full, idx, out_sparse, workspace, workspace_bytes,
                    stream=None) -> int:
    """Lists of tensors (or device addresses) are passed as host arrays of pointers.
    The arrays are built here and live only for the call (the library keeps none)."""
    arrays = [_ptr_array(v) for v in (q_full, q_sparse, k_caches, v_caches, k_scales, v_scales,
                                      out_full, idx, out_sparse)]
    ptrs = [ctypes.cast(a, ctypes.c_void_p) if a is not None else None for a in arrays]
    return load_library().hs2_decode_step(
        ctypes.byref(plan), _ptr(x), _ptr(w), ptrs[0], ptrs[1], ptrs[2], ptrs[3], ptrs[4],
        ptrs[5], _ptr(ctx_len), ptrs[6], ptrs[7], ptrs[8], _ptr(workspace), int(workspace_bytes),
        _stream(stream))


def hs2_sparse_attn_swa_workspace_size(desc, local_window, local_rows):
    """Returns (status, bytes)."""
    n = ctypes.c_size_t(0)
    st = load_library().hs2_sparse_attn_swa_workspace_size(ctypes.byref(desc), int(local_window),
                                                           int(local_rows), ctypes.byref(n))
    return st, n.value


def hs2_sparse_attn_swa(desc, q, k, v, k_scale, v_scale, ctx_len, idx, k_local, v_local, kl_scale,
                        vl_scale, local_window, local_rows, out, workspace, workspace_bytes,
                        stream=None) -> int:
    return load_library().hs2_sparse_attn_swa(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(k_scale), _ptr(v_scale), _ptr(ctx_len),
        _ptr(idx), _ptr(k_local), _ptr(v_local), _ptr(kl_scale), _ptr(vl_scale), int(local_window),
        int(local_rows), _ptr(out), _ptr(workspace), int(workspace_bytes), _stream(stream))


def hs2_status_string(status: int) -> str:
    return load_library().hs2_status_string(int(status)).decode()


def hs2_build_id() -> str:
    """Hash of the sources libhs2.so was built from."""
    return load_library().hs2_build_id().decode()
