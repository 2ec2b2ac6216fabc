"""CPU-only checks of the C ABI: the library loads, exports what include/hs2.h declares,
and every argument check returns its status before anything is enqueued.

No call here reaches a kernel launch: each one fails validation first, so these
run without a GPU.  Fake device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import long_context_decode_full_amd as hs2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs2.h")


@pytest.fixture(scope="module")
def lib():
    host = os.environ.get("HS2_HOST_LIB")   # the sanitizer run loads a host-only build
    if host:
        return hs2.load_library(host)
    if not os.path.exists(hs2.library_path()):
        import __graft_entry__
        __graft_entry__.build()
    return hs2.load_library()


def _desc(**kw):
    base = dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=1 << 20,
                max_ctx_len=1 << 20)
    base.update(kw)
    return hs2.make_desc(**base)


def test_header_symbols_are_exported(lib):
    text = open(HEADER).read()
    declared = sorted(set(re.findall(r"\b(hs2_[a-z_]+)\s*\(", text)))
    assert declared, "no declarations found"
    assert sorted(hs2.EXPORTED_SYMBOLS) == declared
    for name in declared:
        assert hasattr(lib, name), f"{name} not exported"
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_status_strings(lib):
    for st in range(7):
        assert hs2.hs2_status_string(st)
    assert hs2.hs2_status_string(0) == "ok"
    assert hs2.hs2_status_string(99) == "unknown status"


def test_desc_struct_layout_matches_header():
    # int32 x6, int64 x2, int32 x5, float, then the options: uint32 flags, int32 x3
    # -> 24 + 16 + 20 + 4 + 16 = 80 bytes
    assert ctypes.sizeof(hs2.Hs2AttnDesc) == 80
    assert hs2.Hs2AttnDesc.kv_capacity.offset == 24
    assert hs2.Hs2AttnDesc.sm_scale.offset == 60
    assert hs2.Hs2AttnDesc.flags.offset == 64
    assert hs2.Hs2AttnDesc.cand_workgroups.offset == 76


def test_build_id_names_the_current_sources(lib):
    """The library embeds a hash of the sources it was built from; a stale libhs2.so
    (sources edited after the build) shows here instead of running old kernels."""
    from long_context_decode_full_amd import build
    if os.environ.get("HS2_HOST_LIB"):
        assert hs2.hs2_build_id() == "host-sanitizer-build"
        return
    assert hs2.hs2_build_id() == build.source_hash()


@pytest.mark.parametrize("kw,status", [
    (dict(), hs2.HS2_OK),
    (dict(batch=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(q_len=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(n_q_heads=30), hs2.HS2_ERR_INVALID_ARG),          # Hq % Hkv != 0
    (dict(n_q_heads=64, n_kv_heads=4), hs2.HS2_OK),              # G = 16: wide groups
    (dict(n_q_heads=32, n_kv_heads=1), hs2.HS2_OK),              # MQA, G = 32
    (dict(n_q_heads=64, n_kv_heads=1), hs2.HS2_ERR_UNSUPPORTED), # G = 64 > 32
    (dict(n_q_heads=32, n_kv_heads=1, select_mode=1), hs2.HS2_OK),  # G > 8 block mode: the scans' block sums
    (dict(head_dim=64), hs2.HS2_ERR_UNSUPPORTED),
    (dict(kv_dtype=7), hs2.HS2_ERR_INVALID_ARG),
    (dict(max_ctx_len=(1 << 20) + 1), hs2.HS2_ERR_INVALID_ARG),   # beyond capacity
    (dict(q_len=64, max_ctx_len=32), hs2.HS2_ERR_INVALID_ARG),    # chunk longer than context
    (dict(window=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(window=0, topk=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(window=128, topk=4000), hs2.HS2_ERR_UNSUPPORTED),
    (dict(select_mode=5), hs2.HS2_ERR_INVALID_ARG),
    (dict(select_mode=1, block_size=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(select_mode=1, block_size=64, n_blocks=100), hs2.HS2_ERR_UNSUPPORTED),
    (dict(select_mode=1, block_size=16, n_blocks=18), hs2.HS2_ERR_UNSUPPORTED),  # > 16384 blocks
    (dict(select_mode=1), hs2.HS2_OK),
    (dict(sm_scale=0.0), hs2.HS2_ERR_INVALID_ARG),
    (dict(sm_scale=float("nan")), hs2.HS2_ERR_INVALID_ARG),
    (dict(kv_capacity=1 << 31, max_ctx_len=1 << 20), hs2.HS2_ERR_UNSUPPORTED),
    (dict(batch=1100, q_len=64, kv_capacity=4096, max_ctx_len=4096), hs2.HS2_ERR_UNSUPPORTED),
    # options
    (dict(flags=hs2.HS2_FLAGS_ALL & ~(hs2.HS2_FLAG_SPARSE_FUSED | hs2.HS2_FLAG_SPARSE_HEAD)), hs2.HS2_OK),
    (dict(flags=0x100), hs2.HS2_ERR_INVALID_ARG),                 # unknown flag bit
    (dict(flags=1 << 31), hs2.HS2_ERR_INVALID_ARG),
    (dict(flags=hs2.HS2_FLAG_SPARSE_FUSED | hs2.HS2_FLAG_SPARSE_SPLIT), hs2.HS2_ERR_INVALID_ARG),
    (dict(flags=hs2.HS2_FLAG_SPARSE_HEAD | hs2.HS2_FLAG_SPARSE_SPLIT), hs2.HS2_ERR_INVALID_ARG),
    (dict(flags=hs2.HS2_FLAG_SPARSE_HEAD | hs2.HS2_FLAG_SPARSE_FUSED), hs2.HS2_ERR_INVALID_ARG),
    (dict(flags=hs2.HS2_FLAG_SPARSE_HEAD), hs2.HS2_OK),
    (dict(split_len=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(sparse_split_len=-32), hs2.HS2_ERR_INVALID_ARG),
    (dict(cand_workgroups=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(split_len=1, sparse_split_len=1, cand_workgroups=1), hs2.HS2_OK),   # clamped upwards
])
def test_validate(lib, kw, status):
    assert hs2.hs2_validate(_desc(**kw)) == status


def test_validate_checks_the_workspace_size(lib):
    """hs2_validate(desc, bytes) is the descriptor check plus the workspace check that
    every call makes."""
    for kw in (dict(), dict(q_len=64, max_ctx_len=300000, kv_capacity=300000),
               dict(select_mode=hs2.HS2_SELECT_BLOCK, max_ctx_len=5000, kv_capacity=5000)):
        d = _desc(**kw)
        st, need = hs2.hs2_workspace_size(d)
        assert st == hs2.HS2_OK
        assert hs2.hs2_validate(d, need) == hs2.HS2_OK
        assert hs2.hs2_validate(d, need - 1) == hs2.HS2_ERR_WORKSPACE
        assert _full(d, workspace_bytes=need - 1) == hs2.HS2_ERR_WORKSPACE
    assert hs2.hs2_validate(_desc(head_dim=64), 0) == hs2.HS2_ERR_UNSUPPORTED   # descriptor first


def test_validate_null_desc(lib):
    assert lib.hs2_validate(None, 0) == hs2.HS2_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert lib.hs2_workspace_size(None, ctypes.byref(n)) == hs2.HS2_ERR_INVALID_ARG
    assert lib.hs2_workspace_size(ctypes.byref(_desc()), None) == hs2.HS2_ERR_INVALID_ARG


def test_workspace_monotone_in_context(lib):
    prev = 0
    for ctx in [1, 100, 4096, 65536, 1 << 20]:
        st, nbytes = hs2.hs2_workspace_size(_desc(kv_capacity=1 << 20, max_ctx_len=ctx))
        assert st == hs2.HS2_OK
        assert nbytes >= prev
        prev = nbytes
    # logits (32 B per position per KV head) dominate at long context
    st, nbytes = hs2.hs2_workspace_size(_desc())
    assert nbytes >= 4 * (1 << 20) * 8 * 4


def test_selection_row_limit(lib):
    """batch * q_len * n_kv_heads beyond 65535 * 1024 rows is reported, not launched."""
    assert hs2.hs2_validate(_desc(batch=1000, q_len=64, n_q_heads=2048, n_kv_heads=2048,
                                  max_ctx_len=64, kv_capacity=64)) == hs2.HS2_ERR_UNSUPPORTED
    assert hs2.hs2_validate(_desc(batch=1000, q_len=64, n_q_heads=512, n_kv_heads=512,
                                  max_ctx_len=64, kv_capacity=64)) == hs2.HS2_OK


@pytest.mark.parametrize("field", ["split_len", "sparse_split_len", "cand_workgroups"])
def test_size_options_follow_the_descriptor(lib, field, monkeypatch):
    """Split sizes come from the descriptor only: 0 means automatic, tiny values are
    clamped to the kernels' minimum, and the environment is never read (a variable set
    between hs2_workspace_size and a call cannot change the layout)."""
    base = _desc(kv_capacity=1 << 16, max_ctx_len=50000)
    st0, n0 = hs2.hs2_workspace_size(base)
    for v in (0, 1, 7, 256, 4096):
        st, nbytes = hs2.hs2_workspace_size(_desc(kv_capacity=1 << 16, max_ctx_len=50000, **{field: v}))
        assert st == hs2.HS2_OK and nbytes > 0
        if v == 0:
            assert nbytes == n0
    for var in ("HS2_SPLIT_LEN", "HS2_SPARSE_SPLIT_LEN", "HS2_CAND_WGS_TOTAL", "HS2_SCAN_VALU",
                "HS2_FORCE_LOGITS", "HS2_CHUNK_PER_TOKEN", "HS2_SPARSE_FUSED"):
        monkeypatch.setenv(var, "1")
    assert hs2.hs2_workspace_size(base) == (st0, n0)


def test_library_reads_no_environment():
    """No getenv in the host layer: every option travels in the descriptor."""
    src = open(os.path.join(ROOT, "long_context_decode_full_amd", "csrc", "hs2_api.cpp")).read()
    assert "getenv" not in src


FAKE = 0x7F0000000000   # 16-byte aligned fake device address, never dereferenced


def _full(d, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, k_scale=None, v_scale=None, ctx_len=FAKE, out=FAKE,
                idx=FAKE, probs=None, workspace=FAKE, workspace_bytes=1 << 40)
    args.update(over)
    return hs2.hs2_full_attn_select(d, stream=0, **args)


def _sparse(d, **over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, k_scale=None, v_scale=None, ctx_len=FAKE, idx=FAKE,
                out=FAKE, workspace=FAKE, workspace_bytes=1 << 40)
    args.update(over)
    return hs2.hs2_sparse_attn(d, stream=0, **args)


@pytest.mark.parametrize("field", ["q", "k", "v", "ctx_len", "out", "idx", "workspace"])
def test_null_pointers_rejected(lib, field):
    assert _full(_desc(), **{field: None}) == hs2.HS2_ERR_INVALID_ARG
    assert _sparse(_desc(), **{field: None}) == hs2.HS2_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["q", "k", "v", "out", "idx", "workspace"])
def test_misaligned_pointers_rejected(lib, field):
    assert _full(_desc(), **{field: FAKE + 4}) == hs2.HS2_ERR_ALIGNMENT
    assert _sparse(_desc(), **{field: FAKE + 8}) == hs2.HS2_ERR_ALIGNMENT
    assert _full(_desc(), probs=FAKE + 2) == hs2.HS2_ERR_ALIGNMENT


def test_fp8_needs_scales(lib):
    d = _desc(kv_dtype=hs2.HS2_KV_FP8_E4M3FN)
    assert _full(d) == hs2.HS2_ERR_INVALID_ARG
    assert _full(d, k_scale=FAKE) == hs2.HS2_ERR_INVALID_ARG
    assert _sparse(d, v_scale=FAKE) == hs2.HS2_ERR_INVALID_ARG
    assert _full(d, k_scale=FAKE + 2, v_scale=FAKE) == hs2.HS2_ERR_ALIGNMENT


def test_workspace_too_small(lib):
    d = _desc()
    st, nbytes = hs2.hs2_workspace_size(d)
    assert st == 0
    assert _full(d, workspace_bytes=nbytes - 1) == hs2.HS2_ERR_WORKSPACE
    assert _sparse(d, workspace_bytes=16) == hs2.HS2_ERR_WORKSPACE


def test_noalloc_checks_before_touching_a_device(lib):
    """The no-allocation entry point checks its arguments like hs2_full_attn_select and
    refuses calls beyond its fixed scratch before any HIP call (no GPU needed here)."""
    def noalloc(d, **over):
        args = dict(q=FAKE, k=FAKE, v=FAKE, k_scale=None, v_scale=None, ctx_len=FAKE, out=FAKE, idx=FAKE,
                    probs=None)
        args.update(over)
        return hs2.hs2_full_attn_select_noalloc(d, stream=0, **args)
    assert noalloc(_desc(head_dim=64)) == hs2.HS2_ERR_UNSUPPORTED
    assert noalloc(_desc(), q=None) == hs2.HS2_ERR_INVALID_ARG
    assert noalloc(_desc(), out=FAKE + 4) == hs2.HS2_ERR_ALIGNMENT
    assert noalloc(_desc(), probs=FAKE + 2) == hs2.HS2_ERR_ALIGNMENT
    assert noalloc(_desc(kv_dtype=hs2.HS2_KV_FP8_E4M3FN)) == hs2.HS2_ERR_INVALID_ARG
    # the 64-token chunk at 500K positions, or every logit of a million positions
    assert noalloc(_desc(batch=16, q_len=64, kv_capacity=502710, max_ctx_len=502710)) == \
        hs2.HS2_ERR_SCRATCH_LIMIT
    assert noalloc(_desc(), probs=FAKE) == hs2.HS2_ERR_SCRATCH_LIMIT
    assert "scratch" in hs2.hs2_status_string(hs2.HS2_ERR_SCRATCH_LIMIT)


def test_invalid_desc_checked_before_pointers(lib):
    assert _full(_desc(head_dim=96), q=None) == hs2.HS2_ERR_UNSUPPORTED


def test_wide_groups_have_no_logits_path(lib):
    """More than 8 query heads per KV head: token mode on the record path, block mode on
    the scans' block sums (probs from a re-score pass), and every call that only the
    logits path (8 head slots) could serve is refused before anything is enqueued (fake
    device pointers, never touched)."""
    mqa = dict(n_q_heads=32, n_kv_heads=1, kv_capacity=65536, max_ctx_len=65536)
    assert _full(_desc(select_mode=1, flags=hs2.HS2_FLAG_FORCE_LOGITS, **mqa)) == hs2.HS2_ERR_UNSUPPORTED
    assert _full(_desc(select_mode=1, flags=hs2.HS2_FLAG_SCAN_VALU, **mqa)) == hs2.HS2_ERR_UNSUPPORTED
    assert _full(_desc(select_mode=1, block_size=48, n_blocks=18, **mqa)) == hs2.HS2_ERR_UNSUPPORTED
    # a chunk: 96-position blocks take the per-token scan's block sums (a multiple of
    # 32), 48-position blocks would need the logits path
    g16 = dict(n_q_heads=64, n_kv_heads=4, q_len=64, kv_capacity=65536, max_ctx_len=65536)
    assert _full(_desc(select_mode=1, block_size=48, n_blocks=18, **g16)) == hs2.HS2_ERR_UNSUPPORTED


def test_timed_calls_check_like_the_plain_ones(lib):
    """The _timed variants take caller-owned events; argument checks come first and
    return before any event is recorded (fake handles here are never touched)."""
    ev = (0x1234, 0x5678)
    d = _desc()
    assert hs2.hs2_full_attn_select_timed(d, *([FAKE] * 3), None, None, FAKE, FAKE, FAKE, None, FAKE, 16,
                                          stream=0, events=ev) == hs2.HS2_ERR_WORKSPACE
    assert hs2.hs2_sparse_attn_timed(d, FAKE, FAKE, FAKE, None, None, FAKE, FAKE, FAKE, None, 1 << 40,
                                     stream=0, events=ev) == hs2.HS2_ERR_INVALID_ARG
    assert hs2.hs2_full_attn_select_timed(_desc(head_dim=64), *([FAKE] * 3), None, None, FAKE, FAKE,
                                          FAKE, None, FAKE, 1 << 40, stream=0, events=ev) == hs2.HS2_ERR_UNSUPPORTED


def test_product_path_has_no_fallback():
    """The binding and runner must not reach the CPU oracle."""
    pkg = os.path.dirname(hs2.__file__)
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), name
            assert "hybrid_block(" not in src, name


# ----------------------------------------------------------------------------- KV Bridging
def test_bridge_desc_struct_layout_matches_header():
    # int32 x7, then int64 aligned to 8 -> 28 + 4 pad + 8 = 40 bytes, then two int32
    assert ctypes.sizeof(hs2.Hs2BridgeDesc) == 48
    assert hs2.Hs2BridgeDesc.kv_capacity.offset == 32
    assert hs2.Hs2BridgeDesc.gemv_max_tokens.offset == 40


_GOOD = 0x10000000          # fake 4 KiB-aligned device addresses, never dereferenced


def _bridge(lib_unused=None, desc=None, fp8=True, n_layers=2, **over):
    d = desc if desc is not None else hs2.make_bridge_desc(
        300, 512, n_layers, 2, 4, 4096, kv_dtype=hs2.HS2_KV_FP8_E4M3FN if fp8 else hs2.HS2_KV_BF16)
    args = dict(x=_GOOD, w=_GOOD + 0x1000000, seq=_GOOD + 0x2000000, pos=_GOOD + 0x3000000,
                k_caches=[_GOOD + 0x4000000 * (i + 1) for i in range(d.n_layers)],
                v_caches=[_GOOD + 0x4000000 * (i + 1) + 0x2000000 for i in range(d.n_layers)],
                k_scales=[_GOOD + 0x100000 * (i + 1) for i in range(d.n_layers)] if fp8 else None,
                v_scales=[_GOOD + 0x100000 * (i + 1) + 0x80000 for i in range(d.n_layers)] if fp8 else None)
    args.update(over)
    return hs2.hs2_kv_bridge(d, **args, stream=0)


@pytest.mark.parametrize("field,value,status", [
    ("n_tokens", -1, hs2.HS2_ERR_INVALID_ARG),
    ("hidden", 0, hs2.HS2_ERR_INVALID_ARG),
    ("hidden", 100, hs2.HS2_ERR_UNSUPPORTED),
    ("hidden", 65536 + 64, hs2.HS2_ERR_UNSUPPORTED),
    ("head_dim", 64, hs2.HS2_ERR_UNSUPPORTED),
    ("n_layers", 0, hs2.HS2_ERR_INVALID_ARG),
    ("n_layers", 17, hs2.HS2_ERR_UNSUPPORTED),
    ("n_kv_heads", 0, hs2.HS2_ERR_INVALID_ARG),
    ("kv_dtype", 7, hs2.HS2_ERR_INVALID_ARG),
    ("batch", 0, hs2.HS2_ERR_INVALID_ARG),
    ("kv_capacity", 0, hs2.HS2_ERR_INVALID_ARG),
    ("kv_capacity", 1 << 31, hs2.HS2_ERR_UNSUPPORTED),
    ("gemv_max_tokens", -2, hs2.HS2_ERR_INVALID_ARG),
    ("gemv_max_tokens", 1025, hs2.HS2_ERR_INVALID_ARG),
    ("reserved", 1, hs2.HS2_ERR_INVALID_ARG),
])
def test_bridge_desc_checks(lib, field, value, status):
    d = hs2.make_bridge_desc(300, 512, 2, 2, 4, 4096)
    setattr(d, field, value)
    over = {}
    if field == "n_layers" and value > 0:
        over = dict(k_caches=[_GOOD] * value, v_caches=[_GOOD] * value, k_scales=[_GOOD] * value,
                    v_scales=[_GOOD] * value)
    assert _bridge(desc=d, **over) == status


def test_bridge_null_desc(lib):
    assert lib.hs2_kv_bridge(None, None, None, None, None, None, None, None, None, None) == \
        hs2.HS2_ERR_INVALID_ARG


@pytest.mark.parametrize("field", ["x", "w", "seq", "pos", "k_caches", "v_caches", "k_scales", "v_scales"])
def test_bridge_null_pointers_rejected(lib, field):
    assert _bridge(**{field: None}) == hs2.HS2_ERR_INVALID_ARG


def test_bridge_null_layer_pointer_rejected(lib):
    assert _bridge(v_caches=[_GOOD, 0]) == hs2.HS2_ERR_INVALID_ARG
    assert _bridge(k_scales=[_GOOD, 0]) == hs2.HS2_ERR_INVALID_ARG


@pytest.mark.parametrize("field,addr", [("x", _GOOD + 8), ("w", _GOOD + 2), ("seq", _GOOD + 2),
                                        ("pos", _GOOD + 1)])
def test_bridge_misaligned_pointers_rejected(lib, field, addr):
    assert _bridge(**{field: addr}) == hs2.HS2_ERR_ALIGNMENT


def test_bridge_misaligned_layer_pointers_rejected(lib):
    assert _bridge(k_caches=[_GOOD, _GOOD + 8]) == hs2.HS2_ERR_ALIGNMENT
    assert _bridge(v_scales=[_GOOD, _GOOD + 2]) == hs2.HS2_ERR_ALIGNMENT


def test_bridge_bf16_needs_no_scales_and_zero_tokens_enqueue_nothing(lib):
    # a bf16 call with no scale arrays passes every check; with zero tokens it returns
    # before any launch (no GPU is touched)
    d = hs2.make_bridge_desc(0, 512, 2, 2, 4, 4096, kv_dtype=hs2.HS2_KV_BF16)
    assert _bridge(desc=d, fp8=False) == hs2.HS2_OK
    d8 = hs2.make_bridge_desc(0, 512, 2, 2, 4, 4096)
    assert _bridge(desc=d8, fp8=True, k_scales=None) == hs2.HS2_ERR_INVALID_ARG


# ----------------------------------------------------------------------------- decode step
def test_decode_plan_struct_layout_matches_header():
    # hs2_attn_desc (80 bytes) then four int32
    assert ctypes.sizeof(hs2.Hs2DecodePlan) == 96
    assert hs2.Hs2DecodePlan.n_blocks.offset == 80
    assert hs2.Hs2DecodePlan.hidden.offset == 88


def _plan(**kw):
    attn = _desc(kv_capacity=8192, max_ctx_len=8192)
    p = dict(n_blocks=2, n_sparse=3, hidden=512)
    p.update(kw)
    return hs2.make_decode_plan(attn, p["n_blocks"], p["n_sparse"], p["hidden"])


def _step(plan, **over):
    nb, ns = plan.n_blocks, plan.n_sparse
    st, need = hs2.hs2_decode_workspace_size(plan)
    need = need if st == hs2.HS2_OK else 1 << 20
    args = dict(x=_GOOD, w=_GOOD + 0x1000000, q_full=[_GOOD + 0x10000 * (i + 1) for i in range(nb)],
                q_sparse=[_GOOD + 0x20000 * (i + 1) for i in range(nb * ns)],
                k_caches=[_GOOD + 0x4000000 * (i + 1) for i in range(nb)],
                v_caches=[_GOOD + 0x4000000 * (i + 1) + 0x2000000 for i in range(nb)],
                k_scales=None, v_scales=None, ctx_len=_GOOD + 0x3000000,
                out_full=[_GOOD + 0x40000 * (i + 1) for i in range(nb)],
                idx=[_GOOD + 0x80000 * (i + 1) for i in range(nb)],
                out_sparse=[_GOOD + 0x100000 * (i + 1) for i in range(nb * ns)],
                workspace=_GOOD + 0x8000000, workspace_bytes=need)
    args.update(over)
    return hs2.hs2_decode_step(plan, stream=0, **args)


def test_decode_workspace_size_covers_attention(lib):
    st, n = hs2.hs2_decode_workspace_size(_plan())
    st2, n_attn = hs2.hs2_workspace_size(_desc(kv_capacity=8192, max_ctx_len=8192))
    assert st == st2 == hs2.HS2_OK and n >= n_attn + 2 * 4


@pytest.mark.parametrize("kw,status", [
    (dict(n_blocks=0), hs2.HS2_ERR_INVALID_ARG),
    (dict(n_blocks=17), hs2.HS2_ERR_UNSUPPORTED),
    (dict(n_sparse=-1), hs2.HS2_ERR_INVALID_ARG),
    (dict(n_sparse=9), hs2.HS2_ERR_UNSUPPORTED),
    (dict(hidden=0), hs2.HS2_ERR_INVALID_ARG),
])
def test_decode_plan_checks(lib, kw, status):
    p = _plan(**kw)
    assert hs2.hs2_decode_workspace_size(p)[0] == status
    assert _step(p) == status


def test_decode_step_needs_single_query_token(lib):
    p = _plan()
    p.attn.q_len = 2
    assert _step(p) == hs2.HS2_ERR_INVALID_ARG


def test_decode_step_argument_checks_before_any_launch(lib):
    p = _plan()
    assert _step(p, workspace_bytes=100) == hs2.HS2_ERR_WORKSPACE
    assert _step(p, ctx_len=None) == hs2.HS2_ERR_INVALID_ARG
    assert _step(p, q_sparse=None) == hs2.HS2_ERR_INVALID_ARG
    assert _step(p, idx=[_GOOD, 0]) == hs2.HS2_ERR_INVALID_ARG
    assert _step(p, out_sparse=[_GOOD] * 5 + [0]) == hs2.HS2_ERR_INVALID_ARG
    assert _step(p, x=_GOOD + 8) == hs2.HS2_ERR_ALIGNMENT           # bridge source row
    assert _step(_plan(hidden=100)) == hs2.HS2_ERR_UNSUPPORTED                # bridge hidden size
    assert _step(p, k_caches=[_GOOD, _GOOD + 8]) == hs2.HS2_ERR_ALIGNMENT
    p8 = _plan()
    p8.attn.kv_dtype = hs2.HS2_KV_FP8_E4M3FN
    assert _step(p8) == hs2.HS2_ERR_INVALID_ARG                      # fp8 without scales


# ----------------------------------------------------------------------------- first-generation comparator
def _swa(d, **over):
    st, need = hs2.hs2_sparse_attn_swa_workspace_size(d, over.pop("W", 128), over.get("R", 140))
    args = dict(q=_GOOD, k=_GOOD + 0x1000000, v=_GOOD + 0x2000000, k_scale=None, v_scale=None,
                ctx_len=_GOOD + 0x3000000, idx=_GOOD + 0x4000000, k_local=_GOOD + 0x5000000,
                v_local=_GOOD + 0x6000000, kl_scale=None, vl_scale=None, local_window=128,
                local_rows=140, out=_GOOD + 0x7000000, workspace=_GOOD + 0x8000000,
                workspace_bytes=need if st == hs2.HS2_OK else 1 << 20)
    args.update(over)
    args.pop("R", None)
    return hs2.hs2_sparse_attn_swa(d, stream=0, **args)


def test_swa_workspace_and_ring_limits(lib):
    d = _desc(q_len=16, kv_capacity=8192, max_ctx_len=8192, select_mode=hs2.HS2_SELECT_BLOCK)
    assert hs2.hs2_sparse_attn_swa_workspace_size(d, 128, 143)[0] == hs2.HS2_OK
    assert hs2.hs2_sparse_attn_swa_workspace_size(d, 128, 142)[0] == hs2.HS2_ERR_UNSUPPORTED  # < W + Lq - 1
    assert hs2.hs2_sparse_attn_swa_workspace_size(d, 0, 143)[0] == hs2.HS2_ERR_INVALID_ARG
    assert hs2.hs2_sparse_attn_swa_workspace_size(d, 4097, 5000)[0] == hs2.HS2_ERR_UNSUPPORTED


def test_swa_argument_checks_before_any_launch(lib):
    d = _desc(kv_capacity=8192, max_ctx_len=8192, select_mode=hs2.HS2_SELECT_BLOCK)
    assert _swa(d, k_local=None) == hs2.HS2_ERR_INVALID_ARG
    assert _swa(d, v_local=_GOOD + 8) == hs2.HS2_ERR_ALIGNMENT
    assert _swa(d, idx=None) == hs2.HS2_ERR_INVALID_ARG
    assert _swa(d, workspace_bytes=64) == hs2.HS2_ERR_WORKSPACE
    assert _swa(d, local_rows=100) == hs2.HS2_ERR_UNSUPPORTED
    d8 = _desc(kv_capacity=8192, max_ctx_len=8192, kv_dtype=hs2.HS2_KV_FP8_E4M3FN,
               select_mode=hs2.HS2_SELECT_BLOCK)
    assert _swa(d8, k_scale=_GOOD, v_scale=_GOOD) == hs2.HS2_ERR_INVALID_ARG   # local scales missing
