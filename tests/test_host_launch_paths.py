"""Every launch sequence of the C-ABI host layer, run against the host-only build of
hs2_api.cpp with stand-in launchers (tests/host/launch_stubs.cpp) -- never against the
GPU library.  The stand-ins check on the host that every workspace array a kernel would
touch lies inside the workspace the call was given; test_host_sanitizers.py runs this
module (and test_boundary.py) in a process with AddressSanitizer and
UndefinedBehaviorSanitizer on that build.  Fake device addresses are never
dereferenced.  Skipped unless HS2_HOST_LIB names such a build."""
import ctypes
import os

import pytest

import long_context_decode_full_amd as hs2

HOST = os.environ.get("HS2_HOST_LIB")
pytestmark = pytest.mark.skipif(not HOST, reason="needs the host-only sanitizer build (HS2_HOST_LIB)")

WS = 0x7E0000000000          # fake 256-byte aligned workspace base
BUF = 0x100000000            # fake device buffers, 16-byte aligned


@pytest.fixture(scope="module")
def lib():
    lib = hs2.load_library(HOST)
    assert hasattr(lib, "hs2_stub_set_workspace"), "not the host-only build"
    lib.hs2_stub_set_workspace.argtypes = [ctypes.c_void_p, ctypes.c_uint64]
    lib.hs2_stub_set_workspace.restype = None
    lib.hs2_stub_first_error.restype = ctypes.c_char_p
    return lib


def _expect_clean(lib, status, what):
    assert status == hs2.HS2_OK, f"{what}: status {status}"
    assert lib.hs2_stub_launches() > 0, f"{what}: nothing launched"
    assert lib.hs2_stub_errors() == 0, f"{what}: {lib.hs2_stub_first_error().decode()}"


DESCS = {
    "million": dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=1 << 20, max_ctx_len=1 << 20),
    "fp8_256k": dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=1 << 18, max_ctx_len=1 << 18,
                     kv_dtype=hs2.HS2_KV_FP8_E4M3FN),
    "batched": dict(batch=8, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=32768, max_ctx_len=32768),
    "tiny": dict(batch=1, q_len=1, n_q_heads=16, n_kv_heads=2, kv_capacity=4096, max_ctx_len=4096),
    "chunk": dict(batch=16, q_len=64, n_q_heads=32, n_kv_heads=4, kv_capacity=502710, max_ctx_len=502710),
    "chunk_block": dict(batch=16, q_len=64, n_q_heads=32, n_kv_heads=4, kv_capacity=502710,
                        max_ctx_len=502710, select_mode=hs2.HS2_SELECT_BLOCK),
    "decode_block": dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=1 << 20,
                         max_ctx_len=1 << 20, select_mode=hs2.HS2_SELECT_BLOCK),
    "mqa": dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=1, kv_capacity=1 << 20, max_ctx_len=1 << 20),
    "g16_chunk": dict(batch=2, q_len=6, n_q_heads=64, n_kv_heads=4, kv_capacity=9000, max_ctx_len=9000),
    "many_rows": dict(batch=64, q_len=256, n_q_heads=8, n_kv_heads=4, kv_capacity=600, max_ctx_len=600),
    "short": dict(batch=3, q_len=4, n_q_heads=16, n_kv_heads=2, kv_capacity=100, max_ctx_len=70),
    "valu_scan": dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=70000, max_ctx_len=70000,
                      flags=hs2.HS2_FLAG_SCAN_VALU),
    "force_logits": dict(batch=2, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=70000, max_ctx_len=70000,
                         flags=hs2.HS2_FLAG_FORCE_LOGITS),
    "chunk_per_token": dict(batch=2, q_len=64, n_q_heads=32, n_kv_heads=4, kv_capacity=9000, max_ctx_len=9000,
                            flags=hs2.HS2_FLAG_CHUNK_PER_TOKEN),
    "splits": dict(batch=1, q_len=1, n_q_heads=32, n_kv_heads=4, kv_capacity=70000, max_ctx_len=70000,
                   split_len=300, sparse_split_len=40, cand_workgroups=7,
                   flags=hs2.HS2_FLAG_DETERMINISTIC | hs2.HS2_FLAG_SPARSE_FUSED),
    "sparse_split": dict(batch=16, q_len=64, n_q_heads=32, n_kv_heads=4, kv_capacity=20000, max_ctx_len=20000,
                         flags=hs2.HS2_FLAG_SPARSE_SPLIT),
    "sparse_head": dict(batch=4, q_len=64, n_q_heads=32, n_kv_heads=4, kv_capacity=20000, max_ctx_len=20000,
                        flags=hs2.HS2_FLAG_SPARSE_HEAD),
}


@pytest.mark.parametrize("name", list(DESCS))
@pytest.mark.parametrize("probs", [False, True])
def test_full_and_sparse_launch_sequences(lib, name, probs):
    d = hs2.make_desc(**DESCS[name])
    st, need = hs2.hs2_workspace_size(d)
    assert st == hs2.HS2_OK
    fp8 = d.kv_dtype == hs2.HS2_KV_FP8_E4M3FN
    sc = BUF + 0x10000000 if fp8 else None
    lib.hs2_stub_set_workspace(WS, need)
    st = hs2.hs2_full_attn_select(d, BUF, BUF, BUF, sc, sc, BUF, BUF, BUF, BUF if probs else None, WS, need,
                                  stream=0)
    wide = d.n_q_heads // d.n_kv_heads > 8
    if st == hs2.HS2_ERR_UNSUPPORTED:
        # the logits path (probs, decode block mode) keeps 8 head slots and a 16 GiB budget
        assert probs or d.select_mode == hs2.HS2_SELECT_BLOCK
        assert wide or d.q_len > 1
    else:
        _expect_clean(lib, st, f"{name} full layer")
    lib.hs2_stub_set_workspace(WS, need)
    _expect_clean(lib, hs2.hs2_sparse_attn(d, BUF, BUF, BUF, sc, sc, BUF, BUF, BUF, WS, need, stream=0),
                  f"{name} sparse layer")


SCRATCH = 0x7D0000000000     # the stand-ins' scratch address


@pytest.mark.parametrize("name", ["million", "fp8_256k", "batched", "tiny", "mqa", "decode_block", "short",
                                  "force_logits", "splits"])
@pytest.mark.parametrize("probs", [False, True])
def test_noalloc_launch_sequence_fits_the_scratch(lib, name, probs):
    """hs2_full_attn_select_noalloc: every array its kernels index lies inside the
    library's fixed scratch, or the call is refused with HS2_ERR_SCRATCH_LIMIT."""
    d = hs2.make_desc(**DESCS[name])
    fp8 = d.kv_dtype == hs2.HS2_KV_FP8_E4M3FN
    sc = BUF + 0x10000000 if fp8 else None
    lib.hs2_stub_set_workspace(SCRATCH, hs2.HS2_NOALLOC_SCRATCH_BYTES)
    st = hs2.hs2_full_attn_select_noalloc(d, BUF, BUF, BUF, sc, sc, BUF, BUF, BUF, BUF if probs else None,
                                          stream=0)
    if st == hs2.HS2_ERR_SCRATCH_LIMIT:
        assert probs or d.select_mode == hs2.HS2_SELECT_BLOCK or d.flags & hs2.HS2_FLAG_FORCE_LOGITS, name
        assert lib.hs2_stub_launches() == 0
    elif st == hs2.HS2_ERR_UNSUPPORTED:
        assert probs and d.n_q_heads // d.n_kv_heads > 8
    else:
        _expect_clean(lib, st, f"{name} no-allocation full layer")
    if name == "million" and not probs:
        assert st == hs2.HS2_OK   # the benchmark's decode fits


def test_decode_step_launch_sequence(lib):
    attn = hs2.make_desc(2, 1, 32, 4, 40000, 39000)
    plan = hs2.make_decode_plan(attn, 3, 3, 2048)
    st, need = hs2.hs2_decode_workspace_size(plan)
    assert st == hs2.HS2_OK
    lib.hs2_stub_set_workspace(WS, need)
    ptrs = lambda n, base: [base + 0x1000000 * i for i in range(n)]
    st = hs2.hs2_decode_step(plan, BUF, BUF, ptrs(3, BUF), ptrs(9, BUF), ptrs(3, BUF), ptrs(3, BUF), None, None,
                             BUF, ptrs(3, BUF), ptrs(3, BUF), ptrs(9, BUF), WS, need, stream=0)
    _expect_clean(lib, st, "decode step")
    assert lib.hs2_stub_launches() == 2 + 3 * (1 + 1 + 2 + 3 * 1)   # advance, bridge, blocks


def test_bridge_and_first_generation_launch_sequences(lib):
    for T in (1, 16, 17, 5000):
        d = hs2.make_bridge_desc(T, 512, 2, 2, 4, 8192)
        lib.hs2_stub_set_workspace(WS, 0)
        st = hs2.hs2_kv_bridge(d, BUF, BUF, BUF, BUF, [BUF, BUF], [BUF, BUF], [BUF, BUF], [BUF, BUF], stream=0)
        _expect_clean(lib, st, f"bridge T={T}")
    d = hs2.make_desc(2, 16, 32, 4, 9000, 9000, select_mode=hs2.HS2_SELECT_BLOCK)
    st, need = hs2.hs2_sparse_attn_swa_workspace_size(d, 128, 143)
    assert st == hs2.HS2_OK
    lib.hs2_stub_set_workspace(WS, need)
    st = hs2.hs2_sparse_attn_swa(d, BUF, BUF, BUF, None, None, BUF, BUF, BUF, BUF, None, None, 128, 143, BUF,
                                 WS, need, stream=0)
    _expect_clean(lib, st, "first-generation sparse layer")
    # decode sizes: both branches in one launch (the window rows formed in the kernel)
    for fp8 in (False, True):
        d = hs2.make_desc(2, 1, 32, 4, 9000, 9000, select_mode=hs2.HS2_SELECT_BLOCK,
                          kv_dtype=hs2.HS2_KV_FP8_E4M3FN if fp8 else hs2.HS2_KV_BF16)
        st, need = hs2.hs2_sparse_attn_swa_workspace_size(d, 128, 128)
        assert st == hs2.HS2_OK
        lib.hs2_stub_set_workspace(WS, need)
        sc = BUF if fp8 else None
        st = hs2.hs2_sparse_attn_swa(d, BUF, BUF, BUF, sc, sc, BUF, BUF, BUF, BUF, sc, sc, 128, 128, BUF,
                                     WS, need, stream=0)
        _expect_clean(lib, st, f"first-generation sparse layer at decode (fp8={fp8})")
        assert lib.hs2_stub_launches() == 1


def test_stub_catches_a_short_workspace(lib):
    """The extent checks themselves: a workspace announced one byte short is reported."""
    d = hs2.make_desc(**DESCS["tiny"])
    st, need = hs2.hs2_workspace_size(d)
    lib.hs2_stub_set_workspace(WS, need - 256)
    assert hs2.hs2_full_attn_select(d, BUF, BUF, BUF, None, None, BUF, BUF, BUF, None, WS, need, stream=0) == 0
    assert lib.hs2_stub_errors() > 0
