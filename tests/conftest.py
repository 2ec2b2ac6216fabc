import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


_BUILD_CHECKED = {}


@pytest.fixture(autouse=True)
def _library_matches_sources(request):
    """GPU tests run the in-tree libhs2.so; it must have been built from the sources in
    the tree (its embedded build id equals their hash), else every GPU test fails here
    instead of silently running older kernels."""
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    if "ok" not in _BUILD_CHECKED:
        import long_context_decode_full_amd as hs2
        from long_context_decode_full_amd import build
        built, want = hs2.hs2_build_id(), build.source_hash()
        _BUILD_CHECKED["ok"] = built == want
        _BUILD_CHECKED["msg"] = (f"libhs2.so was built from other sources (build id {built}, "
                                 f"sources {want}): rebuild with __graft_entry__.build()")
    assert _BUILD_CHECKED["ok"], _BUILD_CHECKED["msg"]
    yield
