"""CPU oracle for the HySparse2 Hybrid-Block decode path and the KV Bridging
projection that fills its caches -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import anything from this package; the HIP
library and its Python binding never do, and this package imports nothing
from them.

Every function states the passage of the HySparse2 article (Xiaomi MiMo,
"HySparse2" for MiMo-V3, as reprinted by IT Home and translated by AIHOT.vn
with sections 01-05) that it follows, or the reading adopted where the article
is silent.  Parity status: every function here is pinned by tests in
tests/test_oracle_pins.py (the KV Bridging functions of oracle/bridge.py in
tests/test_oracle_bridge_pins.py) against closed forms, brute force, hand-worked
cases or library routines; none is "parity unpinned".  What is unpinned is whether
the score-to-selection rule is the one the article's model uses: the article
gives no formula for it, so the rule is the specified one (group-summed
softmax probabilities, ties to the lower index).
"""
from .hybrid_block import (  # noqa: F401
    bf16_to_f64,
    e4m3fn_value,
    e4m3fn_table,
    dequant_fp8,
    kv_rows,
    full_attention,
    group_scores,
    select_tokens,
    sparse_attention,
    block_select,
    hybrid_block,
    hybrid_block_token,
)
from .gen1 import (  # noqa: F401
    local_rows,
    local_kv,
    swa_branch,
    gen1_sparse_layer,
)
from .bridge import (  # noqa: F401
    bf16_rne,
    e4m3fn_encode,
    quantize_rows,
    project,
    kv_bridge,
)
