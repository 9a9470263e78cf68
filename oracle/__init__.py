"""Float64 CPU oracle of the ARL2 hybrid attention layer.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg; never by the library.
"""
from .arl2_oracle import (  # noqa: F401
    L2_EPS,
    delta_update,
    feature_map,
    frame_forward,
    gate_projections,
    gate_state,
    head_forward,
    inter_read,
    intra_attention,
    kv_cache_attention,
    l2_normalize_rows,
    output_rows,
    row_softmax,
    sigmoid,
    token_level_frame_forward,
    token_level_head_forward,
    token_level_update,
)
