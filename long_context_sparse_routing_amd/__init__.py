"""MI355X-native shared-routing sparse decode attention (CLSA).

The compute path is libclsa.so (hand-written HIP for gfx950) behind a C ABI
(include/clsa.h); `binding` marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    ClsaError,
    csa_build,
    csa_route,
    LouverIndex,
    Prepared,
    kv_append,
    load_library,
    prepare_csa_route,
    prepare_kv_append,
    prepare_route,
    prepare_route_aggregated,
    prepare_route_static,
    prepare_route_threshold,
    prepare_sparse_attn,
    route,
    route_aggregated,
    route_static,
    route_threshold,
    route_threshold_workspace_size,
    route_workspace_size,
    sparse_attn,
    sparse_attn_workspace_size,
)
