"""MoE token dispatch and combine on one MI355X (gfx950).

``ops`` holds the thin binding of the C ABI in ``include/epdc.h``
(``ep_compute_send_counts``, ``ep_build_send_layout``,
``ep_dispatch_permute``, ``ep_batched_prepare``, ``ep_combine``);
``dispatch`` holds the dispatcher-level functions (``dispatch``,
``combine``, ``dispatch_chunked_forward``, ``batched_prepare`` ...).
Importing the package does not load the library; the first call does, and
fails loudly if ``libepdc.so`` has not been built.
"""

from ._lib import LIB_PATH, header_functions, lib  # noqa: F401
from .dispatch import (  # noqa: F401
    ChunkedDispatcher,
    DispatchHandle,
    batched_finalize,
    batched_prepare,
    build_send_layout,
    chunk_bounds,
    combine,
    compute_send_counts,
    dispatch,
    dispatch_chunked_forward,
    permute_by_expert,
    restore_by_expert,
    to_host,
)
from .ops import (  # noqa: F401
    Counts,
    Regrouped,
    SendLayout,
    ep_batched_prepare,
    ep_batched_prepare_fp8,
    batched_scale_like,
    ep_batched_workspace_bytes,
    ep_build_send_layout,
    ep_combine,
    ep_compute_send_counts,
    ep_dispatch_layout,
    ep_dispatch_layout_workspace_bytes,
    ep_dispatch_layout_noalloc,
    ep_dispatch_layout_chunked,
    ep_dispatch_layout_chunked_workspace_bytes,
    library_scratch_status,
    ep_counts_workspace_bytes,
    ep_dispatch_permute,
    ep_layout_workspace_bytes,
    ep_regroup_by_expert,
    ep_regroup_workspace_bytes,
    workspace_for,
    ep_workspace_status,
    check_workspaces,
    workspace_flags,
    WaitGaveUpError,
)
