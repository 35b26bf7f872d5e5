"""libspecverify: the verify step of speculative sampling on AMD MI355X (gfx950).

The work happens in hand-written HIP kernels behind a C ABI
(``include/specverify.h``).  ``binding`` marshals torch tensors to that ABI;
``workloads`` builds the seeded synthetic inputs used by tests and the
benchmark.
"""
from .binding import (  # noqa: F401
    SV_BF16,
    SV_F32,
    SV_GAMMA_BY_BATCH,
    SV_GAMMA_EMA,
    SV_GAMMA_RATE_WINDOW,
    GammaPolicy,
    LibraryMissing,
    SpecVerifyError,
    load_library,
    new_workspace,
    spec_sample,
    spec_sample_filtered_workspace_bytes,
    spec_sample_workspace_bytes,
    spec_verify,
    spec_verify_ex,
    spec_verify_noalloc,
    spec_verify_filtered,
    spec_verify_filtered_workspace_bytes,
    spec_verify_tree,
    spec_verify_tree_workspace_bytes,
    spec_verify_strerror,
    spec_verify_workspace_bytes,
)
