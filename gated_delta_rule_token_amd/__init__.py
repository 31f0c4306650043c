"""gated_delta_rule_token_amd -- a gated delta-rule (Gated DeltaNet) engine for
AMD MI355X (gfx950).

The compute path is the C-ABI library ``libgdr.so`` (hand-written HIP
kernels, declared in ``include/gdr.h``); ``api`` is a thin ctypes binding
that marshals torch tensors into it.  Importing this package loads nothing;
the library is opened on the first call and a missing library is an error,
never a fallback.
"""
from .api import (  # noqa: F401
    GDRError,
    forward,
    gate,
    library_path,
    load_library,
    workspace_size,
)

__all__ = ["GDRError", "forward", "gate", "library_path", "load_library", "workspace_size"]
