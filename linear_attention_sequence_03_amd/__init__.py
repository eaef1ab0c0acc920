"""Gated delta rule forward pass (Gated DeltaNet / KDA / channel-wise write
rates as in FG2-GDN) for MI355X (gfx950).

The compute path is a C-ABI shared library (``libgdr.so``, declared in
``include/gdr.h``) of hand-written HIP kernels; :mod:`.gdr` is a thin ctypes
binding with the same entry-point names.  PyTorch is used only for device
memory and streams.
"""
from .gdr import (  # noqa: F401
    GdrError,
    gdr_chunk_fwd,
    gdr_chunk_fwd_noalloc,
    gdr_chunk_fwd_prologue_workspace_size,
    gdr_chunk_fwd_workspace_size,
    gdr_decode_multi,
    gdr_decode_step,
    gdr_decode_tree,
    gdr_decode_tree_commit,
    gdr_fg2_chunk_fwd,
    gdr_fg2_chunk_fwd_workspace_size,
    gdr_fg2_decode_step,
    gdr_gdn2_chunk_fwd,
    gdr_gdn2_chunk_fwd_workspace_size,
    gdr_gdn2_fwd,
    gdr_status_string,
    load_library,
)
