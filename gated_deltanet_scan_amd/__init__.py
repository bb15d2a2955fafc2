"""Frame-wise Gated DeltaNet scan (forward and backward) for AMD MI355X (gfx950).

The compute path is libgdn.so (HIP kernels behind the C ABI in include/gdn.h);
``api`` marshals torch tensors across it.  ``inputs`` draws seeded synthetic
workloads and is importable without a GPU.
"""
from . import inputs  # noqa: F401

__all__ = ["frame_scan", "frame_scan_fwd", "frame_scan_fwd_static", "frame_scan_fwd_fp8", "frame_scan_fwd_fp4", "frame_scan_bwd", "frame_scan_fwd_save", "frame_step", "block_in_proj", "block_out_proj", "profile_begin", "profile_end", "workspace_size",
           "make_desc", "GdnError", "inputs"]


def __getattr__(name):
    # The HIP binding loads on first use so that CPU-only tools (the input
    # recipe, the oracle tests) can import the package without a GPU.
    if name in ("frame_scan_fwd", "frame_scan_fwd_static", "frame_scan_fwd_fp8", "frame_scan_fwd_fp4", "frame_scan_bwd", "frame_scan_fwd_save", "saved_size", "workspace_size_bwd_saved", "workspace_size_bwd", "frame_step", "block_in_proj", "block_out_proj", "block_workspace_size", "profile_begin", "profile_end",
                "workspace_size", "make_desc", "alloc_workspace"):
        from . import api
        return getattr(api, name)
    if name == "frame_scan":
        from .autograd import frame_scan
        return frame_scan
    if name == "GdnError":
        from ._lib import GdnError
        return GdnError
    raise AttributeError(name)
