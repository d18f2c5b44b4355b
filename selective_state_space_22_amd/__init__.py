"""MI355X (gfx950) selective scan (S6): HIP kernels behind a C ABI.

    from selective_state_space_22_amd import mamba_scan_fwd, mamba_scan_bwd, mamba_state_update

The functions are thin ctypes wrappers of libmamba_mi355x.so (see
include/mamba_mi355x.h); build the library with
``python -m selective_state_space_22_amd.build``.
"""
from .binding import (MAMBA_IO_BF16, MAMBA_IO_F32, MambaError, load_library, mamba_block_fwd,
                      mamba_get_option, mamba_set_option, mamba_stream_status,
                      mamba_block_fwd_workspace_size, mamba_scan_bwd,
                      mamba_scan_bwd_workspace_size, mamba_scan_fwd, mamba_scan_fwd_complex,
                      mamba_scan_fwd_complex_workspace_size, mamba_scan_fwd_noalloc, mamba_scan_fwd_workspace_size,
                      mamba_selection_fwd, mamba_selection_fwd_workspace_size, mamba_ssm_fwd,
                      mamba_ssm_fwd_workspace_size, mamba_state_update, mamba_state_update_complex, mamba_version,
                      status_string)

__all__ = ["mamba_block_fwd", "mamba_block_fwd_workspace_size", "mamba_scan_fwd", "mamba_scan_fwd_complex", "mamba_scan_fwd_complex_workspace_size", "mamba_scan_bwd",
           "mamba_state_update", "mamba_state_update_complex", "mamba_scan_fwd_workspace_size",
           "mamba_scan_bwd_workspace_size", "mamba_selection_fwd", "mamba_selection_fwd_workspace_size",
           "mamba_ssm_fwd", "mamba_ssm_fwd_workspace_size", "mamba_version", "status_string", "load_library", "MambaError",
           "MAMBA_IO_F32", "MAMBA_IO_BF16", "mamba_set_option", "mamba_get_option", "mamba_stream_status",
           "mamba_scan_fwd_noalloc"]
