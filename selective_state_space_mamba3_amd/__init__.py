"""MI355X (gfx950) Mamba-3 selective-state path: forward, decode and backward.

The compute lives in libm3.so (hand-written HIP kernels behind a C ABI, see
include/m3.h); this package is its thin ctypes binding, with torch used for
device memory and streams only.  Entry points carry the C names:
m3_preprocess, m3_siso_fwd, m3_mimo_fwd, m3_siso_step, m3_mimo_step,
m3_siso_fwd_packed, m3_siso_bwd, m3_mimo_bwd, m3_preprocess_bwd.
"""

from ._binding import (  # noqa: F401
    LIB_PATH,
    M3Error,
    PreprocessConfig,
    SsmConfig,
    header_functions,
    last_error,
    lib,
    m3_mimo_bwd,
    m3_mimo_fwd,
    m3_mimo_step,
    m3_preprocess,
    m3_preprocess_bwd,
    m3_siso_bwd,
    m3_siso_fwd,
    m3_siso_fwd_noalloc,
    m3_siso_fwd_packed,
    m3_siso_step,
    mimo_bwd_workspace_bytes,
    mimo_fwd_workspace_bytes,
    scan_segments,
    set_scan_segments,
    siso_bwd_workspace_bytes,
    siso_fwd_packed_workspace_bytes,
    siso_fwd_workspace_bytes,
)
