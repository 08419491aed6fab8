"""MI355X-native (gfx950) selective-scan library.

The compute path is libmamba_scan.so: hand-written HIP kernels behind the C
ABI declared in include/mamba_scan.h.  This package holds its sources
(csrc/), the in-tree build step (build.py), a ctypes binding that only
marshals arguments (_binding.py), and the seeded input generator used by the
tests and the benchmark (inputs.py).
"""
from ._binding import (DIR_BIDIR, DIR_BWD, DIR_CROSS2D, DIR_FWD, DTYPE_BF16, DTYPE_F32, EXPORTED, LIB_PATH,
                       MambaDims, MambaError, ScanStepper, bwd_workspace_bytes, conv1d_silu, load_library, make_dims, num_dirs,
                       saved_bytes, scan_bwd, scan_fwd, scan_fwd_noalloc, scan_fwd_save, scan_step, status_string, workspace_bytes)

__all__ = ["DIR_BIDIR", "DIR_BWD", "DIR_CROSS2D", "DIR_FWD", "DTYPE_BF16", "DTYPE_F32", "EXPORTED", "LIB_PATH",
           "MambaDims", "MambaError", "ScanStepper", "bwd_workspace_bytes", "conv1d_silu", "load_library", "make_dims", "num_dirs",
           "saved_bytes", "scan_bwd", "scan_fwd", "scan_fwd_noalloc", "scan_fwd_save", "scan_step", "status_string", "workspace_bytes"]
