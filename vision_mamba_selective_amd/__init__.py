"""MI355X (gfx950) selective scan for Vision Mamba and VMamba.

The scan itself lives in libvimscan.so (HIP kernels behind a C ABI,
include/vimscan.h). This package holds the in-tree build step, the ctypes
binding with the same entry-point names, and the seeded workload generator.
The binding is imported lazily so that the generator can be used without the
library.
"""

__all__ = ["vim_scan_bidir", "vim_scan_bidir_noalloc", "vim_scan_bidir_chunked", "vim_scan_bidir_dirs", "vim_scan_bidir_conv", "vim_scan_bidir_grad",
           "vim_scan_bidir_fwd_saved", "vim_scan_bidir_grad_saved",
           "VimScanFunction", "vim_scan_bidir_autograd",
           "vmamba_cross_scan4", "s6_scan_1d", "workspace_bytes", "vim_x_proj", "vim_dt_proj",
           "vim_out_proj"]


def __getattr__(name):
    if name in __all__:
        from . import scan
        return getattr(scan, name)
    raise AttributeError(name)
