"""ctypes binding of libvimscan.so.

Argument marshalling only: shapes, dtypes and device pointers of torch tensors
are turned into the C ABI's plain sizes and pointers, and every step of the
scan runs in the library's HIP kernels. There is no fallback: if the library
is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libvimscan.so")

VS_F32, VS_BF16 = 0, 1
VS_OP_VIM_BIDIR, VS_OP_CROSS4, VS_OP_1D, VS_OP_VIM_GRAD = 0, 1, 2, 3
VS_OP_VIM_SAVED, VS_OP_VIM_GRAD_SAVED = 4, 5
VS_NOALLOC_MAX_ELEMS = 1 << 25

# names and argument types of every entry point declared in include/vimscan.h
_I64 = ctypes.c_int64
_I = ctypes.c_int
_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
SIGNATURES = {
    "vs_workspace_bytes": (_SZ, [_I, _I64, _I64, _I64, _I]),
    "vim_scan_bidir": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                            _P, _P, _SZ, _P]),
    "vim_scan_bidir_chunked": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _I, _I, _P, _P, _SZ, _P]),
    "vim_scan_bidir_noalloc": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                    _I, _P, _P]),
    "vim_scan_bidir_dirs": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                                 _P, _P, _SZ, _P]),
    "vim_scan_bidir_conv": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P, _P,
                                 _P, _P, _I, _P, _P, _SZ, _P]),
    "vim_scan_bidir_grad": (_I, [_I64, _I64, _I64, _I64, _I] + [_P] * 8 + [_I] + [_P] * 9 +
                            [_P, _SZ, _P]),
    "vim_scan_bidir_fwd_saved": (_I, [_I64, _I64, _I64, _I64, _I] + [_P] * 8 + [_I] +
                                 [_P, _P, _SZ, _P]),
    "vim_scan_bidir_grad_saved": (_I, [_I64, _I64, _I64, _I64, _I] + [_P] * 8 + [_I] +
                                  [_P, _SZ] + [_P] * 9 + [_P, _SZ, _P]),
    "vmamba_cross_scan4": (_I, [_I64, _I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P, _P,
                                _P, _I, _P, _P, _SZ, _P]),
    "s6_scan_1d": (_I, [_I64, _I64, _I64, _I64, _I, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I,
                        _P, _P]),
    "vim_x_proj": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P]),
    "vim_dt_proj": (_I, [_I64, _I64, _I64, _I, _P, _P, _P, _P]),
    "vim_out_proj": (_I, [_I64, _I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P]),
    "vs_strerror": (ctypes.c_char_p, [_I]),
    "vs_last_error": (ctypes.c_char_p, []),
    "vs_abi_version": (_I, []),
}


class LibraryMissing(ImportError):
    pass


def load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise LibraryMissing(
            "libvimscan.so not found at %s; build it first with "
            "`python -c 'import __graft_entry__ as g; g.build()'` or "
            "`python vision_mamba_selective_amd/build.py`" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class ScanError(RuntimeError):
    def __init__(self, fn, code):
        name = lib.vs_strerror(code).decode()
        detail = lib.vs_last_error().decode()
        super().__init__("%s failed: %s (%d): %s" % (fn, name, code, detail))
        self.code = code


def check(fn, code):
    if code != 0:
        raise ScanError(fn, code)
