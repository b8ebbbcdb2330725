"""ctypes declarations of include/la.h and the loader of libla.so.

The library is loaded after ``import torch`` so that the process maps a
single HIP runtime: torch's ``libamdhip64.so`` carries the same soname
(``libamdhip64.so.7``) that libla.so was linked against.  There is no fallback
of any kind: if libla.so is missing the import of an entry point raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede the dlopen, see above)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libla.so")

LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EHIP = 0, 1, 2, 3
LA_NORMALIZED, LA_GATED, LA_GATED_DELTA, LA_RETENTION, LA_KDA = 0, 1, 2, 3, 4
LA_F32, LA_BF16 = 0, 1
LA_PHI_IDENTITY, LA_PHI_ELU1 = 0, 1
LA_ABI_VERSION = 3

EXPORTED = ("la_chunk_fwd_workspace", "la_chunk_fwd", "la_chunk_fwd_noalloc",
            "la_chunk_bwd_workspace", "la_chunk_bwd", "la_decode_step", "la_verify", "la_commit",
            "la_status_str", "la_last_error", "la_abi_version")
LA_NOALLOC_SCRATCH_BYTES = 32 << 20


class LaDesc(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("dtype", ctypes.c_int32), ("phi", ctypes.c_int32),
                ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libla.so (once) and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            "libla.so is not built (%s); run `python -m gated_delta_rule_causal_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, fp, sz = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t
    dp = ctypes.POINTER(LaDesc)
    lib.la_chunk_fwd_workspace.argtypes = [dp]
    lib.la_chunk_fwd_workspace.restype = sz
    lib.la_chunk_fwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, vp, fp, fp, vp, sz, vp]
    lib.la_chunk_fwd.restype = ctypes.c_int
    lib.la_chunk_bwd_workspace.argtypes = [dp]
    lib.la_chunk_bwd_workspace.restype = sz
    lib.la_chunk_bwd.argtypes = [dp, vp, vp, vp, fp, fp, fp, vp, fp, fp, vp, vp, vp, fp, fp, fp, vp, sz, vp]
    lib.la_chunk_bwd.restype = ctypes.c_int
    lib.la_chunk_fwd_noalloc.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, vp, fp, fp, vp]
    lib.la_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.la_decode_step.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, vp, vp]
    lib.la_decode_step.restype = ctypes.c_int
    lib.la_verify.argtypes = [dp, vp, vp, vp, fp, fp, fp, fp, vp, vp]
    lib.la_verify.restype = ctypes.c_int
    lib.la_commit.argtypes = [dp, vp, vp, fp, fp, vp, fp, fp, vp]
    lib.la_commit.restype = ctypes.c_int
    lib.la_status_str.argtypes = [ctypes.c_int]
    lib.la_status_str.restype = ctypes.c_char_p
    lib.la_last_error.argtypes = []
    lib.la_last_error.restype = ctypes.c_char_p
    lib.la_abi_version.argtypes = []
    lib.la_abi_version.restype = ctypes.c_int
    if lib.la_abi_version() != LA_ABI_VERSION:
        raise RuntimeError("libla.so ABI %d, binding expects %d" % (lib.la_abi_version(), LA_ABI_VERSION))
    _lib = lib
    return lib


class LaError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__("%s (%s)" % (load().la_status_str(status).decode(), detail))


def check(status: int):
    if status != LA_OK:
        raise LaError(status, load().la_last_error().decode())
