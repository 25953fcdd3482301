"""Host (CPU) build of the library's quantiser helpers for the CPU tests.

Compiles ``tests/host/quant_host.cpp`` -- which includes the library's own
``sq_device.h`` -- with hipcc in host-only mode into a shared library under
``tests/host/_build/`` (git-ignored), so that the quotient arithmetic the
kernels run can be replayed without a GPU.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "host", "quant_host.cpp")
CSRC = os.path.join(ROOT, "w8a8_int8_post_amd", "csrc")
OUT_DIR = os.path.join(HERE, "host", "_build")
LIB = os.path.join(OUT_DIR, "libquant_host.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    deps = [SRC, os.path.join(CSRC, "sq_device.h")]
    if os.path.exists(LIB) and os.path.getmtime(LIB) >= max(os.path.getmtime(d) for d in deps):
        return LIB
    os.makedirs(OUT_DIR, exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    # the kernels' own options that bear on the arithmetic: no contraction
    cmd = [HIPCC, "-x", "hip", "--cuda-host-only", "-O2", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-I", CSRC, SRC, "-o", tmp]
    subprocess.run(cmd, check=True, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        lib.hq_codes.argtypes = [P, P, ctypes.c_long, ctypes.c_int, P]
        lib.hq_codes.restype = None
        lib.hq_row_step.argtypes = [ctypes.c_float]
        lib.hq_row_step.restype = ctypes.c_float
        lib.hq_rounding_mismatches.argtypes = [ctypes.c_uint, ctypes.c_ulong]
        lib.hq_rounding_mismatches.restype = ctypes.c_long
        _lib = lib
    return _lib
