"""MI355X (gfx950) deformable 3x3 convolution: fused offset-conv + bilinear
sampling, MFMA GEMM main convolution and backward, behind the C ABI of
include/deft.h (libdeft.so).  ``_lib`` is the ctypes binding, ``layer`` a thin
plan/workspace helper, ``synth`` the seeded synthetic workloads."""
from . import _lib  # noqa: F401
from ._lib import DeftError, load  # noqa: F401
