"""CPU oracle for the deformable 3x3 convolution layer -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package.  The product path (``irregular_gather_cnn_amd``) never
imports it and shares no code with it.

``deft_oracle.c`` holds the arithmetic (fp64 direct loops, see its header for
the definition and its citations of the DefT explainer page).  This module only
compiles it, loads it with ctypes and marshals numpy arrays in and out.
``ref_np`` is a second, independently written numpy formulation of the forward
pass used to cross-check the C one on small shapes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "deft_oracle.c")
_LIB = os.path.join(_HERE, "libdeft_oracle.so")


def build(force: bool = False) -> str:
    """Compile deft_oracle.c into libdeft_oracle.so (gcc, OpenMP, no fast-math,
    no FMA contraction so the fp32 index stage is a single rounded add)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
               "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n", "c_in", "h", "w", "c_out", "kh", "kw", "stride_h", "stride_w", "pad_h", "pad_w",
        "dil_h", "dil_w", "groups")]


@dataclass(frozen=True)
class Shape:
    """Layer hyper-parameters.  ``groups`` is the offset-group count."""
    n: int
    c_in: int
    h: int
    w: int
    c_out: int
    kh: int = 3
    kw: int = 3
    stride: tuple = (1, 1)
    pad: tuple = (1, 1)
    dil: tuple = (1, 1)
    groups: int = 1

    @property
    def ho(self) -> int:
        return (self.h + 2 * self.pad[0] - self.dil[0] * (self.kh - 1) - 1) // self.stride[0] + 1

    @property
    def wo(self) -> int:
        return (self.w + 2 * self.pad[1] - self.dil[1] * (self.kw - 1) - 1) // self.stride[1] + 1

    @property
    def taps(self) -> int:
        return self.kh * self.kw

    @property
    def oc(self) -> int:
        return 2 * self.groups * self.taps

    def cdesc(self) -> _Desc:
        return _Desc(self.n, self.c_in, self.h, self.w, self.c_out, self.kh, self.kw,
                     self.stride[0], self.stride[1], self.pad[0], self.pad[1], self.dil[0],
                     self.dil[1], self.groups)


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        dp = ctypes.POINTER(ctypes.c_double)
        vp = ctypes.c_void_p
        desc = ctypes.POINTER(_Desc)
        lib.oracle_offset_conv.argtypes = [desc, dp, dp, dp, dp]
        lib.oracle_sample_cols.argtypes = [desc, dp, dp, dp]
        lib.oracle_main_conv.argtypes = [desc, dp, dp, dp, dp]
        lib.oracle_forward.argtypes = [desc, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_backward.argtypes = [desc, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp]
        lib.oracle_sample_index_f32.argtypes = [desc, vp, vp, vp, vp]
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        for f in (lib.oracle_offset_conv, lib.oracle_sample_cols, lib.oracle_main_conv,
                  lib.oracle_forward, lib.oracle_backward, lib.oracle_sample_index_f32):
            f.restype = None
        _lib = lib
    return _lib


def threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().oracle_threads())


def _d(a, shape=None):
    """fp64, C-contiguous copy of ``a`` (exact for fp32 and bf16-valued input)."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError("expected shape %s, got %s" % (tuple(shape), a.shape))
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def offset_conv(s: Shape, x, w_off, b_off=None):
    lib = _load()
    x = _d(x, (s.n, s.c_in, s.h, s.w))
    w_off = _d(w_off, (s.oc, s.c_in, s.kh, s.kw))
    b_off = None if b_off is None else _d(b_off, (s.oc,))
    off = np.empty((s.n, s.oc, s.ho, s.wo))
    d = s.cdesc()
    lib.oracle_offset_conv(ctypes.byref(d), _p(x), _p(w_off), _p(b_off), _p(off))
    return off


def sample_cols(s: Shape, x, off):
    """Deformed columns, laid out [N][Ho*Wo][Cin][K]."""
    lib = _load()
    x = _d(x, (s.n, s.c_in, s.h, s.w))
    off = _d(off, (s.n, s.oc, s.ho, s.wo))
    col = np.empty((s.n, s.ho * s.wo, s.c_in, s.taps))
    d = s.cdesc()
    lib.oracle_sample_cols(ctypes.byref(d), _p(x), _p(off), _p(col))
    return col


def main_conv(s: Shape, col, w, b=None):
    lib = _load()
    col = _d(col, (s.n, s.ho * s.wo, s.c_in, s.taps))
    w = _d(w, (s.c_out, s.c_in, s.kh, s.kw))
    b = None if b is None else _d(b, (s.c_out,))
    y = np.empty((s.n, s.c_out, s.ho, s.wo))
    d = s.cdesc()
    lib.oracle_main_conv(ctypes.byref(d), _p(col), _p(w), _p(b), _p(y))
    return y


def forward(s: Shape, x, w_off, b_off, w, b, want_cols: bool = False):
    """Returns (y, offsets[, cols]) in fp64."""
    lib = _load()
    x = _d(x, (s.n, s.c_in, s.h, s.w))
    w_off = _d(w_off, (s.oc, s.c_in, s.kh, s.kw))
    b_off = None if b_off is None else _d(b_off, (s.oc,))
    w = _d(w, (s.c_out, s.c_in, s.kh, s.kw))
    b = None if b is None else _d(b, (s.c_out,))
    y = np.empty((s.n, s.c_out, s.ho, s.wo))
    off = np.empty((s.n, s.oc, s.ho, s.wo))
    col = np.empty((s.n, s.ho * s.wo, s.c_in, s.taps)) if want_cols else None
    d = s.cdesc()
    lib.oracle_forward(ctypes.byref(d), _p(x), _p(w_off), _p(b_off), _p(w), _p(b), _p(y),
                       _p(off), _p(col))
    return (y, off, col) if want_cols else (y, off)


def backward(s: Shape, x, w_off, w, off, dy):
    """Returns dict with dx, dw_off, db_off, dw, db, doff (fp64).  ``off`` are
    the forward's offsets; pass the ones the path under test used."""
    lib = _load()
    x = _d(x, (s.n, s.c_in, s.h, s.w))
    w_off = _d(w_off, (s.oc, s.c_in, s.kh, s.kw))
    w = _d(w, (s.c_out, s.c_in, s.kh, s.kw))
    off = _d(off, (s.n, s.oc, s.ho, s.wo))
    dy = _d(dy, (s.n, s.c_out, s.ho, s.wo))
    out = dict(dx=np.empty((s.n, s.c_in, s.h, s.w)), dw_off=np.empty((s.oc, s.c_in, s.kh, s.kw)),
               db_off=np.empty((s.oc,)), dw=np.empty((s.c_out, s.c_in, s.kh, s.kw)),
               db=np.empty((s.c_out,)), doff=np.empty((s.n, s.oc, s.ho, s.wo)))
    d = s.cdesc()
    lib.oracle_backward(ctypes.byref(d), _p(x), _p(w_off), _p(w), _p(off), _p(dy),
                        _p(out["dx"]), _p(out["dw_off"]), _p(out["db_off"]), _p(out["dw"]),
                        _p(out["db"]), _p(out["doff"]))
    return out


def sample_index_f32(s: Shape, off_f32):
    """Integer tap index / corner mask from fp32 offsets; arrays [N][G][K][Ho][Wo]."""
    lib = _load()
    off = np.ascontiguousarray(np.asarray(off_f32, dtype=np.float32))
    if off.shape != (s.n, s.oc, s.ho, s.wo):
        raise ValueError("offsets must be [N][Oc][Ho][Wo]")
    shp = (s.n, s.groups, s.taps, s.ho, s.wo)
    y0 = np.empty(shp, np.int32)
    x0 = np.empty(shp, np.int32)
    m = np.empty(shp, np.uint8)
    d = s.cdesc()
    lib.oracle_sample_index_f32(ctypes.byref(d), off.ctypes.data, y0.ctypes.data,
                                x0.ctypes.data, m.ctypes.data)
    return y0, x0, m
