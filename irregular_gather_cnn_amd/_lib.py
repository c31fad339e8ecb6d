"""ctypes binding of libdeft.so (include/deft.h): argument marshalling only.

Every function keeps the C name and signature; device pointers may be passed
as torch tensors (their ``data_ptr()``), plain integers or ``None`` (NULL).
A non-zero status raises :class:`DeftError`.  Nothing here computes any part
of the layer: all of it runs in the HIP library, and loading fails loudly if
the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# DEFT_LIB names another build of the same library (e.g. a measurement
# variant); the default is the in-tree libdeft.so
LIB_PATH = os.environ.get("DEFT_LIB") or os.path.join(_PKG, "libdeft.so")

DEFT_F32, DEFT_BF16 = 0, 1
STATUS = {0: "DEFT_OK", -1: "DEFT_ERR_BAD_DESC", -2: "DEFT_ERR_GROUPS", -3: "DEFT_ERR_SHAPE",
          -4: "DEFT_ERR_NULLPTR", -5: "DEFT_ERR_WORKSPACE", -6: "DEFT_ERR_DTYPE", -7: "DEFT_ERR_ALIGN",
          -8: "DEFT_ERR_HIP", -9: "DEFT_ERR_PLAN", -10: "DEFT_ERR_UNSUPPORTED",
          -11: "DEFT_ERR_SCRATCH"}
EXPORTED = ["deft_desc_validate", "deft_plan_create", "deft_plan_create_forced", "deft_plan_get_info",
            "deft_plan_destroy", "deft_workspace_bytes", "deft_forward", "deft_forward_hist", "deft_forward_unfused",
            "deft_forward_noalloc",
            "deft_backward",
            "deft_debug_sample_index", "deft_debug_sample", "deft_halo_histogram", "deft_error_string",
            "deft_last_hip_error", "deft_timing_start", "deft_timing_stop", "deft_timing_count",
            "deft_timing_get", "deft_dwconv1d_forward", "deft_dwpw1d_forward"]


class DeftError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = "%s failed: %s (%s)" % (where, STATUS.get(code, code), deft_error_string(code))
        if code == -8:
            msg += ": " + deft_last_hip_error()
        super().__init__(msg)


class deft_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "n", "c_in", "h", "w", "c_out", "kh", "kw", "stride_h", "stride_w", "pad_h", "pad_w", "dil_h",
        "dil_w", "offset_groups", "dtype")]


class deft_plan_info(ctypes.Structure):
    _fields_ = [("tile_h", ctypes.c_int), ("tile_w", ctypes.c_int), ("halo", ctypes.c_int),
                ("chunk", ctypes.c_int), ("groups_per_wg", ctypes.c_int), ("num_workgroups", ctypes.c_int),
                ("ho", ctypes.c_int), ("wo", ctypes.c_int), ("oc", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("est_miss_fraction", ctypes.c_double), ("ws_forward", ctypes.c_size_t),
                ("ws_training", ctypes.c_size_t), ("ws_cols_offset", ctypes.c_size_t),
                ("bwd_tile_h", ctypes.c_int), ("bwd_tile_w", ctypes.c_int), ("bwd_chunk", ctypes.c_int),
                ("gemm_direct", ctypes.c_int), ("dw_splits", ctypes.c_int), ("gather_direct", ctypes.c_int),
                ("gather_gemm", ctypes.c_int), ("bwd_halo", ctypes.c_int)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libdeft.so; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libdeft.so is not built (%s); run irregular_gather_cnn_amd/build.py or "
                           "__graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dp = ctypes.POINTER(deft_desc)
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "deft_desc_validate": (i, [dp]),
        "deft_plan_create": (i, [dp, vp, i, pp]),
        "deft_plan_create_forced": (i, [dp, i, i, i, i, pp]),
        "deft_plan_get_info": (i, [vp, ctypes.POINTER(deft_plan_info)]),
        "deft_plan_destroy": (None, [vp]),
        "deft_workspace_bytes": (sz, [vp, i]),
        "deft_forward": (i, [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "deft_forward_unfused": (i, [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "deft_forward_noalloc": (i, [vp, vp, vp, vp, vp, vp, vp, vp, vp]),
        "deft_forward_hist": (i, [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i, vp]),
        "deft_dwconv1d_forward": (i, [vp, vp, vp, i, i, i, i, i, vp]),
        "deft_dwpw1d_forward": (i, [vp, vp, vp, vp, i, i, i, i, i, i, vp]),
        "deft_backward": (i, [vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp]),
        "deft_debug_sample_index": (i, [dp, vp, vp, vp, vp, vp]),
        "deft_debug_sample": (i, [vp, vp, vp, vp, vp]),
        "deft_halo_histogram": (i, [dp, vp, vp, i, vp]),
        "deft_error_string": (ctypes.c_char_p, [i]),
        "deft_last_hip_error": (ctypes.c_char_p, []),
        "deft_timing_start": (i, [i]),
        "deft_timing_stop": (i, []),
        "deft_timing_count": (i, []),
        "deft_timing_get": (i, [i, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    if isinstance(t, ctypes.c_void_p):
        return t.value
    raise TypeError("expected a tensor, int or None, got %r" % type(t))


def _check(code: int, where: str):
    if code != 0:
        raise DeftError(code, where)


def make_desc(n, c_in, h, w, c_out, kh=3, kw=3, stride=(1, 1), pad=(1, 1), dil=(1, 1), groups=1,
              dtype=DEFT_BF16) -> deft_desc:
    return deft_desc(n, c_in, h, w, c_out, kh, kw, stride[0], stride[1], pad[0], pad[1], dil[0], dil[1],
                     groups, dtype)


def deft_desc_validate(desc: deft_desc) -> int:
    return load().deft_desc_validate(ctypes.byref(desc))


def deft_plan_create(desc: deft_desc, halo_hist=None) -> ctypes.c_void_p:
    """halo_hist: None or a host sequence of uint32 counts."""
    lib = load()
    out = ctypes.c_void_p()
    if halo_hist is None:
        _check(lib.deft_plan_create(ctypes.byref(desc), None, 0, ctypes.byref(out)), "deft_plan_create")
    else:
        arr = (ctypes.c_uint32 * len(halo_hist))(*[int(v) for v in halo_hist])
        _check(lib.deft_plan_create(ctypes.byref(desc), ctypes.cast(arr, ctypes.c_void_p), len(halo_hist),
                                    ctypes.byref(out)), "deft_plan_create")
    return out


def deft_plan_create_forced(desc: deft_desc, tile_h: int, tile_w: int, halo: int, chunk: int = 0):
    out = ctypes.c_void_p()
    _check(load().deft_plan_create_forced(ctypes.byref(desc), tile_h, tile_w, halo, chunk, ctypes.byref(out)),
           "deft_plan_create_forced")
    return out


def deft_plan_get_info(plan) -> dict:
    info = deft_plan_info()
    _check(load().deft_plan_get_info(plan, ctypes.byref(info)), "deft_plan_get_info")
    return {f: getattr(info, f) for f, _ in deft_plan_info._fields_}


def deft_plan_destroy(plan) -> None:
    load().deft_plan_destroy(plan)


def deft_workspace_bytes(plan, training: int) -> int:
    return int(load().deft_workspace_bytes(plan, int(training)))


def deft_forward(plan, x, w_off, b_off, w, b, y, offsets_out, workspace, ws_bytes, stream=None) -> None:
    _check(load().deft_forward(plan, _ptr(x), _ptr(w_off), _ptr(b_off), _ptr(w), _ptr(b), _ptr(y),
                               _ptr(offsets_out), _ptr(workspace), int(ws_bytes), _ptr(stream)), "deft_forward")


def deft_forward_noalloc(plan, x, w_off, b_off, w, b, y, offsets_out, stream=None) -> None:
    _check(load().deft_forward_noalloc(plan, _ptr(x), _ptr(w_off), _ptr(b_off), _ptr(w), _ptr(b), _ptr(y),
                                       _ptr(offsets_out), _ptr(stream)), "deft_forward_noalloc")


# Bytes of the static scratch behind deft_forward_noalloc (DEFT_NOALLOC_SCRATCH_BYTES in deft.h).
NOALLOC_SCRATCH_BYTES = 64 << 20


def deft_forward_hist(plan, x, w_off, b_off, w, b, y, offsets_out, workspace, ws_bytes, hist, hist_len,
                      stream=None) -> None:
    _check(load().deft_forward_hist(plan, _ptr(x), _ptr(w_off), _ptr(b_off), _ptr(w), _ptr(b), _ptr(y),
                                    _ptr(offsets_out), _ptr(workspace), int(ws_bytes), _ptr(hist), int(hist_len),
                                    _ptr(stream)), "deft_forward_hist")


def deft_dwconv1d_forward(x, w, y, batch, steps, channels, ksize, dilation, stream=None) -> None:
    _check(load().deft_dwconv1d_forward(_ptr(x), _ptr(w), _ptr(y), int(batch), int(steps), int(channels),
                                        int(ksize), int(dilation), _ptr(stream)), "deft_dwconv1d_forward")


def deft_dwpw1d_forward(x, w_dw, w_pw, z, batch, steps, channels, out_channels, ksize, dilation,
                        stream=None) -> None:
    _check(load().deft_dwpw1d_forward(_ptr(x), _ptr(w_dw), _ptr(w_pw), _ptr(z), int(batch), int(steps),
                                      int(channels), int(out_channels), int(ksize), int(dilation), _ptr(stream)),
           "deft_dwpw1d_forward")


def deft_forward_unfused(plan, x, w_off, b_off, w, b, y, offsets, workspace, ws_bytes, stream=None) -> None:
    _check(load().deft_forward_unfused(plan, _ptr(x), _ptr(w_off), _ptr(b_off), _ptr(w), _ptr(b), _ptr(y),
                                       _ptr(offsets), _ptr(workspace), int(ws_bytes), _ptr(stream)),
           "deft_forward_unfused")


def deft_backward(plan, x, w_off, w, offsets, dy, workspace, ws_bytes, dx, dw_off, db_off, dw, db,
                  stream=None) -> None:
    _check(load().deft_backward(plan, _ptr(x), _ptr(w_off), _ptr(w), _ptr(offsets), _ptr(dy), _ptr(workspace),
                                int(ws_bytes), _ptr(dx), _ptr(dw_off), _ptr(db_off), _ptr(dw), _ptr(db),
                                _ptr(stream)), "deft_backward")


def deft_debug_sample_index(desc: deft_desc, offsets, y0, x0, mask, stream=None) -> None:
    _check(load().deft_debug_sample_index(ctypes.byref(desc), _ptr(offsets), _ptr(y0), _ptr(x0), _ptr(mask),
                                          _ptr(stream)), "deft_debug_sample_index")


def deft_debug_sample(plan, x, offsets, cols, stream=None) -> None:
    _check(load().deft_debug_sample(plan, _ptr(x), _ptr(offsets), _ptr(cols), _ptr(stream)), "deft_debug_sample")


def deft_halo_histogram(desc: deft_desc, offsets, hist, hist_len: int, stream=None) -> None:
    _check(load().deft_halo_histogram(ctypes.byref(desc), _ptr(offsets), _ptr(hist), int(hist_len),
                                      _ptr(stream)), "deft_halo_histogram")


def deft_error_string(code: int) -> str:
    return load().deft_error_string(int(code)).decode()


def deft_last_hip_error() -> str:
    return load().deft_last_hip_error().decode()


def deft_timing_start(capacity: int) -> None:
    _check(load().deft_timing_start(int(capacity)), "deft_timing_start")


def deft_timing_stop() -> None:
    _check(load().deft_timing_stop(), "deft_timing_stop")


def deft_timing_count() -> int:
    return int(load().deft_timing_count())


def deft_timing_get(i: int):
    name = ctypes.c_char_p()
    ms = ctypes.c_float()
    _check(load().deft_timing_get(int(i), ctypes.byref(name), ctypes.byref(ms)), "deft_timing_get")
    return name.value.decode(), float(ms.value)
