"""Independent numpy formulation of the deformable layer's forward pass.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Written separately from
``deft_oracle.c`` to cross-check it on small shapes: the bilinear gather is
written here in its separable "tent" form,
    v(py, px) = sum over image pixels (qy, qx) of
                max(0, 1-|qy-py|) * max(0, 1-|qx-px|) * x[qy, qx],
which equals the four-neighbour blend described on the DefT explainer page
(section "Why it fell short": gather the four neighbours of a fractional point
and average them by weight) with zero padding outside the image, and needs no
floor, no corner enumeration and no fully-outside test (a NaN coordinate is
treated as fully outside).  The offset and main convolutions are an explicit
im2col followed by a matrix product (numpy's matmul is the library step).
"""
from __future__ import annotations

import numpy as np


def _im2col(s, x):
    """Plain (undeformed) patches: [N][Ho*Wo][Cin][K]."""
    n, c, h, w = x.shape
    out = np.zeros((n, s.ho, s.wo, c, s.taps))
    for i in range(s.kh):
        for j in range(s.kw):
            k = i * s.kw + j
            for ho in range(s.ho):
                yy = ho * s.stride[0] - s.pad[0] + i * s.dil[0]
                if not 0 <= yy < h:
                    continue
                xs = np.arange(s.wo) * s.stride[1] - s.pad[1] + j * s.dil[1]
                ok = (xs >= 0) & (xs < w)
                view = out[:, ho, :, :, k]                                   # [N][Wo][Cin]
                view[:, ok, :] = np.transpose(x[:, :, yy, xs[ok]], (0, 2, 1))
    return out.reshape(n, s.ho * s.wo, c, s.taps)


def offset_conv(s, x, w_off, b_off=None):
    cols = _im2col(s, np.asarray(x, np.float64)).reshape(s.n, s.ho * s.wo, -1)
    wm = np.asarray(w_off, np.float64).reshape(s.oc, -1)
    off = cols @ wm.T
    if b_off is not None:
        off = off + np.asarray(b_off, np.float64)[None, None, :]
    return np.transpose(off, (0, 2, 1)).reshape(s.n, s.oc, s.ho, s.wo)


def sample_cols(s, x, off):
    """Deformed columns [N][Ho*Wo][Cin][K] via the tent-function form."""
    x = np.asarray(x, np.float64)
    off = np.asarray(off, np.float64)
    cg = s.c_in // s.groups
    col = np.zeros((s.n, s.ho, s.wo, s.c_in, s.taps))
    qy = np.arange(s.h, dtype=np.float64)
    qx = np.arange(s.w, dtype=np.float64)
    hob = np.arange(s.ho) * s.stride[0] - s.pad[0]
    wob = np.arange(s.wo) * s.stride[1] - s.pad[1]
    for g in range(s.groups):
        xg = x[:, g * cg:(g + 1) * cg]                               # [N][Cg][H][W]
        for k in range(s.taps):
            i, j = divmod(k, s.kw)
            py = hob[None, :, None] + i * s.dil[0] + off[:, 2 * (g * s.taps + k)]      # [N][Ho][Wo]
            px = wob[None, None, :] + j * s.dil[1] + off[:, 2 * (g * s.taps + k) + 1]
            bad = np.isnan(py) | np.isnan(px)
            py = np.where(bad, -10.0, py)
            px = np.where(bad, -10.0, px)
            wy = np.maximum(0.0, 1.0 - np.abs(qy[None, None, None, :] - py[..., None]))  # [N][Ho][Wo][H]
            wx = np.maximum(0.0, 1.0 - np.abs(qx[None, None, None, :] - px[..., None]))  # [N][Ho][Wo][W]
            col[:, :, :, g * cg:(g + 1) * cg, k] = np.einsum("nabh,nchw,nabw->nabc", wy, xg, wx)
    return col.reshape(s.n, s.ho * s.wo, s.c_in, s.taps)


def main_conv(s, col, w, b=None):
    cm = np.asarray(col, np.float64).reshape(s.n, s.ho * s.wo, -1)
    wm = np.asarray(w, np.float64).reshape(s.c_out, -1)
    y = cm @ wm.T
    if b is not None:
        y = y + np.asarray(b, np.float64)[None, None, :]
    return np.transpose(y, (0, 2, 1)).reshape(s.n, s.c_out, s.ho, s.wo)


def forward(s, x, w_off, b_off, w, b):
    off = offset_conv(s, x, w_off, b_off)
    col = sample_cols(s, x, off)
    return main_conv(s, col, w, b), off, col
