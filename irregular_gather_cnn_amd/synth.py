"""Seeded synthetic workloads for the deformable 3x3 layer.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the layer's arithmetic, so both the HIP path and the CPU oracle
can be fed from it.

The DefT explainer page measures on detection and classification models whose
datasets and weights are not available here; it states only that learned
offsets form a tight distribution near zero, mostly within about a pixel, and
smaller in deeper layers (section "How DefT works", "The idea").  The
workloads below stand in for them with the shapes listed and:
  x      ~ U(-1, 1)
  w      ~ N(0, sqrt(2 / (Cin*K)))            (Kaiming normal, fan-in)
  w_off  ~ N(0, t * sqrt(3 / (Cin*K)))        so an interior offset has std t
           (a sum of Cin*K terms w*x with Var(x) = 1/3); t = 1 px, or 4 px for
           the wide-offset workload
  biases   0, except in the wide-offset workload, where two seeded
           (group, tap) pairs get a dy bias of +2H, which pushes their taps
           fully outside the image (2/36 = 5.6% of taps)
  dy     ~ N(0, 1)
Each tensor has its own stream: numpy PCG64 seeded with [workload id, tensor
id] (x=1, w=2, w_off=3, dy=4, push choice=5).  bf16 workloads round the fp32
draws to bf16 (round to nearest even).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # stream id mixed into every seed
    n: int
    c_in: int
    c_out: int
    h: int
    w: int
    kh: int = 3
    kw: int = 3
    stride: int = 1
    pad: int = 1
    dil: int = 1
    groups: int = 1
    dtype: str = "f32"       # "f32" or "bf16"
    offset_std: float = 1.0  # pixels
    pushed_pairs: int = 0    # (group, tap) pairs pushed fully outside
    train: bool = False

    @property
    def ho(self) -> int:
        return (self.h + 2 * self.pad - self.dil * (self.kh - 1) - 1) // self.stride + 1

    @property
    def wo(self) -> int:
        return (self.w + 2 * self.pad - self.dil * (self.kw - 1) - 1) // self.stride + 1

    @property
    def taps(self) -> int:
        return self.kh * self.kw

    @property
    def oc(self) -> int:
        return 2 * self.groups * self.taps

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32_n1_c16_16x16", 1, n=1, c_in=16, c_out=16, h=16, w=16, dtype="f32"),
        Workload("fp32_n8_c128_64x64", 2, n=8, c_in=128, c_out=128, h=64, w=64, dtype="f32"),
        Workload("bf16_n16_c256_56x56", 3, n=16, c_in=256, c_out=256, h=56, w=56, dtype="bf16"),
        Workload("bf16_n16_c512_28x28_g4_wide", 4, n=16, c_in=512, c_out=512, h=28, w=28,
                 groups=4, dtype="bf16", offset_std=4.0, pushed_pairs=2),
        Workload("train_bf16_n16_c256_56x56_s1", 5, n=16, c_in=256, c_out=256, h=56, w=56,
                 dtype="bf16", train=True),
        Workload("train_bf16_n16_c256_56x56_s2", 6, n=16, c_in=256, c_out=256, h=56, w=56,
                 stride=2, dtype="bf16", train=True),
    ]
}


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest-even bf16 value, returned as fp32 (exactly representable)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Bit patterns (uint16) of bf16-valued fp32 data (already rounded)."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _rng(wl: Workload, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([wl.wid, tensor]))


def make_inputs(wl: Workload, with_dy: bool | None = None) -> dict:
    """fp32 numpy arrays on the storage grid of ``wl.dtype``:
    x [N][Cin][H][W], w_off [Oc][Cin][kh][kw], b_off [Oc], w [Cout][Cin][kh][kw],
    b [Cout] and, for training workloads, dy [N][Cout][Ho][Wo]."""
    ck = wl.c_in * wl.taps
    x = _rng(wl, 1).uniform(-1.0, 1.0, size=(wl.n, wl.c_in, wl.h, wl.w)).astype(np.float32)
    w = _rng(wl, 2).standard_normal((wl.c_out, wl.c_in, wl.kh, wl.kw), dtype=np.float32)
    w *= np.float32(np.sqrt(2.0 / ck))
    sigma = wl.offset_std * np.sqrt(3.0 / ck)
    w_off = _rng(wl, 3).standard_normal((wl.oc, wl.c_in, wl.kh, wl.kw), dtype=np.float32)
    w_off *= np.float32(sigma)
    b_off = np.zeros((wl.oc,), np.float32)
    if wl.pushed_pairs:
        pairs = _rng(wl, 5).choice(wl.groups * wl.taps, size=wl.pushed_pairs, replace=False)
        for gk in pairs:
            b_off[2 * int(gk)] = 2.0 * wl.h
    b = np.zeros((wl.c_out,), np.float32)
    out = dict(x=x, w=w, w_off=w_off, b_off=b_off, b=b)
    if with_dy if with_dy is not None else wl.train:
        out["dy"] = _rng(wl, 4).standard_normal((wl.n, wl.c_out, wl.ho, wl.wo), dtype=np.float32)
    if wl.dtype == "bf16":
        out = {k: round_bf16(v) for k, v in out.items()}
    return out
