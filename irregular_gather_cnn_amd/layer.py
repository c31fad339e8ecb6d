"""DeformConv: a plan plus a workspace around the C ABI.

PyTorch only supplies device memory and the stream; every step of the layer
runs in libdeft.so through the binding in ``_lib``.
"""
from __future__ import annotations

import torch

from . import _lib


def _tdtype(dtype: str):
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


class DeformConv:
    """Deformable kh x kw convolution (offset conv -> bilinear sampling -> GEMM).

    ``plan``: None (planner default halo), a halo histogram (list of uint32) or
    a (tile_h, tile_w, halo, chunk) tuple for a forced plan.

    ``replan_every`` > 0: every forward also adds the required-halo histogram
    of its taps (emitted by the fused sampling kernel) to a device buffer;
    after that many forwards the next forward first re-plans from the
    accumulated histogram (the plan, and the workspace if it must grow, are
    swapped only between a backward and the next forward)."""

    def __init__(self, n, c_in, h, w, c_out, kh=3, kw=3, stride=(1, 1), pad=(1, 1), dil=(1, 1), groups=1,
                 dtype="bf16", plan=None, training=False, device="cuda", replan_every=0, hist_len=16):
        self.dtype = dtype
        self.tdtype = _tdtype(dtype)
        self.desc = _lib.make_desc(n, c_in, h, w, c_out, kh, kw, stride, pad, dil, groups,
                                   _lib.DEFT_BF16 if dtype == "bf16" else _lib.DEFT_F32)
        if isinstance(plan, tuple):
            self.plan = _lib.deft_plan_create_forced(self.desc, *plan)
        else:
            self.plan = _lib.deft_plan_create(self.desc, plan)
        self.info = _lib.deft_plan_get_info(self.plan)
        self.training = training
        self.ws_bytes = _lib.deft_workspace_bytes(self.plan, 1 if training else 0)
        self.device = device
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.ho, self.wo, self.oc = self.info["ho"], self.info["wo"], self.info["oc"]
        self.n, self.c_in, self.h, self.w, self.c_out = n, c_in, h, w, c_out
        self.kh, self.kw, self.groups = kh, kw, groups
        self.replan_every, self.hist_len = replan_every, hist_len
        self.hist = torch.zeros((hist_len,), dtype=torch.int32, device=device) if replan_every else None
        self.observed_calls, self.replans = 0, 0

    PLAN_KEYS = ("tile_h", "tile_w", "halo", "chunk", "gather_direct", "bwd_tile_h", "bwd_tile_w", "bwd_chunk",
                 "bwd_halo")

    def observed_histogram(self):
        """The required-halo histogram accumulated since the last re-plan."""
        return [int(v) & 0xFFFFFFFF for v in self.hist.cpu().tolist()]

    def _replan(self):
        hist = self.observed_histogram()
        self.hist.zero_()
        self.observed_calls = 0
        new = _lib.deft_plan_create(self.desc, hist)
        info = _lib.deft_plan_get_info(new)
        if all(info[k] == self.info[k] for k in self.PLAN_KEYS):
            _lib.deft_plan_destroy(new)
            return False
        _lib.deft_plan_destroy(self.plan)
        self.plan, self.info = new, info
        self.ws_bytes = _lib.deft_workspace_bytes(self.plan, 1 if self.training else 0)
        if self.ws_bytes > self.ws.numel():
            self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.replans += 1
        return True

    def __del__(self):
        try:
            _lib.deft_plan_destroy(self.plan)
        except Exception:
            pass

    def stream(self):
        return torch.cuda.current_stream().cuda_stream

    def forward(self, x, w_off, b_off, w, b, y=None, offsets=None, want_offsets=None):
        if y is None:
            y = torch.empty((self.n, self.c_out, self.ho, self.wo), dtype=self.tdtype, device=self.device)
        if want_offsets is None:
            want_offsets = self.training
        if offsets is None and want_offsets:
            offsets = torch.empty((self.n, self.oc, self.ho, self.wo), dtype=torch.float32, device=self.device)
        if self.replan_every:
            if self.observed_calls >= self.replan_every:
                self._replan()
            _lib.deft_forward_hist(self.plan, x, w_off, b_off, w, b, y, offsets, self.ws, self.ws_bytes, self.hist,
                                   self.hist_len, self.stream())
            self.observed_calls += 1
        else:
            _lib.deft_forward(self.plan, x, w_off, b_off, w, b, y, offsets, self.ws, self.ws_bytes, self.stream())
        return y, offsets

    def forward_unfused(self, x, w_off, b_off, w, b, y=None, offsets=None):
        """The three-operator form: offsets written to and read back from HBM."""
        if y is None:
            y = torch.empty((self.n, self.c_out, self.ho, self.wo), dtype=self.tdtype, device=self.device)
        if offsets is None:
            offsets = torch.empty((self.n, self.oc, self.ho, self.wo), dtype=torch.float32, device=self.device)
        _lib.deft_forward_unfused(self.plan, x, w_off, b_off, w, b, y, offsets, self.ws, self.ws_bytes,
                                  self.stream())
        return y, offsets

    def backward(self, x, w_off, w, offsets, dy, with_bias=True, out=None):
        if out is None:
            out = dict(dx=torch.empty_like(x), dw_off=torch.empty_like(w_off), dw=torch.empty_like(w),
                       db_off=torch.empty((self.oc,), dtype=self.tdtype, device=self.device) if with_bias else None,
                       db=torch.empty((self.c_out,), dtype=self.tdtype, device=self.device) if with_bias else None)
        _lib.deft_backward(self.plan, x, w_off, w, offsets, dy, self.ws, self.ws_bytes, out["dx"], out["dw_off"],
                           out["db_off"], out["dw"], out["db"], self.stream())
        return out

    def sample(self, x, offsets, cols=None):
        """Unfused sampling from given offsets: cols [N][Ho*Wo][kh*kw][Cin]."""
        if cols is None:
            cols = torch.empty((self.n, self.ho * self.wo, self.kh * self.kw, self.c_in), dtype=self.tdtype,
                               device=self.device)
        _lib.deft_debug_sample(self.plan, x, offsets, cols, self.stream())
        return cols

    def cols_view(self):
        """The deformed columns [N][Ho*Wo][kh*kw][Cin] the last forward left in the workspace."""
        elems = self.n * self.ho * self.wo * self.kh * self.kw * self.c_in
        esz = 2 if self.dtype == "bf16" else 4
        start = self.info["ws_cols_offset"]
        raw = self.ws[start:start + elems * esz]
        return raw.view(self.tdtype).view(self.n, self.ho * self.wo, self.kh * self.kw, self.c_in)


def index_stage(desc, offsets, groups, taps, ho, wo, n):
    """Tap index / corner mask from fp32 device offsets (deft_debug_sample_index)."""
    shp = (n, groups, taps, ho, wo)
    y0 = torch.empty(shp, dtype=torch.int32, device=offsets.device)
    x0 = torch.empty(shp, dtype=torch.int32, device=offsets.device)
    m = torch.empty(shp, dtype=torch.uint8, device=offsets.device)
    _lib.deft_debug_sample_index(desc, offsets, y0, x0, m, torch.cuda.current_stream().cuda_stream)
    return y0, x0, m


def halo_histogram(desc, offsets, hist_len=16):
    hist = torch.empty((hist_len,), dtype=torch.int32, device=offsets.device)
    _lib.deft_halo_histogram(desc, offsets, hist, hist_len, torch.cuda.current_stream().cuda_stream)
    return [int(v) & 0xFFFFFFFF for v in hist.cpu().tolist()]
