"""GPU parity of the dilated depthwise 1-D convolution (deft_dwconv1d_forward)
against the fp64 oracle, on the JAX issue page's shapes.

The page's script feeds ramps (arange(size) / size) of shape (batch,
steps + dilation*(kernel-1), channels) and (kernel, 1, channels), batch 32,
1024 steps, kernel sizes 1/4/16/64, 32/128/512 channels, dilations 1..128 in
float32; these tests use the same generator and shapes (fewer batches where
the oracle would be slow), plus seeded normal inputs and ragged shapes.
Tolerance: rel-L2 1e-5 (fp32).
"""
import numpy as np
import pytest
import torch

from irregular_gather_cnn_amd import _lib as L
from oracle import dwconv as dw

pytestmark = pytest.mark.gpu


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (nb if nb > 0 else 1.0))


def ramp(shape):
    size = int(np.prod(shape))
    return (np.arange(size, dtype=np.float32) / size).reshape(shape)


def run(x, w, d):
    B, Lx, C = x.shape
    K = w.shape[0]
    T = Lx - d * (K - 1)
    xd, wd = torch.from_numpy(np.ascontiguousarray(x)).cuda(), torch.from_numpy(np.ascontiguousarray(w)).cuda()
    y = torch.full((B, T, C), float("nan"), dtype=torch.float32, device="cuda")
    L.deft_dwconv1d_forward(xd, wd, y, B, T, C, K, d, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("K", [1, 4, 16, 64])
@pytest.mark.parametrize("C", [32, 128, 512])
@pytest.mark.parametrize("d", [1, 3, 128])
def test_dwconv1d_page_grid(K, C, d):
    T, B = 1024, 2
    x = ramp((B, T + d * (K - 1), C))
    w = ramp((K, C))
    print("dwconv1d K=%d C=%d d=%d" % (K, C, d), flush=True)
    y = run(x, w, d)
    ref = dw.dwconv1d(x, w, d)
    assert np.isfinite(y).all()
    assert rel(y, ref) <= 1e-5


@pytest.mark.parametrize("B,T,C,K,d", [
    (3, 1000, 36, 5, 7),     # T not a multiple of d; 9 float4 lanes
    (2, 517, 68, 3, 2),      # 17 float4 lanes: a full and a one-lane channel slice
    (2, 5, 8, 3, 16),        # fewer steps than phases
    (1, 1, 4, 64, 1),        # a single output step
    (2, 300, 64, 200, 1),    # a long kernel: the tile shrinks to fit LDS
    (4, 96, 16, 7, 33),
])
def test_dwconv1d_ragged(B, T, C, K, d):
    r = np.random.default_rng(B * 1000 + T + C + K + d)
    x = r.standard_normal((B, T + d * (K - 1), C)).astype(np.float32)
    w = r.standard_normal((K, C)).astype(np.float32)
    print("dwconv1d ragged", (B, T, C, K, d), flush=True)
    y = run(x, w, d)
    assert rel(y, dw.dwconv1d(x, w, d)) <= 1e-5


def test_dwconv1d_full_page_size():
    """The page's largest case (batch 32, 1024 steps, 512 channels, kernel 64,
    dilation 128) at full size; two batches compared with the oracle, the
    others against the first through the ramp's structure-free check that
    every output is finite."""
    B, T, C, K, d = 32, 1024, 512, 64, 128
    x = ramp((B, T + d * (K - 1), C))
    w = ramp((K, C))
    print("dwconv1d full size", flush=True)
    y = run(x, w, d)
    assert np.isfinite(y).all()
    for b in (0, B - 1):
        assert rel(y[b:b + 1], dw.dwconv1d(x[b:b + 1], w, d)) <= 1e-5


def test_dwconv1d_empty_is_a_no_op():
    y = torch.full((1,), 7.0, device="cuda")
    L.deft_dwconv1d_forward(None, None, y, 0, 16, 8, 3, 2, torch.cuda.current_stream().cuda_stream)
    L.deft_dwconv1d_forward(None, None, y, 2, 0, 8, 3, 2, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert float(y.item()) == 7.0


# --- fused depthwise + pointwise ------------------------------------------------

def run_dwpw(x, wd, wp, d):
    B, Lx, C = x.shape
    K, O = wd.shape[0], wp.shape[1]
    T = Lx - d * (K - 1)
    t = [torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in (x, wd, wp)]
    z = torch.full((B, T, O), float("nan"), dtype=torch.float32, device="cuda")
    L.deft_dwpw1d_forward(t[0], t[1], t[2], z, B, T, C, O, K, d, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return z.cpu().numpy()


@pytest.mark.parametrize("B,T,C,O,K,d", [
    (2, 1024, 512, 512, 4, 1),   # the benchmark shape, fewer batches
    (2, 1024, 128, 128, 16, 8),
    (3, 100, 64, 288, 3, 2),     # ragged steps, output channels past one 256-wide tile
    (1, 7, 32, 32, 1, 1),
    (2, 70, 96, 64, 64, 3),
])
def test_dwpw1d_matches_oracle(B, T, C, O, K, d):
    r = np.random.default_rng(B + T + C + O + K + d)
    x = r.standard_normal((B, T + d * (K - 1), C)).astype(np.float32)
    wd = r.standard_normal((K, C)).astype(np.float32)
    wp = (r.standard_normal((C, O)) / np.sqrt(C)).astype(np.float32)
    print("dwpw1d", (B, T, C, O, K, d), flush=True)
    z = run_dwpw(x, wd, wp, d)
    assert np.isfinite(z).all()
    assert rel(z, dw.dwpw1d(x, wd, wp, d)) <= 1e-5


def test_dwpw1d_page_ramps():
    """The JAX page's ramp inputs through the fused module (channel mix by a
    ramp kernel too)."""
    B, T, C, O, K, d = 2, 256, 128, 64, 4, 16
    x = ramp((B, T + d * (K - 1), C))
    wd = ramp((K, C))
    wp = ramp((C, O))
    z = run_dwpw(x, wd, wp, d)
    assert rel(z, dw.dwpw1d(x, wd, wp, d)) <= 1e-5
