"""Pins for the CPU oracle: checks against what the definition and mathematics
fix, independent of the oracle's own formulation.

The DefT explainer page prints no formula and no worked example, so the pins
are special cases that reduce to a library routine (an ordinary convolution),
closed forms (integer shifts, affine images), invariants (partition of unity,
offset-group replication, adjointness) and brute force (finite differences).
Each is chosen so that a plausible mistake (dy/dx swapped, wrong sign, wrong
tap order, a dropped corner, a wrong gradient term) fails at least one.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import Shape, ref_np

pytestmark = pytest.mark.filterwarnings("ignore")


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b.ravel())
    return np.linalg.norm((a - b).ravel()) / (nb if nb > 0 else 1.0)


def rand_layer(s: Shape, seed: int, off_scale: float = 0.5):
    r = np.random.default_rng(seed)
    x = r.uniform(-1, 1, (s.n, s.c_in, s.h, s.w))
    w = r.standard_normal((s.c_out, s.c_in, s.kh, s.kw)) * 0.3
    b = r.standard_normal(s.c_out)
    w_off = r.standard_normal((s.oc, s.c_in, s.kh, s.kw)) * off_scale
    b_off = r.standard_normal(s.oc) * 0.7
    return x, w_off, b_off, w, b


def torch_conv(s: Shape, x, w, b):
    return F.conv2d(torch.from_numpy(np.asarray(x, np.float64)), torch.from_numpy(np.asarray(w, np.float64)),
                    None if b is None else torch.from_numpy(np.asarray(b, np.float64)),
                    stride=s.stride, padding=s.pad, dilation=s.dil).numpy()


SHAPES = [
    Shape(2, 4, 7, 6, 3),
    Shape(1, 6, 9, 8, 5, stride=(2, 2)),
    Shape(2, 4, 8, 9, 3, pad=(2, 2), dil=(2, 2)),
    Shape(1, 4, 6, 7, 2, pad=(0, 0), groups=2),
    Shape(1, 8, 5, 5, 4, stride=(2, 1), pad=(1, 0), dil=(1, 2), groups=4),
    Shape(1, 4, 6, 6, 3, kh=3, kw=2, pad=(1, 0)),
]


# --- library special cases -------------------------------------------------

@pytest.mark.parametrize("s", SHAPES)
def test_zero_offsets_reproduce_plain_convolution(oracle, s):
    """W_off = 0, b_off = 0: every sample lands on the grid, so the layer is an
    ordinary convolution (torch.conv2d, fp64) and the columns are torch's
    unfold (channel-major, tap-minor per output pixel)."""
    x, w_off, b_off, w, b = rand_layer(s, 1)
    y, off, col = oracle.forward(s, x, np.zeros_like(w_off), np.zeros_like(b_off), w, b, want_cols=True)
    assert np.all(off == 0)
    assert rel(y, torch_conv(s, x, w, b)) < 1e-12
    unf = F.unfold(torch.from_numpy(x), (s.kh, s.kw), dilation=s.dil, padding=s.pad, stride=s.stride).numpy()
    # unfold: [N][Cin*K][L] -> [N][L][Cin][K]
    unf = np.transpose(unf, (0, 2, 1)).reshape(s.n, s.ho * s.wo, s.c_in, s.taps)
    assert np.array_equal(col, unf)


@pytest.mark.parametrize("s", SHAPES)
def test_offset_conv_is_plain_convolution(oracle, s):
    x, w_off, b_off, _, _ = rand_layer(s, 2)
    assert rel(oracle.offset_conv(s, x, w_off, b_off), torch_conv(s, x, w_off, b_off)) < 1e-12


# --- closed forms ------------------------------------------------------------

def shifted_conv(s, x, w, b, dys, dxs):
    """Integer offsets (dy_gk, dx_gk), identical at every output pixel: each tap
    reads x at its grid position shifted by an integer, zero outside."""
    M = 16
    xp = np.zeros((s.n, s.c_in, s.h + 2 * M, s.w + 2 * M))
    xp[:, :, M:M + s.h, M:M + s.w] = x
    cg = s.c_in // s.groups
    y = np.zeros((s.n, s.c_out, s.ho, s.wo)) + b[None, :, None, None]
    for g in range(s.groups):
        for i in range(s.kh):
            for j in range(s.kw):
                k = i * s.kw + j
                ys = np.arange(s.ho) * s.stride[0] - s.pad[0] + i * s.dil[0] + dys[g, k] + M
                xs = np.arange(s.wo) * s.stride[1] - s.pad[1] + j * s.dil[1] + dxs[g, k] + M
                patch = xp[:, g * cg:(g + 1) * cg][:, :, ys][:, :, :, xs]       # [N][Cg][Ho][Wo]
                y += np.einsum("oc,nchw->nohw", w[:, g * cg:(g + 1) * cg, i, j], patch)
    return y


@pytest.mark.parametrize("s", SHAPES)
def test_integer_offsets_reproduce_shifted_convolution(oracle, s):
    x, w_off, _, w, b = rand_layer(s, 3)
    r = np.random.default_rng(33)
    dys = r.integers(-3, 4, (s.groups, s.taps))
    dxs = r.integers(-3, 4, (s.groups, s.taps))
    b_off = np.zeros(s.oc)
    b_off[0::2] = dys.ravel()
    b_off[1::2] = dxs.ravel()
    y, _ = oracle.forward(s, x, np.zeros_like(w_off), b_off, w, b)
    assert rel(y, shifted_conv(s, x, w, b, dys, dxs)) < 1e-12


@pytest.mark.parametrize("s", SHAPES)
def test_affine_image_reproduced_exactly(oracle, s):
    """Bilinear interpolation reproduces affine functions: on
    x[c, y, x] = a_c*y + b_c*x + e_c every tap whose four corners are in the
    image yields a_c*py + b_c*px + e_c.  Pins the dy/dx order and sign and the
    fractional weights."""
    r = np.random.default_rng(4)
    a, bb, e = r.standard_normal(s.c_in), r.standard_normal(s.c_in), r.standard_normal(s.c_in)
    yy, xx = np.meshgrid(np.arange(s.h), np.arange(s.w), indexing="ij")
    img = a[:, None, None] * yy + bb[:, None, None] * xx + e[:, None, None]
    x = np.broadcast_to(img, (s.n,) + img.shape).copy()
    off = r.uniform(-1.5, 1.5, (s.n, s.oc, s.ho, s.wo))
    col = oracle.sample_cols(s, x, off)
    cg = s.c_in // s.groups
    checked = 0
    for g in range(s.groups):
        for k in range(s.taps):
            i, j = divmod(k, s.kw)
            py = (np.arange(s.ho) * s.stride[0] - s.pad[0] + i * s.dil[0])[None, :, None] + off[:, 2 * (g * s.taps + k)]
            px = (np.arange(s.wo) * s.stride[1] - s.pad[1] + j * s.dil[1])[None, None, :] + off[:, 2 * (g * s.taps + k) + 1]
            inside = (np.floor(py) >= 0) & (np.floor(py) + 1 <= s.h - 1) & (np.floor(px) >= 0) & (np.floor(px) + 1 <= s.w - 1)
            for c in range(g * cg, (g + 1) * cg):
                expect = a[c] * py + bb[c] * px + e[c]
                got = col[:, :, c, k].reshape(s.n, s.ho, s.wo)
                assert np.allclose(got[inside], expect[inside], rtol=0, atol=1e-12)
                checked += int(inside.sum())
    assert checked > 0


def test_partition_of_unity(oracle):
    """A constant image (per channel) is reproduced exactly by every tap whose
    corners are all in the image: the four weights sum to one."""
    s = Shape(2, 5, 9, 9, 2, pad=(0, 0), groups=1)
    r = np.random.default_rng(5)
    const = r.standard_normal(s.c_in)
    x = np.broadcast_to(const[None, :, None, None], (s.n, s.c_in, s.h, s.w)).copy()
    off = r.uniform(-0.99, 0.99, (s.n, s.oc, s.ho, s.wo))
    col = oracle.sample_cols(s, x, off)
    for k in range(s.taps):
        i, j = divmod(k, s.kw)
        py = np.arange(s.ho)[None, :, None] + i + off[:, 2 * k]
        px = np.arange(s.wo)[None, None, :] + j + off[:, 2 * k + 1]
        inside = (np.floor(py) >= 0) & (np.floor(py) <= s.h - 2) & (np.floor(px) >= 0) & (np.floor(px) <= s.w - 2)
        assert inside.sum() > 0
        for c in range(s.c_in):
            got = col[:, :, c, k].reshape(s.n, s.ho, s.wo)[inside]
            assert np.max(np.abs(got - const[c])) <= 4 * np.finfo(np.float64).eps * abs(const[c])


def test_fully_outside_taps_read_zero(oracle):
    """Pushing every tap beyond the image (dy = +2H) leaves only the bias; NaN
    offsets are fully outside too; pushing one tap equals a convolution with
    that tap's weights zeroed."""
    s = Shape(2, 4, 7, 7, 3, groups=2)
    x, w_off, _, w, b = rand_layer(s, 6)
    b_off = np.zeros(s.oc)
    b_off[0::2] = 2 * s.h
    y, _ = oracle.forward(s, x, np.zeros_like(w_off), b_off, w, b)
    assert np.array_equal(y, np.broadcast_to(b[None, :, None, None], y.shape))
    b_nan = np.full(s.oc, np.nan)
    y2, _ = oracle.forward(s, x, np.zeros_like(w_off), b_nan, w, b)
    assert np.array_equal(y2, np.broadcast_to(b[None, :, None, None], y.shape))
    for push in [(-1.0 - 0.0, "dy"), (float(s.w), "dx")]:
        kstar = 4
        for g in range(s.groups):
            b_off = np.zeros(s.oc)
            i, j = divmod(kstar, s.kw)
            # dy so that py <= -1 for every output row: base row >= -1, so shift by -(H+2)
            if push[1] == "dy":
                b_off[2 * (g * s.taps + kstar)] = -(s.h + 2)
            else:
                b_off[2 * (g * s.taps + kstar) + 1] = s.w + 2
            y3, _ = oracle.forward(s, x, np.zeros_like(w_off), b_off, w, b)
            wz = w.copy()
            cg = s.c_in // s.groups
            wz[:, g * cg:(g + 1) * cg, i, j] = 0
            assert rel(y3, torch_conv(s, x, wz, b)) < 1e-12


def test_offset_groups_replicated_equal_single_group(oracle):
    """G = 4 with identical per-group offset-conv rows equals G = 1."""
    s1 = Shape(2, 8, 7, 7, 3, groups=1)
    s4 = Shape(2, 8, 7, 7, 3, groups=4)
    x, w_off, b_off, w, b = rand_layer(s1, 7, off_scale=0.2)
    w_off4 = np.concatenate([w_off] * 4, axis=0)
    b_off4 = np.concatenate([b_off] * 4, axis=0)
    y1, _ = oracle.forward(s1, x, w_off, b_off, w, b)
    y4, _ = oracle.forward(s4, x, w_off4, b_off4, w, b)
    assert rel(y4, y1) < 1e-13


@pytest.mark.parametrize("s", SHAPES)
def test_c_oracle_matches_numpy_tent_formulation(oracle, s):
    x, w_off, b_off, w, b = rand_layer(s, 8)
    y, off, col = oracle.forward(s, x, w_off, b_off, w, b, want_cols=True)
    y2, off2, col2 = ref_np.forward(s, x, w_off, b_off, w, b)
    assert rel(off, off2) < 1e-13
    assert rel(col, col2) < 1e-13
    assert rel(y, y2) < 1e-13


# --- backward ------------------------------------------------------------------

def _loss(s, x, w_off, b_off, w, b, dy):
    y, _ = oracle.forward(s, x, w_off, b_off, w, b)
    return float(np.sum(y * dy))


def _kink_distance(s, x, w_off, b_off):
    """Distance of the nearest sample coordinate to an integer line (where the
    bilinear value has a kink)."""
    off = oracle.offset_conv(s, x, w_off, b_off)
    d = np.inf
    for k in range(s.taps):
        i, j = divmod(k, s.kw)
        for g in range(s.groups):
            py = (np.arange(s.ho) * s.stride[0] - s.pad[0] + i * s.dil[0])[None, :, None] + off[:, 2 * (g * s.taps + k)]
            px = (np.arange(s.wo) * s.stride[1] - s.pad[1] + j * s.dil[1])[None, None, :] + off[:, 2 * (g * s.taps + k) + 1]
            for p in (py, px):
                d = min(d, float(np.min(np.abs(p - np.round(p)))))
    return d


FD_SHAPES = [
    Shape(2, 4, 6, 6, 3),
    Shape(1, 4, 7, 5, 3, stride=(2, 2), pad=(0, 1)),
    Shape(2, 4, 6, 6, 2, dil=(2, 2), pad=(2, 1), groups=2),
    Shape(1, 4, 5, 7, 3, stride=(1, 2), groups=2),
    # non-square and larger kernels (the shapes the GPU edge tests use)
    Shape(1, 4, 6, 5, 2, kh=3, kw=2, pad=(1, 1)),
    Shape(1, 4, 7, 7, 2, kh=5, kw=5, pad=(2, 2)),
]


@pytest.mark.parametrize("s", FD_SHAPES)
def test_gradients_match_central_differences(oracle, s):
    """Directional central differences (h = 1e-7, fp64) of L = <dY, y> along
    random directions agree with the analytic gradient for every input, plus
    single-coordinate checks.  Seeds with a sample coordinate within 1e-5 of an
    integer line (a kink of the bilinear interpolation) are skipped."""
    for seed in range(100, 200):
        x, w_off, b_off, w, b = rand_layer(s, seed, off_scale=0.3)
        if _kink_distance(s, x, w_off, b_off) > 1e-5:
            break
    else:
        pytest.fail("no kink-free seed")
    r = np.random.default_rng(seed + 1000)
    dy = r.standard_normal((s.n, s.c_out, s.ho, s.wo))
    _, off = oracle.forward(s, x, w_off, b_off, w, b)
    g = oracle.backward(s, x, w_off, w, off, dy)
    assert np.allclose(g["db"], dy.sum(axis=(0, 2, 3)), rtol=1e-12, atol=1e-12)
    params = dict(x=x, w_off=w_off, b_off=b_off, w=w, b=b)
    names = dict(x="dx", w_off="dw_off", b_off="db_off", w="dw", b="db")
    h = 1e-7
    for pname, val in params.items():
        grad = g[names[pname]]
        for trial in range(3):
            v = r.standard_normal(val.shape)
            pp = dict(params)
            pp[pname] = val + h * v
            lp = _loss(s, dy=dy, **pp)
            pp[pname] = val - h * v
            lm = _loss(s, dy=dy, **pp)
            fd = (lp - lm) / (2 * h)
            an = float(np.sum(grad * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (pname, fd, an)
        flat = val.ravel()
        for idx in r.choice(flat.size, size=min(4, flat.size), replace=False):
            pp = dict(params)
            e = np.zeros(flat.size)
            e[idx] = 1.0
            e = e.reshape(val.shape)
            pp[pname] = val + h * e
            lp = _loss(s, dy=dy, **pp)
            pp[pname] = val - h * e
            lm = _loss(s, dy=dy, **pp)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad.ravel()[idx]) <= 1e-6 * max(1.0, abs(fd)), (pname, idx)


@pytest.mark.parametrize("s", SHAPES[:4])
def test_sampling_adjoint(oracle, s):
    """With the offset convolution's weights zero the layer is linear in x for
    fixed (fractional) offsets: <dY, y(v) - b> = <dx(dY), v> exactly (the
    scatter of the backward is the adjoint of the gather)."""
    x, w_off, b_off, w, b = rand_layer(s, 9)
    r = np.random.default_rng(99)
    b_off = r.uniform(-2.5, 2.5, s.oc)
    v = r.standard_normal(x.shape)
    dy = r.standard_normal((s.n, s.c_out, s.ho, s.wo))
    z = np.zeros_like(w_off)
    yv, off = oracle.forward(s, v, z, b_off, w, b)
    g = oracle.backward(s, x, z, w, off, dy)
    lhs = float(np.sum(dy * (yv - b[None, :, None, None])))
    rhs = float(np.sum(g["dx"] * v))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))


def test_grad_offsets_on_affine_image(oracle):
    """On x[c,y,x] = a_c*y + b_c*x + e_c, with one output channel, W[0,c,k] =
    w_ck and dY = 1, the offset gradient of every interior tap is
    ddy = sum_{c in group} w_ck*a_c and ddx = sum_{c in group} w_ck*b_c."""
    s = Shape(1, 6, 9, 9, 1, pad=(0, 0), groups=2)
    r = np.random.default_rng(10)
    a, bb, e = r.standard_normal(s.c_in), r.standard_normal(s.c_in), r.standard_normal(s.c_in)
    yy, xx = np.meshgrid(np.arange(s.h), np.arange(s.w), indexing="ij")
    x = (a[:, None, None] * yy + bb[:, None, None] * xx + e[:, None, None])[None]
    w = r.standard_normal((1, s.c_in, s.kh, s.kw))
    off = r.uniform(-0.9, 0.9, (s.n, s.oc, s.ho, s.wo))
    off[np.abs(off - np.round(off)) < 1e-3] += 0.01
    dy = np.ones((1, 1, s.ho, s.wo))
    g = oracle.backward(s, x, np.zeros((s.oc, s.c_in, s.kh, s.kw)), w, off, dy)
    cg = s.c_in // s.groups
    for gi in range(s.groups):
        for k in range(s.taps):
            i, j = divmod(k, s.kw)
            py = np.arange(s.ho)[:, None] + i + off[0, 2 * (gi * s.taps + k)]
            px = np.arange(s.wo)[None, :] + j + off[0, 2 * (gi * s.taps + k) + 1]
            inside = (np.floor(py) >= 0) & (np.floor(py) <= s.h - 2) & (np.floor(px) >= 0) & (np.floor(px) <= s.w - 2)
            wk = w[0, gi * cg:(gi + 1) * cg, i, j]
            ey = float(np.sum(wk * a[gi * cg:(gi + 1) * cg]))
            ex = float(np.sum(wk * bb[gi * cg:(gi + 1) * cg]))
            assert np.allclose(g["doff"][0, 2 * (gi * s.taps + k)][inside], ey, atol=1e-12)
            assert np.allclose(g["doff"][0, 2 * (gi * s.taps + k) + 1][inside], ex, atol=1e-12)


def test_grad_offsets_cell_chosen_on_fp32_coordinate(oracle):
    """The offset gradient is one-sided at a cell edge, so it depends on which
    cell the sample point is put in; that choice is made on the fp32
    coordinate (the index stage's rule).  On x[y,x] = y^2 + 10 x^2 with one
    1x1 tap, W = 1 and dY = 1, a point in cell (y0, x0) has ddy = 2*y0 + 1
    and ddx = 10*(2*x0 + 1).  dy = 1 - 2^-24 on base row 2 sums to 3.0 in
    fp32 (cell row 3: 7, where an fp64 floor would give row 2: 5); on base row
    0 the fp32 sum stays below 1 (cell row 0: 1).  The value itself is
    continuous across the edge."""
    s = Shape(1, 1, 6, 6, 1, kh=1, kw=1, pad=(0, 0))
    yy, xx = np.meshgrid(np.arange(6.0), np.arange(6.0), indexing="ij")
    x = (yy ** 2 + 10 * xx ** 2)[None, None]
    e = float(np.float32(1.0 - 2.0 ** -24))
    off = np.zeros((1, 2, 6, 6))
    off[0, 0, 2, 1] = e      # row 2 + e -> 3.0 in fp32
    off[0, 0, 0, 0] = e      # row 0 + e stays in cell 0
    off[0, 1, 1, 2] = e      # column 2 + e -> 3.0 in fp32
    g = oracle.backward(s, x, np.zeros((2, 1, 1, 1)), np.ones((1, 1, 1, 1)), off, np.ones((1, 1, 6, 6)))
    cases = {(2, 1): (3, 1), (0, 0): (0, 0), (1, 2): (1, 3), (4, 4): (4, 4)}
    for (ho, wo), (y0, x0) in cases.items():
        assert g["doff"][0, 0, ho, wo] == 2 * y0 + 1, (ho, wo)
        assert g["doff"][0, 1, ho, wo] == 10 * (2 * x0 + 1), (ho, wo)
    iy, ix, _ = oracle.sample_index_f32(s, off.astype(np.float32))
    for (ho, wo), (y0, x0) in cases.items():
        assert (iy[0, 0, 0, ho, wo], ix[0, 0, 0, ho, wo]) == (y0, x0)
    # bilinear interpolation of y^2 between rows 2 and 3 is 4 + 5*e
    col = oracle.sample_cols(s, x, off)
    assert abs(col[0, 2 * 6 + 1, 0, 0] - (4 + 5 * e + 10)) < 1e-6
    assert abs(col[0, 1 * 6 + 2, 0, 0] - (1 + 10 * (4 + 5 * e))) < 1e-5


# --- the fp32 index stage ---------------------------------------------------------

def test_index_stage_hand_cases(oracle):
    """Hand-derived cases of the fp32 tap index / corner mask (bit 0 = (y0,x0),
    1 = (y0,x0+1), 2 = (y0+1,x0), 3 = (y0+1,x0+1); fully outside -> 0,0,0)."""
    s = Shape(1, 8, 4, 4, 8, kh=1, kw=1, pad=(0, 0))     # one tap, base = (ho, wo)
    off = np.zeros((1, 2, 4, 4), np.float32)
    cases = {
        (0, 0): ((0.0, 0.0), (0, 0, 0b1111)),            # on the grid
        (0, 1): ((-0.5, 0.25), (-1, 1, 0b1100)),         # above row 0: top corners out
        (0, 2): ((-1.0, 0.0), (0, 0, 0)),                # py = -1 exactly: fully outside
        (3, 3): ((0.5, 0.5), (3, 3, 0b0001)),            # bottom-right: only (y0,x0) in
        (1, 3): ((0.0, 1.0), (0, 0, 0)),                 # px = 4 = W: fully outside
        (2, 0): ((np.nan, 0.0), (0, 0, 0)),              # NaN: fully outside
        (2, 1): ((-1e-8, 0.0), (2, 1, 0b1111)),          # 2 + (-1e-8) rounds to 2.0 in fp32
        (1, 1): ((-1.75, -1.75), (-1, -1, 0b1000)),      # only corner (0,0) is in the image
        (1, 2): ((0.0, -2.5), (1, -1, 0b1010)),          # px = -0.5: x0 = -1, left corners out
    }
    for (ho, wo), ((dy, dx), _) in cases.items():
        off[0, 0, ho, wo] = dy
        off[0, 1, ho, wo] = dx
    y0, x0, m = oracle.sample_index_f32(s, off)
    for (ho, wo), ((dy, dx), (ey, ex, em)) in cases.items():
        got = (int(y0[0, 0, 0, ho, wo]), int(x0[0, 0, 0, ho, wo]), int(m[0, 0, 0, ho, wo]))
        assert got == (ey, ex, em), ((ho, wo), got, (ey, ex, em))


def test_index_stage_matches_fp64_floor_away_from_rounding(oracle):
    """Where the fp32 add cannot change the floor (offsets on a 1/1024 grid,
    exactly representable), the index stage equals floor of the exact sample
    point and the mask equals the in-image test of each corner."""
    s = Shape(2, 8, 6, 7, 4, stride=(2, 1), pad=(1, 2), dil=(1, 2), groups=2)
    r = np.random.default_rng(11)
    off = (r.integers(-3000, 3000, (s.n, s.oc, s.ho, s.wo)) / 1024.0).astype(np.float32)
    y0, x0, m = oracle.sample_index_f32(s, off)
    for g in range(s.groups):
        for k in range(s.taps):
            i, j = divmod(k, s.kw)
            py = (np.arange(s.ho) * 2 - 1 + i)[None, :, None] + off[:, 2 * (g * s.taps + k)].astype(np.float64)
            px = (np.arange(s.wo) * 1 - 2 + 2 * j)[None, None, :] + off[:, 2 * (g * s.taps + k) + 1].astype(np.float64)
            out = ~((py > -1) & (py < s.h) & (px > -1) & (px < s.w))
            fy, fx = np.floor(py).astype(int), np.floor(px).astype(int)
            em = (((fy >= 0) & (fx >= 0)) * 1 + ((fy >= 0) & (fx + 1 < s.w)) * 2 +
                  ((fy + 1 < s.h) & (fx >= 0)) * 4 + ((fy + 1 < s.h) & (fx + 1 < s.w)) * 8)
            ey = np.where(out, 0, fy)
            ex = np.where(out, 0, fx)
            em = np.where(out, 0, em)
            assert np.array_equal(y0[:, g, k], ey)
            assert np.array_equal(x0[:, g, k], ex)
            assert np.array_equal(m[:, g, k], em)


# --- dilated depthwise 1-D convolution (JAX issue page workload) ---------------

from oracle import dwconv as dw  # noqa: E402


@pytest.mark.parametrize("K,C,d", [(1, 4, 1), (4, 8, 1), (4, 8, 3), (16, 5, 8), (3, 6, 64)])
def test_dwconv1d_equals_grouped_conv(K, C, d):
    """Library special case: torch's grouped conv1d with groups = channels and
    the same dilation, in fp64, on the NCT layout."""
    r = np.random.default_rng(K * 100 + C * 10 + d)
    T = 37
    x = r.standard_normal((2, T + d * (K - 1), C))
    w = r.standard_normal((K, C))
    y = dw.dwconv1d(x, w, d)
    ref = F.conv1d(torch.from_numpy(x).permute(0, 2, 1), torch.from_numpy(w.T.copy()).unsqueeze(1),
                   dilation=d, groups=C).permute(0, 2, 1).numpy()
    assert y.shape == (2, T, C)
    assert rel(y, ref) <= 1e-13


def test_dwconv1d_closed_forms():
    """K = 1 scales the input; a one-hot kernel at tap k0 shifts it by k0*d;
    channels never mix."""
    r = np.random.default_rng(7)
    x = r.standard_normal((3, 50, 4))
    w1 = r.standard_normal((1, 4))
    assert np.array_equal(dw.dwconv1d(x, w1, 5), x * w1[0])
    K, d, k0 = 5, 3, 2
    T = 50 - d * (K - 1)
    w = np.zeros((K, 4))
    w[k0] = 1.0
    assert np.array_equal(dw.dwconv1d(x, w, d), x[:, k0 * d:k0 * d + T, :])
    x2 = x.copy()
    x2[:, :, 1] += 100.0  # perturbing channel 1 leaves the other channels unchanged
    wf = r.standard_normal((K, 4))
    a, b = dw.dwconv1d(x, wf, d), dw.dwconv1d(x2, wf, d)
    assert np.array_equal(a[:, :, [0, 2, 3]], b[:, :, [0, 2, 3]])


def test_dwconv1d_phase_decomposition():
    """Outputs whose step has residue r modulo d read only inputs with residue
    r: the dilated conv equals d undilated convs on the phase subsequences."""
    r = np.random.default_rng(11)
    K, d, C = 4, 5, 3
    T = 23
    x = r.standard_normal((2, T + d * (K - 1), C))
    w = r.standard_normal((K, C))
    y = dw.dwconv1d(x, w, d)
    for ph in range(d):
        sub = dw.dwconv1d(x[:, ph::d, :], w, 1)
        n = len(range(ph, T, d))
        assert np.allclose(y[:, ph::d, :], sub[:, :n, :], rtol=0, atol=1e-12)


def test_dwpw1d_equals_grouped_then_pointwise_conv():
    """Library composition: torch's grouped conv1d (groups = channels) followed
    by a 1x1 conv1d, in fp64; an identity pointwise kernel leaves the
    depthwise result; a pointwise kernel that selects one channel picks it."""
    r = np.random.default_rng(21)
    B, T, C, O, K, d = 2, 29, 8, 12, 3, 4
    x = r.standard_normal((B, T + d * (K - 1), C))
    wd = r.standard_normal((K, C))
    wp = r.standard_normal((C, O))
    z = dw.dwpw1d(x, wd, wp, d)
    xt = torch.from_numpy(x).permute(0, 2, 1)
    y = F.conv1d(xt, torch.from_numpy(wd.T.copy()).unsqueeze(1), dilation=d, groups=C)
    ref = F.conv1d(y, torch.from_numpy(wp.T.copy()).unsqueeze(2)).permute(0, 2, 1).numpy()
    assert z.shape == (B, T, O)
    assert rel(z, ref) <= 1e-13
    assert np.allclose(dw.dwpw1d(x, wd, np.eye(C), d), dw.dwconv1d(x, wd, d), rtol=0, atol=1e-12)
    sel = np.zeros((C, 1))
    sel[5, 0] = 1.0
    assert np.allclose(dw.dwpw1d(x, wd, sel, d)[:, :, 0], dw.dwconv1d(x, wd, d)[:, :, 5], rtol=0, atol=1e-12)
