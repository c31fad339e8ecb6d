"""C-ABI checks that need no GPU: the library loads, exports every function
include/deft.h declares, and every validation error is returned before any
launch (so fake, never-dereferenced pointers are safe here)."""
import ctypes
import os
import re

import pytest

from irregular_gather_cnn_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    txt = open(os.path.join(ROOT, "include", "deft.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(deft_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = L.load()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTED) == names


def desc(**kw):
    base = dict(n=2, c_in=32, h=9, w=11, c_out=8, kh=3, kw=3, stride=(1, 1), pad=(1, 1), dil=(1, 1), groups=1,
                dtype=L.DEFT_BF16)
    base.update(kw)
    return L.make_desc(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(), 0),
    (dict(dtype=7), -6),
    (dict(c_in=0), -1),
    (dict(h=0), -1),
    (dict(stride=(0, 1)), -1),
    (dict(dil=(1, 0)), -1),
    (dict(pad=(-1, 0)), -1),
    (dict(kh=0), -1),
    (dict(groups=0), -2),
    (dict(groups=3), -2),
    (dict(h=2, pad=(0, 0)), -3),
    (dict(c_in=24), -10),
    (dict(c_in=32, groups=4), -10),
    (dict(n=0), 0),
])
def test_descriptor_validation(kw, code):
    assert L.deft_desc_validate(desc(**kw)) == code


def test_plan_and_workspace_sizes():
    d = desc()
    p = L.deft_plan_create(d)
    info = L.deft_plan_get_info(p)
    assert info["ho"] == 9 and info["wo"] == 11 and info["oc"] == 18
    assert info["halo"] == 2 and info["bwd_halo"] == 4  # defaults without a histogram
    cols = 2 * 9 * 11 * 9 * 32 * 2
    assert info["ws_forward"] >= cols and info["ws_training"] >= info["ws_forward"] + cols
    assert L.deft_workspace_bytes(p, 0) == info["ws_forward"]
    assert L.deft_workspace_bytes(p, 1) == info["ws_training"]
    assert info["ws_cols_offset"] % 256 == 0 and info["ws_cols_offset"] + cols <= info["ws_forward"]
    L.deft_plan_destroy(p)


def test_planner_sizes_halo_from_histogram():
    d = desc(n=16, c_in=256, h=56, w=56, c_out=256)
    tight = [900, 90, 9, 1, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0]
    wide = [100, 100, 100, 100, 100, 100, 100, 100, 100, 100, 100, 100, 100, 100, 100, 0]
    pt = L.deft_plan_get_info(L.deft_plan_create(d, tight))
    pw = L.deft_plan_get_info(L.deft_plan_create(d, wide))
    assert pt["halo"] <= 3
    assert pw["halo"] > pt["halo"]
    # backward: the smallest halo leaving no tap outside but the open-ended bin
    assert pt["bwd_halo"] == 3 and pt["est_miss_fraction"] == 0.0
    assert pw["bwd_halo"] == 13 and abs(pw["est_miss_fraction"] - 100 / 1500) < 1e-12
    # 1e-5 of the taps may stay outside
    assert L.deft_plan_get_info(L.deft_plan_create(d, [10 ** 6, 5, 0, 0, 0, 0, 0, 0]))["bwd_halo"] == 0
    assert L.deft_plan_get_info(L.deft_plan_create(d, [10 ** 6, 20, 0, 0, 0, 0, 0, 0]))["bwd_halo"] == 1
    # degenerate histograms: every tap fully outside, or every tap in the open-ended bin (no halo helps)
    assert L.deft_plan_get_info(L.deft_plan_create(d, [0, 0, 0, 0, 0, 0, 0, 50]))["bwd_halo"] == 0
    assert L.deft_plan_get_info(L.deft_plan_create(d, [0, 0, 0, 0, 0, 0, 50, 0]))["bwd_halo"] == 0
    # a tail reaching the open-ended bin: the last bin a halo can take in
    assert L.deft_plan_get_info(L.deft_plan_create(d, [10, 10, 10, 10, 10, 10, 10, 0]))["bwd_halo"] == 5
    # a histogram that counted no tap at all (e.g. a forward whose launch emitted none) carries no
    # information: the same plan as without a histogram
    none = L.deft_plan_get_info(L.deft_plan_create(d))
    empty = L.deft_plan_get_info(L.deft_plan_create(d, [0] * 16))
    assert empty["bwd_halo"] == none["bwd_halo"] == 4
    assert empty["est_miss_fraction"] == none["est_miss_fraction"]
    assert (empty["tile_h"], empty["tile_w"], empty["halo"]) == (none["tile_h"], none["tile_w"], none["halo"])


@pytest.mark.fake_pointers
@pytest.mark.parametrize("kw,dtype", [(dict(w=320), L.DEFT_F32), (dict(w=400, dil=(4, 4), pad=(4, 4)), L.DEFT_BF16)])
def test_wide_image_plan_without_backward(kw, dtype):
    """Images so wide that not even a one-row band of the offset-weight
    backward's staged input fits the LDS: the plan is made (the forward runs)
    but has no backward, and deft_backward refuses it before any launch."""
    d = desc(n=1, c_in=32, h=4, c_out=16, dtype=dtype, **kw)
    p = L.deft_plan_create(d)
    info = L.deft_plan_get_info(p)
    assert info["bwd_chunk"] == 0 and info["ws_forward"] > 0
    big = 1 << 40
    with pytest.raises(L.DeftError) as e:
        # pointers are never dereferenced: validation refuses the plan first
        L.deft_backward(p, 16, 16, 16, 16, 16, 16, big, 16, 16, None, 16, None)
    assert e.value.code == -9
    L.deft_plan_destroy(p)
    # a slightly narrower image keeps its backward
    d2 = desc(n=1, c_in=32, h=4, c_out=16, dtype=dtype, **dict(kw, w=kw["w"] // 2))
    assert L.deft_plan_get_info(L.deft_plan_create(d2))["bwd_chunk"] > 0


def test_forward_halo_avoids_single_workgroup_occupancy():
    """fp32 64 x 64 with offsets of about a pixel: halo 4 needs more than
    80 KB of LDS (one workgroup per CU, measured 1.8x slower than halo 2 at
    two per CU), so the forward takes a smaller halo while the backward's
    halo still covers every tap."""
    d = desc(n=8, c_in=128, h=64, w=64, c_out=128, dtype=L.DEFT_F32)
    hist = [33919, 161534, 80818, 12822, 729, 15, 0, 0, 0, 0, 0, 0, 0, 0, 0, 5075]
    info = L.deft_plan_get_info(L.deft_plan_create(d, hist))
    assert info["lds_bytes"] <= 80 * 1024 and info["halo"] >= 1
    assert info["bwd_halo"] == 5


def test_forced_plan_limits():
    d = desc()
    with pytest.raises(L.DeftError) as e:
        L.deft_plan_create_forced(d, 16, 8, 2, 0)
    assert e.value.code == -9
    with pytest.raises(L.DeftError):
        L.deft_plan_create_forced(d, 8, 8, 2, 48)
    p = L.deft_plan_create_forced(d, 8, 8, 0, 16)
    info = L.deft_plan_get_info(p)
    assert (info["tile_h"], info["tile_w"], info["halo"], info["chunk"]) == (8, 8, 0, 16)


def test_direct_gather_selection():
    """The planner takes the direct-gather forward exactly where it applies:
    at most 9 taps, a power-of-two number of 16-byte channel slices per
    offset group (8 bf16 or 4 fp32 channels); the forced plan's chunk -1 asks
    for it and is refused elsewhere.  The direct variant's workspace holds
    the channel-minor copy of x (one extra zero pixel per image)."""
    def info(**kw):
        return L.deft_plan_get_info(L.deft_plan_create(desc(**kw)))
    assert info(n=2, c_in=32, dtype=L.DEFT_BF16)["gather_direct"] == 1
    assert info(n=2, c_in=32, dtype=L.DEFT_F32)["gather_direct"] == 1  # 8 slices of 4 channels
    assert info(n=2, c_in=32, kh=5, kw=5, pad=(2, 2), dtype=L.DEFT_BF16)["gather_direct"] == 0
    assert info(n=2, c_in=48, dtype=L.DEFT_BF16)["gather_direct"] == 0  # 6 slices of 8 channels
    assert info(n=2, c_in=48, dtype=L.DEFT_F32)["gather_direct"] == 0  # 12 slices of 4 channels
    assert info(n=2, c_in=64, groups=4, dtype=L.DEFT_BF16)["gather_direct"] == 1  # 2 slices per group
    dd = desc(n=2, c_in=32, dtype=L.DEFT_BF16)
    halo_plan = L.deft_plan_get_info(L.deft_plan_create_forced(dd, 8, 8, 2, 32))
    direct_plan = L.deft_plan_get_info(L.deft_plan_create_forced(dd, 8, 8, 2, -1))
    assert halo_plan["gather_direct"] == 0 and direct_plan["gather_direct"] == 1
    copy_bytes = 2 * (9 * 11 + 1) * 32 * 2
    assert direct_plan["ws_forward"] >= halo_plan["ws_forward"] + copy_bytes - 256
    for bad in (desc(n=2, c_in=48, dtype=L.DEFT_F32), desc(n=2, c_in=48, dtype=L.DEFT_BF16)):
        with pytest.raises(L.DeftError) as e:
            L.deft_plan_create_forced(bad, 8, 8, 2, -1)
        assert e.value.code == -9


def test_planner_direct_tile_avoids_ragged_edges():
    """The direct-gather tile is costed with the empty pixel slots of ragged
    edge tiles: on 56 x 56 and 28 x 28 outputs it picks a tile that divides the
    output (7 x 7), not 4 x 16 (whose last tile column would be half empty)."""
    for kw in (dict(n=16, c_in=256, c_out=256, h=56, w=56),
               dict(n=16, c_in=512, c_out=512, h=28, w=28, groups=4)):
        i = L.deft_plan_get_info(L.deft_plan_create(desc(**kw)))
        assert i["gather_direct"] == 1
        assert (i["tile_h"], i["tile_w"]) == (7, 7)
        assert i["ho"] % i["tile_h"] == 0 and i["wo"] % i["tile_w"] == 0


@pytest.mark.parametrize("h,w,stride,dil,groups", [
    (5, 5, 1, 1, 1), (9, 11, 1, 1, 2), (13, 70, 1, 2, 1), (56, 56, 2, 1, 1), (31, 17, 2, 1, 4), (64, 64, 1, 1, 1),
])
def test_planner_tiles_are_valid(h, w, stride, dil, groups):
    """Every automatic plan has a tile of at most 64 pixels, at least one
    workgroup and a workspace; the direct gather covers the output."""
    d = desc(n=2, c_in=64, c_out=24, h=h, w=w, stride=(stride, stride), pad=(dil, dil), dil=(dil, dil),
             groups=groups)
    i = L.deft_plan_get_info(L.deft_plan_create(d))
    assert 1 <= i["tile_h"] * i["tile_w"] <= 64
    assert i["num_workgroups"] >= 1 and i["ws_forward"] > 0
    tiles = -(-i["ho"] // i["tile_h"]) * -(-i["wo"] // i["tile_w"])
    if i["gather_direct"]:
        assert i["num_workgroups"] == 2 * groups * tiles


def test_forced_gather_gemm_plan():
    """chunk -2 selects the forward that gathers straight into the main GEMM;
    it needs bf16, the direct gather, 32-channel slices and 8-pixel runs."""
    ok = L.deft_plan_get_info(L.deft_plan_create_forced(desc(n=2, c_in=64, c_out=40, h=10, w=12), 7, 7, 2, -2))
    assert ok["gather_gemm"] == 1 and ok["gather_direct"] == 1
    plain = L.deft_plan_get_info(L.deft_plan_create_forced(desc(n=2, c_in=64, c_out=40, h=10, w=12), 7, 7, 2, -1))
    assert plain["gather_gemm"] == 0
    assert ok["ws_forward"] > plain["ws_forward"] - 1  # room for the offsets when the caller keeps none
    for bad in (desc(n=2, c_in=64, dtype=L.DEFT_F32), desc(n=2, c_in=16, c_out=8), desc(n=2, c_in=64, h=9, w=11)):
        with pytest.raises(L.DeftError) as e:
            L.deft_plan_create_forced(bad, 7, 7, 2, -2)
        assert e.value.code == -9


FAKE = 1 << 40  # 16-byte aligned, never dereferenced (validation fails first)


@pytest.mark.fake_pointers
def test_forward_validation_before_launch():
    d = desc()
    p = L.deft_plan_create(d)
    ws = L.deft_workspace_bytes(p, 0)
    lib = L.load()
    ok = [p, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, ws, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return lib.deft_forward(*a)

    assert call(1, None) == -4   # x
    assert call(2, None) == -4   # w_off
    assert call(4, None) == -4   # w
    assert call(6, None) == -4   # y
    assert call(8, None) == -5   # workspace
    assert call(9, ws - 1) == -5  # too small
    assert call(1, FAKE + 8) == -7  # misaligned x
    assert call(7, FAKE + 4) == -7  # misaligned offsets_out
    assert call(3, FAKE + 1) == -7  # bias not element aligned
    assert lib.deft_forward(None, *ok[1:]) == -4


@pytest.mark.fake_pointers
def test_forward_hist_validation_before_launch():
    d = desc()
    p = L.deft_plan_create(d)
    ws = L.deft_workspace_bytes(p, 0)
    lib = L.load()
    ok = [p, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, ws, FAKE, 16, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return lib.deft_forward_hist(*a)

    assert call(11, 2) == -1      # too few bins
    assert call(11, 65) == -1     # more bins than lanes
    assert call(10, None) == -4   # histogram buffer
    assert call(10, FAKE + 2) == -7
    assert call(1, None) == -4    # then the forward's own checks
    assert call(8, None) == -5
    assert lib.deft_forward_hist(None, *ok[1:]) == -4


@pytest.mark.fake_pointers
def test_unfused_forward_validation_before_launch():
    d = desc()
    p = L.deft_plan_create(d)
    ws = L.deft_workspace_bytes(p, 0)
    lib = L.load()
    ok = [p, FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE, ws, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return lib.deft_forward_unfused(*a)

    assert call(7, None) == -4   # the offsets buffer is required here
    assert call(1, None) == -4
    assert call(6, None) == -4
    assert call(8, None) == -5
    assert call(9, ws - 1) == -5
    assert call(7, FAKE + 4) == -7
    assert lib.deft_forward_unfused(None, *ok[1:]) == -4
    e = L.deft_plan_create(desc(n=0))
    assert lib.deft_forward_unfused(e, None, None, None, None, None, None, None, None, 0, None) == 0


@pytest.mark.fake_pointers
def test_empty_batch_is_a_no_op():
    d = desc(n=0)
    p = L.deft_plan_create(d)
    lib = L.load()
    assert lib.deft_forward(p, None, None, None, None, None, None, None, None, 0, None) == 0
    assert lib.deft_backward(p, *([None] * 6), 0, *([None] * 6)) == 0
    assert lib.deft_debug_sample(p, None, None, None, None) == 0


@pytest.mark.fake_pointers
def test_backward_validation_before_launch():
    d = desc()
    p = L.deft_plan_create(d)
    ws = L.deft_workspace_bytes(p, 1)
    lib = L.load()
    ok = [p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, FAKE, FAKE, None, FAKE, None, None]
    for i in (1, 2, 3, 4, 5, 8, 9, 11):
        a = list(ok)
        a[i] = None
        assert lib.deft_backward(*a) == -4, i
    a = list(ok)
    a[7] = L.deft_workspace_bytes(p, 0)
    assert lib.deft_backward(*a) == -5
    a = list(ok)
    a[8] = FAKE + 2
    assert lib.deft_backward(*a) == -7


@pytest.mark.fake_pointers
def test_other_entry_points_validate():
    lib = L.load()
    d = desc()
    assert lib.deft_debug_sample_index(ctypes.byref(d), None, FAKE, FAKE, FAKE, None) == -4
    assert lib.deft_halo_histogram(ctypes.byref(d), FAKE, FAKE, 2, None) == -1
    assert lib.deft_halo_histogram(ctypes.byref(d), FAKE, None, 16, None) == -4
    bad = desc(groups=3)
    assert lib.deft_debug_sample_index(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == -2
    p = L.deft_plan_create(d)
    assert lib.deft_debug_sample(p, FAKE, FAKE, None, None) == -4


@pytest.mark.fake_pointers
def test_dwconv1d_validation_before_launch():
    lib = L.load()
    ok = [FAKE, FAKE, FAKE, 2, 16, 8, 3, 2, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return lib.deft_dwconv1d_forward(*a)

    assert call(5, 6) == -1        # channels not a multiple of 4
    assert call(5, 0) == -1
    assert call(6, 0) == -1        # ksize
    assert call(6, 257) == -1
    assert call(7, 0) == -1        # dilation
    assert call(3, -1) == -1       # batch
    assert call(7, 1 << 30) == -1  # input longer than 2^31 - 1 steps
    assert call(0, None) == -4
    assert call(2, None) == -4
    assert call(1, FAKE + 4) == -7
    assert call(3, 0) == 0 and call(4, 0) == 0  # empty: nothing launched


@pytest.mark.fake_pointers
def test_dwpw1d_validation_before_launch():
    lib = L.load()
    ok = [FAKE, FAKE, FAKE, FAKE, 2, 16, 64, 32, 3, 2, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return lib.deft_dwpw1d_forward(*a)

    assert call(6, 48) == -1   # channels not a multiple of 32
    assert call(7, 40) == -1   # out_channels
    assert call(8, 0) == -1
    assert call(9, 0) == -1
    assert call(2, None) == -4
    assert call(3, FAKE + 8) == -7
    assert call(4, 0) == 0


def test_error_strings():
    for code in range(-10, 1):
        s = L.deft_error_string(code)
        assert s and s != "unknown error"
    assert L.deft_error_string(-99) == "unknown error"
    assert L.deft_last_hip_error() == ""
