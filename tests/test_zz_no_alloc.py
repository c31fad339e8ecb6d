"""deft_forward_noalloc (the forward whose scratch is a static device array of
the library) against deft_forward with a caller workspace, through the C ABI:
two calls in a row on one GPU, the second with a smaller input, so the second
runs on the scratch contents the first left behind.  Same plan, same kernels:
y and the offsets must be bit-identical.  A plan whose forward scratch exceeds
the static buffer is refused before anything is launched."""
import numpy as np
import pytest
import torch

from irregular_gather_cnn_amd import _lib as L
from irregular_gather_cnn_amd.synth import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def tensors(wl):
    inp = make_inputs(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    return {k: torch.from_numpy(v).to(dt).cuda() for k, v in inp.items()}


def run_pair(wl):
    desc = L.make_desc(wl.n, wl.c_in, wl.h, wl.w, wl.c_out, wl.kh, wl.kw, (wl.stride,) * 2, (wl.pad,) * 2,
                       (wl.dil,) * 2, wl.groups, L.DEFT_BF16 if wl.dtype == "bf16" else L.DEFT_F32)
    plan = L.deft_plan_create(desc)
    try:
        need = L.deft_workspace_bytes(plan, 0)
        assert need <= L.NOALLOC_SCRATCH_BYTES, (wl.name, need)
        t = tensors(wl)
        dt = t["x"].dtype
        shp_y = (wl.n, wl.c_out, wl.ho, wl.wo)
        shp_o = (wl.n, wl.oc, wl.ho, wl.wo)
        stream = torch.cuda.current_stream().cuda_stream
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        y_ref = torch.empty(shp_y, dtype=dt, device="cuda")
        o_ref = torch.empty(shp_o, dtype=torch.float32, device="cuda")
        L.deft_forward(plan, t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y_ref, o_ref, ws, need, stream)
        y = torch.full(shp_y, float("nan"), dtype=dt, device="cuda")
        o = torch.full(shp_o, float("nan"), dtype=torch.float32, device="cuda")
        L.deft_forward_noalloc(plan, t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y, o, stream)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16) if dt == torch.bfloat16 else y.view(torch.int32),
                           y_ref.view(torch.int16) if dt == torch.bfloat16 else y_ref.view(torch.int32)), wl.name
        assert torch.equal(o.view(torch.int32), o_ref.view(torch.int32)), wl.name
        assert bool(torch.isfinite(y.float()).all())
        # without offsets_out as well
        y2 = torch.full(shp_y, float("nan"), dtype=dt, device="cuda")
        L.deft_forward_noalloc(plan, t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y2, None, stream)
        torch.cuda.synchronize()
        assert torch.equal(y2.float(), y_ref.float()), wl.name
    finally:
        L.deft_plan_destroy(plan)


def test_noalloc_forward_equals_workspace_forward_two_calls():
    big = WORKLOADS["bf16_n16_c256_56x56"].scaled(n=3)
    small = WORKLOADS["tiny_fp32_n1_c16_16x16"].scaled(dtype="bf16", c_in=32, c_out=24, h=13, w=11)
    for wl in (big, small):
        say("noalloc forward vs workspace forward:", wl.name, "n=%d c=%d %dx%d" % (wl.n, wl.c_in, wl.h, wl.w))
        run_pair(wl)


def test_noalloc_forward_fp32_after_bf16():
    wl = WORKLOADS["tiny_fp32_n1_c16_16x16"].scaled(n=2)
    say("noalloc forward vs workspace forward:", wl.name, "fp32 n=2")
    run_pair(wl)


def test_noalloc_refuses_oversize_plan_before_launch():
    wl = WORKLOADS["bf16_n16_c256_56x56"]
    desc = L.make_desc(wl.n, wl.c_in, wl.h, wl.w, wl.c_out, dtype=L.DEFT_BF16)
    plan = L.deft_plan_create(desc)
    try:
        assert L.deft_workspace_bytes(plan, 0) > L.NOALLOC_SCRATCH_BYTES
        t = tensors(wl)
        y = torch.full((wl.n, wl.c_out, wl.ho, wl.wo), 7.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(L.DeftError) as e:
            L.deft_forward_noalloc(plan, t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y, None,
                                   torch.cuda.current_stream().cuda_stream)
        assert e.value.code == -11
        torch.cuda.synchronize()
        assert bool((y.float() == 7.0).all())
    finally:
        L.deft_plan_destroy(plan)
