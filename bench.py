"""Benchmark: one training step (forward + backward) of the deformable 3x3
layer at N=16, Cin=Cout=256, 56x56, bf16 on one MI355X, through the C ABI.

A step runs every stage of the hot path: the fused offset-conv + bilinear
sampling kernel, the main-convolution MFMA GEMM, and the backward (dCol and dW
GEMMs, sampling backward, offset-conv backward).  Inputs are seeded synthetic
tensors already resident in HBM; the plan's halo comes from the offset
histogram of a warm-up forward.  Prints one JSON line on stdout.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}  # dense MFMA


FORWARD_KERNELS = ("prep_forward", "x_channel_minor", "fused_offset_sample", "gemm_forward")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(wl):
    """Algorithmic bytes and flops per launch of each kernel (see the header of
    each kernel for what it must move).  bf16 = 2 bytes, fp32 accumulators 4."""
    esz = 2 if wl.dtype == "bf16" else 4
    P = wl.n * wl.ho * wl.wo
    ck = wl.c_in * wl.taps
    x = wl.n * wl.c_in * wl.h * wl.w
    cols = P * ck * esz
    offs = P * wl.oc * 4
    gemm_flop = 2.0 * wl.c_out * ck * P
    off_flop = 2.0 * wl.oc * ck * P
    return {
        "x_channel_minor": (2 * x * esz, 0.0),
        "fused_offset_sample": (x * esz + cols + wl.oc * ck * esz + (offs if wl.train else 0), off_flop),
        "gemm_forward": (cols + wl.c_out * ck * esz + P * wl.c_out * esz, gemm_flop),
        "gemm_dcol": (P * wl.c_out * esz + wl.c_out * ck * esz + cols, gemm_flop),
        "gemm_dw": (cols + P * wl.c_out * esz + wl.c_out * ck * 4, gemm_flop),
        "sample_backward": (cols + x * esz + offs + offs + x * 4, 0.0),
        "offset_weight_backward": (offs + x * esz + wl.oc * ck * 4, off_flop),
        "dx_final": (offs + wl.c_in * wl.oc * wl.taps * esz + x * 4 + x * esz, off_flop),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="train_bf16_n16_c256_56x56_s1")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU-baseline time budget")
    ap.add_argument("--no-dwconv", action="store_true", help="skip the dilated depthwise conv timings")
    ap.add_argument("--no-other", action="store_true", help="skip the forward at the other configurations")
    ap.add_argument("--no-libgemm", action="store_true",
                    help="skip timing the library GEMM (torch.matmul) on the three GEMM shapes")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times) after the timed steps, as the "
                         "reference kernel for scaling hardware byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from irregular_gather_cnn_amd import _lib as L
    from irregular_gather_cnn_amd.layer import DeformConv, halo_histogram
    from irregular_gather_cnn_amd.synth import WORKLOADS, make_inputs

    wl = WORKLOADS[args.workload]
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    inp = make_inputs(wl, with_dy=True)
    t = {k: torch.from_numpy(v).to(tdt).to(dev) for k, v in inp.items()}
    geo = dict(n=wl.n, c_in=wl.c_in, h=wl.h, w=wl.w, c_out=wl.c_out, kh=wl.kh, kw=wl.kw,
               stride=(wl.stride,) * 2, pad=(wl.pad,) * 2, dil=(wl.dil,) * 2, groups=wl.groups, dtype=wl.dtype)
    log("bench: %s on %s" % (wl.name, torch.cuda.get_device_name(0)))

    # plan from the measured offset distribution
    probe = DeformConv(**geo, training=True, device=dev)
    _, off = probe.forward(t["x"], t["w_off"], t["b_off"], t["w"], t["b"])
    hist = halo_histogram(probe.desc, off, 16)
    off_h = off.cpu().numpy()
    del probe
    layer = DeformConv(**geo, plan=hist, training=True, device=dev)
    info = layer.info
    tot = float(sum(hist))
    log("offset std %.3f px; fully outside taps %.4f; required-halo histogram %s"
        % (float(off_h.std()), hist[-1] / tot, hist))
    log("plan: tile %dx%d halo %d chunk %d, %d workgroups, %d B LDS; backward tile %dx%d chunk %d halo %d, "
        "est. miss %.6f"
        % (info["tile_h"], info["tile_w"], info["halo"], info["chunk"], info["num_workgroups"], info["lds_bytes"],
           info["bwd_tile_h"], info["bwd_tile_w"], info["bwd_chunk"], info["bwd_halo"], info["est_miss_fraction"]))

    y = torch.empty((wl.n, wl.c_out, wl.ho, wl.wo), dtype=tdt, device=dev)
    offs = torch.empty((wl.n, wl.oc, wl.ho, wl.wo), dtype=torch.float32, device=dev)
    grads = dict(dx=torch.empty_like(t["x"]), dw_off=torch.empty_like(t["w_off"]), dw=torch.empty_like(t["w"]),
                 db_off=torch.empty_like(t["b_off"]), db=torch.empty_like(t["b"]))

    def step():
        layer.forward(t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y=y, offsets=offs)
        layer.backward(t["x"], t["w_off"], t["w"], offs, t["dy"], out=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done (%d steps)" % args.warmup)

    # timed region: exactly K steps, with an event between consecutive steps
    # for the per-step spread (events are recorded on the launch stream)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = ev[0].elapsed_time(ev[-1]) / args.steps
    warm = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    log("timed: %d steps, %.3f ms/step (host wall %.3f s)" % (args.steps, ms_step, wall))

    def spread(v):
        q = np.percentile(np.asarray(v, np.float64), [10, 50, 90])
        return {"p10": round(float(q[0]), 4), "median": round(float(q[1]), 4), "p90": round(float(q[2]), 4)}

    # cold caches: before every step, outside its events, 512 MiB are written
    # (twice the 256 MB Infinity Cache, far more than the L2s), so the step
    # starts with none of its inputs cached and the caches full of dirty lines
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(args.steps):
        flush.fill_(1)
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        step()
        b_.record()
        torch.cuda.synchronize()
        cold.append(a_.elapsed_time(b_))
    del flush
    step_spread = {"warm": spread(warm), "cold": spread(cold)}
    log("per-step ms: %s" % step_spread)

    # measured HBM rates on this device: a 1 GiB device copy (read + write)
    # and a 1 GiB fill (write only)
    def hbm_rates():
        nb = 1 << 30
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dstc = torch.empty_like(src)
        dstc.copy_(src)
        src.fill_(0)
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        for _ in range(5):
            dstc.copy_(src)
        b_.record()
        torch.cuda.synchronize()
        copy = 5 * 2 * nb / (a_.elapsed_time(b_) * 1e-3) / 1e9
        a_.record()
        for _ in range(5):
            src.fill_(3)
        b_.record()
        torch.cuda.synchronize()
        fill = 5 * nb / (a_.elapsed_time(b_) * 1e-3) / 1e9
        del src, dstc
        return {"copy_gbs": round(copy, 1), "fill_gbs": round(fill, 1), "bytes": nb}
    hbm_meas = hbm_rates()
    log("measured HBM: %s" % hbm_meas)

    # Context for the three GEMMs: the vendor library (torch.matmul, i.e.
    # hipBLASLt) on the same bf16 shapes with contiguous row-major operands:
    # y = cols @ W^T, dCol = dY @ W, dW = dY^T @ cols (median of 10 calls).
    libgemm = None
    if not args.no_libgemm and wl.dtype == "bf16":
        P_, K_, O_ = wl.n * info["ho"] * info["wo"], wl.c_in * wl.kh * wl.kw, wl.c_out
        g = torch.Generator(device=dev).manual_seed(0)
        colsm = torch.randn(P_, K_, device=dev, generator=g).bfloat16()
        wtm = torch.randn(K_, O_, device=dev, generator=g).bfloat16()
        wm = wtm.t().contiguous()
        dym = torch.randn(P_, O_, device=dev, generator=g).bfloat16()
        dytm = dym.t().contiguous()
        ym = torch.empty(P_, O_, device=dev, dtype=torch.bfloat16)
        dcm = torch.empty(P_, K_, device=dev, dtype=torch.bfloat16)
        dwm = torch.empty(O_, K_, device=dev, dtype=torch.bfloat16)

        def lib_time(fn):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(10):
                a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a_.record()
                fn()
                b_.record()
                torch.cuda.synchronize()
                ts.append(a_.elapsed_time(b_) * 1000)
            return round(sorted(ts)[5], 1)
        libgemm = {"forward_us": lib_time(lambda: torch.matmul(colsm, wtm, out=ym)),
                   "dcol_us": lib_time(lambda: torch.matmul(dym, wm, out=dcm)),
                   "dw_us": lib_time(lambda: torch.matmul(dytm, colsm, out=dwm)),
                   "operands": "contiguous row-major bf16, torch.matmul"}
        del colsm, wtm, wm, dym, dytm, ym, dcm, dwm
        log("library GEMMs: %s" % libgemm)

    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device=dev)
        dstc = torch.empty_like(src)
        for _ in range(3):
            dstc.copy_(src)
        torch.cuda.synchronize()
        del src, dstc

    # instrumented pass: per-kernel durations from events around each launch
    L.deft_timing_start(64 * args.steps)
    for _ in range(args.steps):
        step()
    L.deft_timing_stop()
    per = {}
    for i in range(L.deft_timing_count()):
        name, ms = L.deft_timing_get(i)
        per.setdefault(name, []).append(ms)
    work = kernel_work(wl)
    kernels = {}
    for name, v in per.items():
        avg = sum(v) / len(v)
        launches = len(v) / args.steps
        rec = {"avg_ms": round(avg, 5), "launches_per_step": launches, "ms_per_step": round(avg * launches, 5)}
        if name in work:
            b, f = work[name]
            rec["gbs"] = round(b / (avg * 1e-3) / 1e9, 1)
            rec["hbm_frac"] = round(rec["gbs"] / HBM_PEAK_GBS, 4)
            if f:
                rec["tflops"] = round(f / (avg * 1e-3) / 1e12, 2)
                rec["mfma_frac"] = round(rec["tflops"] / MFMA_PEAK_TFLOPS[wl.dtype], 4)
        kernels[name] = rec
    for name, rec in sorted(kernels.items(), key=lambda kv: -kv[1]["ms_per_step"]):
        log("  %-24s %s" % (name, rec))
    fwd_ms = sum(kernels[k]["ms_per_step"] for k in FORWARD_KERNELS if k in kernels)
    bwd_ms = sum(r["ms_per_step"] for k, r in kernels.items()
                 if k not in FORWARD_KERNELS)

    dom = max((k for k in kernels if k in work), key=lambda k: kernels[k]["ms_per_step"])
    b, f = work[dom]
    avg = kernels[dom]["avg_ms"]
    gbs = b / (avg * 1e-3) / 1e9
    if f and (f / b) > MFMA_PEAK_TFLOPS[wl.dtype] * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = {"bound": "mfma", "achieved": round(f / (avg * 1e-3) / 1e12, 2),
                "peak": MFMA_PEAK_TFLOPS[wl.dtype], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = int(b)
    # HBM traffic from the committed rocprofv3 counter summary of this
    # workload, if the dominant kernel's sources still match it
    roof["traffic"] = None
    from irregular_gather_cnn_amd import profiling
    tr = profiling.read_traffic(os.path.join(ROOT, "profiles", "hbm_traffic_%s.md" % wl.name))
    if dom in tr and tr[dom][1] == profiling.source_hash(dom):
        roof["traffic"] = tr[dom][0]

    # The fused forward against the unfused three-operator forward (offset conv
    # -> offsets through HBM -> sampling -> GEMM) on the same plan and inputs:
    # what fusing the offset convolution into the sampling kernel buys here.
    def time_forward(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b_.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / args.steps

    fused_fn = lambda: layer.forward(t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y=y, offsets=offs)
    unfused_fn = lambda: layer.forward_unfused(t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y=y, offsets=offs)
    fusion = {"fused_fwd_ms": round(time_forward(fused_fn), 4), "unfused_fwd_ms": round(time_forward(unfused_fn), 4)}
    # the forward whose gather feeds the main GEMM directly (same tile and halo)
    try:
        gg = DeformConv(**geo, plan=(info["tile_h"], info["tile_w"], info["halo"], -2), training=True, device=dev)
    except L.DeftError:
        gg = None
    if gg is not None:
        gg_fn = lambda: gg.forward(t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y=y, offsets=offs)
        fusion["gather_gemm_fwd_ms"] = round(time_forward(gg_fn), 4)
        del gg
    # The pages' own staging (tile + halo of the input in LDS, out-of-halo
    # taps from global memory) on the same inputs, under a few forced plans:
    # the forward the default direct gather replaced, re-measured.
    if wl.dtype == "bf16":
        lds = {}
        for th, tw, hh, ch in ((8, 8, 2, 64), (8, 8, 3, 64), (8, 8, 2, 32), (4, 16, 2, 64)):
            try:
                lh = DeformConv(**geo, plan=(th, tw, hh, ch), training=False, device=dev)
            except L.DeftError:
                continue
            lh_fn = lambda: lh.forward(t["x"], t["w_off"], t["b_off"], t["w"], t["b"], y=y)
            lds["%dx%d_halo%d_chunk%d" % (th, tw, hh, ch)] = round(time_forward(lh_fn), 4)
            del lh
        if lds:
            fusion["lds_halo_fwd_ms"] = lds
    L.deft_timing_start(8 * args.steps)
    for _ in range(args.steps):
        unfused_fn()
    L.deft_timing_stop()
    un = {}
    for i in range(L.deft_timing_count()):
        name, ms = L.deft_timing_get(i)
        un.setdefault(name, []).append(ms)
    fusion["unfused_kernels_ms"] = {k: round(sum(v) / len(v), 5) for k, v in un.items()}
    log("fusion: %s" % fusion)

    # The forward at the other configurations of the layer (fp32, wide offsets
    # with 4 groups and pushed taps, stride 2): fused sampling kernel GB/s and
    # main GEMM MFMA share against the peak of each dtype, planned from each
    # workload's own offset histogram.
    others = {}
    if not args.no_other:
        for oname in ("fp32_n8_c128_64x64", "bf16_n16_c512_28x28_g4_wide", "train_bf16_n16_c256_56x56_s2"):
            owl = WORKLOADS[oname]
            otd = torch.bfloat16 if owl.dtype == "bf16" else torch.float32
            oin = make_inputs(owl)
            ot = {k: torch.from_numpy(v).to(otd).to(dev) for k, v in oin.items()}
            ogeo = dict(n=owl.n, c_in=owl.c_in, h=owl.h, w=owl.w, c_out=owl.c_out, kh=owl.kh, kw=owl.kw,
                        stride=(owl.stride,) * 2, pad=(owl.pad,) * 2, dil=(owl.dil,) * 2, groups=owl.groups,
                        dtype=owl.dtype)
            oprobe = DeformConv(**ogeo, training=True, device=dev)
            _, ooff = oprobe.forward(ot["x"], ot["w_off"], ot["b_off"], ot["w"], ot["b"])
            ohist = halo_histogram(oprobe.desc, ooff, 16)
            del oprobe
            olayer = DeformConv(**ogeo, plan=ohist, training=owl.train, device=dev)
            oy = torch.empty((owl.n, owl.c_out, owl.ho, owl.wo), dtype=otd, device=dev)
            oof = torch.empty((owl.n, owl.oc, owl.ho, owl.wo), dtype=torch.float32, device=dev)
            ofn = lambda: olayer.forward(ot["x"], ot["w_off"], ot["b_off"], ot["w"], ot["b"], y=oy,
                                         offsets=oof if owl.train else None)
            fwd_ms_o = time_forward(ofn)
            train_ms_o = None
            if owl.train:
                # the whole training step at this configuration (forward + backward)
                ody = torch.from_numpy(make_inputs(owl, with_dy=True)["dy"]).to(otd).to(dev)
                og = dict(dx=torch.empty_like(ot["x"]), dw_off=torch.empty_like(ot["w_off"]),
                          dw=torch.empty_like(ot["w"]), db_off=torch.empty_like(ot["b_off"]),
                          db=torch.empty_like(ot["b"]))

                def ostep():
                    ofn()
                    olayer.backward(ot["x"], ot["w_off"], ot["w"], oof, ody, out=og)
                train_ms_o = time_forward(ostep)
                del ody, og
            L.deft_timing_start(8 * args.steps)
            for _ in range(args.steps):
                ofn()
            L.deft_timing_stop()
            oper = {}
            for i in range(L.deft_timing_count()):
                name, ms = L.deft_timing_get(i)
                oper.setdefault(name, []).append(ms)
            owork = kernel_work(owl)
            rec = {"fwd_ms": round(fwd_ms_o, 4), "plan": {k: olayer.info[k] for k in ("tile_h", "tile_w", "halo",
                                                                                          "gather_direct")}}
            if train_ms_o is not None:
                rec["fwd_bwd_ms"] = round(train_ms_o, 4)
            pro = [sum(v) / len(v) for k, v in oper.items() if k in ("x_channel_minor", "prep_forward")]
            if pro:
                rec["prologue_us"] = round(sum(pro) * 1e3, 1)
            if not owl.train:
                # the pages' staging (tile + halo of the input in LDS) on the same
                # inputs, for comparison with the planned direct gather
                try:
                    lh = DeformConv(**ogeo, plan=(8, 8, max(1, olayer.info["halo"]), 32), training=False, device=dev)
                    lh_fn = lambda: lh.forward(ot["x"], ot["w_off"], ot["b_off"], ot["w"], ot["b"], y=oy)
                    rec["lds_halo_fwd_ms"] = round(time_forward(lh_fn), 4)
                    del lh
                except L.DeftError:
                    pass
            for kname in ("fused_offset_sample", "gemm_forward"):
                if kname in oper:
                    avg = sum(oper[kname]) / len(oper[kname])
                    b_, f_ = owork[kname]
                    rec[kname] = {"us": round(avg * 1e3, 1), "gbs": round(b_ / (avg * 1e-3) / 1e9, 1),
                                  "hbm_frac": round(b_ / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                    if kname == "gemm_forward":
                        tf = f_ / (avg * 1e-3) / 1e12
                        rec[kname]["tflops"] = round(tf, 1)
                        rec[kname]["mfma_frac"] = round(tf / MFMA_PEAK_TFLOPS[owl.dtype], 4)
            others[oname] = rec
            del olayer, ot, oy, oof
        log("other configurations (forward): %s" % others)

    # Second workload: the dilated depthwise 1-D convolution of the JAX issue
    # page (batch 32, 1024 steps, 512 channels, fp32, ramp inputs as there),
    # timed per kernel size and dilation; algorithmic bytes = x + y + w once.
    dwc = {}
    if not args.no_dwconv:
        B_, T_, C_ = 32, 1024, 512
        for K_ in (4, 16, 64):
            row = {}
            for d_ in (1, 2, 4, 8, 16, 32, 64, 128):
                L_ = T_ + d_ * (K_ - 1)
                xd = torch.arange(B_ * L_ * C_, dtype=torch.float32, device=dev).div_(B_ * L_ * C_).view(B_, L_, C_)
                wd = torch.arange(K_ * C_, dtype=torch.float32, device=dev).div_(K_ * C_).view(K_, C_)
                yd = torch.empty((B_, T_, C_), dtype=torch.float32, device=dev)
                fn = lambda: L.deft_dwconv1d_forward(xd, wd, yd, B_, T_, C_, K_, d_,
                                                     torch.cuda.current_stream().cuda_stream)
                ms_ = time_forward(fn)
                nbytes = 4.0 * (B_ * L_ * C_ + B_ * T_ * C_ + K_ * C_)
                row[str(d_)] = {"us": round(ms_ * 1e3, 1), "gbs": round(nbytes / (ms_ * 1e-3) / 1e9, 1)}
                del xd, wd, yd
            dwc["k%d" % K_] = row
        # fused depthwise + pointwise (512 -> 512 channels) against the
        # depthwise kernel followed by a library fp32 matmul for the mix
        O_ = 512
        for K_, d_ in ((4, 1), (16, 8)):
            L_ = T_ + d_ * (K_ - 1)
            xd = torch.arange(B_ * L_ * C_, dtype=torch.float32, device=dev).div_(B_ * L_ * C_).view(B_, L_, C_)
            wd = torch.arange(K_ * C_, dtype=torch.float32, device=dev).div_(K_ * C_).view(K_, C_)
            wp = torch.arange(C_ * O_, dtype=torch.float32, device=dev).div_(C_ * O_).view(C_, O_)
            yd = torch.empty((B_, T_, C_), dtype=torch.float32, device=dev)
            zd = torch.empty((B_, T_, O_), dtype=torch.float32, device=dev)
            st_ = torch.cuda.current_stream().cuda_stream
            fused_ = time_forward(lambda: L.deft_dwpw1d_forward(xd, wd, wp, zd, B_, T_, C_, O_, K_, d_, st_))

            def unfused_():
                L.deft_dwconv1d_forward(xd, wd, yd, B_, T_, C_, K_, d_, st_)
                torch.matmul(yd.view(-1, C_), wp, out=zd.view(-1, O_))
            unf_ = time_forward(unfused_)
            flop = 2.0 * B_ * T_ * C_ * (O_ + K_)
            dwc["dwpw_k%d_d%d" % (K_, d_)] = {"fused_us": round(fused_ * 1e3, 1), "unfused_us": round(unf_ * 1e3, 1),
                                              "fused_tflops": round(flop / (fused_ * 1e-3) / 1e12, 1)}
            del xd, wd, wp, yd, zd
        log("dilated depthwise conv (32x1024x512 fp32), fused depthwise+pointwise: %s" % dwc)

    # the fused sampling kernel together with the prologue launch it cannot
    # run without (channel-minor copy of x and weight layouts): bytes of both
    # over the time of both
    prologue_frac = None
    if "fused_offset_sample" in kernels:
        pk = [k for k in ("x_channel_minor", "prep_forward") if k in kernels]
        tb = sum(work[k][0] for k in ["fused_offset_sample"] + pk if k in work)
        tt = sum(kernels[k]["avg_ms"] for k in ["fused_offset_sample"] + pk)
        prologue_frac = round(tb / (tt * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    total_flop = sum(f for k, (b_, f) in work.items())
    gflops = total_flop / (ms_step * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu:
        import oracle
        s1 = oracle.Shape(1, wl.c_in, wl.h, wl.w, wl.c_out, wl.kh, wl.kw, (wl.stride,) * 2, (wl.pad,) * 2,
                          (wl.dil,) * 2, wl.groups)
        done, t_cpu = 0, 0.0
        while done < wl.n and t_cpu < args.cpu_seconds:
            sl = slice(done, done + 1)
            c0 = time.perf_counter()
            _, o = oracle.forward(s1, inp["x"][sl], inp["w_off"], inp["b_off"], inp["w"], inp["b"])
            oracle.backward(s1, inp["x"][sl], inp["w_off"], inp["w"], o, inp["dy"][sl])
            t_cpu += time.perf_counter() - c0
            done += 1
        cpu_ms = t_cpu / done * wl.n * 1e3
        model = ""
        try:
            with open("/proc/cpuinfo") as fh:
                for ln in fh:
                    if ln.startswith("model name"):
                        model = ln.split(":", 1)[1].strip()
                        break
        except OSError:
            pass
        cpu = {"value": round(cpu_ms, 1), "unit": "ms", "cores": oracle.threads(), "kind": "oracle",
               "cpu_model": model,
               "sample": "fp64 forward+backward of %d of the %d images (%.1f s), scaled x%d/%d to one full step"
                         % (done, wl.n, t_cpu, wl.n, done)}
        log("cpu baseline: %s" % cpu)

    line = {
        "metric": "deformable 3x3 layer fwd+bwd ms & GB/s / MFMA % (N=16,C=256,56x56,bf16)",
        "value": round(ms_step, 4), "unit": "ms", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "n": wl.n, "c_in": wl.c_in, "c_out": wl.c_out, "h": wl.h, "w": wl.w,
                   "kernel": [wl.kh, wl.kw], "stride": wl.stride, "pad": wl.pad, "dilation": wl.dil,
                   "offset_groups": wl.groups, "offset_std_px": wl.offset_std,
                   "plan": {k: info[k] for k in ("tile_h", "tile_w", "halo", "chunk", "gather_direct", "bwd_tile_h",
                                                 "bwd_tile_w", "bwd_chunk", "bwd_halo")}},
        "fwd_ms": round(fwd_ms, 4), "bwd_ms": round(bwd_ms, 4), "layer_gflops": round(gflops, 1),
        "step_ms_spread": step_spread,
        "hbm_measured": hbm_meas,
        "fused_sample_hbm_frac": kernels.get("fused_offset_sample", {}).get("hbm_frac"),
        "fused_sample_with_prologue_hbm_frac": prologue_frac,
        "main_gemm_mfma_frac": kernels.get("gemm_forward", {}).get("mfma_frac"),
        "fusion": fusion,
        "library_gemm": libgemm,
        "depthwise_dilated_1d": dwc or None,
        "other_configs_forward": others or None,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
