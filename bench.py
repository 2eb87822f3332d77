"""Throughput of the single-GPU K-FAC step on ResNet-50 shapes at 32 samples per GPU.

One step = Kronecker factors of all 54 layers (53 convolutions and the classifier,
fp16 inputs) -> unpack to full symmetric -> 108 damped inverses -> G^-1 dW A^-1 for
all 54 layers (fp32 gradients) with the update w <- w - lr P of every weight in the
same kernel -> diagonal Fisher of all 53 BatchNorm layers with the gamma/beta update.
Inputs are synthetic and seeded, resident in HBM before timing starts.

Prints one JSON line: steps/s (`value`), the roofline of the kernel that takes the
most time (algorithmic work / its average launch duration from HIP events recorded
on its launch stream inside the timed region) and the fp64 oracle timed on the host
cores on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

PEAK_FP32_MFMA = 157.3   # TFLOP/s, MI355X dense fp32 matrix
PEAK_FP16_MFMA = 2516.6  # TFLOP/s, MI355X dense fp16 matrix
PEAK_HBM = 8000.0        # GB/s
TB = 128                 # block of the inverse
LR = 0.01                # learning rate of the parameter update

# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE), calibrated by a plain 1 GiB device copy (fetch x2.0,
# write x1.0) and summarised in profiles/resnet50_step_hbm_counters.md. Reported only
# while the kernel's source text still hashes to the value it was measured with.
MEASURED_TRAFFIC = {"inv_update_kernel": (970451456, "3d5e4963843e59a4a5a228c1bd1c9c537f3130f2")}
CSRC = os.path.join(ROOT, "fac_second_order_amd", "csrc")


def kernel_source_sha(name):
    """Hash of the update kernel's own source: its tile routine, the kernel, and the
    tile engine headers they use."""
    import hashlib
    if name != "inv_update_kernel":
        return None
    inv = open(os.path.join(CSRC, "invert.hip")).read()
    tile = inv[inv.index("// Update of step k:"):inv.index("// Pivot of step k. Sub-step J runs")]
    kern = inv[inv.index("// Update after the group of steps"):inv.index("// Bordered last column")]
    text = tile + kern + open(os.path.join(CSRC, "tile_f32.hpp")).read() + \
        open(os.path.join(CSRC, "common.hpp")).read()
    return hashlib.sha1(text.encode()).hexdigest()


def measured_traffic(name):
    rec = MEASURED_TRAFFIC.get(name)
    if rec is None or kernel_source_sha(name) != rec[1]:
        return None
    return rec[0]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=None, help="default 32 (128 for --workload stale)")
    ap.add_argument("--workload", choices=["resnet50", "stale", "capture"], default="resnet50",
                    help="resnet50: one full K-FAC step per step (batch 32); stale: refresh "
                         "every 10 steps with EMA 0.95, preconditioning only otherwise (batch 128); "
                         "capture: training iterations of a randomly initialised ResNet-50 on "
                         "synthetic 224x224 images, factors from its own activations (batch 32)")
    ap.add_argument("--precond-accum", choices=["f32", "f64"], default="f32",
                    help="accumulation of the preconditioning products (f64: kfac_precondition_ex)")
    ap.add_argument("--refine-inverse", action="store_true",
                    help="one fp64-residual refinement step of every inverse (kfac_invert_refine)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="time the steps without per-kernel events (roofline then null)")
    ap.add_argument("--copy-calibration", type=float, default=0.0,
                    help="also run a plain copy of this many GiB (for counter calibration)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# algorithmic work (what the method must do), per step
# ---------------------------------------------------------------------------

def inverse_update_flops(n_all, group=2):
    """Algorithmic flops of the inverse's update launches and of its row updates per
    call, for block steps taken in groups of `group` (kfac_invert_schedule).

    Before pivot k = kg + s of a group starting at kg, block row k takes the group's
    earlier steps (rows kg+s' of the group take only the steps after s', having been
    rewritten by that step's panel; of the diagonal block, the pivot takes step k-1 and
    the panel launches the steps before it). After the group, one update gives every other
    upper tile the group's steps it has not had: all of them outside the group's
    rows, the steps after the latest of its own rows inside them. A tile counts its
    entries on or above the diagonal, 2 flops per multiply-add. An order 128m + 1 takes
    m block steps; its last column is a bordered step of the finish kernel."""
    upd = row = 0
    for n in n_all:
        nb = -(-n // TB)
        ns = n // TB if (n > TB and n % TB == 1) else nb  # block steps (bordered last column)
        bs = [min(TB, n - i * TB) for i in range(nb)]

        def area(i, j):
            return bs[i] * bs[j] if i < j else bs[i] * (bs[i] + 1) // 2

        for kg in range(0, ns, group):
            g = min(group, ns - kg)
            for s in range(1, g):
                k = kg + s
                for j in range(nb):
                    lo = j - kg + 1 if kg <= j < k else 0
                    kk = sum(bs[kg + t] for t in range(lo, s))
                    if kk:
                        row += 2 * area(min(j, k), max(j, k)) * kk
            for i in range(nb):
                for j in range(i, nb):
                    m = max([x - kg for x in (i, j) if kg <= x < kg + g], default=-1)
                    kk = sum(bs[kg + t] for t in range(m + 1, g))
                    if kk:
                        upd += 2 * area(i, j) * kk
    return upd, row


def work(layers, bns, group=2):
    syrk = sum(l.rows * l.d_a * (l.d_a + 1) + l.rows * l.d_g * (l.d_g + 1) for l in layers)
    n_all = [l.d_a for l in layers] + [l.d_g for l in layers]
    inv = sum(n ** 3 for n in n_all)
    pre = sum(2 * l.d_g ** 2 * l.d_a + 2 * l.d_g * l.d_a ** 2 for l in layers)
    # the step unpacks the upper triangle only (the inverse reads no more): read + write
    pack_bytes = sum(2 * (n * (n + 1) // 2 * 4) for n in n_all)
    finish_bytes = sum(n * (n + 1) // 2 * 4 + n * n * 4 for n in n_all)
    bn_bytes = sum(2 * b.n * b.hw * b.c * 2 + 4 * b.c * 4 for b in bns)
    upd, row = inverse_update_flops(n_all, group)
    return {"syrk_flop": syrk, "inv_flop": inv, "pre_flop": pre, "pack_bytes": pack_bytes,
            "finish_bytes": finish_bytes, "bn_bytes": bn_bytes, "update_flop": upd, "rowupd_flop": row}


def stage_rates(kern, w):
    """Per-stage rates from the per-kernel breakdown (ms per step): algorithmic work of
    the stage over the summed time of its kernels, against the stage's bound."""
    def ms(*names):
        return sum(kern.get(n, (0.0, 0))[0] for n in names)
    out = {}
    for stage, names, work_, unit, peak in (
            ("factors", ("syrk_tile_kernel", "syrk_reduce_kernel"), w["syrk_flop"], "TFLOP/s", PEAK_FP16_MFMA),
            ("inverse", ("inv_prep_kernel", "inv_pivot_kernel", "inv_panel_kernel",
                         "inv_update_kernel", "inv_finish_kernel"), w["inv_flop"], "TFLOP/s", PEAK_FP32_MFMA),
            ("precondition", ("gemm_tn_kernel",), w["pre_flop"], "TFLOP/s", PEAK_FP32_MFMA),
            ("bn", ("bn_partial_kernel", "bn_finish_kernel"), w["bn_bytes"], "GB/s", PEAK_HBM),
            ("unpack", ("unpack_kernel",), w["pack_bytes"], "GB/s", PEAK_HBM),
            ("inverse_finish", ("inv_finish_kernel",), w["finish_bytes"], "GB/s", PEAK_HBM)):
        t = ms(*names)
        if t <= 0:
            continue
        rate = work_ / (t * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
        out[stage] = {"ms": round(t, 4), "achieved": round(rate, 1), "unit": unit, "peak": peak,
                      "frac": round(rate / peak, 4)}
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample, scaled stage by stage
# ---------------------------------------------------------------------------

def cpu_baseline(layers, bns, budget_s=25.0):
    """Times the fp64 oracle on every third layer (factors, inverses, preconditioning)
    and every third BatchNorm layer, and scales each stage by its share of the
    algorithmic work (flops for the matrix stages, bytes for BN) to a full step."""
    import oracle
    seed = 300
    samp = layers[::3]
    samp_bn = bns[::3]
    s = float(np.float32(np.sqrt(1e-3)))
    t = {"factors": 0.0, "invert": 0.0, "precondition": 0.0, "bn": 0.0}
    w_full = work(layers, bns)
    w_samp = work(samp, samp_bn)
    t_start = time.perf_counter()
    for i, l in enumerate(samp):
        rng = synth.layer_rng(seed, i)
        act = synth.relu_normal_f16(rng, l.act_shape)
        gout = synth.normal_f16(rng, l.gout_shape)
        grad = synth.normal_f32(rng, (l.d_g, l.d_a), 0.1)
        wt = synth.normal_f32(rng, (l.d_g, l.d_a), 0.05)
        t0 = time.perf_counter()
        A, G = oracle.conv_factors(act, gout, l.kh, l.kw, l.sh, l.sw, l.ph, l.pw, l.bias)
        t1 = time.perf_counter()
        Ai, _ = oracle.damped_inverse(A.astype(np.float32), s)
        Gi, _ = oracle.damped_inverse(G.astype(np.float32), s)
        t2 = time.perf_counter()
        oracle.sgd_update(wt, oracle.precondition(Gi, grad, Ai), LR)
        t3 = time.perf_counter()
        t["factors"] += t1 - t0
        t["invert"] += t2 - t1
        t["precondition"] += t3 - t2
        if time.perf_counter() - t_start > 4 * budget_s:
            raise RuntimeError("oracle sample exceeded its time budget")
    for i, b in enumerate(samp_bn):
        rng = synth.layer_rng(seed + 1, i)
        x = synth.normal_f16(rng, b.shape)
        g = synth.normal_f16(rng, b.shape)
        prm = np.stack([np.ones(b.c), np.zeros(b.c)])
        t0 = time.perf_counter()
        oracle.sgd_update(prm, oracle.bn_diag_fisher(x, g, 1e-3)["precond"], LR)
        t["bn"] += time.perf_counter() - t0
    scale = {"factors": w_full["syrk_flop"] / w_samp["syrk_flop"],
             "invert": w_full["inv_flop"] / w_samp["inv_flop"],
             "precondition": w_full["pre_flop"] / w_samp["pre_flop"],
             "bn": w_full["bn_bytes"] / w_samp["bn_bytes"]}
    est = sum(t[k] * scale[k] for k in t)
    sampled = sum(t.values())
    cores = len(os.sched_getaffinity(0))
    return {"value": 1.0 / est, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": (f"fp64 oracle on every third of the 54 K-FAC layers ({len(samp)}) and of the "
                       f"53 BN layers ({len(samp_bn)}), {sampled:.1f} s measured; each stage scaled by "
                       f"its share of algorithmic work to a full step of {est:.1f} s "
                       f"(factors {t['factors']*scale['factors']:.1f}, inverses "
                       f"{t['invert']*scale['invert']:.1f}, precondition and update "
                       f"{t['precondition']*scale['precondition']:.1f}, BN {t['bn']*scale['bn']:.1f} s)")}


# ---------------------------------------------------------------------------
# GPU step
# ---------------------------------------------------------------------------

def make_inputs(layers, bns, device, seed=3, grad_dtype=None, gout_std=1.0):
    import torch
    grad_dtype = grad_dtype or torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def normal(shape, std, dtype):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
        return x.to(dtype)

    act = [normal(l.act_shape, 1.0, torch.float16).relu_() for l in layers]
    gout = [normal(l.gout_shape, gout_std, torch.float16) for l in layers]
    grads = [normal((l.d_g, l.d_a), 0.1, grad_dtype) for l in layers]
    xhat = [normal(b.shape, 1.0, torch.float16) for b in bns]
    bgout = [normal(b.shape, gout_std, torch.float16) for b in bns]
    return act, gout, grads, xhat, bgout


def make_params(layers, bns, device, seed=4):
    """fp32 weights N(0, 0.05^2) per layer ([d_g, d_a], bias in the last column) and
    BatchNorm parameters gamma = 1, beta = 0, the tensors the update writes."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    weights = [torch.randn((l.d_g, l.d_a), generator=g, device=device) * 0.05 for l in layers]
    bn_params = [torch.stack([torch.ones(b.c, device=device), torch.zeros(b.c, device=device)])
                 for b in bns]
    return weights, bn_params


def run_stale(args):
    """Stale curvature at batch 128: every 10th step refreshes the factors (EMA 0.95,
    the first refresh overwrites) and the inverses; every step preconditions one of
    ten fp16 N(0,1e-2) gradient sets. Two activation/gradient sets alternate across
    refreshes. Reports amortised steps/s over `steps` steps."""
    import torch
    import fac_second_order_amd as kfac
    dev = torch.device("cuda:0")
    batch = args.batch or 128
    layers = synth.conv_layers(batch)
    bns = synth.bn_layers(batch)
    sets = [make_inputs(layers, bns, dev, seed=50 + s, grad_dtype=torch.float16, gout_std=0.1)
            for s in range(2)]
    gen = torch.Generator(device=dev)
    gen.manual_seed(60)
    grads = [[(torch.randn((l.d_g, l.d_a), generator=gen, device=dev) * 0.1).half() for l in layers]
             for _ in range(10)]
    st = kfac.KfacStep(layers, bns, dev)
    weights, bn_params = make_params(layers, bns, dev)
    nref = [0]

    def step(t):
        refresh = t % 10 == 0
        s = nref[0] % 2 if refresh else (nref[0] - 1) % 2
        act, gout, _, xhat, bgout = sets[s]
        decay = 0.0 if (refresh and nref[0] == 0) else 0.95
        st.step(act, gout, grads[t % 10], xhat, bgout, ema_decay=decay, refresh=refresh,
                weights=weights, bn_params=bn_params, lr=LR)
        if refresh:
            nref[0] += 1

    steps = args.steps if args.steps % 10 == 0 else 100   # whole refresh cycles only
    for t in range(10):          # one warm-up cycle (refresh + 9 stale steps)
        step(t)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(steps):
        step(t)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if int(st.info.abs().sum()) != 0:
        raise RuntimeError("Cholesky breakdown on a damped factor")
    out = {
        "metric": "K-FAC amortised steps/sec (ResNet-50 shapes, batch 128, refresh every 10, EMA 0.95, 1 GPU)",
        "value": round(steps / elapsed, 3), "unit": "steps/s", "n_gpus": 1, "steps": steps, "warmup": 10,
        "ms_per_step": round(1e3 * elapsed / steps, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "resnet50_kfac_stale_schedule", "batch_per_gpu": batch, "refresh_every": 10,
                   "ema_decay": 0.95, "grad_dtype": "f16", "lr": LR},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def run_capture(args):
    """Training iterations of a randomly initialised ResNet-50 (PyTorch forward and
    backward, fp32, channels-last) on one fixed batch of synthetic 224x224 images with
    random labels; each iteration's K-FAC step (factors from the captured activations
    and output gradients, inverses, preconditioning and update of every weight and
    BatchNorm parameter) runs in libkfac. Reports iterations/s and the K-FAC step's
    share, timed with events on the stream the library runs on."""
    import torch
    import torch.nn.functional as F
    from fac_second_order_amd.capture import KfacCapture, ResNet50
    dev = torch.device("cuda:0")
    batch = args.batch or 32
    torch.manual_seed(5)
    model = ResNet50(1000).to(dev).to(memory_format=torch.channels_last)
    cap = KfacCapture(model, damping=1e-3, ema_decay=0.95)
    g = torch.Generator(device=dev)
    g.manual_seed(6)
    x = torch.randn(batch, 3, 224, 224, generator=g, device=dev).to(memory_format=torch.channels_last)
    y = torch.randint(0, 1000, (batch,), generator=g, device=dev)
    ev = []

    def it(timed):
        model.zero_grad(set_to_none=True)
        F.cross_entropy(model(x), y).backward()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cap.step(lr=1e-3)
        e1.record()
        if timed:
            ev.append((e0, e1))

    for _ in range(args.warmup):
        it(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        it(True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    if int(cap.kstep.info.abs().sum()) != 0:
        raise RuntimeError("Cholesky breakdown on a damped factor")
    kfac_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    out = {
        "metric": "ResNet-50 training iterations/sec with K-FAC (batch 32, factors from the network's "
                  "own activations, 1 GPU)",
        "value": round(args.steps / elapsed, 3), "unit": "iterations/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(1e3 * elapsed / args.steps, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "resnet50_capture", "batch_per_gpu": batch, "image": 224, "classes": 1000,
                   "damping": 1e-3, "lr": 1e-3, "ema_decay": 0.95,
                   "kfac_ms_per_step": round(kfac_ms, 3),
                   "forward_backward_ms_per_step": round(1e3 * elapsed / args.steps - kfac_ms, 3)},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's K-FAC step; runs on more than one GPU are not "
              "part of this build (the multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)
    import torch
    import fac_second_order_amd as kfac

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "stale":
        run_stale(args)
        return
    if args.workload == "capture":
        run_capture(args)
        return
    args.batch = args.batch or 32
    layers = synth.conv_layers(args.batch)
    bns = synth.bn_layers(args.batch)
    w = work(layers, bns, kfac.kfac_invert_schedule()[1])
    act, gout, grads, xhat, bgout = make_inputs(layers, bns, dev)
    weights, bn_params = make_params(layers, bns, dev)
    st = kfac.KfacStep(layers, bns, dev, precond_accum=args.precond_accum, refine_inverse=args.refine_inverse)

    def step():
        st.step(act, gout, grads, xhat, bgout, weights=weights, bn_params=bn_params, lr=LR)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(st.info.abs().sum()) != 0:
        raise RuntimeError("Cholesky breakdown on a damped factor: " + str(st.info.tolist()))

    timing = not args.no_kernel_timing
    kern, dominant = {}, None
    if timing:
        # breakdown pass (untimed): every launch bracketed by events, over two steps
        kfac.kfac_timing_reset()
        kfac.kfac_timing_only(-1)
        kfac.kfac_timing_enable(True)
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        kfac.kfac_timing_enable(False)
        for i in range(kfac.kfac_timing_kernels()):
            ms, n = kfac.kfac_timing_read(i)
            if n:
                kern[kfac.kfac_kernel_name(i)] = (ms / 2, n // 2)
        kfac.kfac_timing_reset()
        dominant = max(range(kfac.kfac_timing_kernels()),
                       key=lambda i: kern.get(kfac.kfac_kernel_name(i), (0.0, 0))[0])
        # timed region: events around the dominant kernel's launches only
        kfac.kfac_timing_only(dominant)
        kfac.kfac_timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    live = None
    if timing:
        kfac.kfac_timing_enable(False)
        live = (kfac.kfac_kernel_name(dominant),) + tuple(kfac.kfac_timing_read(dominant))
        kfac.kfac_timing_reset()
        kfac.kfac_timing_only(-1)

    ms_step = 1e3 * elapsed / args.steps
    value = args.steps / elapsed

    roofline = None
    if live:
        name, ms, n = live  # summed over the timed steps, measured in the timed region
        per_launch = {  # algorithmic work of one average launch, and its bound
            "inv_update_kernel": (w["update_flop"] * args.steps, "mfma", PEAK_FP32_MFMA),
            "syrk_tile_kernel": (w["syrk_flop"] * args.steps, "mfma", PEAK_FP16_MFMA),
            "gemm_tn_kernel": (w["pre_flop"] * args.steps, "mfma", PEAK_FP32_MFMA),
        }
        if name in per_launch:
            total_work, bound, peak = per_launch[name]
            achieved = total_work / (ms * 1e-3) / 1e12      # = per-launch work / average duration
            roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(achieved / peak, 4), "traffic": measured_traffic(name), "kernel": name,
                        "launches": n, "avg_launch_us": round(1e3 * ms / n, 2),
                        "algorithmic_per_launch": total_work / n}
        elif name in ("bn_partial_kernel", "unpack_kernel"):
            b = w["bn_bytes"] if name == "bn_partial_kernel" else w["pack_bytes"]
            achieved = b * args.steps / (ms * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM, 4), "traffic": None, "kernel": name,
                        "launches": n, "avg_launch_us": round(1e3 * ms / n, 2),
                        "algorithmic_per_launch": b * args.steps / n}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(layers, bns)

    if args.copy_calibration > 0:
        nbytes = int(args.copy_calibration * (1 << 30))
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    out = {
        "metric": "K-FAC steps/sec (ResNet-50 shapes, batch 32, 1 GPU); TFLOP/s vs MFMA peak",
        "value": round(value, 3), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "resnet50_kfac_step", "batch_per_gpu": args.batch,
                   "kfac_layers": len(layers), "factors": 2 * len(layers), "bn_layers": len(bns),
                   "damping": 1e-3, "lr": LR, "precond_accum": args.precond_accum, "refine_inverse": args.refine_inverse, "inputs": "fp16 ReLU(N(0,1)) activations, fp16 N(0,1) "
                   "output and BN gradients, fp32 N(0,1e-2) weight gradients, fp32 N(0,2.5e-3) weights"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_ms_per_step": {k: round(v[0], 4) for k, v in
                                sorted(kern.items(), key=lambda kv: -kv[1][0])},
        "stage_rates": stage_rates(kern, w) if kern else None,
        "step_tflop": round((w["syrk_flop"] + w["inv_flop"] + w["pre_flop"]) / 1e12, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
