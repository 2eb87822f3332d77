"""Throughput of the single-GPU K-FAC step on ResNet-50 shapes at 32 samples per GPU.

One step = Kronecker factors of all 54 layers (53 convolutions and the classifier,
fp16 inputs, also written as the upper triangles the inversion reads) -> 108 damped inverses -> G^-1 dW A^-1 for
all 54 layers (fp32 gradients) with the update w <- w - lr P of every weight in the
same kernel -> diagonal Fisher of all 53 BatchNorm layers with the gamma/beta update.
Inputs are synthetic and seeded, resident in HBM before timing starts.

Prints one JSON line: steps/s (`value`, K steps over the wall clock between two
device synchronisations) with the per-step median, p10 and p90 from HIP events, the
roofline of the kernel that takes the most time (algorithmic work / its average
launch duration from HIP events recorded on its launch stream inside the timed
region), the fp64 oracle timed on the host cores on one full step of the same inputs,
and extra keys for the other workloads: the fully connected layer (32x64 / 32x16,
fp32), the 3x3 convolution 64->64 at 56x56 batch 32, batched inversion of all 108
ResNet-50-sized stress factors at condition numbers 1e2, 1e3, 1e4, and the
stale-curvature schedule at batch 128 (100 steps, refresh every 10, EMA 0.95).

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra-configs]
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

PEAK_FP16_MFMA = 2516.6  # TFLOP/s, MI355X dense fp16 (and bf16) matrix
# fp32 products formed from six bf16 MFMA products of exactly split operands (the
# update, the preconditioning and the refinement's correction): the bf16 peak over six
# is the bound of their algorithmic fp32 flops.
PEAK_X3 = round(PEAK_FP16_MFMA / 6, 1)
PEAK_FP32_MFMA = 157.3   # TFLOP/s, MI355X dense fp32 matrix (the same products on fp32 MFMA)

# kernels whose algorithmic work per launch bench.py models (roofline candidates)
MODELLED = {"inv_update_kernel", "syrk_tile_kernel", "gemm_tn_kernel", "gemm_tn64_kernel",
            "refine_residual_gemm_tn64_kernel", "refine_correction_gemm_tn_kernel", "bn_partial_kernel",
            "unpack_kernel"}
PEAK_HBM = 8000.0        # GB/s
TB = 128                 # block of the inverse
LR = 0.01                # learning rate of the parameter update

# HBM bytes per launch of the dominant kernel in the timed steps, from two rocprofv3
# --pmc passes (FETCH_SIZE, then WRITE_SIZE) over the launches of the timed steps,
# calibrated by a plain 1 GiB device copy (fetch x2.0, write x1.0) and summarised in
# profiles/resnet50_step_hbm_counters.md; keyed by kernel and by whether the step ran
# on two streams (the launches then hold fewer tiles each). Reported only while the
# kernel's source text still hashes to the value it was measured with.
MEASURED_TRAFFIC = {("inv_update_kernel", True): (829600000, "1882cb717ea2a1ce25667bf516af88a5691a2c8f")}
CSRC = os.path.join(ROOT, "fac_second_order_amd", "csrc")


def kernel_source_sha(name, group):
    """Hash of the update kernel's own source (its tile routine, the kernel and the tile
    engine headers they use) and of the group size the library was built with (the block
    steps one launch applies, from kfac_invert_schedule)."""
    import hashlib
    if name != "inv_update_kernel":
        return None
    inv = open(os.path.join(CSRC, "invert.hip")).read()
    tile = inv[inv.index("// Update of step k:"):inv.index("// Pivot of step k. Sub-step J runs")]
    kern = inv[inv.index("// Update after the group of steps"):inv.index("// Bordered last column")]
    text = tile + kern + open(os.path.join(CSRC, "tile_f32.hpp")).read() + \
        open(os.path.join(CSRC, "common.hpp")).read() + f"\ngroup {group}"
    return hashlib.sha1(text.encode()).hexdigest()


def measured_traffic(name, side_stream, group):
    rec = MEASURED_TRAFFIC.get((name, side_stream))
    if rec is None or kernel_source_sha(name, group) != rec[1]:
        return None
    return rec[0]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=10)
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
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="only the ResNet-50 step (no fc, 3x3, inversion-stress and stale-schedule keys)")
    ap.add_argument("--no-side-stream", action="store_true",
                    help="run the whole step on one stream (default: the 4609-order inverses and "
                         "their layers' preconditioning on a second stream)")
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
    # one refinement step of every inverse: the residual F X (fp64 sums) and the
    # correction X E (fp32 sums), 2 n^3 each
    refine = sum(2 * n ** 3 for n in n_all)
    return {"syrk_flop": syrk, "inv_flop": inv, "pre_flop": pre, "pack_bytes": pack_bytes, "refine_flop": refine,
            "finish_bytes": finish_bytes, "bn_bytes": bn_bytes, "update_flop": upd, "rowupd_flop": row}


PEAK_FP64_MFMA = 78.6    # TFLOP/s, MI355X dense fp64 matrix


def stage_rates(kern, w, precond_accum="f32"):
    """Per-stage rates from the per-kernel breakdown (ms per step): algorithmic work of
    the stage over the summed time of its kernels, against the stage's bound."""
    def ms(*names):
        return sum(kern.get(n, (0.0, 0))[0] for n in names)
    pre_peak = PEAK_FP64_MFMA if precond_accum == "f64" else PEAK_X3
    out = {}
    for stage, names, work_, unit, peak in (
            ("factors", ("syrk_tile_kernel", "syrk_reduce_kernel", "shift_assemble_kernel"), w["syrk_flop"], "TFLOP/s",
             PEAK_FP16_MFMA),
            ("inverse", ("inv_prep_kernel", "inv_pivot_kernel", "inv_panel_kernel",
                         "inv_update_kernel", "inv_finish_kernel"), w["inv_flop"], "TFLOP/s", PEAK_X3),
            ("precondition", ("gemm_tn_kernel", "gemm_tn64_kernel"), w["pre_flop"], "TFLOP/s", pre_peak),
            ("refine_residual", ("refine_residual_gemm_tn64_kernel",), w["refine_flop"] / 2, "TFLOP/s",
             PEAK_FP64_MFMA),
            ("refine_correction", ("refine_correction_gemm_tn_kernel",), w["refine_flop"] / 2, "TFLOP/s",
             PEAK_X3),
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


def percentiles(ms_list):
    a = np.asarray(ms_list, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4), "n": int(a.size)}


def timed_calls(fn, reps, warm=3):
    """Runs fn warm + reps times on the current stream, HIP events around each of the
    timed calls; returns their durations in ms."""
    import torch
    for _ in range(warm):
        fn()
    ev = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ev.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def progress(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [x for x in threadpool_info() if x.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"])
    except Exception:  # noqa: BLE001 - threadpoolctl is optional
        pass
    return len(os.sched_getaffinity(0))


def one_thread():
    """Context that limits BLAS to one thread (threadpoolctl)."""
    from threadpoolctl import threadpool_limits
    return threadpool_limits(limits=1, user_api="blas")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on one full step of the bench's own inputs
# ---------------------------------------------------------------------------

def cpu_baseline(layers, bns, host_in):
    """Times the fp64 oracle on one complete step of the workload (every layer's factors,
    damped inverses, preconditioned gradient and update; every BatchNorm layer's
    diagonal Fisher and update) on host copies of the inputs the GPU step used."""
    import oracle
    s = float(np.float32(np.sqrt(1e-3)))
    t = {"factors": 0.0, "invert": 0.0, "precondition": 0.0, "bn": 0.0}
    for l, layer in enumerate(layers):
        if l % 10 == 0:
            progress(f"oracle step: layer {l} of {len(layers)}")
        t0 = time.perf_counter()
        A, G = oracle.conv_factors(host_in["act"][l], host_in["gout"][l], layer.kh, layer.kw, layer.sh,
                                   layer.sw, layer.ph, layer.pw, layer.bias)
        t1 = time.perf_counter()
        Ai, _ = oracle.damped_inverse(A, s)
        Gi, _ = oracle.damped_inverse(G, s)
        t2 = time.perf_counter()
        oracle.sgd_update(host_in["w"][l], oracle.precondition(Gi, host_in["grad"][l], Ai), LR)
        t3 = time.perf_counter()
        t["factors"] += t1 - t0
        t["invert"] += t2 - t1
        t["precondition"] += t3 - t2
        del A, G, Ai, Gi
    for i in range(len(bns)):
        t0 = time.perf_counter()
        oracle.sgd_update(host_in["bn_w"][i], oracle.bn_diag_fisher(host_in["xhat"][i], host_in["bgout"][i],
                                                                       1e-3)["precond"], LR)
        t["bn"] += time.perf_counter() - t0
    total = sum(t.values())
    return {"value": round(1.0 / total, 5), "unit": "steps/s", "cores": blas_threads(), "kind": "oracle",
            "cpu_model": cpu_model(), "seconds_per_step": round(total, 3),
            "stage_seconds": {k: round(v, 3) for k, v in t.items()},
            "sample": (f"one full step of the fp64 oracle (all {len(layers)} K-FAC layers: factors, damped "
                       f"inverses, preconditioned gradient and update; all {len(bns)} BatchNorm layers) on host "
                       f"copies of the GPU step's inputs, NumPy BLAS on {blas_threads()} threads")}


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


def stale_schedule(batch=128, steps=100):
    """Stale curvature at batch `batch`: every 10th step refreshes the factors (EMA 0.95,
    the first refresh overwrites) and the inverses; every step preconditions one of ten
    fp16 N(0,1e-2) gradient sets. Two activation/gradient sets alternate across
    refreshes. Returns amortised steps/s over `steps` steps after one warm-up cycle."""
    import torch
    import fac_second_order_amd as kfac
    dev = torch.device("cuda:0")
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

    steps = steps if steps % 10 == 0 else 100   # whole refresh cycles only
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
    return {"value": round(steps / elapsed, 3), "unit": "steps/s", "steps": steps, "warmup": 10,
            "ms_per_step": round(1e3 * elapsed / steps, 3), "batch_per_gpu": batch, "refresh_every": 10,
            "ema_decay": 0.95, "grad_dtype": "f16"}


def run_stale(args):
    r = stale_schedule(args.batch or 128, args.steps)
    out = {
        "metric": "K-FAC amortised steps/sec (ResNet-50 shapes, batch 128, refresh every 10, EMA 0.95, 1 GPU)",
        "value": r["value"], "unit": "steps/s", "n_gpus": 1, "steps": r["steps"], "warmup": 10,
        "ms_per_step": r["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "resnet50_kfac_stale_schedule", "batch_per_gpu": r["batch_per_gpu"],
                   "refresh_every": 10, "ema_decay": 0.95, "grad_dtype": "f16", "lr": LR},
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
    cap = KfacCapture(model, damping=1e-3, ema_decay=0.95, precond_accum=args.precond_accum,
                      refine_inverse=args.refine_inverse)
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
                   "damping": 1e-3, "lr": 1e-3, "ema_decay": 0.95, "precond_accum": args.precond_accum,
                   "refine_inverse": args.refine_inverse, "kfac_ms_per_step": round(kfac_ms, 3),
                   "forward_backward_ms_per_step": round(1e3 * elapsed / args.steps - kfac_ms, 3)},
        "roofline": None, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# the other workloads, as extra keys of the same line
# ---------------------------------------------------------------------------

def run_fc(dev, with_oracle):
    """Fully connected layer, fp32: a[32x64], g[32x16] N(0,1) (seeded), dW = g^T a / 32,
    no bias, damping 1e-3: factors, both damped inverses and G^-1 dW A^-1 per call."""
    import torch
    import fac_second_order_amd as kfac
    seed = synth.config_seed("fc")
    a = synth.normal_f32(synth.layer_rng(seed, 0), (32, 64))
    g = synth.normal_f32(synth.layer_rng(seed, 1), (32, 16))
    dW = (g.astype(np.float64).T @ a.astype(np.float64)) / 32.0
    layer = synth.Layer("fc", 32, 1, 1, 64, 1, 1, 16, 1, 1, 1, 1, 0, 0, 0)
    st = kfac.KfacStep([layer], [], dev, in_dtype=torch.float32)
    da = torch.from_numpy(a.reshape(32, 1, 1, 64)).to(dev)
    dg = torch.from_numpy(g.reshape(32, 1, 1, 16)).to(dev)
    dw = torch.from_numpy(dW.astype(np.float32)).to(dev)

    def chain():
        st.factors([da], [dg])
        st.invert()
        st.precondition([dw])

    ms = timed_calls(chain, 50)
    out = {"gpu_us_per_call": percentiles([1e3 * x for x in ms]),
           "what": "factors + unpack + 2 damped inverses + G^-1 dW A^-1 (5 library calls)"}
    if with_oracle:
        import oracle
        s = float(np.float32(np.sqrt(1e-3)))

        def ref():
            A, G = oracle.conv_factors(a.reshape(32, 1, 1, 64), g.reshape(32, 1, 1, 16), 1, 1, 1, 1, 0, 0, 0)
            return oracle.precondition(oracle.damped_inverse(G, s)[0], dW, oracle.damped_inverse(A, s)[0])

        P = ref()
        for key, ctx in (("oracle_us_1thread", one_thread), ("oracle_us_all_threads", None)):
            reps = []
            for _ in range(5):
                if ctx:
                    with ctx():
                        t0 = time.perf_counter(); ref(); reps.append(time.perf_counter() - t0)  # noqa: E702
                else:
                    t0 = time.perf_counter(); ref(); reps.append(time.perf_counter() - t0)  # noqa: E702
            out[key] = round(1e6 * float(np.median(reps)), 1)
        out["p_relF_vs_oracle"] = float(np.linalg.norm(st.out[0].cpu().numpy() - P) / np.linalg.norm(P))
    return out


def run_conv3x3(dev, with_oracle):
    """One 3x3 convolution 64->64, stride 1, pad 1, 56x56, batch 32 (R = 100,352 patch rows,
    A 577 x 577, G 64 x 64): activations fp16(ReLU(N(0,1))), output gradients
    fp16(N(0,1e-2)), dW the layer's true weight gradient; damping 1e-3."""
    import torch
    import fac_second_order_amd as kfac
    layer = synth.Layer("s2b0.c2", 32, 56, 56, 64, 56, 56, 64, 3, 3, 1, 1, 1, 1, 1)
    seed = synth.config_seed("conv3x3")
    act = synth.relu_normal_f16(synth.layer_rng(seed, 0), layer.act_shape)
    gout = synth.normal_f16(synth.layer_rng(seed, 1), layer.gout_shape, 0.1)
    da, dg = torch.from_numpy(act).to(dev), torch.from_numpy(gout).to(dev)
    st = kfac.KfacStep([layer], [], dev)
    # dW = (1/N) Gamma^T X, from the library's own inputs (a plain matrix product of the
    # gradient and the patch rows; it is an input of the preconditioning, not timed)
    X = torch.nn.functional.unfold(da.permute(0, 3, 1, 2).float(), 3, padding=1)       # [N, 64*9, HW] (c, kh, kw)
    X = X.view(32, 64, 9, 3136).permute(0, 3, 2, 1).reshape(-1, 576)                   # rows, (kh, kw, c)
    X = torch.cat([X, torch.ones(X.shape[0], 1, device=dev)], 1)
    dW = (dg.float().reshape(-1, 64).t() @ X) / 32.0
    del X
    rows = layer.rows
    flop_a, flop_g = rows * 577 * 578, rows * 64 * 65
    f_ms = timed_calls(lambda: st.factors([da], [dg]), 50)
    i_ms = timed_calls(st.invert, 50)
    p_ms = timed_calls(lambda: st.precondition([dW]), 50)
    c_ms = timed_calls(lambda: (st.factors([da], [dg]), st.invert(), st.precondition([dW])), 50)
    fmed = float(np.median(f_ms))
    rate = (flop_a + flop_g) / (fmed * 1e-3) / 1e12
    out = {"factors_us": percentiles([1e3 * x for x in f_ms]),
           "factors_tflops": round(rate, 1), "factors_frac_fp16_peak": round(rate / PEAK_FP16_MFMA, 4),
           "factors_algorithmic_gflop": round((flop_a + flop_g) / 1e9, 3),
           "invert_us": percentiles([1e3 * x for x in i_ms]),
           "precondition_us": percentiles([1e3 * x for x in p_ms]),
           "chain_us": percentiles([1e3 * x for x in c_ms]),
           "what": "factors (A 577, G 64) / unpack + 2 damped inverses / G^-1 dW A^-1 / all three"}
    if with_oracle:
        import oracle
        s = float(np.float32(np.sqrt(1e-3)))
        dWh = dW.cpu().numpy().astype(np.float64)

        def ref():
            A, G = oracle.conv_factors(act, gout, 3, 3, 1, 1, 1, 1, 1)
            return oracle.precondition(oracle.damped_inverse(G, s)[0], dWh, oracle.damped_inverse(A, s)[0])

        t0 = time.perf_counter()
        P = ref()
        out["oracle_s_all_threads"] = round(time.perf_counter() - t0, 3)
        with one_thread():
            t0 = time.perf_counter()
            ref()
            out["oracle_s_1thread"] = round(time.perf_counter() - t0, 3)
        out["p_relF_vs_oracle"] = float(np.linalg.norm(st.out[0].cpu().numpy() - P) / np.linalg.norm(P))
    return out


def stress_factors(dims, kappa, dev, seed):
    """Damped-Gram stress factors on the device, one per order in `dims`: X = Z diag(s),
    Z N(0,1) with 4n rows, s log-spaced from 1 to 1e-3, F = X^T X / (4n) made exactly
    symmetric and scaled so that cond(F + 1e-3 I) <= kappa (largest eigenvalue by power
    iteration, rounded up)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = []
    for n in dims:
        sig = torch.logspace(0, -3, n, device=dev)
        X = torch.randn(4 * n, n, generator=g, device=dev) * sig
        F = (X.t() @ X) / (4 * n)
        F = 0.5 * (F + F.t())
        v = torch.ones(n, 1, device=dev)
        for _ in range(60):
            v = F @ v
            lam = v.norm()
            v = v / lam
        F *= (kappa - 1.0) * 1e-3 / (float(lam) * 1.01)
        out.append(F.contiguous())
        del X
    return out


def run_invert_stress(dev, with_oracle):
    """Batched damped inversion of one stress factor per ResNet-50 factor (108 matrices,
    orders 64 ... 4609), shift 1e-3, at cond <= 1e2, 1e3, 1e4: time of the whole batch per
    condition number, time per size class (a call with that class's matrices only) at
    1e4, and the error against the oracle, which inverts the same fp32 matrices, for
    five sizes at each condition number."""
    import torch
    import fac_second_order_amd as kfac
    layers = synth.conv_layers(32)
    dims = [l.d_a for l in layers] + [l.d_g for l in layers]
    out = {"matrices": len(dims), "sum_n3_tflop": round(sum(n ** 3 for n in dims) / 1e12, 4), "by_kappa": {}}
    err_dims = (64, 577, 1025, 2049, 4609)
    for kappa in (1e2, 1e3, 1e4):
        mats = stress_factors(dims, kappa, dev, seed=int(np.log10(kappa)) + 400)
        inv = [torch.empty_like(m) for m in mats]
        info = torch.zeros(len(dims), dtype=torch.int32, device=dev)
        ws = torch.empty(kfac.kfac_invert_workspace(dims) + 256, dtype=torch.uint8, device=dev)
        ms = timed_calls(lambda: kfac.kfac_invert(dims, mats, inv, [1e-3] * len(dims), info, workspace=ws), 10)
        if int(info.abs().sum()) != 0:
            raise RuntimeError("breakdown in the stress inversion")
        med = float(np.median(ms))
        rec = {"batch_ms": percentiles(ms),
               "tflops": round(sum(n ** 3 for n in dims) / (med * 1e-3) / 1e12, 2)}
        rec["frac_peak"] = round(rec["tflops"] / PEAK_X3, 4)
        if kappa == 1e4:
            per = {}
            for n in sorted(set(dims)):
                idx = [i for i, d in enumerate(dims) if d == n]
                sub_d = [n] * len(idx)
                sub_m, sub_i = [mats[i] for i in idx], [inv[i] for i in idx]
                t = timed_calls(lambda: kfac.kfac_invert(sub_d, sub_m, sub_i, [1e-3] * len(idx), info,
                                                         workspace=ws), 10)
                per[str(n)] = {"count": len(idx), "ms": round(float(np.median(t)), 4)}
            rec["per_size_class_ms"] = per
        if with_oracle:
            import oracle
            errs = {}
            for n in err_dims:
                i = dims.index(n)
                F = mats[i].cpu().numpy()
                ref, _ = oracle.damped_inverse(F, 1e-3)
                errs[str(n)] = float(np.linalg.norm(inv[i].cpu().numpy() - ref) / np.linalg.norm(ref))
            rec["relF_vs_oracle"] = errs
        out["by_kappa"][f"{kappa:.0e}"] = rec
        del mats, inv
        torch.cuda.empty_cache()
    return out


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
    group = kfac.kfac_invert_schedule()[1]
    w = work(layers, bns, group)
    progress("drawing inputs")
    act, gout, grads, xhat, bgout = make_inputs(layers, bns, dev)
    weights, bn_params = make_params(layers, bns, dev)
    st = kfac.KfacStep(layers, bns, dev, precond_accum=args.precond_accum, refine_inverse=args.refine_inverse,
                       side_stream=not args.no_side_stream)
    host_in = None
    if not args.no_cpu_baseline:   # the oracle's copy of the very inputs of the timed steps
        host_in = {"act": [a.cpu().numpy() for a in act], "gout": [g.cpu().numpy() for g in gout],
                   "grad": [g.cpu().numpy() for g in grads], "xhat": [x.cpu().numpy() for x in xhat],
                   "bgout": [g.cpu().numpy() for g in bgout], "w": [x.cpu().numpy() for x in weights],
                   "bn_w": [x.cpu().numpy() for x in bn_params]}

    def step():
        st.step(act, gout, grads, xhat, bgout, weights=weights, bn_params=bn_params, lr=LR)

    progress(f"warm-up {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if int(st.info.abs().sum()) != 0:
        raise RuntimeError("Cholesky breakdown on a damped factor: " + str(st.info.tolist()))

    timing = not args.no_kernel_timing
    kern, dominant, top = {}, None, None
    if timing:
        # breakdown pass (untimed): every launch bracketed by events, over two steps of
        # the one-stream schedule, so that a launch's time is its own and not time spent
        # waiting behind the other stream's work
        bst = st if not st.side else kfac.KfacStep(layers, bns, dev, precond_accum=args.precond_accum,
                                                   refine_inverse=args.refine_inverse, side_stream=False)
        bst.step(act, gout, grads, xhat, bgout, weights=weights, bn_params=bn_params, lr=LR)
        torch.cuda.synchronize()
        kfac.kfac_timing_reset()
        kfac.kfac_timing_only(-1)
        kfac.kfac_timing_enable(True)
        for _ in range(2):
            bst.step(act, gout, grads, xhat, bgout, weights=weights, bn_params=bn_params, lr=LR)
        torch.cuda.synchronize()
        kfac.kfac_timing_enable(False)
        for i in range(kfac.kfac_timing_kernels()):
            ms, n = kfac.kfac_timing_read(i)
            if n:
                kern[kfac.kfac_kernel_name(i)] = (ms / 2, n // 2)
        kfac.kfac_timing_reset()
        del bst
        torch.cuda.empty_cache()
        ids = range(kfac.kfac_timing_kernels())
        by_time = lambda i: kern.get(kfac.kfac_kernel_name(i), (0.0, 0))[0]  # noqa: E731
        top = kfac.kfac_kernel_name(max(ids, key=by_time))
        # the roofline kernel: the largest one with an algorithmic work model (the
        # pivot and panel launches are latency-bound steps of the sweep and have none)
        dominant = max((i for i in ids if kfac.kfac_kernel_name(i) in MODELLED), key=by_time)
        # timed region: events around the dominant kernel's launches only
        kfac.kfac_timing_only(dominant)
        kfac.kfac_timing_enable(True)
    progress(f"timing {args.steps} steps")
    step_ev = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step()
        b.record()
        step_ev.append((a, b))
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    live = None
    if timing:
        kfac.kfac_timing_enable(False)
        live = (kfac.kfac_kernel_name(dominant),) + tuple(kfac.kfac_timing_read(dominant))
        kfac.kfac_timing_reset()
        kfac.kfac_timing_only(-1)
    step_ms = [x.elapsed_time(y) for x, y in step_ev]

    ms_step = 1e3 * elapsed / args.steps
    value = args.steps / elapsed

    roofline = None
    if live:
        name, ms, n = live  # summed over the timed steps, measured in the timed region
        per_launch = {  # algorithmic work of all the kernel's launches in the timed steps, and its bound
            "inv_update_kernel": (w["update_flop"] * args.steps, "mfma", PEAK_X3),
            "syrk_tile_kernel": (w["syrk_flop"] * args.steps, "mfma", PEAK_FP16_MFMA),
            "gemm_tn_kernel": (w["pre_flop"] * args.steps, "mfma", PEAK_X3),
            "gemm_tn64_kernel": (w["pre_flop"] * args.steps, "mfma", PEAK_FP64_MFMA),
            "refine_residual_gemm_tn64_kernel": (w["refine_flop"] / 2 * args.steps, "mfma", PEAK_FP64_MFMA),
            "refine_correction_gemm_tn_kernel": (w["refine_flop"] / 2 * args.steps, "mfma", PEAK_X3),
        }
        assert set(per_launch) | {"bn_partial_kernel", "unpack_kernel"} == MODELLED
        if name in per_launch:
            total_work, bound, peak = per_launch[name]
            achieved = total_work / (ms * 1e-3) / 1e12      # = per-launch work / average duration
            roofline = {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                        "frac": round(achieved / peak, 4), "traffic": measured_traffic(name, bool(st.side), group), "kernel": name,
                        "launches": n, "avg_launch_us": round(1e3 * ms / n, 2),
                        "algorithmic_per_launch": total_work / n}
            if peak == PEAK_X3:
                roofline["peak_basis"] = "bf16 MFMA peak / 6: each fp32 product is six bf16 MFMA products"
                roofline["frac_fp32_mfma_peak"] = round(achieved / PEAK_FP32_MFMA, 4)
        if roofline and top != name:
            roofline["largest_kernel"] = top
        elif name in ("bn_partial_kernel", "unpack_kernel"):
            b = w["bn_bytes"] if name == "bn_partial_kernel" else w["pack_bytes"]
            achieved = b * args.steps / (ms * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM, "unit": "GB/s",
                        "frac": round(achieved / PEAK_HBM, 4), "traffic": None, "kernel": name,
                        "launches": n, "avg_launch_us": round(1e3 * ms / n, 2),
                        "algorithmic_per_launch": b * args.steps / n}

    if args.copy_calibration > 0:
        nbytes = int(args.copy_calibration * (1 << 30))
        a = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    side_stream = bool(st.side)
    extra = {}
    if not args.no_extra_configs:
        with_oracle = not args.no_cpu_baseline
        del st
        torch.cuda.empty_cache()
        progress("fc layer (fp32)")
        extra["fc_fp32"] = run_fc(dev, with_oracle)
        progress("3x3 convolution 64->64 at 56x56, batch 32")
        extra["conv3x3_64_b32"] = run_conv3x3(dev, with_oracle)
        progress("inversion stress set (108 factors, cond 1e2 / 1e3 / 1e4)")
        extra["invert_stress"] = run_invert_stress(dev, with_oracle)
        torch.cuda.empty_cache()
        progress("stale-curvature schedule, batch 128, 100 steps")
        extra["stale_schedule_b128"] = stale_schedule(128, 100)

    cpu = None
    if host_in is not None:
        progress("oracle on one full step (CPU)")
        cpu = cpu_baseline(layers, bns, host_in)

    out = {
        "metric": "K-FAC steps/sec (ResNet-50 shapes, batch 32, 1 GPU); TFLOP/s vs MFMA peak",
        "value": round(value, 3), "unit": "steps/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "step_ms_events": percentiles(step_ms), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "resnet50_kfac_step", "batch_per_gpu": args.batch,
                   "kfac_layers": len(layers), "factors": 2 * len(layers), "bn_layers": len(bns),
                   "damping": 1e-3, "lr": LR, "precond_accum": args.precond_accum, "refine_inverse": args.refine_inverse,
                   "side_stream": side_stream, "inputs": "fp16 ReLU(N(0,1)) activations, fp16 N(0,1) "
                   "output and BN gradients, fp32 N(0,1e-2) weight gradients, fp32 N(0,2.5e-3) weights"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels_ms_per_step": {k: round(v[0], 4) for k, v in
                                sorted(kern.items(), key=lambda kv: -kv[1][0])},
        "stage_rates": stage_rates(kern, w, args.precond_accum) if kern else None,
        "step_tflop": round((w["syrk_flop"] + w["inv_flop"] + w["pre_flop"]) / 1e12, 4),
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
