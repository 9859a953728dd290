"""Benchmark: AlexNet training step (forward, loss, backward, SGD) at batch 128
on one MI355X, bf16 with fp32 accumulation and fp32 master weights, synthetic
inputs resident in HBM.

Prints one JSON line.  `value` is training images/s over the timed steps.
Beside it: the forward pass alone at batch 128 (single tower and two-tower),
per-kernel MFMA / HBM fractions from HIP events recorded around each kernel
(one untimed diagnostic pass without the side stream, so that each kernel has
the GPU to itself), the roofline figure of the dominant kernel (the longest
one on the step's main stream, i.e. not one of the conv weight gradients that
run beside it on the side stream) measured with HIP events inside the timed
region, and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E

CONV = {  # name: (Cin, Cout, k, Ho, grouped)
    "CONV1": (3, 96, 11, 55, False), "CONV2": (96, 256, 5, 27, True), "CONV3": (256, 384, 3, 13, False),
    "CONV4": (384, 384, 3, 13, True), "CONV5": (384, 256, 3, 13, True),
}
FC = {"FC6": (9216, 4096), "FC7": (4096, 4096), "FC8": (4096, 1000)}


def conv_flops(name, n, groups):
    cin, cout, k, ho, grouped = CONV[name]
    g = groups if grouped else 1
    return 2.0 * cout * (cin // g) * k * k * n * ho * ho


def conv_wcount(name, groups):
    cin, cout, k, _, grouped = CONV[name]
    return cout * (cin // (groups if grouped else 1)) * k * k


def kernel_work(kt, n, groups, train=True):
    """Algorithmic work of one launch: ("mfma", FLOP) or ("hbm", bytes).
    Bytes count each input read once and each output written once (bf16
    activations, uint8 argmax, fp32 optimizer state)."""
    e = 2
    layer, _, op = kt.partition("_")
    if layer.startswith("CONV") and op in ("FWD", "WGRAD", "DGRAD"):
        return "mfma", conv_flops(layer, n, groups)
    if kt.startswith("FC"):
        fin, fout = FC[layer]
        # weight streaming bound at this batch: weights + activations once
        if op == "FWD":
            return "hbm", e * (fin * fout + n * fin + n * fout)
        if op == "DGRAD":
            return "hbm", e * (fin * fout + n * fout + n * fin)
        # WGRAD with the SGD update fused: activations in; fp32 w, v in and out; bf16 w out
        return "hbm", e * (n * fout + n * fin) + 18 * fin * fout
    act = {"55x96": n * 55 * 55 * 96, "27x96": n * 27 * 27 * 96, "27x256": n * 27 * 27 * 256,
           "13x256": n * 13 * 13 * 256, "6x256": n * 6 * 6 * 256}
    table = {
        # layer-1 input staging, and in the same launch the weight re-layouts:
        # each OIHW source read once; the layer-1 block layout, the forward copies
        # of conv2..5 and, for a training step, their data-gradient copies written
        "S2D": e * (n * 3 * 227 * 227 + n * 57 * 57 * 48 + 96 * 3 * 11 * 11 + 96 * 432
                    + (3 if train else 2) * sum(conv_wcount(c, groups) for c in CONV if c != "CONV1")),
        # LRN + max-pool fused: LRN input read once, pooled values and argmax written
        "LRNPOOL1_FWD": e * act["55x96"] + (e + 1) * act["27x96"],
        "LRNPOOL2_FWD": e * act["27x256"] + (e + 1) * act["13x256"],
        # pool, LRN and ReLU backward fused: pooled gradient, argmax and LRN input
        # read, da written, and (training) da's fp32 column sums per row
        "POOLLRN1_BWD": (e + 1) * act["27x96"] + 2 * e * act["55x96"] + (4 * n * 55 * 96 if train else 0),
        "POOLLRN2_BWD": (e + 1) * act["13x256"] + 2 * e * act["27x256"] + (4 * n * 27 * 256 if train else 0),
        "POOL5_FWD": e * act["13x256"] + (e + 1) * act["6x256"],
        "POOL5_BWD": (e + 1) * act["6x256"] + 2 * e * act["13x256"],
        # bias gradients of layers 3-8: their output gradients read once (the
        # block partials and the 22 B per bias of the update are below 0.2%)
        "BIAS": e * (2 * n * 13 * 13 * 384 + act["13x256"] + n * (2 * 4096 + 1000)),
        # layers 1 and 2 from their per-row fp32 sums
        "BIAS12": 4 * n * (55 * 96 + 27 * 256),
    }
    return "hbm", float(table[kt])


def kernel_source_sha256():
    """sha256 over the HIP kernel sources (name + bytes, sorted): the identity
    of the build that HBM counters in profiles/ were taken on."""
    import hashlib
    d = os.path.join(ROOT, "deep_cnn_image_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".cpp", ".h")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic.json (two rocprofv3
    --pmc runs, FETCH_SIZE and WRITE_SIZE, scaled by a plain copy), or None if
    the counters were taken on other kernel sources or do not cover `kernel`."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    t = json.load(open(path))
    k = t.get("kernels", {}).get(kernel)
    if k is None or t.get("source_sha256") != kernel_source_sha256():
        return None
    return int(k["read_bytes"] + k["write_bytes"])


def cpu_model():
    """The host CPU's model name (what lscpu reports), from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=64, help="images in the CPU-oracle sample")
    ap.add_argument("--train-only", action="store_true",
                    help="time the training step only (for short profiled runs) and print its kernels")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--cache-probe", action="store_true",
                    help="only time a streaming read of FC6's weight-matrix size after the last-level "
                         "cache holds clean or dirty lines, and print that")
    return ap.parse_args()


def cache_probe(dev):
    """Streaming-read time of a 75.5 MB bf16 matrix (the size of FC6's
    weights, 4096 x 9216) by a plain reduction, after a 400 MB read has filled
    the last-level cache with clean lines and after a 400 MB write has filled it
    with dirty ones, and with the matrix itself just read (cached).  Medians of
    10 reps with torch events, whose span includes a cache write-back fence of a
    few microseconds; the kernel trace of the same run has the kernel alone."""
    import torch
    m = torch.ones(4096, 9216, dtype=torch.bfloat16, device=dev)
    big = torch.empty(100 << 20, dtype=torch.float32, device=dev)
    res = {}
    for state in ("after_400MB_read", "after_400MB_write", "after_reading_itself"):
        ts = []
        for _ in range(10):
            if state == "after_400MB_read":
                big.sum()
            elif state == "after_400MB_write":
                big.fill_(1.0)
            else:
                big.fill_(1.0)
                m.sum(dtype=torch.float32)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            m.sum(dtype=torch.float32)
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        med = sorted(ts)[len(ts) // 2]
        res[state] = {"us": round(med, 2), "GB/s": round(m.numel() * 2 / med / 1e3, 1)}
    return {"cache_probe": res, "bytes": m.numel() * 2}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU "
              "data parallelism is not implemented.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from deep_cnn_image_amd import binding as B
    from deep_cnn_image_amd import inputs as I
    from deep_cnn_image_amd.session import Session, SideStream, Timer, stream_handle, to_device

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.cache_probe:
        print(json.dumps(cache_probe(dev)))
        return
    B.lib()
    h = I.TRAIN_HYPER

    def copy_calibration():
        # a plain 512 MiB device copy, the reference for the HBM byte counters
        src = torch.ones(256 << 20, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        return {"read": src.numel() * 2, "write": dst.numel() * 2}

    def new_events(k):
        # start/stop pairs without the system-scope fence of a default event,
        # which would add a cache write-back to every timed span
        return [Timer() for _ in range(k)]

    # ---------------------------------------------------------------- training step
    syn = I.workload_inputs("train_batch128")
    n = syn.x.shape[0]
    sess = Session(n, 1, B.BF16, B.MODE_TRAIN, dev)
    master = []
    for w, b in zip(syn.master_w, syn.biases):
        master += [torch.from_numpy(w).to(dev), torch.from_numpy(b).to(dev)]
    mom = [torch.zeros_like(m) for m in master]
    work = [torch.empty(m.shape, dtype=torch.bfloat16, device=dev) for m in master]
    B.alexnet_cast_weights(sess.cfg, master, work, stream_handle())
    x = to_device(syn.x, B.BF16, dev)
    labels = torch.from_numpy(syn.labels).to(dev)
    loss = torch.zeros(1, dtype=torch.float32, device=dev)
    stream = stream_handle()
    # the caller's second stream: the weight gradients run on it beside the
    # data-gradient chain (alexnet_train_step_ex)
    side = SideStream(dev)

    def train(i, timers=(), serial=False):
        # serial: no side stream, so that every timed kernel has the GPU to itself
        B.alexnet_train_step_ex(sess.cfg, master, mom, work, x, None, 0, 0, labels, h["lr"], h["momentum"],
                                h["weight_decay"], h["dropout_seed"], i, loss, None, sess.ws, sess.ws_bytes,
                                stream, 0 if serial else side.handle, () if serial else side.event_handles,
                                list(timers))

    step = 0
    for _ in range(args.warmup):
        train(step); step += 1
    torch.cuda.synchronize()

    # diagnostic pass (untimed, serial): every kernel bracketed by its own events
    diag_steps = 3
    names = [k for k in B.KERNELS if k != "RGB_PCA"]   # every kernel of the training step
    evs = [new_events(len(names)) for _ in range(diag_steps)]
    for d in range(diag_steps):
        train(step, [(B.KT[nm], evs[d][j].start, evs[d][j].stop)
                     for j, nm in enumerate(names)], serial=True)
        step += 1
    torch.cuda.synchronize()
    per_kernel = {}
    for j, nm in enumerate(names):
        ms = [evs[d][j].elapsed_ms() for d in range(diag_steps)]
        if min(ms) > 0:
            per_kernel[nm] = sum(ms) / len(ms)
    # the dominant kernel: the longest of those on the step's main stream.  The
    # conv weight gradients run on the side stream beside that chain, so their
    # time inside the real step includes the GPU they share; their own rates
    # are the isolated ones in kernels_train.
    on_side = {f"CONV{i}_WGRAD" for i in range(1, 6)}
    dominant = max((nm for nm in per_kernel if nm not in on_side), key=per_kernel.get)

    # timed region: events only around the dominant kernel, on the main stream
    # (the order of the step is the same as without them)
    tev = new_events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        train(step, [(B.KT[dominant], tev[i].start, tev[i].stop)])
        step += 1
    torch.cuda.synchronize()
    train_s = (time.perf_counter() - t0) / args.steps
    dom_ms = sum(t.elapsed_ms() for t in tev) / args.steps
    final_loss = float(loss.item())
    if args.train_only:
        # the training step alone (short runs under a profiler): its per-kernel
        # fractions and the dominant kernel's figure, nothing else
        out = {"ms_per_step": round(train_s * 1e3, 4), "value": round(n / train_s, 1), "unit": "images/s",
               "loss": round(final_loss, 5), "dominant": dominant, "dominant_us": round(dom_ms * 1e3, 2),
               "kernels_train_us": {nm: round(ms * 1e3, 2) for nm, ms in per_kernel.items()}}
        if args.copy_calibration:
            out["copy_calibration_bytes"] = copy_calibration()
        print(json.dumps(out), flush=True)
        return

    # ---------------------------------------------------------------- augmented training step
    # Same step fed by the section-4.1 augmentation: 227x227 patches of 256x256
    # sources with mirror flags and PCA colour shifts, read by the layer-1
    # staging.  The principal components come from alexnet_rgb_pca on the batch.
    aug_in = I.augment_inputs(5, n)
    src = to_device(aug_in.src, B.BF16, dev)
    crop = torch.from_numpy(aug_in.crop).to(dev)
    alpha = torch.from_numpy(aug_in.alpha).to(dev)
    eigval = torch.empty(3, dtype=torch.float32, device=dev)
    eigvec = torch.empty(9, dtype=torch.float32, device=dev)
    pca_ws_bytes = B.alexnet_rgb_pca_workspace_bytes()
    pca_ws = torch.empty(pca_ws_bytes, dtype=torch.uint8, device=dev)
    hs, ws_ = aug_in.src.shape[2], aug_in.src.shape[3]

    def pca(timers=()):
        B.alexnet_rgb_pca_timed(sess.cfg, src, n, hs, ws_, eigval, eigvec, pca_ws, pca_ws_bytes, stream,
                                list(timers))

    for _ in range(args.warmup):
        pca()
    pev = new_events(args.steps)
    for i in range(args.steps):
        pca([(B.KT["RGB_PCA"], pev[i].start, pev[i].stop)])
    torch.cuda.synchronize()
    pca_ms = sum(t.elapsed_ms() for t in pev) / args.steps
    aug = B.augment(crop, alpha, eigval, eigvec)

    def train_aug(i, timers=()):
        B.alexnet_train_step_ex(sess.cfg, master, mom, work, src, aug, hs, ws_, labels, h["lr"], h["momentum"],
                                h["weight_decay"], h["dropout_seed"], i, loss, None, sess.ws, sess.ws_bytes,
                                stream, side.handle, side.event_handles, list(timers))

    for _ in range(args.warmup):
        train_aug(step); step += 1
    sev = new_events(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        train_aug(step, [(B.KT["S2D"], sev[i].start, sev[i].stop)])
        step += 1
    torch.cuda.synchronize()
    aug_s = (time.perf_counter() - t0) / args.steps
    aug_stage_ms = sum(t.elapsed_ms() for t in sev) / args.steps
    del sess, src, pca_ws

    # ---------------------------------------------------------------- forward passes
    fwd = {}
    fwd_kernels = {}
    for wl, key in (("bf16_batch128", "single"), ("two_tower_batch128", "two_tower")):
        s2 = I.workload_inputs(wl)
        n2 = s2.x.shape[0]
        fs = Session(n2, s2.groups, B.BF16, B.MODE_FORWARD, dev)
        params = fs.upload_params(s2.weights, s2.biases)
        x2 = to_device(s2.x, B.BF16, dev)
        probs = torch.empty((n2, 1000), dtype=torch.float32, device=dev)

        def fwd_call(timers=()):
            B.alexnet_forward_timed(fs.cfg, params, x2, probs, fs.ws, fs.ws_bytes, stream, list(timers))

        for _ in range(args.warmup):
            fwd_call()
        fnames = [nm for nm in names if nm.endswith("_FWD") or nm == "S2D"]
        fev = new_events(len(fnames))
        fwd_call([(B.KT[nm], fev[j].start, fev[j].stop) for j, nm in enumerate(fnames)])
        torch.cuda.synchronize()
        fwd_kernels[key] = {nm: fev[j].elapsed_ms() for j, nm in enumerate(fnames)}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fwd_call()
        torch.cuda.synchronize()
        fwd[key] = (time.perf_counter() - t0) / args.steps
        del fs

    # ---------------------------------------------------------------- ten-view inference
    # 256 sources of 3x256x256; each call runs the forward pass on the 2560
    # views (four corners and the centre, each also mirrored) and averages
    # the ten softmax outputs per source.
    s5 = I.workload_inputs("tenview_256_sources")
    n5 = s5.x.shape[0]
    ts = Session(n5, 1, B.BF16, B.MODE_TENVIEW, dev)
    params5 = ts.upload_params(s5.weights, s5.biases)
    src5 = to_device(s5.x, B.BF16, dev)
    probs5 = torch.empty((n5, 1000), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        B.alexnet_forward_tenview(ts.cfg, params5, src5, probs5, ts.ws, ts.ws_bytes, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        B.alexnet_forward_tenview(ts.cfg, params5, src5, probs5, ts.ws, ts.ws_bytes, stream)
    torch.cuda.synchronize()
    tenview_s = (time.perf_counter() - t0) / args.steps
    del ts, src5, params5

    # ---------------------------------------------------------------- batch-1 fp32 forward (latency)
    # One image, fp32 weights and activations: each call is waited for on
    # its own, so the figure is the latency of one call, launches included.
    s1 = I.workload_inputs("fp32_batch1")
    ls = Session(1, 1, B.F32, B.MODE_FORWARD, dev)
    params1 = ls.upload_params(s1.weights, s1.biases)
    x1 = to_device(s1.x, B.F32, dev)
    probs1 = torch.empty((1, 1000), dtype=torch.float32, device=dev)
    for _ in range(args.warmup):
        B.alexnet_forward(ls.cfg, params1, x1, probs1, ls.ws, ls.ws_bytes, stream)
    torch.cuda.synchronize()
    lat = []
    for _ in range(max(args.steps, 5)):
        t0 = time.perf_counter()
        B.alexnet_forward(ls.cfg, params1, x1, probs1, ls.ws, ls.ws_bytes, stream)
        torch.cuda.synchronize()
        lat.append(time.perf_counter() - t0)
    lat_s = float(np.median(lat))
    # the same call captured once into a HIP graph and replayed: the launch
    # work of its ~30 kernels is done once at capture, not per call
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.alexnet_forward(ls.cfg, params1, x1, probs1, ls.ws, ls.ws_bytes, stream_handle())
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    glat = []
    for _ in range(max(args.steps, 5)):
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        glat.append(time.perf_counter() - t0)
    glat_s = float(np.median(glat))
    del graph, ls, params1

    # ---------------------------------------------------------------- fractions of roofline
    def frac(nm, ms, groups=1, train=True):
        kind, work = kernel_work(nm, n, groups, train)
        if kind == "mfma":
            return {"bound": "mfma", "TFLOP/s": round(work / (ms * 1e-3) / 1e12, 1),
                    "frac": round(work / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "us": round(ms * 1e3, 2)}
        return {"bound": "hbm", "GB/s": round(work / (ms * 1e-3) / 1e9, 1),
                "frac": round(work / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "us": round(ms * 1e3, 2)}

    def frac_pca(ms):
        # one read of every source pixel; the 9 fp64 moments per workgroup are negligible
        b = n * 3 * hs * ws_ * 2
        return {"bound": "hbm", "GB/s": round(b / (ms * 1e-3) / 1e9, 1),
                "frac": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "us": round(ms * 1e3, 2)}

    kernels_train = {nm: frac(nm, ms) for nm, ms in per_kernel.items()}
    conv_fwd_flops = sum(conv_flops(c, n, 1) for c in CONV)
    conv_fwd_ms = sum(fwd_kernels["single"][c + "_FWD"] for c in CONV)
    conv_train_flops = conv_fwd_flops * 3 - conv_flops("CONV1", n, 1)   # fwd + wgrad + dgrad (no conv1 dgrad)
    conv_train_ms = sum(ms for nm, ms in per_kernel.items() if nm.startswith("CONV"))

    kind, work = kernel_work(dominant, n, 1)
    achieved = work / (dom_ms * 1e-3) / (1e12 if kind == "mfma" else 1e9)
    peak = PEAK_BF16_TFLOPS if kind == "mfma" else PEAK_HBM_GBS
    roofline = {"kernel": dominant, "bound": kind, "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s" if kind == "mfma" else "GB/s", "frac": round(achieved / peak, 4),
                "traffic": measured_traffic(dominant), "avg_launch_us": round(dom_ms * 1e3, 2),
                "work_per_launch": work}

    rec = {
        "metric": "images/s AlexNet bs128 fwd and train step; conv MFMA % of bf16 peak",
        "value": round(n / train_s, 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(train_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "AlexNet training step (forward, cross-entropy, backward, SGD momentum "
                               "0.9 wd 5e-4), batch 128, single tower, 3x227x227 N(0,1) images, "
                               "bf16 activations/weights with fp32 accumulate and fp32 master weights",
                   "global_batch": n},
        "loss": round(final_loss, 5),
        "forward": {"images_per_s": round(n / fwd["single"], 1), "ms": round(fwd["single"] * 1e3, 4),
                    "conv_mfma_frac": round(conv_fwd_flops / (conv_fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)},
        "forward_two_tower": {"images_per_s": round(n / fwd["two_tower"], 1),
                              "ms": round(fwd["two_tower"] * 1e3, 4)},
        "train_conv_mfma_frac": round(conv_train_flops / (conv_train_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "kernels_train": kernels_train,
        "kernels_forward": {nm: frac(nm, ms, train=False) for nm, ms in fwd_kernels["single"].items()},
        "roofline": roofline,
        "train_augmented": {
            "images_per_s": round(n / aug_s, 1), "ms": round(aug_s * 1e3, 4),
            "workload": "the training step on 227x227 patches of 3x256x256 sources (random offsets, mirror "
                        "flags, PCA colour shifts with alpha ~ N(0, 0.1)), staged straight from the sources",
            "staging": frac("S2D", aug_stage_ms)},
        "rgb_pca": dict(frac_pca(pca_ms), images=n, size=f"3x{hs}x{ws_}"),
        "tenview": {"views_per_s": round(10 * n5 / tenview_s, 1), "source_images_per_s": round(n5 / tenview_s, 1),
                    "ms": round(tenview_s * 1e3, 4),
                    "workload": f"{n5} sources of 3x256x256, ten 227x227 views each (bf16, single tower)"},
        "forward_bs1_fp32": {"latency_ms": round(lat_s * 1e3, 4), "images_per_s": round(1.0 / lat_s, 1),
                             "graph_latency_ms": round(glat_s * 1e3, 4),
                             "workload": "one 3x227x227 image, fp32 weights and activations, single tower; "
                                         "median of calls each waited for"},
    }

    if args.copy_calibration:
        rec["copy_calibration_bytes"] = copy_calibration()

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        k = args.cpu_sample
        s3 = I.workload_inputs("train_batch128", batch=k)
        zw = [np.zeros(w.shape) for w in s3.master_w]
        zb = [np.zeros(b.shape) for b in s3.biases]
        t0 = time.perf_counter()
        oracle.alexnet.train_step(s3.weights, s3.biases, s3.master_w, s3.biases, zw, zb, s3.x, s3.labels, 1,
                                  seed=3, step=0, store="bf16")
        cpu_s = time.perf_counter() - t0
        rec["cpu_baseline"] = {"value": round(k / cpu_s, 3), "unit": "images/s", "cores": oracle.num_threads(),
                               "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"one training step (forward, loss, backward, SGD) on {k} images of the "
                                         f"batch-128 workload, float64 direct loops, {cpu_s:.1f} s"}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
