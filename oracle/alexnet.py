"""The AlexNet network, composed from the oracle's per-layer functions.

Test infrastructure only.  The order of operations follows the pages:
paper-graph-ui "Overall Architecture (Layer-by-Layer Specification)" and its
per-layer summary (Conv -> ReLU -> LRN -> MaxPool for layers 1 and 2; Conv ->
ReLU for 3 and 4; Conv -> ReLU -> MaxPool for 5; FC -> ReLU -> Dropout for 6
and 7; FC -> softmax for 8), the fermi.ai ALEXNET_FORWARD / TRAIN_STEP
description (paddings 0/2/1/1/1, 227x227 input, flatten to 9216), the dropout
rule (train: zero with probability 0.5; test: keep all, multiply by 0.5) and
the SGD update in "Training Procedure Details".

Readings where the pages leave a step open (each is listed with its reason in
the design notes): input 227x227; conv paddings 0, 2, 1, 1, 1; the two-tower
net is groups=2 on conv2/conv4/conv5; LRN runs across all channels of the layer
with half-width 2 and alpha not divided by n; pool argmax is the first maximum
of a row-major window scan; flatten in (c, h, w) order; ReLU'(0) = 0; dropout
masks from Philox4x32-10 without rescaling at train time and a 0.5 scale at
test time; loss is the batch mean; weight decay applies to every parameter
tensor, biases included.

Storage precision.  The bf16 workloads define the network with bf16
activations and fp32 accumulation.  With ``store="bf16"`` every tensor that
one layer hands to the next (activations in the forward pass, activation
gradients in the backward pass) is rounded to the nearest bf16 value, ties to
even, straight from float64; the arithmetic inside each layer stays float64.
Max-pool argmaxes and ReLU masks are then decided on the same bf16 values the
network stores.  Weight gradients, logits and probabilities are not rounded.
With ``store=None`` nothing is rounded.
"""
from __future__ import annotations

import numpy as np

from . import lib as L

# (stride, pad, grouped) per conv layer, from the pages' layer list.
CONV_GEOM = ((4, 0, False), (1, 2, True), (1, 1, False), (1, 1, True), (1, 1, True))
LRN = dict(k=2.0, alpha=1e-4, beta=0.75, n=5)
DROPOUT_P = 0.5
TEST_SCALE = 0.5


def _g(groups, grouped):
    return groups if grouped else 1


def round_bf16(a):
    """Nearest bf16 value of each float64 (ties to even), as float64.  Keeps 8
    significant bits by rounding away the low 45 bits of the float64 mantissa
    (normal range only; values here stay far above bf16's subnormal range)."""
    a = np.ascontiguousarray(a, np.float64)
    u = a.view(np.uint64)
    low = np.uint64((1 << 45) - 1)
    r = (u + (low >> np.uint64(1)) + ((u >> np.uint64(45)) & np.uint64(1))) & ~low
    return r.view(np.float64)


def _quant(store):
    if store is None:
        return lambda a: a
    if store == "bf16":
        return round_bf16
    raise ValueError(store)


def forward(weights, biases, x, groups=1, train=False, seed=0, step=0, masks=None, store=None):
    """Forward pass.  Returns a dict holding every intermediate (NCHW / [N, F]).

    weights/biases: 8 arrays each (conv OIHW, FC [out][in]).  In train mode the
    FC6/FC7 outputs are multiplied by the Philox keep-masks of (seed, step), or
    by ``masks`` = (mask6, mask7) when given (rows of a larger batch's masks).
    ``store``: None or "bf16", the storage precision of tensors between layers.
    """
    q = _quant(store)
    t = {}
    n = x.shape[0]
    a = np.asarray(x, np.float64)
    t["x"] = a
    for li in range(5):
        s, p, grouped = CONV_GEOM[li]
        z = L.conv2d(a, weights[li], biases[li], s, p, _g(groups, grouped))
        a = q(L.relu(z))
        t[f"conv{li + 1}"] = a                     # ReLU output
        if li in (0, 1):
            b = q(L.lrn(a, **LRN))
            t[f"lrn{li + 1}"] = b
            a, am = L.maxpool(b, 3, 2)
            t[f"pool{li + 1}"], t[f"arg{li + 1}"] = a, am
        elif li == 4:
            a, am = L.maxpool(a, 3, 2)
            t["pool5"], t["arg5"] = a, am
    h = a.reshape(n, -1)                            # (c, h, w) flatten -> 9216
    t["flat"] = h
    for fi, li in enumerate((5, 6)):
        hz = q(L.relu(L.fc(h, weights[li], biases[li])))
        t[f"fc{li + 1}"] = hz                       # ReLU output before dropout
        if train:
            m = (L.dropout_mask(seed, step, fi, n, hz.shape[1], DROPOUT_P) if masks is None
                 else np.asarray(masks[fi], np.uint8))
            t[f"mask{li + 1}"] = m
            h = hz * m
        else:
            h = hz * TEST_SCALE
        t[f"drop{li + 1}"] = h
    z = L.fc(h, weights[7], biases[7])
    t["logits"] = z
    t["probs"] = L.softmax(z)
    return t


def backward(weights, t, labels, groups=1, store=None):
    """Gradients of the mean cross-entropy w.r.t. all 16 parameter tensors.

    Returns (loss, grads_w, grads_b, gtaps) where gtaps holds the gradient
    w.r.t. each saved activation (named d<activation>).  ``store`` as in
    forward(): the precision of the activation gradients handed between
    layers."""
    q = _quant(store)
    g = {}
    loss, dz = L.ce_loss_grad(t["probs"], labels)
    dz = q(dz)
    g["dlogits"] = dz
    gw, gb = [None] * 8, [None] * 8
    dh, gw[7], gb[7] = L.fc_bwd(dz, t["drop7"], weights[7])
    for li in (6, 5):
        name = f"fc{li + 1}"
        dh = dh * t[f"mask{li + 1}"]                # dropout: no gradient to dropped units
        dh = q(L.relu_bwd(t[name], dh))
        g["d" + name] = dh                          # gradient w.r.t. the FC pre-activation
        x_in = t["drop6"] if li == 6 else t["flat"]
        dh, gw[li], gb[li] = L.fc_bwd(dh, x_in, weights[li])
    dh = q(dh)
    g["dflat"] = dh
    da = dh.reshape(t["pool5"].shape)
    da = L.maxpool_bwd(da, t["arg5"], t["conv5"].shape)
    for li in (4, 3, 2, 1, 0):
        s, p, grouped = CONV_GEOM[li]
        gg = _g(groups, grouped)
        act = t[f"conv{li + 1}"]
        if li in (0, 1):
            # pool -> LRN -> ReLU backward
            da = q(L.maxpool_bwd(da, t[f"arg{li + 1}"], act.shape))
            g[f"dlrn{li + 1}"] = da
            da = L.lrn_bwd(act, da, **LRN)
        dzc = q(L.relu_bwd(act, da))
        g[f"dconv{li + 1}"] = dzc                   # gradient w.r.t. the conv pre-activation
        x_in = t["x"] if li == 0 else (t["pool1"] if li == 1 else
                                       t["pool2"] if li == 2 else t[f"conv{li}"])
        gw[li], gb[li] = L.conv2d_bwd_weight(dzc, x_in, weights[li].shape, s, p, gg)
        if li > 0:
            da = L.conv2d_bwd_data(dzc, weights[li], x_in.shape, s, p, gg)
            if li in (1, 2):                        # input of a pooling layer: stored as is
                da = q(da)
            g[f"din{li + 1}"] = da
    return loss, gw, gb, g


def train_step(work_w, work_b, master_w, master_b, vel_w, vel_b, x, labels, groups=1,
               lr=0.01, momentum=0.9, weight_decay=5e-4, seed=3, step=0, store=None):
    """One TRAIN_STEP: forward (train mode), loss, backward, SGD on every tensor.

    The forward/backward use the working weights (the bf16-rounded copies in
    the bf16 configuration); SGD updates the master weights and velocities.
    Returns a dict with loss, taps, gradients and the updated state."""
    t = forward(work_w, work_b, x, groups, train=True, seed=seed, step=step, store=store)
    loss, gw, gb, gt = backward(work_w, t, labels, groups, store=store)
    new_w, new_vw, new_b, new_vb = [], [], [], []
    for i in range(8):
        w1, v1 = L.sgd(master_w[i], vel_w[i], gw[i], lr, momentum, weight_decay)
        b1, u1 = L.sgd(master_b[i], vel_b[i], gb[i], lr, momentum, weight_decay)
        new_w.append(w1); new_vw.append(v1); new_b.append(b1); new_vb.append(u1)
    return dict(loss=loss, taps=t, gtaps=gt, grad_w=gw, grad_b=gb,
                w=new_w, vw=new_vw, b=new_b, vb=new_vb)


def forward_tenview(weights, biases, src, groups=1, crop=227, store=None):
    """Ten-patch test-time averaging: crop, forward, mean of the softmaxes."""
    views = L.tenview_crop(src, crop)
    t = forward(weights, biases, views, groups, store=store)
    t["views"] = views
    t["mean_probs"] = L.view_mean(t["probs"])
    return t
