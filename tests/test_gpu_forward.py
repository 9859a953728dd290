"""GPU parity of the forward pass (through the C ABI) against the CPU oracle.

Small batches are compared element by element, end to end and layer by layer
(each layer of the oracle fed the HIP path's own stored input, so pool argmax
indices must match bit for bit).  Full-size batches are compared on sampled
images, which the oracle can compute on their own because images are
independent in the forward pass."""
import numpy as np
import pytest
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, Timer, stream_handle, to_device

from gpu_helpers import (DEV, TOL_BF16, TOL_F32, TOL_F32_OUT, TOL_LAYER_BF16, flat, host, nchw,
                         rel_l2, say)

pytestmark = pytest.mark.gpu

FWD_TAPS = ("conv1", "lrn1", "pool1", "arg1", "conv2", "lrn2", "pool2", "arg2", "conv3", "conv4",
            "conv5", "pool5", "arg5", "drop6", "drop7", "logits")


def run_forward(syn, dtype, mode=B.MODE_FORWARD, batch=None, lrn_taps=True):
    n = syn.x.shape[0] if batch is None else batch
    say(f"[gpu] forward mode={mode} batch={n} groups={syn.groups} dtype={dtype} seed={syn.seed} "
        f"lrn_taps={lrn_taps}")
    sess = Session(n, syn.groups, dtype, mode, DEV, lrn_taps=lrn_taps)
    params = sess.upload_params(syn.weights, syn.biases)
    x = to_device(syn.x, dtype, DEV)
    probs = sess.forward(params, x)
    torch.cuda.synchronize()
    g = {name: sess.tap(name).clone() for name in FWD_TAPS if lrn_taps or not name.startswith("lrn")}
    if mode == B.MODE_TENVIEW:
        g["view_probs"] = sess.tap("view_probs").clone()
    g["probs"] = probs.clone()
    return g


NHWC_TAPS = {"conv1", "lrn1", "pool1", "arg1", "conv2", "lrn2", "pool2", "arg2", "conv3", "conv4",
             "conv5", "arg5"}


def hostify(g, rows=None):
    """Taps of the selected images as float64 NCHW / [N, F] host arrays."""
    out = {}
    for k, v in g.items():
        if k == "view_probs":
            continue
        t = v if rows is None else v[torch.as_tensor(rows, device=v.device)]
        out[k] = nchw(t) if k in NHWC_TAPS else flat(t)
    return out


def layerwise(orc, syn, h, groups, tol, rows=None):
    """Each layer of the oracle on the HIP path's stored input of that layer."""
    W, Bb = syn.weights, syn.biases
    x = syn.x if rows is None else syn.x[rows]
    lay = {}
    lay["conv1"] = rel_l2(h["conv1"], orc.relu(orc.conv2d(x, W[0], Bb[0], 4, 0)))
    lay["lrn1"] = rel_l2(h["lrn1"], orc.lrn(h["conv1"]))
    p1, a1 = orc.maxpool(h["lrn1"])
    assert np.array_equal(h["pool1"], p1), "pool1 values"
    assert np.array_equal(h["arg1"], a1), "pool1 argmax"
    lay["conv2"] = rel_l2(h["conv2"], orc.relu(orc.conv2d(h["pool1"], W[1], Bb[1], 1, 2, groups)))
    lay["lrn2"] = rel_l2(h["lrn2"], orc.lrn(h["conv2"]))
    p2, a2 = orc.maxpool(h["lrn2"])
    assert np.array_equal(h["pool2"], p2), "pool2 values"
    assert np.array_equal(h["arg2"], a2), "pool2 argmax"
    lay["conv3"] = rel_l2(h["conv3"], orc.relu(orc.conv2d(h["pool2"], W[2], Bb[2], 1, 1)))
    lay["conv4"] = rel_l2(h["conv4"], orc.relu(orc.conv2d(h["conv3"], W[3], Bb[3], 1, 1, groups)))
    lay["conv5"] = rel_l2(h["conv5"], orc.relu(orc.conv2d(h["conv4"], W[4], Bb[4], 1, 1, groups)))
    p5, a5 = orc.maxpool(h["conv5"])
    assert np.array_equal(h["pool5"], p5.reshape(p5.shape[0], -1)), "pool5 values"
    assert np.array_equal(h["arg5"], a5), "pool5 argmax"
    lay["drop6"] = rel_l2(h["drop6"], 0.5 * orc.relu(orc.fc(h["pool5"], W[5], Bb[5])))
    lay["drop7"] = rel_l2(h["drop7"], 0.5 * orc.relu(orc.fc(h["drop6"], W[6], Bb[6])))
    lay["logits"] = rel_l2(h["logits"], orc.fc(h["drop7"], W[7], Bb[7]))
    say("[gpu] layer-isolated rel-L2:", {k: f"{v:.2e}" for k, v in lay.items()})
    for k, v in lay.items():
        limit = TOL_F32_OUT if k == "logits" else tol
        assert v <= limit, (k, v)
    return lay


def end_to_end(orc, syn, h, groups, tol, rows=None, store=None):
    """store=None: float64 oracle; store="bf16": the oracle with bf16 storage
    between layers (the precision the bf16 workloads define)."""
    x = syn.x if rows is None else syn.x[rows]
    t = orc.alexnet.forward(syn.weights, syn.biases, x, groups, store=store)
    e = {}
    for name in ("conv1", "lrn1", "pool1", "conv2", "lrn2", "pool2", "conv3", "conv4", "conv5"):
        e[name] = rel_l2(h[name], t[name])
    e["pool5"] = rel_l2(h["pool5"], t["flat"])
    for name in ("drop6", "drop7", "logits", "probs"):
        e[name] = rel_l2(h[name], t[name])
    # argmax agreement end to end is a diagnostic: near-ties may round apart.
    agree = {k: float(np.mean(h[k] == t[k])) for k in ("arg1", "arg2", "arg5")}
    say(f"[gpu] end-to-end rel-L2 (oracle storage {store}):", {k: f"{v:.2e}" for k, v in e.items()},
        "argmax agreement:", agree)
    for k, v in e.items():
        assert v <= tol, (k, v)
    return t


# ---------------------------------------------------------------- fp32, batch 1
def test_fp32_batch1_matches_oracle(orc):
    syn = I.workload_inputs("fp32_batch1")
    g = run_forward(syn, B.F32)
    h = hostify(g)
    layerwise(orc, syn, h, 1, TOL_F32)
    t = end_to_end(orc, syn, h, 1, TOL_F32)
    for k in ("arg1", "arg2", "arg5"):      # near-ties may round apart end to end
        assert np.mean(h[k] == t[k]) >= 0.999, k
    np.testing.assert_allclose(host(g["probs"]).sum(1), 1.0, atol=1e-5)


def test_fp32_two_tower_batch2_matches_oracle(orc):
    """fp32 grouped network at batch 2: the small-batch paths with two groups
    (split-K partials and their reduction per group, the FC row kernel)."""
    syn = I.synthetic(12, 2, groups=2, bf16=False)
    g = run_forward(syn, B.F32)
    h = hostify(g)
    layerwise(orc, syn, h, 2, TOL_F32)
    t = end_to_end(orc, syn, h, 2, TOL_F32)
    for k in ("arg1", "arg2", "arg5"):      # near-ties may round apart end to end
        assert np.mean(h[k] == t[k]) >= 0.999, k
    np.testing.assert_allclose(host(g["probs"]).sum(1), 1.0, atol=1e-5)


# ---------------------------------------------------------------- bf16, small batches
@pytest.mark.parametrize("wl,batch", [("bf16_batch128", 3), ("two_tower_batch128", 2), ("bf16_batch128", 1),
                                      ("bf16_batch128", 4), ("bf16_batch128", 5)])
def test_bf16_small_batch_layerwise_and_end_to_end(orc, wl, batch):
    syn = I.workload_inputs(wl, batch=batch)
    g = run_forward(syn, B.BF16)
    h = hostify(g)
    layerwise(orc, syn, h, syn.groups, TOL_LAYER_BF16)
    end_to_end(orc, syn, h, syn.groups, TOL_BF16, store="bf16")
    end_to_end(orc, syn, h, syn.groups, TOL_BF16)
    probs = host(g["probs"])
    np.testing.assert_allclose(probs.sum(1), 1.0, atol=1e-5)
    # probabilities are the fp32 softmax of the stored fp32 logits
    assert rel_l2(probs, orc.softmax(flat(g["logits"]))) <= 1e-5


def test_tenview_small(orc):
    syn = I.workload_inputs("tenview_256_sources", batch=2)
    g = run_forward(syn, B.BF16, B.MODE_TENVIEW, batch=2)
    views = orc.tenview_crop(syn.x)
    # layer 1 reads the crops and mirrors straight from the sources
    assert rel_l2(nchw(g["conv1"]), orc.relu(orc.conv2d(views, syn.weights[0], syn.biases[0], 4, 0))) <= TOL_LAYER_BF16
    t = orc.alexnet.forward_tenview(syn.weights, syn.biases, syn.x, store="bf16")
    e_views = rel_l2(flat(g["view_probs"]), t["probs"])
    e_mean = rel_l2(host(g["probs"]), t["mean_probs"])
    say(f"[gpu] ten-view rel-L2 views={e_views:.2e} mean={e_mean:.2e}")
    assert e_views <= TOL_BF16 and e_mean <= TOL_BF16
    vp = flat(g["view_probs"]).reshape(2, 10, 1000)
    np.testing.assert_allclose(host(g["probs"]), vp.sum(1) / 10.0, rtol=1e-6, atol=1e-9)


def test_fused_lrn_pool_equals_stored_path():
    """The default forward (LRN and max-pool fused, LRN output never stored)
    gives bit-identical pooled values, argmax and probabilities."""
    syn = I.workload_inputs("bf16_batch128", batch=3)
    a = run_forward(syn, B.BF16, lrn_taps=True)
    b = run_forward(syn, B.BF16, lrn_taps=False)
    for k in b:
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype != torch.uint8 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype != torch.uint8 else b[k]), k


def test_forward_is_deterministic():
    syn = I.workload_inputs("bf16_batch128", batch=4)
    a = run_forward(syn, B.BF16)
    b = run_forward(syn, B.BF16)
    for k in FWD_TAPS + ("probs",):
        assert torch.equal(a[k].view(torch.uint8) if a[k].dtype != torch.uint8 else a[k],
                           b[k].view(torch.uint8) if b[k].dtype != torch.uint8 else b[k]), k


def test_timers_time_their_kernels_and_change_no_result():
    """Timers from alexnet_event_create around three kernels of a forward
    pass: each span is positive and below a second, and the probabilities are
    bit-identical to those of the untimed call."""
    syn = I.workload_inputs("bf16_batch128", batch=8)
    sess = Session(8, 1, B.BF16, B.MODE_FORWARD, DEV)
    params = sess.upload_params(syn.weights, syn.biases)
    x = to_device(syn.x, B.BF16, DEV)
    plain = sess.forward(params, x).clone()
    names = ("S2D", "CONV2_FWD", "FC6_FWD")
    timers = [Timer() for _ in names]
    probs = torch.empty_like(plain)
    B.alexnet_forward_timed(sess.cfg, params, x, probs, sess.ws, sess.ws_bytes, stream_handle(),
                            [(B.KT[nm], t.start, t.stop) for nm, t in zip(names, timers)])
    torch.cuda.synchronize()
    ms = [t.elapsed_ms() for t in timers]
    say(f"[gpu] timed spans (ms) {dict(zip(names, ms))}")
    assert all(0.0 < m < 1000.0 for m in ms), ms
    assert torch.equal(probs, plain)


# ---------------------------------------------------------------- full-size, sampled images
@pytest.mark.parametrize("wl", ["bf16_batch128", "two_tower_batch128"])
def test_full_batch128_sampled_images(orc, wl):
    syn = I.workload_inputs(wl)
    g = run_forward(syn, B.BF16)
    rows = np.array([0, 77, 127])
    h = hostify(g, rows)
    layerwise(orc, syn, h, syn.groups, TOL_LAYER_BF16, rows=rows)
    end_to_end(orc, syn, h, syn.groups, TOL_BF16, rows=rows, store="bf16")
    end_to_end(orc, syn, h, syn.groups, TOL_BF16, rows=rows)
    np.testing.assert_allclose(host(g["probs"]).sum(1), 1.0, atol=1e-5)


def test_full_tenview_256_sources_sampled(orc):
    syn = I.workload_inputs("tenview_256_sources")
    g = run_forward(syn, B.BF16, B.MODE_TENVIEW, batch=256)
    for src in (0, 255):
        t = orc.alexnet.forward_tenview(syn.weights, syn.biases, syn.x[src:src + 1], store="bf16")
        e_mean = rel_l2(host(g["probs"])[src:src + 1], t["mean_probs"])
        e_views = rel_l2(flat(g["view_probs"])[src * 10:src * 10 + 10], t["probs"])
        say(f"[gpu] ten-view source {src}: mean {e_mean:.2e} views {e_views:.2e}")
        assert e_mean <= TOL_BF16 and e_views <= TOL_BF16
    np.testing.assert_allclose(host(g["probs"]).sum(1), 1.0, atol=1e-5)
