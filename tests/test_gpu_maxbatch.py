"""The largest batch the library accepts for a training step (4096) on the GPU,
where several tensors pass 1-2 GB and every buffer offset is at its widest.

The oracle cannot afford a 4096-image step, so the checks are invariants of
a batch made of 32 copies of the 128-image batch, with dropout off
(cfg.dropout_p = 0):
  - within the 4096 run every copy carries bit-identical values and
    gradients: no kernel's result depends on where a row sits in the batch;
  - the conv1 weight gradient -- the largest reduction (12.4M output pixels,
    split-K over the largest buffers) -- equals 32 times the oracle's conv1
    weight gradient of one copy, taken from the run's own stored dconv1;
  - against the 128-image run: the convolution stack (through pool5) is bit
    for bit the same (each output element is the same dot product in the same
    order whatever the batch); the FC outputs, probabilities, loss and
    gradients agree up to summation order.  The FC split-K count follows the
    batch, so the logits differ in the last bits, and every bf16-stored
    activation gradient after them can round the other way: the differences
    grow by about 5e-4 per layer down the backward pass (printed), which
    bounds them at 1e-2 at the conv1 end."""
import numpy as np
import pytest
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, stream_handle, to_device

from gpu_helpers import DEV, host, nchw, params_f32, rel_l2, say

pytestmark = pytest.mark.gpu

REPS = 32                  # 32 x 128 = 4096, the largest training batch
# activation gradients along the backward pass (bf16), first copy of the batch
CHAIN = ("dlogits", "dfc7", "dfc6", "dflat", "dconv5", "dconv4", "dconv3", "din3", "dconv2", "din2", "dconv1")
TOL_SUM_ORDER = 1e-3       # FC outputs and probabilities: fp32 sums in another order
TOL_CHAIN = 1e-2           # gradients: bf16 rounding flips compounding down the backward pass
TOL_WGRAD = 1e-4           # conv1 weight gradient vs the oracle on the same dconv1 (fp32 accumulation)


def train_repeated(syn, reps):
    base = syn.x.shape[0]
    n = base * reps
    say(f"[gpu] max-batch train: batch={n} ({reps} copies of {base}), dropout off")
    sess = Session(n, 1, B.BF16, B.MODE_TRAIN, DEV)
    sess.cfg.dropout_p = 0.0
    master = params_f32(syn.master_w, syn.biases)
    mom = [torch.zeros_like(m) for m in master]
    work = [torch.empty(m.shape, dtype=torch.bfloat16, device=DEV) for m in master]
    B.alexnet_cast_weights(sess.cfg, master, work, stream_handle())
    x = to_device(syn.x, B.BF16, DEV).repeat(reps, 1, 1, 1).contiguous()
    labels = torch.from_numpy(syn.labels.astype(np.int32)).to(DEV).repeat(reps).contiguous()
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    probs = torch.empty((n, 1000), dtype=torch.float32, device=DEV)
    sess.train_step(master, mom, work, x, labels, loss, probs, lr=0.01, momentum_coef=0.9,
                    weight_decay=5e-4, seed=3, step=0)
    torch.cuda.synchronize()
    r = dict(loss=float(loss.item()), probs=probs.cpu().numpy(),
             dlogits=host(sess.tap("dlogits")), pool5=sess.tap("pool5")[:base].clone(),
             pool5_last=sess.tap("pool5")[n - base:].clone(),
             gw=[host(sess.tap(f"gw{i + 1}")) for i in range(5)],
             gb=[host(sess.tap(f"gb{i + 1}")).ravel() for i in range(8)],
             chain={k: host(sess.tap(k)[:base]) for k in CHAIN},
             dconv1=nchw(sess.tap("dconv1")[:base]),
             copies_equal=all(torch.equal(sess.tap(k)[:base], sess.tap(k)[n - base:])
                              for k in ("pool5", "drop7", "dlogits", "dfc6", "dconv3", "dconv1")),
             mom=[host(v) for v in mom], master=[host(m) for m in master],
             work=[w.float().cpu().numpy() for w in work])
    del sess, x, probs
    torch.cuda.empty_cache()
    return r


def test_max_batch_is_32_copies_of_the_base_batch(orc):
    syn = I.workload_inputs("train_batch128")                      # the 128-image training workload
    base = train_repeated(syn, 1)
    big = train_repeated(syn, REPS)
    n = syn.x.shape[0]
    # within the 4096 run: the first and the last copy agree bit for bit
    assert big["copies_equal"]
    # conv1 weight gradient at 4096 rows vs the oracle on the run's own dconv1
    ref, _ = orc.conv2d_bwd_weight(big["dconv1"], syn.x, syn.weights[0].shape, 4, 0)
    e1 = rel_l2(big["gw"][0], REPS * ref)
    say(f"[gpu] max-batch gw1 vs oracle on the same dconv1: {e1:.1e}")
    assert e1 <= TOL_WGRAD
    # convolution stack: bit-identical rows in the first and last copy
    assert torch.equal(big["pool5"], base["pool5"]) and torch.equal(big["pool5_last"], base["pool5"])
    # probabilities and loss gradients of every copy
    p = big["probs"].reshape(REPS, n, 1000)
    dl = big["dlogits"].reshape(REPS, n, 1000)
    for k in range(REPS):
        assert rel_l2(p[k], base["probs"]) <= TOL_SUM_ORDER, k
        assert rel_l2(dl[k] * REPS, base["dlogits"]) <= TOL_SUM_ORDER, k
    # the loss: the mean of the same row losses, whose logits differ by the FC sum order
    assert abs(big["loss"] - base["loss"]) <= 1e-4 * abs(base["loss"])
    chain = {k: rel_l2(big["chain"][k] * REPS, base["chain"][k]) for k in CHAIN}
    say("[gpu] max-batch activation-gradient chain, relative L2 vs base:",
        {k: f"{v:.1e}" for k, v in chain.items()})
    # gradients, momentum and weights after the update
    errs = {}
    for i in range(5):
        errs[f"gw{i + 1}"] = rel_l2(big["gw"][i], base["gw"][i])
    for i in range(8):
        errs[f"gb{i + 1}"] = rel_l2(big["gb"][i], base["gb"][i])
    for j in range(16):
        errs[f"v{j}"] = rel_l2(big["mom"][j], base["mom"][j])
    say("[gpu] max-batch relative L2 vs base:", {k: f"{v:.1e}" for k, v in errs.items()})
    for k, e in errs.items():
        assert e <= TOL_CHAIN, (k, e)
    for k, e in chain.items():
        assert e <= TOL_CHAIN, (k, e)
    for j in range(16):
        assert rel_l2(big["master"][j] - syn_master(syn, j), base["master"][j] - syn_master(syn, j)) \
            <= TOL_CHAIN, j


def syn_master(syn, j):
    i = j // 2
    return np.asarray(syn.master_w[i] if j % 2 == 0 else syn.biases[i], np.float64)


# ---------------------------------------------------------------- forward at the largest sizes
def forward_taps(syn_weights, syn_biases, x_host, n, mode, groups=1):
    sess = Session(n, groups, B.BF16, mode, DEV)
    params = sess.upload_params(syn_weights, syn_biases)
    x = to_device(x_host, B.BF16, DEV) if isinstance(x_host, np.ndarray) else x_host
    probs = sess.forward(params, x)
    torch.cuda.synchronize()
    return sess, probs


def test_forward_batch4096_is_32_copies_of_batch128():
    """Forward pass at the largest batch (4096 = 32 copies of the 128-image
    workload): the first and last copies are bit-identical to each other and
    to the 128-image run through pool5 (each conv output is the same dot
    product in the same order whatever the batch); the probabilities of every
    copy agree with the 128-image run up to the FC layers' summation order."""
    syn = I.workload_inputs("bf16_batch128")
    n = syn.x.shape[0]
    say(f"[gpu] forward batch {n}")
    s1, p1 = forward_taps(syn.weights, syn.biases, syn.x, n, B.MODE_FORWARD)
    pool5_base, probs_base = s1.tap("pool5").clone(), p1.cpu().numpy()
    del s1
    say(f"[gpu] forward batch {n * REPS} ({REPS} copies)")
    xb = to_device(syn.x, B.BF16, DEV).repeat(REPS, 1, 1, 1).contiguous()
    s2, p2 = forward_taps(syn.weights, syn.biases, xb, n * REPS, B.MODE_FORWARD)
    pool5 = s2.tap("pool5")
    assert torch.equal(pool5[:n], pool5_base) and torch.equal(pool5[-n:], pool5_base)
    assert torch.equal(s2.tap("drop7")[:n], s2.tap("drop7")[-n:])
    p = p2.cpu().numpy().reshape(REPS, n, 1000)
    e = max(rel_l2(p[k], probs_base) for k in range(REPS))
    say(f"[gpu] batch-4096 probabilities vs batch 128: max rel-L2 {e:.1e}")
    assert e <= TOL_SUM_ORDER
    np.testing.assert_allclose(p.sum(-1), 1.0, atol=1e-5)
    del s2, xb
    torch.cuda.empty_cache()


def test_tenview_512_sources(orc):
    """Ten-view inference at the largest count the library accepts, 512
    sources (5120 views, the conv1 output alone about 3 GB, byte offsets near
    the top of the 32-bit buffer range): the first 256 sources are the
    256-source workload and give bit-identical conv stacks to its own run;
    sources from the second half, the last one included, match the oracle."""
    syn = I.workload_inputs("tenview_256_sources")
    extra = I.synthetic(14, 256, image=256, with_labels=False).x
    say("[gpu] ten-view 256 sources")
    s1, _ = forward_taps(syn.weights, syn.biases, syn.x, 256, B.MODE_TENVIEW)
    pool5_base = s1.tap("pool5").clone()
    del s1
    torch.cuda.empty_cache()
    say("[gpu] ten-view 512 sources (5120 views)")
    x512 = np.concatenate([syn.x, extra])
    s2, p2 = forward_taps(syn.weights, syn.biases, x512, 512, B.MODE_TENVIEW)
    assert torch.equal(s2.tap("pool5")[:2560], pool5_base)
    probs = host(p2)
    vp = host(s2.tap("view_probs"))
    np.testing.assert_allclose(probs.sum(1), 1.0, atol=1e-5)
    for src in (300, 511):
        t = orc.alexnet.forward_tenview(syn.weights, syn.biases, x512[src:src + 1], store="bf16")
        e_mean = rel_l2(probs[src:src + 1], t["mean_probs"])
        e_views = rel_l2(vp[src * 10:src * 10 + 10], t["probs"])
        say(f"[gpu] ten-view 512 sources, source {src}: mean {e_mean:.2e} views {e_views:.2e}")
        assert e_mean <= 2e-2 and e_views <= 2e-2
    del s2
    torch.cuda.empty_cache()
