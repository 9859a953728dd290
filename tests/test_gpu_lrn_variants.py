"""The LRN constants the C ABI accepts besides the pages' (n = 5, k = 2,
alpha = 1e-4, beta = 0.75): window sizes 1, 3, 7 and 9 and other exponents
select other instantiations of the fused LRN + pool kernels (forward and
backward).  Each is checked layer by layer against the oracle's LRN
(paper-graph-ui "Local Response Normalization") on the HIP path's own stored
LRN input, in a training step with the LRN taps stored:
  - LRN output of layers 1 and 2 (forward), pool values and argmax bit-exact;
  - gradient w.r.t. the LRN input times the ReLU mask (backward).
Tolerances are the layer-isolated ones: one bf16 rounding of the output
(rel-L2 5e-3) or fp32 (1e-5)."""
import numpy as np
import pytest
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, stream_handle, to_device

from gpu_helpers import DEV, TOL_LAYER_BF16, nchw, params_f32, rel_l2, say

pytestmark = pytest.mark.gpu

CASES = [  # dtype, n, k, alpha, beta
    (B.BF16, 3, 2.0, 1e-4, 0.75),
    (B.BF16, 1, 1.0, 1e-3, 0.75),
    (B.BF16, 7, 1.0, 5e-4, 0.5),
    (B.BF16, 9, 2.0, 1e-3, 0.6),
    (B.F32, 3, 1.0, 1e-3, 0.6),
    (B.F32, 5, 2.0, 1e-4, 0.5),
]


@pytest.mark.parametrize("dtype,n,k,alpha,beta", CASES)
def test_lrn_variant_layerwise(orc, dtype, n, k, alpha, beta):
    syn = I.synthetic(13, 2, groups=1, bf16=dtype == B.BF16)
    say(f"[gpu] LRN variant dtype={dtype} n={n} k={k} alpha={alpha} beta={beta}")
    sess = Session(2, 1, dtype, B.MODE_TRAIN, DEV, lrn_taps=True)
    sess.cfg.lrn_n, sess.cfg.lrn_k, sess.cfg.lrn_alpha, sess.cfg.lrn_beta = n, k, alpha, beta
    master = params_f32(syn.master_w, syn.biases)
    mom = [torch.zeros_like(m) for m in master]
    tdt = torch.bfloat16 if dtype == B.BF16 else torch.float32
    work = [torch.empty(m.shape, dtype=tdt, device=DEV) for m in master]
    B.alexnet_cast_weights(sess.cfg, master, work, stream_handle())
    x = to_device(syn.x, dtype, DEV)
    labels = torch.from_numpy(syn.labels.astype(np.int32)).to(DEV)
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    sess.train_step(master, mom, work, x, labels, loss, None)
    torch.cuda.synchronize()
    h = {t: nchw(sess.tap(t)) for t in ("conv1", "lrn1", "pool1", "arg1", "conv2", "lrn2", "pool2", "arg2",
                                        "dlrn1", "dconv1", "dlrn2", "dconv2")}
    # the cfg values as the library holds them (fp32)
    kk, aa, bb = float(sess.cfg.lrn_k), float(sess.cfg.lrn_alpha), float(sess.cfg.lrn_beta)
    lrn = lambda a: orc.lrn(a, kk, aa, bb, n)
    e = {}
    for l in ("1", "2"):
        e["lrn" + l] = rel_l2(h["lrn" + l], lrn(h["conv" + l]))
        p, a = orc.maxpool(h["lrn" + l])
        assert np.array_equal(h["pool" + l], p), "pool" + l
        assert np.array_equal(h["arg" + l], a), "arg" + l
        want = orc.lrn_bwd(h["conv" + l], h["dlrn" + l], kk, aa, bb, n) * (h["conv" + l] > 0)
        e["dconv" + l] = rel_l2(h["dconv" + l], want)
    say("[gpu] LRN variant rel-L2:", {q: f"{v:.1e}" for q, v in e.items()})
    tol = TOL_LAYER_BF16 if dtype == B.BF16 else 1e-5
    for q, v in e.items():
        assert v <= tol, (q, v)
    assert np.isfinite(float(loss.item()))
