"""Layer 1's bf16 kernels (the direct forward and weight-gradient convolutions)
at a batch whose tiles do not spread evenly: 37 images make 37 x 14 = 518
tiles of 4 output rows, so the XCDs get 64 or 65 tiles and their workgroups
two or three, and the double-buffered block rows alternate an odd number of
times in some workgroups and an even number in others.  The forward output of
sampled images (first, middle, last) and the weight gradient of the whole
batch are compared with the oracle, each computed from the HIP path's own
input of that layer (ImageNet Classification with Deep Convolutional Neural
Networks, section 3.5: layer 1 applies 96 kernels of 11x11x3 at stride 4 to
the RGB image, 227x227 here)."""
import numpy as np
import pytest
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, stream_handle, to_device

from gpu_helpers import DEV, TOL_LAYER_BF16, host, nchw, params_f32, rel_l2, say

pytestmark = pytest.mark.gpu

BATCH = 37
ROWS = [0, BATCH // 2, BATCH - 1]
TOL_WGRAD = 1e-4   # fp32 accumulation of the same bf16 products, in another order


def test_layer1_forward_uneven_tiles(orc):
    syn = I.synthetic(41, BATCH, groups=1, bf16=True)
    say(f"[gpu] layer-1 forward, batch {BATCH} bf16 (518 tiles over 256 workgroups)")
    sess = Session(BATCH, 1, B.BF16, B.MODE_FORWARD, DEV)
    params = sess.upload_params(syn.weights, syn.biases)
    x = to_device(syn.x, B.BF16, DEV)
    sess.forward(params, x)
    torch.cuda.synchronize()
    got = nchw(sess.tap("conv1")[torch.as_tensor(ROWS, device=DEV)])
    want = orc.relu(orc.conv2d(syn.x[ROWS], syn.weights[0], syn.biases[0], 4, 0))
    e = rel_l2(got, want)
    say(f"[gpu]   conv1 of images {ROWS} vs oracle: rel-L2 {e:.2e}")
    assert e <= TOL_LAYER_BF16


def test_layer1_weight_gradient_uneven_tiles(orc):
    syn = I.synthetic(43, BATCH, groups=1, bf16=True)
    say(f"[gpu] layer-1 weight gradient, batch {BATCH} bf16 training step")
    sess = Session(BATCH, 1, B.BF16, B.MODE_TRAIN, DEV)
    master = params_f32(syn.master_w, syn.biases)
    mom = [torch.zeros_like(m) for m in master]
    work = [torch.empty(m.shape, dtype=torch.bfloat16, device=DEV) for m in master]
    B.alexnet_cast_weights(sess.cfg, master, work, stream_handle())
    x = to_device(syn.x, B.BF16, DEV)
    labels = torch.from_numpy(syn.labels.astype(np.int32)).to(DEV)
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    probs = torch.empty((BATCH, 1000), dtype=torch.float32, device=DEV)
    sess.train_step(master, mom, work, x, labels, loss, probs, lr=0.01, momentum_coef=0.9,
                    weight_decay=5e-4, seed=5, step=0)
    torch.cuda.synchronize()
    gw1 = host(sess.tap("gw1"))
    dconv1 = nchw(sess.tap("dconv1"))
    assert np.any(gw1 != 0.0)
    # the input as the step stored it: bf16 images (the oracle widens them exactly)
    ref, _ = orc.conv2d_bwd_weight(dconv1, syn.x, syn.weights[0].shape, 4, 0)
    e = rel_l2(gw1, ref)
    say(f"[gpu]   gw1 vs oracle on the run's own dconv1: rel-L2 {e:.2e}")
    assert e <= TOL_WGRAD
