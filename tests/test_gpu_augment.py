"""GPU parity of the training-time augmentation and the RGB principal
components (paper-graph-ui "Data Augmentation", Forms 1 and 2) through the C
ABI, against the CPU oracle.

- alexnet_augment_images against the oracle's patches, element by element:
  the HIP path forms the colour shift and the pixel sum in fp32 and rounds
  once to bf16, the oracle works in float64 and rounds to bf16 at the end, so
  an element may differ by one bf16 unit in the last place when the float64
  value sits within fp32 rounding of a bf16 rounding boundary; all others are
  identical (fp32 workload: relative 1e-6).
- alexnet_train_step_augmented, whose layer-1 staging reads the patches
  straight from the sources, is bit-identical to alexnet_train_step fed the
  materialised patches (same per-element arithmetic); the training step itself
  is pinned against the oracle in test_gpu_train.
- alexnet_rgb_pca against the oracle's covariance eigen-decomposition: the
  fp64 moments of bf16 inputs are exact, so eigenvalues and eigenvectors agree
  to fp32 rounding (tolerances 1e-6 relative and 1e-5 absolute)."""
import numpy as np
import pytest
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, stream_handle, to_device

from gpu_helpers import DEV, host, params_f32, say

pytestmark = pytest.mark.gpu

BF16_SAME_FRACTION = 1e-3   # at most this share of elements one bf16 ulp apart


def dev_aug(a: I.AugInputs, eigval, eigvec):
    t = dict(crop=torch.from_numpy(np.ascontiguousarray(a.crop, np.int32)).to(DEV),
             alpha=torch.from_numpy(np.ascontiguousarray(a.alpha, np.float32)).to(DEV),
             eigval=torch.from_numpy(np.ascontiguousarray(eigval, np.float32)).to(DEV),
             eigvec=torch.from_numpy(np.ascontiguousarray(eigvec, np.float32)).to(DEV))
    return t, B.augment(t["crop"], t["alpha"], t["eigval"], t["eigvec"])


def pca_basis(orc, a: I.AugInputs):
    lam, vec, _ = orc.rgb_pca(a.src)
    return lam.astype(np.float32), vec.astype(np.float32)


def gpu_augment(a: I.AugInputs, eigval, eigvec, dtype):
    n, _, hs, ws = a.src.shape
    say(f"[gpu] augment_images batch={n} src={hs}x{ws} dtype={dtype}")
    cfg = B.alexnet_default_cfg(n, 1, dtype)
    src = to_device(a.src, dtype, DEV)
    keep, aug = dev_aug(a, eigval, eigvec)
    x = torch.empty((n, 3, 227, 227), dtype=torch.bfloat16 if dtype == B.BF16 else torch.float32, device=DEV)
    B.alexnet_augment_images(cfg, src, hs, ws, aug, x, stream_handle())
    torch.cuda.synchronize()
    return x


def oracle_augment(orc, a: I.AugInputs, eigval, eigvec):
    return orc.augment(a.src, a.crop, a.alpha.astype(np.float64), eigvec.astype(np.float64),
                       eigval.astype(np.float64))


def bf16_ulp(v):
    e = np.floor(np.log2(np.maximum(np.abs(v), 1e-30)))
    return np.exp2(e - 7)


def check_bf16(gpu, want):
    g = host(gpu)
    w = orc_round(want)
    diff = np.abs(g - w)
    off = diff > 0
    assert np.all(diff[off] <= bf16_ulp(np.maximum(np.abs(g), np.abs(w)))[off]), float(diff.max())
    frac = off.mean()
    say(f"[gpu] augment: {off.sum()} of {off.size} elements one bf16 ulp from the oracle ({frac:.1e})")
    assert frac <= BF16_SAME_FRACTION


def orc_round(a):
    import oracle
    return oracle.alexnet.round_bf16(a)


@pytest.mark.parametrize("hs,ws,batch", [(256, 256, 128), (240, 300, 5), (227, 227, 3)])
def test_augment_images_bf16(orc, hs, ws, batch):
    a = I.augment_inputs(21, batch, hs, ws)
    lam, vec = pca_basis(orc, a)
    x = gpu_augment(a, lam, vec, B.BF16)
    check_bf16(x, oracle_augment(orc, a, lam, vec))


def test_augment_images_fp32(orc):
    a = I.augment_inputs(22, 4, 256, 256, bf16=False)
    lam, vec = pca_basis(orc, a)
    x = host(gpu_augment(a, lam, vec, B.F32))
    want = oracle_augment(orc, a, lam, vec)
    shift = np.abs(want - orc.augment(a.src, a.crop, 0 * a.alpha.astype(np.float64),
                                      vec.astype(np.float64), lam.astype(np.float64)))
    err = np.abs(x - want)
    assert np.all(err <= 4e-7 * (np.abs(want) + shift) + 1e-30), float(err.max())


def test_augment_clamps_out_of_range_offsets(orc):
    a = I.augment_inputs(23, 4, 256, 300)
    a.crop[:] = np.array([[-5, 1000, 0], [999, -3, 1], [29, 73, 1], [-1, -1, 0]], np.int32)
    lam, vec = pca_basis(orc, a)
    got = host(gpu_augment(a, lam, vec, B.BF16))
    clamped = I.AugInputs(a.seed, a.bf16, a.src, np.array([[0, 73, 0], [29, 0, 1], [29, 73, 1], [0, 0, 0]],
                                                            np.int32), a.alpha, a.labels)
    want = host(gpu_augment(clamped, lam, vec, B.BF16))
    assert np.array_equal(got, want)
    check_bf16(torch.from_numpy(got), oracle_augment(orc, a, lam, vec))


def run_train(a: I.AugInputs, syn, eigval, eigvec, fused: bool):
    n, _, hs, ws = a.src.shape
    say(f"[gpu] train {'augmented' if fused else 'on materialised patches'} batch={n}")
    sess = Session(n, 1, B.BF16, B.MODE_TRAIN, DEV)
    master = params_f32(syn.master_w, syn.biases)
    mom = [torch.zeros_like(m) for m in master]
    work = [torch.empty(m.shape, dtype=torch.bfloat16, device=DEV) for m in master]
    B.alexnet_cast_weights(sess.cfg, master, work, stream_handle())
    labels = torch.from_numpy(a.labels.astype(np.int32)).to(DEV)
    loss = torch.zeros(1, dtype=torch.float32, device=DEV)
    probs = torch.empty((n, 1000), dtype=torch.float32, device=DEV)
    keep, aug = dev_aug(a, eigval, eigvec)
    src = to_device(a.src, B.BF16, DEV)
    hyper = (0.01, 0.9, 5e-4, 3, 0)
    if fused:
        B.alexnet_train_step_augmented(sess.cfg, master, mom, work, src, hs, ws, aug, labels, *hyper, loss,
                                       probs, sess.ws, sess.ws_bytes, stream_handle())
    else:
        x = torch.empty((n, 3, 227, 227), dtype=torch.bfloat16, device=DEV)
        B.alexnet_augment_images(sess.cfg, src, hs, ws, aug, x, stream_handle())
        B.alexnet_train_step(sess.cfg, master, mom, work, x, labels, *hyper, loss, probs, sess.ws,
                             sess.ws_bytes, stream_handle())
    torch.cuda.synchronize()
    out = dict(loss=loss.clone(), probs=probs.clone(), master=[m.clone() for m in master],
               mom=[v.clone() for v in mom], work=[w.clone() for w in work],
               taps={k: sess.tap(k).clone() for k in ("conv1", "pool1", "dconv1", "gw1", "gb1", "gw2")})
    del sess
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("batch", [4, 128])
def test_train_step_augmented_equals_materialised(orc, batch):
    a = I.augment_inputs(24, batch)
    syn = I.synthetic(3, batch)
    lam, vec = pca_basis(orc, a)
    f = run_train(a, syn, lam, vec, fused=True)
    m = run_train(a, syn, lam, vec, fused=False)
    assert torch.equal(f["loss"], m["loss"]) and torch.equal(f["probs"], m["probs"])
    for k in f["taps"]:
        assert torch.equal(f["taps"][k], m["taps"][k]), k
    for i in range(16):
        assert torch.equal(f["master"][i], m["master"][i]), i
        assert torch.equal(f["mom"][i], m["mom"][i]), i
        assert torch.equal(f["work"][i], m["work"][i]), i
    assert np.isfinite(float(f["loss"].item()))


def gpu_pca(images: np.ndarray, dtype):
    n, _, h, w = images.shape
    say(f"[gpu] rgb_pca n={n} {h}x{w} dtype={dtype}")
    cfg = B.alexnet_default_cfg(1, 1, dtype)
    x = to_device(images, dtype, DEV)
    lam = torch.empty(3, dtype=torch.float32, device=DEV)
    vec = torch.empty(9, dtype=torch.float32, device=DEV)
    nb = B.alexnet_rgb_pca_workspace_bytes()
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    B.alexnet_rgb_pca(cfg, x, n, h, w, lam, vec, ws, nb, stream_handle())
    torch.cuda.synchronize()
    return host(lam), host(vec).reshape(3, 3)


@pytest.mark.parametrize("dtype,n,h,w", [(B.BF16, 128, 256, 256), (B.BF16, 3, 31, 17), (B.F32, 4, 256, 256)])
def test_rgb_pca(orc, dtype, n, h, w):
    a = I.augment_inputs(25, n, max(h, 227), max(w, 227), bf16=dtype == B.BF16)
    imgs = np.ascontiguousarray(a.src[:, :, :h, :w])
    lam, vec = gpu_pca(imgs, dtype)
    want_lam, want_vec, _ = orc.rgb_pca(imgs)
    say(f"[gpu] rgb_pca eigenvalues {lam} oracle {want_lam}")
    assert np.allclose(lam, want_lam, rtol=1e-6, atol=0)
    assert np.allclose(vec, want_vec, rtol=0, atol=1e-5)


def test_rgb_pca_degenerate_inputs(orc):
    # a constant image: zero covariance, all eigenvalues 0
    lam, vec = gpu_pca(np.full((2, 3, 8, 8), 0.75, np.float32), B.BF16)
    assert np.array_equal(lam, np.zeros(3))
    assert np.allclose(vec.T @ vec, np.eye(3), atol=1e-6)
    # one pixel
    lam, _ = gpu_pca(np.array([1.0, 2.0, 3.0], np.float32).reshape(1, 3, 1, 1), B.F32)
    assert np.array_equal(lam, np.zeros(3))
