"""Pins of the CPU oracle's per-layer functions against things other than itself:
torch float64 library routines, closed forms, invariants, central differences
and hand-worked values.  CPU only."""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------- conv
CONV_CASES = [
    # N, Cin, H, W, Cout, K, stride, pad, G
    (2, 2, 5, 5, 3, 3, 1, 0, 1),
    (1, 2, 5, 5, 4, 3, 2, 1, 2),
    (2, 3, 23, 23, 5, 11, 4, 0, 1),     # conv1 geometry, small
    (1, 4, 9, 9, 6, 5, 1, 2, 2),        # conv2 geometry, grouped
    (2, 6, 7, 7, 4, 3, 1, 1, 2),        # conv4/5 geometry, grouped
    (1, 3, 8, 6, 2, 3, 1, 1, 1),        # non-square
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_fwd_matches_torch(orc, case):
    N, Cin, H, W, Cout, K, s, p, G = case
    rng = np.random.default_rng(1)
    x = rng.standard_normal((N, Cin, H, W))
    w = rng.standard_normal((Cout, Cin // G, K, K))
    b = rng.standard_normal(Cout)
    y = orc.conv2d(x, w, b, s, p, G)
    ref = F.conv2d(_t(x), _t(w), _t(b), stride=s, padding=p, groups=G).numpy()
    assert y.shape == ref.shape
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CONV_CASES)
def test_conv_bwd_matches_torch_autograd(orc, case):
    N, Cin, H, W, Cout, K, s, p, G = case
    rng = np.random.default_rng(2)
    x = rng.standard_normal((N, Cin, H, W))
    w = rng.standard_normal((Cout, Cin // G, K, K))
    b = rng.standard_normal(Cout)
    xt, wt, bt = (_t(a).requires_grad_() for a in (x, w, b))
    yt = F.conv2d(xt, wt, bt, stride=s, padding=p, groups=G)
    dy = rng.standard_normal(tuple(yt.shape))
    yt.backward(_t(dy))
    dx = orc.conv2d_bwd_data(dy, w, x.shape, s, p, G)
    dw, db = orc.conv2d_bwd_weight(dy, x, w.shape, s, p, G)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-11, atol=1e-11)


def test_conv_delta_kernel_shifts_input(orc):
    """A kernel that is 1 at (kh, kw) and 0 elsewhere copies the input shifted
    by (kh - p, kw - p), with zeros where the shift leaves the image."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 1, 6, 7))
    for kh, kw in [(0, 0), (1, 2), (2, 1)]:
        w = np.zeros((1, 1, 3, 3))
        w[0, 0, kh, kw] = 1.0
        y = orc.conv2d(x, w, None, 1, 1, 1)
        exp = np.zeros_like(x)
        for h in range(6):
            for ww in range(7):
                hi, wi = h + kh - 1, ww + kw - 1
                if 0 <= hi < 6 and 0 <= wi < 7:
                    exp[0, 0, h, ww] = x[0, 0, hi, wi]
        np.testing.assert_array_equal(y, exp)


def test_conv_constant_input_closed_form(orc):
    """Constant input c: interior outputs equal b + c * sum(W); with padding the
    border outputs see only the in-image part of the kernel."""
    c = 0.75
    x = np.full((1, 2, 7, 7), c)
    w = np.arange(2 * 2 * 3 * 3, dtype=np.float64).reshape(2, 2, 3, 3) / 10.0
    b = np.array([0.5, -1.0])
    y = orc.conv2d(x, w, b, 1, 1, 1)
    for co in range(2):
        assert np.allclose(y[0, co, 1:-1, 1:-1], b[co] + c * w[co].sum(), rtol=0, atol=1e-13)
        # corner (0,0): only kernel rows/cols 1..2 are in the image
        assert math.isclose(y[0, co, 0, 0], b[co] + c * w[co, :, 1:, 1:].sum(), abs_tol=1e-13)


def test_conv_grouped_blocks_cross_group(orc):
    """groups=2: an output of group 0 does not change when group-1 inputs do."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((1, 4, 6, 6))
    w = rng.standard_normal((6, 2, 3, 3))
    y0 = orc.conv2d(x, w, None, 1, 1, 2)
    x2 = x.copy()
    x2[:, 2:] += 5.0
    y1 = orc.conv2d(x2, w, None, 1, 1, 2)
    np.testing.assert_array_equal(y0[:, :3], y1[:, :3])
    assert not np.allclose(y0[:, 3:], y1[:, 3:])


def test_conv_bwd_central_differences(orc):
    """Backward pinned independently of torch: central differences of
    L = sum(dy * conv(x, w, b))."""
    rng = np.random.default_rng(5)
    N, Cin, H, W, Cout, K, s, p, G = 1, 4, 9, 9, 4, 3, 2, 1, 2
    x = rng.standard_normal((N, Cin, H, W))
    w = rng.standard_normal((Cout, Cin // G, K, K))
    b = rng.standard_normal(Cout)
    dy = rng.standard_normal(orc.conv2d(x, w, b, s, p, G).shape)
    f = lambda xx, ww, bb: float((orc.conv2d(xx, ww, bb, s, p, G) * dy).sum())
    dx = orc.conv2d_bwd_data(dy, w, x.shape, s, p, G)
    dw, db = orc.conv2d_bwd_weight(dy, x, w.shape, s, p, G)
    h = 1e-6
    for idx in [(0, 0, 0, 0), (0, 3, 4, 5), (0, 2, 8, 8)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += h; xm[idx] -= h
        assert math.isclose((f(xp, w, b) - f(xm, w, b)) / (2 * h), dx[idx], rel_tol=1e-6, abs_tol=1e-8)
    for idx in [(0, 0, 0, 0), (3, 1, 2, 1)]:
        wp, wm = w.copy(), w.copy()
        wp[idx] += h; wm[idx] -= h
        assert math.isclose((f(x, wp, b) - f(x, wm, b)) / (2 * h), dw[idx], rel_tol=1e-6, abs_tol=1e-8)
    bp, bm = b.copy(), b.copy()
    bp[2] += h; bm[2] -= h
    assert math.isclose((f(x, w, bp) - f(x, w, bm)) / (2 * h), db[2], rel_tol=1e-6)


# --------------------------------------------------------------------------- relu
def test_relu_invariants(orc):
    rng = np.random.default_rng(6)
    x = rng.standard_normal(1000)
    x[:5] = 0.0
    y = orc.relu(x)
    assert (y >= 0).all()
    np.testing.assert_array_equal(y[x > 0], x[x > 0])
    assert (y[x <= 0] == 0).all()
    g = rng.standard_normal(1000)
    gz = orc.relu_bwd(y, g)
    np.testing.assert_array_equal(gz[x > 0], g[x > 0])
    assert (gz[x <= 0] == 0).all()        # subgradient 0 at 0


# --------------------------------------------------------------------------- LRN
def test_lrn_matches_torch(orc):
    rng = np.random.default_rng(7)
    a = np.abs(rng.standard_normal((2, 11, 4, 5))) * 30.0
    b = orc.lrn(a, k=2.0, alpha=1e-4, beta=0.75, n=5)
    # torch divides alpha by the window size; the pages' formula does not.
    ref = F.local_response_norm(_t(a), size=5, alpha=5 * 1e-4, beta=0.75, k=2.0).numpy()
    np.testing.assert_allclose(b, ref, rtol=1e-12)


def test_lrn_closed_forms(orc):
    k, alpha, beta = 2.0, 1e-4, 0.75
    # zero input -> zero
    assert (orc.lrn(np.zeros((1, 8, 2, 2))) == 0).all()
    # single active channel i: b_i = a/(k + alpha a^2)^beta; neighbours stay 0
    a = np.zeros((1, 8, 1, 1)); a[0, 3] = 40.0
    b = orc.lrn(a)
    assert math.isclose(b[0, 3, 0, 0], 40.0 / (k + alpha * 1600.0) ** beta, rel_tol=1e-14)
    assert (np.delete(b[0, :, 0, 0], 3) == 0).all()
    # constant c on all N channels: window holds 3, 4, 5, 5, ..., 5, 4, 3 channels
    c = 25.0
    a = np.full((1, 9, 1, 1), c)
    b = orc.lrn(a)[0, :, 0, 0]
    counts = [3, 4, 5, 5, 5, 5, 5, 4, 3]
    for i, m in enumerate(counts):
        assert math.isclose(b[i], c / (k + alpha * m * c * c) ** beta, rel_tol=1e-14)


@pytest.mark.parametrize("params", [dict(k=2.0, alpha=1e-4, beta=0.75, n=5),
                                    dict(k=1.0, alpha=0.3, beta=0.75, n=5),
                                    dict(k=0.5, alpha=0.7, beta=1.3, n=3)])
def test_lrn_bwd_matches_torch_autograd(orc, params):
    rng = np.random.default_rng(8)
    a = np.abs(rng.standard_normal((2, 10, 3, 3))) * 3.0
    g = rng.standard_normal(a.shape)
    at = _t(a).requires_grad_()
    n = params["n"]
    out = F.local_response_norm(at, size=n, alpha=params["alpha"] * n, beta=params["beta"], k=params["k"])
    out.backward(_t(g))
    da = orc.lrn_bwd(a, g, **params)
    np.testing.assert_allclose(da, at.grad.numpy(), rtol=1e-10, atol=1e-12)


def test_lrn_bwd_central_differences(orc):
    rng = np.random.default_rng(9)
    prm = dict(k=1.0, alpha=0.4, beta=0.75, n=5)
    a = np.abs(rng.standard_normal((1, 7, 2, 2))) * 2.0
    g = rng.standard_normal(a.shape)
    da = orc.lrn_bwd(a, g, **prm)
    f = lambda aa: float((orc.lrn(aa, **prm) * g).sum())
    h = 1e-6
    for idx in [(0, 0, 0, 0), (0, 3, 1, 0), (0, 6, 1, 1)]:
        ap, am = a.copy(), a.copy()
        ap[idx] += h; am[idx] -= h
        assert math.isclose((f(ap) - f(am)) / (2 * h), da[idx], rel_tol=1e-6, abs_tol=1e-9)


# --------------------------------------------------------------------------- pool
def test_pool_matches_torch_on_tie_free_input(orc):
    rng = np.random.default_rng(10)
    x = rng.permutation(2 * 3 * 13 * 13).reshape(2, 3, 13, 13).astype(np.float64)
    y, am = orc.maxpool(x, 3, 2)
    ref, idx = F.max_pool2d(_t(x), 3, 2, return_indices=True)
    np.testing.assert_array_equal(y, ref.numpy())
    Ho = y.shape[2]
    ii, jj = np.meshgrid(np.arange(Ho), np.arange(Ho), indexing="ij")
    flat = (2 * ii + am // 3) * 13 + (2 * jj + am % 3)
    np.testing.assert_array_equal(flat, idx.numpy())


def test_pool_sizes_and_overlap(orc):
    for H, Ho in [(55, 27), (27, 13), (13, 6)]:
        y, _ = orc.maxpool(np.zeros((1, 1, H, H)), 3, 2)
        assert y.shape[-1] == Ho
    # adjacent windows share exactly one column: a single large value at column 2
    # (row 0) is the max of output windows j=0 and j=1.
    x = np.zeros((1, 1, 5, 5)); x[0, 0, 0, 2] = 9.0
    y, am = orc.maxpool(x, 3, 2)
    assert y[0, 0, 0, 0] == 9.0 and y[0, 0, 0, 1] == 9.0
    assert am[0, 0, 0, 0] == 2 and am[0, 0, 0, 1] == 0


def test_pool_invariants_and_tie_rule(orc):
    rng = np.random.default_rng(11)
    x = np.round(rng.standard_normal((2, 4, 27, 27)) * 2) / 2   # many ties
    y, am = orc.maxpool(x, 3, 2)
    for n, c, i, j in [(0, 0, 0, 0), (1, 3, 12, 12), (0, 2, 5, 7)]:
        win = x[n, c, 2 * i:2 * i + 3, 2 * j:2 * j + 3].ravel()
        assert y[n, c, i, j] == win.max()
        assert win[am[n, c, i, j]] == y[n, c, i, j]
        assert am[n, c, i, j] == int(np.argmax(win))            # first maximum
    yc, amc = orc.maxpool(np.full((1, 2, 13, 13), 3.0), 3, 2)
    assert (amc == 0).all() and (yc == 3.0).all()


def test_pool_bwd(orc):
    rng = np.random.default_rng(12)
    x = rng.permutation(3 * 27 * 27).reshape(1, 3, 27, 27).astype(np.float64)
    xt = _t(x).requires_grad_()
    yt = F.max_pool2d(xt, 3, 2)
    g = rng.standard_normal(tuple(yt.shape))
    yt.backward(_t(g))
    _, am = orc.maxpool(x, 3, 2)
    dx = orc.maxpool_bwd(g, am, x.shape, 3, 2)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-14, atol=1e-14)
    assert math.isclose(dx.sum(), g.sum(), rel_tol=1e-12)      # gradient is routed, not created


# --------------------------------------------------------------------------- fc, softmax, loss
def test_fc_fwd_bwd_matches_torch(orc):
    rng = np.random.default_rng(13)
    x, w, b = rng.standard_normal((5, 17)), rng.standard_normal((9, 17)), rng.standard_normal(9)
    xt, wt, bt = (_t(a).requires_grad_() for a in (x, w, b))
    yt = F.linear(xt, wt, bt)
    np.testing.assert_allclose(orc.fc(x, w, b), yt.detach().numpy(), rtol=1e-13)
    dy = rng.standard_normal((5, 9))
    yt.backward(_t(dy))
    dx, dw, db = orc.fc_bwd(dy, x, w)
    np.testing.assert_allclose(dx, xt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(db, bt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_softmax_distribution_and_shift(orc):
    rng = np.random.default_rng(14)
    z = rng.standard_normal((4, 1000)) * 5
    p = orc.softmax(z)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=0, atol=1e-14)
    assert (p > 0).all()
    np.testing.assert_allclose(orc.softmax(z + 123.0), p, rtol=1e-12)
    np.testing.assert_allclose(p, torch.softmax(_t(z), 1).numpy(), rtol=1e-12)


def test_softmax_worked_example_from_pages(orc):
    g = json.load(open(os.path.join(GOLDEN, "softmax_logit_pair.json")))
    rng = np.random.default_rng(15)
    lo, hi = g["others_range"]
    z = rng.uniform(lo, hi, (1, g["classes"]))
    for k, v in g["logits"].items():
        z[0, int(k)] = v
    p = orc.softmax(z)[0]
    assert math.isclose(p[250] / p[248], math.exp(8.7 - 7.9), rel_tol=1e-12)
    assert p.argmax() == 250 and np.argsort(p)[-2] == 248


def test_cross_entropy_matches_torch(orc):
    rng = np.random.default_rng(16)
    z = rng.standard_normal((6, 1000)) * 3
    y = rng.integers(0, 1000, 6).astype(np.int32)
    zt = _t(z).requires_grad_()
    lt = F.cross_entropy(zt, torch.from_numpy(y.astype(np.int64)))
    lt.backward()
    loss, dz = orc.ce_loss_grad(orc.softmax(z), y)
    assert math.isclose(loss, lt.item(), rel_tol=1e-12)
    np.testing.assert_allclose(dz, zt.grad.numpy(), rtol=1e-10, atol=1e-15)


def test_cross_entropy_uniform_closed_form(orc):
    p = np.full((4, 1000), 1e-3)
    y = np.array([0, 5, 999, 3], np.int32)
    loss, dz = orc.ce_loss_grad(p, y)
    assert math.isclose(loss, math.log(1000.0), rel_tol=1e-12)
    exp = np.full((4, 1000), 1e-3 / 4)
    exp[np.arange(4), y] = (1e-3 - 1.0) / 4
    np.testing.assert_allclose(dz, exp, rtol=1e-12)


# --------------------------------------------------------------------------- sgd
def test_sgd_closed_forms(orc):
    lr, mu, wd = 0.01, 0.9, 5e-4
    w = np.array([1.0, -2.0, 0.5])
    # g = 0, v = 0 -> pure weight decay: w1 = w (1 - lr wd)
    w1, v1 = orc.sgd(w, np.zeros(3), np.zeros(3), lr, mu, wd)
    np.testing.assert_allclose(w1, w * (1 - lr * wd), rtol=1e-15)
    # w = 0, v = 0 -> v1 = -lr g
    g = np.array([3.0, -1.0, 0.25])
    w1, v1 = orc.sgd(np.zeros(3), np.zeros(3), g, lr, mu, wd)
    np.testing.assert_allclose(v1, -lr * g, rtol=1e-15)
    np.testing.assert_allclose(w1, v1, rtol=1e-15)


def test_sgd_two_steps_by_hand(orc):
    g = json.load(open(os.path.join(GOLDEN, "sgd_two_steps.json")))
    w, v = np.array([g["w0"]]), np.array([g["v0"]])
    w, v = orc.sgd(w, v, np.array([g["grads"][0]]), g["lr"], g["momentum"], g["weight_decay"])
    assert math.isclose(v[0], g["v1"], rel_tol=1e-13) and math.isclose(w[0], g["w1"], rel_tol=1e-13)
    w, v = orc.sgd(w, v, np.array([g["grads"][1]]), g["lr"], g["momentum"], g["weight_decay"])
    assert math.isclose(v[0], g["v2"], rel_tol=1e-12) and math.isclose(w[0], g["w2"], rel_tol=1e-12)


# --------------------------------------------------------------------------- philox / dropout
def test_dropout_mask_statistics(orc):
    """The bit stream itself is pinned in test_oracle_philox.py; these pin the
    mask semantics: keep probability 1/2, independence across layers, steps, seeds
    and neighbouring elements, determinism."""
    rows, cols = 128, 4096
    n = rows * cols
    sigma = math.sqrt(n * 0.25)
    m0 = orc.dropout_mask(3, 0, 0, rows, cols, 0.5)
    m1 = orc.dropout_mask(3, 0, 1, rows, cols, 0.5)
    m2 = orc.dropout_mask(3, 1, 0, rows, cols, 0.5)
    m3 = orc.dropout_mask(4, 0, 0, rows, cols, 0.5)
    for m in (m0, m1, m2, m3):
        assert set(np.unique(m)) <= {0, 1}
        assert abs(int(m.sum()) - n / 2) < 5 * sigma
    for a, b in ((m0, m1), (m0, m2), (m0, m3), (m1, m2)):
        agree = int((a == b).sum())
        assert abs(agree - n / 2) < 5 * sigma
    f = m0.ravel().astype(np.int64)
    same_next = int((f[1:] == f[:-1]).sum())
    assert abs(same_next - (n - 1) / 2) < 5 * math.sqrt((n - 1) * 0.25)
    np.testing.assert_array_equal(m0, orc.dropout_mask(3, 0, 0, rows, cols, 0.5))
    # p controls the drop rate
    q = orc.dropout_mask(3, 0, 0, rows, cols, 0.25)
    assert abs(int((q == 0).sum()) - n / 4) < 5 * math.sqrt(n * 0.1875)


def test_philox_output_words_uniform(orc):
    """Byte histogram of 4096 Philox blocks is uniform (chi-square, 255 dof)."""
    words = []
    for i in range(4096):
        words.append(orc.philox4x32_10([i, 7, 0, 0], [3, 0]))
    b = np.array(words, np.uint32).ravel().view(np.uint8)
    hist = np.bincount(b, minlength=256)
    exp = b.size / 256
    chi2 = float(((hist - exp) ** 2 / exp).sum())
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)
    # a single-bit change of the counter or the key changes every word
    base = orc.philox4x32_10([1, 2, 3, 4], [5, 6])
    for ctr, key in (([1, 2, 3, 5], [5, 6]), ([1, 2, 3, 4], [5, 7])):
        assert (orc.philox4x32_10(ctr, key) != base).all()


# --------------------------------------------------------------------------- ten-view
def test_tenview_offsets_and_mirrors(orc):
    S, P = 256, 227
    yy, xx = np.meshgrid(np.arange(S), np.arange(S), indexing="ij")
    src = np.stack([yy * 1000.0 + xx, -(yy * 1000.0 + xx)])[None]      # [1, 2, S, S]
    v = orc.tenview_crop(src, P)
    assert v.shape == (10, 2, P, P)
    corners = [(0, 0), (0, 29), (29, 0), (29, 29), (14, 14)]
    for i, (y0, x0) in enumerate(corners):
        assert v[i, 0, 0, 0] == y0 * 1000 + x0
        assert v[i, 0, P - 1, P - 1] == (y0 + P - 1) * 1000 + x0 + P - 1
        assert v[5 + i, 0, 0, 0] == y0 * 1000 + x0 + P - 1                 # mirrored
        assert v[5 + i, 0, 3, P - 1] == (y0 + 3) * 1000 + x0
        assert v[5 + i, 1, 0, 0] == -(y0 * 1000 + x0 + P - 1)


def test_tenview_constant_image(orc):
    src = np.full((2, 3, 256, 256), 0.25)
    v = orc.tenview_crop(src)
    assert (v == 0.25).all()
    p = np.random.default_rng(17).random((20, 7))
    p = np.tile(p[:1], (10, 1))
    p = np.concatenate([p, np.tile(np.arange(7.0)[None], (10, 1))])
    m = orc.view_mean(p)
    np.testing.assert_allclose(m[0], p[0], rtol=1e-15)
    np.testing.assert_allclose(m[1], np.arange(7.0), rtol=1e-15)
