"""Pins of the oracle's training-time augmentation and RGB principal
components (paper-graph-ui "Data Augmentation", Forms 1 and 2; the paper's
section 4.1) against values fixed by the definitions themselves: identity and
mirror cases, the ten-view crops, closed-form colour shifts, and images whose
colour covariance is known exactly."""
import numpy as np
import pytest

from oracle import lib as L

RNG = np.random.default_rng(12)
ZERO3 = np.zeros(3)
EYE = np.eye(3)


def test_identity_patch_is_the_source():
    src = RNG.standard_normal((2, 3, 227, 227))
    out = L.augment(src, np.zeros((2, 3), np.int32), np.zeros((2, 3)), EYE, np.ones(3))
    assert np.array_equal(out, src)


def test_patch_offsets_and_mirror():
    src = RNG.standard_normal((2, 3, 240, 251))
    crop = np.array([[5, 17, 0], [13, 24, 1]], np.int32)
    out = L.augment(src, crop, np.zeros((2, 3)), EYE, np.ones(3))
    assert np.array_equal(out[0], src[0, :, 5:232, 17:244])
    assert np.array_equal(out[1], src[1, :, 13:240, 24:251][:, :, ::-1])


def test_mirror_twice_restores():
    src = RNG.standard_normal((1, 3, 227, 227))
    f = np.array([[0, 0, 1]], np.int32)
    once = L.augment(src, f, np.zeros((1, 3)), EYE, np.ones(3))
    assert not np.array_equal(once, src)
    assert np.array_equal(L.augment(once, f, np.zeros((1, 3)), EYE, np.ones(3)), src)


def test_tenview_crops_are_special_cases():
    src = RNG.standard_normal((2, 3, 256, 256))
    views = L.tenview_crop(src)
    offs = [(0, 0), (0, 29), (29, 0), (29, 29), (14, 14)]
    for n in range(2):
        for v in range(10):
            y0, x0 = offs[v % 5]
            crop = np.array([[y0, x0, 1 if v >= 5 else 0]], np.int32)
            out = L.augment(src[n:n + 1], crop, np.zeros((1, 3)), EYE, np.ones(3))
            assert np.array_equal(out[0], views[n * 10 + v])


def test_out_of_range_offsets_clamp_to_the_edge():
    src = RNG.standard_normal((1, 3, 256, 300))
    a = L.augment(src, np.array([[-7, 999, 0]], np.int32), np.zeros((1, 3)), EYE, np.ones(3))
    b = L.augment(src, np.array([[0, 73, 0]], np.int32), np.zeros((1, 3)), EYE, np.ones(3))
    assert np.array_equal(a, b)


def test_colour_shift_closed_form():
    # constant image: every pixel of channel c becomes k_c + sum_i P[c][i] a_i l_i
    k = np.array([0.5, -1.0, 2.0])
    src = np.broadcast_to(k[None, :, None, None], (1, 3, 230, 230)).copy()
    P = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 1.0], [0.0, 1.0, 0.0]])   # columns p_1 = e_r, p_2 = e_b, p_3 = e_g
    lam = np.array([1.0, 2.0, 3.0])
    alpha = np.array([[0.1, -0.2, 0.3]])
    out = L.augment(src, np.array([[1, 2, 1]], np.int32), alpha, P, lam)
    # shift: r += 0.1*1, b += -0.2*2, g += 0.3*3
    want = k + np.array([0.1, 0.9, -0.4])
    for c in range(3):
        assert np.allclose(out[0, c], want[c], rtol=0, atol=1e-15)


def test_shift_is_linear_in_alpha():
    src = RNG.standard_normal((1, 3, 227, 227))
    P, _ = np.linalg.qr(RNG.standard_normal((3, 3)))
    lam = np.array([0.9, 0.3, 0.05])
    a1, a2 = RNG.standard_normal((1, 3)) * 0.1, RNG.standard_normal((1, 3)) * 0.1
    z = np.zeros((1, 3), np.int32)
    base = L.augment(src, z, np.zeros((1, 3)), P, lam)
    d1 = L.augment(src, z, a1, P, lam) - base
    d2 = L.augment(src, z, a2, P, lam) - base
    d12 = L.augment(src, z, a1 + a2, P, lam) - base
    assert np.allclose(d1 + d2, d12, rtol=0, atol=1e-14)
    # the shift is the same at every pixel of a channel
    assert np.allclose(d1, d1[:, :, :1, :1], rtol=0, atol=1e-14)


def _pattern_images(mix, offset, h=6, w=8):
    """Channels = mix @ (u1, u2, u3) + offset with u1 = (-1)^(y+x),
    u2 = (-1)^y, u3 = (-1)^x: zero-mean, unit-variance, mutually orthogonal
    patterns over an even grid, so the RGB covariance is exactly mix mix^T."""
    y, x = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    u = np.stack([(-1.0) ** (y + x), (-1.0) ** y, (-1.0) ** x])
    img = np.einsum("ck,khw->chw", mix, u) + np.asarray(offset)[:, None, None]
    return img[None]


def test_pca_recovers_a_known_covariance():
    R, _ = np.linalg.qr(np.array([[2.0, 1.0, 0.5], [0.3, -1.0, 2.0], [1.0, 0.2, -0.7]]))
    s = np.array([1.5, 0.6, 0.2])
    imgs = np.concatenate([_pattern_images(R @ np.diag(s), [0.3, -2.0, 5.0]),
                           _pattern_images(R @ np.diag(s), [0.3, -2.0, 5.0])])
    lam, vec, cov = L.rgb_pca(imgs)
    assert np.allclose(cov, R @ np.diag(s ** 2) @ R.T, rtol=0, atol=1e-13)
    assert np.allclose(lam, s ** 2, rtol=0, atol=1e-13)
    for i in range(3):
        r = R[:, i] * np.sign(R[np.argmax(np.abs(R[:, i])), i])
        assert np.allclose(vec[:, i], r, rtol=0, atol=1e-10)
    # unit vectors, largest entry positive, descending eigenvalues
    assert np.allclose(vec.T @ vec, EYE, atol=1e-12)
    assert all(vec[np.argmax(np.abs(vec[:, i])), i] > 0 for i in range(3))
    assert lam[0] >= lam[1] >= lam[2]


def test_pca_two_pixel_closed_form():
    # pixels (0,0,0) and (2,2,2): mean (1,1,1), covariance = all-ones matrix,
    # eigenvalues 3, 0, 0; the top component is (1,1,1)/sqrt(3)
    img = np.zeros((1, 3, 1, 2))
    img[0, :, 0, 1] = 2.0
    lam, vec, cov = L.rgb_pca(img)
    assert np.allclose(cov, np.ones((3, 3)), rtol=0, atol=1e-15)
    assert np.allclose(lam, [3.0, 0.0, 0.0], rtol=0, atol=1e-14)
    assert np.allclose(vec[:, 0], np.ones(3) / np.sqrt(3), rtol=0, atol=1e-14)


def test_pca_four_pixel_closed_form():
    # (1,0,0), (0,1,0), (0,0,1), (1,1,1): centred vectors +-0.5 with zero
    # cross terms, covariance 0.25 I
    img = np.zeros((1, 3, 2, 2))
    img[0, 0, 0, 0] = img[0, 1, 0, 1] = img[0, 2, 1, 0] = 1.0
    img[0, :, 1, 1] = 1.0
    lam, _, cov = L.rgb_pca(img)
    assert np.allclose(cov, 0.25 * EYE, rtol=0, atol=1e-15)
    assert np.allclose(lam, 0.25, rtol=0, atol=1e-15)


@pytest.mark.parametrize("scale", [1.0, 1e-3, 1e3])
def test_pca_shift_and_scale(scale):
    # adding a constant colour leaves the covariance alone; scaling scales it by scale^2
    imgs = RNG.standard_normal((2, 3, 5, 7))
    lam0, vec0, cov0 = L.rgb_pca(imgs)
    lam1, vec1, cov1 = L.rgb_pca(imgs * scale + np.array([1.0, -3.0, 0.5])[None, :, None, None])
    assert np.allclose(cov1, cov0 * scale ** 2, rtol=1e-9, atol=0)
    assert np.allclose(lam1, lam0 * scale ** 2, rtol=1e-9, atol=0)
    assert np.allclose(vec1, vec0, rtol=0, atol=1e-8)
