"""ctypes bindings for oracle/liboracle.so (float64 NumPy in, float64 NumPy out).

Test infrastructure only; see the package docstring.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# ORACLE_LIB selects another build of the same source (the sanitizer test uses it)
_LIB_PATH = os.environ.get("ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_D = C.POINTER(C.c_double)
_U8 = C.POINTER(C.c_uint8)
_U32 = C.POINTER(C.c_uint32)
_I32 = C.POINTER(C.c_int32)
_i = C.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build(verbose=False)
    lib = C.CDLL(_LIB_PATH)
    sig = {
        "orc_conv2d_fwd": [_D, _i, _i, _i, _i, _D, _D, _i, _i, _i, _i, _i, _D],
        "orc_conv2d_bwd_data": [_D, _i, _i, _i, _i, _D, _i, _i, _i, _i, _i, _D],
        "orc_conv2d_bwd_weight": [_D, _D, _i, _i, _i, _i, _i, _i, _i, _i, _i, _D, _D],
        "orc_relu": [_D, C.c_int64, _D],
        "orc_relu_bwd": [_D, _D, C.c_int64, _D],
        "orc_lrn_fwd": [_D, _i, _i, _i, C.c_double, C.c_double, C.c_double, _i, _D],
        "orc_lrn_bwd": [_D, _D, _i, _i, _i, C.c_double, C.c_double, C.c_double, _i, _D],
        "orc_maxpool_fwd": [_D, _i, _i, _i, _i, _i, _i, _D, _U8],
        "orc_maxpool_bwd": [_D, _U8, _i, _i, _i, _i, _i, _i, _D],
        "orc_fc_fwd": [_D, _i, _i, _D, _D, _i, _D],
        "orc_fc_bwd": [_D, _D, _D, _i, _i, _i, _D, _D, _D],
        "orc_softmax": [_D, _i, _i, _D],
        "orc_ce_loss_grad": [_D, _I32, _i, _i, _D],
        "orc_sgd": [_D, _D, _D, C.c_int64, C.c_double, C.c_double, C.c_double],
        "orc_philox4x32_10": [_U32, _U32, _U32],
        "orc_dropout_mask": [C.c_uint64, C.c_uint64, _i, _i, _i, C.c_double, _U8],
        "orc_tenview_crop": [_D, _i, _i, _i, _i, _D],
        "orc_view_mean": [_D, _i, _i, _D],
        "orc_augment": [_D, _i, _i, _i, _i, _I32, _D, _D, _D, _i, _D],
        "orc_num_threads": [],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = None
    lib.orc_ce_loss_grad.restype = C.c_double
    lib.orc_num_threads.restype = C.c_int
    _lib = lib
    return lib


def _d(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: np.ndarray, t=_D):
    return a.ctypes.data_as(t)


def num_threads() -> int:
    return _load().orc_num_threads()


def conv2d(x, w, b, stride, pad, groups=1):
    x, w = _d(x), _d(w)
    N, Cin, H, W = x.shape
    Cout, _, K, _ = w.shape
    Ho, Wo = (H + 2 * pad - K) // stride + 1, (W + 2 * pad - K) // stride + 1
    y = np.empty((N, Cout, Ho, Wo), np.float64)
    bb = None if b is None else _d(b)
    _load().orc_conv2d_fwd(_p(x), N, Cin, H, W, _p(w), None if bb is None else _p(bb),
                           Cout, K, stride, pad, groups, _p(y))
    return y


def conv2d_bwd_data(dy, w, in_shape, stride, pad, groups=1):
    dy, w = _d(dy), _d(w)
    N, Cin, H, W = in_shape
    Cout, _, K, _ = w.shape
    dx = np.empty((N, Cin, H, W), np.float64)
    _load().orc_conv2d_bwd_data(_p(dy), N, Cin, H, W, _p(w), Cout, K, stride, pad, groups, _p(dx))
    return dx


def conv2d_bwd_weight(dy, x, w_shape, stride, pad, groups=1):
    dy, x = _d(dy), _d(x)
    N, Cin, H, W = x.shape
    Cout, _, K, _ = w_shape
    dw = np.empty(w_shape, np.float64)
    db = np.empty((Cout,), np.float64)
    _load().orc_conv2d_bwd_weight(_p(dy), _p(x), N, Cin, H, W, Cout, K, stride, pad, groups,
                                  _p(dw), _p(db))
    return dw, db


def relu(x):
    x = _d(x)
    y = np.empty_like(x)
    _load().orc_relu(_p(x), x.size, _p(y))
    return y


def relu_bwd(a, g):
    a, g = _d(a), _d(g)
    out = np.empty_like(a)
    _load().orc_relu_bwd(_p(a), _p(g), a.size, _p(out))
    return out


def lrn(a, k=2.0, alpha=1e-4, beta=0.75, n=5):
    a = _d(a)
    N, Cc = a.shape[:2]
    HW = int(np.prod(a.shape[2:])) if a.ndim > 2 else 1
    b = np.empty_like(a)
    _load().orc_lrn_fwd(_p(a), N, Cc, HW, k, alpha, beta, n, _p(b))
    return b


def lrn_bwd(a, g, k=2.0, alpha=1e-4, beta=0.75, n=5):
    a, g = _d(a), _d(g)
    N, Cc = a.shape[:2]
    HW = int(np.prod(a.shape[2:])) if a.ndim > 2 else 1
    da = np.empty_like(a)
    _load().orc_lrn_bwd(_p(a), _p(g), N, Cc, HW, k, alpha, beta, n, _p(da))
    return da


def maxpool(x, z=3, s=2):
    x = _d(x)
    N, Cc, H, W = x.shape
    Ho, Wo = (H - z) // s + 1, (W - z) // s + 1
    y = np.empty((N, Cc, Ho, Wo), np.float64)
    am = np.empty((N, Cc, Ho, Wo), np.uint8)
    _load().orc_maxpool_fwd(_p(x), N, Cc, H, W, z, s, _p(y), _p(am, _U8))
    return y, am


def maxpool_bwd(dy, am, in_shape, z=3, s=2):
    dy = _d(dy)
    am = np.ascontiguousarray(am, dtype=np.uint8)
    N, Cc, H, W = in_shape
    dx = np.empty(in_shape, np.float64)
    _load().orc_maxpool_bwd(_p(dy), _p(am, _U8), N, Cc, H, W, z, s, _p(dx))
    return dx


def fc(x, w, b):
    x, w = _d(x), _d(w)
    M, K = x.shape
    O = w.shape[0]
    y = np.empty((M, O), np.float64)
    bb = None if b is None else _d(b)
    _load().orc_fc_fwd(_p(x), M, K, _p(w), None if bb is None else _p(bb), O, _p(y))
    return y


def fc_bwd(dy, x, w, want_dx=True):
    dy, x, w = _d(dy), _d(x), _d(w)
    M, K = x.shape
    O = w.shape[0]
    dx = np.empty((M, K), np.float64) if want_dx else None
    dw = np.empty((O, K), np.float64)
    db = np.empty((O,), np.float64)
    _load().orc_fc_bwd(_p(dy), _p(x), _p(w), M, K, O, None if dx is None else _p(dx),
                       _p(dw), _p(db))
    return dx, dw, db


def softmax(z):
    z = _d(z)
    M, O = z.shape
    p = np.empty_like(z)
    _load().orc_softmax(_p(z), M, O, _p(p))
    return p


def ce_loss_grad(p, labels):
    p = _d(p)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    M, O = p.shape
    dz = np.empty_like(p)
    loss = _load().orc_ce_loss_grad(_p(p), _p(labels, _I32), M, O, _p(dz))
    return loss, dz


def sgd(w, v, g, lr, momentum, weight_decay):
    """Returns (w_new, v_new); the inputs are not modified."""
    w = _d(w).copy()
    v = _d(v).copy()
    g = _d(g)
    _load().orc_sgd(_p(w), _p(v), _p(g), w.size, lr, momentum, weight_decay)
    return w, v


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.empty(4, np.uint32)
    _load().orc_philox4x32_10(_p(c, _U32), _p(k, _U32), _p(out, _U32))
    return out


def dropout_mask(seed, step, layer, rows, cols, p=0.5):
    m = np.empty((rows, cols), np.uint8)
    _load().orc_dropout_mask(seed, step, layer, rows, cols, p, _p(m, _U8))
    return m


def tenview_crop(src, crop=227):
    src = _d(src)
    N, Cc, S, _ = src.shape
    out = np.empty((N * 10, Cc, crop, crop), np.float64)
    _load().orc_tenview_crop(_p(src), N, Cc, S, crop, _p(out))
    return out


def view_mean(p):
    p = _d(p)
    M, O = p.shape
    out = np.empty((M // 10, O), np.float64)
    _load().orc_view_mean(_p(p), M // 10, O, _p(out))
    return out


def augment(src, crop, alpha, eigvec, eigval, patch=227):
    """Augmented patches of src [N][3][Hs][Ws] (see orc_augment)."""
    src = _d(src)
    N, Cc, Hs, Ws = src.shape
    crop = np.ascontiguousarray(crop, dtype=np.int32).reshape(N, 3)
    out = np.empty((N, Cc, patch, patch), np.float64)
    _load().orc_augment(_p(src), N, Cc, Hs, Ws, _p(crop, _I32), _p(_d(alpha).reshape(N, 3)),
                        _p(_d(eigvec).reshape(3, 3)), _p(_d(eigval).reshape(3)), patch, _p(out))
    return out


def rgb_pca(images):
    """Principal components of the RGB values of every pixel of images [n][3][h][w]
    (paper-graph-ui "Data Augmentation", Form 2, steps 1-2; the paper's
    section 4.1): the 3 x 3 covariance of the pixels' RGB vectors (the mean of
    the outer products of the centred vectors, dividing by the pixel count),
    then its eigenvectors and eigenvalues.  Sums are plain float64 sums over
    all pixels; the eigen-decomposition is LAPACK's
    symmetric solver (numpy.linalg.eigh).  Returned in descending order of
    eigenvalue, each eigenvector (column i of the 3 x 3 result) signed so that
    its largest-magnitude entry is positive (the first such entry on a tie).
    Pinned by: images built from orthogonal patterns with an exactly known
    covariance, and brute force on a tiny image."""
    x = _d(images)
    n, c, h, w = x.shape
    assert c == 3
    pix = np.moveaxis(x, 1, -1).reshape(-1, 3)       # one RGB vector per pixel
    P = pix.shape[0]
    mean = pix.sum(axis=0) / P
    d = pix - mean                                    # centred RGB vectors
    cov = d.T @ d / P
    lam, vec = np.linalg.eigh(cov)
    order = np.argsort(-lam, kind="stable")
    lam, vec = lam[order], vec[:, order]
    for i in range(3):
        big = int(np.argmax(np.abs(vec[:, i])))
        if vec[big, i] < 0:
            vec[:, i] = -vec[:, i]
    return lam, vec, cov
