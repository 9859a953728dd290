"""ctypes binding of libalexnet.so: one Python function per C entry point, same
names, argument marshalling only.  Device buffers are passed as integer
addresses (``tensor.data_ptr()``) and streams as ``hipStream_t`` handles
(``torch.cuda.current_stream().cuda_stream``).

Importing this module does not need a GPU; loading fails loudly if the
library has not been built (``python -m deep_cnn_image_amd.build``).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# ALEXNET_LIB selects another build of the same sources (the sanitizer test uses it)
LIB_PATH = os.environ.get("ALEXNET_LIB") or os.path.join(_HERE, "lib", "libalexnet.so")

OK, E_NULL, E_SHAPE, E_DTYPE, E_WORKSPACE, E_ALIGN, E_DEVICE, E_HIP, E_ARG, E_SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
NOALLOC_SCRATCH_BYTES = 64 << 20   # ALEXNET_NOALLOC_SCRATCH_BYTES
F32, BF16, U8 = 0, 1, 2
MODE_FORWARD, MODE_TRAIN, MODE_TENVIEW = 0, 1, 2

EXPORTED = (
    "alexnet_default_cfg", "alexnet_workspace_bytes", "alexnet_forward", "alexnet_forward_tenview",
    "alexnet_train_step", "alexnet_cast_weights", "alexnet_dropout_mask", "alexnet_tap",
    "alexnet_tap_count", "alexnet_tap_name", "alexnet_status_string", "alexnet_forward_timed",
    "alexnet_train_step_timed", "alexnet_augment_images", "alexnet_train_step_augmented",
    "alexnet_train_step_augmented_timed", "alexnet_rgb_pca_workspace_bytes", "alexnet_rgb_pca",
    "alexnet_rgb_pca_timed", "alexnet_train_step_ex", "alexnet_forward_noalloc", "alexnet_event_create",
    "alexnet_event_destroy", "alexnet_event_elapsed_ms",
)

# alexnet_kernel ids (kernel-timing hooks)
KERNELS = (
    "S2D", "CONV1_FWD", "CONV2_FWD", "CONV3_FWD", "CONV4_FWD", "CONV5_FWD", "LRNPOOL1_FWD",
    "LRNPOOL2_FWD", "POOL5_FWD", "FC6_FWD", "FC7_FWD", "FC8_FWD", "FC8_DGRAD", "FC7_DGRAD",
    "FC6_DGRAD", "FC8_WGRAD", "FC7_WGRAD", "FC6_WGRAD", "POOL5_BWD", "CONV5_WGRAD", "CONV4_WGRAD",
    "CONV3_WGRAD", "CONV2_WGRAD", "CONV1_WGRAD", "CONV5_DGRAD", "CONV4_DGRAD", "CONV3_DGRAD",
    "CONV2_DGRAD", "POOLLRN2_BWD", "POOLLRN1_BWD", "BIAS", "RGB_PCA", "BIAS12",
)
KT = {name: i + 1 for i, name in enumerate(KERNELS)}


class Cfg(C.Structure):
    _fields_ = [("batch", C.c_int32), ("groups", C.c_int32), ("dtype", C.c_int32),
                ("lrn_n", C.c_int32), ("lrn_k", C.c_float), ("lrn_alpha", C.c_float),
                ("lrn_beta", C.c_float), ("dropout_p", C.c_float), ("lrn_taps", C.c_int32)]


class Timer(C.Structure):
    _fields_ = [("kernel", C.c_int32), ("start", C.c_void_p), ("stop", C.c_void_p)]


SIDE_EVENTS = 10   # ALEXNET_SIDE_EVENTS


class Exec(C.Structure):
    """alexnet_exec: side stream and its fork/join events (hipStream_t and
    hipEvent_t handles), kernel timers."""
    _fields_ = [("side_stream", C.c_void_p), ("events", C.c_void_p * SIDE_EVENTS),
                ("timers", C.POINTER(Timer)), ("n_timers", C.c_int32)]


class Augment(C.Structure):
    """alexnet_augment: device addresses of crop [N][3] int32, alpha [N][3],
    eigval [3] and eigvec [3][3] (fp32)."""
    _fields_ = [("crop", C.c_void_p), ("alpha", C.c_void_p), ("eigval", C.c_void_p),
                ("eigvec", C.c_void_p)]


def augment(crop, alpha, eigval, eigvec) -> Augment:
    return Augment(_ptr(crop) or None, _ptr(alpha) or None, _ptr(eigval) or None, _ptr(eigvec) or None)


class AlexNetError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


_lib = None
_PTR16 = C.c_void_p * 16


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m deep_cnn_image_amd.build`")
    L = C.CDLL(LIB_PATH)
    vp, cfgp = C.c_void_p, C.POINTER(Cfg)
    L.alexnet_default_cfg.argtypes = [cfgp, C.c_int32, C.c_int32, C.c_int32]
    L.alexnet_default_cfg.restype = None
    L.alexnet_workspace_bytes.argtypes = [cfgp, C.c_int]
    L.alexnet_workspace_bytes.restype = C.c_size_t
    L.alexnet_forward.argtypes = [cfgp, _PTR16, vp, vp, vp, C.c_size_t, vp]
    L.alexnet_forward.restype = C.c_int
    L.alexnet_forward_noalloc.argtypes = [cfgp, _PTR16, vp, vp, vp]
    L.alexnet_forward_noalloc.restype = C.c_int
    L.alexnet_forward_tenview.argtypes = [cfgp, _PTR16, vp, vp, vp, C.c_size_t, vp]
    L.alexnet_forward_tenview.restype = C.c_int
    L.alexnet_train_step.argtypes = [cfgp, _PTR16, _PTR16, _PTR16, vp, vp, C.c_float, C.c_float,
                                     C.c_float, C.c_uint64, C.c_uint64, vp, vp, vp, C.c_size_t, vp]
    L.alexnet_train_step.restype = C.c_int
    tp = C.POINTER(Timer)
    L.alexnet_forward_timed.argtypes = [cfgp, _PTR16, vp, vp, vp, C.c_size_t, vp, tp, C.c_int32]
    L.alexnet_forward_timed.restype = C.c_int
    L.alexnet_train_step_timed.argtypes = [cfgp, _PTR16, _PTR16, _PTR16, vp, vp, C.c_float, C.c_float,
                                           C.c_float, C.c_uint64, C.c_uint64, vp, vp, vp, C.c_size_t,
                                           vp, tp, C.c_int32]
    L.alexnet_train_step_timed.restype = C.c_int
    augp = C.POINTER(Augment)
    L.alexnet_augment_images.argtypes = [cfgp, vp, C.c_int32, C.c_int32, augp, vp, vp]
    L.alexnet_augment_images.restype = C.c_int
    L.alexnet_train_step_augmented.argtypes = [cfgp, _PTR16, _PTR16, _PTR16, vp, C.c_int32, C.c_int32, augp,
                                               vp, C.c_float, C.c_float, C.c_float, C.c_uint64, C.c_uint64,
                                               vp, vp, vp, C.c_size_t, vp]
    L.alexnet_train_step_augmented.restype = C.c_int
    L.alexnet_train_step_augmented_timed.argtypes = L.alexnet_train_step_augmented.argtypes + [tp, C.c_int32]
    L.alexnet_train_step_augmented_timed.restype = C.c_int
    L.alexnet_train_step_ex.argtypes = [cfgp, _PTR16, _PTR16, _PTR16, vp, augp, C.c_int32, C.c_int32, vp,
                                        C.c_float, C.c_float, C.c_float, C.c_uint64, C.c_uint64, vp, vp, vp,
                                        C.c_size_t, vp, C.POINTER(Exec)]
    L.alexnet_train_step_ex.restype = C.c_int
    L.alexnet_rgb_pca_workspace_bytes.argtypes = []
    L.alexnet_rgb_pca_workspace_bytes.restype = C.c_size_t
    L.alexnet_rgb_pca.argtypes = [cfgp, vp, C.c_int32, C.c_int32, C.c_int32, vp, vp, vp, C.c_size_t, vp]
    L.alexnet_rgb_pca.restype = C.c_int
    L.alexnet_rgb_pca_timed.argtypes = L.alexnet_rgb_pca.argtypes + [tp, C.c_int32]
    L.alexnet_rgb_pca_timed.restype = C.c_int
    L.alexnet_cast_weights.argtypes = [cfgp, _PTR16, _PTR16, vp]
    L.alexnet_cast_weights.restype = C.c_int
    L.alexnet_dropout_mask.argtypes = [C.c_uint64, C.c_uint64, C.c_int32, C.c_int32, C.c_int32,
                                       C.c_float, vp, vp]
    L.alexnet_dropout_mask.restype = C.c_int
    L.alexnet_tap.argtypes = [cfgp, C.c_int, C.c_int, C.POINTER(C.c_size_t), C.POINTER(C.c_int64),
                              C.POINTER(C.c_int), C.POINTER(C.c_int)]
    L.alexnet_tap.restype = C.c_int
    L.alexnet_tap_count.argtypes = []
    L.alexnet_tap_count.restype = C.c_int
    L.alexnet_tap_name.argtypes = [C.c_int]
    L.alexnet_tap_name.restype = C.c_char_p
    L.alexnet_status_string.argtypes = [C.c_int]
    L.alexnet_status_string.restype = C.c_char_p
    L.alexnet_event_create.argtypes = [C.c_int32, C.POINTER(vp)]
    L.alexnet_event_create.restype = C.c_int
    L.alexnet_event_destroy.argtypes = [vp]
    L.alexnet_event_destroy.restype = C.c_int
    L.alexnet_event_elapsed_ms.argtypes = [vp, vp, C.POINTER(C.c_float)]
    L.alexnet_event_elapsed_ms.restype = C.c_int
    _lib = L
    return L


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _ptr16(xs: Sequence) -> "C.Array":
    if len(xs) != 16:
        raise ValueError("expected 16 tensors (w1, b1, ..., w8, b8)")
    return _PTR16(*[_ptr(t) or None for t in xs])


def _check(status: int, where: str) -> int:
    if status != OK:
        raise AlexNetError(status, where)
    return status


def status_string(status: int) -> str:
    return lib().alexnet_status_string(status).decode()


def alexnet_default_cfg(batch: int, groups: int = 1, dtype: int = BF16, lrn_taps: bool = False) -> Cfg:
    cfg = Cfg()
    lib().alexnet_default_cfg(C.byref(cfg), batch, groups, dtype)
    cfg.lrn_taps = 1 if lrn_taps else 0
    return cfg


def alexnet_workspace_bytes(cfg: Cfg, mode: int) -> int:
    return int(lib().alexnet_workspace_bytes(C.byref(cfg), mode))


def alexnet_forward(cfg, params, x, probs, ws, ws_bytes, stream=0, check=True) -> int:
    s = lib().alexnet_forward(C.byref(cfg), _ptr16(params), _ptr(x) or None, _ptr(probs) or None,
                              _ptr(ws) or None, ws_bytes, _ptr(stream) or None)
    return _check(s, "alexnet_forward") if check else s


def alexnet_forward_noalloc(cfg, params, x, probs, stream=0, check=True) -> int:
    s = lib().alexnet_forward_noalloc(C.byref(cfg), _ptr16(params), _ptr(x) or None, _ptr(probs) or None,
                                      _ptr(stream) or None)
    return _check(s, "alexnet_forward_noalloc") if check else s


def alexnet_forward_tenview(cfg, params, src, probs, ws, ws_bytes, stream=0, check=True) -> int:
    s = lib().alexnet_forward_tenview(C.byref(cfg), _ptr16(params), _ptr(src) or None,
                                      _ptr(probs) or None, _ptr(ws) or None, ws_bytes,
                                      _ptr(stream) or None)
    return _check(s, "alexnet_forward_tenview") if check else s


def alexnet_train_step(cfg, master, momentum, work, x, labels, lr, momentum_coef, weight_decay,
                       seed, step, loss, probs, ws, ws_bytes, stream=0, check=True) -> int:
    s = lib().alexnet_train_step(C.byref(cfg), _ptr16(master), _ptr16(momentum), _ptr16(work),
                                 _ptr(x) or None, _ptr(labels) or None, lr, momentum_coef,
                                 weight_decay, seed, step, _ptr(loss) or None, _ptr(probs) or None,
                                 _ptr(ws) or None, ws_bytes, _ptr(stream) or None)
    return _check(s, "alexnet_train_step") if check else s


def _timers(timers):
    """[(kernel id, start event handle, stop event handle), ...] -> (array, n)."""
    if not timers:
        return None, 0
    arr = (Timer * len(timers))(*[Timer(k, s, e) for k, s, e in timers])
    return arr, len(timers)


def alexnet_forward_timed(cfg, params, x, probs, ws, ws_bytes, stream, timers, check=True) -> int:
    arr, n = _timers(timers)
    s = lib().alexnet_forward_timed(C.byref(cfg), _ptr16(params), _ptr(x) or None, _ptr(probs) or None,
                                    _ptr(ws) or None, ws_bytes, _ptr(stream) or None, arr, n)
    return _check(s, "alexnet_forward_timed") if check else s


def alexnet_train_step_timed(cfg, master, momentum, work, x, labels, lr, momentum_coef, weight_decay,
                             seed, step, loss, probs, ws, ws_bytes, stream, timers, check=True) -> int:
    arr, n = _timers(timers)
    s = lib().alexnet_train_step_timed(C.byref(cfg), _ptr16(master), _ptr16(momentum), _ptr16(work),
                                       _ptr(x) or None, _ptr(labels) or None, lr, momentum_coef,
                                       weight_decay, seed, step, _ptr(loss) or None, _ptr(probs) or None,
                                       _ptr(ws) or None, ws_bytes, _ptr(stream) or None, arr, n)
    return _check(s, "alexnet_train_step_timed") if check else s


def alexnet_train_step_ex(cfg, master, momentum, work, x, aug, src_h, src_w, labels, lr, momentum_coef,
                          weight_decay, seed, step, loss, probs, ws, ws_bytes, stream=0, side_stream=0,
                          events=(), timers=(), check=True) -> int:
    """aug: an Augment or None; side_stream: a hipStream_t handle or 0;
    events: SIDE_EVENTS hipEvent_t handles when side_stream is given."""
    arr, n = _timers(timers)
    ev = list(events) + [0] * (SIDE_EVENTS - len(events))
    ex = Exec(_ptr(side_stream) or None, (C.c_void_p * SIDE_EVENTS)(*[e or None for e in ev[:SIDE_EVENTS]]),
              arr, n)
    s = lib().alexnet_train_step_ex(
        C.byref(cfg), _ptr16(master), _ptr16(momentum), _ptr16(work), _ptr(x) or None,
        C.byref(aug) if aug is not None else None, src_h, src_w, _ptr(labels) or None, lr, momentum_coef,
        weight_decay, seed, step, _ptr(loss) or None, _ptr(probs) or None, _ptr(ws) or None, ws_bytes,
        _ptr(stream) or None, C.byref(ex))
    return _check(s, "alexnet_train_step_ex") if check else s


def alexnet_augment_images(cfg, src, src_h, src_w, aug: Augment, x, stream=0, check=True) -> int:
    s = lib().alexnet_augment_images(C.byref(cfg), _ptr(src) or None, src_h, src_w,
                                     C.byref(aug) if aug is not None else None, _ptr(x) or None,
                                     _ptr(stream) or None)
    return _check(s, "alexnet_augment_images") if check else s


def alexnet_train_step_augmented(cfg, master, momentum, work, src, src_h, src_w, aug: Augment, labels, lr,
                                 momentum_coef, weight_decay, seed, step, loss, probs, ws, ws_bytes, stream=0,
                                 check=True) -> int:
    s = lib().alexnet_train_step_augmented(
        C.byref(cfg), _ptr16(master), _ptr16(momentum), _ptr16(work), _ptr(src) or None, src_h, src_w,
        C.byref(aug) if aug is not None else None, _ptr(labels) or None, lr, momentum_coef, weight_decay,
        seed, step, _ptr(loss) or None, _ptr(probs) or None, _ptr(ws) or None, ws_bytes, _ptr(stream) or None)
    return _check(s, "alexnet_train_step_augmented") if check else s


def alexnet_train_step_augmented_timed(cfg, master, momentum, work, src, src_h, src_w, aug: Augment, labels,
                                       lr, momentum_coef, weight_decay, seed, step, loss, probs, ws, ws_bytes,
                                       stream, timers, check=True) -> int:
    arr, n = _timers(timers)
    s = lib().alexnet_train_step_augmented_timed(
        C.byref(cfg), _ptr16(master), _ptr16(momentum), _ptr16(work), _ptr(src) or None, src_h, src_w,
        C.byref(aug) if aug is not None else None, _ptr(labels) or None, lr, momentum_coef, weight_decay,
        seed, step, _ptr(loss) or None, _ptr(probs) or None, _ptr(ws) or None, ws_bytes, _ptr(stream) or None,
        arr, n)
    return _check(s, "alexnet_train_step_augmented_timed") if check else s


def alexnet_rgb_pca_workspace_bytes() -> int:
    return int(lib().alexnet_rgb_pca_workspace_bytes())


def alexnet_rgb_pca(cfg, images, n, h, w, eigval, eigvec, ws, ws_bytes, stream=0, check=True) -> int:
    s = lib().alexnet_rgb_pca(C.byref(cfg), _ptr(images) or None, n, h, w, _ptr(eigval) or None,
                              _ptr(eigvec) or None, _ptr(ws) or None, ws_bytes, _ptr(stream) or None)
    return _check(s, "alexnet_rgb_pca") if check else s


def alexnet_rgb_pca_timed(cfg, images, n, h, w, eigval, eigvec, ws, ws_bytes, stream, timers,
                          check=True) -> int:
    arr, k = _timers(timers)
    s = lib().alexnet_rgb_pca_timed(C.byref(cfg), _ptr(images) or None, n, h, w, _ptr(eigval) or None,
                                    _ptr(eigvec) or None, _ptr(ws) or None, ws_bytes, _ptr(stream) or None,
                                    arr, k)
    return _check(s, "alexnet_rgb_pca_timed") if check else s


def alexnet_cast_weights(cfg, master, work, stream=0, check=True) -> int:
    s = lib().alexnet_cast_weights(C.byref(cfg), _ptr16(master), _ptr16(work), _ptr(stream) or None)
    return _check(s, "alexnet_cast_weights") if check else s


def alexnet_dropout_mask(seed, step, layer, rows, cols, p, mask, stream=0, check=True) -> int:
    s = lib().alexnet_dropout_mask(seed, step, layer, rows, cols, p, _ptr(mask) or None,
                                   _ptr(stream) or None)
    return _check(s, "alexnet_dropout_mask") if check else s


def alexnet_tap(cfg, mode: int, tap_id: int):
    """(byte offset, shape tuple, dtype, layout) of a workspace tap."""
    off = C.c_size_t()
    shape = (C.c_int64 * 4)()
    dt, lay = C.c_int(), C.c_int()
    _check(lib().alexnet_tap(C.byref(cfg), mode, tap_id, C.byref(off), shape, C.byref(dt),
                             C.byref(lay)), "alexnet_tap")
    return off.value, tuple(shape), dt.value, lay.value


def alexnet_event_create(timing: bool) -> int:
    e = C.c_void_p()
    _check(lib().alexnet_event_create(1 if timing else 0, C.byref(e)), "alexnet_event_create")
    return int(e.value)


def alexnet_event_destroy(event: int) -> None:
    _check(lib().alexnet_event_destroy(event), "alexnet_event_destroy")


def alexnet_event_elapsed_ms(start: int, stop: int) -> float:
    ms = C.c_float()
    _check(lib().alexnet_event_elapsed_ms(start, stop, C.byref(ms)), "alexnet_event_elapsed_ms")
    return float(ms.value)


def alexnet_tap_count() -> int:
    return int(lib().alexnet_tap_count())


def alexnet_tap_name(tap_id: int):
    r = lib().alexnet_tap_name(tap_id)
    return None if r is None else r.decode()


def tap_ids() -> dict:
    return {alexnet_tap_name(i): i for i in range(alexnet_tap_count())}
