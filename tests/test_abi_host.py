"""Host-only tests of the C ABI: the library loads without a GPU, exports every
symbol the header declares, validates arguments before any launch, and plans
a consistent workspace.  No compute call reaches the device here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from deep_cnn_image_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "alexnet.h")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(alexnet_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.EXPORTED)


def test_default_cfg_holds_page_constants():
    c = B.alexnet_default_cfg(128, 2, B.BF16)
    assert (c.batch, c.groups, c.dtype, c.lrn_n) == (128, 2, B.BF16, 5)
    assert c.lrn_k == 2.0 and c.lrn_alpha == float(np.float32(1e-4)) and c.lrn_beta == 0.75
    assert c.dropout_p == 0.5


@pytest.mark.parametrize("field,value", [("batch", 0), ("batch", -1), ("batch", 5000), ("groups", 3),
                                         ("groups", 0), ("dtype", 7), ("lrn_n", 4), ("lrn_n", 11),
                                         ("lrn_k", 0.0), ("dropout_p", 1.0), ("lrn_taps", 2)])
def test_invalid_cfg_gives_zero_workspace(field, value):
    c = B.alexnet_default_cfg(4, 1, B.BF16)
    setattr(c, field, value)
    assert B.alexnet_workspace_bytes(c, B.MODE_FORWARD) == 0


def test_tenview_batch_limit():
    c = B.alexnet_default_cfg(512, 1, B.BF16)
    assert B.alexnet_workspace_bytes(c, B.MODE_TENVIEW) > 0
    c.batch = 513
    assert B.alexnet_workspace_bytes(c, B.MODE_TENVIEW) == 0
    assert B.alexnet_workspace_bytes(c, 3) == 0


FAKE = 1 << 40          # a 256-aligned non-null address; never dereferenced on error paths


def fake_params(align=256):
    return [FAKE + i * 4096 for i in range(16)]


def test_forward_validation_errors_before_launch():
    c = B.alexnet_default_cfg(2, 1, B.BF16)
    ws = B.alexnet_workspace_bytes(c, B.MODE_FORWARD)
    p = fake_params()
    f = lambda **kw: B.alexnet_forward(kw.get("cfg", c), kw.get("params", p), kw.get("x", FAKE),
                                       kw.get("probs", FAKE), kw.get("ws", FAKE),
                                       kw.get("wsb", ws), 0, check=False)
    assert f(ws=0) == B.E_NULL
    assert f(ws=FAKE + 16) == B.E_ALIGN
    assert f(wsb=ws - 1) == B.E_WORKSPACE
    assert f(x=0) == B.E_NULL
    assert f(x=FAKE + 2) == B.E_ALIGN
    assert f(params=p[:15] + [0]) == B.E_NULL
    assert f(params=p[:15] + [FAKE + 8]) == B.E_ALIGN
    bad = B.alexnet_default_cfg(2, 3, B.BF16)
    assert f(cfg=bad) == B.E_SHAPE
    bad = B.alexnet_default_cfg(2, 1, 9)
    assert f(cfg=bad) == B.E_DTYPE
    null_cfg = B.lib().alexnet_forward(None, B._ptr16(p), FAKE, FAKE, FAKE, ws, None)
    assert null_cfg == B.E_NULL


def test_train_validation_errors_before_launch():
    c = B.alexnet_default_cfg(2, 1, B.BF16)
    ws = B.alexnet_workspace_bytes(c, B.MODE_TRAIN)
    p = fake_params()
    f = lambda **kw: B.alexnet_train_step(c, kw.get("m", p), kw.get("v", p), kw.get("w", p),
                                          kw.get("x", FAKE), kw.get("y", FAKE), 0.01, 0.9, 5e-4, 3, 0,
                                          kw.get("loss", FAKE), None, FAKE, kw.get("wsb", ws), 0,
                                          check=False)
    assert f(wsb=ws - 256) == B.E_WORKSPACE
    assert f(y=0) == B.E_NULL
    assert f(loss=0) == B.E_NULL
    assert f(m=p[:3] + [0] + p[4:]) == B.E_NULL
    assert f(w=p[:3] + [FAKE + 4] + p[4:]) == B.E_ALIGN
    assert B.alexnet_train_step(c, p, p, p, FAKE, FAKE, float("nan"), 0.9, 5e-4, 3, 0, FAKE, None,
                                FAKE, ws, 0, check=False) == B.E_ARG


def test_dropout_mask_validation():
    assert B.alexnet_dropout_mask(3, 0, 0, 4, 4096, 0.5, 0, check=False) == B.E_NULL
    assert B.alexnet_dropout_mask(3, 0, 0, 4, 4095, 0.5, FAKE, check=False) == B.E_SHAPE
    assert B.alexnet_dropout_mask(3, 0, 0, 4, 4096, 1.5, FAKE, check=False) == B.E_ARG
    assert B.alexnet_dropout_mask(3, 0, 0, 0, 4096, 0.5, FAKE, check=False) == B.OK   # empty: no launch


@pytest.mark.parametrize("mode", [B.MODE_FORWARD, B.MODE_TRAIN, B.MODE_TENVIEW])
@pytest.mark.parametrize("groups", [1, 2])
def test_taps_are_disjoint_and_inside_workspace(mode, groups):
    c = B.alexnet_default_cfg(3, groups, B.BF16)
    total = B.alexnet_workspace_bytes(c, mode)
    n_img = 30 if mode == B.MODE_TENVIEW else 3
    spans = []
    esz = {B.F32: 4, B.BF16: 2, B.U8: 1}
    for name, i in B.tap_ids().items():
        try:
            off, shape, dt, layout = B.alexnet_tap(c, mode, i)
        except B.AlexNetError as e:
            assert e.status == B.E_ARG
            continue
        assert off % 256 == 0
        nbytes = int(np.prod(shape)) * esz[dt]
        spans.append((off, off + nbytes, name))
        if layout == 0:
            assert shape[0] == n_img
    spans.sort()
    for (a0, a1, na), (b0, b1, nb) in zip(spans, spans[1:]):
        assert a1 <= b0, (na, nb)
    assert spans[-1][1] <= total


def test_tap_shapes_follow_the_layer_list():
    c = B.alexnet_default_cfg(2, 2, B.BF16)
    ids = B.tap_ids()
    get = lambda n: B.alexnet_tap(c, B.MODE_TRAIN, ids[n])[1]
    assert get("conv1") == (2, 55, 55, 96) and get("pool1") == (2, 27, 27, 96)
    assert get("conv2") == (2, 27, 27, 256) and get("pool2") == (2, 13, 13, 256)
    assert get("conv3") == (2, 13, 13, 384) and get("conv5") == (2, 13, 13, 256)
    assert get("pool5") == (2, 9216, 1, 1) and get("logits") == (2, 1000, 1, 1)
    assert get("gw2") == (256, 48, 5, 5) and get("gw4") == (384, 192, 3, 3)
    assert get("gw3") == (384, 256, 3, 3) and get("gb6") == (4096, 1, 1, 1)
    with pytest.raises(B.AlexNetError):
        B.alexnet_tap(c, B.MODE_FORWARD, ids["gw1"])
    # FC weight gradients are applied inside their GEMM: never stored
    for name in ("gw6", "gw7", "gw8"):
        with pytest.raises(B.AlexNetError):
            B.alexnet_tap(c, B.MODE_TRAIN, ids[name])


def test_lrn_taps_only_on_request():
    ids = B.tap_ids()
    for mode in (B.MODE_FORWARD, B.MODE_TRAIN):
        c = B.alexnet_default_cfg(2, 1, B.BF16)
        assert c.lrn_taps == 0
        with pytest.raises(B.AlexNetError):
            B.alexnet_tap(c, mode, ids["lrn1"])
        c = B.alexnet_default_cfg(2, 1, B.BF16, lrn_taps=True)
        assert B.alexnet_tap(c, mode, ids["lrn1"])[1] == (2, 55, 55, 96)
        assert B.alexnet_tap(c, mode, ids["lrn2"])[1] == (2, 27, 27, 256)
    c = B.alexnet_default_cfg(2, 1, B.BF16)
    for name in ("dlrn1", "dlrn2"):
        with pytest.raises(B.AlexNetError):
            B.alexnet_tap(c, B.MODE_TRAIN, ids[name])
    c = B.alexnet_default_cfg(2, 1, B.BF16, lrn_taps=True)
    assert B.alexnet_tap(c, B.MODE_TRAIN, ids["dlrn1"])[1] == (2, 55, 55, 96)


def test_kernel_ids_match_header():
    txt = open(HEADER).read()
    body = txt[txt.index("typedef enum {\n  ALEXNET_KT_S2D"):txt.index("} alexnet_kernel;")]
    names = re.findall(r"ALEXNET_KT_([A-Z0-9_]+)", body)
    assert names[-1] == "COUNT"
    assert tuple(names[:-1]) == B.KERNELS


def test_timer_validation_before_launch():
    c = B.alexnet_default_cfg(2, 1, B.BF16)
    ws = B.alexnet_workspace_bytes(c, B.MODE_FORWARD)
    p = fake_params()
    f = lambda t: B.alexnet_forward_timed(c, p, FAKE, FAKE, FAKE, ws, 0, t, check=False)
    assert f([(0, FAKE, FAKE)]) == B.E_ARG                       # id out of range
    assert f([(len(B.KERNELS) + 1, FAKE, FAKE)]) == B.E_ARG
    assert f([(B.KT["CONV2_FWD"], 0, FAKE)]) == B.E_NULL
    arr, _ = B._timers([(B.KT["CONV2_FWD"], FAKE, FAKE)])
    assert B.lib().alexnet_forward_timed(C.byref(c), B._ptr16(p), FAKE, FAKE, FAKE, ws, None, arr, -1) == B.E_ARG


def test_event_helpers_validate_pointers():
    lib = B.lib()
    assert lib.alexnet_event_create(1, None) == B.E_NULL
    assert lib.alexnet_event_destroy(None) == B.E_NULL
    ms = C.c_float()
    assert lib.alexnet_event_elapsed_ms(None, FAKE, C.byref(ms)) == B.E_NULL
    assert lib.alexnet_event_elapsed_ms(FAKE, None, C.byref(ms)) == B.E_NULL
    assert lib.alexnet_event_elapsed_ms(FAKE, FAKE, None) == B.E_NULL


def test_augment_validation_errors_before_launch():
    c = B.alexnet_default_cfg(2, 1, B.BF16)
    aug = B.Augment(FAKE, FAKE + 256, FAKE + 512, FAKE + 768)
    f = lambda **kw: B.alexnet_augment_images(kw.get("cfg", c), kw.get("src", FAKE), kw.get("h", 256),
                                              kw.get("w", 256), kw.get("aug", aug), kw.get("x", FAKE), 0,
                                              check=False)
    assert f(aug=None) == B.E_NULL
    assert f(aug=B.Augment(FAKE, 0, FAKE, FAKE)) == B.E_NULL
    assert f(aug=B.Augment(FAKE + 2, FAKE, FAKE, FAKE)) == B.E_ALIGN
    assert f(h=226) == B.E_SHAPE and f(w=100) == B.E_SHAPE and f(h=9000) == B.E_SHAPE
    assert f(src=0) == B.E_NULL and f(x=0) == B.E_NULL
    assert f(src=FAKE + 8) == B.E_ALIGN
    assert f(cfg=B.alexnet_default_cfg(0, 1, B.BF16)) == B.E_SHAPE
    ws = B.alexnet_workspace_bytes(c, B.MODE_TRAIN)
    p = fake_params()
    t = lambda **kw: B.alexnet_train_step_augmented(c, p, p, p, FAKE, kw.get("h", 256), 256, kw.get("aug", aug),
                                                    FAKE, 0.01, 0.9, 5e-4, 3, 0, FAKE, None, FAKE,
                                                    kw.get("wsb", ws), 0, check=False)
    assert t(aug=None) == B.E_NULL
    assert t(h=200) == B.E_SHAPE
    assert t(wsb=ws - 256) == B.E_WORKSPACE


def test_rgb_pca_validation_errors_before_launch():
    c = B.alexnet_default_cfg(1, 1, B.BF16)
    nb = B.alexnet_rgb_pca_workspace_bytes()
    assert nb >= 9 * 8
    f = lambda **kw: B.alexnet_rgb_pca(kw.get("cfg", c), kw.get("x", FAKE), kw.get("n", 4), kw.get("h", 8),
                                       kw.get("w", 8), kw.get("lam", FAKE), kw.get("vec", FAKE),
                                       kw.get("ws", FAKE), kw.get("wsb", nb), 0, check=False)
    assert f(n=0) == B.E_SHAPE and f(h=0) == B.E_SHAPE and f(w=-1) == B.E_SHAPE
    assert f(x=0) == B.E_NULL and f(lam=0) == B.E_NULL and f(vec=0) == B.E_NULL and f(ws=0) == B.E_NULL
    assert f(wsb=nb - 1) == B.E_WORKSPACE
    assert f(ws=FAKE + 64) == B.E_ALIGN and f(lam=FAKE + 2) == B.E_ALIGN
    assert f(cfg=B.alexnet_default_cfg(1, 1, 7)) == B.E_DTYPE


def test_train_step_ex_side_stream_validation():
    """alexnet_train_step_ex: the side stream must differ from the main one
    and come with all ALEXNET_SIDE_EVENTS events; checked before any launch."""
    c = B.alexnet_default_cfg(2, 1, B.BF16)
    ws = B.alexnet_workspace_bytes(c, B.MODE_TRAIN)
    p = fake_params()
    evs = [FAKE + 512 * i for i in range(B.SIDE_EVENTS)]
    f = lambda **kw: B.alexnet_train_step_ex(c, p, p, p, FAKE, None, 0, 0, FAKE, 0.01, 0.9, 5e-4, 3, 0, FAKE,
                                             None, FAKE, kw.get("wsb", ws), kw.get("stream", FAKE + 64),
                                             kw.get("side", FAKE + 128), kw.get("events", evs), check=False)
    assert f(side=FAKE + 64) == B.E_ARG                    # same stream as the main one
    assert f(events=evs[:-1]) == B.E_NULL                   # one event missing
    assert f(events=evs[:3] + [0] + evs[4:]) == B.E_NULL
    assert f(wsb=ws - 256) == B.E_WORKSPACE                 # the usual checks still run
    assert f(side=0, events=(), wsb=ws - 256) == B.E_WORKSPACE
    txt = open(HEADER).read()
    assert int(re.search(r"#define ALEXNET_SIDE_EVENTS (\d+)", txt).group(1)) == B.SIDE_EVENTS


def test_library_creates_no_streams_events_or_memory():
    """The caller owns every buffer, stream and event: the library's sources
    call no HIP allocation or stream/event creation routine, apart from the
    event helpers that make and destroy an event at the caller's request."""
    csrc = os.path.join(ROOT, "deep_cnn_image_amd", "csrc")
    banned = re.compile(r"\bhip(Malloc\w*|Free\w*|HostMalloc|ExtMalloc\w*|StreamCreate\w*|"
                        r"EventCreate\w*|StreamDestroy|EventDestroy)\s*\(")
    helpers = re.compile(r"int alexnet_event_create\(.*?\n}\n\nint alexnet_event_destroy\(.*?\n}\n", re.S)
    for name in sorted(os.listdir(csrc)):
        txt = open(os.path.join(csrc, name)).read()
        if name == "alexnet.cpp":
            assert len(helpers.findall(txt)) == 1
            txt = helpers.sub("", txt)
        assert not banned.search(txt), (name, banned.search(txt).group(0))


def test_noalloc_forward_refuses_oversized_configurations_before_launch():
    """alexnet_forward_noalloc keeps its workspace in a static device array of
    ALEXNET_NOALLOC_SCRATCH_BYTES; larger configurations are refused on the
    host with ALEXNET_E_SCRATCH, smaller ones reach the usual checks."""
    txt = open(HEADER).read()
    m = re.search(r"#define ALEXNET_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES
    p = fake_params()
    for dtype, n in ((B.F32, 16), (B.BF16, 64), (B.BF16, 4096)):
        c = B.alexnet_default_cfg(n, 1, dtype)
        assert B.alexnet_workspace_bytes(c, B.MODE_FORWARD) > B.NOALLOC_SCRATCH_BYTES
        assert B.alexnet_forward_noalloc(c, p, FAKE, FAKE, 0, check=False) == B.E_SCRATCH
    for dtype in (B.F32, B.BF16):
        c = B.alexnet_default_cfg(8, 2, dtype)
        assert B.alexnet_workspace_bytes(c, B.MODE_FORWARD) <= B.NOALLOC_SCRATCH_BYTES
        assert B.alexnet_forward_noalloc(c, p, 0, FAKE, 0, check=False) == B.E_NULL
        assert B.alexnet_forward_noalloc(c, p, FAKE + 2, FAKE, 0, check=False) == B.E_ALIGN
    assert B.status_string(B.E_SCRATCH).startswith("configuration needs more")
