"""Seeded synthetic inputs for the AlexNet path.

This module only draws numbers: images, weights, labels and source images for
the ten-view batch.  It performs none of the network's arithmetic, so both the
HIP library's callers and the CPU oracle can take their inputs from here.

Recipe (one ``numpy.random.default_rng(seed)`` stream, drawn in this order):
  1. images  x ~ N(0, 1), float32, shape [N, 3, S, S]  (S = 227, or 256 for
     ten-view sources);
  2. for each learned layer in order conv1..conv5, fc6..fc8: weights
     ~ N(0, 1) * sqrt(2 / fan_in), float32 (He), fan_in = (Cin/G)*k*k or
     in_features.  Biases are constants: 1 for conv2, conv4, conv5 and the
     three FC layers, 0 for conv1 and conv3 (the paper's rule for which layers
     start at 1; the fermi.ai wiki lists "the FC layers" among them);
  3. labels uniform in [0, 1000), int32, shape [N].

bf16 values are produced from float32 by round-to-nearest-even on the bit
pattern; the float32 copy of a bf16 tensor holds exactly the bf16 value.

Augmentation workload (``augment_inputs``, its own stream of ``seed``):
  1. sources z ~ N(0, 1), float32 [N, 3, Hs, Ws], mixed across the colour
     channels by the fixed matrix AUG_MIX = R diag(AUG_SPREAD) (R a rotation
     by fixed angles), so the RGB covariance of the sources is close to
     R diag(AUG_SPREAD^2) R^T with well separated eigenvalues, as in natural
     images, where one colour component dominates;
  2. per image: crop offsets y0 in [0, Hs - 227], x0 in [0, Ws - 227] and a
     mirror flag, uniform; colour draws alpha ~ N(0, 0.1) (the pages'
     standard deviation), float32 [N, 3];
  3. labels uniform in [0, 1000).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

# Parameter shapes only (name, Cin, Cout, kernel, grouped-in-two-tower-net);
# strides and paddings belong to the network code, not to the input draw.
CONV_SHAPES = (
    ("conv1", 3, 96, 11, False),
    ("conv2", 96, 256, 5, True),
    ("conv3", 256, 384, 3, False),
    ("conv4", 384, 384, 3, True),
    ("conv5", 384, 256, 3, True),
)
FC_SHAPES = (("fc6", 9216, 4096), ("fc7", 4096, 4096), ("fc8", 4096, 1000))
BIAS_ONE = {"conv2", "conv4", "conv5", "fc6", "fc7", "fc8"}

IMAGE = 227
SOURCE = 256
CLASSES = 1000


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array holding exactly the bf16-rounded values of ``a``."""
    return bf16_to_f32(bf16_bits(a))


def weight_shapes(groups: int = 1):
    """Shapes of the 16 parameter tensors, conv weights OIHW, FC [out][in]."""
    shapes = []
    for name, cin, cout, k, grouped in CONV_SHAPES:
        g = groups if grouped else 1
        shapes.append((name, (cout, cin // g, k, k), (cout,)))
    for name, fin, fout in FC_SHAPES:
        shapes.append((name, (fout, fin), (fout,)))
    return shapes


@dataclass
class Synthetic:
    seed: int
    groups: int
    bf16: bool
    x: np.ndarray                      # float32 (bf16-exact when bf16)
    weights: List[np.ndarray]          # 8 float32 weight tensors (bf16-exact when bf16)
    biases: List[np.ndarray]           # 8 float32 bias vectors
    master_w: List[np.ndarray]         # unrounded float32 weights (fp32 master copy)
    labels: np.ndarray                 # int32 [N]
    names: List[str] = field(default_factory=list)

    def x_bits(self) -> np.ndarray:
        return bf16_bits(self.x)


def synthetic(seed: int, batch: int, groups: int = 1, bf16: bool = True,
              image: int = IMAGE, with_labels: bool = True) -> Synthetic:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, 3, image, image), dtype=np.float32)
    ws, bs, masters, names = [], [], [], []
    for name, wshape, bshape in weight_shapes(groups):
        fan_in = int(np.prod(wshape[1:]))
        w = rng.standard_normal(wshape, dtype=np.float32) * np.float32(np.sqrt(2.0 / fan_in))
        w = w.astype(np.float32)
        b = np.full(bshape, 1.0 if name in BIAS_ONE else 0.0, dtype=np.float32)
        masters.append(w)
        ws.append(round_bf16(w) if bf16 else w)
        bs.append(b)
        names.append(name)
    labels = (rng.integers(0, CLASSES, size=batch, dtype=np.int32)
              if with_labels else np.zeros(batch, np.int32))
    if bf16:
        x = round_bf16(x)
    return Synthetic(seed, groups, bf16, x, ws, bs, masters, labels, names)


# The five workloads, by name: (seed, batch, groups, bf16, mode)
WORKLOADS = {
    "fp32_batch1": dict(seed=0, batch=1, groups=1, bf16=False, mode="forward"),
    "bf16_batch128": dict(seed=1, batch=128, groups=1, bf16=True, mode="forward"),
    "two_tower_batch128": dict(seed=2, batch=128, groups=2, bf16=True, mode="forward"),
    "train_batch128": dict(seed=3, batch=128, groups=1, bf16=True, mode="train"),
    "tenview_256_sources": dict(seed=4, batch=256, groups=1, bf16=True, mode="tenview"),
}

TRAIN_HYPER = dict(lr=0.01, momentum=0.9, weight_decay=5e-4, dropout_seed=3, step=0)


def workload_inputs(name: str, batch: Optional[int] = None) -> Synthetic:
    """Seeded inputs and weights of a named workload (optionally fewer or more
    images, same seed and distributions)."""
    c = WORKLOADS[name]
    n = c["batch"] if batch is None else batch
    image = SOURCE if c["mode"] == "tenview" else IMAGE
    return synthetic(c["seed"], n, c["groups"], c["bf16"], image=image)


# ---------------------------------------------------------------- augmentation
AUG_SPREAD = (1.0, 0.45, 0.2)
AUG_ALPHA_STD = 0.1


def _rotation(a: float, b: float, c: float) -> np.ndarray:
    ca, sa, cb, sb, cc, sc = np.cos(a), np.sin(a), np.cos(b), np.sin(b), np.cos(c), np.sin(c)
    rz = np.array([[ca, -sa, 0], [sa, ca, 0], [0, 0, 1]])
    ry = np.array([[cb, 0, sb], [0, 1, 0], [-sb, 0, cb]])
    rx = np.array([[1, 0, 0], [0, cc, -sc], [0, sc, cc]])
    return rz @ ry @ rx


AUG_MIX = (_rotation(0.5, -0.7, 0.3) @ np.diag(AUG_SPREAD)).astype(np.float32)


@dataclass
class AugInputs:
    seed: int
    bf16: bool
    src: np.ndarray       # float32 [N, 3, Hs, Ws] (bf16-exact when bf16)
    crop: np.ndarray      # int32 [N, 3]: y0, x0, flip
    alpha: np.ndarray     # float32 [N, 3]
    labels: np.ndarray    # int32 [N]


def augment_inputs(seed: int, batch: int, src_h: int = SOURCE, src_w: int = SOURCE,
                   bf16: bool = True) -> AugInputs:
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((batch, 3, src_h, src_w), dtype=np.float32)
    src = np.einsum("cd,ndhw->nchw", AUG_MIX, z).astype(np.float32)
    y0 = rng.integers(0, src_h - IMAGE + 1, size=batch)
    x0 = rng.integers(0, src_w - IMAGE + 1, size=batch)
    flip = rng.integers(0, 2, size=batch)
    crop = np.stack([y0, x0, flip], axis=1).astype(np.int32)
    alpha = (rng.standard_normal((batch, 3)) * AUG_ALPHA_STD).astype(np.float32)
    labels = rng.integers(0, CLASSES, size=batch, dtype=np.int32)
    if bf16:
        src = round_bf16(src)
    return AugInputs(seed, bf16, src, crop, alpha, labels)
