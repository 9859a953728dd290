"""Helpers shared by the GPU parity tests (no tests here)."""
import sys

import numpy as np
import torch

from deep_cnn_image_amd import binding as B
from deep_cnn_image_amd import inputs as I
from deep_cnn_image_amd.session import Session, to_device

DEV = "cuda:0"

# Tolerances.  The bf16 bar is the relative L2 error the workload states for
# activations and gradients; the fp32 bar applies to the fp32 configuration.
# A single layer fed the HIP path's own stored input differs from the float64
# oracle only by fp32 accumulation order and the final rounding of its
# output to bf16 (unit roundoff 2^-9, i.e. a relative L2 of at most ~2e-3).
TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_LAYER_BF16 = 5e-3
TOL_F32_OUT = 1e-5   # fp32 outputs (weight gradients, logits) of one layer fed the same bf16 inputs


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b) -> float:
    """||a - b|| / ||b||; a is reshaped to b's shape (same element count)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size != b.size:
        raise ValueError(f"size mismatch {a.shape} vs {b.shape}")
    a = a.reshape(b.shape)
    nb = np.linalg.norm(b)
    if nb == 0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / nb)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


def nchw(t: torch.Tensor) -> np.ndarray:
    """NHWC tap -> NCHW float64 (or uint8) array."""
    a = host(t)
    return np.ascontiguousarray(a.transpose(0, 3, 1, 2))


def flat(t: torch.Tensor) -> np.ndarray:
    a = host(t)
    return a.reshape(a.shape[0], -1)


def taps(sess: Session, names):
    return {n: sess.tap(n) for n in names}


def params_f32(weights, biases, dev=DEV):
    out = []
    for w, b in zip(weights, biases):
        out.append(torch.from_numpy(np.ascontiguousarray(w, np.float32)).to(dev))
        out.append(torch.from_numpy(np.ascontiguousarray(b, np.float32)).to(dev))
    return out
