"""torch-side plumbing around the C ABI: device buffers for parameters,
workspace and outputs, and typed views of workspace taps.  torch only
allocates memory and supplies the stream; every step of the network runs in
libalexnet.so."""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

from . import binding as B
from .inputs import bf16_bits

TORCH_DT = {B.F32: torch.float32, B.BF16: torch.bfloat16, B.U8: torch.uint8}


def to_device(a: np.ndarray, dtype: int, device) -> torch.Tensor:
    """Upload a float32 array as fp32, or as bf16 (round to nearest even)."""
    if dtype == B.BF16:
        bits = bf16_bits(np.ascontiguousarray(a, np.float32))
        return torch.from_numpy(bits.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)


def stream_handle() -> int:
    return int(torch.cuda.current_stream().cuda_stream)


def _destroy_event(e) -> None:
    # also runs at interpreter exit, when the runtime may already be gone
    if e:
        try:
            B.lib().alexnet_event_destroy(e)
        except Exception:
            pass


class SideStream:
    """A caller-owned second stream and the fork/join events the training
    step uses with it (alexnet_train_step_ex).  The stream has the default
    priority; the events come from alexnet_event_create (timing disabled, no
    system-scope fence: they only order the two streams)."""

    def __init__(self, device: str = "cuda:0"):
        self.stream = torch.cuda.Stream(device=device)
        with torch.cuda.device(device):
            self.events = [B.alexnet_event_create(False) for _ in range(B.SIDE_EVENTS)]

    def __del__(self):
        for e in getattr(self, "events", ()):
            _destroy_event(e)

    @property
    def handle(self) -> int:
        return int(self.stream.cuda_stream)

    @property
    def event_handles(self) -> List[int]:
        return list(self.events)


class Timer:
    """A start/stop pair of timing events from alexnet_event_create, for the
    *_timed calls' timers (no system-scope fence, so the timed span holds the
    kernel alone)."""

    def __init__(self):
        self.start = B.alexnet_event_create(True)
        self.stop = B.alexnet_event_create(True)

    def elapsed_ms(self) -> float:
        return B.alexnet_event_elapsed_ms(self.start, self.stop)

    def __del__(self):
        for e in (getattr(self, "start", None), getattr(self, "stop", None)):
            _destroy_event(e)


class Session:
    """One configuration (batch, groups, dtype, mode) with its workspace."""

    def __init__(self, batch: int, groups: int = 1, dtype: int = B.BF16, mode: int = B.MODE_FORWARD,
                 device: str = "cuda:0", lrn_taps: bool = False):
        self.cfg = B.alexnet_default_cfg(batch, groups, dtype, lrn_taps)
        self.mode = mode
        self.dtype = dtype
        self.device = torch.device(device)
        self.ws_bytes = B.alexnet_workspace_bytes(self.cfg, mode)
        if self.ws_bytes == 0:
            raise B.AlexNetError(B.E_ARG, "alexnet_workspace_bytes")
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self._taps = B.tap_ids()

    # ------------------------------------------------------------- taps
    def tap(self, name: str) -> torch.Tensor:
        off, shape, dt, _layout = B.alexnet_tap(self.cfg, self.mode, self._taps[name])
        tdt = TORCH_DT[dt]
        n = int(np.prod(shape))
        nbytes = n * torch.empty((), dtype=tdt).element_size()
        return self.ws[off:off + nbytes].view(tdt).view(*[int(s) for s in shape])

    # ------------------------------------------------------------- params
    def upload_params(self, weights: Sequence[np.ndarray], biases: Sequence[np.ndarray],
                      dtype: Optional[int] = None) -> List[torch.Tensor]:
        dt = self.dtype if dtype is None else dtype
        out = []
        for w, b in zip(weights, biases):
            out.append(to_device(w, dt, self.device))
            out.append(to_device(b, dt, self.device))
        return out

    # ------------------------------------------------------------- calls
    def forward(self, params, x: torch.Tensor, probs: Optional[torch.Tensor] = None) -> torch.Tensor:
        if probs is None:
            probs = torch.empty((self.cfg.batch, 1000), dtype=torch.float32, device=self.device)
        fn = B.alexnet_forward_tenview if self.mode == B.MODE_TENVIEW else B.alexnet_forward
        fn(self.cfg, params, x, probs, self.ws, self.ws_bytes, stream_handle())
        return probs

    def train_step(self, master, momentum, work, x, labels, loss, probs=None, lr=0.01,
                   momentum_coef=0.9, weight_decay=5e-4, seed=3, step=0,
                   side: Optional[SideStream] = None, timers=()):
        """alexnet_train_step, or with a side stream (or timers)
        alexnet_train_step_ex."""
        if side is None and not timers:
            B.alexnet_train_step(self.cfg, master, momentum, work, x, labels, lr, momentum_coef,
                                 weight_decay, seed, step, loss, probs, self.ws, self.ws_bytes,
                                 stream_handle())
            return
        B.alexnet_train_step_ex(self.cfg, master, momentum, work, x, None, 0, 0, labels, lr,
                                momentum_coef, weight_decay, seed, step, loss, probs, self.ws,
                                self.ws_bytes, stream_handle(),
                                side.handle if side is not None else 0,
                                side.event_handles if side is not None else (), timers)
