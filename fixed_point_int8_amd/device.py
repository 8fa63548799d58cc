"""Device plumbing around the C ABI: an artifact and its engine in GPU
memory, and a batch of run states in one device arena.  PyTorch provides
the device memory and the stream; every computation is a libfpi8 call.
"""
from __future__ import annotations

import numpy as np

from . import binding as B


def _torch():
    import torch
    return torch


def section_zero(blob: np.ndarray) -> np.ndarray:
    n = int(blob[128 + 8: 128 + 16].view(np.uint64)[0])
    return blob[:n]


class DeviceModel:
    """An artifact copied to the GPU and the engine bound to it."""

    def __init__(self, blob: np.ndarray, max_runs: int, device: str = "cuda"):
        torch = _torch()
        if not torch.cuda.is_available():
            raise RuntimeError("no GPU: the fixed-point core runs only on the GPU")
        self.blob_len = int(blob.size)
        self.d_blob = torch.from_numpy(blob).to(device)
        e, self.engine = B.fpi8_engine_create(section_zero(blob), self.d_blob, self.blob_len, max_runs)
        if e:
            self.engine = None
            raise RuntimeError(f"fpi8_engine_create failed with error {e}")
        self.max_runs = max_runs

    def close(self):
        if self.engine is not None:
            B.fpi8_engine_destroy(self.engine)
            self.engine = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class DeviceBatch:
    """n runs at a fixed stride in one device buffer.

    runs: list of (ids, max_tokens, temperature_q16, seed).
    """

    def __init__(self, cfg, runs, device: str = "cuda", stride: int | None = None):
        torch = _torch()
        self.cfg = tuple(int(v) for v in cfg)
        self.n = len(runs)
        self.sizes = []
        for ids, mx, t, s in runs:
            n = B.fpi8_state_size(self.cfg, len(ids), mx)
            if n == B.UINT64_MAX:
                raise ValueError("state_size out of range")
            self.sizes.append(n)
        need = (max(self.sizes) + 255) // 256 * 256
        self.stride = stride or need
        if self.stride < need or self.stride % 8:
            raise ValueError("stride too small or misaligned")
        self.d_states = torch.zeros(self.n * self.stride, dtype=torch.uint8, device=device)
        host = None
        for i, (ids, mx, t, s) in enumerate(runs):
            size = self.sizes[i]
            if host is None or host.size < size:
                raw = np.empty(size + 64, dtype=np.uint8)
                off = (-raw.ctypes.data) % 64
                host = raw[off: off + size]
            st = host[:size]
            e = B.fpi8_init_state(self.cfg, st, ids, mx, t, s)
            if e:
                raise ValueError(f"fpi8_init_state failed with error {e}")
            # Beyond the ids the fresh state is zero, as the device buffer is.
            head = B.fpi8_state_offsets(self.cfg, len(ids), mx)["out"]
            self.d_states[i * self.stride: i * self.stride + head].copy_(
                torch.from_numpy(st[:head].copy()))

    def turn(self, model: DeviceModel, max_positions: int, stream=None):
        return B.fpi8_turn(model.engine, self.d_states, self.stride, self.n, max_positions, stream)

    def turn_phases(self, model: DeviceModel, max_phases: int, stream=None):
        return B.fpi8_turn_phases(model.engine, self.d_states, self.stride, self.n, max_phases,
                                  stream)

    def turn_units(self, model: DeviceModel, max_units: int, stream=None):
        return B.fpi8_turn_units(model.engine, self.d_states, self.stride, self.n, max_units,
                                 stream)

    def state(self, i: int) -> np.ndarray:
        """A host copy of run i's state (8-byte aligned)."""
        size = self.sizes[i]
        t = self.d_states[i * self.stride: i * self.stride + size].cpu().numpy()
        raw = np.empty(size + 64, dtype=np.uint8)
        off = (-raw.ctypes.data) % 64
        out = raw[off: off + size]
        out[:] = t
        return out

    def header(self, i: int) -> np.ndarray:
        t = self.d_states[i * self.stride: i * self.stride + 128].cpu().numpy()
        out = np.zeros(128 + 64, dtype=np.uint8)
        off = (-out.ctypes.data) % 64
        h = out[off: off + 128]
        h[:] = t
        return h

    def info(self, i: int) -> dict:
        h = self.header(i)
        e, d = B.fpi8_state_info(h)
        if e:
            raise ValueError(f"state {i}: error {e}")
        return d
