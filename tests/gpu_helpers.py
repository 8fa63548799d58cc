"""Helpers of the GPU parity tests: run a batch on the GPU through the C ABI
and the same runs through the oracle, and compare states byte for byte."""
from __future__ import annotations

import sys

import numpy as np

import oracle as O
from fixed_point_int8_amd import binding as B
from fixed_point_int8_amd.device import DeviceBatch, DeviceModel

REGIONS = ("ids", "out", "x", "w1", "w2", "w3", "gate", "up", "logits", "scores", "keys",
           "values")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    return torch


def diff_report(cfg, run_spec, a: np.ndarray, b: np.ndarray) -> str:
    ids, mx = run_spec[0], run_spec[1]
    off = B.fpi8_state_offsets(cfg, len(ids), mx)
    bounds = [("header", 0, 128)]
    for i, name in enumerate(REGIONS):
        end = off[REGIONS[i + 1]] if i + 1 < len(REGIONS) else off["total"]
        bounds.append((name, off[name], end))
    msgs = []
    for name, lo, hi in bounds:
        if not np.array_equal(a[lo:hi], b[lo:hi]):
            d = np.nonzero(a[lo:hi] != b[lo:hi])[0]
            msgs.append(f"{name}: {d.size} bytes differ, first at +{d[0]}")
    return "; ".join(msgs)


class Pair:
    """The same runs on the GPU (one batch) and in the oracle (one by one)."""

    def __init__(self, shape, blob, runs, model=None, max_runs=None):
        self.cfg = shape.as_tuple()
        self.blob = blob
        self.runs = runs
        self.model = model or DeviceModel(blob, max_runs or len(runs))
        self.batch = DeviceBatch(self.cfg, runs)
        self.ref = []
        for ids, mx, t, s in runs:
            e, st = O.init_state(self.cfg, ids, mx, t, s)
            assert e == 0
            self.ref.append(st)
        self.ref_err = [0] * len(runs)

    def turn(self, k, oracle_runs=None):
        e, errs = self.batch.turn(self.model, k)
        assert e < 100, f"HIP failure {e}"
        for i in (range(len(self.runs)) if oracle_runs is None else oracle_runs):
            self.ref_err[i] = O.turn(self.blob, self.ref[i], k)
        return errs

    def compare(self, runs=None):
        for i in (range(len(self.runs)) if runs is None else runs):
            g = self.batch.state(i)
            r = self.ref[i]
            if not np.array_equal(g, r):
                raise AssertionError(f"run {i}: " + diff_report(self.cfg, self.runs[i], g, r))

    def load(self, i, st):
        """Run i becomes the oracle state st, on both sides."""
        import torch
        assert st.size == self.ref[i].size
        self.ref[i][:] = st
        b = self.batch
        b.d_states[i * b.stride: i * b.stride + st.size].copy_(torch.from_numpy(st.copy()))

    def complete(self):
        return all(O.state_info(s)[1]["complete"] or O.state_info(s)[1]["error"] for s in self.ref)
