"""Parity over the decode windows of the full-size workloads, through the C ABI.

Every workload's model and batch width runs on the GPU through its prompt
and into (or through) its decode window; a run of the batch is run by the
oracle from the same start and the two states are compared byte for byte:
the header and cursor, every activation and working vector, the logits,
the scores buffer and every key and value word of the cache ("The resumable
state" lists them).  The page's own invariant is the same one: every target
produces the same tokens and text bytes from the same state.

* 1.1B-shaped, 32 runs of 128 prompt ids and 128 generated tokens, run to
  completion; two runs compared.
* 7B-shaped, 64 runs of 512 prompt ids, through position 663, past the
  decode positions the benchmark times (it centres them on the window's
  middle, position 639); one run compared.
* The long-context layer shape (dim 2048, 16 heads of 128, FFN 5632, vocab
  32000, context 8192) with 2 layers instead of 16, 16 runs of 7,936 prompt
  ids, through position 7,945: attention over up to 7,946 cached positions
  per head.  One run compared with the oracle, and a second run fed the
  same ids compared with it on the GPU.

The oracle runs its heads and matrix rows on 16 host threads (each word is
still computed whole).  These take minutes: marked slow as well as gpu.
"""
import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads import blob as Bl
from workloads.configs import Shape
from fixed_point_int8_amd.device import DeviceBatch, DeviceModel
from gpu_helpers import diff_report, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def oracle_run(cfg, blob, spec, positions):
    ids, mx, t, s = spec
    e, st = O.init_state(cfg, ids, mx, t, s)
    assert e == 0
    assert O.turn(blob, st, positions) == 0
    return st


def compare(cfg, spec, got, want, label):
    if not np.array_equal(got, want):
        raise AssertionError(f"{label}: " + diff_report(cfg, spec, got, want))


def test_decode_window_1b_to_completion():
    w = W.by_name("1.1B-shaped-d2048-L22")
    shape, cfg = w.shape, w.shape.as_tuple()
    say("decode window 1.1B: artifact")
    blob = Bl.build_blob(shape, w.blob_seed)
    runs = [(W.prompt_ids(shape.vocab, w.prompt, w.ids_seed, r), w.max_tokens, w.temperature_q16,
             w.run_seed + r) for r in range(w.runs)]
    model = DeviceModel(blob, w.runs)
    O.set_threads(16)
    try:
        batch = DeviceBatch(cfg, runs)
        positions = w.prompt + w.max_tokens - 1
        say(f"decode window 1.1B: {positions} positions x {w.runs} runs on the GPU")
        e, errs = batch.turn(model, positions)
        assert e == 0 and not any(errs), (e, list(errs))
        for r in (0, w.runs - 1):
            say(f"decode window 1.1B: oracle run {r}")
            want = oracle_run(cfg, blob, runs[r], positions)
            info = O.state_info(want)[1]
            assert info["complete"] and not info["error"]
            compare(cfg, runs[r], batch.state(r), want, f"1.1B run {r}")
    finally:
        model.close()
        O.set_threads(1)


def test_decode_window_7b_through_benchmark_steps():
    w = W.by_name("7B-shaped-d4096-L32")
    shape, cfg = w.shape, w.shape.as_tuple()
    say("decode window 7B: artifact")
    blob = Bl.build_blob(shape, w.blob_seed)
    runs = [(W.prompt_ids(shape.vocab, w.prompt, w.ids_seed, r), w.max_tokens, w.temperature_q16,
             w.run_seed + r) for r in range(w.runs)]
    model = DeviceModel(blob, w.runs)
    O.set_threads(16)
    try:
        batch = DeviceBatch(cfg, runs)
        positions = 664  # positions 0 .. 663
        say(f"decode window 7B: {positions} positions x {w.runs} runs on the GPU")
        e, errs = batch.turn(model, positions)
        assert e == 0 and not any(errs), (e, list(errs))
        assert batch.info(0)["position"] == positions
        got = batch.state(0)
        del batch
        say("decode window 7B: oracle run 0 (about 2.5 minutes)")
        want = oracle_run(cfg, blob, runs[0], positions)
        assert O.state_info(want)[1]["position"] == positions
        compare(cfg, runs[0], got, want, "7B run 0")
    finally:
        model.close()
        O.set_threads(1)


def test_decode_window_long_context_layers():
    full = W.by_name("long-context-8k-d2048-L16")
    fs = full.shape
    shape = Shape(fs.dim, fs.hidden, 2, fs.heads, fs.kv_heads, fs.vocab, fs.context)
    cfg = shape.as_tuple()
    say("decode window long context, 2 layers: artifact")
    blob = Bl.build_blob(shape, full.blob_seed)
    runs = [(W.prompt_ids(shape.vocab, full.prompt, full.ids_seed, r), full.max_tokens,
             full.temperature_q16, full.run_seed + r) for r in range(full.runs)]
    # the last run is fed run 0's ids (and seed): its state must be run 0's
    runs[-1] = runs[0]
    model = DeviceModel(blob, full.runs)
    O.set_threads(16)
    try:
        batch = DeviceBatch(cfg, runs)
        positions = full.prompt + 10  # positions 0 .. 7945
        say(f"decode window long context: {positions} positions x {full.runs} runs on the GPU")
        e, errs = batch.turn(model, positions)
        assert e == 0 and not any(errs), (e, list(errs))
        got0 = batch.state(0)
        compare(cfg, runs[0], batch.state(full.runs - 1), got0, "long context, same ids")
        say("decode window long context: oracle run 0")
        want = oracle_run(cfg, blob, runs[0], positions)
        assert O.state_info(want)[1]["position"] == positions
        compare(cfg, runs[0], got0, want, "long context run 0")
    finally:
        model.close()
        O.set_threads(1)
