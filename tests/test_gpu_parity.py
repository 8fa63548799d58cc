"""Parity of the HIP path with the oracle, bit for bit, through the C ABI.

Small shapes run whole (every state byte after every turn); the row kernel
is checked on ragged shapes, adversarial 64-bit inputs (which take the exact
64-bit path) and the full 4096 x 4096 sweep.
"""
import math

import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads import blob as Bl
from workloads.configs import Shape
from fixed_point_int8_amd import binding as B
from fixed_point_int8_amd.device import DeviceModel
from gpu_helpers import Pair, require_gpu, say

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# The matrix row, standalone

def gpu_rows_packed(Wm, s, x):
    torch = require_gpu()
    rows, cols = Wm.shape
    batch = x.shape[0]
    dW = torch.from_numpy(np.ascontiguousarray(Wm)).cuda()
    n_p = B.fpi8_matrix_packed_size(rows, cols)
    dP = torch.empty(n_p, dtype=torch.uint8, device="cuda")
    assert B.fpi8_matrix_pack(dW, rows, cols, dP, n_p) == 0
    del dW  # the packed copy alone serves the calls
    dS = torch.from_numpy(np.ascontiguousarray(s).view(np.int32)).cuda()
    dX = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    dY = torch.zeros((batch, rows), dtype=torch.int64, device="cuda")
    n = B.fpi8_matrix_rows_workspace_size(rows, cols, batch)
    dWk = torch.zeros(n, dtype=torch.uint8, device="cuda")
    assert B.fpi8_matrix_rows_packed(dP, dS, rows, cols, dX, batch, dY, dWk, n) == 0
    torch.cuda.synchronize()
    return dY.cpu().numpy()


@pytest.mark.parametrize("rows,cols,batch", [
    (1, 1, 1), (37, 172, 3), (100, 300, 17), (129, 4096, 64), (33, 64, 128), (48, 11008, 8),
    (200, 2048, 65), (4096, 4096, 128), (12000, 384, 50), (12290, 128, 33), (4096, 4096, 1),
    (4096, 4096, 8), (100, 4096, 8), (7, 100, 2), (40, 1000, 5), (24, 2752, 2), (20, 40000, 2)])
def test_matrix_rows_packed(rows, cols, batch):
    # (12000, 384, 50) takes the shared-digit kernel with three row-owning
    # waves, its last workgroup ending inside the matrix; (12290, 128, 33)
    # four row-owning waves with rows past the last full tile.
    say(f"matrix_rows_packed {rows}x{cols} batch {batch}")
    Wm, s, x = W.row_operands(rows, cols, batch, rows * 1000 + cols + batch + 5)
    assert np.array_equal(gpu_rows_packed(Wm, s, x), O.rows(Wm, s, x))


def test_matrix_rows_packed_exact_path():
    Wm, s, _ = W.row_operands(40, 200, 5, 9)
    x = W.adversarial_row_inputs(5, 200, 10)
    assert np.array_equal(gpu_rows_packed(Wm, s, x), O.rows(Wm, s, x))


# Matrices of 65,536 rows or more (the stream launch's threshold on 256
# compute units: every wave gets a tile of 64 rows) with a multiple of 8
# blocks of 64 columns take the persistent streaming kernels: the
# digit-sharing shapes up to 64 inputs, the weight-sharing one from 65 to
# 128.  Rows past the last full tile, columns inside the last block, inputs
# that end inside a run tile, and every launch-shape boundary.
@pytest.mark.parametrize("rows,cols,batch", [
    (65573, 4066, 1), (65536, 4096, 8), (65552, 512, 16), (65536, 4096, 17), (65600, 4096, 32),
    (65536, 2048, 33), (65541, 4096, 64), (65536, 512, 65), (65536, 512, 100), (65536, 4096, 128),
    (65573, 4066, 97), (66000, 1024, 128), (131072, 512, 3)])
def test_matrix_rows_packed_stream(rows, cols, batch):
    say(f"matrix_rows_packed stream {rows}x{cols} batch {batch}")
    O.set_threads(16)
    try:
        Wm, s, x = W.row_operands(rows, cols, batch, rows + cols * 7 + batch)
        assert np.array_equal(gpu_rows_packed(Wm, s, x), O.rows(Wm, s, x))
    finally:
        O.set_threads(1)


@pytest.mark.parametrize("batch", [5, 40, 100])
def test_matrix_rows_packed_stream_exact_path(batch):
    # A word beyond three digits sends the whole streaming launch down the
    # exact 64-bit loop; extreme weights and scales in the first rows.
    rows, cols = 65536, 512
    O.set_threads(16)
    try:
        Wm, s, x = W.row_operands(rows, cols, batch, 77 + batch)
        x[batch - 1, cols - 1] = -(2**45) + 3
        x[0, :64] = W.adversarial_row_inputs(1, 64, batch)[0]
        Wm[0, :] = 0
        Wm[1, :] = 255
        s[0] = 2**32 - 1
        s[2] = 0
        assert np.array_equal(gpu_rows_packed(Wm, s, x), O.rows(Wm, s, x))
    finally:
        O.set_threads(1)


# The vector-ALU streaming kernel (fpi8_matrix_rows_set_path(2)): 1 to 4
# inputs whose digits sit in LDS, v_dot4 over the packed tiles.  Rows past
# the last full tile, columns inside the last block, the largest column
# count its LDS holds for four inputs, a word beyond three digits (the exact
# loop), and five inputs (not taken: the matrix-core kernel runs).
@pytest.mark.parametrize("rows,cols,batch,big", [
    (65573, 4066, 1, False), (65536, 1000, 2, False), (65600, 4096, 3, False),
    (65536, 4096, 4, False), (65536, 12288, 4, False), (65536, 512, 2, True), (65536, 512, 5, False)])
def test_matrix_rows_packed_stream_valu(rows, cols, batch, big):
    say(f"matrix_rows_packed stream, vector ALU, {rows}x{cols} batch {batch} big {big}")
    O.set_threads(16)
    assert B.fpi8_matrix_rows_set_path(B.PATH_VALU) == 0
    try:
        Wm, s, x = W.row_operands(rows, cols, batch, rows + cols * 11 + batch)
        if big:
            x[batch - 1, 7] = 2**40 + 5
            x[0, :64] = W.adversarial_row_inputs(1, 64, batch)[0]
            Wm[0, :] = 255
            s[1] = 2**32 - 1
        assert np.array_equal(gpu_rows_packed(Wm, s, x), O.rows(Wm, s, x))
    finally:
        B.fpi8_matrix_rows_set_path(B.PATH_AUTO)
        O.set_threads(1)


def test_matrix_rows_set_path_rejects_unknown():
    assert B.fpi8_matrix_rows_set_path(3) == 102
    assert B.fpi8_matrix_rows_set_path(-1) == 102
    assert B.fpi8_matrix_rows_set_path(B.PATH_AUTO) == 0


def gpu_rows(Wm, s, x, work=None):
    torch = require_gpu()
    rows, cols = Wm.shape
    batch = x.shape[0]
    dW = torch.from_numpy(np.ascontiguousarray(Wm)).cuda()
    dS = torch.from_numpy(np.ascontiguousarray(s).view(np.int32)).cuda()
    dX = torch.from_numpy(np.ascontiguousarray(x)).cuda()
    dY = torch.zeros((batch, rows), dtype=torch.int64, device="cuda")
    n = B.fpi8_matrix_rows_workspace_size(rows, cols, batch)
    dWk = work if work is not None else torch.zeros(n, dtype=torch.uint8, device="cuda")
    e = B.fpi8_matrix_rows(dW, dS, rows, cols, dX, batch, dY, dWk, n)
    assert e == 0
    torch.cuda.synchronize()
    return dY.cpu().numpy()


@pytest.mark.parametrize("rows,cols,batch", [
    (16, 64, 1), (1, 1, 1), (37, 172, 3), (100, 300, 17), (256, 512, 32), (129, 4096, 64),
    (64, 128, 100), (33, 64, 128), (48, 11008, 8), (200, 2048, 65), (24, 65536, 3),
    (20, 40000, 2), (20, 40000, 1), (20, 16384, 2)])
def test_matrix_rows_random(rows, cols, batch):
    say(f"matrix_rows {rows}x{cols} batch {batch}")
    Wm, s, x = W.row_operands(rows, cols, batch, rows * 1000 + cols + batch)
    assert np.array_equal(gpu_rows(Wm, s, x), O.rows(Wm, s, x))


@pytest.mark.parametrize("rows,cols,batch", [(16, 64, 2), (40, 100, 5), (64, 256, 33)])
def test_matrix_rows_adversarial_inputs(rows, cols, batch):
    say(f"matrix_rows adversarial {rows}x{cols} batch {batch}")
    Wm, s, _ = W.row_operands(rows, cols, batch, 7)
    x = W.adversarial_row_inputs(batch, cols, rows + cols)
    Wm[0, :] = 0
    Wm[1, :] = 255
    s[0] = 2**32 - 1
    s[2] = 0
    assert np.array_equal(gpu_rows(Wm, s, x), O.rows(Wm, s, x))


@pytest.mark.parametrize("batch,packed", [(1, False), (2, True), (8, False), (8, True)])
def test_matrix_rows_one_wave_exact(batch, packed):
    # Calls of at most 8 inputs split their digits per wave; one word too
    # wide for three digits, in the last wave's columns only, sends that wave
    # alone down the exact path.
    rows, cols = 64, 4096
    Wm, s, x = W.row_operands(rows, cols, batch, 41 + batch)
    x[batch - 1, cols - 5] = 2**40 + 12345
    ref = O.rows(Wm, s, x)
    got = gpu_rows_packed(Wm, s, x) if packed else gpu_rows(Wm, s, x)
    assert np.array_equal(got, ref)


def test_matrix_rows_three_digit_edges():
    # Inputs at the edges of the three-digit range, and one just outside it.
    Wm, s, _ = W.row_operands(32, 128, 4, 3)
    edge = np.array([-8421504, 8355711, -8421505, 8355712, 8388607, -8388608], dtype=np.int64)
    x = np.resize(edge, (4, 128)).astype(np.int64)
    assert np.array_equal(gpu_rows(Wm, s, x), O.rows(Wm, s, x))
    x2 = np.resize(edge[:2], (4, 128)).astype(np.int64)
    assert np.array_equal(gpu_rows(Wm, s, x2), O.rows(Wm, s, x2))


@pytest.mark.parametrize("batch", [3, 40])
def test_matrix_rows_reused_workspace(batch):
    # One workspace (filled with 0xFF, not zeros) across calls whose inputs
    # alternately need and do not need the exact path: the overflow mark of
    # one call must not leak into the next.
    torch = require_gpu()
    rows, cols = 48, 320
    Wm, s, x = W.row_operands(rows, cols, batch, 31)
    xa = W.adversarial_row_inputs(batch, cols, 32)
    n = B.fpi8_matrix_rows_workspace_size(rows, cols, batch)
    work = torch.full((n,), 255, dtype=torch.uint8, device="cuda")
    for xi in (x, xa, x, x, xa, xa, x):
        assert np.array_equal(gpu_rows(Wm, s, xi, work), O.rows(Wm, s, xi))


@pytest.mark.parametrize("batch", W.ROW_SWEEP_BATCHES)
def test_matrix_rows_4096_sweep(batch):
    say(f"matrix_rows 4096x4096 batch {batch}")
    O.set_threads(16)
    Wm, s, x = W.row_operands(W.ROW_SWEEP_ROWS, W.ROW_SWEEP_COLS, batch, W.ROW_SWEEP_SEED)
    try:
        assert np.array_equal(gpu_rows(Wm, s, x), O.rows(Wm, s, x))
    finally:
        O.set_threads(1)


# ---------------------------------------------------------------------------
# The whole pass on small shapes

def spec(shape, n_runs, prompt, max_tokens, seed=0, temps=None, seeds=None):
    runs = []
    for r in range(n_runs):
        p = prompt[r] if isinstance(prompt, (list, tuple)) else prompt
        m = max_tokens[r] if isinstance(max_tokens, (list, tuple)) else max_tokens
        ids = W.prompt_ids(shape.vocab, p, 100 + seed, r)
        t = temps[r] if temps else 0
        sd = seeds[r] if seeds else 42 + r
        runs.append((ids, m, t, sd))
    return runs


def run_pair(shape, blob, runs, cuts, compare_every=True, row_kernel=0, streams=0, graph=True):
    pair = Pair(shape, blob, runs)
    assert B.fpi8_engine_set_row_kernel(pair.model.engine, row_kernel) == 0
    assert B.fpi8_engine_set_streams(pair.model.engine, streams) == 0
    assert B.fpi8_engine_set_graph(pair.model.engine, graph) == 0
    try:
        for k in cuts:
            pair.turn(k)
            if compare_every:
                pair.compare()
            if pair.complete():
                break
        while not pair.complete():
            pair.turn(1 << 20)
        pair.compare()
    finally:
        pair.model.close()
    return pair


def test_tiny_workload_position_by_position():
    w = W.TINY
    say("tiny workload")
    blob = Bl.build_blob(w.shape, w.blob_seed)
    runs = [(W.prompt_ids(w.shape.vocab, w.prompt, w.ids_seed, 0), w.max_tokens, 0, w.run_seed)]
    pair = run_pair(w.shape, blob, runs, [1] * 31)
    info = O.state_info(pair.ref[0])[1]
    assert info["complete"] and info["generated"] == 16


def test_tiny_prefix_runs_in_one_batch():
    # P = k ids and one generated token, k = 1..16: runs of sixteen sizes at
    # one stride; a greedy token at every fed position.
    w = W.TINY
    say("tiny prefix runs")
    blob = Bl.build_blob(w.shape, w.blob_seed)
    ids = W.prompt_ids(w.shape.vocab, w.prompt, w.ids_seed, 0)
    runs = [(ids[:k], 1, 0, 0) for k in range(1, 17)]
    run_pair(w.shape, blob, runs, [3, 5, 100])


def test_tiny_context_fills_exactly():
    w = W.TINY
    blob = Bl.build_blob(w.shape, w.blob_seed)
    ids = W.prompt_ids(w.shape.vocab, 16, w.ids_seed, 0)
    run_pair(w.shape, blob, [(ids, 17, 0, 0)], [40])


@pytest.mark.parametrize("name", ["gqa", "ragged", "wide", "h8", "h256", "h4"])
def test_small_shapes_greedy(name):
    shape = W.SMALL_SHAPES[name]
    say(f"small shape {name}")
    blob = Bl.build_blob(shape, 11)
    runs = spec(shape, 5, [1, 4, 7, 2, 9], [9, 5, 3, 12, 1])
    run_pair(shape, blob, runs, [1, 2, 3, 1, 5])


@pytest.mark.parametrize("name", ["h256", "h4", "gqa", "split"])
def test_small_shapes_one_layout(name):
    # Every run of the batch with the same layout: the normalization and
    # attention read through the common offsets (queries and first keys
    # requested before the run descriptors), at head sizes 256, 4, 16
    # (grouped) and 128.
    shape = W.SMALL_SHAPES[name]
    say(f"small shape {name}, one layout")
    blob = Bl.build_blob(shape, 13)
    runs = spec(shape, 6, 5, 8, seed=9)
    run_pair(shape, blob, runs, [1, 3, 2, 6])


def test_one_arena_across_layouts():
    # The engine records a position as a graph per (arena, run count, score
    # slots, layout).  When every run of a batch has the same buffer offsets,
    # the normalization and attention read through those offsets before the
    # run descriptors arrive; the same arena then holds batches whose runs
    # differ (the descriptors' path) and another common layout: each must
    # record its own graph, or the step reads the previous batch's offsets.
    torch = require_gpu()
    shape = W.SMALL_SHAPES["wide"]
    cfg = shape.as_tuple()
    say("one arena across layouts")
    blob = Bl.build_blob(shape, 31)
    batches = [spec(shape, 4, 5, 6, seed=1),                  # one layout
               spec(shape, 4, [3, 4, 5, 7], [6, 5, 4, 3], seed=2),  # four layouts
               spec(shape, 4, 9, 4, seed=3),                  # one layout, other offsets
               spec(shape, 4, 5, 6, seed=4)]                  # the first layout again
    stride = max(B.fpi8_state_size(cfg, len(ids), mx) for b in batches for ids, mx, _, _ in b)
    stride = (stride + 255) // 256 * 256
    model = DeviceModel(blob, 4)
    try:
        arena = None
        for k, runs in enumerate(batches):
            pair = Pair(shape, blob, runs, model=model)
            if arena is None:
                arena = torch.zeros(4 * stride, dtype=torch.uint8, device="cuda")
            # the batch's fresh states, moved into the one arena at the one stride
            arena.zero_()
            b = pair.batch
            for i in range(4):
                arena[i * stride: i * stride + b.sizes[i]].copy_(b.d_states[i * b.stride: i * b.stride + b.sizes[i]])
            b.d_states, b.stride = arena, stride
            for cut in (2, 3):
                pair.turn(cut)
                pair.compare()
            say(f"batch {k} matches")
    finally:
        model.close()


@pytest.mark.parametrize("n_runs", [3, 20, 40, 70])
def test_split_contraction_whole_pass(n_runs):
    # dim 1024 and hidden 2816: every matrix's columns are shared by several
    # workgroups; 20, 40 and 70 runs take the wider tiles.
    shape = W.SMALL_SHAPES["split"]
    say(f"split shape, {n_runs} runs")
    blob = Bl.build_blob(shape, 21)
    runs = spec(shape, n_runs, [1 + (r % 5) for r in range(n_runs)], [2 + (r % 4) for r in range(n_runs)])
    run_pair(shape, blob, runs, [2, 3])


@pytest.mark.parametrize("row_kernel", [1, 2, 3, 4, 5, 6, 7])
@pytest.mark.parametrize("n_runs", [3, 20, 70])
def test_row_kernels_whole_pass(n_runs, row_kernel):
    # Every matrix of the split shape has a column count that is a multiple
    # of 128, so both row kernels can run all of them: 1 forces the kernel
    # whose waves split the contraction, 2 the one that shares digits in LDS,
    # 3 that one with three row-owning waves, so that workgroups end inside
    # a matrix and span the Q/K and K/V boundaries, 4 to 6 that one with 3,
    # 6 or 12 waves all owning rows (16, 32 or 64 runs per workgroup), 7 the
    # default's multi-wave shapes (seven stages in flight) at this width.
    shape = W.SMALL_SHAPES["split"]
    say(f"split shape, {n_runs} runs, row kernel {row_kernel}")
    blob = Bl.build_blob(shape, 22)
    runs = spec(shape, n_runs, [1 + (r % 4) for r in range(n_runs)], [2 + (r % 3) for r in range(n_runs)])
    run_pair(shape, blob, runs, [1, 3], row_kernel=row_kernel)


@pytest.mark.parametrize("streams,n_runs,graph,one_layout", [
    (2, 5, True, False), (2, 20, True, False), (1, 70, True, False), (1, 20, False, False),
    (2, 20, False, False), (2, 20, True, True), (2, 7, False, True)])
def test_run_groups_on_two_streams(streams, n_runs, graph, one_layout):
    # The batch split in two groups, each advanced on its own stream, and a
    # wide batch on one stream; runs of several layouts, or of one (the
    # second group then reads through the common offsets from its own first
    # run on).
    shape = W.SMALL_SHAPES["gqa"]
    say(f"{n_runs} runs on {streams} stream(s), graph {graph}, one layout {one_layout}")
    blob = Bl.build_blob(shape, 25)
    if one_layout:
        runs = spec(shape, n_runs, 4, 5)
    else:
        runs = spec(shape, n_runs, [1 + (r % 6) for r in range(n_runs)], [1 + (r % 5) for r in range(n_runs)])
    run_pair(shape, blob, runs, [1, 2, 4], streams=streams, graph=graph)


@pytest.mark.parametrize("row_kernel", [2, 3, 4, 5, 6, 7])
def test_shared_kernel_exact_path(row_kernel):
    shape = W.SMALL_SHAPES["split"]
    say(f"exact path, shared-digit row kernel {row_kernel}")
    norm = np.full((2 * shape.layers + 1) * shape.dim, 1 << 30, dtype=np.int32)
    blob = Bl.build_blob(shape, 23, tables={"norm": norm})
    runs = spec(shape, 5, [2, 3, 1, 4, 2], 3)
    run_pair(shape, blob, runs, [1, 10], row_kernel=row_kernel)


def test_long_context_attention():
    # Attention over thousands of cached positions, with a shorter run
    # beside the long one.
    shape = Shape(256, 512, 2, 2, 2, 300, 4096)
    say("long context 4096, 3000 ids")
    blob = Bl.build_blob(shape, 24)
    runs = [(W.prompt_ids(shape.vocab, 3000, 124, 0), 3, 0, 1),
            (W.prompt_ids(shape.vocab, 700, 124, 1), 2, 0, 2)]
    O.set_threads(16)
    try:
        run_pair(shape, blob, runs, [1500, 100000], compare_every=False)
    finally:
        O.set_threads(1)


def test_full_context_score_buffer():
    # A run whose cache spans the whole 8192-entry context (the long-context
    # workload's): 8192 prompt ids and one generated token, so the last
    # position attends over all 8192 cached positions and attention keeps
    # 8192 scores in LDS, the largest buffer.  Checked halfway and at the end.
    shape = Shape(128, 256, 1, 1, 1, 300, 8192)
    say("full 8192 context")
    blob = Bl.build_blob(shape, 26)
    runs = [(W.prompt_ids(shape.vocab, 8192, 126, 0), 1, 0, 1),
            (W.prompt_ids(shape.vocab, 100, 126, 1), 3, 0, 2)]
    O.set_threads(16)
    pair = Pair(shape, blob, runs)
    try:
        pair.turn(4096)
        pair.compare()
        pair.turn(4096)
        pair.compare()
        info = O.state_info(pair.ref[0])[1]
        assert info["position"] == 8192 and info["generated"] == 1 and info["complete"]
    finally:
        pair.model.close()
        O.set_threads(1)


def test_argmax_ties_across_sampling_chunks():
    # Classifier rows repeat with period 7 (weights and scales), so every
    # logit value occurs at indices k, k + 7, k + 14, ... spread over all of
    # the sampler's per-thread chunks: at temperature zero the lowest index
    # of the largest value must win ("Sampling": lowest index on ties), and
    # above zero the draw walks the tied entries in index order.  A second
    # model repeats its rows with period 300, so tied maxima sit in chunks
    # far apart.
    for period, vocab in ((7, 1000), (300, 32000)):
        shape = Shape(64, 172, 1, 4, 4, vocab, 32)
        say(f"argmax ties, period {period}, vocab {vocab}")
        blob = Bl.build_blob(shape, 40 + period)
        Wc, Sc = Bl.matrix_view(blob, shape, Bl.KIND_CLS)
        for r in range(period, vocab):
            Wc[r] = Wc[r % period]
            Sc[r] = Sc[r % period]
        runs = [(W.prompt_ids(vocab, 3 + r % 4, 50 + period, r), 6, (0, 0, 65536, 45000)[r % 4],
                 r + 1) for r in range(8)]
        pair = run_pair(shape, blob, runs, [1, 2, 100])
        for r, (ids, mx, t, _) in enumerate(runs):
            st = pair.ref[r]
            lay = O.state_layout(shape.as_tuple(), len(ids), mx)
            n = O.state_info(st)[1]["generated"]
            toks = st[lay["out"]: lay["out"] + 4 * n].view(np.uint32)
            assert n > 0
            if t == 0:  # every greedy token is the first of its tied maxima
                assert np.all(toks < period), (period, toks)


@pytest.mark.parametrize("name", ["1.1B-shaped-d2048-L22", "7B-shaped-d4096-L32",
                                  "long-context-8k-d2048-L16"])
def test_full_size_first_positions(name):
    # The model and batch width of the workload; prompts of 1 to 3 ids so
    # that the first positions generate (classifier and sampling at full
    # size).  Every run advances on the GPU; a sample of runs is checked
    # against the oracle, state for state.
    w = W.by_name(name)
    shape = w.shape
    say(f"full size {name}: artifact")
    blob = Bl.build_blob(shape, w.blob_seed)
    runs = [(W.prompt_ids(shape.vocab, 1 + (r % 3), w.ids_seed, r), 3, 0, w.run_seed + r)
            for r in range(w.runs)]
    sample = sorted({0, 1, 2, w.runs // 2 + 1, w.runs - 1})
    O.set_threads(16)
    pair = Pair(shape, blob, runs)
    try:
        for k in (1, 2):
            say(f"full size {name}: turn of {k}")
            pair.turn(k, oracle_runs=sample)
            pair.compare(sample)
    finally:
        pair.model.close()
        O.set_threads(1)


def test_full_size_7b_longer_prompts():
    # The benchmark's model and batch width (64 runs, graph replay) with
    # prompts of 66 to 70 ids, so attention at head size 128 loops over
    # several batches of cached positions before sampling; two runs are
    # checked against the oracle, state for state, at the end.
    w = W.by_name("7B-shaped-d4096-L32")
    shape = w.shape
    say("full size 7B, longer prompts: artifact")
    blob = Bl.build_blob(shape, w.blob_seed)
    runs = [(W.prompt_ids(shape.vocab, 66 + (r % 5), w.ids_seed, 200 + r), 2, 0, w.run_seed + r)
            for r in range(w.runs)]
    sample = [4, w.runs - 2]
    O.set_threads(16)
    pair = Pair(shape, blob, runs)
    try:
        say("full size 7B, longer prompts: 71 positions")
        pair.turn(71, oracle_runs=sample)
        pair.compare(sample)
    finally:
        pair.model.close()
        O.set_threads(1)


def test_planned_turns():
    # Turns as the planner plans them ("The turn planner"): each turn runs
    # the planned units of work (or finishes the position when it ends with
    # a draw), the GPU state equals the oracle's after every turn, and the
    # run takes the quoted number of turns when it reaches max tokens.
    from oracle import planner as PL
    shape = Shape(96, 160, 3, 8, 2, 300, 64)
    blob = Bl.build_blob(shape, 61)
    s0 = np.ascontiguousarray(Bl.section_zero(blob))
    for temp in (0, 45000):
        say(f"planned turns, temperature {temp}")
        runs = [(W.prompt_ids(shape.vocab, 9, 62, temp), 7, temp, 5)]
        pair = Pair(shape, blob, runs)
        try:
            quote = PL.quote_turns(s0, pair.ref[0])
            e, q = B.fpi8_quote_turns(s0, pair.ref[0])
            assert e == 0 and q == quote
            turns = 0
            while True:
                e, plan = B.fpi8_plan_turn(s0, pair.ref[0])
                assert e == 0
                if plan["units"] == 0:
                    break
                if plan["ends_with_draw"]:
                    pair.turn(1)
                else:
                    e, errs = pair.batch.turn_units(pair.model, plan["units"])
                    assert e == 0 and not any(errs), (e, errs)
                    assert O.turn_units(blob, pair.ref[0], plan["units"]) == 0
                pair.compare()
                turns += 1
            info = O.state_info(pair.ref[0])[1]
            assert info["complete"]
            if info["generated"] == 7:
                assert turns == quote
        finally:
            pair.model.close()


def test_queued_turns():
    # Turns queued back to back on a stream (fpi8_turn_bind, then
    # fpi8_turn_async with no synchronization in between), from a cursor
    # inside a position: the states equal the oracle's, and the per-run
    # errors land in a device array (a run with a broken header keeps its
    # error 3 and is not advanced).
    torch = require_gpu()
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 71)
    runs = [(W.prompt_ids(shape.vocab, 3 + r, 72, r), 6, (0, 65536)[r % 2], r + 1) for r in range(5)]
    pair = Pair(shape, blob, runs)
    try:
        # stop every run inside a position first
        e, errs = pair.batch.turn_units(pair.model, 777)
        assert e == 0
        for i in range(len(runs)):
            assert O.turn_units(blob, pair.ref[i], 777) == 0
        pair.compare()
        bad = pair.batch.d_states[4 * pair.batch.stride: 4 * pair.batch.stride + 8]
        bad.fill_(0)  # run 4: not a state
        stream = torch.cuda.Stream()
        e, herrs = B.fpi8_turn_bind(pair.model.engine, pair.batch.d_states, pair.batch.stride,
                                    len(runs), stream)
        assert e == 3 and list(herrs) == [0, 0, 0, 0, 3]
        derr = torch.full((len(runs),), -1, dtype=torch.int32, device="cuda")
        for k in (1, 2, 1, 3):
            assert B.fpi8_turn_async(pair.model.engine, k, stream, derr) == 0
        stream.synchronize()
        assert derr.cpu().tolist() == [0, 0, 0, 0, 3]
        for i in range(4):
            for k in (1, 2, 1, 3):  # one turn each, as on the GPU
                assert O.turn(blob, pair.ref[i], k) == 0
        pair.compare(range(4))
        # a turn of another kind unbinds the batch
        pair.batch.turn(pair.model, 1)
        assert B.fpi8_turn_async(pair.model.engine, 1, stream, derr) == 102
    finally:
        pair.model.close()


def test_queued_turns_across_layouts():
    # Queued turns over one arena whose batches change layout between binds:
    # one common layout, another common layout, then runs of several
    # layouts.  Each bind decides whether the normalization and attention
    # may read through common offsets, and the recorded graph follows it.
    torch = require_gpu()
    shape = W.SMALL_SHAPES["wide"]
    cfg = shape.as_tuple()
    say("queued turns across layouts")
    blob = Bl.build_blob(shape, 41)
    batches = [spec(shape, 4, 5, 6, seed=5), spec(shape, 4, 7, 5, seed=6),
               spec(shape, 4, [3, 4, 5, 6], [7, 6, 5, 4], seed=7)]
    stride = max(B.fpi8_state_size(cfg, len(ids), mx) for b in batches for ids, mx, _, _ in b)
    stride = (stride + 255) // 256 * 256
    model = DeviceModel(blob, 4)
    arena = torch.zeros(4 * stride, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    derr = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    try:
        for k, runs in enumerate(batches):
            pair = Pair(shape, blob, runs, model=model)
            arena.zero_()
            b = pair.batch
            for i in range(4):
                arena[i * stride: i * stride + b.sizes[i]].copy_(b.d_states[i * b.stride: i * b.stride + b.sizes[i]])
            b.d_states, b.stride = arena, stride
            torch.cuda.synchronize()
            e, herrs = B.fpi8_turn_bind(model.engine, arena, stride, 4, stream)
            assert e == 0 and list(herrs) == [0, 0, 0, 0]
            for cut in (2, 1, 3):
                assert B.fpi8_turn_async(model.engine, cut, stream, derr) == 0
            stream.synchronize()
            assert derr.cpu().tolist() == [0, 0, 0, 0]
            for i in range(4):
                for cut in (2, 1, 3):
                    assert O.turn(blob, pair.ref[i], cut) == 0
            pair.compare()
            say(f"batch {k} matches")
    finally:
        model.close()


def test_full_size_units():
    # Turns of unit budgets at the 1.1B shape and its batch width: the
    # budgets stop runs inside matrices, attention stages and sampling
    # passes at full size, and a sample of runs is checked against the
    # oracle, state for state.
    w = W.by_name("1.1B-shaped-d2048-L22")
    shape = w.shape
    say("full size units: artifact")
    blob = Bl.build_blob(shape, w.blob_seed)
    runs = [(W.prompt_ids(shape.vocab, 1 + (r % 2), w.ids_seed, r), 3, 65536 * (r % 2),
             w.run_seed + r) for r in range(w.runs)]
    sample = [0, 1, 5, w.runs - 1]
    O.set_threads(16)
    pair = Pair(shape, blob, runs)
    try:
        # about a third of a layer, a whole position and a few layers, into
        # the classifier, into sampling
        for k in (7_001, 300_000, 223_400, 30_000, 60_000, 100_000):
            say(f"full size units: turn of {k}")
            e, errs = pair.batch.turn_units(pair.model, k)
            assert e == 0 and not any(errs), (e, errs)
            for i in sample:
                assert O.turn_units(blob, pair.ref[i], k) == 0
            pair.compare(sample)
    finally:
        pair.model.close()
        O.set_threads(1)


def test_generic_head_size():
    shape = Shape(120, 200, 2, 6, 3, 300, 24)  # head 20: the generic attention path
    say("generic head size 20")
    blob = Bl.build_blob(shape, 12)
    runs = spec(shape, 4, [3, 6, 1, 10], [6, 4, 9, 2])
    run_pair(shape, blob, runs, [2, 2, 4])


def test_temperature_sampling():
    shape = W.SMALL_SHAPES["gqa"]
    say("temperature sampling")
    blob = Bl.build_blob(shape, 13)
    temps = [65536, 3 * 65536 // 2, 16 << 16, 1, 0, 32768]
    seeds = [0, 1, 2**64 - 1, 12345, 7, 99]
    runs = spec(shape, 6, [2, 5, 3, 8, 4, 1], 10, temps=temps, seeds=seeds)
    run_pair(shape, blob, runs, [1, 4, 2])


def test_wide_batch_two_chunks():
    # 70 runs: four 16-run tiles per workgroup and a second batch chunk.
    shape = W.SMALL_SHAPES["tiny"]
    say("70 runs")
    blob = Bl.build_blob(shape, 14)
    runs = spec(shape, 70, [1 + (r % 9) for r in range(70)], [1 + (r % 7) for r in range(70)])
    run_pair(shape, blob, runs, [2, 3], compare_every=True)


def test_exact_path_inside_the_model():
    # Normalization weights of 64.0 push the normalized vector beyond the
    # three-digit range, so the matrices take the exact 64-bit path.
    shape = W.SMALL_SHAPES["ragged"]
    say("exact path in the model")
    norm = np.full((2 * shape.layers + 1) * shape.dim, 1 << 30, dtype=np.int32)
    blob = Bl.build_blob(shape, 15, tables={"norm": norm})
    runs = spec(shape, 3, [2, 3, 4], 4)
    run_pair(shape, blob, runs, [1, 1, 10])


# ---------------------------------------------------------------------------
# Errors: the 32-bit cache fit check, invalid states, complete runs

def fit_blob(shape, kind, layer=0, seed=1000):
    bl = Bl.build_blob(shape, seed)
    w, s = Bl.matrix_view(bl, shape, kind, layer)
    w[:] = 255
    s[:] = 2**32 - 1
    return bl


@pytest.mark.parametrize("kind,layer,phase", [(Bl.KIND_K, 0, 6), (Bl.KIND_V, 0, 7), (Bl.KIND_K, 1, 6)])
def test_cache_fit_failure(kind, layer, phase):
    shape = W.SMALL_SHAPES["gqa"]
    say(f"fit failure kind {kind} layer {layer}")
    blob = fit_blob(shape, kind, layer)
    runs = spec(shape, 3, [1, 2, 3], 3)
    pair = Pair(shape, blob, runs)
    try:
        errs = pair.turn(5)
        assert list(errs) == [8, 8, 8]
        for i in range(3):
            gi = pair.batch.info(i)
            ri = O.state_info(pair.ref[i])[1]
            assert pair.ref_err[i] == 8
            assert (gi["error"], gi["phase"], gi["layer"], gi["position"]) == \
                   (ri["error"], ri["phase"], ri["layer"], ri["position"]) == (8, phase, layer, 0)
        errs = pair.turn(1)
        assert list(errs) == [3, 3, 3]
    finally:
        pair.model.close()


def test_rotary_fit_failure():
    shape = Shape(8, 16, 1, 1, 1, 16, 4)
    cos, sin = Bl.rope_tables(shape)
    c45 = round(2**24 * math.sqrt(0.5))
    cos[0, :] = c45
    sin[0, :] = c45
    bl = Bl.build_blob(shape, 5, tables={"cos": cos, "sin": sin,
                                         "norm": np.full(3 * 8, 1 << 24, np.int32)})
    w, s = Bl.matrix_view(bl, shape, Bl.KIND_K, 0)
    E, sE = Bl.matrix_view(bl, shape, Bl.KIND_EMBED, 0)
    E[:] = 129
    sE[:] = 1 << 24
    w[0::2, :] = 255
    w[1::2, :] = 1
    s[:] = int((2**31 - 2**20) / (127 * 8) * 2**24 / 65536)
    pair = Pair(shape, bl, [(np.array([3], np.uint32), 2, 0, 0)])
    try:
        errs = pair.turn(1)
        assert list(errs) == [8] and pair.ref_err[0] == 8
        gi = pair.batch.info(0)
        assert (gi["phase"], gi["layer"], gi["error"]) == (8, 0, 8)
    finally:
        pair.model.close()


def test_invalid_and_complete_runs_in_a_batch():
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 16)
    runs = spec(shape, 4, [3, 3, 3, 3], [1, 4, 4, 4])
    pair = Pair(shape, blob, runs)
    try:
        # break run 2's tag on the device
        pair.batch.d_states[2 * pair.batch.stride] = 0
        errs = pair.turn(1)
        assert list(errs) == [0, 0, 3, 0]
        pair.turn(100, oracle_runs=[0, 1, 3])
        pair.compare(runs=[0, 1, 3])
        # run 0 completed in the first turn; a later turn leaves it as it is
        before = pair.batch.state(0)
        errs = pair.turn(1, oracle_runs=[])
        assert errs[0] == 0 and np.array_equal(before, pair.batch.state(0))
    finally:
        pair.model.close()


# ---------------------------------------------------------------------------
# States that stand between two phases ("The resumable state")

def cut_at(blob, st, position, phase, layer):
    """Advances an oracle state one phase at a time to the cursor."""
    while True:
        i = O.state_info(st)[1]
        if (i["position"], i["phase"], i["layer"]) == (position, phase, layer):
            return
        assert not i["complete"] and i["position"] <= position
        assert O.turn_phases(blob, st, 1) == 0


def phase_cuts(shape, prompt):
    """Every cursor a position has, at a prompt position and at a generating
    one: (position, phase, layer)."""
    out = []
    for t in (1, prompt + 1):
        out.append((t, 3, 0))
        for l in range(shape.layers):
            out += [(t, p, l) for p in range(4, 17)]
    for t in (prompt - 1, prompt + 1):
        out += [(t, p, 0) for p in (17, 18, 19)]
    return out


@pytest.mark.parametrize("row_kernel,streams", [(0, 0), (1, 0), (2, 2), (5, 0)])
def test_resume_between_phases(row_kernel, streams):
    # Oracle runs stopped after every phase of a position, one per run, on
    # the GPU in one batch: the first turn finishes each run's position, and
    # every later word matches the oracle's uninterrupted arithmetic.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 51)
    prompt = 4
    cuts = phase_cuts(shape, prompt)
    n = len(cuts)
    say(f"resume between phases: {n} runs, row kernel {row_kernel}, streams {streams}")
    temps = [0 if r % 3 else 65536 for r in range(n)]
    runs = spec(shape, n, prompt, 5, seed=3, temps=temps)
    pair = Pair(shape, blob, runs)
    assert B.fpi8_engine_set_row_kernel(pair.model.engine, row_kernel) == 0
    assert B.fpi8_engine_set_streams(pair.model.engine, streams) == 0
    try:
        for i, (t, p, l) in enumerate(cuts):
            st = pair.ref[i].copy()
            cut_at(blob, st, t, p, l)
            pair.load(i, st)
        for k in (1, 1, 2):
            errs = pair.turn(k)
            assert not any(errs), errs
            pair.compare()
        while not pair.complete():
            pair.turn(1 << 20)
        pair.compare()
    finally:
        pair.model.close()


# Cursors where the engine's launches meet, so where a turn of phases may
# stop a run: every boundary between two phases but the one inside phase 11.
STOPS = {3, 4, 5, 9, 10, 12, 15, 17, 18, 19}


def cursor(st):
    i = O.state_info(st)[1]
    return i["position"], i["phase"], i["layer"], i["complete"]


def same_but_turns(pair, i, turns):
    """Run i's states agree byte for byte outside the turn counter, which
    counts the GPU's turns (the oracle took one per phase)."""
    g, r = pair.batch.state(i), pair.ref[i].copy()
    assert O.state_info(g)[1]["turns"] == turns
    g[80:88] = 0
    r[80:88] = 0
    if not np.array_equal(g, r):
        from gpu_helpers import diff_report
        raise AssertionError(f"run {i}: " + diff_report(pair.cfg, pair.runs[i], g, r))


@pytest.mark.parametrize("row_kernel,streams", [(0, 0), (2, 2)])
def test_stop_between_phases(row_kernel, streams):
    # Turns of k phases on the GPU: each run stops at the last launch
    # boundary within k phases of the oracle's count, in the state the oracle
    # has at that cursor; runs start at every cursor, including those inside
    # a launch, which make no progress until k reaches the next boundary.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 53)
    prompt = 4
    cuts = phase_cuts(shape, prompt)[::3]
    n = len(cuts)
    say(f"stop between phases: {n} runs, row kernel {row_kernel}, streams {streams}")
    temps = [0 if r % 4 else 65536 for r in range(n)]
    runs = spec(shape, n, prompt, 5, seed=5, temps=temps)
    pair = Pair(shape, blob, runs)
    assert B.fpi8_engine_set_row_kernel(pair.model.engine, row_kernel) == 0
    assert B.fpi8_engine_set_streams(pair.model.engine, streams) == 0
    rng = np.random.default_rng(row_kernel * 10 + streams)
    try:
        turns = []
        for i, (t, p, l) in enumerate(cuts):
            st = pair.ref[i].copy()
            cut_at(blob, st, t, p, l)
            pair.load(i, st)
            turns.append(O.state_info(st)[1]["turns"])
        for rounds in range(200):
            if pair.complete():
                break
            live = [i for i in range(n) if not cursor(pair.ref[i])[3]]
            if rng.random() < 0.15:
                errs = pair.turn(1)
                assert not any(errs), errs
                for i in range(n):
                    turns[i] += 1 if i in live else 0
                    same_but_turns(pair, i, turns[i])
                continue
            # small budgets first (every boundary gets its turn), then any
            k = 1 + rounds % 8 if rounds < 40 else int(rng.integers(1, 45))
            e, errs = pair.batch.turn_phases(pair.model, k)
            assert e == 0 and not any(errs), (e, errs)
            for i in range(n):
                want = cursor(pair.batch.state(i))
                ref = pair.ref[i]
                used = 0
                while cursor(ref) != want:
                    assert used < k and not cursor(ref)[3], (i, k, cursor(ref), want)
                    assert O.turn_phases(blob, ref, 1) == 0
                    used += 1
                # the GPU stopped at the last boundary the budget reaches
                probe = ref.copy()
                for _ in range(k - used):
                    if cursor(probe)[3]:
                        break
                    assert O.turn_phases(blob, probe, 1) == 0
                    c = cursor(probe)
                    assert c[1] not in STOPS or c[3], (i, k, used, want, c)
                turns[i] += 1 if i in live else 0
                same_but_turns(pair, i, turns[i])
        assert pair.complete()
    finally:
        pair.model.close()


def test_stop_at_each_boundary():
    # From the start of a prompt position and of a generating one, a turn
    # of k phases for every k up to a position and a half: the cursor is the
    # last boundary within k phases, the state the oracle's at that cursor.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 54)
    prompt = 4
    runs = spec(shape, 2, prompt, 4, seed=6, temps=[0, 65536])
    starts = [(1, 3, 0), (prompt - 1, 3, 0)]
    pair = Pair(shape, blob, runs)
    try:
        cut = []
        for i, (t, p, l) in enumerate(starts):
            st = pair.ref[i].copy()
            cut_at(blob, st, t, p, l)
            cut.append(st)
        per_position = 1 + 13 * shape.layers + 3
        seen = set()
        for k in range(1, per_position * 3 // 2 + 1):
            for i in range(2):
                pair.load(i, cut[i])
            e, errs = pair.batch.turn_phases(pair.model, k)
            assert e == 0 and not any(errs), (k, e, errs)
            for i in range(2):
                ref = cut[i].copy()
                last = ref.copy()
                for _ in range(k):
                    assert O.turn_phases(blob, ref, 1) == 0
                    if cursor(ref)[1] in STOPS:
                        last = ref.copy()
                turns = O.state_info(cut[i])[1]["turns"] + 1
                pair.ref[i][:] = last
                assert cursor(pair.batch.state(i)) == cursor(last), (k, i)
                same_but_turns(pair, i, turns)
                seen.add(cursor(last)[1])
        assert seen == STOPS, seen
    finally:
        pair.model.close()


@pytest.mark.parametrize("row_kernel", [0, 2])
def test_resume_inside_phases(row_kernel):
    # Oracle runs stopped inside a phase (a row of a matrix, a unit of an
    # attention stage, an entry of a sampling pass), from every phase of a
    # prompt and of a generating position: the GPU finishes each position
    # and every later word matches the oracle's.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 55)
    prompt = 4
    cuts = phase_cuts(shape, prompt)
    n = len(cuts)
    say(f"resume inside phases: {n} runs, row kernel {row_kernel}")
    temps = [65536 if r % 2 else 0 for r in range(n)]
    runs = spec(shape, n, prompt, 5, seed=7, temps=temps)
    pair = Pair(shape, blob, runs)
    assert B.fpi8_engine_set_row_kernel(pair.model.engine, row_kernel) == 0
    rng = np.random.default_rng(row_kernel + 1)
    try:
        inside = 0
        for i, (t, p, l) in enumerate(cuts):
            st = pair.ref[i].copy()
            cut_at(blob, st, t, p, l)
            # into the phase: up to a few hundred units (a sampling pass is
            # one unit per vocabulary entry, attention one per position or
            # element)
            assert O.turn_units(blob, st, int(rng.integers(1, 320 if p == 19 else 40))) == 0
            h = st[:128]
            inside += bool(h[16:20].view(np.uint32)[0] or h[100:104].view(np.uint32)[0]
                           or h[120:128].view(np.uint32).any())
            pair.load(i, st)
        assert inside >= n // 3, inside
        for k in (1, 1, 3):
            errs = pair.turn(k)
            assert not any(errs), errs
            pair.compare()
        while not pair.complete():
            pair.turn(1 << 20)
        pair.compare()
    finally:
        pair.model.close()


def test_resume_inside_sampling():
    # Above temperature zero, runs stopped in each sampling pass: in the
    # maximum pass, the sum pass, and the draw pass before and after its
    # first entry (the generator has advanced there; the GPU must not again).
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 56)
    V = shape.vocab
    units = [1, V + 1, 2 * V, 2 * V + 1]
    runs = spec(shape, len(units), 4, 3, seed=8, temps=[65536 * 3 // 2] * len(units))
    pair = Pair(shape, blob, runs)
    try:
        for i, u in enumerate(units):
            st = pair.ref[i].copy()
            cut_at(blob, st, 3, 19, 0)
            assert O.turn_units(blob, st, u) == 0
            assert O.state_info(st)[1]["phase"] == 19, (i, u)
            pair.load(i, st)
        passes = [int(pair.ref[i][100:104].view(np.uint32)[0]) for i in range(len(units))]
        assert passes == [0, 1, 2, 2], passes
        errs = pair.turn(1)
        assert not any(errs), errs
        pair.compare()
        while not pair.complete():
            pair.turn(1 << 20)
        pair.compare()
    finally:
        pair.model.close()


def units_pair_turn(pair, k, blob):
    """A turn of k units on both sides; every run's state must agree."""
    e, errs = pair.batch.turn_units(pair.model, k)
    assert e == 0 and not any(errs), (k, e, errs)
    for i in range(len(pair.runs)):
        if not (O.state_info(pair.ref[i])[1]["complete"]):
            assert O.turn_units(blob, pair.ref[i], k) == 0
    pair.compare()


def test_units_one_at_a_time():
    # Turns of one unit of work each, through a generating position and on,
    # at temperature zero and above: the GPU stops after every row of every
    # matrix, every unit of every attention stage and every vocabulary entry
    # of every sampling pass, in the state the oracle's turn leaves.
    shape = W.TINY.shape
    blob = Bl.build_blob(shape, 57)
    runs = spec(shape, 2, 3, 3, seed=9, temps=[0, 65536])
    pair = Pair(shape, blob, runs)
    try:
        for i in range(2):
            st = pair.ref[i].copy()
            cut_at(blob, st, 2, 3, 0)        # the last prompt position, which generates
            pair.load(i, st)
        seen = set()
        n = 0
        while cursor(pair.ref[0])[0] < 4 or cursor(pair.ref[1])[0] < 4:
            units_pair_turn(pair, 1, blob)
            n += 1
            h = pair.ref[1][:128]
            seen.add((int(h[8:12].view(np.uint32)[0]), int(h[120:124].view(np.uint32)[0]),
                      int(h[100:104].view(np.uint32)[0])))
            assert n < 6000
        say(f"{n} one-unit turns")
        # every phase, every attention stage and every sampling pass stopped in
        assert {p for p, _, _ in seen} >= set(range(3, 20)), seen
        assert {(9, sg) for sg in range(4)} <= {(p, sg) for p, sg, _ in seen}
        assert {(19, ps) for ps in range(3)} <= {(p, ps) for p, _, ps in seen}
        while not pair.complete():
            units_pair_turn(pair, 997, blob)
    finally:
        pair.model.close()


@pytest.mark.parametrize("row_kernel,streams", [(0, 0), (2, 0), (0, 2), (4, 0), (7, 0)])
def test_units_random_budgets(row_kernel, streams):
    # Random budgets over a batch of runs that start at every cursor of a
    # position (between phases and inside them), grouped heads, temperature
    # zero and above.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 58)
    prompt = 4
    cuts = phase_cuts(shape, prompt)[::2]
    n = len(cuts)
    temps = [65536 if r % 2 else 0 for r in range(n)]
    runs = spec(shape, n, prompt, 4, seed=10, temps=temps)
    pair = Pair(shape, blob, runs)
    assert B.fpi8_engine_set_row_kernel(pair.model.engine, row_kernel) == 0
    assert B.fpi8_engine_set_streams(pair.model.engine, streams) == 0
    rng = np.random.default_rng(20 + row_kernel)
    try:
        for i, (t, p, l) in enumerate(cuts):
            st = pair.ref[i].copy()
            cut_at(blob, st, t, p, l)
            assert O.turn_units(blob, st, int(rng.integers(0, 60))) == 0
            pair.load(i, st)
        turns = 0
        while not pair.complete():
            turns += 1
            assert turns < 400
            units_pair_turn(pair, int(rng.choice([rng.integers(1, 50), rng.integers(1, 900),
                                                  rng.integers(1, 5000)])), blob)
        say(f"{turns} turns of units")
    finally:
        pair.model.close()


def test_text_prompt_end_to_end():
    # Text in, text out: prompts tokenized by the library's host tokenizer,
    # the pass on the GPU, the generated tokens' text read back from the
    # device states; against the oracle's tokenizer, turns and text.
    from oracle import tokenizer as T
    from workloads import vocab as V
    shape = W.SMALL_SHAPES["ragged"]
    blob = Bl.build_blob(shape, 67)
    s0 = Bl.section_zero(blob)
    v = T.Vocab(s0)
    runs = []
    for r in range(6):
        prompt = V.sample_text(5 + 3 * r, 80 + r)
        e, ids = B.fpi8_tokenize(s0, prompt, 6)
        assert e == 0 and list(ids) == T.encode(v, prompt, 6)[1]
        runs.append((np.asarray(ids, np.uint32), 6, 0 if r % 2 else 65536, 90 + r))
    say("text prompts end to end")
    pair = run_pair(shape, blob, runs, [2, 3])
    for i, (ids, mx, t, sd) in enumerate(runs):
        g = pair.batch.state(i)
        gen = B.fpi8_output_tokens(g)
        assert B.fpi8_output_text(s0, g) == (0, T.output_text(v, ids, gen))


def test_page_format_round_trip_on_the_gpu():
    # Runs stopped by unit budgets on the GPU, written out in the page's
    # state format and read back (host), then continued on the GPU: every
    # word as the oracle's uninterrupted runs have it.
    from oracle import tokenizer as T
    shape = W.SMALL_SHAPES["ragged"]
    blob = Bl.build_blob(shape, 68)
    s0 = Bl.section_zero(blob)
    cfg = shape.as_tuple()
    prompt = b"Once upon a time"
    e, ids = T.encode(T.Vocab(s0), prompt, 5)
    assert e == 0
    runs = [(np.asarray(ids, np.uint32), 5, 65536 * (r % 2), 100 + r) for r in range(4)]
    pair = Pair(shape, blob, runs)
    try:
        for k in (9_001, 2_500, 17_777):
            units_pair_turn(pair, k, blob)
            for i in range(len(runs)):
                g = pair.batch.state(i)
                e, pg = B.fpi8_state_export(s0, g, prompt, cfg)
                assert e == 0
                e, back = B.fpi8_state_import(cfg, pg)
                assert e == 0 and np.array_equal(back, g)
                pair.load(i, back)
        while not pair.complete():
            pair.turn(1 << 20)
        pair.compare()
    finally:
        pair.model.close()


def test_page_state_from_text_on_the_gpu():
    # Text to text through the page's state format: a fresh page state
    # (library), phases 0-2 in random unit budgets (library, against the
    # oracle's page tokenizer after every call), imported to the GPU and
    # run there to the end, then exported in the page's format: byte for
    # byte the oracle's export of the oracle's run.
    from oracle import pages as OP
    from workloads import vocab as V
    shape = W.SMALL_SHAPES["ragged"]
    blob = Bl.build_blob(shape, 70)
    s0 = Bl.section_zero(blob)
    cfg = shape.as_tuple()
    rng = np.random.default_rng(12)
    prompts = [V.sample_text(int(n), 120 + r) for r, n in enumerate(rng.integers(0, 14, 5))]
    prompts[0] = b""
    runs, imported = [], []
    for r, prompt in enumerate(prompts):
        temp, seed = 65536 * (r % 2), 130 + r
        e, pg = B.fpi8_pages_init(cfg, prompt, 5, temp, seed)
        e2, ref = OP.init(cfg, prompt, 5, temp, seed)
        assert e == e2 == 0 and np.array_equal(pg, ref)
        while OP._u32(ref, 8) < 3:
            b = int(rng.integers(1, 12))
            assert B.fpi8_pages_tokenize(s0, pg, b)[0] == 0
            assert OP.tokenize_units(s0, cfg, ref, b) == 0
            assert np.array_equal(pg, ref)
        e, st = B.fpi8_state_import(cfg, pg)
        assert e == 0
        n = OP._u32(pg, 32)
        L = O.state_layout(cfg, n, 5)
        ids = st[L["ids"]: L["ids"] + 4 * n].view(np.uint32).copy()
        runs.append((ids, 5, temp, seed))
        imported.append(st)
    say("page states from text, on the GPU")
    pair = Pair(shape, blob, runs)
    try:
        for i, st in enumerate(imported):
            assert np.array_equal(st, pair.ref[i])
            pair.load(i, st)
        while not pair.complete():
            pair.turn(3)
        pair.compare()
        for i, prompt in enumerate(prompts):
            e, pg = B.fpi8_state_export(s0, pair.batch.state(i), prompt, cfg)
            assert e == 0
            assert np.array_equal(pg, OP.export(s0, cfg, pair.ref[i], prompt))
    finally:
        pair.model.close()


def test_units_budget_edges():
    # A budget of 0 changes nothing but the turn count; a budget past the
    # end completes a run as a turn of positions does; a complete run is
    # left as it is; a broken state gets error 3 beside runs that go on.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 69)
    runs = spec(shape, 3, 3, 3, seed=11, temps=[0, 65536, 0])
    pair = Pair(shape, blob, runs)
    try:
        before = [pair.batch.state(i) for i in range(3)]
        units_pair_turn(pair, 0, blob)
        for i in range(3):
            g = pair.batch.state(i)
            assert np.array_equal(g[88:], before[i][88:]) and np.array_equal(g[:80], before[i][:80])
        units_pair_turn(pair, 700, blob)
        pair.batch.d_states[2 * pair.batch.stride] = 0          # break run 2's tag
        e, errs = pair.batch.turn_units(pair.model, (1 << 64) - 1)
        assert list(errs) == [0, 0, 3]
        for i in (0, 1):
            assert O.turn_units(blob, pair.ref[i], (1 << 64) - 2) == 0
            assert O.state_info(pair.ref[i])[1]["complete"]
        pair.compare(runs=[0, 1])
        done = pair.batch.state(0)
        e, errs = pair.batch.turn_units(pair.model, 5)
        assert errs[0] == 0 and np.array_equal(done, pair.batch.state(0))
    finally:
        pair.model.close()


def test_resume_cursor_checks():
    # Cursors no turn can leave in the state ("The resumable state") get
    # error 3, on the GPU as in the oracle; the run is left as it is.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 52)
    bad = [(17, 0, 0), (4, shape.layers, 0), (3, 1, 0), (2, 0, 0), (9, 0, shape.heads),
           (21, 0, 0), (5, 0, shape.dim), (4, 0, 1)]
    runs = spec(shape, len(bad), 4, 3, seed=4)
    pair = Pair(shape, blob, runs)
    try:
        for i, (p, l, row) in enumerate(bad):
            st = pair.ref[i].copy()
            cut_at(blob, st, 1, 5, 0)
            st[8:12] = np.frombuffer(np.uint32(p).tobytes(), np.uint8)
            st[12:16] = np.frombuffer(np.uint32(l).tobytes(), np.uint8)
            st[16:20] = np.frombuffer(np.uint32(row).tobytes(), np.uint8)
            assert O.turn(blob, st.copy(), 1) == 3
            pair.load(i, st)
        before = [pair.batch.state(i) for i in range(len(bad))]
        errs = pair.turn(1, oracle_runs=[])
        assert list(errs) == [3] * len(bad)
        for i in range(len(bad)):
            assert np.array_equal(before[i], pair.batch.state(i))
    finally:
        pair.model.close()


def test_stop_token_completes_a_run():
    from test_oracle_pins import stop_token_blob
    shape = W.TINY.shape
    bl = stop_token_blob(shape)
    runs = spec(shape, 2, [2, 5], 6)
    pair = run_pair(shape, bl, runs, [1, 1, 3])
    for i in range(2):
        info = O.state_info(pair.ref[i])[1]
        assert info["complete"] and info["generated"] == 1


def test_engine_rejects_bad_artifacts():
    require_gpu()
    import torch
    shape = W.SMALL_SHAPES["gqa"]
    bl = Bl.build_blob(shape, 17)
    s0 = Bl.section_zero(bl)
    d = torch.from_numpy(bl).cuda()
    bad = s0.copy(); bad[0] = 0
    assert B.fpi8_engine_create(bad, d, bl.size, 4)[0] == 2
    assert B.fpi8_engine_create(s0, d, int(Bl.plan(shape).sections[-1][0]) + 8, 4)[0] == 5
    e, h = B.fpi8_engine_create(s0, d, bl.size, 4)
    assert e == 0
    B.fpi8_engine_destroy(h)


def test_turn_rejects_bad_batches():
    # An empty batch and one wider than the engine are argument errors
    # before anything is read; a misaligned stride, or one shorter than a
    # state, fails every run with error 3 and leaves the states unchanged.
    shape = W.SMALL_SHAPES["gqa"]
    blob = Bl.build_blob(shape, 18)
    runs = spec(shape, 3, 4, 3, seed=12)
    say("turn argument checks")
    pair = Pair(shape, blob, runs, max_runs=3)
    try:
        b, eng = pair.batch, pair.model.engine
        before = [b.state(i).copy() for i in range(3)]
        assert B.fpi8_turn(eng, b.d_states, b.stride, 0, 1)[0] == B.ERR_ARGUMENT
        assert B.fpi8_turn(eng, b.d_states, b.stride, 4, 1)[0] == B.ERR_ARGUMENT
        for stride in (b.stride - 4, 128, b.sizes[0] - 8):
            e, errs = B.fpi8_turn(eng, b.d_states, stride, 3, 1)
            assert e == 3 and list(errs) == [3, 3, 3], (stride, e, list(errs))
        for i in range(3):
            assert np.array_equal(b.state(i), before[i])
        # the same batch with its own stride goes on as the oracle does
        pair.turn(2)
        pair.compare()
    finally:
        pair.model.close()
