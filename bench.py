"""Benchmark: decode throughput of the fixed-point forward pass on one MI355X.

One step is one position of every run of the batch through the whole path:
embedding, every layer (normalization, query/key/value rows with rotary and
the cache store, attention, output rows, normalization, gate/up rows with
SiLU, down rows), the final normalization, the classifier rows and sampling.
The workload is the 7B-shaped model (dim 4096, 32 layers, 32 heads of 128,
FFN 11008, vocab 32000) with 64 runs of 512 prompt ids each; the prompts
are prefilled first (untimed), then W warm-up steps and K timed decode
steps run (by default K covers the rest of the 255-step decode window but
for 8 kernel-timed steps at its end).  Inputs are seeded and synthetic and
already in HBM when the timed region starts.

Also measured: the standalone matrix row at 4096 x 4096 for batches of 1,
8, 32 and 128 input vectors over a pool of distinct matrices larger than the
last-level cache, and (unless --no-cpu) the oracle on the host cores over a
bounded sample of the same workload.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode tokens/s at batch B, bit-exact; int8 row-kernel HBM GB/s vs peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_matrices(shape, generating=True):
    """(rows, cols) of every matrix one step multiplies."""
    d, f, kvd, v, L = shape.dim, shape.hidden, shape.kv_dim, shape.vocab, shape.layers
    mats = [(d, d), (kvd, d), (kvd, d), (d, d), (f, d), (f, d), (d, f)] * L
    if generating:
        mats.append((v, d))
    return mats


def rows_bytes(shape, batch, generating=True):
    """Algorithmic bytes of every row-kernel launch of one step: weight bytes,
    Q24 scales, i64 inputs and i64 outputs of each matrix."""
    total = 0
    for rows, cols in step_matrices(shape, generating):
        total += rows * cols + 4 * rows + 8 * batch * cols + 8 * batch * rows
    return total


def attention_bytes(shape, batch, npos):
    """Algorithmic bytes of one attention launch (one layer): every cached key
    and value word of the positions so far, the queries read and the outputs
    written."""
    return batch * (shape.kv_heads * npos * shape.head_size * 4 * 2 + shape.dim * 8 * 2)


def measured_traffic(kernel, workload, positions):
    """HBM bytes per launch of attention over `positions` (one launch per layer
    and step), from the committed rocprofv3 counter runs (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's readings): their ratio to the
    algorithmic bytes of the launches they counted, times the algorithmic
    bytes of these launches.  None when there are none for this workload or
    the kernel's source has changed since they were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}-7B-decode-b64.traffic.json")
    if workload != "7B-shaped-d4096-L32" or not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    src = open(os.path.join(ROOT, "fixed_point_int8_amd", "csrc", "fpi8_kernels.hip")).read()
    a = src.find("// Phase 9, one workgroup per (run, head)")
    b = src.find("// Phase 19 and the end of a position")
    if a < 0 or b < 0 or hashlib.sha256(src[a:b].encode()).hexdigest() != t["source_sha256"]:
        return None
    import workloads as Wl
    shape = Wl.by_name(workload).shape

    def mean_alg(pr):
        ps = range(pr[0], pr[1] + 1)
        return sum(attention_bytes(shape, 64, p + 1) for p in ps) / len(ps)

    ratio = t["traffic_bytes_per_launch"] / mean_alg(t["positions"])
    return int(ratio * mean_alg(positions))


STREAM_SRC = os.path.join(ROOT, "fixed_point_int8_amd", "csrc", "fpi8_rows_stream.hip")
MFMA_I8_PEAK_OPS = 5.0e15  # MI355X dense int8 matrix-core peak, ops/s


def mfma_ops(rows, cols, batch):
    """Int8 matrix-core operations the row kernels issue for one matrix: three
    digit passes of 16x16x64 MFMAs over 16-run tiles (a partial run tile is
    issued whole)."""
    return 2 * 3 * 16 * ((batch + 15) // 16) * rows * 64 * ((cols + 63) // 64)


def source_sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def pool_traffic(batch):
    """HBM bytes per launch of the pooled row kernel at this batch, from the
    committed rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE, scaled by a
    plain copy's readings), or None when there are none or the kernel source
    has changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "k_rows_stream-4096-pool.traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_sha(STREAM_SRC):
        return None
    b = t.get("batches", {}).get(str(batch))
    return None if b is None else b["traffic_bytes_per_launch"]


def row_sweep(torch, reps=5):
    """The standalone matrix row at 4096 columns over a pool of 48 distinct
    4096 x 4096 matrices (805 MB, over three times the 256 MB last-level
    cache), packed beforehand (fpi8_matrix_pack, outside the timed region:
    weights are prepared once and used many times).

    pool: the 48 matrices are one stacked matrix of 196,608 rows of 4096
      columns, and one call streams them all: a launch that splits the
      inputs into digits, then one launch of the persistent row kernel.  The
      row kernel's own duration comes from HIP events the library records
      around its launch on the call's stream (fpi8_matrix_rows_timing).
    per_matrix: one call per 4096 x 4096 matrix, 48 calls back to back
      (each a short launch, bound by its ramp rather than by bandwidth).
    valu_vs_mfma: the pooled call at 1, 2 and 4 inputs with the digits on
      the vector ALU (v_dot4) and on the matrix cores, kernel time of each."""
    from fixed_point_int8_amd import binding as B
    rows1 = cols = 4096
    pool = 48
    rows = rows1 * pool
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    n_p1 = B.fpi8_matrix_packed_size(rows1, cols)
    Pk = torch.empty((pool, n_p1), dtype=torch.uint8, device="cuda")
    for i in range(pool):
        Wi = torch.randint(0, 256, (rows1, cols), dtype=torch.uint8, device="cuda", generator=g)
        assert B.fpi8_matrix_pack(Wi, rows1, cols, Pk[i], n_p1) == 0
        del Wi
    S = torch.randint(1 << 14, (1 << 18) + 1, (pool, rows1), dtype=torch.int64, device="cuda",
                      generator=g).to(torch.int32)
    # 16-row tiles stack: the packed pool is the packed stacked matrix
    assert B.fpi8_matrix_packed_size(rows, cols) == pool * n_p1
    out = {}
    stream = torch.cuda.current_stream()
    for batch in (1, 8, 32, 128):
        x = (torch.randn((batch, cols), device="cuda", generator=g) * 2.0 * 65536).round().to(torch.int64)
        y = torch.zeros((batch, rows), dtype=torch.int64, device="cuda")
        n = B.fpi8_matrix_rows_workspace_size(rows, cols, batch)
        work = torch.zeros(n, dtype=torch.uint8, device="cuda")
        alg1 = rows1 * cols + 4 * rows1 + 8 * batch * cols + 8 * batch * rows1
        alg = rows * cols + 4 * rows + 8 * batch * cols + 8 * batch * rows
        ops = mfma_ops(rows, cols, batch)

        def pooled():
            return B.fpi8_matrix_rows_packed(Pk, S, rows, cols, x, batch, y, work, n, stream)

        assert pooled() == 0
        torch.cuda.synchronize()
        B.fpi8_matrix_rows_set_timing(True)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            pooled()
        t1.record(stream)
        torch.cuda.synchronize()
        call_ms = t0.elapsed_time(t1) / reps
        e, kern_ms, launches = B.fpi8_matrix_rows_timing()
        B.fpi8_matrix_rows_set_timing(False)
        assert e == 0 and launches == reps
        kern_ms /= launches

        yp = y[:, (pool - 1) * rows1:].clone()
        y1 = torch.zeros((batch, rows1), dtype=torch.int64, device="cuda")

        def single(i):
            return B.fpi8_matrix_rows_packed(Pk[i], S[i], rows1, cols, x, batch, y1, work, n, stream)

        for i in range(pool):
            assert single(i) == 0
        torch.cuda.synchronize()
        # the pooled call's last matrix equals the last single call's
        assert torch.equal(yp, y1), "pooled and single calls disagree"
        t0.record(stream)
        for _ in range(3):
            for i in range(pool):
                single(i)
        t1.record(stream)
        torch.cuda.synchronize()
        single_ms = t0.elapsed_time(t1) / (3 * pool)
        out[str(batch)] = {
            "pool": {"rows": rows, "kernel_us": round(kern_ms * 1e3, 2),
                     "GB/s": round(alg / kern_ms / 1e6, 1),
                     "frac": round(alg / kern_ms / 1e6 / HBM_PEAK_GBS, 4),
                     "weight_GB/s": round(rows * cols / kern_ms / 1e6, 1),
                     "call_us": round(call_ms * 1e3, 2),
                     "call_GB/s": round(alg / call_ms / 1e6, 1),
                     "mfma_util": round(ops / (kern_ms * 1e-3) / MFMA_I8_PEAK_OPS, 4),
                     "bytes_per_launch": alg, "traffic": pool_traffic(batch)},
            "per_matrix": {"us_per_call": round(single_ms * 1e3, 3),
                           "GB/s": round(alg1 / single_ms / 1e6, 1),
                           "frac": round(alg1 / single_ms / 1e6 / HBM_PEAK_GBS, 4)},
        }
        del x, y, y1, yp, work

    # The same pooled call on the vector ALU (v_dot4 over the same digits,
    # held in LDS) beside the matrix cores, at the batches the vector-ALU
    # kernel takes: the arithmetic closer to the HBM roof is the default.
    cmp = {}
    for batch in (1, 2, 4):
        x = (torch.randn((batch, cols), device="cuda", generator=g) * 2.0 * 65536).round().to(torch.int64)
        n = B.fpi8_matrix_rows_workspace_size(rows, cols, batch)
        work = torch.zeros(n, dtype=torch.uint8, device="cuda")
        alg = rows * cols + 4 * rows + 8 * batch * cols + 8 * batch * rows
        ys, row = [], {}
        for name, path in (("mfma", B.PATH_MFMA), ("valu", B.PATH_VALU)):
            y = torch.zeros((batch, rows), dtype=torch.int64, device="cuda")
            assert B.fpi8_matrix_rows_set_path(path) == 0
            assert B.fpi8_matrix_rows_packed(Pk, S, rows, cols, x, batch, y, work, n, stream) == 0
            torch.cuda.synchronize()
            B.fpi8_matrix_rows_set_timing(True)
            for _ in range(reps):
                B.fpi8_matrix_rows_packed(Pk, S, rows, cols, x, batch, y, work, n, stream)
            e, kern_ms, launches = B.fpi8_matrix_rows_timing()
            B.fpi8_matrix_rows_set_timing(False)
            assert e == 0 and launches == reps
            kern_ms /= launches
            row[name + "_us"] = round(kern_ms * 1e3, 2)
            row[name + "_frac"] = round(alg / kern_ms / 1e6 / HBM_PEAK_GBS, 4)
            ys.append(y)
        B.fpi8_matrix_rows_set_path(B.PATH_AUTO)
        assert torch.equal(ys[0], ys[1]), "vector-ALU and matrix-core rows disagree"
        cmp[str(batch)] = row
        del x, work, ys
    out["valu_vs_mfma"] = cmp
    del Pk, S
    torch.cuda.empty_cache()
    return out


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth of a plain device copy (bytes read plus bytes
    written per second), measured beside the nominal peak."""
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        b.copy_(a)
    t1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (t0.elapsed_time(t1) * 1e6)
    del a, b
    torch.cuda.empty_cache()
    return round(gbs, 1)


def cpu_baseline(blob, shape, name, seconds=12.0, max_positions=64):
    """The oracle on the host: one run of the same model from a one-id prompt,
    generating (classifier included) in turns of 4 positions until about
    `seconds` of wall time have passed, on as many threads as the host gives
    this job (at most 16)."""
    import oracle as O
    import workloads as Wl
    threads = min(16, os.cpu_count() or 1)
    O.set_threads(threads)
    ids = Wl.prompt_ids(shape.vocab, 1, 2003, 0)
    max_positions = min(max_positions, shape.context - 1)
    e, st = O.init_state(shape.as_tuple(), ids, max_positions, 0, 1)
    assert e == 0
    t0 = time.perf_counter()
    while True:
        assert O.turn(blob, st, 4) == 0
        info = O.state_info(st)[1]
        if info["complete"] or time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    gen = info["generated"]
    O.set_threads(1)
    return {"value": round(gen / dt, 4), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"one run of the {name} model, a 1-id prompt, {gen} generating positions "
                      f"(classifier included), {dt:.1f} s wall; runs are independent, so B runs take "
                      f"B times as long"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="decode steps timed (default: every decode position after the warm-up "
                         "and before the kernel-timed steps)")
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--kernel-steps", type=int, default=8,
                    help="extra steps after the timed ones, with per-launch kernel timing")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--workload", default="7B-shaped-d4096-L32")
    ap.add_argument("--only-sweep", action="store_true",
                    help="only the standalone 4096-column row sweep and the device copy (for "
                         "profiler runs of the row kernel); prints their JSON")
    ap.add_argument("--eager", action="store_true",
                    help="launch every kernel itself instead of replaying a recorded position "
                         "(for profilers that cannot follow graph launches)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the runs of a batch are "
              f"independent, and the library has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.only_sweep:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        print(json.dumps({"hbm_copy_GB/s": copy_bandwidth(torch, 1 << 28),
                          "row_sweep_4096": row_sweep(torch)}), flush=True)
        return
    import workloads as Wl
    from workloads import blob as Bl
    from fixed_point_int8_amd import binding as B
    from fixed_point_int8_amd.device import DeviceBatch, DeviceModel

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = Wl.by_name(args.workload)
    shape = w.shape
    if args.steps is None:
        args.steps = w.max_tokens - 1 - args.warmup - args.kernel_steps
    window = w.max_tokens - 1  # decode positions of the workload
    if args.warmup + args.steps + args.kernel_steps > window:
        # more than the window holds: keep the order (warm-up, timed, kernel-timed)
        # and time what is left, saying so
        args.warmup = min(args.warmup, window - 2)
        args.kernel_steps = max(1, min(args.kernel_steps, window - args.warmup - 1))
        asked = args.steps
        args.steps = window - args.warmup - args.kernel_steps
        log(f"{asked} timed steps do not fit the {window} decode positions with the warm-up and "
            f"kernel-timed steps; timing {args.steps}")
    if args.steps < 1 or args.warmup < 0:
        raise SystemExit("warmup + steps + kernel steps exceed the decode positions of the workload")

    t = time.perf_counter()
    blob = Bl.build_blob(shape, w.blob_seed)
    log(f"artifact {blob.size / 1e9:.3f} GB in {time.perf_counter() - t:.1f} s")
    model = DeviceModel(blob, max_runs=w.runs)
    if args.eager:
        B.fpi8_engine_set_graph(model.engine, False)
    runs = [(Wl.prompt_ids(shape.vocab, w.prompt, w.ids_seed, r), w.max_tokens, w.temperature_q16,
             w.run_seed + r) for r in range(w.runs)]
    t = time.perf_counter()
    batch = DeviceBatch(shape.as_tuple(), runs)
    log(f"{w.runs} states of {batch.sizes[0] / 1e6:.1f} MB in {time.perf_counter() - t:.1f} s")
    stream = torch.cuda.current_stream()

    # Prefill: positions 0 .. prompt-1 (the last one generates the first token).
    torch.cuda.synchronize()
    t = time.perf_counter()
    e, errs = batch.turn(model, w.prompt, stream)
    torch.cuda.synchronize()
    prefill_s = time.perf_counter() - t
    assert e == 0, (e, list(errs))
    log(f"prefill {w.prompt} positions x {w.runs} runs in {prefill_s:.2f} s")

    gen_prefill = sum(batch.info(i)["generated"] for i in range(w.runs))
    # By default the timed steps are the whole decode window (positions
    # prompt .. prompt + max_tokens - 2) less the warm-up steps before them
    # and the kernel-timed steps after them.  A shorter run of steps sits
    # around the window's middle, where a step reads its mean cache length;
    # the steps before them are untimed (warm-up included).
    first_dec, last_dec = w.prompt, w.prompt + w.max_tokens - 2
    mid = (first_dec + last_dec) // 2
    start = max(first_dec + args.warmup, mid - args.steps // 2)
    start = min(start, last_dec + 1 - args.steps - args.kernel_steps)
    t = time.perf_counter()
    e, errs = batch.turn(model, start - first_dec, stream)
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - t
    assert e == 0, (e, list(errs))
    gen0 = sum(batch.info(i)["generated"] for i in range(w.runs))
    pos0 = batch.info(0)["position"]
    assert pos0 == start, (pos0, start)

    # The timed steps: nothing but the launches of the path.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e, errs = batch.turn(model, args.steps, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    assert e == 0, (e, list(errs))
    gen1 = sum(batch.info(i)["generated"] for i in range(w.runs))
    tokens = gen1 - gen0

    # Kernel times: a few more steps with every row-kernel and attention
    # launch bracketed by HIP events on its stream.
    pos1 = batch.info(0)["position"]
    ks = args.kernel_steps
    # One stream here, so that no other kernel runs beside the one timed.
    B.fpi8_engine_set_streams(model.engine, 1)
    for k in (B.T_ROWS, B.T_ATTN, B.T_NORM):
        B.fpi8_engine_set_timing(model.engine, k, True)
    torch.cuda.synchronize()
    tk = time.perf_counter()
    e, errs = batch.turn(model, ks, stream)
    torch.cuda.synchronize()
    dk = time.perf_counter() - tk
    assert e == 0, (e, list(errs))
    _, rows_ms, rows_n = B.fpi8_engine_timing(model.engine, B.T_ROWS)
    _, attn_ms, attn_n = B.fpi8_engine_timing(model.engine, B.T_ATTN)
    _, norm_ms, norm_n = B.fpi8_engine_timing(model.engine, B.T_NORM)
    for k in (B.T_ROWS, B.T_ATTN, B.T_NORM):
        B.fpi8_engine_set_timing(model.engine, k, False)

    # Algorithmic bytes over the kernel-timed steps (positions pos1 .. pos1+ks-1).
    rows_alg = rows_bytes(shape, w.runs) * ks
    rows_ops = sum(mfma_ops(r, c, w.runs) for r, c in step_matrices(shape)) * ks
    attn_alg = sum(attention_bytes(shape, w.runs, pos1 + k + 1) * shape.layers for k in range(ks))
    kern = {
        "steps": ks, "positions": [pos1, pos1 + ks - 1],
        "rows": {"launches": rows_n, "avg_us": round(rows_ms * 1e3 / max(rows_n, 1), 2),
                 "GB/s": round(rows_alg / (rows_ms * 1e6), 1),
                 "frac": round(rows_alg / (rows_ms * 1e6) / HBM_PEAK_GBS, 4),
                 "mfma_util": round(rows_ops / (rows_ms * 1e-3) / MFMA_I8_PEAK_OPS, 4),
                 "bytes_per_launch": int(rows_alg / max(rows_n, 1))},
        "attention": {"launches": attn_n, "avg_us": round(attn_ms * 1e3 / max(attn_n, 1), 2),
                      "GB/s": round(attn_alg / (attn_ms * 1e6), 1),
                      "frac": round(attn_alg / (attn_ms * 1e6) / HBM_PEAK_GBS, 4),
                      "bytes_per_launch": int(attn_alg / max(attn_n, 1))},
        "norm": {"launches": norm_n, "avg_us": round(norm_ms * 1e3 / max(norm_n, 1), 2)},
        "share_of_step": {"rows": round(rows_ms / (dk * 1e3), 3),
                          "attention": round(attn_ms / (dk * 1e3), 3),
                          "norm": round(norm_ms / (dk * 1e3), 3)},
    }
    roofline_attention = {"kernel": "k_attention", "bound": "hbm",
                          "achieved": kern["attention"]["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                          "frac": kern["attention"]["frac"],
                          "traffic": measured_traffic("k_attention", w.name, [pos1, pos1 + ks - 1])}

    model.close()
    del batch, model
    torch.cuda.empty_cache()
    copy_gbs = copy_bandwidth(torch)
    sweep = None if args.no_sweep else row_sweep(torch)
    cpu = None if args.no_cpu else cpu_baseline(blob, shape, w.name)

    # The int8 row kernel's roofline: one launch over the pooled 4096-column
    # sweep, at the HBM-bound batch (1, 8 or 32) where it is furthest from
    # peak.  (At 128 inputs the three digit passes make it matrix-core bound;
    # that batch reports its int8 MFMA utilization in the sweep.)
    roofline = None
    if sweep:
        bsel = min(("1", "8", "32"), key=lambda b: sweep[b]["pool"]["frac"])
        pl = sweep[bsel]["pool"]
        roofline = {"kernel": "k_rows_stream_shared",
                    "bound": "hbm", "achieved": pl["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": pl["frac"], "traffic": pl["traffic"],
                    "workload": f"4096-column rows, 48 stacked 4096x4096 matrices, batch {bsel}",
                    "bytes_per_launch": pl["bytes_per_launch"]}

    res = {
        "metric": METRIC, "value": round(tokens / dt, 2), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3 / args.steps, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int64",
        "data": "synthetic",
        "config": {"workload": f"{w.name} decode", "global_batch": w.runs,
                   "prompt": w.prompt, "decode_positions": [pos0, pos0 + args.steps - 1],
                   "decode_window": [first_dec, last_dec],
                   "seq_len": w.prompt + w.max_tokens - 1, "parallelism": "none (one GPU)"},
        "roofline": roofline, "roofline_attention": roofline_attention,
        "cpu_baseline": cpu, "kernels": kern,
        "prefill_s": round(prefill_s, 2),
        # every token the runs hold over prefill, the untimed and the timed steps, over their wall time
        "prefill_and_decode_tokens_per_s": round(gen1 / (prefill_s + warm_s + dt), 2),
        "first_tokens": gen_prefill,
        "hbm_copy_GB/s": copy_gbs, "row_sweep_4096": sweep,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
