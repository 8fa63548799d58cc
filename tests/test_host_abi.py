"""The C ABI of libfpi8 on the CPU: the library loads, exports what
include/fpi8.h declares, and its host functions (state size, state init,
state info, artifact checks) agree with the oracle.  No GPU call is made."""
import re
import os

import numpy as np
import pytest

import oracle as O
import workloads as W
from workloads import blob as Bl
from workloads.configs import Shape
from fixed_point_int8_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "fpi8.h")).read()
    declared = set(re.findall(r"\b(fpi8_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(B.EXPORTS)
    L = B.lib()
    for name in declared:
        assert getattr(L, name) is not None


def test_library_has_gfx950_code():
    data = open(B.LIB_PATH, "rb").read()
    assert b"gfx950" in data


CFGS = [W.TINY.shape.as_tuple(), W.M1B.shape.as_tuple(), W.M7B.shape.as_tuple(),
        W.LONG8K.shape.as_tuple(), (288, 768, 6, 6, 6, 32000, 256), (64, 172, 5, 8, 4, 512, 512)]


@pytest.mark.parametrize("cfg", CFGS)
def test_state_size_matches_oracle(cfg):
    for n_ids, mx in [(1, 1), (3, 5), (16, 16), (cfg[6], 1), (1, cfg[6]), (cfg[6], 2), (0, 3),
                      (2, 0), (5, cfg[6] + 1)]:
        assert B.fpi8_state_size(cfg, n_ids, mx) == O.state_size(cfg, n_ids, mx), (n_ids, mx)
    bad = list(cfg)
    bad[0] += 1
    assert B.fpi8_state_size(bad, 2, 2) == O.state_size(bad, 2, 2) == B.UINT64_MAX


def test_state_offsets_match_oracle():
    for cfg in CFGS:
        a = B.fpi8_state_offsets(cfg, 7, 9)
        b = O.state_layout(cfg, 7, 9)
        for k in B.OFFSET_NAMES:
            assert a[k] == b[k], k


def aligned(n):
    return O.aligned_zeros(n)


def test_init_state_matches_oracle_byte_for_byte():
    rng = np.random.default_rng(1)
    cfg = W.SMALL_SHAPES["gqa"].as_tuple()
    for trial in range(30):
        n = int(rng.integers(1, 20))
        mx = int(rng.integers(1, 21))
        ids = rng.integers(0, cfg[5], n).astype(np.uint32)
        t = int(rng.choice([0, 1, 65536, 16 << 16]))
        seed = int(rng.choice([0, 1, 2**64 - 1, int(rng.integers(0, 2**63))]))
        eo, so = O.init_state(cfg, ids, mx, t, seed)
        size = B.fpi8_state_size(cfg, n, mx)
        if size == B.UINT64_MAX:
            sp = aligned(8)
            assert B.fpi8_init_state(cfg, sp, ids, mx, t, seed) == eo != 0
            continue
        sp = aligned(size)
        ep = B.fpi8_init_state(cfg, sp, ids, mx, t, seed)
        assert ep == eo
        if ep == 0:
            assert np.array_equal(sp, so)
            assert B.fpi8_state_info(sp)[1] == {k: v for k, v in O.state_info(so)[1].items()}


def test_init_state_errors_match_oracle():
    cfg = W.TINY.shape.as_tuple()
    cases = [([5] * 4, 0, 0), ([5] * 4, 33, 0), ([], 4, 0), ([512], 4, 0), ([5], 4, (16 << 16) + 1),
             ([5] * 16, 17, 0), ([5] * 16, 18, 0), ([5] * 32, 1, 0), ([5] * 33, 1, 0)]
    for ids, mx, t in cases:
        eo, _ = O.init_state(cfg, ids, mx, t, 0)
        size = B.fpi8_state_size(cfg, len(ids), mx)
        buf = aligned(8 if size == B.UINT64_MAX else size)
        assert B.fpi8_init_state(cfg, buf, ids, mx, t, 0) == eo, (len(ids), mx, t)
    size = B.fpi8_state_size(cfg, 3, 4)
    assert B.fpi8_init_state(cfg, aligned(size + 8), [5] * 3, 4) == 4
    assert B.fpi8_init_state(cfg, aligned(size + 8)[1:size + 1], [5] * 3, 4) == 3
    assert B.fpi8_init_state((0,) + cfg[1:], aligned(size), [5] * 3, 4) == 1


def test_blob_check_matches_oracle():
    shape = W.SMALL_SHAPES["ragged"]
    bl = Bl.build_blob(shape, 3)
    lay = Bl.plan(shape)
    variants = [bl]
    bad = bl.copy(); bad[0] ^= 1; variants.append(bad)
    bad = bl.copy(); bad[8:12] = np.frombuffer(np.uint32(161).tobytes(), np.uint8); variants.append(bad)
    bad = bl.copy(); bad[lay.offsets["exp"]:lay.offsets["exp"] + 4] = 0; variants.append(bad)
    variants.append(bl[: lay.sections[-1][0] + 10].copy())
    variants.append(bl[: lay.section0_len].copy())
    bad = bl.copy(); bad[40] += 1; variants.append(bad)
    d0 = lay.offsets["desc"]
    for field in range(0, 32, 4):
        bad = bl.copy(); bad[d0 + 32 * 4 + field] ^= 0x10; variants.append(bad)
    for sec in (1, 5, 9):
        bad = bl.copy()
        o = Bl.SECTION_TABLE + 16 * sec + 8
        bad[o:o + 8] = np.frombuffer(np.uint64(64).tobytes(), np.uint8)
        variants.append(bad)
    for off in range(48, 112, 8):
        bad = bl.copy(); bad[off] ^= 4; variants.append(bad)
    for i, v in enumerate(variants):
        assert B.fpi8_blob_check(v) == O.blob_check(v), i


def test_output_tokens_of_a_fresh_state():
    cfg = W.TINY.shape.as_tuple()
    size = B.fpi8_state_size(cfg, 4, 6)
    st = aligned(size)
    assert B.fpi8_init_state(cfg, st, [3, 4, 5, 6], 6, 0, 9) == 0
    assert B.fpi8_output_tokens(st).size == 0
    o = B.fpi8_state_offsets(cfg, 4, 6)
    st[o["out"]: o["out"] + 8] = np.frombuffer(np.array([11, 12], np.uint32).tobytes(), np.uint8)
    st[44:48] = np.frombuffer(np.uint32(2).tobytes(), np.uint8)
    assert list(B.fpi8_output_tokens(st)) == [11, 12]


def test_oracle_turn_after_library_init():
    # A state written by the library's init is one the oracle runs.
    shape = W.SMALL_SHAPES["gqa"]
    cfg = shape.as_tuple()
    bl = Bl.build_blob(shape, 4)
    st = aligned(B.fpi8_state_size(cfg, 5, 3))
    assert B.fpi8_init_state(cfg, st, [3, 4, 5, 6, 7], 3, 0, 0) == 0
    assert O.run_to_end(bl, st) == 0
    assert B.fpi8_state_info(st)[1]["complete"] == 1


def test_matrix_rows_rejects_bad_arguments_before_any_launch():
    # Sizes, null pointers and alignments are checked on the host before the
    # call touches the GPU (the pointers here are never dereferenced).
    need = B.fpi8_matrix_rows_workspace_size(16, 64, 2)
    ok = dict(d_W=0x10000, d_scale=0x20000, rows=16, cols=64, d_x=0x30000, batch=2, d_y=0x40000,
              d_work=0x50000, work_len=need)
    bad = [dict(rows=0), dict(cols=0), dict(batch=0), dict(cols=65537), dict(d_W=0), dict(d_x=0),
           dict(d_y=0), dict(d_work=0), dict(work_len=need - 1), dict(d_work=0x50010),
           dict(d_x=0x30004), dict(d_y=0x40002)]
    for change in bad:
        args = dict(ok, **change)
        assert B.fpi8_matrix_rows(**args) == B.ERR_ARGUMENT, change
        pk = dict(args, d_P=args.pop("d_W"))
        assert B.fpi8_matrix_rows_packed(**pk) == B.ERR_ARGUMENT, change
    # a packed copy must be 16-byte aligned
    pk = dict(ok, d_P=0x10008)
    del pk["d_W"]
    assert B.fpi8_matrix_rows_packed(**pk) == B.ERR_ARGUMENT
