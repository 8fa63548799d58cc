"""The oracle: a plain, slow CPU implementation of the fixed-point forward
pass of the curta-core inference core ("The inference core" page), in C.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The GPU library does
not use it, and it does not use the GPU library.

Functions:
  isqrt, row, rows, rmsnorm, rotate, exp_index, silu, attention_head,
  xorshift64s, sample                    -- the primitives, one by one
  blob_check, state_size, pages_state_size, init_state, state_info,
  state_layout, turn                     -- the artifact, the state, a turn

Parity unpinned (stated in the C file too): the pairing of rotary elements
(adjacent pairs inside each head) and the reading of "divides by the
temperature" have no value on the pages to check them against.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfpi8_ref.so")
_SRC = os.path.join(_HERE, "fpi8_ref.c")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, OpenMP over matrix rows)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fopenmp", "-shared", "-fPIC",
               _SRC, "-o", _LIB_PATH + ".tmp"]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class Info(C.Structure):
    _fields_ = [(n, C.c_uint32) for n in
                ("phase", "layer", "position", "token", "n_ids", "max_tokens",
                 "temperature_q16", "generated", "cache_positions", "error", "complete",
                 "reserved")] + [("generator", C.c_uint64), ("turns", C.c_uint64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}


class Layout(C.Structure):
    _fields_ = [(n, C.c_uint64) for n in
                ("ids", "out", "x", "w1", "w2", "w3", "gate", "up", "logits", "scores",
                 "keys", "values", "total")] + [("cache_positions", C.c_uint32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None
_P = C.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = C.CDLL(_LIB_PATH)
        sig = {
            "fpi8_ref_isqrt": (C.c_uint64, [C.c_uint64]),
            "fpi8_ref_row": (C.c_int64, [_P, C.c_uint32, _P, C.c_uint32]),
            "fpi8_ref_rows": (None, [_P, _P, C.c_uint32, C.c_uint32, _P, C.c_uint32, _P]),
            "fpi8_ref_rmsnorm": (None, [_P, _P, C.c_uint32, _P]),
            "fpi8_ref_rotate": (None, [_P, _P, C.c_int32, C.c_int32]),
            "fpi8_ref_exp_index": (C.c_uint32, [C.c_uint64]),
            "fpi8_ref_silu": (C.c_int64, [C.c_int64, _P]),
            "fpi8_ref_attention_head": (None, [_P, _P, _P, C.c_uint32, C.c_uint32, C.c_uint64,
                                               C.c_uint32, _P, _P, _P, _P, _P]),
            "fpi8_ref_xorshift64s": (C.c_uint64, [_P]),
            "fpi8_ref_sample": (C.c_uint32, [_P, C.c_uint32, C.c_uint32, _P, _P]),
            "fpi8_ref_blob_check": (C.c_int32, [_P, C.c_uint64, _P]),
            "fpi8_ref_state_size": (C.c_uint64, [_P, C.c_uint32, C.c_uint32]),
            "fpi8_ref_pages_state_size": (C.c_uint64, [_P, C.c_uint32, C.c_uint32]),
            "fpi8_ref_init_state": (C.c_int32, [_P, _P, C.c_uint64, _P, C.c_uint32, C.c_uint32,
                                                C.c_uint32, C.c_uint64]),
            "fpi8_ref_state_info": (C.c_int32, [_P, C.c_uint64, C.POINTER(Info)]),
            "fpi8_ref_state_layout": (C.c_int32, [_P, C.c_uint32, C.c_uint32, C.POINTER(Layout)]),
            "fpi8_ref_turn": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.c_uint32]),
            "fpi8_ref_turn_phases": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.c_uint32]),
            "fpi8_ref_turn_units": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.c_uint64]),
            "fpi8_ref_set_threads": (C.c_int32, [C.c_int32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _cfg(cfg) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cfg, dtype=np.uint32).reshape(7))


# ---- primitives --------------------------------------------------------------

def set_threads(n: int) -> int:
    return lib().fpi8_ref_set_threads(int(n))


def isqrt(n: int) -> int:
    return lib().fpi8_ref_isqrt(C.c_uint64(n))


def row(w: np.ndarray, scale: int, x: np.ndarray) -> int:
    w = np.ascontiguousarray(w, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.int64)
    assert w.size == x.size
    return lib().fpi8_ref_row(_ptr(w), scale, _ptr(x), w.size)


def rows(W: np.ndarray, s: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y[b, r] for W [rows, cols] uint8, s [rows] uint32, x [batch, cols] int64."""
    W = np.ascontiguousarray(W, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint32)
    x = np.ascontiguousarray(np.atleast_2d(x), dtype=np.int64)
    R, K = W.shape
    assert x.shape[1] == K and s.size == R
    y = np.zeros((x.shape[0], R), dtype=np.int64)
    lib().fpi8_ref_rows(_ptr(W), _ptr(s), R, K, _ptr(x), x.shape[0], _ptr(y))
    return y


def rmsnorm(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.int64)
    w = np.ascontiguousarray(w, dtype=np.int32)
    y = np.zeros_like(x)
    lib().fpi8_ref_rmsnorm(_ptr(x), _ptr(w), x.size, _ptr(y))
    return y


def rotate(a: int, b: int, c: int, s: int):
    A = np.array([a], dtype=np.int64)
    B = np.array([b], dtype=np.int64)
    lib().fpi8_ref_rotate(_ptr(A), _ptr(B), c, s)
    return int(A[0]), int(B[0])


def exp_index(d: int) -> int:
    return lib().fpi8_ref_exp_index(C.c_uint64(d & (2**64 - 1)))


def silu(x: int, tab: np.ndarray) -> int:
    tab = np.ascontiguousarray(tab, dtype=np.int32)
    return lib().fpi8_ref_silu(x, _ptr(tab))


def attention_head(q, K, V, inv, exp_tab):
    """One head: q [head] int64, K and V [npos, head] int32.  Returns
    (out [head], probabilities [npos], max score, sum of exponentials)."""
    q = np.ascontiguousarray(q, dtype=np.int64)
    K = np.ascontiguousarray(K, dtype=np.int32)
    V = np.ascontiguousarray(V, dtype=np.int32)
    exp_tab = np.ascontiguousarray(exp_tab, dtype=np.uint32)
    npos, head = K.shape
    scores = np.zeros(npos, dtype=np.int64)
    out = np.zeros(head, dtype=np.int64)
    m = np.zeros(1, dtype=np.int64)
    ssum = np.zeros(1, dtype=np.uint64)
    lib().fpi8_ref_attention_head(_ptr(q), _ptr(K), _ptr(V), npos, head, head, inv,
                                  _ptr(exp_tab), _ptr(scores), _ptr(out), _ptr(m), _ptr(ssum))
    return out, scores, int(m[0]), int(ssum[0])


def xorshift64s(state: int):
    st = np.array([state], dtype=np.uint64)
    out = lib().fpi8_ref_xorshift64s(_ptr(st))
    return int(st[0]), out


def sample(logits, temperature_q16, exp_tab, generator):
    logits = np.ascontiguousarray(logits, dtype=np.int64)
    exp_tab = np.ascontiguousarray(exp_tab, dtype=np.uint32)
    g = np.array([generator], dtype=np.uint64)
    tok = lib().fpi8_ref_sample(_ptr(logits), logits.size, temperature_q16, _ptr(exp_tab), _ptr(g))
    return tok, int(g[0])


# ---- artifact and state ---------------------------------------------------------

def blob_check(blob: np.ndarray):
    cfg = np.zeros(7, dtype=np.uint32)
    e = lib().fpi8_ref_blob_check(_ptr(blob), blob.size, _ptr(cfg))
    return e, tuple(int(v) for v in cfg)


def state_size(cfg, n_ids, max_tokens) -> int:
    return lib().fpi8_ref_state_size(_ptr(_cfg(cfg)), n_ids, max_tokens)


def pages_state_size(cfg, prompt_bytes, max_tokens) -> int:
    return lib().fpi8_ref_pages_state_size(_ptr(_cfg(cfg)), prompt_bytes, max_tokens)


def state_layout(cfg, n_ids, max_tokens) -> dict:
    L = Layout()
    e = lib().fpi8_ref_state_layout(_ptr(_cfg(cfg)), n_ids, max_tokens, C.byref(L))
    if e:
        raise ValueError(f"state_layout error {e}")
    return L.as_dict()


def aligned_zeros(n: int) -> np.ndarray:
    """A uint8 buffer of n bytes whose start is 64-byte aligned."""
    raw = np.zeros(n + 64, dtype=np.uint8)
    off = (-raw.ctypes.data) % 64
    return raw[off:off + n]


def init_state(cfg, ids, max_tokens, temperature_q16=0, seed=0, state=None):
    """Returns (error, state array)."""
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    n = state_size(cfg, ids.size, max_tokens)
    if state is None:
        state = aligned_zeros(0 if n == 2**64 - 1 else n)
    e = lib().fpi8_ref_init_state(_ptr(_cfg(cfg)), _ptr(state), state.size, _ptr(ids), ids.size,
                                  max_tokens, temperature_q16, C.c_uint64(seed))
    return e, state


def state_info(state: np.ndarray):
    I = Info()
    e = lib().fpi8_ref_state_info(_ptr(state), state.size, C.byref(I))
    return e, I.as_dict()


def turn(blob: np.ndarray, state: np.ndarray, max_positions: int) -> int:
    return lib().fpi8_ref_turn(_ptr(blob), blob.size, _ptr(state), state.size, max_positions)


def turn_phases(blob: np.ndarray, state: np.ndarray, max_phases: int) -> int:
    """Runs up to max_phases single phases from the state's cursor."""
    return lib().fpi8_ref_turn_phases(_ptr(blob), blob.size, _ptr(state), state.size, max_phases)


def turn_units(blob: np.ndarray, state: np.ndarray, max_units: int) -> int:
    """Runs up to max_units units of work from the state's cursor."""
    return lib().fpi8_ref_turn_units(_ptr(blob), blob.size, _ptr(state), state.size, max_units)


def run_to_end(blob, state, chunk=1 << 30):
    """Turns until the run is complete or fails; returns the last error."""
    while True:
        e = turn(blob, state, chunk)
        if e:
            return e
        if state_info(state)[1]["complete"]:
            return 0
