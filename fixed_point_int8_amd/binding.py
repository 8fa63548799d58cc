"""Python binding of libfpi8 (include/fpi8.h): the same names, argument
marshalling only.  Every step of the forward pass runs in the library's HIP
kernels; this module converts numpy arrays, torch tensors and integers to
pointers and back.

Loading fails loudly when libfpi8.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfpi8.so")

# Core error numbers ("Core errors") and the library's own.
OK, INVALID_CONFIG, INVALID_FORMAT, INVALID_STATE, BUFFER_TOO_SMALL = 0, 1, 2, 3, 4
MISSING_WEIGHTS, INVALID_PROMPT, CONTEXT_EXCEEDED, ARITHMETIC = 5, 6, 7, 8
ERR_HIP, ERR_UNSUPPORTED, ERR_ARGUMENT = 100, 101, 102

# Kernel classes of fpi8_engine_set_timing.
T_ROWS, T_ATTN, T_NORM, T_SAMPLE, T_EMBED = range(5)

UINT64_MAX = (1 << 64) - 1

# Symbols include/fpi8.h declares.
EXPORTS = ("fpi8_blob_check", "fpi8_state_size", "fpi8_state_offsets", "fpi8_init_state",
           "fpi8_state_info", "fpi8_output_tokens", "fpi8_engine_create",
           "fpi8_engine_destroy", "fpi8_turn", "fpi8_turn_phases", "fpi8_turn_units",
           "fpi8_engine_set_row_kernel", "fpi8_engine_set_graph", "fpi8_tokenize",
           "fpi8_token_text", "fpi8_output_text", "fpi8_pages_state_size", "fpi8_state_export",
           "fpi8_state_import", "fpi8_pages_init", "fpi8_pages_tokenize", "fpi8_position_charges",
           "fpi8_engine_set_streams",
           "fpi8_engine_set_timing",
           "fpi8_engine_timing",
           "fpi8_matrix_rows_workspace_size", "fpi8_matrix_rows", "fpi8_matrix_packed_size",
           "fpi8_matrix_pack", "fpi8_matrix_rows_packed", "fpi8_matrix_rows_set_timing",
           "fpi8_matrix_rows_timing", "fpi8_matrix_rows_packed_noalloc", "fpi8_plan_turn",
           "fpi8_quote_turns", "fpi8_turn_bind", "fpi8_turn_async", "fpi8_matrix_rows_set_path")


class fpi8_info(C.Structure):
    _fields_ = [(n, C.c_uint32) for n in
                ("phase", "layer", "position", "token", "n_ids", "max_tokens",
                 "temperature_q16", "generated", "cache_positions", "error", "complete",
                 "reserved")] + [("generator", C.c_uint64), ("turns", C.c_uint64)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}


class fpi8_turn_plan(C.Structure):
    _fields_ = [("sections", C.c_uint32 * 2), ("section_count", C.c_uint32),
                ("estimated_cu", C.c_uint32), ("max_generated", C.c_uint32),
                ("ends_with_draw", C.c_uint32), ("units", C.c_uint64)]


_P = C.c_void_p
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        sig = {
            "fpi8_blob_check": (C.c_int32, [_P, C.c_uint64, _P]),
            "fpi8_state_size": (C.c_uint64, [_P, C.c_uint32, C.c_uint32]),
            "fpi8_state_offsets": (C.c_int32, [_P, C.c_uint32, C.c_uint32, _P]),
            "fpi8_init_state": (C.c_int32, [_P, _P, C.c_uint64, _P, C.c_uint32, C.c_uint32,
                                            C.c_uint32, C.c_uint64]),
            "fpi8_state_info": (C.c_int32, [_P, C.c_uint64, C.POINTER(fpi8_info)]),
            "fpi8_output_tokens": (_P, [_P, C.c_uint64, C.POINTER(C.c_uint32)]),
            "fpi8_engine_create": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.c_uint32,
                                               C.POINTER(_P)]),
            "fpi8_engine_destroy": (None, [_P]),
            "fpi8_turn": (C.c_int32, [_P, _P, C.c_uint64, C.c_uint32, C.c_uint32, _P, _P]),
            "fpi8_turn_phases": (C.c_int32, [_P, _P, C.c_uint64, C.c_uint32, C.c_uint32, _P, _P]),
            "fpi8_turn_units": (C.c_int32, [_P, _P, C.c_uint64, C.c_uint32, C.c_uint64, _P, _P]),
            "fpi8_tokenize": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint32, C.c_uint32, _P,
                                          C.c_uint32, C.POINTER(C.c_uint32)]),
            "fpi8_token_text": (C.c_int32, [_P, C.c_uint64, C.c_uint32, C.c_uint32, _P,
                                            C.c_uint32, C.POINTER(C.c_uint32)]),
            "fpi8_output_text": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, _P, C.c_uint64,
                                             C.POINTER(C.c_uint64)]),
            "fpi8_pages_state_size": (C.c_uint64, [_P, C.c_uint32, C.c_uint32]),
            "fpi8_state_export": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, _P, C.c_uint32, _P,
                                              C.c_uint64]),
            "fpi8_state_import": (C.c_int32, [_P, _P, C.c_uint64, _P, C.c_uint64]),
            "fpi8_pages_init": (C.c_int32, [_P, _P, C.c_uint32, C.c_uint32, C.c_uint32,
                                            C.c_uint64, _P, C.c_uint64]),
            "fpi8_pages_tokenize": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.c_uint64, _P]),
            "fpi8_position_charges": (C.c_int32, [_P, C.c_uint32, C.c_int32, C.c_uint32, _P]),
            "fpi8_engine_set_row_kernel": (C.c_int32, [_P, C.c_int32]),
            "fpi8_engine_set_streams": (C.c_int32, [_P, C.c_int32]),
            "fpi8_engine_set_graph": (C.c_int32, [_P, C.c_int32]),
            "fpi8_engine_set_timing": (C.c_int32, [_P, C.c_int32, C.c_int32]),
            "fpi8_engine_timing": (C.c_int32, [_P, C.c_int32, C.POINTER(C.c_double),
                                               C.POINTER(C.c_uint64)]),
            "fpi8_matrix_rows_workspace_size": (C.c_uint64, [C.c_uint32, C.c_uint32, C.c_uint32]),
            "fpi8_matrix_rows": (C.c_int32, [_P, _P, C.c_uint32, C.c_uint32, _P, C.c_uint32, _P,
                                             _P, C.c_uint64, _P]),
            "fpi8_matrix_packed_size": (C.c_uint64, [C.c_uint32, C.c_uint32]),
            "fpi8_matrix_pack": (C.c_int32, [_P, C.c_uint32, C.c_uint32, _P, C.c_uint64, _P]),
            "fpi8_matrix_rows_packed": (C.c_int32, [_P, _P, C.c_uint32, C.c_uint32, _P, C.c_uint32,
                                                    _P, _P, C.c_uint64, _P]),
            "fpi8_matrix_rows_set_timing": (C.c_int32, [C.c_int32]),
            "fpi8_matrix_rows_set_path": (C.c_int32, [C.c_int32]),
            "fpi8_turn_bind": (C.c_int32, [_P, _P, C.c_uint64, C.c_uint32, _P, _P]),
            "fpi8_turn_async": (C.c_int32, [_P, C.c_uint32, _P, _P]),
            "fpi8_plan_turn": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.POINTER(fpi8_turn_plan)]),
            "fpi8_quote_turns": (C.c_int32, [_P, C.c_uint64, _P, C.c_uint64, C.POINTER(C.c_uint64)]),
            "fpi8_matrix_rows_packed_noalloc": (C.c_int32, [_P, _P, C.c_uint32, C.c_uint32, _P,
                                                            C.c_uint32, _P, _P]),
            "fpi8_matrix_rows_timing": (C.c_int32, [C.POINTER(C.c_double), C.POINTER(C.c_uint64)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(_P)


def _cfg(cfg) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(cfg, dtype=np.uint32).reshape(7))


def _dev_ptr(t) -> int:
    """Device address of a torch tensor or a plain integer address."""
    return t if isinstance(t, int) else int(t.data_ptr())


def _stream_ptr(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


# ---- host functions ------------------------------------------------------------

def fpi8_blob_check(blob: np.ndarray):
    cfg = np.zeros(7, dtype=np.uint32)
    e = lib().fpi8_blob_check(_np_ptr(blob), blob.size, _np_ptr(cfg))
    return e, tuple(int(v) for v in cfg)


def fpi8_state_size(cfg, n_ids: int, max_tokens: int) -> int:
    return lib().fpi8_state_size(_np_ptr(_cfg(cfg)), n_ids, max_tokens)


OFFSET_NAMES = ("ids", "out", "x", "w1", "w2", "w3", "gate", "up", "logits", "scores", "keys",
                "values", "total")


def fpi8_state_offsets(cfg, n_ids: int, max_tokens: int) -> dict:
    out = np.zeros(13, dtype=np.uint64)
    e = lib().fpi8_state_offsets(_np_ptr(_cfg(cfg)), n_ids, max_tokens, _np_ptr(out))
    if e:
        raise ValueError(f"fpi8_state_offsets: error {e}")
    return dict(zip(OFFSET_NAMES, (int(v) for v in out)))


def fpi8_init_state(cfg, state: np.ndarray, ids, max_tokens: int, temperature_q16: int = 0,
                    seed: int = 0) -> int:
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    return lib().fpi8_init_state(_np_ptr(_cfg(cfg)), _np_ptr(state), state.size, _np_ptr(ids),
                                 ids.size, max_tokens, temperature_q16, C.c_uint64(seed))


def fpi8_state_info(state: np.ndarray):
    info = fpi8_info()
    e = lib().fpi8_state_info(_np_ptr(state), state.size, C.byref(info))
    return e, info.as_dict()


def fpi8_output_tokens(state: np.ndarray) -> np.ndarray:
    n = C.c_uint32(0)
    p = lib().fpi8_output_tokens(_np_ptr(state), state.size, C.byref(n))
    if not p:
        raise ValueError("fpi8_output_tokens: invalid state")
    off = p - state.ctypes.data
    return state[off: off + 4 * n.value].view(np.uint32).copy()


# ---- the GPU engine ---------------------------------------------------------------

def fpi8_engine_create(section0: np.ndarray, d_blob, blob_len: int, max_runs: int):
    h = _P()
    e = lib().fpi8_engine_create(_np_ptr(section0), section0.size, _dev_ptr(d_blob), blob_len,
                                 max_runs, C.byref(h))
    return e, h


def fpi8_engine_destroy(engine) -> None:
    lib().fpi8_engine_destroy(engine)


def fpi8_turn(engine, d_states, state_stride: int, n_runs: int, max_positions: int,
              stream=None):
    errs = np.zeros(n_runs, dtype=np.int32)
    e = lib().fpi8_turn(engine, _dev_ptr(d_states), state_stride, n_runs, max_positions,
                        _stream_ptr(stream), _np_ptr(errs))
    return e, errs


def fpi8_turn_bind(engine, d_states, state_stride: int, n_runs: int, stream=None):
    errs = np.zeros(n_runs, dtype=np.int32)
    e = lib().fpi8_turn_bind(engine, _dev_ptr(d_states), state_stride, n_runs, _stream_ptr(stream),
                             _np_ptr(errs))
    return e, errs


def fpi8_turn_async(engine, max_positions: int, stream=None, d_run_errors=None) -> int:
    return lib().fpi8_turn_async(engine, max_positions, _stream_ptr(stream),
                                 None if d_run_errors is None else _dev_ptr(d_run_errors))


def fpi8_turn_phases(engine, d_states, state_stride: int, n_runs: int, max_phases: int,
                     stream=None):
    errs = np.zeros(n_runs, dtype=np.int32)
    e = lib().fpi8_turn_phases(engine, _dev_ptr(d_states), state_stride, n_runs, max_phases,
                               _stream_ptr(stream), _np_ptr(errs))
    return e, errs


def fpi8_turn_units(engine, d_states, state_stride: int, n_runs: int, max_units: int,
                    stream=None):
    errs = np.zeros(n_runs, dtype=np.int32)
    e = lib().fpi8_turn_units(engine, _dev_ptr(d_states), state_stride, n_runs, max_units,
                              _stream_ptr(stream), _np_ptr(errs))
    return e, errs


def fpi8_tokenize(section0: np.ndarray, prompt: bytes, max_tokens: int):
    """(error, ids) of phases 0 to 2 for a prompt of bytes."""
    s0 = np.ascontiguousarray(section0, dtype=np.uint8)
    p = np.frombuffer(bytes(prompt), dtype=np.uint8).copy()
    n = C.c_uint32(0)
    ids = np.zeros(len(prompt) + 2, dtype=np.uint32)
    e = lib().fpi8_tokenize(_np_ptr(s0), s0.size, _np_ptr(p) if p.size else None, p.size,
                            max_tokens, _np_ptr(ids), ids.size, C.byref(n))
    return e, (ids[: n.value].copy() if e == 0 else None)


def fpi8_token_text(section0: np.ndarray, prev: int, token: int):
    """(error, bytes) a generated token adds after prev."""
    s0 = np.ascontiguousarray(section0, dtype=np.uint8)
    out = np.zeros(128, dtype=np.uint8)
    n = C.c_uint32(0)
    e = lib().fpi8_token_text(_np_ptr(s0), s0.size, prev, token, _np_ptr(out), out.size,
                              C.byref(n))
    return e, (out[: n.value].tobytes() if e == 0 else None)


def fpi8_output_text(section0: np.ndarray, state: np.ndarray):
    """(error, bytes) of a host state's generated tokens."""
    s0 = np.ascontiguousarray(section0, dtype=np.uint8)
    n = C.c_uint64(0)
    e = lib().fpi8_output_text(_np_ptr(s0), s0.size, _np_ptr(state), state.size, None, 0,
                               C.byref(n))
    if e not in (0, 4):
        return e, None
    out = np.zeros(max(n.value, 1), dtype=np.uint8)
    e = lib().fpi8_output_text(_np_ptr(s0), s0.size, _np_ptr(state), state.size, _np_ptr(out),
                               out.size, C.byref(n))
    return e, (out[: n.value].tobytes() if e == 0 else None)


def fpi8_pages_state_size(cfg, prompt_bytes: int, max_tokens: int) -> int:
    return lib().fpi8_pages_state_size(_np_ptr(_cfg(cfg)), prompt_bytes, max_tokens)


def fpi8_state_export(section0: np.ndarray, state: np.ndarray, prompt: bytes, cfg):
    """(error, bytes of the state in the page's format)."""
    s0 = np.ascontiguousarray(section0, dtype=np.uint8)
    info = fpi8_state_info(state)[1]
    n = fpi8_pages_state_size(cfg, len(prompt), info["max_tokens"])
    if n == UINT64_MAX:
        return 6, None
    out = np.zeros(n, dtype=np.uint8)
    p = np.frombuffer(bytes(prompt), dtype=np.uint8).copy()
    e = lib().fpi8_state_export(_np_ptr(s0), s0.size, _np_ptr(state), state.size,
                                _np_ptr(p) if p.size else None, p.size, _np_ptr(out), out.size)
    return e, (out if e == 0 else None)


def fpi8_state_import(cfg, pages: np.ndarray):
    """(error, state in this library's format, 8-byte aligned)."""
    n_ids = int(pages[32:36].view(np.uint32)[0])
    mx = int(pages[36:40].view(np.uint32)[0])
    size = fpi8_state_size(cfg, n_ids, mx)
    if size == UINT64_MAX:
        return 3, None
    raw = np.zeros(size + 64, dtype=np.uint8)
    off = (-raw.ctypes.data) % 64
    st = raw[off: off + size]
    e = lib().fpi8_state_import(_np_ptr(_cfg(cfg)), _np_ptr(pages), pages.size, _np_ptr(st), size)
    return e, (st if e == 0 else None)


def fpi8_pages_init(cfg, prompt: bytes, max_tokens: int, temperature_q16: int = 0, seed: int = 0):
    """(error, a fresh state in the page's format, before tokenizing)."""
    n = fpi8_pages_state_size(cfg, len(prompt), max_tokens)
    out = np.zeros(0 if n == UINT64_MAX else n, dtype=np.uint8)
    buf = C.create_string_buffer(bytes(prompt), max(len(prompt), 1))
    e = lib().fpi8_pages_init(_np_ptr(_cfg(cfg)), buf, len(prompt), max_tokens, temperature_q16,
                              C.c_uint64(seed), _np_ptr(out), out.size)
    return e, (out if e == 0 else None)


def fpi8_position_charges(cfg, position: int, generating: bool, temperature_q16: int = 0):
    """(error, compute units of phases 3 to 19 of one position, uint64[17])."""
    out = np.zeros(17, dtype=np.uint64)
    e = lib().fpi8_position_charges(_np_ptr(_cfg(cfg)), position, 1 if generating else 0,
                                    temperature_q16, _np_ptr(out))
    return e, out


def fpi8_pages_tokenize(section0: np.ndarray, pages: np.ndarray, max_units: int):
    """Runs up to max_units units of phases 0 to 2 in place: (error, units run)."""
    s0 = np.ascontiguousarray(section0, dtype=np.uint8)
    done = C.c_uint64(0)
    e = lib().fpi8_pages_tokenize(_np_ptr(s0), s0.size, _np_ptr(pages), pages.size,
                                  C.c_uint64(max_units), C.byref(done))
    return e, done.value


def fpi8_engine_set_row_kernel(engine, kind: int) -> int:
    return lib().fpi8_engine_set_row_kernel(engine, kind)


def fpi8_engine_set_graph(engine, enable: bool) -> int:
    return lib().fpi8_engine_set_graph(engine, 1 if enable else 0)


def fpi8_engine_set_streams(engine, streams: int) -> int:
    return lib().fpi8_engine_set_streams(engine, streams)


def fpi8_engine_set_timing(engine, kernel: int, enable: bool) -> int:
    return lib().fpi8_engine_set_timing(engine, kernel, 1 if enable else 0)


def fpi8_engine_timing(engine, kernel: int):
    ms = C.c_double(0)
    n = C.c_uint64(0)
    e = lib().fpi8_engine_timing(engine, kernel, C.byref(ms), C.byref(n))
    return e, ms.value, n.value


def fpi8_plan_turn(section_zero: np.ndarray, state: np.ndarray):
    """(error, plan dict) of the next turn of the run in a host state."""
    p = fpi8_turn_plan()
    e = lib().fpi8_plan_turn(_np_ptr(section_zero), section_zero.size, _np_ptr(state), state.size,
                             C.byref(p))
    return e, {"sections": list(p.sections)[:p.section_count], "estimated_cu": p.estimated_cu,
               "max_generated": p.max_generated, "units": p.units,
               "ends_with_draw": p.ends_with_draw}


def fpi8_quote_turns(section_zero: np.ndarray, state: np.ndarray):
    n = C.c_uint64(0)
    e = lib().fpi8_quote_turns(_np_ptr(section_zero), section_zero.size, _np_ptr(state), state.size,
                               C.byref(n))
    return e, n.value


NOALLOC_MAX_BATCH = 128
NOALLOC_MAX_COLS = 16384


def fpi8_matrix_rows_packed_noalloc(d_P, d_scale, rows: int, cols: int, d_x, batch: int, d_y,
                                    stream=None) -> int:
    return lib().fpi8_matrix_rows_packed_noalloc(_dev_ptr(d_P), _dev_ptr(d_scale), rows, cols,
                                                 _dev_ptr(d_x), batch, _dev_ptr(d_y),
                                                 _stream_ptr(stream))


def fpi8_matrix_rows_set_timing(enable: bool) -> int:
    return lib().fpi8_matrix_rows_set_timing(1 if enable else 0)


# fpi8_matrix_rows_set_path values
PATH_AUTO, PATH_MFMA, PATH_VALU = 0, 1, 2


def fpi8_matrix_rows_set_path(path: int) -> int:
    return lib().fpi8_matrix_rows_set_path(path)


def fpi8_matrix_rows_timing():
    ms = C.c_double(0)
    n = C.c_uint64(0)
    e = lib().fpi8_matrix_rows_timing(C.byref(ms), C.byref(n))
    return e, ms.value, n.value


def fpi8_matrix_rows_workspace_size(rows: int, cols: int, batch: int) -> int:
    return lib().fpi8_matrix_rows_workspace_size(rows, cols, batch)


def fpi8_matrix_rows(d_W, d_scale, rows: int, cols: int, d_x, batch: int, d_y, d_work,
                     work_len: int, stream=None) -> int:
    return lib().fpi8_matrix_rows(_dev_ptr(d_W), _dev_ptr(d_scale), rows, cols, _dev_ptr(d_x),
                                  batch, _dev_ptr(d_y), _dev_ptr(d_work), work_len,
                                  _stream_ptr(stream))


def fpi8_matrix_packed_size(rows: int, cols: int) -> int:
    return lib().fpi8_matrix_packed_size(rows, cols)


def fpi8_matrix_pack(d_W, rows: int, cols: int, d_P, p_len: int, stream=None) -> int:
    return lib().fpi8_matrix_pack(_dev_ptr(d_W), rows, cols, _dev_ptr(d_P), p_len, _stream_ptr(stream))


def fpi8_matrix_rows_packed(d_P, d_scale, rows: int, cols: int, d_x, batch: int, d_y, d_work,
                            work_len: int, stream=None) -> int:
    return lib().fpi8_matrix_rows_packed(_dev_ptr(d_P), _dev_ptr(d_scale), rows, cols, _dev_ptr(d_x),
                                         batch, _dev_ptr(d_y), _dev_ptr(d_work), work_len,
                                         _stream_ptr(stream))
