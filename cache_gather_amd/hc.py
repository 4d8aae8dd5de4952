"""ctypes binding of libhc.so (include/hc.h), with the same entry-point names.

Argument marshalling only: every step of the decode path runs in the HIP
kernels of libhc.so.  There is no fallback: if the library is missing or
cannot be loaded, every call raises.  torch is imported before the library
is loaded so that the process uses the one HIP runtime torch ships with;
torch only provides device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libhc.so")
HEADER = os.path.join(ROOT, "include", "hc.h")

ROW_BYTES = 656
OUT_ELEMS = 576
ATTEND_STATIC_BYTES = 32 << 20   # HC_ATTEND_STATIC_BYTES
TRACE_HEADER = 8
NUM_STAGES = 3
STAGES = ("topk_scan", "select", "gather")
STATUS = {0: "HC_OK", -1: "HC_E_INVAL", -2: "HC_E_NOMEM", -3: "HC_E_HIP", -4: "HC_E_STATE",
          -5: "HC_E_CONSISTENCY", -6: "HC_E_DEVICE"}
NO_APPEND = (1 << 64) - 1


def trace_ints(k: int) -> int:
    return TRACE_HEADER + 4 * k


class HcError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (fn, STATUS.get(status, "?"), status))


class hc_config(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("n_sessions", ctypes.c_uint32),
                ("n_layers", ctypes.c_uint32), ("layers_per_select", ctypes.c_uint32),
                ("cache_slots", ctypes.c_uint32), ("top_k", ctypes.c_uint32),
                ("max_positions", ctypes.c_uint64), ("device", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("ring_rows", ctypes.c_uint32),
                ("copyback_rows", ctypes.c_uint32), ("queries", ctypes.c_uint32),
                ("replacement", ctypes.c_uint32)]


CONFIG_SIZE_NO_RING = hc_config.ring_rows.offset
CONFIG_SIZE_ONE_QUERY = hc_config.queries.offset
LRU, CIRCULAR, CLOCK = 0, 1, 2   # hc_config.replacement


def make_config(n_sessions, n_layers, layers_per_select, cache_slots, top_k, max_positions,
                device=0, flags=0, ring_rows=0, copyback_rows=0, queries=1,
                replacement=LRU) -> hc_config:
    return hc_config(ctypes.sizeof(hc_config), n_sessions, n_layers, layers_per_select,
                     cache_slots, top_k, max_positions, device, flags, ring_rows,
                     copyback_rows, queries, replacement)


_LIB = None
_TEST_LIB = None
_vp = ctypes.c_void_p
TEST_LIB_PATH = os.path.join(HERE, "libhc_test.so")


def lib():
    """The loaded libhc.so; raises if it was not built."""
    global _LIB
    if _LIB is None:
        _LIB = _load(LIB_PATH)
    return _LIB


def test_lib():
    """The test build libhc_test.so (the same entry points plus hc_test_hook,
    include/hc_test.h), loaded beside libhc.so; for the tests of failure paths."""
    global _TEST_LIB
    if _TEST_LIB is None:
        L = _load(TEST_LIB_PATH)
        L.hc_test_hook.argtypes = [_vp, ctypes.c_int, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)]
        L.hc_test_hook.restype = ctypes.c_int
        _TEST_LIB = L
    return _TEST_LIB


class using:
    """with using(test_lib()): every hc_* call of this module goes to that
    library (contexts are not shared between libraries)."""

    def __init__(self, L):
        self.L = L

    def __enter__(self):
        global _LIB
        lib()
        self.prev, _LIB = _LIB, self.L
        return self.L

    def __exit__(self, *exc):
        global _LIB
        _LIB = self.prev


def _load(path):
    import torch  # noqa: F401  (its HIP runtime must be the one in the process)
    if not os.path.exists(path):
        raise RuntimeError("%s is not built; run __graft_entry__.build()" % path)
    L = ctypes.CDLL(path)
    st = ctypes.c_int
    L.hc_workspace_bytes.argtypes = [ctypes.POINTER(hc_config), ctypes.POINTER(ctypes.c_uint64)]
    L.hc_workspace_bytes.restype = st
    L.hc_create.argtypes = [ctypes.POINTER(hc_config), _vp, ctypes.c_uint64, ctypes.POINTER(_vp)]
    L.hc_create.restype = st
    L.hc_host_rows.argtypes = [_vp, ctypes.c_uint32, ctypes.c_uint32]
    L.hc_host_rows.restype = _vp
    L.hc_step.argtypes = [_vp, _vp, _vp, ctypes.c_uint64, ctypes.POINTER(ctypes.c_uint64),
                          _vp, _vp, _vp]
    L.hc_step.restype = st
    L.hc_append.argtypes = [_vp, _vp, _vp, ctypes.POINTER(ctypes.c_uint64)]
    L.hc_append.restype = st
    L.hc_flush.argtypes = [_vp, _vp, _vp]
    L.hc_flush.restype = st
    L.hc_attend_workspace_bytes.argtypes = [_vp, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint64)]
    L.hc_attend_workspace_bytes.restype = st
    L.hc_attend.argtypes = [_vp, _vp, _vp, ctypes.c_uint32, ctypes.c_float, _vp, _vp,
                            ctypes.c_uint64, _vp]
    L.hc_attend.restype = st
    L.hc_attend_cached.argtypes = [_vp, _vp, _vp, ctypes.c_uint32, ctypes.c_float, _vp,
                                   ctypes.c_uint64, _vp]
    L.hc_attend_cached.restype = st
    L.hc_attend_cached_noalloc.argtypes = [_vp, _vp, _vp, ctypes.c_uint32, ctypes.c_float, _vp]
    L.hc_attend_cached_noalloc.restype = st
    L.hc_export_state.argtypes = [_vp, ctypes.c_uint32, ctypes.c_uint32, _vp, _vp, _vp, _vp]
    L.hc_export_state.restype = st
    L.hc_profile_enable.argtypes = [_vp, ctypes.c_uint32]
    L.hc_profile_enable.restype = st
    L.hc_profile_read.argtypes = [_vp, ctypes.POINTER(ctypes.c_double), _vp, ctypes.c_uint64,
                                  ctypes.POINTER(ctypes.c_uint64)]
    L.hc_profile_read.restype = st
    L.hc_steps_done.argtypes = [_vp, ctypes.POINTER(ctypes.c_uint64)]
    L.hc_steps_done.restype = st
    L.hc_destroy.argtypes = [_vp]
    L.hc_destroy.restype = st
    L.hc_status_str.argtypes = [ctypes.c_int]
    L.hc_status_str.restype = ctypes.c_char_p
    return L


def declared_functions() -> list[str]:
    """Names of the functions include/hc.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(hc_\w+)\s*\(", text, re.M)))


def _check(fn, status):
    if status != 0:
        raise HcError(fn, status)


def _ptr(x):
    """Raw address of a torch tensor, numpy array, int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(type(x))


# ---------------------------------------------------------- entry points ---

def hc_workspace_bytes(cfg: hc_config) -> int:
    n = ctypes.c_uint64()
    _check("hc_workspace_bytes", lib().hc_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def hc_create(cfg: hc_config, dev_workspace, ws_bytes: int) -> int:
    out = _vp()
    _check("hc_create", lib().hc_create(ctypes.byref(cfg), _ptr(dev_workspace), ws_bytes,
                                        ctypes.byref(out)))
    return out.value


def hc_host_rows(ctx: int, session: int, layer: int, max_positions: int) -> np.ndarray:
    """The pinned host rows of (session, layer) as a writable uint8 [Hcap, 656] view."""
    p = lib().hc_host_rows(ctx, session, layer)
    if not p:
        raise HcError("hc_host_rows", -1)
    buf = (ctypes.c_uint8 * (max_positions * ROW_BYTES)).from_address(p)
    return np.frombuffer(buf, dtype=np.uint8).reshape(max_positions, ROW_BYTES)


def hc_step(ctx: int, stream, d_scores, score_stride: int, hist_len, d_out, d_sel,
            d_trace=None) -> None:
    hl = np.ascontiguousarray(hist_len, dtype=np.uint64)
    _check("hc_step", lib().hc_step(ctx, _ptr(stream), _ptr(d_scores), score_stride,
                                    hl.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)),
                                    _ptr(d_out), _ptr(d_sel), _ptr(d_trace)))


def hc_append(ctx: int, stream, d_rows, pos) -> None:
    """pos: one position per session, or NO_APPEND (None is accepted too)."""
    p = np.array([NO_APPEND if x is None else x for x in pos], dtype=np.uint64)
    _check("hc_append", lib().hc_append(ctx, _ptr(stream), _ptr(d_rows),
                                        p.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))))


def hc_flush(ctx: int, stream, n_sessions: int, check=True):
    """Returns (status, host row count per session); raises on a failure other
    than HC_E_CONSISTENCY unless check is False."""
    counts = np.zeros(n_sessions, np.uint64)
    r = lib().hc_flush(ctx, _ptr(stream), _ptr(counts))
    if check and r not in (0, -5):
        raise HcError("hc_flush", r)
    return r, counts


def hc_attend_workspace_bytes(ctx: int, heads: int) -> int:
    n = ctypes.c_uint64()
    _check("hc_attend_workspace_bytes", lib().hc_attend_workspace_bytes(ctx, heads, ctypes.byref(n)))
    return n.value


def hc_attend(ctx: int, stream, d_q, heads: int, scale: float, d_rows, d_work, work_bytes: int,
              d_out) -> None:
    _check("hc_attend", lib().hc_attend(ctx, _ptr(stream), _ptr(d_q), heads, scale,
                                        _ptr(d_rows), _ptr(d_work), work_bytes, _ptr(d_out)))


def hc_attend_cached(ctx: int, stream, d_q, heads: int, scale: float, d_work, work_bytes: int,
                     d_out) -> None:
    _check("hc_attend_cached", lib().hc_attend_cached(ctx, _ptr(stream), _ptr(d_q), heads, scale,
                                                      _ptr(d_work), work_bytes, _ptr(d_out)))


def hc_attend_cached_noalloc(ctx: int, stream, d_q, heads: int, scale: float, d_out) -> None:
    _check("hc_attend_cached_noalloc", lib().hc_attend_cached_noalloc(ctx, _ptr(stream), _ptr(d_q),
                                                                      heads, scale, _ptr(d_out)))


def hc_export_state(ctx: int, session: int, layer: int, slots: int, max_positions: int,
                    pos2slot=False, hot_rows=False):
    slot2pos = np.empty(slots, np.int32)
    last_use = np.empty(slots, np.int32)
    p2s = np.empty(max_positions, np.int32) if pos2slot else None
    hot = np.empty((slots, ROW_BYTES), np.uint8) if hot_rows else None
    _check("hc_export_state", lib().hc_export_state(ctx, session, layer, _ptr(slot2pos),
                                                    _ptr(last_use), _ptr(p2s), _ptr(hot)))
    return {"slot2pos": slot2pos, "last_use": last_use, "pos2slot": p2s, "hot": hot}


def hc_profile_enable(ctx: int, max_steps: int) -> None:
    _check("hc_profile_enable", lib().hc_profile_enable(ctx, max_steps))


def hc_profile_read(ctx: int, max_steps: int = 0):
    """(summed ms per stage, n timed steps, per-step ms [n, stages] or None)."""
    ms = (ctypes.c_double * NUM_STAGES)()
    n = ctypes.c_uint64()
    per = np.zeros((max_steps, NUM_STAGES), np.float64) if max_steps else None
    _check("hc_profile_read", lib().hc_profile_read(ctx, ms, _ptr(per), max_steps,
                                                    ctypes.byref(n)))
    if per is not None:
        per = per[:min(n.value, max_steps)]
    return dict(zip(STAGES, list(ms))), n.value, per


def hc_steps_done(ctx: int) -> int:
    n = ctypes.c_uint64()
    _check("hc_steps_done", lib().hc_steps_done(ctx, ctypes.byref(n)))
    return n.value


def hc_test_hook(ctx, kind: int, arg: int = 0) -> int:
    """The test build's hook (include/hc_test.h); returns its output value."""
    out = ctypes.c_uint64()
    _check("hc_test_hook", test_lib().hc_test_hook(ctx, kind, arg, ctypes.byref(out)))
    return out.value


(TEST_FAIL_LAUNCH, TEST_FORCE_SELECT, TEST_CORRUPT_LRU, TEST_FAIL_PINNED, TEST_PINNED_BYTES,
 TEST_POISON_VICTIMS) = 1, 2, 3, 4, 5, 6


def hc_destroy(ctx: int) -> None:
    _check("hc_destroy", lib().hc_destroy(ctx))


def hc_status_str(status: int) -> str:
    return lib().hc_status_str(status).decode()


# ------------------------------------------------- torch-owned resources ---

class HotCache:
    """One context plus its torch-allocated device workspace.

    torch supplies only device memory and the stream; the library does the rest.
    """

    def __init__(self, n_sessions, n_layers, layers_per_select, cache_slots, top_k,
                 max_positions, device=0, ring_rows=0, copyback_rows=0, queries=1,
                 replacement=LRU):
        import torch
        self.cfg = make_config(n_sessions, n_layers, layers_per_select, cache_slots, top_k,
                               max_positions, device, 0, ring_rows, copyback_rows, queries,
                               replacement)
        self.Q = queries
        self.S, self.L, self.R = n_sessions, n_layers, layers_per_select
        self.G = -(-n_layers // layers_per_select)
        self.C, self.K, self.hcap = cache_slots, top_k, max_positions
        self.device = torch.device("cuda", device)
        self.ctx = 0
        self._L = lib()   # the library the context belongs to (see `using`)
        self.ws_bytes = hc_workspace_bytes(self.cfg)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        assert self.workspace.data_ptr() % 256 == 0
        self.ctx = hc_create(self.cfg, self.workspace, self.ws_bytes)

    def host_rows(self, s, l) -> np.ndarray:
        return hc_host_rows(self.ctx, s, l, self.hcap)

    def step(self, scores, score_stride, hist_len, out, sel, trace=None, stream=None):
        import torch
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        hc_step(self.ctx, st.cuda_stream, scores, score_stride, hist_len, out, sel, trace)

    def _stream(self, stream):
        import torch
        return (stream if stream is not None else torch.cuda.current_stream(self.device)).cuda_stream

    def append(self, rows, pos, stream=None):
        """rows: device uint8 [S, L, 656]; pos: position per session or None."""
        hc_append(self.ctx, self._stream(stream), rows, pos)

    def flush(self, stream=None):
        """(status, host row count per session) after the consistency boundary."""
        return hc_flush(self.ctx, self._stream(stream), self.S)

    def attention_buffers(self, heads):
        """(scratch, out fp32 [S, L, (Q,) heads, 512]) for hc_attend*."""
        import torch
        nbytes = hc_attend_workspace_bytes(self.ctx, heads)
        work = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        q = (self.Q,) if self.Q > 1 else ()
        out = torch.empty((self.S, self.L) + q + (heads, 512), dtype=torch.float32,
                          device=self.device)
        return work, out

    def attend(self, q, heads, scale, rows, work, out, stream=None):
        """Attention over the last step's gathered bf16 rows."""
        hc_attend(self.ctx, self._stream(stream), q, heads, scale, rows, work, work.numel(), out)

    def attend_cached(self, q, heads, scale, work, out, stream=None):
        """Attention reading the last step's rows from the slots (no bf16 buffer)."""
        hc_attend_cached(self.ctx, self._stream(stream), q, heads, scale, work, work.numel(), out)

    def attend_cached_noalloc(self, q, heads, scale, out, stream=None):
        """attend_cached with the library's own scratch (no allocation)."""
        hc_attend_cached_noalloc(self.ctx, self._stream(stream), q, heads, scale, out)

    def export_state(self, s, l, pos2slot=False, hot_rows=False):
        return hc_export_state(self.ctx, s, l, self.C, self.hcap, pos2slot, hot_rows)

    def alloc_outputs(self, trace=False):
        """out [S, L, K, 576] and sel [S, G, K]; with Q > 1 query rows per
        round, out [S, L, Q, K, 576] and sel [S, G, Q, K]."""
        import torch
        q = (self.Q,) if self.Q > 1 else ()
        out = torch.empty((self.S, self.L) + q + (self.K, OUT_ELEMS), dtype=torch.int16,
                          device=self.device)
        sel = torch.empty((self.S, self.G) + q + (self.K,), dtype=torch.int32,
                          device=self.device)
        tr = (torch.empty((self.S * self.G, trace_ints(self.Q * self.K)), dtype=torch.int32,
                          device=self.device) if trace else None)
        return out, sel, tr

    def close(self):
        if self.ctx:
            with using(self._L):
                hc_destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
