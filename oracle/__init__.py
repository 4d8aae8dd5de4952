"""ctypes binding of the plain-C CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py may import this package; the HIP product path
never does.  The oracle shares no code with the HIP library.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)

ROW_BYTES = 656
OUT_ELEMS = 576
LRU, CIRCULAR, CLOCK = 0, 1, 2   # replacement policies


class StepInfo(ctypes.Structure):
    _fields_ = [("n_hit", ctypes.c_int32), ("n_miss", ctypes.c_int32),
                ("n_evict", ctypes.c_int32),
                ("slot", _i32p), ("miss_pos", _i32p),
                ("victim", _i32p), ("evicted", _i32p),
                ("n_ring", ctypes.c_int32)]


def lib():
    global _LIB
    if _LIB is None:
        # ORACLE_LIB lets the mutation tests load a deliberately broken copy
        path = os.environ.get("ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.orc_topk.argtypes = [_f32p, ctypes.c_int64, ctypes.c_int32, _i32p]
        L.orc_topk.restype = ctypes.c_int
        L.orc_dequant_elem.argtypes = [ctypes.c_int8, ctypes.c_uint16]
        L.orc_dequant_elem.restype = ctypes.c_uint16
        L.orc_dequant_row.argtypes = [_u8p, _u16p]
        L.orc_dequant_row.restype = None
        L.orc_attend.argtypes = [_u16p, _u16p, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                 ctypes.POINTER(ctypes.c_double)]
        L.orc_attend.restype = None
        L.orc_dequant_table.argtypes = [_u16p]
        L.orc_dequant_table.restype = None
        L.orc_cache_new.argtypes = [ctypes.c_int32, ctypes.c_int64]
        L.orc_cache_new.restype = ctypes.c_void_p
        L.orc_cache_new_policy.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
        L.orc_cache_new_policy.restype = ctypes.c_void_p
        L.orc_cache_ref.argtypes = [ctypes.c_void_p]
        L.orc_cache_ref.restype = _u8p
        L.orc_cache_hand.argtypes = [ctypes.c_void_p]
        L.orc_cache_hand.restype = ctypes.c_int32
        L.orc_cache_free.argtypes = [ctypes.c_void_p]
        L.orc_cache_free.restype = None
        L.orc_cache_step.argtypes = [ctypes.c_void_p, ctypes.c_int32, _i32p, ctypes.c_int32,
                                     _u8p, ctypes.c_void_p, ctypes.POINTER(StepInfo)]
        L.orc_cache_step.restype = ctypes.c_int
        L.orc_gather.argtypes = [ctypes.c_void_p, ctypes.c_void_p, _i32p, ctypes.c_int32, _u16p]
        L.orc_gather.restype = ctypes.c_int
        for name in ("orc_cache_slot_of", "orc_cache_pos_of", "orc_cache_last"):
            getattr(L, name).argtypes = [ctypes.c_void_p]
            getattr(L, name).restype = _i32p
        L.orc_cache_hot.argtypes = [ctypes.c_void_p]
        L.orc_cache_hot.restype = _u8p
        L.orc_ring_new.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.orc_ring_new.restype = ctypes.c_void_p
        L.orc_ring_free.argtypes = [ctypes.c_void_p]
        L.orc_ring_free.restype = None
        L.orc_ring_append.argtypes = [ctypes.c_void_p, ctypes.c_int64, _u8p, _u8p]
        L.orc_ring_append.restype = ctypes.c_int
        L.orc_ring_flush.argtypes = [ctypes.c_void_p, _u8p]
        L.orc_ring_flush.restype = ctypes.c_int64
        L.orc_ring_row.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        L.orc_ring_row.restype = _u8p
        L.orc_ring_copied.argtypes = [ctypes.c_void_p]
        L.orc_ring_copied.restype = ctypes.c_int64
        L.orc_model_step.argtypes = [
            ctypes.POINTER(ctypes.c_void_p), ctypes.POINTER(_u8p), ctypes.POINTER(ctypes.c_void_p),
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32, ctypes.POINTER(_f32p), ctypes.POINTER(ctypes.c_int64),
            _i32p, _u16p, ctypes.POINTER(StepInfo), ctypes.c_int32]
        L.orc_model_step.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def topk(scores, k):
    """Exact top-k positions of fp32 scores (totalOrder, ties to lower
    position), ascending."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    sel = np.empty(k, dtype=np.int32)
    if lib().orc_topk(_ptr(s, _f32p), s.size, k, _ptr(sel, _i32p)) != 0:
        raise ValueError("orc_topk: need 1 <= k <= len(scores)")
    return sel


def dequant_elem(q, scale_bits):
    return lib().orc_dequant_elem(int(q), int(scale_bits))


def dequant_row(row):
    r = np.ascontiguousarray(row, dtype=np.uint8)
    assert r.size == ROW_BYTES
    out = np.empty(OUT_ELEMS, dtype=np.uint16)
    lib().orc_dequant_row(_ptr(r, _u8p), _ptr(out, _u16p))
    return out


def attend(q, rows, scale):
    """MLA decode attention: q uint16 bf16 bits [H, 576], rows uint16 bf16
    bits [K, 576] -> float64 [H, 512]."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    H, K = q.shape[0], rows.shape[0]
    assert q.shape[1] == OUT_ELEMS and rows.shape[1] == OUT_ELEMS
    out = np.empty((H, 512), np.float64)
    lib().orc_attend(_ptr(q, _u16p), _ptr(rows, _u16p), H, K, float(scale),
                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def dequant_table():
    """table[q + 128, scale_bits] for every int8 q and every fp16 bit pattern."""
    t = np.empty((256, 65536), dtype=np.uint16)
    lib().orc_dequant_table(_ptr(t, _u16p))
    return t


class _InfoBufs:
    def __init__(self, k):
        self.slot = np.empty(k, np.int32)
        self.miss_pos = np.empty(k, np.int32)
        self.victim = np.empty(k, np.int32)
        self.evicted = np.empty(k, np.int32)
        self.info = StepInfo(0, 0, 0, _ptr(self.slot, _i32p), _ptr(self.miss_pos, _i32p),
                             _ptr(self.victim, _i32p), _ptr(self.evicted, _i32p), 0)

    def result(self):
        n = self.info.n_miss
        return {"n_hit": self.info.n_hit, "n_miss": n, "n_evict": self.info.n_evict,
                "n_ring": self.info.n_ring,
                "slot": self.slot.copy(), "miss_pos": self.miss_pos.copy(),
                "victim": self.victim.copy(), "evicted": self.evicted.copy()}


class Ring:
    """Recent ring of one (session, layer): the last `rows` appended rows, a
    batched copyback of every `batch` rows into the host row store."""

    def __init__(self, rows, batch):
        self.rows, self.batch = int(rows), int(batch)
        self._p = lib().orc_ring_new(self.rows, self.batch)
        if not self._p:
            raise ValueError("orc_ring_new: need 1 <= batch <= rows")

    def close(self):
        if self._p:
            lib().orc_ring_free(self._p)
            self._p = None

    def __del__(self):
        self.close()

    def append(self, p, row, host_rows):
        r = np.ascontiguousarray(row, dtype=np.uint8)
        assert r.size == ROW_BYTES and host_rows.flags.c_contiguous and host_rows.dtype == np.uint8
        if lib().orc_ring_append(self._p, int(p), _ptr(r, _u8p), _ptr(host_rows, _u8p)) != 0:
            raise ValueError("orc_ring_append: position out of order")

    def flush(self, host_rows):
        assert host_rows.flags.c_contiguous and host_rows.dtype == np.uint8
        return int(lib().orc_ring_flush(self._p, _ptr(host_rows, _u8p)))

    def holds(self, p):
        return bool(lib().orc_ring_row(self._p, int(p)))

    def copied(self):
        return int(lib().orc_ring_copied(self._p))


class Cache:
    """Hot cache of one (session, layer); replacement LRU, CIRCULAR or CLOCK."""

    def __init__(self, slots, hcap, policy=LRU):
        self.C, self.hcap = int(slots), int(hcap)
        self._p = lib().orc_cache_new_policy(self.C, self.hcap, int(policy))
        if not self._p:
            raise MemoryError("orc_cache_new failed")

    def close(self):
        if self._p:
            lib().orc_cache_free(self._p)
            self._p = None

    def __del__(self):
        self.close()

    def step(self, t, sel, host_rows, ring=None):
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        rows = np.ascontiguousarray(host_rows, dtype=np.uint8)
        assert rows.size >= self.hcap * ROW_BYTES
        bufs = _InfoBufs(sel.size)
        rc = lib().orc_cache_step(self._p, int(t), _ptr(sel, _i32p), sel.size,
                                  _ptr(rows, _u8p), ring._p if ring else None,
                                  ctypes.byref(bufs.info))
        if rc != 0:
            raise ValueError("orc_cache_step rejected its input")
        return bufs.result()

    def gather(self, sel, ring=None):
        sel = np.ascontiguousarray(sel, dtype=np.int32)
        out = np.empty((sel.size, OUT_ELEMS), dtype=np.uint16)
        if lib().orc_gather(self._p, ring._p if ring else None, _ptr(sel, _i32p), sel.size,
                            _ptr(out, _u16p)) != 0:
            raise ValueError("orc_gather: a selected position is not resident")
        return out

    def slot_of(self):
        return np.ctypeslib.as_array(lib().orc_cache_slot_of(self._p), (self.hcap,)).copy()

    def pos_of(self):
        return np.ctypeslib.as_array(lib().orc_cache_pos_of(self._p), (self.C,)).copy()

    def last(self):
        return np.ctypeslib.as_array(lib().orc_cache_last(self._p), (self.C,)).copy()

    def hot(self):
        return np.ctypeslib.as_array(lib().orc_cache_hot(self._p),
                                     (self.C, ROW_BYTES)).copy()

    def ref(self):
        return np.ctypeslib.as_array(lib().orc_cache_ref(self._p), (self.C,)).copy()

    def hand(self):
        return int(lib().orc_cache_hand(self._p))


class Model:
    """S sessions x L layers, one selection per group of R layers; each layer
    keeps its own LRU cache.  host_rows[s][l] is a uint8 [hcap, 656] array.
    With ring_rows > 0 every layer also has a recent ring (batch copyback_rows)
    that append() feeds and whose copybacks write into host_rows (which must
    then be writable C-contiguous uint8 arrays: they are used in place)."""

    def __init__(self, n_sessions, n_layers, layers_per_select, top_k, slots, hcap, host_rows,
                 ring_rows=0, copyback_rows=0, queries=1, replacement=LRU):
        self.S, self.L, self.R = int(n_sessions), int(n_layers), int(layers_per_select)
        self.G = -(-self.L // self.R)
        self.K, self.C, self.hcap = int(top_k), int(slots), int(hcap)
        self.Q = int(queries)
        self.caches = [Cache(slots, hcap, replacement) for _ in range(self.S * self.L)]
        self.rows = [np.ascontiguousarray(host_rows[s][l], dtype=np.uint8)
                     for s in range(self.S) for l in range(self.L)]
        for r in self.rows:
            assert r.size >= self.hcap * ROW_BYTES
        n = self.S * self.L
        self._cache_arr = (ctypes.c_void_p * n)(*[c._p for c in self.caches])
        self._rows_arr = (_u8p * n)(*[_ptr(r, _u8p) for r in self.rows])
        self.rings = None
        self._ring_arr = None
        if ring_rows:
            for s in range(self.S):
                for l in range(self.L):
                    assert self.rows[s * self.L + l] is host_rows[s][l], \
                        "ring copybacks need the caller's host arrays in place"
            self.rings = [Ring(ring_rows, copyback_rows) for _ in range(n)]
            self._ring_arr = (ctypes.c_void_p * n)(*[r._p for r in self.rings])

    def cache(self, s, l):
        return self.caches[s * self.L + l]

    def ring(self, s, l):
        return self.rings[s * self.L + l]

    def append(self, pos, new_rows):
        """Appends position pos[s] of every session (None: skip the session);
        new_rows[s][l] is that position's 656-B row of layer l."""
        for s in range(self.S):
            if pos[s] is None:
                continue
            for l in range(self.L):
                self.ring(s, l).append(pos[s], new_rows[s][l], self.rows[s * self.L + l])

    def flush(self):
        """Copies every appended row not yet in host RAM; returns the host row
        frontier of each session (all layers agree)."""
        out = []
        for s in range(self.S):
            f = {self.ring(s, l).flush(self.rows[s * self.L + l]) for l in range(self.L)}
            assert len(f) == 1
            out.append(f.pop())
        return out

    def step(self, t, scores, hist_len, gather=True, info=True, nthreads=1):
        """scores[(s*G + g)*Q + q]: fp32 array of at least hist_len[s] entries.
        Returns (sel [S,G,K] or [S,G,Q,K] when Q > 1, out [S,L,K,576] or
        [S,L,Q,K,576] or None, infos list or None); with Q > 1 the infos cover
        the union of the group's Q selections (Q*K entries per array)."""
        units = self.S * self.G * self.Q
        sc = [np.ascontiguousarray(x, dtype=np.float32) for x in scores]
        assert len(sc) == units
        for u, x in enumerate(sc):
            assert x.size >= hist_len[u // (self.G * self.Q)]
        sc_arr = (_f32p * units)(*[_ptr(x, _f32p) for x in sc])
        hl = np.ascontiguousarray(hist_len, dtype=np.int64)
        QK = self.Q * self.K
        sel = np.empty((self.S, self.G, self.Q, self.K), np.int32)
        out = (np.empty((self.S, self.L, self.Q, self.K, OUT_ELEMS), np.uint16)
               if gather else None)
        bufs = [_InfoBufs(QK) for _ in range(self.S * self.L)] if info else None
        info_arr = (StepInfo * (self.S * self.L))(*[b.info for b in bufs]) if info else None
        rc = lib().orc_model_step(
            self._cache_arr, self._rows_arr, self._ring_arr, self.S, self.L, self.R, self.K,
            self.Q, int(t), sc_arr, _ptr(hl, ctypes.POINTER(ctypes.c_int64)), _ptr(sel, _i32p),
            _ptr(out, _u16p) if gather else None, info_arr, int(nthreads))
        if rc != 0:
            raise ValueError("orc_model_step failed")
        infos = None
        if info:
            # the structs were copied into info_arr; read counts back from there
            infos = []
            for i, b in enumerate(bufs):
                b.info = info_arr[i]
                infos.append(b.result())
        if self.Q == 1:
            sel = sel[:, :, 0]
            out = out[:, :, 0] if gather else None
        return sel, out, infos

    def close(self):
        for c in self.caches:
            c.close()
        for r in self.rings or ():
            r.close()
