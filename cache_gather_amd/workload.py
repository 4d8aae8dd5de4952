"""Seeded synthetic inputs for the hot-cache decode step.

This module only draws random inputs; it holds none of the step's arithmetic
(no ranking, no cache logic, no dequantisation).  Both the HIP path and the
CPU oracle take their inputs from here.

The inputs stand in for the page "From 1M Total to 15+ × 1M Contexts: GLM-5.3
KV Cache Offloading" (zhuai.tech), whose runs used a private 50,023-token
prompt with a 32,768-row hot cache and DSA top-2,048 selection (sections
"Separate historical capacity from the current working set" and "Six
interleaved pairs establish the nearly lossless result").  No real selection
trace exists, so scores are a persistent per-position bias plus per-step
noise, which gives selections that overlap from one step to the next.

Recipe (all seeded; numpy PCG64 via default_rng with a tuple seed):
  rows of (session s, layer l), block b of 65,536 positions:
      rng((seed, 1, s, l, b)):
      latent  int8 uniform over [-127, 127] (random bytes, -128 redrawn)
      scales  fp16 of uniform[1e-3, 1e-1)  (numpy float32 -> float16 cast)
      RoPE    bf16 of N(0, 1) float32     (torch float32 -> bfloat16 cast)
  bias of unit (s, g):   sigma_b * N(0,1) float32, Hcap values, rng((seed, 2, s, g))
  noise of step t:       sigma_n * N(0,1) float32, H_t values, rng((seed, 3, s, g, t))
  scores(s, g, t) = bias[:H_t] + noise   (one float32 add)
  H_t = H0 + t: one position is appended per decode step; Hcap = H0 + steps.
  Multi-query rounds (MTP verification, Q query rows): query 0 has the scores
  above; query q > 0 adds its own draft noise, one more float32 add:
      sigma_draft * N(0,1) float32, H_t values, rng((seed, 4, s, g, q, t))
  so the Q selections overlap heavily without being equal.
  Attention queries (the consumer of the gathered rows), per (s, l, t):
      bf16 of N(0,1) float32 (torch float32 -> bfloat16), [Q][heads][576],
      rng((seed, 5, s, l, t)).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_BYTES = 656
BLOCK_ROWS = 65536


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_sessions: int
    n_layers: int
    layers_per_select: int
    hist0: int
    steps: int
    cache_slots: int
    top_k: int
    sigma_bias: tuple      # per session
    sigma_noise: tuple     # per session
    seed: int
    note: str = ""

    @property
    def n_groups(self) -> int:
        return -(-self.n_layers // self.layers_per_select)

    @property
    def hcap(self) -> int:
        return self.hist0 + self.steps

    @property
    def n_units(self) -> int:
        return self.n_sessions * self.n_groups

    def hist_len(self, t: int) -> np.ndarray:
        return np.full(self.n_sessions, self.hist0 + t, dtype=np.uint64)

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _rep(x, n):
    return tuple([x] * n)


# The workloads, named by what they are.
TINY = Workload("tiny_4k", 1, 1, 1, 4096, 16, 1024, 256, (0.5,), (1.0,), 1001,
                "history 4,096, 1,024 slots, top-256, 16 steps")
PAGE_50K = Workload("page_50k", 1, 1, 1, 50023, 1024, 32768, 2048, (1.0,), (0.3,), 1002,
                    "one layer, history 50,023, 32,768 slots, top-2,048, 1,024 steps")
MODEL78_50K = Workload("model78_50k", 1, 78, 4, 50023, 64, 32768, 2048, (1.0,), (0.3,), 1003,
                       "78 layers, selection every 4th layer, history 50,023, 64 steps")
LONG_1M = Workload("long_1m", 1, 1, 1, 1048576, 256, 32768, 2048, (0.2,), (1.0,), 1004,
                   "one layer, history 1,048,576, low locality, 256 steps")
BATCH16_1M = Workload("batch16_1m", 16, 1, 1, 1048576, 128, 32768, 2048,
                      _rep(1.0, 8) + _rep(0.2, 8), _rep(0.3, 8) + _rep(1.0, 8), 1005,
                      "16 sessions of 1,048,576 positions, 8 high + 8 low locality")
# Calibrated variants reproducing the stated overlap / miss statistics.
PAGE_50K_CAL = PAGE_50K.with_(name="page_50k_cal", sigma_noise=(0.075,), seed=1012,
                              note="page_50k with noise sigma 0.075 (about 0.9 overlap)")
LONG_1M_CAL = LONG_1M.with_(name="long_1m_cal", sigma_bias=(1.2,), seed=1014,
                            note="long_1m with bias sigma 1.2 (about 30% misses)")
BATCH16_1M_CAL = BATCH16_1M.with_(name="batch16_1m_cal",
                                  sigma_bias=_rep(1.0, 8) + _rep(1.2, 8), seed=1015,
                                  note="batch16_1m with the low half at bias sigma 1.2")

ALL = {w.name: w for w in (TINY, PAGE_50K, MODEL78_50K, LONG_1M, BATCH16_1M,
                           PAGE_50K_CAL, LONG_1M_CAL, BATCH16_1M_CAL)}


def _workers():
    return max(1, min(16, os.cpu_count() or 1))


# ------------------------------------------------------------------ rows ---

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    import torch  # library conversion float32 -> bfloat16 (round to nearest even)
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy()


def _fill_block(out: np.ndarray, seed: int, s: int, l: int, b: int) -> None:
    n = out.shape[0]
    rng = np.random.default_rng((seed, 1, s, l, b))
    q = np.frombuffer(rng.bytes(n * 512), dtype=np.int8).copy()
    bad = np.flatnonzero(q == -128)
    while bad.size:
        q[bad] = np.frombuffer(rng.bytes(bad.size), dtype=np.int8)
        bad = bad[q[bad] == -128]
    scales = rng.uniform(1e-3, 1e-1, size=(n, 8)).astype(np.float32).astype(np.float16)
    rope = _bf16_bits(rng.standard_normal((n, 64), dtype=np.float32))
    out[:, 0:512] = q.view(np.uint8).reshape(n, 512)
    out[:, 512:528] = scales.view(np.uint8).reshape(n, 16)
    out[:, 528:656] = rope.view(np.uint8).reshape(n, 128)


def fill_rows(wl: Workload, s: int, l: int, out: np.ndarray | None = None,
              n_rows: int | None = None) -> np.ndarray:
    """Rows [0, n_rows) of (session s, layer l) as uint8 [n_rows, 656], written
    into `out` when given (e.g. a view of pinned host memory)."""
    n_rows = wl.hcap if n_rows is None else n_rows
    if out is None:
        out = np.empty((n_rows, ROW_BYTES), dtype=np.uint8)
    assert out.shape[0] >= n_rows and out.shape[1] == ROW_BYTES and out.dtype == np.uint8
    blocks = range(0, -(-n_rows // BLOCK_ROWS))

    def one(b):
        lo, hi = b * BLOCK_ROWS, min(n_rows, (b + 1) * BLOCK_ROWS)
        _fill_block(out[lo:hi], wl.seed, s, l, b)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, blocks))
    return out


def fill_all_rows(wl: Workload, dest=None) -> list:
    """Rows of every (session, layer), generated in parallel over (s, l, block).
    dest(s, l) may return a uint8 [>= Hcap, 656] array to fill (e.g. pinned
    host memory); otherwise new arrays are made.  Returns rows[s][l]."""
    n = wl.hcap
    rows = [[dest(s, l) if dest else np.empty((n, ROW_BYTES), np.uint8)
             for l in range(wl.n_layers)] for s in range(wl.n_sessions)]
    jobs = [(s, l, b) for s in range(wl.n_sessions) for l in range(wl.n_layers)
            for b in range(-(-n // BLOCK_ROWS))]

    def one(job):
        s, l, b = job
        lo, hi = b * BLOCK_ROWS, min(n, (b + 1) * BLOCK_ROWS)
        _fill_block(rows[s][l][lo:hi], wl.seed, s, l, b)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(one, jobs))
    return rows


# ---------------------------------------------------------------- scores ---

class Scores:
    """Per-step scores of every unit (s, g); the bias vectors are kept."""

    def __init__(self, wl: Workload):
        self.wl = wl
        self._bias = {}

    def bias(self, s: int, g: int) -> np.ndarray:
        key = (s, g)
        if key not in self._bias:
            rng = np.random.default_rng((self.wl.seed, 2, s, g))
            self._bias[key] = (np.float32(self.wl.sigma_bias[s])
                               * rng.standard_normal(self.wl.hcap, dtype=np.float32))
        return self._bias[key]

    def unit(self, s: int, g: int, t: int) -> np.ndarray:
        h = self.wl.hist0 + t
        rng = np.random.default_rng((self.wl.seed, 3, s, g, t))
        noise = np.float32(self.wl.sigma_noise[s]) * rng.standard_normal(h, dtype=np.float32)
        return self.bias(s, g)[:h] + noise

    def step(self, t: int, stride: int | None = None, queries: int = 1,
             sigma_draft: float = 0.1) -> np.ndarray:
        """float32 [S*G*Q, stride] for step t (entries past H_t are zero);
        row (s*G + g)*Q + q is query q of unit (s, g)."""
        wl = self.wl
        stride = wl.hcap if stride is None else stride
        out = np.zeros((wl.n_units * queries, stride), dtype=np.float32)

        def one(uq):
            u, q = divmod(uq, queries)
            s, g = divmod(u, wl.n_groups)
            x = self.unit(s, g, t)
            if q:
                h = x.size
                rng = np.random.default_rng((self.wl.seed, 4, s, g, q, t))
                x = x + np.float32(sigma_draft) * rng.standard_normal(h, dtype=np.float32)
            out[uq, :x.size] = x

        for u in range(wl.n_units):   # bias vectors first, then parallel noise
            self.bias(*divmod(u, wl.n_groups))
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(wl.n_units * queries)))
        return out


def queries(wl: Workload, t: int, heads: int, n_queries: int = 1) -> np.ndarray:
    """bf16 bit patterns (uint16) [S, L, Q, heads, 576] of step t's attention
    queries (or [S, L, heads, 576] for one query row)."""
    out = np.empty((wl.n_sessions, wl.n_layers, n_queries, heads, 576), np.uint16)
    for s in range(wl.n_sessions):
        for l in range(wl.n_layers):
            rng = np.random.default_rng((wl.seed, 5, s, l, t))
            x = rng.standard_normal((n_queries, heads, 576), dtype=np.float32)
            out[s, l] = _bf16_bits(x).view(np.uint16)
    return out if n_queries > 1 else out[:, :, 0]
