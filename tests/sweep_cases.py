"""Seeded random configurations for the GPU parity sweep.

Each draw fixes sessions, layers, layers per selection, top-K, query rows,
slots, history lengths (a different start per session, some sessions pausing
on some steps), the replacement policy, the score row stride and, for some
draws, a recent ring with its copyback batch.  The draws stay inside the
limits the C ABI states, which a CPU test checks through hc_workspace_bytes.
Nothing here computes any part of the method.
"""
import dataclasses
import math

import numpy as np

from cache_gather_amd import workload as W

N_CASES = 48
LRU, CIRCULAR, CLOCK = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Case:
    seed: int
    wl: W.Workload
    queries: int
    policy: int
    ring_rows: int
    copyback_rows: int
    stride_pad: int            # score row stride = Hcap rounded to 4, plus this
    start_back: tuple          # per session: history at step 0 is hist0 - this
    pause: tuple               # per session: probability of not growing in a step

    @property
    def name(self):
        wl = self.wl
        return "s%d_S%dL%dR%d_K%dQ%dC%d_H%d_p%d%s" % (
            self.seed, wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k,
            self.queries, wl.cache_slots, wl.hist0, self.policy,
            "_ring%dx%d" % (self.ring_rows, self.copyback_rows) if self.ring_rows else "")

    def hist_len(self, t):
        """History per session at step t (rings: set by the appends instead).
        Starts at hist0 - start_back[s]; grows by one on every step after
        the first that the session does not pause; never exceeds hist0 + t."""
        out = np.empty(self.wl.n_sessions, np.uint64)
        for s in range(self.wl.n_sessions):
            rng = np.random.default_rng((self.seed, 7, s))
            grow = rng.random(self.wl.steps) >= self.pause[s]
            out[s] = self.wl.hist0 - self.start_back[s] + int(grow[1:t + 1].sum())
        return out

    def skip(self, t, s):
        """Ring draws: session s appends nothing at step t."""
        return bool(np.random.default_rng((self.seed, 8, s, t)).random() < self.pause[s])


def draw(seed):
    rng = np.random.default_rng((0x5EE9, seed))
    S = int(rng.integers(1, 5))
    L = int(rng.integers(1, 6))
    R = int(rng.integers(1, L + 1))
    Q = int(rng.choice([1, 1, 1, 2, 3, 4]))
    K = int(math.exp(rng.uniform(0.0, math.log(4096.0))))
    K = max(1, min(K, 8192 // Q))
    C = min(Q * K + int(rng.integers(0, 3 * Q * K + 64)), 65536)
    H0 = max(K + 1, int(math.exp(rng.uniform(math.log(K + 1.0), math.log(120000.0)))))
    steps = int(rng.integers(6, 15))
    policy = int(rng.choice([LRU, LRU, CIRCULAR, CLOCK]))
    ring = batch = 0
    if rng.random() < 0.3:
        ring = int(rng.choice([8, 16, 64, 256]))
        batch = int(rng.integers(1, ring + 1))
    pad = int(rng.choice([0, 0, 0, 1, 2, 3]))
    back = tuple(int(rng.integers(0, (H0 - K) // 2 + 1)) if (ring == 0 and s > 0) else 0
                 for s in range(S))
    pause = tuple(float(rng.choice([0.0, 0.0, 0.3])) for _ in range(S))
    sb = tuple(float(x) for x in rng.uniform(0.1, 1.2, S))
    sn = tuple(float(x) for x in rng.uniform(0.3, 1.0, S))
    wl = W.Workload("sweep_%d" % seed, S, L, R, H0, steps, C, K, sb, sn, 7000 + seed)
    return Case(seed, wl, Q, policy, ring, batch, pad, back, pause)


CASES = [draw(i) for i in range(N_CASES)]
