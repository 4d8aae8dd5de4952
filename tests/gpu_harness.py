"""Drives the HIP library and the CPU oracle side by side on one workload.

Both sides get the same seeded inputs from cache_gather_amd.workload; the
oracle keeps its own copy of the host rows, so nothing it reads can be touched
by the GPU path.
"""
import sys
import time

import numpy as np
import torch

import oracle
from cache_gather_amd import hc
from cache_gather_amd import workload as W


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def align4(n):
    return (n + 3) // 4 * 4


class Pair:
    def __init__(self, wl: W.Workload, score_stride=None, rows_fn=None, device=0, queries=1,
                 replacement=0):
        self.wl = wl
        self.Q = queries
        self.dev = torch.device("cuda", device)
        say("workload", wl.name, "S=%d L=%d R=%d K=%d C=%d H0=%d steps=%d" % (
            wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k, wl.cache_slots,
            wl.hist0, wl.steps))
        self.stride = align4(wl.hcap) if score_stride is None else score_stride
        self.hc = hc.HotCache(wl.n_sessions, wl.n_layers, wl.layers_per_select,
                              wl.cache_slots, wl.top_k, wl.hcap, device, queries=queries,
                              replacement=replacement)
        t0 = time.time()
        self.rows = [[None] * wl.n_layers for _ in range(wl.n_sessions)]
        for s in range(wl.n_sessions):
            for l in range(wl.n_layers):
                r = rows_fn(s, l) if rows_fn else W.fill_rows(wl, s, l)
                self.rows[s][l] = r
                np.copyto(self.hc.host_rows(s, l), r)
        say("rows ready in %.1fs" % (time.time() - t0))
        self.orc = oracle.Model(wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k,
                                wl.cache_slots, wl.hcap, self.rows, queries=queries,
                                replacement=replacement)
        self.scores = W.Scores(wl)
        self.out, self.sel, self.trace = self.hc.alloc_outputs(trace=True)
        self.d_scores = torch.empty((wl.n_units * queries, self.stride), dtype=torch.float32,
                                    device=self.dev)
        self.evictions = 0   # over all compared steps and units, as the oracle counts them

    def scores_for(self, t):
        return self.scores.step(t, self.stride, queries=self.Q)

    fill_only = False   # steps without a gathered output (hc_step with d_out = NULL)

    def gpu_step(self, t, scores_np, hist_len):
        self.d_scores.copy_(torch.from_numpy(scores_np))
        self.hc.step(self.d_scores, self.stride, hist_len, None if self.fill_only else self.out,
                     self.sel, self.trace)

    def step(self, t, scores_np=None, hist_len=None, gather=True, nthreads=16):
        """One step on both sides; returns (gpu dict, oracle tuple)."""
        wl = self.wl
        if scores_np is None:
            scores_np = self.scores_for(t)
        if hist_len is None:
            hist_len = wl.hist_len(t)
        self.gpu_step(t, scores_np, hist_len)
        o_sel, o_out, o_inf = self.orc.step(t, list(scores_np), np.asarray(hist_len, np.int64),
                                            gather=gather, nthreads=nthreads)
        torch.cuda.synchronize()
        g = {"sel": self.sel.cpu().numpy(), "trace": self.trace.cpu().numpy()}
        if gather and not self.fill_only:
            g["out"] = self.out.cpu().numpy().view(np.uint16)
        return g, (o_sel, o_out, o_inf)

    def compare(self, t, g, o, gather=True):
        wl = self.wl
        o_sel, o_out, o_inf = o
        K = wl.top_k * self.Q    # trace entries per unit: the round's union
        np.testing.assert_array_equal(g["sel"], o_sel, err_msg="selection, step %d" % t)
        for s in range(wl.n_sessions):
            for gi in range(wl.n_groups):
                u = s * wl.n_groups + gi
                tr = g["trace"][u]
                info = o_inf[s * wl.n_layers + gi * wl.layers_per_select]
                msg = "step %d unit %d" % (t, u)
                assert tr[0] == info["n_hit"] and tr[1] == info["n_miss"], msg
                assert tr[2] == info["n_evict"] and tr[3] == info["n_ring"], msg
                self.evictions += int(info["n_evict"])
                # the data movement the gather's lanes counted: each missing row
                # read from host RAM once per layer and written into its slot;
                # further query rows of a missing position read host RAM again;
                # every other selected row comes from HBM (slot or ring)
                nl = min(wl.layers_per_select, wl.n_layers - gi * wl.layers_per_select)
                n_miss = int(info["n_miss"])
                dup = 0
                if self.Q > 1:
                    sel_u = np.asarray(g["sel"]).reshape(wl.n_units, K)[u]
                    dup = int(np.isin(sel_u, np.asarray(info["miss_pos"][:n_miss])).sum()) - n_miss
                gathered = not self.fill_only
                assert tr[4] == (n_miss + (dup if gathered else 0)) * nl, msg + " host rows"
                assert tr[5] == ((K - n_miss - dup) * nl if gathered else 0), msg + " HBM rows"
                assert tr[6] == n_miss * nl, msg + " slot fills"
                assert tr[7] == (K * nl if gathered else 0), msg + " output rows"
                base = hc.TRACE_HEADER
                np.testing.assert_array_equal(tr[base:base + K], info["slot"], err_msg=msg)
                np.testing.assert_array_equal(tr[base + K:base + 2 * K], info["miss_pos"],
                                              err_msg=msg)
                np.testing.assert_array_equal(tr[base + 2 * K:base + 3 * K], info["victim"],
                                              err_msg=msg)
                np.testing.assert_array_equal(tr[base + 3 * K:base + 4 * K], info["evicted"],
                                              err_msg=msg)
        if gather and "out" in g:
            bad = np.argwhere(g["out"] != o_out)
            assert bad.size == 0, "output differs at step %d, first [s,l,i,j]=%s (%d values)" % (
                t, bad[0].tolist(), bad.shape[0])

    def compare_state(self):
        wl = self.wl
        for s in range(wl.n_sessions):
            for l in range(wl.n_layers):
                st = self.hc.export_state(s, l, pos2slot=True, hot_rows=True)
                c = self.orc.cache(s, l)
                np.testing.assert_array_equal(st["slot2pos"], c.pos_of())
                np.testing.assert_array_equal(st["last_use"], c.last())
                np.testing.assert_array_equal(st["pos2slot"], c.slot_of())
                res = np.flatnonzero(st["slot2pos"] >= 0)
                np.testing.assert_array_equal(st["hot"][res], c.hot()[res])
                # resident bytes equal the host copy
                np.testing.assert_array_equal(st["hot"][res], self.rows[s][l][st["slot2pos"][res]])

    def run(self, steps=None, gather_every=1, nthreads=16):
        steps = self.wl.steps if steps is None else steps
        t0 = time.time()
        for t in range(steps):
            gather = gather_every and (t % gather_every == 0 or t == steps - 1)
            g, o = self.step(t, gather=bool(gather), nthreads=nthreads)
            self.compare(t, g, o, gather=bool(gather))
        say("%s: %d steps bit-exact in %.1fs" % (self.wl.name, steps, time.time() - t0))
        self.compare_state()

    def close(self):
        self.hc.close()
        self.orc.close()


class RingPair(Pair):
    """Both sides with a recent ring.  Prefill rows [0, H0 - 1) are written to
    host RAM up front; step t first appends position H0 - 1 + t for every
    layer (so hist_len(t) = H0 + t as without a ring), and those rows reach
    host RAM only through the copybacks.  recent_boost is added to the scores
    of appended positions so that the ring is selected from."""

    def __init__(self, wl, ring_rows, copyback_rows, recent_boost=1.0, device=0, skip=None,
                 queries=1, replacement=0, score_stride=None):
        self.ring_rows, self.copyback_rows = ring_rows, copyback_rows
        self.Q = queries
        self.first = wl.hist0 - 1
        self.recent_boost = np.float32(recent_boost)
        self.skip = skip or (lambda t, s: False)  # session s appends nothing at step t
        self.wl = wl
        self.dev = torch.device("cuda", device)
        say("ring workload", wl.name, "S=%d L=%d K=%d C=%d H0=%d steps=%d ring=%d batch=%d" % (
            wl.n_sessions, wl.n_layers, wl.top_k, wl.cache_slots, wl.hist0, wl.steps,
            ring_rows, copyback_rows))
        self.stride = align4(wl.hcap) if score_stride is None else score_stride
        self.hc = hc.HotCache(wl.n_sessions, wl.n_layers, wl.layers_per_select,
                              wl.cache_slots, wl.top_k, wl.hcap, device,
                              ring_rows=ring_rows, copyback_rows=copyback_rows, queries=queries,
                              replacement=replacement)
        S, L = wl.n_sessions, wl.n_layers
        self.rows = [[W.fill_rows(wl, s, l) for l in range(L)] for s in range(S)]
        self.orc_host = [[np.zeros_like(self.rows[s][l]) for l in range(L)] for s in range(S)]
        for s in range(S):
            for l in range(L):
                h = self.hc.host_rows(s, l)
                h[:self.first] = self.rows[s][l][:self.first]
                h[self.first:] = 0
                self.orc_host[s][l][:self.first] = self.rows[s][l][:self.first]
        self.evictions = 0
        self.orc = oracle.Model(S, L, wl.layers_per_select, wl.top_k, wl.cache_slots, wl.hcap,
                                self.orc_host, ring_rows=ring_rows, copyback_rows=copyback_rows,
                                queries=queries, replacement=replacement)
        self.end = [self.first] * S
        self.scores = W.Scores(wl)
        self.out, self.sel, self.trace = self.hc.alloc_outputs(trace=True)
        self.d_scores = torch.empty((wl.n_units * queries, self.stride), dtype=torch.float32,
                                    device=self.dev)
        self.d_new = torch.empty((S, L, 656), dtype=torch.uint8, device=self.dev)

    def step(self, t, scores_np=None, hist_len=None, gather=True, nthreads=16):
        wl = self.wl
        S, L = wl.n_sessions, wl.n_layers
        pos = [None if self.skip(t, s) else self.end[s] for s in range(S)]
        new = np.zeros((S, L, 656), np.uint8)
        for s in range(S):
            if pos[s] is not None:
                for l in range(L):
                    new[s, l] = self.rows[s][l][pos[s]]
        self.d_new.copy_(torch.from_numpy(new))
        self.hc.append(self.d_new, pos)
        self.orc.append(pos, new)
        for s in range(S):
            if pos[s] is not None:
                self.end[s] += 1
        if hist_len is None:
            hist_len = np.array(self.end, np.uint64)
        if scores_np is None:
            scores_np = self.scores_for(t)
            for uq in range(wl.n_units * self.Q):
                s_ = uq // (wl.n_groups * self.Q)
                scores_np[uq, self.first:self.end[s_]] += self.recent_boost
        return Pair.step(self, t, scores_np, hist_len, gather, nthreads)

    def compare_host(self, margin=8):
        """Pinned host rows around the appended range equal the oracle's host
        store: copied rows equal, rows not copied yet still zero."""
        torch.cuda.synchronize()
        for s in range(self.wl.n_sessions):
            lo, hi = self.first, min(self.wl.hcap, self.end[s] + margin)
            for l in range(self.wl.n_layers):
                g = self.hc.host_rows(s, l)[lo:hi]
                o = self.orc_host[s][l][lo:hi]
                if not np.array_equal(g, o):
                    bad = np.flatnonzero((g != o).any(axis=1))
                    raise AssertionError("host rows differ: session %d layer %d positions %s"
                                         % (s, l, (lo + bad[:8]).tolist()))

    def flush_both(self):
        status, counts = self.hc.flush()
        o_counts = self.orc.flush()
        return status, counts, o_counts

    def run(self, steps=None, gather_every=1, nthreads=16, host_every=1):
        steps = self.wl.steps if steps is None else steps
        t0 = time.time()
        for t in range(steps):
            gather = gather_every and (t % gather_every == 0 or t == steps - 1)
            g, o = self.step(t, gather=bool(gather), nthreads=nthreads)
            self.compare(t, g, o, gather=bool(gather))
            if host_every and t % host_every == 0:
                self.compare_host()
        n_ring = int(sum(self.trace.cpu().numpy()[:, 3]))
        say("%s ring: %d steps bit-exact in %.1fs (last step read %d rows from the ring)" % (
            self.wl.name, steps, time.time() - t0, n_ring))
        status, counts, o_counts = self.flush_both()
        assert status == 0, hc.STATUS.get(status)
        np.testing.assert_array_equal(counts, o_counts)
        np.testing.assert_array_equal(counts, self.end)
        self.compare_host()
        self.compare_state()
