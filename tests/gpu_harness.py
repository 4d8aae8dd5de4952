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
    def __init__(self, wl: W.Workload, score_stride=None, rows_fn=None, device=0):
        self.wl = wl
        self.dev = torch.device("cuda", device)
        say("workload", wl.name, "S=%d L=%d R=%d K=%d C=%d H0=%d steps=%d" % (
            wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k, wl.cache_slots,
            wl.hist0, wl.steps))
        self.stride = align4(wl.hcap) if score_stride is None else score_stride
        self.hc = hc.HotCache(wl.n_sessions, wl.n_layers, wl.layers_per_select,
                              wl.cache_slots, wl.top_k, wl.hcap, device)
        t0 = time.time()
        self.rows = [[None] * wl.n_layers for _ in range(wl.n_sessions)]
        for s in range(wl.n_sessions):
            for l in range(wl.n_layers):
                r = rows_fn(s, l) if rows_fn else W.fill_rows(wl, s, l)
                self.rows[s][l] = r
                np.copyto(self.hc.host_rows(s, l), r)
        say("rows ready in %.1fs" % (time.time() - t0))
        self.orc = oracle.Model(wl.n_sessions, wl.n_layers, wl.layers_per_select, wl.top_k,
                                wl.cache_slots, wl.hcap, self.rows)
        self.scores = W.Scores(wl)
        self.out, self.sel, self.trace = self.hc.alloc_outputs(trace=True)
        self.d_scores = torch.empty((wl.n_units, self.stride), dtype=torch.float32,
                                    device=self.dev)

    def scores_for(self, t):
        return self.scores.step(t, self.stride)

    def gpu_step(self, t, scores_np, hist_len):
        self.d_scores.copy_(torch.from_numpy(scores_np))
        self.hc.step(self.d_scores, self.stride, hist_len, self.out, self.sel, self.trace)

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
        if gather:
            g["out"] = self.out.cpu().numpy().view(np.uint16)
        return g, (o_sel, o_out, o_inf)

    def compare(self, t, g, o, gather=True):
        wl = self.wl
        o_sel, o_out, o_inf = o
        K = wl.top_k
        np.testing.assert_array_equal(g["sel"], o_sel, err_msg="selection, step %d" % t)
        for s in range(wl.n_sessions):
            for gi in range(wl.n_groups):
                u = s * wl.n_groups + gi
                tr = g["trace"][u]
                info = o_inf[s * wl.n_layers + gi * wl.layers_per_select]
                msg = "step %d unit %d" % (t, u)
                assert tr[0] == info["n_hit"] and tr[1] == info["n_miss"], msg
                assert tr[2] == info["n_evict"], msg
                base = hc.TRACE_HEADER
                np.testing.assert_array_equal(tr[base:base + K], info["slot"], err_msg=msg)
                np.testing.assert_array_equal(tr[base + K:base + 2 * K], info["miss_pos"],
                                              err_msg=msg)
                np.testing.assert_array_equal(tr[base + 2 * K:base + 3 * K], info["victim"],
                                              err_msg=msg)
                np.testing.assert_array_equal(tr[base + 3 * K:base + 4 * K], info["evicted"],
                                              err_msg=msg)
        if gather:
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
