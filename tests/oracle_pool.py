"""The oracle over many rows in a process pool, for the full-size GPU tests.

Workers are started with `spawn`, so none of them inherits the test
process's GPU context; each regenerates its inputs from the seeded generator
(deterministic, so every worker sees the same step) and runs the oracle on
its share of the rows.  The merged result has the layout of one
oracle.verify call over those rows.
"""

import multiprocessing as mp
import os

import numpy as np

WORKERS = 8


def _rows(args):
    import oracle
    from rejection_sampling_verifier_amd import workloads as W

    cfg, step, overrides, rows = args
    inp = W.make_inputs(cfg, step, **overrides)
    return oracle.verify(inp.target, inp.draft, inp.draft_tokens, inp.draft_len, inp.temperature, inp.top_p,
                         inp.seed, rows=rows)


def _merge(parts):
    base = parts[0]
    for p in parts[1:]:
        for b in p.rows:
            base.tokens[b] = p.tokens[b]
            base.n_accepted[b] = p.n_accepted[b]
            base.probe_pos[b] = p.probe_pos[b]
            base.probe_row[b] = p.probe_row[b]
            base.min_margin[b] = p.min_margin[b]
            base.n_decisions[b] = p.n_decisions[b]
            base.n_flagged[b] = p.n_flagged[b]
            base.u_res[b] = p.u_res[b]
            if b in p.margins:
                base.margins[b] = p.margins[b]
                base.accepts[b] = p.accepts[b]
            if b in p.sample_cdf:
                base.sample_cdf[b] = p.sample_cdf[b]
            if b in p.cuts:
                base.cuts[b] = p.cuts[b]
    base.rows = np.sort(np.concatenate([p.rows for p in parts]))
    return base


class OraclePool:
    """with OraclePool() as pool: res = pool.verify(cfg, step, rows)

    Workers regenerate the inputs of the step they are given, so a job per
    (step, chunk of rows) costs one input generation per chunk."""

    def __init__(self, workers=WORKERS):
        self.workers = max(1, min(workers, os.cpu_count() or 1))
        self._pool = None

    def __enter__(self):
        self._pool = mp.get_context("spawn").Pool(self.workers)
        return self

    def __exit__(self, *exc):
        self._pool.close()
        self._pool.join()

    def submit(self, cfg, step, rows, chunks=None, **overrides):
        """Starts the oracle on `rows` of step `step`, split into `chunks`
        jobs (default: one per worker); .get() returns the merged result."""
        rows = np.asarray(rows)
        chunks = [c for c in np.array_split(rows, chunks or self.workers) if c.size]
        return _Job([self._pool.apply_async(_rows, ((cfg, step, overrides, c),)) for c in chunks])

    def verify(self, cfg, step, rows, **overrides):
        return self.submit(cfg, step, rows, **overrides).get()


class _Job:
    def __init__(self, parts):
        self._parts = parts

    def get(self):
        return _merge([p.get() for p in self._parts])
