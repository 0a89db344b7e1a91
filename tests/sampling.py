"""Row and key selection for the full-size GPU parity tests, and a threaded
driver of the oracle over the selected rows.

Full-size shares hold 16K-32K query rows per head over up to 1M keys; the
float64 oracle cannot afford every row, so each share is checked on a seeded
sample of at least MIN_ROWS rows that always includes the rows where the
kernel changes behaviour: the first and last rows of each half of the share
(the zigzag chunks), and rows at in-tile offsets of the 256-row workgroup
tiles (0, 1, 63, 64, 127, 128, 129, 191, 192, 255). For the duplicated-key
stress share, rows whose best visible key has an exact twin (an exact tie in
the row maximum) are added on top.

Nothing here computes an expected value: row choice only, plus scheduling of
``oracle.attention_rows`` calls on worker threads.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import ring_inputs

MIN_ROWS = 1024
TILE_ROWS = 256
TILE_OFFSETS = (0, 1, 63, 64, 127, 128, 129, 191, 192, 255)


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def sample_rows(wl: ring_inputs.Workload, seed: int, n_rows: int = MIN_ROWS, extra=()) -> np.ndarray:
    """Sorted local row indices: boundary rows, tile-offset rows of a few
    tiles (first, last, middle and random ones), ``extra``, then seeded
    random rows up to ``n_rows`` in total."""
    c = wl.local_len
    g = c // 2
    rng = np.random.default_rng(seed)
    base = set()
    for s0 in (0, g):
        base |= {s0, s0 + 1, s0 + g - 2, s0 + g - 1}
    n_tiles = (c + TILE_ROWS - 1) // TILE_ROWS
    tiles = {0, 1, n_tiles // 2 - 1, n_tiles // 2, n_tiles - 2, n_tiles - 1}
    tiles |= set(rng.choice(n_tiles, size=min(6, n_tiles), replace=False).tolist())
    for t in tiles:
        base |= {t * TILE_ROWS + o for o in TILE_OFFSETS}
    base |= {int(r) for r in extra}
    base = {r for r in base if 0 <= r < c}
    need = n_rows - len(base)
    if need > 0:
        pool = np.setdiff1d(np.arange(c, dtype=np.int64), np.fromiter(base, dtype=np.int64))
        base |= set(rng.choice(pool, size=min(need, len(pool)), replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)


def tied_argmax_rows(wl: ring_inputs.Workload, positions: np.ndarray, heads, n_pool: int, seed: int,
                     batch: int = 0) -> np.ndarray:
    """Local rows (from a seeded pool of ``n_pool``) whose highest-scoring
    visible key, for at least one of the query ``heads``, is a duplicated
    key whose twin is visible too, so the row maximum is an exact tie.

    ``positions`` are the global positions of the share's local rows. The
    twins come from ``ring_inputs.duplicate_plan`` (each destination key is
    an exact copy of its source key), so the tie is decided from the plan,
    not from comparing floating-point scores."""
    rng = np.random.default_rng(seed)
    pool = np.sort(rng.choice(len(positions), size=min(n_pool, len(positions)), replace=False))
    pos = positions[pool]
    G = wl.heads_q // wl.heads_kv
    found = set()
    for h in heads:
        g = h // G
        dst, src = ring_inputs.duplicate_plan(wl, batch, g)
        twins = {}
        for a, b in zip(dst.tolist(), src.tolist()):
            twins.setdefault(a, []).append(b)
            twins.setdefault(b, []).append(a)
        k = ring_inputs.head(wl, "k", batch, g).astype(np.float64)
        q = ring_inputs.rows(wl, "q", batch, h, pos).astype(np.float64)
        for r0 in range(0, len(pool), 128):
            sl = slice(r0, r0 + 128)
            s = q[sl] @ k.T
            if wl.causal:
                s[np.arange(k.shape[0])[None, :] > pos[sl, None]] = -np.inf
            best = s.argmax(axis=1)
            for i, j in enumerate(best.tolist()):
                p = int(pos[sl][i])
                if any(t <= p or not wl.causal for t in twins.get(j, ())):
                    found.add(int(pool[sl][i]))
    return np.array(sorted(found), dtype=np.int64)


class OracleRows:
    """Oracle output at chosen local rows of one device share, computed on
    worker threads while the share is being built.

    Pass ``on_head`` to ``harness.build_share``: every KV head's global K/V
    is queued (in row blocks, one job per query head of the group and block)
    as it is drawn; ``result()`` waits and returns (O [B, Hq, R, d],
    LSE [B, Hq, R]) in float64."""

    def __init__(self, wl: ring_inputs.Workload, positions: np.ndarray, block: int = 128):
        self.wl = wl
        self.positions = np.asarray(positions, dtype=np.int64)
        self.block = block
        R = len(self.positions)
        self.o = np.zeros((wl.batch, wl.heads_q, R, wl.head_dim))
        self.lse = np.zeros((wl.batch, wl.heads_q, R))
        self.k_pos = np.arange(wl.total_len, dtype=np.int64)
        self.pool = ThreadPoolExecutor(threads())
        self.jobs = []
        try:
            from threadpoolctl import threadpool_limits
            self._limit = threadpool_limits(limits=1, user_api="blas")
        except Exception:  # BLAS threads stay as they are
            self._limit = None

    def _job(self, b, h, kh, vh, sl):
        q = ring_inputs.rows(self.wl, "q", b, h, self.positions[sl])
        o, s = oracle.attention_rows(q, self.positions[sl], kh, vh, self.k_pos, self.wl.causal)
        self.o[b, h, sl] = o
        self.lse[b, h, sl] = s

    def on_head(self, b, g, kh, vh):
        G = self.wl.heads_q // self.wl.heads_kv
        R = len(self.positions)
        for h in range(g * G, (g + 1) * G):
            for r0 in range(0, R, self.block):
                self.jobs.append(self.pool.submit(self._job, b, h, kh, vh, slice(r0, min(R, r0 + self.block))))

    def result(self):
        try:
            for j in self.jobs:
                j.result()
        finally:
            self.pool.shutdown()
            if self._limit is not None:
                self._limit.restore_original_limits()
        return self.o, self.lse
