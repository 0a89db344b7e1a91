"""Full-softmax attention in float64 at chosen query rows (oracle side).

Test infrastructure only; see the package docstring.

Definition followed (for every batch b, query head h and query row i at
global position p_i):

* kv head g(h) = floor(h / (H_q / H_kv)) — contiguous GQA groups; lecture 30
  (section 8.3, question 1) gives each GPU 8 Q heads and 1 KV head when 64 Q
  heads and 8 KV heads are split 8 ways, which is contiguous grouping.
* visible keys V_i = all global positions j when not causal, else those with
  j <= p_i (lower triangle including the diagonal; lecture 30 section 3.2).
* s_ij = (q_i . k_j) * scale, scale = 1/sqrt(head_dim) ("distributed training
  hands-on code", section 6.2, block_attention).
* O_i = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i), m_i = max_j s_ij
  (the same section: the softmax fold, finished by O / L).
* LSE_i = m_i + ln sum_j exp(s_ij - m_i) (natural log; the pages use torch.exp).
* A row with no visible key gets O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math

import numpy as np

import ring_inputs
from .positions import device_positions


def kv_head_of(h: int, heads_q: int, heads_kv: int) -> int:
    """KV head read by query head h (contiguous groups of H_q / H_kv)."""
    if heads_q % heads_kv:
        raise ValueError("heads_q must be a multiple of heads_kv")
    return h // (heads_q // heads_kv)


def attention_rows(q, q_pos, k, v, k_pos, causal: bool, scale: float | None = None,
                   row_group: int = 64):
    """float64 softmax attention of query rows ``q`` [R, d] over keys ``k`` [L, d].

    Returns (O [R, dv], LSE [R]). Rows are evaluated independently, ``row_group``
    at a time (in order of position), each over all of its visible keys at
    once. When the mask is causal and ``k_pos`` is ascending, keys past the
    last position a group's rows can see carry weight exactly zero for every
    row of the group and are left out of its products.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    R = q.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full(R, -np.inf, dtype=np.float64)
    ascending = bool(causal) and bool(np.all(k_pos[1:] >= k_pos[:-1]))
    order = np.argsort(q_pos, kind="stable")
    for r0 in range(0, R, row_group):
        idx = order[r0:min(R, r0 + row_group)]
        n = len(k_pos)
        if ascending and len(idx):
            n = int(np.searchsorted(k_pos, q_pos[idx].max(), side="right"))
        kk, vv, kp = k[:n], v[:n], k_pos[:n]
        s = q[idx] @ kk.T
        s *= scale
        if causal:
            if ascending:  # each row's visible keys are a prefix of kk
                for i, e in enumerate(np.searchsorted(kp, q_pos[idx], side="right")):
                    s[i, e:] = -np.inf
            else:
                s[kp[None, :] > q_pos[idx, None]] = -np.inf
        m = s.max(axis=1) if n else np.full(len(idx), -np.inf)
        has = np.isfinite(m)
        s -= np.where(has, m, 0.0)[:, None]
        p = np.exp(s, out=s)
        l = p.sum(axis=1)
        o = (p @ vv) / np.where(has, l, 1.0)[:, None]
        o[~has] = 0.0
        out[idx] = o
        with np.errstate(divide="ignore"):
            lse[idx] = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return out, lse


def visible_pair_count(q_pos, k_pos, causal: bool) -> int:
    """Number of (query, key) pairs that attention uses: all pairs, or k_pos <= q_pos."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.sort(np.asarray(k_pos, dtype=np.int64))
    if not causal:
        return int(len(q_pos) * len(k_pos))
    return int(np.searchsorted(k_pos, q_pos, side="right").sum())


def device_share(wl: "ring_inputs.Workload", rank: int, rows=None, heads=None, batches=None):
    """Oracle output of one device's share of a ring workload.

    ``rows`` selects local row indices (default: all ``local_len``); ``heads``
    selects query heads (default: all). Keys and values are the whole global
    sequence, positions 0..L-1, drawn by ``ring_inputs``.

    Returns dict with ``out`` [B', H', R, d], ``lse`` [B', H', R], ``rows``,
    ``positions`` (global position of each returned row) and ``heads``.
    """
    local_pos = device_positions(wl.partition, wl.world, rank, wl.local_len)
    rows = np.arange(wl.local_len) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(wl.heads_q)) if heads is None else list(heads)
    batches = list(range(wl.batch)) if batches is None else list(batches)
    q_pos = local_pos[rows]
    k_pos = np.arange(wl.total_len, dtype=np.int64)
    out = np.zeros((len(batches), len(heads), len(rows), wl.head_dim))
    lse = np.zeros((len(batches), len(heads), len(rows)))
    for bi, b in enumerate(batches):
        cache = {}
        for hi, h in enumerate(heads):
            g = kv_head_of(h, wl.heads_q, wl.heads_kv)
            if g not in cache:
                cache.clear()
                cache[g] = (ring_inputs.head(wl, "k", b, g), ring_inputs.head(wl, "v", b, g))
            k, v = cache[g]
            q = ring_inputs.rows(wl, "q", b, h, q_pos)
            o, s = attention_rows(q, q_pos, k, v, k_pos, wl.causal)
            out[bi, hi] = o
            lse[bi, hi] = s
    return {"out": out, "lse": lse, "rows": rows, "positions": q_pos, "heads": heads}
