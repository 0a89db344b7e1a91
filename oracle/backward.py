"""Gradients of full-softmax attention in float64 (oracle side).

Test infrastructure only; see the package docstring.

The pages give the ring forward only ("distributed training hands-on code",
section 6.2, runs the ring without a backward pass). The backward ring step is
the plain extension of the same fold, and what the ring of backward steps
reaches exactly (up to rounding order) is the gradient of full attention.
That gradient is what this module writes out, by the chain rule applied to
the forward definition of ``attention.py``; for every batch, query head h and
query row i with visible keys V_i, given the upstream gradient dO_i:

* P_ij = exp(s_ij - LSE_i) for j in V_i, else 0 (the forward's softmax);
* dV_j = sum_i P_ij dO_i;
* dP_ij = dO_i . v_j;
* D_i = sum_j P_ij dP_ij, which equals dO_i . O_i;
* dS_ij = P_ij (dP_ij - D_i);
* dQ_i = scale * sum_j dS_ij k_j;   dK_j = scale * sum_i dS_ij q_i.

GQA: a KV head's dK and dV are the sums over the query heads that read it.
A row without visible keys contributes nothing and gets dQ = 0.
"""
from __future__ import annotations

import math

import numpy as np

import ring_inputs
from .attention import attention_rows, kv_head_of
from .positions import device_positions


def attention_backward_rows(q, q_pos, k, v, k_pos, do, causal: bool, scale: float | None = None):
    """Gradients of the attention of rows ``q`` [R, d] over keys ``k`` [L, d].

    ``do`` [R, dv] is the gradient of the loss with respect to the output.
    Returns a dict: ``dq`` [R, d], ``dk`` [L, d], ``dv`` [L, dv] (the part of
    the key/value gradients that these rows produce), ``out`` [R, dv],
    ``lse`` [R] and ``delta`` [R] (= D_i). Two more row terms size the
    rounding error a reduced-precision evaluation of dQ can make (they are
    not gradients): ``p_k`` [R, d] = sum_j P_ij k_j (the attention output
    with the keys as values) and ``abs_ds_k`` [R, d] = sum_j |dS_ij| |k_j|.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    out, lse = attention_rows(q, q_pos, k, v, k_pos, causal, scale)
    s = (q @ k.T) * scale
    visible = np.ones(s.shape, dtype=bool)
    if causal:
        visible = k_pos[None, :] <= q_pos[:, None]
    has = np.isfinite(lse)
    p = np.where(visible & has[:, None], np.exp(s - np.where(has, lse, 0.0)[:, None]), 0.0)
    dv = p.T @ do
    dp = do @ v.T
    delta = np.einsum("rd,rd->r", do, out)
    ds = p * (dp - delta[:, None])
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return {"dq": dq, "dk": dk, "dv": dv, "out": out, "lse": lse, "delta": delta,
            "p_k": p @ k, "abs_ds_k": np.abs(ds) @ np.abs(k)}


def key_gradients(q, q_pos, k, v, k_pos, do, causal: bool, key_index, scale: float | None = None):
    """The part of dK_j and dV_j that rows ``q`` produce, for the keys
    ``key_index`` (indices into ``k``) only.

    The row statistics come from all keys: LSE_i and O_i by ``attention_rows``,
    D_i = dO_i . O_i. Then, at the chosen keys j only: P_ij = exp(s_ij -
    LSE_i) where visible, dP_ij = dO_i . v_j, dS_ij = P_ij (dP_ij - D_i),
    dK_j = scale * sum_i dS_ij q_i and dV_j = sum_i P_ij dO_i — the same chain
    rule as ``attention_backward_rows``, restricted to a few columns, so a few
    keys of a long sequence cost only the rows that can see them.

    Also returns three sums that size the rounding error of a
    reduced-precision evaluation (not gradients), per key and column:
    ``abs_ds_q`` = sum_i |dS_ij| |q_i|, ``p_a_q`` = sum_i P_ij A_i |q_i| with
    A_i = sum_d |dO_id| |O_id|, and ``p_do`` = sum_i P_ij |dO_i|.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    key_index = np.asarray(key_index, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[1])
    out, lse = attention_rows(q, q_pos, k, v, k_pos, causal, scale)
    kj, vj, pj = k[key_index], v[key_index], k_pos[key_index]
    s = (q @ kj.T) * scale
    visible = np.ones(s.shape, dtype=bool)
    if causal:
        visible = pj[None, :] <= q_pos[:, None]
    has = np.isfinite(lse)
    p = np.where(visible & has[:, None], np.exp(s - np.where(has, lse, 0.0)[:, None]), 0.0)
    dp = do @ vj.T
    delta = np.einsum("rd,rd->r", do, out)
    ds = p * (dp - delta[:, None])
    a = (np.abs(do) * np.abs(out)).sum(axis=1)
    return {"dk": scale * (ds.T @ q), "dv": p.T @ do,
            "abs_ds_q": np.abs(ds).T @ np.abs(q), "p_a_q": p.T @ (a[:, None] * np.abs(q)),
            "p_do": p.T @ np.abs(do)}


def upstream_rows(wl: "ring_inputs.Workload", b: int, h: int, positions) -> np.ndarray:
    """The seeded upstream gradient dO at the given global positions (float32)."""
    return ring_inputs.rows(wl, "do", b, h, positions)


def device_backward(wl: "ring_inputs.Workload", rank: int, heads=None):
    """One device's part of the backward pass of a ring workload.

    The device holds the query rows its partition gives it. Returns a dict:
    ``dq`` [B, H', R, d] for those rows (query heads ``heads``, default all),
    ``dk`` and ``dv`` [B, H_kv, L, d]: the device's contribution to the key
    and value gradients of the whole global sequence (indexed by global
    position), summed over the query heads selected; ``positions`` [R].
    Summing ``dk``/``dv`` over all devices gives the full gradient.
    """
    pos = device_positions(wl.partition, wl.world, rank, wl.local_len)
    heads = list(range(wl.heads_q)) if heads is None else list(heads)
    k_pos = np.arange(wl.total_len, dtype=np.int64)
    L, d = wl.total_len, wl.head_dim
    dq = np.zeros((wl.batch, len(heads), len(pos), d))
    dk = np.zeros((wl.batch, wl.heads_kv, L, d))
    dv = np.zeros((wl.batch, wl.heads_kv, L, d))
    for b in range(wl.batch):
        cache = {}
        for hi, h in enumerate(heads):
            g = kv_head_of(h, wl.heads_q, wl.heads_kv)
            if g not in cache:
                cache.clear()
                cache[g] = (ring_inputs.head(wl, "k", b, g), ring_inputs.head(wl, "v", b, g))
            k, v = cache[g]
            q = ring_inputs.rows(wl, "q", b, h, pos)
            do = upstream_rows(wl, b, h, pos)
            r = attention_backward_rows(q, pos, k, v, k_pos, do, wl.causal)
            dq[b, hi] = r["dq"]
            dk[b, g] += r["dk"]
            dv[b, g] += r["dv"]
    return {"dq": dq, "dk": dk, "dv": dv, "positions": pos, "heads": heads}
