"""Pins of the CPU oracle against things other than itself.

Each test names what fixes the expected value: a hand-worked example, a
closed form, a library routine (PyTorch / SciPy), or an invariant of the
method. Chosen so that a dropped scale, a wrong sign, a transposed operand,
an off-by-one causal mask, a wrong GQA head map or a wrong zigzag chunk
order each fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import ring_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- hand example
def test_hand_worked_example():
    g = _load("hand_example.json")
    q, k, v = (np.array(g[x]) for x in ("q", "k", "v"))
    o, lse = oracle.attention_rows(q, [5], k, v, [0, 1], causal=False)
    np.testing.assert_allclose(o, g["noncausal"]["out"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, g["noncausal"]["lse"], rtol=0, atol=1e-12)
    for case in ("causal_query_at_0", "causal_query_at_1"):
        c = g[case]
        o, lse = oracle.attention_rows(q, c["q_pos"], k, v, c["k_pos"], causal=True)
        np.testing.assert_allclose(o, c["out"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, c["lse"], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(0)
    L, d = 37, 8
    q = rng.standard_normal((L, d))
    key = rng.standard_normal(d)
    k = np.tile(key, (L, 1))
    v = rng.standard_normal((L, 5))
    pos = np.arange(L)
    o, lse = oracle.attention_rows(q, pos, k, v, pos, causal=True)
    for i in range(L):
        np.testing.assert_allclose(o[i], v[: i + 1].mean(axis=0), atol=1e-12)
        s = q[i] @ key / math.sqrt(d)
        assert abs(lse[i] - (s + math.log(i + 1))) < 1e-12


def test_causal_first_position_returns_first_value():
    rng = np.random.default_rng(1)
    L, d = 16, 4
    q, k, v = (rng.standard_normal((L, d)) for _ in range(3))
    pos = np.arange(L)
    o, lse = oracle.attention_rows(q, pos, k, v, pos, causal=True)
    np.testing.assert_array_equal(o[0], v[0])
    assert abs(lse[0] - q[0] @ k[0] / 2.0) < 1e-15


def test_constant_values_and_affine_equivariance():
    rng = np.random.default_rng(2)
    L, d = 20, 6
    q, k = rng.standard_normal((L, d)), rng.standard_normal((L, d))
    v = rng.standard_normal((L, d))
    pos = np.arange(L)
    c = rng.standard_normal(d)
    o_const, _ = oracle.attention_rows(q, pos, k, np.tile(c, (L, 1)), pos, causal=True)
    np.testing.assert_allclose(o_const, np.tile(c, (L, 1)), atol=1e-12)
    o, lse = oracle.attention_rows(q, pos, k, v, pos, causal=True)
    o2, lse2 = oracle.attention_rows(q, pos, k, 3.0 * v + c, pos, causal=True)
    np.testing.assert_allclose(o2, 3.0 * o + c, atol=1e-11)
    np.testing.assert_array_equal(lse2, lse)


def test_row_without_visible_keys():
    q = np.ones((1, 4))
    k = np.ones((3, 4))
    v = np.ones((3, 4))
    o, lse = oracle.attention_rows(q, [0], k, v, [1, 2, 3], causal=True)
    assert np.all(o == 0) and lse[0] == -np.inf


# ---------------------------------------------------------------- library routines
def _sdpa_reference(q, k, v, q_pos, k_pos, causal, heads_q, heads_kv):
    """torch float64 scaled_dot_product_attention with an explicit boolean mask."""
    import torch
    G = heads_q // heads_kv
    qt = torch.from_numpy(q)                        # [Hq, R, d]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)   # [Hq, L, d]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)
    if causal:
        mask = torch.from_numpy(k_pos[None, :] <= q_pos[:, None])
    else:
        mask = torch.ones(len(q_pos), len(k_pos), dtype=torch.bool)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    scores = (qt @ kt.transpose(-1, -2)) / math.sqrt(q.shape[-1])
    scores = scores.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    return out.numpy(), lse.numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2), (8, 2)])
def test_matches_torch_sdpa_with_gqa(causal, heads):
    hq, hkv = heads
    rng = np.random.default_rng(3)
    L, R, d = 96, 40, 16
    k = rng.standard_normal((hkv, L, d))
    v = rng.standard_normal((hkv, L, d))
    q_pos = np.sort(rng.choice(L, R, replace=False))
    q = rng.standard_normal((hq, R, d))
    k_pos = np.arange(L)
    ref_o, ref_lse = _sdpa_reference(q, k, v, q_pos, k_pos, causal, hq, hkv)
    for h in range(hq):
        g = oracle.kv_head_of(h, hq, hkv)
        o, lse = oracle.attention_rows(q[h], q_pos, k[g], v[g], k_pos, causal)
        np.testing.assert_allclose(o, ref_o[h], atol=1e-12, rtol=1e-12)
        np.testing.assert_allclose(lse, ref_lse[h], atol=1e-12, rtol=1e-12)
        # rows in shuffled order over several row groups (the causal key
        # prefix of each group is cut at its last visible position), and the
        # keys handed over in shuffled order (no prefix cut): same rows
        perm = rng.permutation(R)
        kperm = rng.permutation(L)
        for kk, vv, kp in ((k[g], v[g], k_pos), (k[g][kperm], v[g][kperm], k_pos[kperm])):
            o2, lse2 = oracle.attention_rows(q[h][perm], q_pos[perm], kk, vv, kp, causal, row_group=7)
            np.testing.assert_allclose(o2, ref_o[h][perm], atol=1e-12, rtol=1e-12)
            np.testing.assert_allclose(lse2, ref_lse[h][perm], atol=1e-12, rtol=1e-12)


def test_lse_matches_scipy_logsumexp_at_large_logits():
    from scipy.special import logsumexp
    rng = np.random.default_rng(4)
    L, d = 64, 16
    q = rng.standard_normal((8, d)) * 300.0
    k = rng.standard_normal((L, d)) * 300.0
    v = rng.standard_normal((L, d))
    pos = np.arange(L)
    o, lse = oracle.attention_rows(q, pos[:8] + 50, k, v, pos, causal=True)
    for i in range(8):
        s = q[i] @ k[: 51 + i].T / 4.0
        assert abs(lse[i] - logsumexp(s)) <= 1e-9 * max(1.0, abs(lse[i]))
        w = np.exp(s - s.max())
        np.testing.assert_allclose(o[i], (w / w.sum()) @ v[: 51 + i], atol=1e-12)
    assert np.all(np.isfinite(o))


# ---------------------------------------------------------------- brute force
def test_brute_force_tiny_cases():
    """Enumerate every visible (row, key) pair with math.exp, no numpy algebra."""
    rng = np.random.default_rng(5)
    for L in (1, 2, 3, 5, 8):
        for d in (1, 2, 4):
            for causal in (False, True):
                q = rng.standard_normal((L, d))
                k = rng.standard_normal((L, d))
                v = rng.standard_normal((L, d))
                perm = rng.permutation(L)          # query rows in arbitrary order
                o, lse = oracle.attention_rows(q[perm], perm, k, v, np.arange(L), causal)
                for a, i in enumerate(perm):
                    terms = []
                    for j in range(L):
                        if causal and j > i:
                            continue
                        dot = 0.0
                        for t in range(d):
                            dot += float(q[i, t]) * float(k[j, t])
                        terms.append((dot / math.sqrt(d), j))
                    top = max(t[0] for t in terms)
                    den = sum(math.exp(t[0] - top) for t in terms)
                    for c in range(d):
                        num = sum(math.exp(t[0] - top) * float(v[t[1], c]) for t in terms)
                        assert abs(o[a, c] - num / den) < 1e-12
                    assert abs(lse[a] - (top + math.log(den))) < 1e-12


# ---------------------------------------------------------------- method invariants
def _online_fold(q, q_pos, kv_blocks, causal, order):
    """The pages' block recurrence (section 6.2 of the hands-on code page),
    written here independently: running max M, sum L, unnormalised O."""
    d = q.shape[1]
    R = q.shape[0]
    M = np.full(R, -np.inf)
    Lsum = np.zeros(R)
    O = np.zeros((R, kv_blocks[0][2].shape[1]))
    for j in order:
        kpos, k, v = kv_blocks[j]
        S = q @ k.T / math.sqrt(d)
        if causal:
            S = np.where(kpos[None, :] <= q_pos[:, None], S, -np.inf)
        Mn = np.maximum(M, S.max(axis=1))
        safe = np.where(np.isfinite(Mn), Mn, 0.0)
        alpha = np.where(np.isfinite(M), np.exp(M - safe), 0.0)
        P = np.exp(S - safe[:, None])
        Lsum = Lsum * alpha + P.sum(axis=1)
        O = O * alpha[:, None] + P @ v
        M = Mn
    return O / Lsum[:, None], M + np.log(Lsum)


@pytest.mark.parametrize("partition", ["contiguous", "zigzag", "striped"])
def test_ring_of_blocks_equals_full_attention_in_any_order(partition):
    rng = np.random.default_rng(6)
    n, c, d = 4, 12, 8
    L = n * c
    q_all, k_all, v_all = (rng.standard_normal((L, d)) for _ in range(3))
    table = oracle.partition_table(partition, n, c)
    blocks = [(table[j], k_all[table[j]], v_all[table[j]]) for j in range(n)]
    for r in range(n):
        pos = table[r]
        o_ref, lse_ref = oracle.attention_rows(q_all[pos], pos, k_all, v_all, np.arange(L), True)
        code_order = [(r - s) % n for s in range(n)]
        text_order = [(r + s) % n for s in range(n)]
        for order in (code_order, text_order, list(rng.permutation(n))):
            o, lse = _online_fold(q_all[pos], pos, blocks, True, order)
            np.testing.assert_allclose(o, o_ref, atol=1e-12)
            np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_partitions_agree_per_global_row():
    wl = ring_inputs.Workload(name="t", batch=1, heads_q=2, heads_kv=1, head_dim=16, dtype="bf16",
                              causal=True, partition="zigzag", world=4, local_len=16, seed=7)
    by_pos = {}
    for part in ("zigzag", "contiguous", "striped"):
        w = wl.with_(partition=part)
        for r in range(w.world):
            res = oracle.device_share(w, r)
            for i, p in enumerate(res["positions"]):
                key = int(p)
                val = (res["out"][0, :, i], res["lse"][0, :, i])
                if key in by_pos:
                    np.testing.assert_allclose(val[0], by_pos[key][0], atol=1e-12)
                    np.testing.assert_allclose(val[1], by_pos[key][1], atol=1e-12)
                else:
                    by_pos[key] = val
    assert sorted(by_pos) == list(range(wl.total_len))


# ---------------------------------------------------------------- positions
def test_zigzag_positions_match_stated_chunks():
    g = _load("zigzag_8dev_chunks.json")
    for r, (a, b) in enumerate(g["device_chunks"]):
        pos = oracle.device_positions("zigzag", g["world"], r, g["local_len"])
        cl = g["chunk_len"]
        expect = np.concatenate([np.arange(a * cl, (a + 1) * cl), np.arange(b * cl, (b + 1) * cl)])
        np.testing.assert_array_equal(pos, expect)


def test_striped_positions_match_stated_tokens():
    """GPU 0 of a 4-GPU striped split holds tokens 0, 4, 8, ... (the page's
    example); together with every position being covered once, this fixes
    the stride and rules out a contiguous or zigzag map under that name."""
    g = _load("striped_4gpu_positions.json")
    for local_len in (3, 8, 64):
        pos = oracle.device_positions("striped", g["world"], g["rank"], local_len)
        np.testing.assert_array_equal(pos[:3], g["first_positions"])
        np.testing.assert_array_equal(np.diff(pos), np.full(local_len - 1, g["world"]))


@pytest.mark.parametrize("partition", ["contiguous", "zigzag", "striped"])
def test_partitions_cover_every_position_once(partition):
    t = oracle.partition_table(partition, 8, 32)
    assert sorted(t.ravel().tolist()) == list(range(256))


# ---------------------------------------------------------------- work counts
def test_visible_pairs_brute_force():
    rng = np.random.default_rng(8)
    for _ in range(20):
        qp = rng.integers(0, 50, size=rng.integers(1, 12))
        kp = rng.integers(0, 50, size=rng.integers(1, 12))
        brute = sum(1 for a in qp for b in kp if b <= a)
        assert oracle.visible_pair_count(qp, kp, True) == brute
        assert oracle.visible_pair_count(qp, kp, False) == len(qp) * len(kp)


def test_visible_pairs_closed_forms():
    for case in _load("work_counts.json")["cases"]:
        pos = oracle.device_positions(case["partition"], case["world"], case["rank"], case["local_len"])
        L = case["world"] * case["local_len"]
        assert oracle.visible_pair_count(pos, np.arange(L), True) == case["pairs_per_head"]


def test_zigzag_work_is_balanced_contiguous_is_not():
    n, c = 16, 64
    L = n * c
    z = [oracle.visible_pair_count(oracle.device_positions("zigzag", n, r, c), np.arange(L), True) for r in range(n)]
    assert len(set(z)) == 1 and z[0] * n == L * (L + 1) // 2
    cont = [oracle.visible_pair_count(oracle.device_positions("contiguous", n, r, c), np.arange(L), True)
            for r in range(n)]
    assert cont == sorted(cont) and cont[-1] > 1.9 * (sum(cont) / n)
