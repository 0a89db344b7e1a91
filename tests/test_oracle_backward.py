"""Pins of the oracle's attention gradients against things other than itself.

Each test names what fixes the expected value: central finite differences of
the (separately pinned) forward oracle, PyTorch autograd in float64 on the
CPU, or an invariant of softmax attention. A dropped scale, a wrong sign in
dS, a D_i taken over the wrong axis, a transposed product, a mask applied to
the wrong side or a GQA sum over the wrong heads each fails at least one.
"""
import math

import numpy as np
import pytest

import oracle
import ring_inputs


def _case(rng, R, L, d, causal, q_scale=1.0):
    q = rng.standard_normal((R, d)) * q_scale
    k = rng.standard_normal((L, d)) * q_scale
    v = rng.standard_normal((L, d))
    do = rng.standard_normal((R, d))
    q_pos = np.sort(rng.choice(L, R, replace=False)) if causal else np.arange(R)
    return q, k, v, do, q_pos, np.arange(L)


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences_of_the_forward(causal):
    """dL/dx for L = sum(dO * O), by central differences of attention_rows."""
    rng = np.random.default_rng(11)
    q, k, v, do, q_pos, k_pos = _case(rng, 4, 6, 5, causal)
    g = oracle.attention_backward_rows(q, q_pos, k, v, k_pos, do, causal)

    def loss(qq, kk, vv):
        o, _ = oracle.attention_rows(qq, q_pos, kk, vv, k_pos, causal)
        return float((o * do).sum())

    h = 1e-6
    for name, x, grad in (("q", q, g["dq"]), ("k", k, g["dk"]), ("v", v, g["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                        loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        np.testing.assert_allclose(grad, num, atol=1e-8, rtol=1e-6, err_msg=name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("heads", [(1, 1), (4, 2), (6, 3)])
def test_matches_torch_autograd_with_gqa(causal, heads):
    import torch
    hq, hkv = heads
    rng = np.random.default_rng(12)
    L, R, d = 80, 48, 16
    q = rng.standard_normal((hq, R, d))
    k = rng.standard_normal((hkv, L, d))
    v = rng.standard_normal((hkv, L, d))
    do = rng.standard_normal((hq, R, d))
    q_pos = np.sort(rng.choice(L, R, replace=False))
    k_pos = np.arange(L)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    group = hq // hkv
    ke = tk.repeat_interleave(group, dim=0)
    ve = tv.repeat_interleave(group, dim=0)
    s = torch.matmul(tq, ke.transpose(1, 2).contiguous()) / math.sqrt(d)
    if causal:
        mask = torch.tensor(k_pos[None, :] <= q_pos[:, None])
        s = s.masked_fill(~mask, float("-inf"))
    out = torch.matmul(torch.softmax(s, dim=-1), ve)
    out.backward(torch.tensor(do))
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for h in range(hq):
        gh = oracle.kv_head_of(h, hq, hkv)
        r = oracle.attention_backward_rows(q[h], q_pos, k[gh], v[gh], k_pos, do[h], causal)
        np.testing.assert_allclose(r["dq"], tq.grad[h].numpy(), atol=1e-12, rtol=1e-10)
        dk[gh] += r["dk"]
        dv[gh] += r["dv"]
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12, rtol=1e-10)
    # the gradients of a few chosen keys alone, rows split in two parts
    pick = np.array([0, 1, 37, L - 2, L - 1, 50])
    dk_p = np.zeros((hkv, len(pick), d))
    dv_p = np.zeros((hkv, len(pick), d))
    for h in range(hq):
        gh = oracle.kv_head_of(h, hq, hkv)
        for rows in (slice(0, 20), slice(20, R)):
            r = oracle.key_gradients(q[h][rows], q_pos[rows], k[gh], v[gh], k_pos, do[h][rows], causal, pick)
            dk_p[gh] += r["dk"]
            dv_p[gh] += r["dv"]
    np.testing.assert_allclose(dk_p, tk.grad.numpy()[:, pick], atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dv_p, tv.grad.numpy()[:, pick], atol=1e-12, rtol=1e-10)


def test_invariants_of_softmax_attention():
    """Shifting every key by one vector leaves O unchanged, so sum_j dK_j = 0;
    each softmax row sums to one, so sum_j dV_j = sum_i dO_i; and
    D_i = sum_j P_ij dP_ij equals dO_i . O_i."""
    from scipy.special import softmax
    rng = np.random.default_rng(13)
    q, k, v, do, q_pos, k_pos = _case(rng, 64, 200, 32, True, q_scale=2.0)
    r = oracle.attention_backward_rows(q, q_pos, k, v, k_pos, do, True)
    np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-10)
    np.testing.assert_allclose(r["dv"].sum(axis=0), do.sum(axis=0), atol=1e-10)
    s = q @ k.T / math.sqrt(q.shape[1])
    s[k_pos[None, :] > q_pos[:, None]] = -np.inf
    p = softmax(s, axis=1)
    dp = do @ v.T
    np.testing.assert_allclose(r["delta"], (p * dp).sum(axis=1), atol=1e-10)


def test_error_terms():
    """p_k is attention with the keys as values; |dQ| <= scale * abs_ds_k
    (triangle inequality), with equality where every dS_ij k_j has one sign."""
    rng = np.random.default_rng(16)
    q, k, v, do, q_pos, k_pos = _case(rng, 16, 40, 8, True)
    r = oracle.attention_backward_rows(q, q_pos, k, v, k_pos, do, True)
    o_k, _ = oracle.attention_rows(q, q_pos, k, k, k_pos, True)
    np.testing.assert_allclose(r["p_k"], o_k, atol=1e-12)
    scale = 1 / math.sqrt(8)
    assert (np.abs(r["dq"]) <= scale * r["abs_ds_k"] + 1e-12).all()
    kp = np.abs(k)
    r2 = oracle.attention_backward_rows(q[:1], [39], kp, v, k_pos, do[:1], True)
    # one row, keys all positive: |sum_j dS_j k_j| < sum_j |dS_j| k_j unless dS has one sign (it never
    # does: the dS of a row sum to zero), so the bound is strict here
    assert (np.abs(r2["dq"]) < scale * r2["abs_ds_k"]).all()


def test_key_error_terms():
    """Over all keys, each row's softmax weights sum to one, so sum_j p_do_j =
    sum_i |dO_i| and sum_j p_a_q_j = sum_i A_i |q_i|; |dK_j| <= scale *
    abs_ds_q_j (triangle inequality), with equality for a single row (one
    term per key) and strict somewhere for many rows."""
    rng = np.random.default_rng(17)
    q, k, v, do, q_pos, k_pos = _case(rng, 24, 50, 8, True)
    q = np.abs(q)
    allk = np.arange(50)
    r = oracle.key_gradients(q, q_pos, k, v, k_pos, do, True, allk)
    out, _ = oracle.attention_rows(q, q_pos, k, v, k_pos, True)
    np.testing.assert_allclose(r["p_do"].sum(axis=0), np.abs(do).sum(axis=0), atol=1e-12)
    a = (np.abs(do) * np.abs(out)).sum(axis=1)
    np.testing.assert_allclose(r["p_a_q"].sum(axis=0), (a[:, None] * q).sum(axis=0), atol=1e-12)
    scale = 1 / math.sqrt(8)
    assert (np.abs(r["dk"]) <= scale * r["abs_ds_q"] + 1e-15).all()
    assert (np.abs(r["dk"]) < scale * r["abs_ds_q"] - 1e-6).any()
    one = oracle.key_gradients(q[:1], [49], k, v, k_pos, do[:1], True, allk)
    np.testing.assert_allclose(np.abs(one["dk"]), scale * one["abs_ds_q"], rtol=1e-12, atol=0)


def test_single_visible_key():
    """A causal row at position 0 sees only key 0: O_0 = v_0, so its dQ is
    zero, it adds dO_0 to dV_0 and nothing to dK."""
    rng = np.random.default_rng(14)
    q, k, v, do = (rng.standard_normal((1, 8)) for _ in range(4))
    kk = np.vstack([k, rng.standard_normal((3, 8))])
    vv = np.vstack([v, rng.standard_normal((3, 8))])
    r = oracle.attention_backward_rows(q, [0], kk, vv, np.arange(4), do, True)
    np.testing.assert_allclose(r["dq"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dk"], 0.0, atol=1e-15)
    np.testing.assert_allclose(r["dv"][0], do[0], atol=1e-15)
    np.testing.assert_allclose(r["dv"][1:], 0.0, atol=1e-15)


def test_row_without_visible_keys_contributes_nothing():
    rng = np.random.default_rng(15)
    q, k, v, do = (rng.standard_normal((2, 4)) for _ in range(4))
    r = oracle.attention_backward_rows(q, [5, 0], k, v, [1, 2], do, True)
    assert np.isfinite(r["dq"]).all() and np.isfinite(r["dk"]).all()
    np.testing.assert_allclose(r["dq"][1], 0.0)
    r1 = oracle.attention_backward_rows(q[:1], [5], k, v, [1, 2], do[:1], True)
    np.testing.assert_allclose(r["dk"], r1["dk"], atol=1e-15)
    np.testing.assert_allclose(r["dv"], r1["dv"], atol=1e-15)


@pytest.mark.parametrize("partition", ["contiguous", "zigzag", "striped"])
def test_device_parts_sum_to_the_full_gradient(partition):
    """The devices' parts of dK/dV add up to the gradient over all rows, and
    each device's dQ rows are the full gradient's rows at its positions."""
    wl = ring_inputs.Workload(name="tiny", batch=1, heads_q=4, heads_kv=2, head_dim=8, dtype="f32",
                              causal=True, partition=partition, world=4, local_len=8, seed=77)
    L = wl.total_len
    dk = np.zeros((1, 2, L, 8))
    dv = np.zeros((1, 2, L, 8))
    parts = [oracle.device_backward(wl, r) for r in range(wl.world)]
    for p in parts:
        dk += p["dk"]
        dv += p["dv"]
    pos = np.arange(L)
    for h in range(4):
        g = h // 2
        r = oracle.attention_backward_rows(ring_inputs.head(wl, "q", 0, h), pos, ring_inputs.head(wl, "k", 0, g),
                                           ring_inputs.head(wl, "v", 0, g), pos,
                                           ring_inputs.head(wl, "do", 0, h), True)
        dk[0, g] -= r["dk"]
        dv[0, g] -= r["dv"]
        for p in parts:
            np.testing.assert_allclose(p["dq"][0, h], r["dq"][p["positions"]], atol=1e-12)
    np.testing.assert_allclose(dk, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv, 0.0, atol=1e-12)


def test_upstream_gradient_is_its_own_stream():
    wl = ring_inputs.WORKLOADS["zigzag8k_8dev_d128"]
    do = ring_inputs.head(wl, "do", 0, 0)
    v = ring_inputs.head(wl, "v", 0, 0)
    assert not np.array_equal(do, v)
    assert abs(do.mean()) < 0.02 and abs(do.std() - 1.0) < 0.02
    np.testing.assert_array_equal(ring_inputs.round_to_bf16(do), do)
