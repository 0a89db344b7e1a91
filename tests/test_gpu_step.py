"""GPU tests of the step, merge and finalize kernels against the oracle on
small seeded inputs that span several tiles and a ragged tail, plus the
method's invariants and edge cases. All calls go through the C ABI."""
import math

import numpy as np
import pytest

import oracle
import ring_inputs
import ring_attention_blockwise_amd as ra
from ring_attention_blockwise_amd import harness

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-3


def _seeded(shape, seed, dtype, std=1.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(std)
    return ring_inputs.round_to_bf16(x) if dtype == "bf16" else x


def _tdt(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _dev(x, dtype, gpu):
    import torch
    return torch.from_numpy(x).to(gpu).to(_tdt(dtype)).contiguous()


def _case(gpu, dtype, d, hq, hkv, q_segs, kv_segs, causal, seed=0, B=1):
    """Run init-step + finalize on the GPU and the oracle on the same inputs."""
    import torch
    nq = sum(s[1] for s in q_segs)
    nk = sum(s[1] for s in kv_segs)
    q = _seeded((B, hq, nq, d), seed, dtype)
    k = _seeded((B, hkv, nk, d), seed + 1, dtype)
    v = _seeded((B, hkv, nk, d), seed + 2, dtype)
    code = ra.BF16 if dtype == "bf16" else ra.F32
    sd = ra.step_desc(B, hq, hkv, d, nq, nk, dtype=code, causal=causal, q_segs=q_segs, kv_segs=kv_segs)
    o = torch.empty((B, hq, nq, d), dtype=torch.float32, device=gpu)
    m = torch.empty((B, hq, nq), dtype=torch.float32, device=gpu)
    l = torch.empty_like(m)
    ra.step(sd, _dev(q, dtype, gpu), _dev(k, dtype, gpu), _dev(v, dtype, gpu), o, m, l, init=True)
    out = torch.empty((B, hq, nq, d), dtype=_tdt(dtype), device=gpu)
    lse = torch.empty((B, hq, nq), dtype=torch.float32, device=gpu)
    ra.finalize(sd, o, m, l, out, lse)
    torch.cuda.synchronize()
    qp, kp = harness.positions(q_segs), harness.positions(kv_segs)
    ref_o = np.zeros((B, hq, nq, d))
    ref_l = np.zeros((B, hq, nq))
    for b in range(B):
        for h in range(hq):
            g = oracle.kv_head_of(h, hq, hkv)
            ref_o[b, h], ref_l[b, h] = oracle.attention_rows(q[b, h], qp, k[b, g], v[b, g], kp, causal)
    return out.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l, (o, m, l)


def _assert_close(out, lse, ref_o, ref_l, dtype):
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.all(out[~fin] == 0)
    err_o = np.abs(out - ref_o).max() if out.size else 0.0
    err_l = np.abs(lse[fin] - ref_l[fin]).max() if fin.any() else 0.0
    assert err_o <= TOL_O[dtype], f"max |O - oracle| = {err_o}"
    assert err_l <= TOL_LSE, f"max |LSE - oracle| = {err_l}"


SEGMENT_CASES = [
    # (q segments, kv segments) — global positions (start, len[, stride])
    ([(0, 200)], [(0, 200)]),                              # diagonal block, ragged tail
    ([(300, 120), (900, 81)], [(0, 150), (850, 183)]),     # two segments each, partial overlap
    ([(1000, 130)], [(0, 333)]),                           # all keys before all queries (full)
    ([(0, 64)], [(64, 64)]),                               # every key after every query
    ([(5, 97, 4)], [(0, 77, 5)]),                          # strided positions
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("segs", range(len(SEGMENT_CASES)))
def test_step_matches_oracle(gpu, dtype, d, causal, segs):
    q_segs, kv_segs = SEGMENT_CASES[segs]
    out, lse, ro, rl, _ = _case(gpu, dtype, d, 4, 2, q_segs, kv_segs, causal, seed=10 * segs + d)
    _assert_close(out, lse, ro, rl, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch_and_gqa_group_of_eight(gpu, dtype):
    out, lse, ro, rl, _ = _case(gpu, dtype, 128, 8, 1, [(200, 257)], [(0, 390)], True, seed=3, B=2)
    _assert_close(out, lse, ro, rl, dtype)


def test_many_tiles_long_rows(gpu):
    out, lse, ro, rl, _ = _case(gpu, "bf16", 128, 2, 2, [(1500, 300)], [(0, 1700)], True, seed=4)
    _assert_close(out, lse, ro, rl, "bf16")


def test_large_logits_do_not_overflow(gpu):
    """Logits of order 1e3 exercise the lazy rescale and the -inf guards."""
    import torch
    d, n = 64, 300
    q = _seeded((1, 1, n, d), 5, "bf16", std=12.0)
    k = _seeded((1, 1, n, d), 6, "bf16", std=12.0)
    v = _seeded((1, 1, n, d), 7, "bf16")
    sd = ra.step_desc(1, 1, 1, d, n, n, q_segs=[(0, n)], kv_segs=[(0, n)])
    o = torch.empty((1, 1, n, d), dtype=torch.float32, device=gpu)
    m = torch.empty((1, 1, n), dtype=torch.float32, device=gpu)
    l = torch.empty_like(m)
    ra.step(sd, _dev(q, "bf16", gpu), _dev(k, "bf16", gpu), _dev(v, "bf16", gpu), o, m, l, init=True)
    out = torch.empty((1, 1, n, d), dtype=torch.bfloat16, device=gpu)
    lse = torch.empty((1, 1, n), dtype=torch.float32, device=gpu)
    ra.finalize(sd, o, m, l, out, lse)
    ro, rl = oracle.attention_rows(q[0, 0], np.arange(n), k[0, 0], v[0, 0], np.arange(n), True)
    assert torch.isfinite(out.float()).all()
    _assert_close(out.double().cpu().numpy()[0, 0], lse.double().cpu().numpy()[0, 0], ro, rl, "bf16")


# ---------------------------------------------------------------- edge cases
def test_empty_block_with_init_gives_empty_state(gpu):
    import torch
    for dtype in ("f32", "bf16"):
        sd = ra.step_desc(1, 2, 1, 64, 40, 0, dtype=ra.BF16 if dtype == "bf16" else ra.F32,
                          q_segs=[(0, 40)], kv_segs=[(0, 0)])
        o = torch.full((1, 2, 40, 64), 7.0, device=gpu)
        m = torch.full((1, 2, 40), 7.0, device=gpu)
        l = torch.full((1, 2, 40), 7.0, device=gpu)
        q = torch.zeros((1, 2, 40, 64), dtype=_tdt(dtype), device=gpu)
        kv = torch.zeros((1, 1, 0, 64), dtype=_tdt(dtype), device=gpu)
        ra.step(sd, q, kv, kv, o, m, l, init=True)
        assert (o == 0).all() and (l == 0).all() and torch.isneginf(m).all()
        out = torch.empty((1, 2, 40, 64), dtype=_tdt(dtype), device=gpu)
        lse = torch.empty((1, 2, 40), device=gpu)
        ra.finalize(sd, o, m, l, out, lse)
        assert (out.float() == 0).all() and torch.isneginf(lse).all()


def test_fully_masked_step_leaves_state_untouched(gpu):
    import torch
    _, _, _, _, (o, m, l) = _case(gpu, "bf16", 128, 2, 2, [(100, 100)], [(0, 150)], True)
    o0, m0, l0 = o.clone(), m.clone(), l.clone()
    q = torch.randn((1, 2, 100, 128), device=gpu).to(torch.bfloat16)
    kv = torch.randn((1, 2, 64, 128), device=gpu).to(torch.bfloat16)
    sd = ra.step_desc(1, 2, 2, 128, 100, 64, q_segs=[(100, 100)], kv_segs=[(500, 64)])
    assert ra.visible_pairs(sd) == 0
    ra.step(sd, q, kv, kv, o, m, l)
    torch.cuda.synchronize()
    assert torch.equal(o, o0) and torch.equal(m, m0) and torch.equal(l, l0)


def test_rows_without_visible_keys_finalize_to_zero(gpu):
    # queries at 0..99 against keys 50..149: rows 0..49 see nothing
    out, lse, ro, rl, _ = _case(gpu, "bf16", 64, 1, 1, [(0, 100)], [(50, 100)], True)
    assert np.isneginf(lse[0, 0, :50]).all() and (out[0, 0, :50] == 0).all()
    _assert_close(out, lse, ro, rl, "bf16")


def test_zero_query_rows_is_a_no_op(gpu):
    import torch
    sd = ra.step_desc(1, 1, 1, 64, 0, 10, q_segs=[(0, 0)], kv_segs=[(0, 10)])
    e = torch.empty((1, 1, 0, 64), dtype=torch.bfloat16, device=gpu)
    kv = torch.zeros((1, 1, 10, 64), dtype=torch.bfloat16, device=gpu)
    f = torch.empty((1, 1, 0), device=gpu)
    ra.step(sd, e, kv, kv, e.float(), f, f, init=True)


# ---------------------------------------------------------------- merge
def _state_for(gpu, q, k, v, q_segs, kv_segs, causal=True, dtype="bf16"):
    import torch
    B, hq, nq, d = q.shape
    hkv, nk = k.shape[1], k.shape[2]
    code = ra.BF16 if dtype == "bf16" else ra.F32
    sd = ra.step_desc(B, hq, hkv, d, nq, nk, dtype=code, causal=causal, q_segs=q_segs, kv_segs=kv_segs)
    o = torch.empty((B, hq, nq, d), dtype=torch.float32, device=gpu)
    m = torch.empty((B, hq, nq), dtype=torch.float32, device=gpu)
    l = torch.empty_like(m)
    ra.step(sd, _dev(q, dtype, gpu), _dev(np.ascontiguousarray(k), dtype, gpu),
            _dev(np.ascontiguousarray(v), dtype, gpu), o, m, l, init=True)
    return o, m, l


def test_merge_is_commutative_bitwise_and_associative(gpu):
    import torch
    d, n, nk = 128, 260, 720
    q = _seeded((1, 2, n, d), 20, "bf16")
    k = _seeded((1, 2, nk, d), 21, "bf16")
    v = _seeded((1, 2, nk, d), 22, "bf16")
    cuts = [(0, 300), (300, 550), (550, 720)]
    qs = [(600, n)]
    states = [_state_for(gpu, q, k[:, :, a:b], v[:, :, a:b], qs, [(a, b - a)]) for a, b in cuts]
    sd = ra.step_desc(1, 2, 2, d, n, 1, q_segs=qs, kv_segs=[(0, 1)])

    def merged(a, b):
        o, m, l = (x.clone() for x in a)
        ra.merge(sd, o, m, l, *b)
        return o, m, l

    ab, ba = merged(states[0], states[1]), merged(states[1], states[0])
    for x, y in zip(ab, ba):
        assert torch.equal(x, y)
    left = merged(merged(states[0], states[1]), states[2])
    right = merged(states[0], merged(states[1], states[2]))
    out_l, lse_l = torch.empty((1, 2, n, d), dtype=torch.bfloat16, device=gpu), torch.empty((1, 2, n), device=gpu)
    out_r, lse_r = torch.empty_like(out_l), torch.empty_like(lse_l)
    ra.finalize(sd, *left, out_l, lse_l)
    ra.finalize(sd, *right, out_r, lse_r)
    assert (out_l.float() - out_r.float()).abs().max().item() <= 1e-2
    assert (lse_l - lse_r).abs().max().item() <= 1e-5
    # the merge of the three partial states is full attention over all keys
    qp = harness.positions(qs)
    ro = np.zeros((1, 2, n, d))
    rl = np.zeros((1, 2, n))
    for h in range(2):
        ro[0, h], rl[0, h] = oracle.attention_rows(q[0, h], qp, k[0, h], v[0, h], np.arange(nk), True)
    _assert_close(out_l.double().cpu().numpy(), lse_l.double().cpu().numpy(), ro, rl, "bf16")


def test_merge_with_empty_state_is_identity(gpu):
    import torch
    q = _seeded((1, 1, 90, 64), 30, "f32")
    k = _seeded((1, 1, 120, 64), 31, "f32")
    v = _seeded((1, 1, 120, 64), 32, "f32")
    o, m, l = _state_for(gpu, q, k, v, [(100, 90)], [(0, 120)], dtype="f32")
    sd = ra.step_desc(1, 1, 1, 64, 90, 1, dtype=ra.F32, q_segs=[(100, 90)], kv_segs=[(0, 1)])
    eo, em, el = torch.zeros_like(o), torch.full_like(m, float("-inf")), torch.zeros_like(l)
    a = [x.clone() for x in (o, m, l)]
    ra.merge(sd, *a, eo, em, el)
    for x, y in zip(a, (o, m, l)):
        assert torch.equal(x, y)
    ra.merge(sd, eo, em, el, o, m, l)
    for x, y in zip((eo, em, el), (o, m, l)):
        assert torch.equal(x, y)
