"""GPU tests of the backward ring step against the oracle's gradients.

The small workloads run the forward and then the backward of every device
(the dK/dV accumulators of each block are shared by all devices, as they
would be after travelling the whole ring) and compare every element of dQ,
dK and dV with the oracle's gradient of full attention. A manual loop of
ring_attn_backward_step must give the driver's result bit for bit. The 128K
GQA share (and device 7 of the d64 numerics-stress share: logits with a
standard deviation near 16, 1 % duplicated keys) runs in the benchmark's
configuration and compares a seeded sample of dQ rows (tile and chunk
boundaries included) with the oracle, and checks
two identities that hold at any size for one device's dK/dV contribution:
sum over keys of dK = 0 and sum over keys of dV = sum over its rows of dO.

Tolerance (bf16 path): the kernels round P and dS to bf16 (relative error
2^-9 each) for the matrix products, and the row terms come from the bf16
forward output (O rounded to bf16, LSE within 1e-3). On the small workloads
errors are measured as max |GPU - oracle| / max |oracle| per tensor and must
stay below 2e-2, the forward's output tolerance (1e-5 for the fp32 path, which
computes in fp32 throughout, like the fp32 forward's bound). On the long rows of the 128K
share, D_i = dO_i . O_i computed from the bf16 output can cancel against
dP_ij (|D_i| up to ~30 next to |dQ_i| ~ 0.01), so dQ is held to a per-element
budget derived from those two roundings:
  scale (2^-7 A_i |sum_j P_ij k_j| + 2^-8 sum_j |dS_ij| |k_j|) + 2^-8 |dQ_i| + 1e-4,
with A_i = sum_d |dO_id| |O_id| bounding |D_i - D~_i| / 2^-7 (O off by at
most 2^-8 relative: its own bf16 rounding plus the forward's)."""
import numpy as np
import pytest

import oracle
import ring_inputs
import ring_attention_blockwise_amd as ra
from ring_attention_blockwise_amd import harness

pytestmark = pytest.mark.gpu

TOL_REL = {"bf16": 2e-2, "f32": 1e-5}
BW = ring_inputs.BACKWARD_WORKLOADS


def _copy_stream():
    import torch
    return torch.cuda.Stream()


def _rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.isfinite(got).all()
    return float(np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30))


def _all_devices(wl):
    import torch
    dev = torch.device("cuda:0")
    dk = dv = None
    dqs, shares = [], []
    for rank in range(wl.world):
        share = harness.build_share(wl, rank, dev)
        if dk is None:
            dk, dv = harness.new_kv_grads(share)
        cs = _copy_stream()
        out, lse = harness.run_forward(share, copy_stream=cs)
        d_out = harness.build_upstream(share)
        dqs.append(harness.run_backward(share, out, lse, d_out, dk, dv, copy_stream=cs))
        shares.append(share)
    torch.cuda.synchronize()
    return shares, dqs, dk, dv


@pytest.mark.parametrize("name", list(BW) + ["zigzag8k_8dev_d128", "ring4_noncausal_f32"])
def test_small_backward_every_element(gpu, name):
    wl = BW.get(name) or ring_inputs.WORKLOADS[name]
    shares, dqs, dk, dv = _all_devices(wl)
    full_dk = full_dv = 0.0
    err_dq = 0.0
    for rank in range(wl.world):
        ref = oracle.device_backward(wl, rank)
        full_dk = full_dk + ref["dk"]
        full_dv = full_dv + ref["dv"]
        err_dq = max(err_dq, _rel_err(dqs[rank].float().cpu().numpy(), ref["dq"]))
    err_dk = err_dv = 0.0
    for j in range(wl.world):
        pos = shares[j].q_positions
        err_dk = max(err_dk, _rel_err(dk[j].cpu().numpy(), full_dk[:, :, pos]))
        err_dv = max(err_dv, _rel_err(dv[j].cpu().numpy(), full_dv[:, :, pos]))
    print(f"  {name}: rel err dQ={err_dq:.3e} dK={err_dk:.3e} dV={err_dv:.3e}", flush=True)
    tol = TOL_REL[wl.dtype]
    assert err_dq <= tol and err_dk <= tol and err_dv <= tol


def test_step_loop_matches_driver_bitwise(gpu):
    """ring_attn_backward_step over the ring order, by hand, equals the driver."""
    import torch
    wl = BW["bwd_zigzag4k_4dev_gqa"]
    dev = torch.device("cuda:0")
    share = harness.build_share(wl, 1, dev)
    out, lse = harness.run_forward(share, copy_stream=_copy_stream())
    d_out = harness.build_upstream(share)
    dk_a, dv_a = harness.new_kv_grads(share)
    dq_a = harness.run_backward(share, out, lse, d_out, dk_a, dv_a, copy_stream=_copy_stream())

    rd = share.ring_desc()
    sd0, _ = ra.ring_step_desc(rd, 0)
    terms = torch.empty((2, wl.batch, wl.heads_q, wl.local_len), dtype=torch.float32, device=dev)
    ra.backward_prep(sd0, out, d_out, lse, terms)
    dq = torch.empty(share.q.shape, dtype=torch.float32, device=dev)
    dk_b, dv_b = harness.new_kv_grads(share)
    first = True
    for s in range(wl.world):
        sd, owner = ra.ring_step_desc(rd, s)
        if ra.visible_pairs(sd) == 0:
            continue
        ra.backward_step(sd, share.q, share.k_blocks[owner], share.v_blocks[owner], d_out, terms, dq,
                         dk_b[owner], dv_b[owner], init_dq=first)
        first = False
    torch.cuda.synchronize()
    assert torch.equal(dq.to(torch.bfloat16), dq_a)
    for j in range(wl.world):
        assert torch.equal(dk_a[j], dk_b[j]) and torch.equal(dv_a[j], dv_b[j])


def test_backward_is_deterministic_and_accumulates(gpu):
    """Two runs give identical bits; running a device twice doubles its dK/dV."""
    import torch
    wl = BW["bwd_striped2k_2dev_b2"]
    dev = torch.device("cuda:0")
    share = harness.build_share(wl, 0, dev)
    out, lse = harness.run_forward(share, copy_stream=_copy_stream())
    d_out = harness.build_upstream(share)
    dk1, dv1 = harness.new_kv_grads(share)
    dk2, dv2 = harness.new_kv_grads(share)
    dq1 = harness.run_backward(share, out, lse, d_out, dk1, dv1, copy_stream=_copy_stream())
    dq2 = harness.run_backward(share, out, lse, d_out, dk2, dv2, copy_stream=_copy_stream())
    harness.run_backward(share, out, lse, d_out, dk2, dv2, copy_stream=_copy_stream())
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2)
    for j in range(wl.world):
        assert torch.equal(2 * dk1[j], dk2[j]) and torch.equal(2 * dv1[j], dv2[j])


@pytest.mark.parametrize("name,rank", [("stress256k_8dev_d64", 7), ("zigzag128k_8dev_gqa", 0)])
def test_full_size_backward_is_deterministic(gpu, name, rank):
    """Repeated backward passes of a full-size share give the same bits in
    every row of dQ, dK and dV (a tile read before every wave's copy of it
    has landed would make some rows change from run to run)."""
    import torch
    wl = ring_inputs.WORKLOADS[name]
    share = harness.build_share(wl, rank, gpu)
    out, lse = harness.run_forward(share)
    d_out = harness.build_upstream(share)
    ref = None
    for rep in range(4):
        dk, dv = harness.new_kv_grads(share)
        dq = harness.run_backward(share, out, lse, d_out, dk, dv, copy_stream=_copy_stream())
        torch.cuda.synchronize()
        if ref is None:
            ref = (dq.clone(), [x.clone() for x in dk], [x.clone() for x in dv])
            continue
        assert torch.equal(dq, ref[0])
        assert all(torch.equal(a, b) for a, b in zip(dk, ref[1]))
        assert all(torch.equal(a, b) for a, b in zip(dv, ref[2]))


KEY_WINDOW = 1024      # sampled keys sit in the last KEY_WINDOW global positions
KEYS_PER_HEAD = 64
DQ_ROWS = 256


def _window_keys(wl, seed):
    """Global positions of the sampled keys: the last KEY_WINDOW positions
    hold them, at the in-tile offsets of the 128-key workgroup tiles there
    and seeded random ones, KEYS_PER_HEAD in all."""
    L = wl.total_len
    lo = L - KEY_WINDOW
    base = {lo, lo + 1, L - 2, L - 1}
    for t in (0, 3, 7):
        base |= {lo + 128 * t + o for o in (0, 1, 31, 32, 63, 64, 127)}
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(lo, L), np.fromiter(base, dtype=np.int64))
    base |= set(rng.choice(pool, size=KEYS_PER_HEAD - len(base), replace=False).tolist())
    return np.array(sorted(base), dtype=np.int64)


def _block_of_positions(wl):
    """global position -> (block, local key index) under the workload's partition."""
    where = np.zeros((wl.total_len, 2), dtype=np.int64)
    for j in range(wl.world):
        p = oracle.device_positions(wl.partition, wl.world, j, wl.local_len)
        where[p, 0] = j
        where[p, 1] = np.arange(wl.local_len)
    return where


@pytest.mark.parametrize("name,rank", [("zigzag128k_8dev_gqa", 0), ("stress256k_8dev_d64", 7)])
def test_full_size_backward_sampled_rows_keys_and_identities(gpu, name, rank):
    """dQ at sampled rows and dK/dV at sampled keys, element by element,
    against per-element error budgets; the sum identities over every key.

    A key's gradient needs the statistics of every row that sees it, so the
    sampled keys come from the last KEY_WINDOW positions of the sequence,
    which only the device's rows at those positions can see; the oracle
    computes those rows over all keys."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    import sampling
    wl = ring_inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    share = harness.build_share(wl, rank, dev)
    cs = _copy_stream()
    out, lse = harness.run_forward(share, copy_stream=cs)
    d_out = harness.build_upstream(share)
    dk, dv = harness.new_kv_grads(share)
    dq = harness.run_backward(share, out, lse, d_out, dk, dv, copy_stream=cs)
    torch.cuda.synchronize()

    c, L = wl.local_len, wl.total_len
    group = wl.heads_q // wl.heads_kv
    scale = 1.0 / np.sqrt(wl.head_dim)
    k_pos = np.arange(L)
    qpos = share.q_positions

    # dQ rows (tile and chunk boundaries included)
    rows = sampling.sample_rows(wl, seed=17, n_rows=DQ_ROWS)
    dq_np = dq[:, :, rows].float().cpu().numpy()
    # the key window: its keys, and the device rows that can see them
    keys = _window_keys(wl, seed=rank)
    where = _block_of_positions(wl)[keys]
    win_rows = np.nonzero(qpos >= keys.min())[0]
    assert 0 < len(win_rows) <= KEY_WINDOW
    dk_np = np.stack([dk[j][0, :, i].double().cpu().numpy() for j, i in where], axis=1)   # [Hkv, K, d]
    dv_np = np.stack([dv[j][0, :, i].double().cpu().numpy() for j, i in where], axis=1)

    def dq_job(g, h, sl, kh, vh):
        r_ = rows[sl]
        q = ring_inputs.rows(wl, "q", 0, h, qpos[r_])
        do = ring_inputs.rows(wl, "do", 0, h, qpos[r_])
        r = oracle.attention_backward_rows(q, qpos[r_], kh, vh, k_pos, do, True)
        a = (np.abs(do.astype(np.float64)) * np.abs(r["out"])).sum(axis=1, keepdims=True)
        budget = (scale * (2.0 ** -7 * a * np.abs(r["p_k"]) + 2.0 ** -8 * r["abs_ds_k"]) +
                  2.0 ** -8 * np.abs(r["dq"]) + 1e-4)
        got = dq_np[0, h, sl]
        assert np.isfinite(got).all()
        return float((np.abs(got - r["dq"]) / budget).max())

    def key_job(g, h, sl, kh, vh):
        r_ = win_rows[sl]
        q = ring_inputs.rows(wl, "q", 0, h, qpos[r_])
        do = ring_inputs.rows(wl, "do", 0, h, qpos[r_])
        return g, oracle.key_gradients(q, qpos[r_], kh, vh, k_pos, do, True, keys)

    from threadpoolctl import threadpool_limits
    dq_err = 0.0
    kg = {}
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(sampling.threads()) as ex:
        for g in range(wl.heads_kv):
            kh = ring_inputs.head(wl, "k", 0, g)
            vh = ring_inputs.head(wl, "v", 0, g)
            jobs_dq, jobs_k = [], []
            for h in range(g * group, (g + 1) * group):
                for r0 in range(0, len(rows), 32):
                    jobs_dq.append(ex.submit(dq_job, g, h, slice(r0, r0 + 32), kh, vh))
                for r0 in range(0, len(win_rows), 128):
                    jobs_k.append(ex.submit(key_job, g, h, slice(r0, r0 + 128), kh, vh))
            for j in jobs_dq:
                dq_err = max(dq_err, j.result())
            for j in jobs_k:
                gg, r = j.result()
                acc = kg.setdefault(gg, {})
                for key_, val in r.items():
                    acc[key_] = acc.get(key_, 0.0) + val
    dk_err = dv_err = 0.0
    for g in range(wl.heads_kv):
        r = kg[g]
        b_dk = scale * (2.0 ** -8 * r["abs_ds_q"] + 2.0 ** -7 * r["p_a_q"]) + 2.0 ** -8 * np.abs(r["dk"]) + 1e-6
        b_dv = 2.0 ** -7 * r["p_do"] + 2.0 ** -8 * np.abs(r["dv"]) + 1e-6
        assert np.isfinite(dk_np[g]).all() and np.isfinite(dv_np[g]).all()
        dk_err = max(dk_err, float((np.abs(dk_np[g] - r["dk"]) / b_dk).max()))
        dv_err = max(dv_err, float((np.abs(dv_np[g] - r["dv"]) / b_dv).max()))

    # Identities of one device's contribution, per KV head and column. Every
    # row's P~ sums to 1 within 2^-8 (LSE within 1e-3, bf16 rounding 2^-9),
    # so |sum dV - sum dO| <= 2^-8 sum |dO|; the dS~ of a row sum to D - D~,
    # far below 1 % of sum |dK| here.
    sum_dk = sum(x.double().sum(dim=2) for x in dk)          # [B, Hkv, d]
    sum_dv = sum(x.double().sum(dim=2) for x in dv)
    abs_dk = sum(x.double().abs().sum(dim=2) for x in dk)
    grouped = d_out.double().reshape(wl.batch, wl.heads_kv, group, wl.local_len, wl.head_dim)
    do_sum = grouped.sum(dim=(2, 3))
    do_abs = grouped.abs().sum(dim=(2, 3))
    id_dk = float((sum_dk.abs() / abs_dk).max())
    id_dv = float(((sum_dv - do_sum).abs() / do_abs).max())
    print(f"  {name}: dQ rows={len(rows)} x {wl.heads_q} heads: max err / budget {dq_err:.3f}; "
          f"dK/dV at {len(keys)} keys x {wl.heads_kv} KV heads ({len(win_rows)} rows see them): "
          f"max err / budget {dk_err:.3f} / {dv_err:.3f}; "
          f"|sum dK|/sum|dK| {id_dk:.3e}; |sum dV - sum dO|/sum|dO| {id_dv:.3e}", flush=True)
    assert dq_err <= 1.0 and dk_err <= 1.0 and dv_err <= 1.0
    assert id_dk <= 1e-2 and id_dv <= 2.0 ** -8


def _bwd_tensors(sd, dev, seed=5):
    import torch
    g = torch.Generator(device="cpu").manual_seed(seed)
    B, Hq, Hk, D = sd.batch, sd.heads_q, sd.heads_kv, sd.head_dim
    dt = torch.bfloat16 if sd.dtype == ra.BF16 else torch.float32
    mk = lambda *shape: torch.randn(*shape, generator=g).to(dev).to(dt)
    q, d_out = mk(B, Hq, sd.q_len, D), mk(B, Hq, sd.q_len, D)
    k, v = mk(B, Hk, sd.kv_len, D), mk(B, Hk, sd.kv_len, D)
    terms = torch.zeros((2, B, Hq, sd.q_len), dtype=torch.float32, device=dev)
    terms[0] = -8.0 / (sd.head_dim ** -0.5)  # LSE = 8 for every row
    return q, k, v, d_out, terms


def test_backward_step_edge_cases(gpu):
    """Empty shapes do nothing; a block that no row sees leaves dQ untouched
    (zeroes it with RA_BWD_INIT_DQ) and dK/dV untouched."""
    import torch
    dev = torch.device("cuda:0")
    f = torch.float32
    for dims in ((1, 4, 2, 128, 0, 64), (1, 4, 2, 128, 64, 0), (0, 4, 2, 128, 64, 64)):
        B, Hq, Hk, D, nq, nk = dims
        sd = ra.step_desc(B, Hq, Hk, D, nq, nk, causal=False)
        q, k, v, d_out, terms = _bwd_tensors(sd, dev)
        dq = torch.full((B, Hq, nq, D), 3.0, dtype=f, device=dev)
        dk = torch.full((B, Hk, nk, D), 5.0, dtype=f, device=dev)
        dv = torch.full((B, Hk, nk, D), 7.0, dtype=f, device=dev)
        ra.backward_step(sd, q, k, v, d_out, terms, dq, dk, dv, init_dq=False)
        torch.cuda.synchronize()
        assert bool((dq == 3.0).all()) and bool((dk == 5.0).all()) and bool((dv == 7.0).all())
    # causal: queries at positions 0..99, keys at 500..563 -> no visible pair
    sd = ra.step_desc(1, 4, 2, 128, 100, 64, q_segs=[(0, 100)], kv_segs=[(500, 64)])
    q, k, v, d_out, terms = _bwd_tensors(sd, dev)
    for init in (False, True):
        dq = torch.full((1, 4, 100, 128), 3.0, dtype=f, device=dev)
        dk = torch.full((1, 2, 64, 128), 5.0, dtype=f, device=dev)
        dv = torch.full((1, 2, 64, 128), 7.0, dtype=f, device=dev)
        ra.backward_step(sd, q, k, v, d_out, terms, dq, dk, dv, init_dq=init)
        torch.cuda.synchronize()
        assert bool((dq == (0.0 if init else 3.0)).all())
        assert bool((dk == 5.0).all()) and bool((dv == 7.0).all())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rows_without_keys_contribute_nothing(gpu, dtype):
    """A row whose forward saw no key (LSE = -inf, row term c = -inf) gets
    dQ = 0 and adds nothing to dK/dV: the result equals the same step with
    that row's dO set to zero."""
    import torch
    dev = torch.device("cuda:0")
    code = ra.BF16 if dtype == "bf16" else ra.F32
    sd = ra.step_desc(1, 2, 1, 128, 300, 200, dtype=code, q_segs=[(100, 300)], kv_segs=[(0, 200)])
    q, k, v, d_out, terms = _bwd_tensors(sd, dev)
    dead = [0, 17, 255, 299]
    t1 = terms.clone()
    t1[0, :, :, dead] = float("-inf")
    t1[1, :, :, dead] = 0.0
    d0 = d_out.clone()
    d0[:, :, dead] = 0
    f = torch.float32
    out = []
    for dd, tt in ((d_out, t1), (d0, t1)):
        dq = torch.empty((1, 2, 300, 128), dtype=f, device=dev)
        dk = torch.zeros((1, 1, 200, 128), dtype=f, device=dev)
        dv = torch.zeros((1, 1, 200, 128), dtype=f, device=dev)
        ra.backward_step(sd, q, k, v, dd, tt, dq, dk, dv, init_dq=True)
        out.append((dq, dk, dv))
    torch.cuda.synchronize()
    (dq_a, dk_a, dv_a), (dq_b, dk_b, dv_b) = out
    assert bool(torch.isfinite(dq_a).all()) and bool((dq_a[:, :, dead] == 0).all())
    assert torch.equal(dq_a, dq_b) and torch.equal(dk_a, dk_b) and torch.equal(dv_a, dv_b)
