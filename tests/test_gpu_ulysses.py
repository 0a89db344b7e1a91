"""GPU tests of ring_attn_ulysses_forward (sequence <-> head all-to-all around
local attention) against the oracle.

The small workloads run every device and compare every row of every output
shard; they also check that Ulysses and the ring (same inputs, contiguous
partition) give the same attention. The 128K workload runs device 0, which
owns query heads 0-3 of every shard, and compares a seeded sample of
sequence positions (shard and tile boundaries always included)."""
import numpy as np
import pytest

import oracle
import ring_inputs
import ring_attention_blockwise_amd as ra
from ring_attention_blockwise_amd import harness

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "bf16": 2e-2}
TOL_LSE = 1e-3
U = ring_inputs.ULYSSES_WORKLOADS


def _desc(wl, rank):
    dtype = ra.BF16 if wl.dtype == "bf16" else ra.F32
    return ra.ulysses_desc(wl.batch, wl.heads_q, wl.heads_kv, wl.head_dim, wl.total_len, wl.world, rank,
                           dtype=dtype, causal=wl.causal)


def _outputs(wl, device):
    import torch
    dt = harness.torch_dtype(wl)
    shape = (wl.batch, wl.heads_q, wl.local_len)
    outs = [torch.full(shape + (wl.head_dim,), float("nan"), dtype=dt, device=device) for _ in range(wl.world)]
    lses = [torch.full(shape, float("nan"), dtype=torch.float32, device=device) for _ in range(wl.world)]
    return outs, lses


def _run(wl, ranks, q, k, v, outs, lses):
    import torch
    for rank in ranks:
        ud = _desc(wl, rank)
        ws = torch.empty(ra.ulysses_workspace_size(ud), dtype=torch.uint8, device=q[0].device)
        ra.ulysses_forward(ud, q, k, v, outs, lses, ws)
    torch.cuda.synchronize()


def _oracle_rows(wl, b, h, positions):
    """Full attention of query head h at global `positions` over the whole sequence."""
    g = h // (wl.heads_q // wl.heads_kv)
    k = ring_inputs.head(wl, "k", b, g)
    v = ring_inputs.head(wl, "v", b, g)
    q = ring_inputs.rows(wl, "q", b, h, positions)
    return oracle.attention_rows(q, positions, k, v, np.arange(wl.total_len), wl.causal)


@pytest.mark.parametrize("name", ["ulysses2k_4dev_gqa", "ulysses512_2dev_f32", "ulysses990_3dev_ragged"])
def test_small_ulysses_every_row(gpu, name):
    import torch
    wl = U[name]
    dev = torch.device("cuda:0")
    q, k, v = harness.build_ulysses_shards(wl, dev)
    outs, lses = _outputs(wl, dev)
    _run(wl, range(wl.world), q, k, v, outs, lses)
    out = torch.cat(outs, dim=2).double().cpu().numpy()  # [B, H, L, d] in token order
    lse = torch.cat(lses, dim=2).double().cpu().numpy()
    positions = np.arange(wl.total_len)
    err_o = err_l = 0.0
    for b in range(wl.batch):
        for h in range(wl.heads_q):
            ref_o, ref_l = _oracle_rows(wl, b, h, positions)
            err_o = max(err_o, np.abs(out[b, h] - ref_o).max())
            err_l = max(err_l, np.abs(lse[b, h] - ref_l).max())
    print(f"  {name}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert err_o <= TOL_O[wl.dtype], err_o
    assert err_l <= TOL_LSE, err_l


def test_ulysses_matches_ring_on_same_inputs(gpu):
    """The two sequence-parallel schemes compute the same attention: Ulysses
    shard j equals the ring's device j output (contiguous partition)."""
    import torch
    wl = U["ulysses2k_4dev_gqa"]
    dev = torch.device("cuda:0")
    q, k, v = harness.build_ulysses_shards(wl, dev)
    outs, lses = _outputs(wl, dev)
    _run(wl, range(wl.world), q, k, v, outs, lses)
    for rank in range(wl.world):
        share = harness.build_share(wl, rank, dev)
        assert torch.equal(share.q, q[rank])
        out_r, lse_r = harness.run_forward(share, copy_stream=torch.cuda.Stream())
        torch.cuda.synchronize()
        d_o = (out_r.double() - outs[rank].double()).abs().max().item()
        d_l = (lse_r.double() - lses[rank].double()).abs().max().item()
        print(f"  device {rank}: ring vs Ulysses max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}", flush=True)
        assert d_o <= TOL_O[wl.dtype] and d_l <= TOL_LSE


def test_ulysses_only_writes_its_heads(gpu):
    """A device writes its own heads of every shard and nothing else."""
    import torch
    wl = U["ulysses2k_4dev_gqa"]
    dev = torch.device("cuda:0")
    q, k, v = harness.build_ulysses_shards(wl, dev)
    outs, lses = _outputs(wl, dev)
    rank = 2
    _run(wl, [rank], q, k, v, outs, lses)
    hr = wl.heads_q // wl.world
    mine = slice(rank * hr, (rank + 1) * hr)
    rest = [h for h in range(wl.heads_q) if not (mine.start <= h < mine.stop)]
    for j in range(wl.world):
        assert torch.isfinite(outs[j][:, mine]).all() and torch.isfinite(lses[j][:, mine]).all()
        assert torch.isnan(outs[j][:, rest].float()).all() and torch.isnan(lses[j][:, rest]).all()


def test_full_size_ulysses_sampled_rows(gpu):
    import torch
    wl = U["ulysses128k_8dev_gqa"]
    dev = torch.device("cuda:0")
    rank = 0
    hr, hkr = wl.heads_q // wl.world, wl.heads_kv // wl.world
    heads = list(range(rank * hr, (rank + 1) * hr))
    q, k, v = harness.build_ulysses_shards(wl, dev, heads_q=heads, heads_kv=list(range(rank * hkr, (rank + 1) * hkr)))
    outs, lses = _outputs(wl, dev)
    _run(wl, [rank], q, k, v, outs, lses)
    c, L = wl.local_len, wl.total_len
    base = {0, 1, 63, 64, 255, 256, L - 1, L - 2, L - 256}
    for j in range(1, wl.world):
        base |= {j * c - 1, j * c, j * c + 1}
    rng = np.random.default_rng(7)
    positions = np.array(sorted(base | set(rng.choice(L, size=120, replace=False).tolist())), dtype=np.int64)
    out = torch.cat(outs, dim=2)[:, :, positions].double().cpu().numpy()
    lse = torch.cat(lses, dim=2)[:, :, positions].double().cpu().numpy()
    err_o = err_l = 0.0
    for h in heads:
        ref_o, ref_l = _oracle_rows(wl, 0, h, positions)
        err_o = max(err_o, np.abs(out[0, h] - ref_o).max())
        err_l = max(err_l, np.abs(lse[0, h] - ref_l).max())
    print(f"  rows={len(positions)} x {len(heads)} heads: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[wl.dtype], err_o
    assert err_l <= TOL_LSE, err_l
