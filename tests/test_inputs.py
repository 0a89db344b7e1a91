"""The seeded input generator: determinism, chunk independence, bf16 rounding, duplicates."""
import numpy as np
import pytest

import ring_inputs


def _small(**kw):
    base = dict(name="t", batch=1, heads_q=2, heads_kv=1, head_dim=8, dtype="bf16", causal=True,
                partition="zigzag", world=4, local_len=16, seed=11)
    base.update(kw)
    return ring_inputs.Workload(**base)


def test_same_seed_same_bytes_and_chunks_regenerate_alone():
    wl = _small()
    a = ring_inputs.head(wl, "k", 0, 0)
    b = ring_inputs.head(wl, "k", 0, 0)
    assert a.tobytes() == b.tobytes()
    g = wl.gen_chunk
    for c in range(wl.n_gen_chunks):
        np.testing.assert_array_equal(ring_inputs.chunks(wl, "k", 0, 0, [c]), a[c * g:(c + 1) * g])
    pos = np.array([3, 0, 31, 17, 63])
    np.testing.assert_array_equal(ring_inputs.rows(wl, "k", 0, 0, pos), a[pos])


def test_streams_differ_by_tensor_head_and_seed():
    wl = _small()
    q0 = ring_inputs.head(wl, "q", 0, 0)
    assert not np.array_equal(q0, ring_inputs.head(wl, "k", 0, 0))
    assert not np.array_equal(q0, ring_inputs.head(wl, "q", 0, 1))
    assert not np.array_equal(q0, ring_inputs.head(wl.with_(seed=12), "q", 0, 0))


def test_bf16_rounding_matches_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ours = ring_inputs.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(ours, ref)
    bits = ring_inputs.bf16_bits(ours)
    back = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(back, ours)


def test_bf16_values_are_exact_and_fp32_untouched():
    wl = _small()
    x = ring_inputs.head(wl, "q", 0, 0)
    np.testing.assert_array_equal(ring_inputs.round_to_bf16(x), x)
    xf = ring_inputs.head(wl.with_(dtype="f32"), "q", 0, 0)
    assert not np.array_equal(ring_inputs.round_to_bf16(xf), xf)


def test_distributions():
    wl = _small(world=8, local_len=4096, head_dim=64, qk_std=4.0, v_dist="uniform")
    q = ring_inputs.head(wl, "q", 0, 0)
    v = ring_inputs.head(wl, "v", 0, 0)
    assert abs(q.std() - 4.0) < 0.05 and abs(q.mean()) < 0.02
    assert v.min() >= -1.0 and v.max() <= 1.0 and abs(v.mean()) < 0.01


def test_duplicated_keys_create_exact_ties():
    wl = _small(world=8, local_len=2000, head_dim=16, dup_frac=0.01)
    k = ring_inputs.head(wl, "k", 0, 0)
    dst, src = ring_inputs.duplicate_plan(wl, 0, 0)
    assert len(dst) == int(0.01 * wl.total_len) == len(np.unique(dst))
    assert np.all(dst != src)
    raw = np.concatenate([ring_inputs._draw_chunk(wl, "k", 0, 0, c) for c in range(wl.n_gen_chunks)])
    np.testing.assert_array_equal(k[dst], raw[src])
    keep = np.setdiff1d(np.arange(wl.total_len), dst)
    np.testing.assert_array_equal(k[keep], raw[keep])


@pytest.mark.parametrize("name", sorted(ring_inputs.WORKLOADS))
def test_presets_are_consistent(name):
    wl = ring_inputs.WORKLOADS[name]
    assert wl.heads_q % wl.heads_kv == 0
    assert wl.local_len % 2 == 0
    assert all(0 <= r < wl.world for r in wl.ranks)
