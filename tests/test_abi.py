"""The C-ABI library on the host: it loads, exports every symbol the header
declares, its host-only helpers agree with the oracle's independent code, and
invalid arguments are rejected before any GPU work (nothing is launched)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import ring_attention_blockwise_amd as ra

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ring_attn.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ring_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ra.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", ra.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ring_attn_\w+)", nm))
    assert set(names) <= exported
    assert set(ra.EXPORTED) == set(names)


def test_abi_version():
    assert ra.lib().ring_attn_abi_version() == 104


def _expand(segs):
    return np.concatenate([np.arange(s, s + n * st, st) for s, n, st in segs]) if segs else np.zeros(0, int)


@pytest.mark.parametrize("partition", ["contiguous", "zigzag", "striped"])
@pytest.mark.parametrize("world,local", [(1, 8), (4, 16), (8, 1024), (64, 16384)])
def test_partition_segments_match_oracle_positions(partition, world, local):
    for rank in sorted({0, world // 2, world - 1}):
        segs = ra.partition_segments(partition, world, rank, local)
        np.testing.assert_array_equal(_expand(segs), oracle.device_positions(partition, world, rank, local))


@pytest.mark.parametrize("partition", ["contiguous", "zigzag", "striped"])
def test_visible_pairs_match_oracle_count(partition):
    n, c = 8, 48
    L = n * c
    for rank in range(n):
        for reverse in (False, True):
            rd = ra.ring_desc(1, 2, 1, 64, c, n, rank, partition, reverse_order=reverse)
            total = 0
            for s in range(n):
                sd, owner = ra.ring_step_desc(rd, s)
                qp = oracle.device_positions(partition, n, rank, c)
                kp = oracle.device_positions(partition, n, owner, c)
                assert ra.visible_pairs(sd) == oracle.visible_pair_count(qp, kp, True)
                total += ra.visible_pairs(sd)
            assert total == oracle.visible_pair_count(oracle.device_positions(partition, n, rank, c),
                                                      np.arange(L), True)


def test_visible_pairs_random_segments():
    rng = np.random.default_rng(0)
    for _ in range(200):
        segs_q = [(int(rng.integers(0, 50)), int(rng.integers(0, 20)), int(rng.integers(1, 4)))
                  for _ in range(int(rng.integers(1, 3)))]
        segs_k = [(int(rng.integers(0, 50)), int(rng.integers(0, 20)), int(rng.integers(1, 4)))
                  for _ in range(int(rng.integers(1, 3)))]
        nq = sum(s[1] for s in segs_q)
        nk = sum(s[1] for s in segs_k)
        sd = ra.step_desc(1, 1, 1, 64, nq, nk, causal=True, q_segs=segs_q, kv_segs=segs_k)
        assert ra.visible_pairs(sd) == oracle.visible_pair_count(_expand(segs_q), _expand(segs_k), True)
    sd = ra.step_desc(1, 1, 1, 64, 7, 5, causal=False)
    assert ra.visible_pairs(sd) == 35


def test_ring_step_owner_order():
    rd = ra.ring_desc(1, 1, 1, 64, 16, 4, 1)
    assert [ra.ring_step_desc(rd, s)[1] for s in range(4)] == [1, 0, 3, 2]
    rd = ra.ring_desc(1, 1, 1, 64, 16, 4, 1, reverse_order=True)
    assert [ra.ring_step_desc(rd, s)[1] for s in range(4)] == [1, 2, 3, 0]


def test_workspace_size_covers_slots_and_state():
    rd = ra.ring_desc(1, 32, 8, 128, 16384, 8, 0)
    ws = ra.forward_workspace_size(rd)
    block = 8 * 16384 * 128 * 2
    state = 32 * 16384 * (128 * 4 + 8)
    assert 4 * block + state <= ws <= 4 * block + state + 8 * 256


# ---- validation: errors come back before anything is enqueued -------------------
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced on the host


def _step_rc(sd, ptrs=(FAKE,) * 6, flags=0):
    return ra.lib().ring_attn_step(ctypes.byref(sd), *ptrs, flags, None)


@pytest.mark.parametrize("field,value,code", [
    ("head_dim", 96, ra.ERR_UNSUPPORTED), ("dtype", 7, ra.ERR_UNSUPPORTED),
    ("heads_kv", 3, ra.ERR_INVALID_ARG), ("heads_q", 0, ra.ERR_INVALID_ARG),
    ("batch", -1, ra.ERR_INVALID_ARG), ("q_len", -5, ra.ERR_INVALID_ARG),
    ("causal", 2, ra.ERR_INVALID_ARG), ("scale", float("nan"), ra.ERR_INVALID_ARG),
])
def test_step_rejects_bad_descriptor(field, value, code):
    sd = ra.step_desc(1, 4, 2, 128, 16, 16, q_segs=[(0, 16)], kv_segs=[(0, 16)])
    setattr(sd, field, value)
    assert _step_rc(sd) == code
    assert ra.last_error() != ""


def test_step_rejects_bad_segments_and_pointers():
    sd = ra.step_desc(1, 1, 1, 64, 16, 16, q_segs=[(0, 15)], kv_segs=[(0, 16)])
    assert _step_rc(sd) == ra.ERR_INVALID_ARG and "add up" in ra.last_error()
    sd = ra.step_desc(1, 1, 1, 64, 16, 16, q_segs=[(0, 16, 0)], kv_segs=[(0, 16)])
    assert _step_rc(sd) == ra.ERR_INVALID_ARG
    sd = ra.step_desc(1, 1, 1, 64, 16, 16, causal=True)          # causal without positions
    assert _step_rc(sd) == ra.ERR_INVALID_ARG
    sd = ra.step_desc(1, 1, 1, 64, 16, 16, q_segs=[(0, 16)], kv_segs=[(0, 16)])
    assert _step_rc(sd, (None,) + (FAKE,) * 5) == ra.ERR_INVALID_ARG
    assert _step_rc(sd, (ctypes.c_void_p(0x10004),) + (FAKE,) * 5) == ra.ERR_INVALID_ARG  # misaligned
    assert _step_rc(sd, flags=4) == ra.ERR_INVALID_ARG
    empty = ra.step_desc(1, 1, 1, 64, 0, 16, q_segs=[(0, 0)], kv_segs=[(0, 16)])
    assert _step_rc(empty, (None,) * 6) == ra.OK                 # no rows: nothing to do


def test_merge_finalize_reject_bad_arguments():
    L = ra.lib()
    sd = ra.step_desc(1, 1, 1, 96, 16, 16, causal=False)
    assert L.ring_attn_merge(ctypes.byref(sd), *(FAKE,) * 6, None) == ra.ERR_UNSUPPORTED
    assert L.ring_attn_finalize(ctypes.byref(sd), *(FAKE,) * 5, None) == ra.ERR_UNSUPPORTED
    sd = ra.step_desc(1, 1, 1, 64, 16, 16, causal=False)
    assert L.ring_attn_merge(ctypes.byref(sd), None, *(FAKE,) * 5, None) == ra.ERR_INVALID_ARG
    assert L.ring_attn_finalize(ctypes.byref(sd), FAKE, FAKE, FAKE, None, None, None) == ra.ERR_INVALID_ARG


def test_forward_rejects_small_workspace_and_bad_desc():
    L = ra.lib()
    rd = ra.ring_desc(1, 2, 1, 64, 16, 4, 0)
    blocks = (ctypes.c_void_p * 4)(*([0x10000] * 4))
    ws = ra.forward_workspace_size(rd)
    rc = L.ring_attn_forward(ctypes.byref(rd), FAKE, blocks, blocks, FAKE, FAKE, FAKE, ws - 1, None, None, None)
    assert rc == ra.ERR_WORKSPACE
    rc = L.ring_attn_forward(ctypes.byref(rd), FAKE, blocks, blocks, FAKE, FAKE, None, ws, None, None, None)
    assert rc == ra.ERR_WORKSPACE
    bad = ra.ring_desc(1, 2, 1, 64, 15, 4, 0, partition="zigzag")   # odd local length
    assert L.ring_attn_forward(ctypes.byref(bad), FAKE, blocks, blocks, FAKE, FAKE, FAKE, ws, None, None,
                               None) == ra.ERR_INVALID_ARG
    bad = ra.ring_desc(1, 2, 1, 64, 16, 4, 4)                      # rank out of range
    assert ra.lib().ring_attn_forward_workspace_size(ctypes.byref(bad)) == 0
    for recv in (-1, 3):                                           # unknown receive mode
        bad = ra.ring_desc(1, 2, 1, 64, 16, 4, 0, receive=recv)
        assert ra.lib().ring_attn_forward_workspace_size(ctypes.byref(bad)) == 0
        assert L.ring_attn_forward(ctypes.byref(bad), FAKE, blocks, blocks, FAKE, FAKE, FAKE, ws, None, None,
                                   None) == ra.ERR_INVALID_ARG
    for recv in ("auto", "memcpy", "fused"):
        assert ra.forward_workspace_size(ra.ring_desc(1, 2, 1, 64, 16, 4, 0, receive=recv)) == ws
    nulls = (ctypes.c_void_p * 4)(*([0x10000] * 3 + [None]))
    assert L.ring_attn_forward(ctypes.byref(rd), FAKE, blocks, nulls, FAKE, FAKE, FAKE, ws, None, None,
                               None) == ra.ERR_INVALID_ARG
    same = ctypes.c_void_p(0x5000)
    assert L.ring_attn_forward(ctypes.byref(rd), FAKE, blocks, blocks, FAKE, FAKE, FAKE, ws, same, same,
                               None) == ra.ERR_INVALID_ARG


def test_key_split_workspace_and_validation():
    """The key split's partial states are sized into the forward workspace:
    k fp32 states (O, m, l) for a split of k; automatic only for small bf16
    shares; a given k is capped at the block's key tiles; out-of-range values
    are rejected before anything is enqueued."""
    L = ra.lib()
    blocks = (ctypes.c_void_p * 8)(*([0x10000] * 8))
    ws = ctypes.c_size_t(1 << 40)

    def size(**kw):
        return ra.forward_workspace_size(ra.ring_desc(1, 8, 8, 128, 1024, 8, 0, **kw))

    rows = 8 * 1024
    def parts(k):
        return k * rows * 128 * 4 + 2 * k * rows * 4   # every region is a multiple of 256 bytes here

    base = size(key_split=1)
    assert size() == base + parts(8)                       # 32 work items: split 8 ways (2 key tiles each)
    assert size(key_split=2) == base + parts(2)
    assert size(key_split=16) == base + parts(16)          # 16 key tiles: one each
    # a 256-row block has 4 key tiles: 16 is capped at 4
    assert (ra.forward_workspace_size(ra.ring_desc(1, 8, 8, 128, 256, 8, 0, key_split=16))
            - ra.forward_workspace_size(ra.ring_desc(1, 8, 8, 128, 256, 8, 0, key_split=1))) == 4 * 2048 * 520
    # fp32 never splits; 128K/8 GQA (2048 work items) is not split automatically
    assert ra.forward_workspace_size(ra.ring_desc(1, 8, 8, 128, 1024, 8, 0, dtype=ra.F32, key_split=8)) == \
        ra.forward_workspace_size(ra.ring_desc(1, 8, 8, 128, 1024, 8, 0, dtype=ra.F32))
    big = dict(batch=1, heads_q=32, heads_kv=8, head_dim=128, local_len=16384, world=8, rank=0)
    assert ra.forward_workspace_size(ra.ring_desc(**big)) == ra.forward_workspace_size(ra.ring_desc(**big, key_split=1))
    for k in (-1, 17):
        bad = ra.ring_desc(1, 8, 8, 128, 1024, 8, 0, key_split=k)
        assert L.ring_attn_forward_workspace_size(ctypes.byref(bad)) == 0
        assert L.ring_attn_forward(ctypes.byref(bad), FAKE, blocks, blocks, FAKE, FAKE, FAKE, ws, None, None,
                                   None) == ra.ERR_INVALID_ARG
        assert "key_split" in ra.last_error()
    # the split share still fits the no-allocation forward's scratch
    assert size() - 256 <= ra.NOALLOC_SCRATCH_BYTES


def test_ulysses_workspace_and_validation():
    """Head counts and sequence length must divide by world; bad arguments are
    rejected on the host before anything is enqueued."""
    L = ra.lib()
    ud = ra.ulysses_desc(1, 8, 4, 128, 2048, 4, 1)
    ws = ra.ulysses_workspace_size(ud)
    # this device: 2 Q heads and 1 KV head over all 2048 tokens (Q, K, V, out bf16, LSE fp32)
    assert ws >= (2 + 1 + 1 + 2) * 2048 * 128 * 2 + 2 * 2048 * 4
    for bad in (ra.ulysses_desc(1, 8, 4, 128, 2048, 8, 0),   # 4 KV heads over 8 devices
                ra.ulysses_desc(1, 6, 3, 128, 2048, 4, 0),   # 6 Q heads over 4 devices
                ra.ulysses_desc(1, 8, 4, 128, 2050, 4, 0),   # 2050 tokens over 4 devices
                ra.ulysses_desc(1, 8, 4, 128, 2048, 4, 4),   # rank out of range
                ra.ulysses_desc(1, 8, 4, 96, 2048, 4, 0)):   # head_dim not 64 or 128
        assert L.ring_attn_ulysses_workspace_size(ctypes.byref(bad)) == 0
    shards = (ctypes.c_void_p * 4)(*([0x10000] * 4))
    rc = L.ring_attn_ulysses_forward(ctypes.byref(ud), shards, shards, shards, shards, None, FAKE, ws - 1, None)
    assert rc == ra.ERR_WORKSPACE
    nulls = (ctypes.c_void_p * 4)(*([0x10000] * 3 + [None]))
    rc = L.ring_attn_ulysses_forward(ctypes.byref(ud), shards, nulls, shards, shards, None, FAKE, ws, None)
    assert rc == ra.ERR_INVALID_ARG
    misaligned = (ctypes.c_void_p * 4)(*([0x10000] * 3 + [0x10008]))
    rc = L.ring_attn_ulysses_forward(ctypes.byref(ud), shards, shards, shards, misaligned, None, FAKE, ws, None)
    assert rc == ra.ERR_INVALID_ARG
    rc = L.ring_attn_ulysses_forward(ctypes.byref(ud), shards, shards, shards, shards, nulls, FAKE, ws, None)
    assert rc == ra.ERR_INVALID_ARG
    rc = L.ring_attn_ulysses_forward(ctypes.byref(ud), None, shards, shards, shards, None, FAKE, ws, None)
    assert rc == ra.ERR_INVALID_ARG
    odd_lse = (ctypes.c_void_p * 4)(*([0x10000] * 3 + [0x10002]))  # fp32 LSE shards must be 4-byte aligned
    rc = L.ring_attn_ulysses_forward(ctypes.byref(ud), shards, shards, shards, shards, odd_lse, FAKE, ws, None)
    assert rc == ra.ERR_INVALID_ARG


def test_backward_workspace_and_validation():
    """The backward entry points check every argument on the host: unsupported
    shapes, bad flags, NULL or misaligned pointers and a small workspace are
    rejected before anything is enqueued."""
    L = ra.lib()
    rd = ra.ring_desc(1, 8, 2, 128, 1024, 4, 1, partition="zigzag")
    ws = ra.backward_workspace_size(rd)
    block = 2 * 1024 * 128 * 2
    rows = 8 * 1024
    assert ws >= 4 * block + rows * 128 * 4 + 2 * rows * 4
    blocks = (ctypes.c_void_p * 4)(*([0x10000] * 4))
    args = (FAKE, blocks, blocks, FAKE, FAKE, FAKE, FAKE, blocks, blocks)
    assert L.ring_attn_backward(ctypes.byref(rd), *args, FAKE, ws - 1, None, None, None) == ra.ERR_WORKSPACE
    nulls = (ctypes.c_void_p * 4)(*([0x10000] * 3 + [None]))
    assert L.ring_attn_backward(ctypes.byref(rd), FAKE, blocks, blocks, FAKE, FAKE, FAKE, FAKE, blocks, nulls,
                                FAKE, ws, None, None, None) == ra.ERR_INVALID_ARG
    bad_dim = ra.ring_desc(1, 8, 2, 96, 1024, 4, 1)
    assert L.ring_attn_backward(ctypes.byref(bad_dim), *args, FAKE, 1 << 40, None, None, None) == ra.ERR_UNSUPPORTED
    sd = ra.step_desc(1, 8, 2, 128, 256, 256, causal=False)
    step_args = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.ring_attn_backward_step(ctypes.byref(sd), *step_args, 2, None) == ra.ERR_INVALID_ARG
    assert L.ring_attn_backward_step(ctypes.byref(sd), None, *step_args[1:], 0, None) == ra.ERR_INVALID_ARG
    mis = ctypes.c_void_p(0x10008)
    assert L.ring_attn_backward_step(ctypes.byref(sd), *step_args[:5], mis, *step_args[6:], 0,
                                     None) == ra.ERR_INVALID_ARG
    sd96 = ra.step_desc(1, 8, 2, 96, 256, 256, causal=False)
    assert L.ring_attn_backward_step(ctypes.byref(sd96), *step_args, 0, None) == ra.ERR_UNSUPPORTED
    assert L.ring_attn_backward_prep(ctypes.byref(sd), None, FAKE, FAKE, FAKE, None) == ra.ERR_INVALID_ARG
    causal_no_segments = ra.step_desc(1, 8, 2, 128, 256, 256)
    assert L.ring_attn_backward_step(ctypes.byref(causal_no_segments), *step_args, 0, None) == ra.ERR_INVALID_ARG


def test_partition_rejects_bad_input():
    with pytest.raises(ra.RingAttnError):
        ra.partition_segments("zigzag", 4, 0, 15)
    with pytest.raises(ra.RingAttnError):
        ra.partition_segments("contiguous", 4, 4, 16)
    with pytest.raises(KeyError):
        ra.partition_segments("diagonal", 4, 0, 16)


def test_mfma_probe_rejects_bad_arguments():
    L = ra.lib()
    fake = ctypes.c_void_p(16)  # never dereferenced: validation comes first
    assert L.ring_attn_mfma_probe(0, 1, fake, fake, None) == ra.ERR_INVALID_ARG
    assert L.ring_attn_mfma_probe(1, 0, fake, fake, None) == ra.ERR_INVALID_ARG
    assert L.ring_attn_mfma_probe(1, 1, None, fake, None) == ra.ERR_INVALID_ARG
    assert L.ring_attn_mfma_probe(1, 1, fake, None, None) == ra.ERR_INVALID_ARG


def test_total_rows_beyond_the_grid_limit_are_rejected():
    """batch x heads x rows above 2^34 would overflow 32-bit launch grids:
    rejected on the host (no GPU work, fake pointers never touched)."""
    L = ra.lib()
    big = ra.step_desc(1 << 13, 1 << 10, 1 << 10, 128, 1 << 12, 1 << 12, causal=False)  # 2^35 rows
    assert L.ring_attn_visible_pairs(ctypes.byref(big)) == -1
    args = [FAKE] * 6
    assert L.ring_attn_step(ctypes.byref(big), *args, 1, None) == ra.ERR_INVALID_ARG
    ok = ra.step_desc(1 << 12, 1 << 10, 1 << 10, 128, 1 << 12, 1 << 12, causal=False)  # 2^34 rows: allowed
    assert L.ring_attn_visible_pairs(ctypes.byref(ok)) == (1 << 12) * (1 << 12)
    rd = ra.ring_desc(1 << 13, 1 << 10, 1 << 10, 128, 1 << 12, 8, 0, partition="contiguous")
    assert L.ring_attn_forward_workspace_size(ctypes.byref(rd)) == 0


def test_release_thread_events_without_events_makes_no_hip_call():
    """A thread that never ran a driver holds no events: the release returns
    OK without touching the (absent) GPU."""
    assert ra.lib().ring_attn_release_thread_events() == ra.OK


def test_forward_noalloc_rejects_before_any_gpu_work():
    """Shares past the scratch size, bad descriptors and NULL blocks are
    rejected on the host (fake pointers: nothing may be touched)."""
    L = ra.lib()
    blocks = (ctypes.c_void_p * 4)(*([0x10000] * 4))
    ok = ra.ring_desc(1, 2, 1, 64, 16, 4, 0)
    assert ra.forward_workspace_size(ok) - 256 <= ra.NOALLOC_SCRATCH_BYTES
    # 128K/8 GQA share: two K/V receive slots and the fp32 state are ~1 GB
    big = ra.ring_desc(1, 32, 8, 128, 16384, 8, 0, partition="zigzag")
    assert ra.forward_workspace_size(big) - 256 > ra.NOALLOC_SCRATCH_BYTES
    blocks8 = (ctypes.c_void_p * 8)(*([0x10000] * 8))
    assert L.ring_attn_forward_noalloc(ctypes.byref(big), FAKE, blocks8, blocks8, FAKE, FAKE, None) == ra.ERR_WORKSPACE
    assert "scratch" in ra.last_error()
    bad = ra.ring_desc(1, 2, 1, 64, 15, 4, 0, partition="zigzag")   # odd local length
    assert L.ring_attn_forward_noalloc(ctypes.byref(bad), FAKE, blocks, blocks, FAKE, FAKE, None) == ra.ERR_INVALID_ARG
    nulls = (ctypes.c_void_p * 4)(*([0x10000] * 3 + [None]))
    assert L.ring_attn_forward_noalloc(ctypes.byref(ok), FAKE, blocks, nulls, FAKE, FAKE, None) == ra.ERR_INVALID_ARG
    assert L.ring_attn_forward_noalloc(None, FAKE, blocks, blocks, FAKE, FAKE, None) == ra.ERR_INVALID_ARG
