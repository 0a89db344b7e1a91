"""Seeded synthetic inputs for the blockwise ring-attention step.

This module only *draws numbers*: workload presets (shapes, distributions,
seeds) and deterministic, chunk-indexed generation of the global Q/K/V
sequences. It holds none of the attention arithmetic and none of the
partitioning logic; both the CPU oracle and the HIP path consume what it
returns and each maps rows to devices with its own code.

Generation recipe (the same for every workload):

* The global sequence of length ``L = world * local_len`` is cut into
  ``2 * world`` generation chunks of ``L / (2 * world)`` tokens.
* Every (tensor, batch, head, chunk) draws from its own PCG64 stream seeded
  by ``SeedSequence([seed, tensor_id, b, h, chunk])``, in float32, so any
  chunk regenerates on its own and the result never depends on the order
  or the threads used to draw it.
* Q and K are ``N(0, qk_std**2)``; V is ``N(0, 1)`` or ``U(-1, 1)``; the
  upstream gradient dO of the backward pass (tensor "do", query heads) is
  ``N(0, 1)``.
* For bf16 workloads every value is then rounded once to bfloat16
  (round-to-nearest-even); both sides consume the rounded values.
* A duplicated-key fraction (the numerics-stress workload) copies K rows
  onto ``floor(dup_frac * L)`` seeded destination positions per
  (batch, kv head) from uniformly drawn *other* positions of the same head,
  using the pre-copy values, so scores tie exactly.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}
_DUP_STREAM = 99


@dataclasses.dataclass(frozen=True)
class Workload:
    """One device-share workload of a simulated ring.

    ``world`` simulated devices each hold ``local_len`` tokens of a global
    sequence of ``world * local_len`` tokens. ``ranks`` lists the device
    shares that are run (the first one is the graded share).
    """

    name: str
    batch: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str          # "f32" or "bf16"
    causal: bool
    partition: str      # "contiguous" or "zigzag"
    world: int
    local_len: int
    seed: int
    qk_std: float = 1.0
    v_dist: str = "normal"   # "normal" -> N(0,1); "uniform" -> U(-1,1)
    dup_frac: float = 0.0
    ranks: tuple = (0,)
    description: str = ""

    @property
    def total_len(self) -> int:
        return self.world * self.local_len

    @property
    def gen_chunk(self) -> int:
        return self.total_len // (2 * self.world)

    @property
    def n_gen_chunks(self) -> int:
        return 2 * self.world

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads, named by what they are.
WORKLOADS = {
    "ring4_noncausal_f32": Workload(
        name="ring4_noncausal_f32", batch=1, heads_q=2, heads_kv=2, head_dim=64, dtype="f32",
        causal=False, partition="contiguous", world=4, local_len=256, seed=1001, ranks=(0,),
        description="non-causal ring of 4 steps, B1 H2 d64 fp32, local Q 256, 4 K/V blocks of 256"),
    "zigzag8k_8dev_d128": Workload(
        name="zigzag8k_8dev_d128", batch=1, heads_q=8, heads_kv=8, head_dim=128, dtype="bf16",
        causal=True, partition="zigzag", world=8, local_len=1024, seed=1002, ranks=(0,),
        description="causal zigzag, 8192 tokens over 8 devices (chunks i and 15-i of 512), H8 d128 bf16"),
    "zigzag128k_8dev_gqa": Workload(
        name="zigzag128k_8dev_gqa", batch=1, heads_q=32, heads_kv=8, head_dim=128, dtype="bf16",
        causal=True, partition="zigzag", world=8, local_len=16384, seed=1003, ranks=(0,),
        description="one device of a 128K causal context over 8 devices, 32 Q / 8 KV heads, d128 bf16, zigzag"),
    "striped128k_8dev_gqa": Workload(
        name="striped128k_8dev_gqa", batch=1, heads_q=32, heads_kv=8, head_dim=128, dtype="bf16",
        causal=True, partition="striped", world=8, local_len=16384, seed=1003, ranks=(0,),
        description="the 128K/8 GQA tensors under the striped partition (token t on device t mod 8)"),
    "zigzag1m_64dev": Workload(
        name="zigzag1m_64dev", batch=1, heads_q=8, heads_kv=8, head_dim=128, dtype="bf16",
        causal=True, partition="zigzag", world=64, local_len=16384, seed=1004, ranks=(0,),
        description="one device of a 1M causal context over 64 devices, H8 d128 bf16, zigzag"),
    "contig1m_64dev": Workload(
        name="contig1m_64dev", batch=1, heads_q=8, heads_kv=8, head_dim=128, dtype="bf16",
        causal=True, partition="contiguous", world=64, local_len=16384, seed=1004, ranks=(63, 0),
        description="one device of a 1M causal context over 64 devices, H8 d128 bf16, contiguous"),
    "stress256k_8dev_d64": Workload(
        name="stress256k_8dev_d64", batch=1, heads_q=16, heads_kv=16, head_dim=64, dtype="bf16",
        causal=True, partition="contiguous", world=8, local_len=32768, seed=1005, qk_std=4.0,
        v_dist="uniform", dup_frac=0.01, ranks=(7, 0),
        description="numerics stress: causal contiguous, local 32768 x 8 steps, H16 d64 bf16, "
                    "Q,K ~ N(0,16), V ~ U(-1,1), 1% duplicated keys"),
}


# Ulysses workloads: the global sequence is split into `world` contiguous
# shards (device j holds tokens j*local_len .. (j+1)*local_len - 1); the
# 128K one draws the same global tensors as the 128K zigzag ring workload.
ULYSSES_WORKLOADS = {
    "ulysses2k_4dev_gqa": Workload(
        name="ulysses2k_4dev_gqa", batch=1, heads_q=8, heads_kv=4, head_dim=128, dtype="bf16",
        causal=True, partition="contiguous", world=4, local_len=512, seed=1006, ranks=(0, 1, 2, 3),
        description="Ulysses, causal, 2048 tokens over 4 devices, 8 Q / 4 KV heads, d128 bf16"),
    "ulysses512_2dev_f32": Workload(
        name="ulysses512_2dev_f32", batch=2, heads_q=4, heads_kv=2, head_dim=64, dtype="f32",
        causal=False, partition="contiguous", world=2, local_len=256, seed=1007, ranks=(0, 1),
        description="Ulysses, non-causal, 512 tokens over 2 devices, B2, 4 Q / 2 KV heads, d64 fp32"),
    "ulysses990_3dev_ragged": Workload(
        name="ulysses990_3dev_ragged", batch=2, heads_q=6, heads_kv=3, head_dim=64, dtype="bf16",
        causal=True, partition="contiguous", world=3, local_len=330, seed=1031, ranks=(0, 1, 2),
        description="Ulysses, causal, 990 tokens over 3 devices (330 per shard: ragged tiles, LSE shards "
                    "not a multiple of 16 bytes), B2, 6 Q / 3 KV heads, d64 bf16"),
    "ulysses128k_8dev_gqa": Workload(
        name="ulysses128k_8dev_gqa", batch=1, heads_q=32, heads_kv=8, head_dim=128, dtype="bf16",
        causal=True, partition="contiguous", world=8, local_len=16384, seed=1003, ranks=(0,),
        description="Ulysses, one device of a 128K causal context over 8 devices, 32 Q / 8 KV heads "
                    "(4 Q / 1 KV head per device), d128 bf16"),
}


# Backward-pass workloads (small enough for the oracle to cover every row):
# GQA zigzag, two batches striped, non-causal, and ragged row counts.
BACKWARD_WORKLOADS = {
    "bwd_zigzag4k_4dev_gqa": Workload(
        name="bwd_zigzag4k_4dev_gqa", batch=1, heads_q=8, heads_kv=2, head_dim=128, dtype="bf16",
        causal=True, partition="zigzag", world=4, local_len=1024, seed=1008, ranks=(0, 1, 2, 3),
        description="backward, causal zigzag, 4096 tokens over 4 devices, 8 Q / 2 KV heads, d128 bf16"),
    "bwd_striped2k_2dev_b2": Workload(
        name="bwd_striped2k_2dev_b2", batch=2, heads_q=4, heads_kv=4, head_dim=128, dtype="bf16",
        causal=True, partition="striped", world=2, local_len=1024, seed=1009, ranks=(0, 1),
        description="backward, causal striped, 2048 tokens over 2 devices, B2, H4, d128 bf16"),
    "bwd_noncausal1k_4dev": Workload(
        name="bwd_noncausal1k_4dev", batch=1, heads_q=4, heads_kv=2, head_dim=128, dtype="bf16",
        causal=False, partition="contiguous", world=4, local_len=256, seed=1010, ranks=(0, 1, 2, 3),
        description="backward, non-causal, 1024 tokens over 4 devices, 4 Q / 2 KV heads, d128 bf16"),
    "bwd_zigzag2k_4dev_d64": Workload(
        name="bwd_zigzag2k_4dev_d64", batch=1, heads_q=4, heads_kv=2, head_dim=64, dtype="bf16",
        causal=True, partition="zigzag", world=4, local_len=512, seed=1012, ranks=(0, 1, 2, 3),
        description="backward, causal zigzag, 2048 tokens over 4 devices, 4 Q / 2 KV heads, d64 bf16"),
    "bwd_f32_zigzag1k_4dev": Workload(
        name="bwd_f32_zigzag1k_4dev", batch=1, heads_q=4, heads_kv=2, head_dim=128, dtype="f32",
        causal=True, partition="zigzag", world=4, local_len=256, seed=1013, ranks=(0, 1, 2, 3),
        description="backward, causal zigzag, 1024 tokens over 4 devices, 4 Q / 2 KV heads, d128 fp32"),
    "bwd_ragged3k_3dev": Workload(
        name="bwd_ragged3k_3dev", batch=1, heads_q=4, heads_kv=1, head_dim=128, dtype="bf16",
        causal=True, partition="zigzag", world=3, local_len=1000, seed=1011, ranks=(0, 1, 2),
        description="backward, causal zigzag, 3000 tokens over 3 devices (ragged tiles), 4 Q / 1 KV head, "
                    "d128 bf16"),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-exact (uint16)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _draw_chunk(wl: Workload, tensor: str, b: int, h: int, chunk: int) -> np.ndarray:
    ss = np.random.SeedSequence([wl.seed, TENSOR_IDS[tensor], b, h, chunk])
    rng = np.random.Generator(np.random.PCG64(ss))
    shape = (wl.gen_chunk, wl.head_dim)
    if tensor == "v" and wl.v_dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    elif tensor in ("v", "do"):
        x = rng.standard_normal(shape, dtype=np.float32)
    else:
        x = rng.standard_normal(shape, dtype=np.float32)
        if wl.qk_std != 1.0:
            x *= np.float32(wl.qk_std)
    if wl.dtype == "bf16":
        x = round_to_bf16(x)
    return x


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def chunks(wl: Workload, tensor: str, b: int, h: int, chunk_ids) -> np.ndarray:
    """Concatenation of the given generation chunks of one head, float32 [len, d]."""
    chunk_ids = list(chunk_ids)
    if tensor == "k" and wl.dup_frac > 0:
        full = head(wl, "k", b, h)
        g = wl.gen_chunk
        return np.concatenate([full[c * g:(c + 1) * g] for c in chunk_ids], axis=0)
    if len(chunk_ids) > 2:
        with ThreadPoolExecutor(_threads()) as ex:
            parts = list(ex.map(lambda c: _draw_chunk(wl, tensor, b, h, c), chunk_ids))
    else:
        parts = [_draw_chunk(wl, tensor, b, h, c) for c in chunk_ids]
    return np.concatenate(parts, axis=0)


def duplicate_plan(wl: Workload, b: int, h: int):
    """(dst, src) positions of the duplicated keys of one (batch, kv head)."""
    L = wl.total_len
    n_dup = int(np.floor(wl.dup_frac * L))
    if n_dup == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, _DUP_STREAM, b, h])))
    dst = rng.choice(L, size=n_dup, replace=False).astype(np.int64)
    src = rng.integers(0, L - 1, size=n_dup).astype(np.int64)
    src = src + (src >= dst)          # uniform over the other L-1 positions
    return dst, src


def head(wl: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """The whole global sequence of one (tensor, batch, head), float32 [L, d]."""
    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(lambda c: _draw_chunk(wl, tensor, b, h, c), range(wl.n_gen_chunks)))
    x = np.concatenate(parts, axis=0)
    if tensor == "k" and wl.dup_frac > 0:
        dst, src = duplicate_plan(wl, b, h)
        x[dst] = x[src].copy()
    return x


def rows(wl: Workload, tensor: str, b: int, h: int, positions: np.ndarray) -> np.ndarray:
    """Rows of one head at the given global positions, float32 [len(positions), d].

    Only the generation chunks that hold those positions are drawn.
    """
    positions = np.asarray(positions, dtype=np.int64)
    g = wl.gen_chunk
    need = np.unique(positions // g)
    if tensor == "k" and wl.dup_frac > 0:
        return head(wl, "k", b, h)[positions]
    block = chunks(wl, tensor, b, h, need)
    return block[_vector_local(positions, need, g)]


def _vector_local(positions, need, g):
    lut = np.full(int(need.max()) + 1, -1, dtype=np.int64)
    lut[need] = np.arange(len(need), dtype=np.int64)
    return lut[positions // g] * g + positions % g
