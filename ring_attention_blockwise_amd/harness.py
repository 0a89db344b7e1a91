"""Build one device's share of a ring workload on the GPU and run it.

Inputs come from ``ring_inputs`` (seeded, chunk-indexed); rows are mapped to
devices with the library's own partition map (ring_attn_partition_segments).
Nothing here computes attention: the step, merge, finalize and the ring
driver all run in libring_attn.
"""
from __future__ import annotations

import dataclasses

import numpy as np

import ring_inputs
from . import (BF16, F32, RingDesc, backward, backward_workspace_size, finalize, forward,
               forward_workspace_size, partition_segments, ring_desc, ring_step_desc, step, visible_pairs)


def positions(segs) -> np.ndarray:
    """Global positions of the rows described by [(start, len[, stride])]."""
    if not segs:
        return np.zeros(0, dtype=np.int64)
    parts = []
    for seg in segs:
        start, n = seg[0], seg[1]
        stride = seg[2] if len(seg) > 2 else 1
        parts.append(np.arange(start, start + n * stride, stride, dtype=np.int64)[:n])
    return np.concatenate(parts)


def dtype_code(wl: ring_inputs.Workload) -> int:
    return BF16 if wl.dtype == "bf16" else F32


def torch_dtype(wl):
    import torch
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def make_ring_desc(wl: ring_inputs.Workload, rank: int, reverse_order: bool = False, receive="auto",
                   key_split=0) -> RingDesc:
    return ring_desc(wl.batch, wl.heads_q, wl.heads_kv, wl.head_dim, wl.local_len, wl.world, rank,
                     wl.partition, dtype=dtype_code(wl), causal=wl.causal, reverse_order=reverse_order,
                     receive=receive, key_split=key_split)


@dataclasses.dataclass
class DeviceShare:
    workload: ring_inputs.Workload
    rank: int
    q: "object"                 # [B, Hq, c, d] on the GPU
    k_blocks: list              # world tensors [B, Hkv, c, d]
    v_blocks: list
    q_positions: np.ndarray     # global position of each local row

    def ring_desc(self, reverse_order=False, receive="auto", key_split=0) -> RingDesc:
        return make_ring_desc(self.workload, self.rank, reverse_order, receive, key_split)


def _to_device(x: np.ndarray, dt, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).to(device=device).to(dt)


def build_share(wl: ring_inputs.Workload, rank: int, device, on_head=None) -> DeviceShare:
    """Q of device ``rank`` and every device's K/V block, resident on ``device``.

    ``on_head(b, g, k_f32, v_f32)``, if given, is called with each KV head's
    whole global K/V (float32 numpy) as it is drawn, so callers can use the
    same draw without holding every head at once.
    """
    import torch
    dt = torch_dtype(wl)
    B, Hq, Hk, d, c, n = wl.batch, wl.heads_q, wl.heads_kv, wl.head_dim, wl.local_len, wl.world
    L = wl.total_len
    qpos = positions(partition_segments(wl.partition, n, rank, c))
    q = torch.empty((B, Hq, c, d), dtype=dt, device=device)
    for b in range(B):
        for h in range(Hq):
            q[b, h] = _to_device(ring_inputs.rows(wl, "q", b, h, qpos), dt, device)
    block_pos = [torch.from_numpy(positions(partition_segments(wl.partition, n, j, c))).to(device)
                 for j in range(n)]
    k_blocks = [torch.empty((B, Hk, c, d), dtype=dt, device=device) for _ in range(n)]
    v_blocks = [torch.empty((B, Hk, c, d), dtype=dt, device=device) for _ in range(n)]
    for b in range(B):
        for g in range(Hk):
            kh = ring_inputs.head(wl, "k", b, g)
            vh = ring_inputs.head(wl, "v", b, g)
            if on_head is not None:
                on_head(b, g, kh, vh)
            kd = _to_device(kh, dt, device)
            vd = _to_device(vh, dt, device)
            assert kd.shape[0] == L
            for j in range(n):
                k_blocks[j][b, g] = kd.index_select(0, block_pos[j])
                v_blocks[j][b, g] = vd.index_select(0, block_pos[j])
            del kd, vd
    return DeviceShare(wl, rank, q, k_blocks, v_blocks, qpos)


def build_ulysses_shards(wl: ring_inputs.Workload, device, heads_q=None, heads_kv=None):
    """Every device's sequence shard of Q, K and V for a Ulysses workload:
    lists of ``world`` tensors [B, H, local_len, d], shard j holding tokens
    j*local_len .. (j+1)*local_len - 1 (only ``heads_q`` / ``heads_kv`` are
    drawn if given; the others stay zero)."""
    import torch
    dt = torch_dtype(wl)
    B, Hq, Hk, d, c, n = wl.batch, wl.heads_q, wl.heads_kv, wl.head_dim, wl.local_len, wl.world
    out = {}
    for name, H, which in (("q", Hq, heads_q), ("k", Hk, heads_kv), ("v", Hk, heads_kv)):
        shards = [torch.zeros((B, H, c, d), dtype=dt, device=device) for _ in range(n)]
        for b in range(B):
            for h in (range(H) if which is None else which):
                full = _to_device(ring_inputs.head(wl, name, b, h), dt, device)
                for j in range(n):
                    shards[j][b, h] = full[j * c:(j + 1) * c]
                del full
        out[name] = shards
    return out["q"], out["k"], out["v"]


def alloc_outputs(share: DeviceShare):
    import torch
    wl = share.workload
    out = torch.empty_like(share.q)
    lse = torch.empty((wl.batch, wl.heads_q, wl.local_len), dtype=torch.float32, device=share.q.device)
    return out, lse


def effective_key_split(share: DeviceShare, key_split=0) -> int:
    """The key split the library gives this share's forward (1: none), read
    from the workspace it asks for: k partial fp32 states of the share's rows."""
    wl = share.workload
    extra = (forward_workspace_size(share.ring_desc(key_split=key_split))
             - forward_workspace_size(share.ring_desc(key_split=1)))
    per = wl.batch * wl.heads_q * wl.local_len * (wl.head_dim + 2) * 4
    return max(1, round(extra / per)) if extra > 0 else 1


def alloc_workspace(share: DeviceShare, reverse_order=False, key_split=0):
    import torch
    n = forward_workspace_size(share.ring_desc(reverse_order, key_split=key_split))
    return torch.empty(n, dtype=torch.uint8, device=share.q.device)


def run_forward(share: DeviceShare, reverse_order=False, copy_stream=None, workspace=None, out=None, lse=None,
                step_events=None, receive="auto", key_split=0):
    """ring_attn_forward on the current stream (receive copies on ``copy_stream``,
    made as ``receive`` says: "auto", "memcpy" or "fused"; ``key_split`` as
    ring_desc)."""
    if out is None:
        out, lse = alloc_outputs(share)
    if workspace is None:
        workspace = alloc_workspace(share, reverse_order, key_split)
    forward(share.ring_desc(reverse_order, receive, key_split), share.q, share.k_blocks, share.v_blocks, out, lse,
            workspace, copy_stream=copy_stream, step_events=step_events)
    return out, lse


def new_state(share: DeviceShare):
    import torch
    wl = share.workload
    dev = share.q.device
    o = torch.zeros((wl.batch, wl.heads_q, wl.local_len, wl.head_dim), dtype=torch.float32, device=dev)
    m = torch.full((wl.batch, wl.heads_q, wl.local_len), float("-inf"), dtype=torch.float32, device=dev)
    l = torch.zeros((wl.batch, wl.heads_q, wl.local_len), dtype=torch.float32, device=dev)
    return o, m, l


def run_steps(share: DeviceShare, steps, state=None, init_first=True):
    """Apply ring steps (indices into the ring order) with ring_attn_step, in the given order."""
    rd = share.ring_desc()
    if state is None:
        state = new_state(share)
    o, m, l = state
    first = init_first
    for s in steps:
        sd, owner = ring_step_desc(rd, s)
        step(sd, share.q, share.k_blocks[owner], share.v_blocks[owner], o, m, l, init=first)
        first = False
    return o, m, l


def finalize_state(share: DeviceShare, state):
    rd = share.ring_desc()
    sd, _ = ring_step_desc(rd, 0)
    out, lse = alloc_outputs(share)
    o, m, l = state
    finalize(sd, o, m, l, out, lse)
    return out, lse


def step_pairs(wl: ring_inputs.Workload, rank: int):
    """Visible (query, key) pairs per (batch, head) of every ring step of a share."""
    rd = make_ring_desc(wl, rank)
    return [visible_pairs(ring_step_desc(rd, s)[0]) for s in range(wl.world)]


def build_upstream(share: DeviceShare):
    """The seeded upstream gradient dO at the device's rows, [B, Hq, c, d] on the GPU."""
    import torch
    wl = share.workload
    dt = torch_dtype(wl)
    d_out = torch.empty_like(share.q)
    for b in range(wl.batch):
        for h in range(wl.heads_q):
            d_out[b, h] = _to_device(ring_inputs.rows(wl, "do", b, h, share.q_positions), dt, share.q.device)
    return d_out


def new_kv_grads(share: DeviceShare):
    """Zeroed fp32 dK and dV accumulators, one pair per K/V block."""
    import torch
    wl = share.workload
    shape = (wl.batch, wl.heads_kv, wl.local_len, wl.head_dim)
    dk = [torch.zeros(shape, dtype=torch.float32, device=share.q.device) for _ in range(wl.world)]
    dv = [torch.zeros(shape, dtype=torch.float32, device=share.q.device) for _ in range(wl.world)]
    return dk, dv


def run_backward(share: DeviceShare, out, lse, d_out, dk_acc, dv_acc, copy_stream=None, workspace=None,
                 step_events=None, receive="auto"):
    """ring_attn_backward on the current stream; returns dQ (input dtype)."""
    import torch
    rd = share.ring_desc(receive=receive)
    if workspace is None:
        workspace = torch.empty(backward_workspace_size(rd), dtype=torch.uint8, device=share.q.device)
    dq = torch.empty_like(share.q)
    backward(rd, share.q, share.k_blocks, share.v_blocks, out, d_out, lse, dq, dk_acc, dv_acc, workspace,
             copy_stream=copy_stream, step_events=step_events)
    return dq
