"""Python binding of libring_attn — the MI355X blockwise ring-attention step.

Argument marshalling only: every step of the path runs in the HIP library
(``csrc/``, declared in ``include/ring_attn.h``). Tensors are torch tensors on
the GPU (PyTorch provides device memory and streams); each call checks device,
dtype, shape and contiguity, then passes raw pointers and the current HIP
stream. Importing works without a GPU (host-only helpers run anywhere); the
library must be built (``python -m ring_attention_blockwise_amd.build``) or
every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RING_ATTN_LIB") or os.path.join(_HERE, "libring_attn.so")

# ---- constants mirrored from ring_attn.h ------------------------------------
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
CONTIGUOUS, ZIGZAG, STRIPED = 0, 1, 2
PARTITIONS = {"contiguous": CONTIGUOUS, "zigzag": ZIGZAG, "striped": STRIPED}
RECV_AUTO, RECV_MEMCPY, RECV_FUSED = 0, 1, 2
RECEIVES = {"auto": RECV_AUTO, "memcpy": RECV_MEMCPY, "fused": RECV_FUSED}
STEP_INIT = 1
BWD_INIT_DQ = 1

EXPORTED = (
    "ring_attn_step", "ring_attn_merge", "ring_attn_finalize", "ring_attn_forward_workspace_size",
    "ring_attn_forward", "ring_attn_partition_segments", "ring_attn_ring_step_desc",
    "ring_attn_visible_pairs", "ring_attn_last_error", "ring_attn_abi_version",
    "ring_attn_events_create", "ring_attn_event_elapsed_ms", "ring_attn_events_destroy",
    "ring_attn_synchronize", "ring_attn_ulysses_workspace_size", "ring_attn_ulysses_forward",
    "ring_attn_backward_prep", "ring_attn_backward_step", "ring_attn_backward_workspace_size",
    "ring_attn_backward", "ring_attn_mfma_probe", "ring_attn_release_thread_events",
    "ring_attn_forward_noalloc",
)


class Segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int64), ("stride", ctypes.c_int64)]


class StepDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
        ("n_q_seg", ctypes.c_int32), ("n_kv_seg", ctypes.c_int32),
        ("q_seg", Segment * 2), ("kv_seg", Segment * 2),
    ]


class RingDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("local_len", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float), ("world", ctypes.c_int32),
        ("rank", ctypes.c_int32), ("partition", ctypes.c_int32), ("reverse_order", ctypes.c_int32),
        ("receive", ctypes.c_int32), ("key_split", ctypes.c_int32),
    ]


class UlyssesDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("scale", ctypes.c_float), ("world", ctypes.c_int32),
        ("rank", ctypes.c_int32),
    ]


class RingAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m ring_attention_blockwise_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        SD, RD, UD = ctypes.POINTER(StepDesc), ctypes.POINTER(RingDesc), ctypes.POINTER(UlyssesDesc)
        sig = {
            "ring_attn_step": (ctypes.c_int, [SD, P, P, P, P, P, P, I32, P]),
            "ring_attn_merge": (ctypes.c_int, [SD, P, P, P, P, P, P, P]),
            "ring_attn_finalize": (ctypes.c_int, [SD, P, P, P, P, P, P]),
            "ring_attn_forward_workspace_size": (SZ, [RD]),
            "ring_attn_forward": (ctypes.c_int, [RD, P, P, P, P, P, P, SZ, P, P, P]),
            "ring_attn_forward_noalloc": (ctypes.c_int, [RD, P, P, P, P, P, P]),
            "ring_attn_partition_segments": (ctypes.c_int, [I32, I32, I32, I64, ctypes.POINTER(Segment),
                                                            ctypes.POINTER(I32)]),
            "ring_attn_ring_step_desc": (ctypes.c_int, [RD, I32, SD, ctypes.POINTER(I32)]),
            "ring_attn_visible_pairs": (I64, [SD]),
            "ring_attn_last_error": (ctypes.c_char_p, []),
            "ring_attn_abi_version": (I32, []),
            "ring_attn_events_create": (ctypes.c_int, [I32, P]),
            "ring_attn_event_elapsed_ms": (ctypes.c_int, [P, P, ctypes.POINTER(ctypes.c_float)]),
            "ring_attn_events_destroy": (ctypes.c_int, [I32, P]),
            "ring_attn_synchronize": (ctypes.c_int, [P]),
            "ring_attn_release_thread_events": (ctypes.c_int, []),
            "ring_attn_mfma_probe": (ctypes.c_int, [I32, I32, P, P, P]),
            "ring_attn_ulysses_workspace_size": (SZ, [UD]),
            "ring_attn_ulysses_forward": (ctypes.c_int, [UD, P, P, P, P, P, P, SZ, P]),
            "ring_attn_backward_prep": (ctypes.c_int, [SD, P, P, P, P, P]),
            "ring_attn_backward_step": (ctypes.c_int, [SD, P, P, P, P, P, P, P, P, I32, P]),
            "ring_attn_backward_workspace_size": (SZ, [RD]),
            "ring_attn_backward": (ctypes.c_int, [RD, P, P, P, P, P, P, P, P, P, P, SZ, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def last_error() -> str:
    return lib().ring_attn_last_error().decode()


def _check(rc: int, what: str):
    if rc != OK:
        raise RingAttnError(rc, f"{what}: {last_error()}")


# ---- descriptors ---------------------------------------------------------------
def _segments(segs):
    arr = (Segment * 2)()
    for i, s in enumerate(segs):
        start, length = s[0], s[1]
        stride = s[2] if len(s) > 2 else 1
        arr[i] = Segment(start, length, stride)
    return arr, len(segs)


def step_desc(batch, heads_q, heads_kv, head_dim, q_len, kv_len, dtype=BF16, causal=True, scale=0.0,
              q_segs=(), kv_segs=()) -> StepDesc:
    """Step descriptor; segments are (start, len[, stride]) tuples of global positions."""
    qa, nq = _segments(q_segs)
    ka, nk = _segments(kv_segs)
    return StepDesc(batch, heads_q, heads_kv, head_dim, q_len, kv_len, dtype, int(causal), scale,
                    nq, nk, qa, ka)


def ring_desc(batch, heads_q, heads_kv, head_dim, local_len, world, rank, partition="zigzag",
              dtype=BF16, causal=True, scale=0.0, reverse_order=False, receive="auto",
              key_split=0) -> RingDesc:
    """key_split: 0 automatic, 1 never, 2..16 that many parts per query tile (bf16)."""
    part = PARTITIONS[partition] if isinstance(partition, str) else int(partition)
    recv = RECEIVES[receive] if isinstance(receive, str) else int(receive)
    return RingDesc(batch, heads_q, heads_kv, head_dim, local_len, dtype, int(causal), scale, world,
                    rank, part, int(reverse_order), recv, int(key_split))


def partition_segments(partition, world: int, rank: int, local_len: int):
    """[(start, len, stride)] of device ``rank``'s local rows (the library's partition map)."""
    part = PARTITIONS[partition] if isinstance(partition, str) else int(partition)
    segs = (Segment * 2)()
    n = ctypes.c_int32()
    _check(lib().ring_attn_partition_segments(part, world, rank, local_len, segs, ctypes.byref(n)),
           "partition_segments")
    return [(segs[i].start, segs[i].len, segs[i].stride) for i in range(n.value)]


def ring_step_desc(rd: RingDesc, step: int):
    """(StepDesc, owner) of ring step ``step``."""
    sd = StepDesc()
    owner = ctypes.c_int32()
    _check(lib().ring_attn_ring_step_desc(ctypes.byref(rd), step, ctypes.byref(sd), ctypes.byref(owner)),
           "ring_step_desc")
    return sd, owner.value


def visible_pairs(sd: StepDesc) -> int:
    n = lib().ring_attn_visible_pairs(ctypes.byref(sd))
    if n < 0:
        raise RingAttnError(ERR_INVALID_ARG, f"visible_pairs: {last_error()}")
    return int(n)


def forward_workspace_size(rd: RingDesc) -> int:
    n = lib().ring_attn_forward_workspace_size(ctypes.byref(rd))
    if n == 0:
        raise RingAttnError(ERR_INVALID_ARG, f"forward_workspace_size: {last_error()}")
    return int(n)


# ---- tensor marshalling ------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_of(code):
    torch = _torch()
    return torch.bfloat16 if code == BF16 else torch.float32


def _ptr(t, dtype, shape, name):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def step(sd: StepDesc, q, k, v, o_acc, m, l, init: bool = False, stream=None):
    """Fold K/V into the state (o_acc, m, l) in place (ring_attn_step)."""
    torch = _torch()
    dt = _dtype_of(sd.dtype)
    B, Hq, Hk, D = sd.batch, sd.heads_q, sd.heads_kv, sd.head_dim
    args = (
        _ptr(q, dt, (B, Hq, sd.q_len, D), "q"), _ptr(k, dt, (B, Hk, sd.kv_len, D), "k"),
        _ptr(v, dt, (B, Hk, sd.kv_len, D), "v"), _ptr(o_acc, torch.float32, (B, Hq, sd.q_len, D), "o_acc"),
        _ptr(m, torch.float32, (B, Hq, sd.q_len), "m"), _ptr(l, torch.float32, (B, Hq, sd.q_len), "l"),
    )
    _check(lib().ring_attn_step(ctypes.byref(sd), *args, STEP_INIT if init else 0, _stream(stream)),
           "ring_attn_step")


def merge(sd: StepDesc, o_a, m_a, l_a, o_b, m_b, l_b, stream=None):
    """(o_a, m_a, l_a) <- (a) merged with (b) (ring_attn_merge)."""
    torch = _torch()
    B, Hq, D, S = sd.batch, sd.heads_q, sd.head_dim, sd.q_len
    f = torch.float32
    _check(lib().ring_attn_merge(
        ctypes.byref(sd), _ptr(o_a, f, (B, Hq, S, D), "o_a"), _ptr(m_a, f, (B, Hq, S), "m_a"),
        _ptr(l_a, f, (B, Hq, S), "l_a"), _ptr(o_b, f, (B, Hq, S, D), "o_b"), _ptr(m_b, f, (B, Hq, S), "m_b"),
        _ptr(l_b, f, (B, Hq, S), "l_b"), _stream(stream)), "ring_attn_merge")


def finalize(sd: StepDesc, o_acc, m, l, out, lse=None, stream=None):
    """out <- o_acc / l in the input dtype; lse <- natural-log LSE (ring_attn_finalize)."""
    torch = _torch()
    B, Hq, D, S = sd.batch, sd.heads_q, sd.head_dim, sd.q_len
    f = torch.float32
    _check(lib().ring_attn_finalize(
        ctypes.byref(sd), _ptr(o_acc, f, (B, Hq, S, D), "o_acc"), _ptr(m, f, (B, Hq, S), "m"),
        _ptr(l, f, (B, Hq, S), "l"), _ptr(out, _dtype_of(sd.dtype), (B, Hq, S, D), "out"),
        _ptr(lse, f, (B, Hq, S), "lse"), _stream(stream)), "ring_attn_finalize")


def forward(rd: RingDesc, q_local, k_blocks: Sequence, v_blocks: Sequence, out, lse, workspace,
            compute_stream=None, copy_stream=None, step_events: Optional["StepEvents"] = None):
    """One device's whole ring (ring_attn_forward). ``workspace`` is a uint8 GPU tensor."""
    torch = _torch()
    dt = _dtype_of(rd.dtype)
    B, Hq, Hk, D, c, n = rd.batch, rd.heads_q, rd.heads_kv, rd.head_dim, rd.local_len, rd.world
    if len(k_blocks) != n or len(v_blocks) != n:
        raise ValueError(f"need {n} K and V blocks")
    kp = (ctypes.c_void_p * n)(*[_ptr(k, dt, (B, Hk, c, D), f"k_blocks[{i}]").value for i, k in enumerate(k_blocks)])
    vp = (ctypes.c_void_p * n)(*[_ptr(v, dt, (B, Hk, c, D), f"v_blocks[{i}]").value for i, v in enumerate(v_blocks)])
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    ev = None
    if step_events is not None:
        if step_events.n != 2 * n:
            raise ValueError("step_events must hold 2 * world events")
        ev = step_events.array
    _check(lib().ring_attn_forward(
        ctypes.byref(rd), _ptr(q_local, dt, (B, Hq, c, D), "q_local"), kp, vp,
        _ptr(out, dt, (B, Hq, c, D), "out"), _ptr(lse, torch.float32, (B, Hq, c), "lse"),
        ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(compute_stream),
        None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream), ev), "ring_attn_forward")


NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024  # RA_NOALLOC_SCRATCH_BYTES


def forward_noalloc(rd: RingDesc, q_local, k_blocks: Sequence, v_blocks: Sequence, out, lse, stream=None):
    """One device's whole ring without a workspace (ring_attn_forward_noalloc):
    the library's per-GPU scratch array holds the receive slots and state."""
    torch = _torch()
    dt = _dtype_of(rd.dtype)
    B, Hq, Hk, D, c, n = rd.batch, rd.heads_q, rd.heads_kv, rd.head_dim, rd.local_len, rd.world
    if len(k_blocks) != n or len(v_blocks) != n:
        raise ValueError(f"need {n} K and V blocks")
    kp = (ctypes.c_void_p * n)(*[_ptr(k, dt, (B, Hk, c, D), f"k_blocks[{i}]").value for i, k in enumerate(k_blocks)])
    vp = (ctypes.c_void_p * n)(*[_ptr(v, dt, (B, Hk, c, D), f"v_blocks[{i}]").value for i, v in enumerate(v_blocks)])
    _check(lib().ring_attn_forward_noalloc(
        ctypes.byref(rd), _ptr(q_local, dt, (B, Hq, c, D), "q_local"), kp, vp,
        _ptr(out, dt, (B, Hq, c, D), "out"), _ptr(lse, torch.float32, (B, Hq, c), "lse"), _stream(stream)),
        "ring_attn_forward_noalloc")


def ulysses_desc(batch, heads_q, heads_kv, head_dim, seq_len, world, rank, dtype=BF16, causal=True,
                 scale=0.0) -> UlyssesDesc:
    return UlyssesDesc(batch, heads_q, heads_kv, head_dim, seq_len, dtype, int(causal), scale, world, rank)


def ulysses_workspace_size(ud: UlyssesDesc) -> int:
    n = lib().ring_attn_ulysses_workspace_size(ctypes.byref(ud))
    if n == 0:
        raise RingAttnError(ERR_INVALID_ARG, f"ulysses_workspace_size: {last_error()}")
    return int(n)


def ulysses_forward(ud: UlyssesDesc, q_shards: Sequence, k_shards: Sequence, v_shards: Sequence,
                    out_shards: Sequence, lse_shards: Optional[Sequence], workspace, stream=None):
    """Device ``ud.rank``'s part of one Ulysses attention (ring_attn_ulysses_forward):
    shards are device j's [B, H, L/world, d] tensors; writes this device's heads of
    every out (and lse) shard. ``workspace`` is a uint8 GPU tensor."""
    torch = _torch()
    dt = _dtype_of(ud.dtype)
    B, Hq, Hk, D, n = ud.batch, ud.heads_q, ud.heads_kv, ud.head_dim, ud.world
    ls = ud.seq_len // n if n > 0 else 0
    for name, arr in (("q", q_shards), ("k", k_shards), ("v", v_shards), ("out", out_shards)):
        if len(arr) != n:
            raise ValueError(f"need {n} {name} shards")
    if lse_shards is not None and len(lse_shards) != n:
        raise ValueError(f"need {n} lse shards")

    def ptrs(arr, dtype, heads, name):
        return (ctypes.c_void_p * n)(*[_ptr(t, dtype, (B, heads, ls, D), f"{name}[{i}]").value
                                      for i, t in enumerate(arr)])

    qp, kp, vp = ptrs(q_shards, dt, Hq, "q_shards"), ptrs(k_shards, dt, Hk, "k_shards"), ptrs(v_shards, dt, Hk, "v_shards")
    op = ptrs(out_shards, dt, Hq, "out_shards")
    lp = None
    if lse_shards is not None:
        lp = (ctypes.c_void_p * n)(*[_ptr(t, torch.float32, (B, Hq, ls), f"lse_shards[{i}]").value
                                     for i, t in enumerate(lse_shards)])
    ws = _ptr(workspace, torch.uint8, (workspace.numel(),), "workspace")
    _check(lib().ring_attn_ulysses_forward(ctypes.byref(ud), qp, kp, vp, op, lp, ws, workspace.numel(),
                                           _stream(stream)), "ring_attn_ulysses_forward")


def backward_prep(sd: StepDesc, out, d_out, lse, terms, stream=None):
    """Row terms of the backward step (ring_attn_backward_prep); ``terms`` is
    fp32 [2, B, Hq, q_len]."""
    torch = _torch()
    dt = _dtype_of(sd.dtype)
    B, Hq, D, S = sd.batch, sd.heads_q, sd.head_dim, sd.q_len
    f = torch.float32
    _check(lib().ring_attn_backward_prep(
        ctypes.byref(sd), _ptr(out, dt, (B, Hq, S, D), "out"), _ptr(d_out, dt, (B, Hq, S, D), "d_out"),
        _ptr(lse, f, (B, Hq, S), "lse"), _ptr(terms, f, (2, B, Hq, S), "terms"), _stream(stream)),
        "ring_attn_backward_prep")


def backward_step(sd: StepDesc, q, k, v, d_out, terms, dq_acc, dk_acc, dv_acc, init_dq: bool = False,
                  stream=None):
    """Add one K/V block's gradient contributions (ring_attn_backward_step)."""
    torch = _torch()
    dt = _dtype_of(sd.dtype)
    f = torch.float32
    B, Hq, Hk, D = sd.batch, sd.heads_q, sd.heads_kv, sd.head_dim
    args = (
        _ptr(q, dt, (B, Hq, sd.q_len, D), "q"), _ptr(k, dt, (B, Hk, sd.kv_len, D), "k"),
        _ptr(v, dt, (B, Hk, sd.kv_len, D), "v"), _ptr(d_out, dt, (B, Hq, sd.q_len, D), "d_out"),
        _ptr(terms, f, (2, B, Hq, sd.q_len), "terms"), _ptr(dq_acc, f, (B, Hq, sd.q_len, D), "dq_acc"),
        _ptr(dk_acc, f, (B, Hk, sd.kv_len, D), "dk_acc"), _ptr(dv_acc, f, (B, Hk, sd.kv_len, D), "dv_acc"),
    )
    _check(lib().ring_attn_backward_step(ctypes.byref(sd), *args, BWD_INIT_DQ if init_dq else 0, _stream(stream)),
           "ring_attn_backward_step")


def backward_workspace_size(rd: RingDesc) -> int:
    n = lib().ring_attn_backward_workspace_size(ctypes.byref(rd))
    if n == 0:
        raise RingAttnError(ERR_INVALID_ARG, f"backward_workspace_size: {last_error()}")
    return int(n)


def backward(rd: RingDesc, q_local, k_blocks: Sequence, v_blocks: Sequence, out, d_out, lse, dq,
             dk_acc: Sequence, dv_acc: Sequence, workspace, compute_stream=None, copy_stream=None,
             step_events: Optional["StepEvents"] = None):
    """One device's backward pass over the whole ring (ring_attn_backward): writes
    ``dq`` and adds this device's contributions to the fp32 accumulators
    ``dk_acc[j]``, ``dv_acc[j]`` of every block j."""
    torch = _torch()
    dt = _dtype_of(rd.dtype)
    f = torch.float32
    B, Hq, Hk, D, c, n = rd.batch, rd.heads_q, rd.heads_kv, rd.head_dim, rd.local_len, rd.world
    for name, arr in (("k_blocks", k_blocks), ("v_blocks", v_blocks), ("dk_acc", dk_acc), ("dv_acc", dv_acc)):
        if len(arr) != n:
            raise ValueError(f"need {n} {name}")

    def ptrs(arr, dtype, name):
        return (ctypes.c_void_p * n)(*[_ptr(t, dtype, (B, Hk, c, D), f"{name}[{i}]").value
                                      for i, t in enumerate(arr)])

    ev = None
    if step_events is not None:
        if step_events.n != 2 * n:
            raise ValueError("step_events must hold 2 * world events")
        ev = step_events.array
    ws = _ptr(workspace, torch.uint8, (workspace.numel(),), "workspace")
    _check(lib().ring_attn_backward(
        ctypes.byref(rd), _ptr(q_local, dt, (B, Hq, c, D), "q_local"), ptrs(k_blocks, dt, "k_blocks"),
        ptrs(v_blocks, dt, "v_blocks"), _ptr(out, dt, (B, Hq, c, D), "out"), _ptr(d_out, dt, (B, Hq, c, D), "d_out"),
        _ptr(lse, f, (B, Hq, c), "lse"), _ptr(dq, dt, (B, Hq, c, D), "dq"), ptrs(dk_acc, f, "dk_acc"),
        ptrs(dv_acc, f, "dv_acc"), ws, workspace.numel(), _stream(compute_stream),
        None if copy_stream is None else ctypes.c_void_p(copy_stream.cuda_stream), ev), "ring_attn_backward")


class StepEvents:
    """A set of timing-enabled HIP events owned by the library."""

    def __init__(self, n: int):
        self.n = n
        self.array = (ctypes.c_void_p * n)()
        _check(lib().ring_attn_events_create(n, self.array), "events_create")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        _check(lib().ring_attn_event_elapsed_ms(self.array[i], self.array[j], ctypes.byref(ms)), "elapsed")
        return float(ms.value)

    def close(self):
        if self.array is not None:
            lib().ring_attn_events_destroy(self.n, self.array)
            self.array = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def synchronize(stream=None):
    _check(lib().ring_attn_synchronize(_stream(stream)), "synchronize")


def release_thread_events():
    """Destroy the drivers' cached ordering events of the calling thread
    (ring_attn_release_thread_events); later driver calls recreate them."""
    _check(lib().ring_attn_release_thread_events(), "release_thread_events")


def mfma_probe(blocks: int, iters: int, sink, stamps, stream=None):
    """Enqueue the matrix-core probe (ring_attn_mfma_probe): ``sink`` float32 [blocks*256] and
    ``stamps`` int64 [blocks*4] on the GPU; it performs blocks*4*iters*4*32768 FLOP."""
    torch = _torch()
    _check(lib().ring_attn_mfma_probe(int(blocks), int(iters), _ptr(sink, torch.float32, (blocks * 256,), "sink"),
                                      _ptr(stamps, torch.int64, (blocks * 4,), "stamps"), _stream(stream)),
           "mfma_probe")
