"""ring_attn_forward_noalloc (the forward for callers that cannot allocate)
against ring_attn_forward on the same inputs, through the C ABI: bit for bit
on two calls in a row, the second on a smaller share (so stale scratch from
the first call must not leak into it), bf16 and fp32; a share past the
scratch size is refused with nothing written."""
import numpy as np
import pytest

import ring_inputs
import ring_attention_blockwise_amd as ra
from ring_attention_blockwise_amd import harness

pytestmark = pytest.mark.gpu

W = ring_inputs.WORKLOADS


def _both(share):
    """(out, lse) of the workspace forward and of the no-allocation forward."""
    import torch
    ref_out, ref_lse = harness.run_forward(share, copy_stream=None)
    out = torch.full_like(ref_out, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    ra.forward_noalloc(share.ring_desc(), share.q, share.k_blocks, share.v_blocks, out, lse)
    torch.cuda.synchronize()
    return (ref_out, ref_lse), (out, lse)


def test_noalloc_matches_forward_on_two_calls_the_second_smaller(gpu):
    import torch
    big = W["zigzag8k_8dev_d128"]                                            # ~12.6 MB of scratch
    small = big.with_(heads_q=4, heads_kv=2, world=4, local_len=512, seed=2024)  # ~1.1 MB, GQA
    for wl, rank in ((big, 0), (small, 3)):
        print(f"no-alloc forward: {wl.name} {wl.heads_q}/{wl.heads_kv} heads, world {wl.world}, "
              f"local {wl.local_len}, rank {rank}", flush=True)
        share = harness.build_share(wl, rank, gpu)
        (ref_out, ref_lse), (out, lse) = _both(share)
        assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)


def test_noalloc_matches_forward_fp32_and_repeats(gpu):
    import torch
    wl = W["ring4_noncausal_f32"]
    share = harness.build_share(wl, 2, gpu)
    first = None
    for _ in range(2):
        (ref_out, ref_lse), (out, lse) = _both(share)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        if first is None:
            first = (out.clone(), lse.clone())
    assert torch.equal(first[0], out) and torch.equal(first[1], lse)


def test_noalloc_refuses_a_share_past_the_scratch(gpu):
    """A 1M-token-style share with a 4096-row local block needs more than the
    scratch holds: refused before anything is enqueued (outputs untouched)."""
    import torch
    wl = W["zigzag8k_8dev_d128"].with_(local_len=8192, world=2, heads_q=8, heads_kv=8)
    rd = harness.make_ring_desc(wl, 0)
    assert ra.forward_workspace_size(rd) - 256 > ra.NOALLOC_SCRATCH_BYTES
    dt = torch.bfloat16
    q = torch.zeros((1, 8, 8192, 128), dtype=dt, device=gpu)
    kv = [torch.zeros((1, 8, 8192, 128), dtype=dt, device=gpu) for _ in range(2)]
    out = torch.full((1, 8, 8192, 128), 7.0, dtype=dt, device=gpu)
    lse = torch.full((1, 8, 8192), 7.0, dtype=torch.float32, device=gpu)
    with pytest.raises(ra.RingAttnError) as err:
        ra.forward_noalloc(rd, q, kv, kv, out, lse)
    assert err.value.code == ra.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())
