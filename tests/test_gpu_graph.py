"""A whole-device forward (ring_attn_forward, two streams) and a whole-device
backward (ring_attn_backward) captured into a HIP graph and replayed give the
eager result bit for bit on every replay, with eager work and
synchronisation between the replays."""
import pytest

import ring_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["zigzag8k_8dev_d128", "ring4_noncausal_f32"])
def test_forward_graph_replays_match_eager(gpu, name):
    import torch
    from ring_attention_blockwise_amd import harness

    wl = ring_inputs.WORKLOADS[name]
    dev = torch.device("cuda:0")
    share = harness.build_share(wl, wl.ranks[0], dev)
    copy_stream = torch.cuda.Stream()

    out_e, lse_e = harness.alloc_outputs(share)
    harness.run_forward(share, copy_stream=copy_stream, workspace=harness.alloc_workspace(share),
                        out=out_e, lse=lse_e)
    torch.cuda.synchronize()

    out_g, lse_g = harness.alloc_outputs(share)
    ws_g = harness.alloc_workspace(share)
    # one eager call first: the library creates its ordering events outside capture
    harness.run_forward(share, copy_stream=copy_stream, workspace=ws_g, out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        harness.run_forward(share, copy_stream=copy_stream, workspace=ws_g, out=out_g, lse=lse_g)
    torch.cuda.synchronize()
    for replay in range(3):
        out_g.fill_(float("nan"))
        lse_g.fill_(float("nan"))
        ws_g.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, out_e), f"replay {replay}: output differs from the eager forward"
        assert torch.equal(lse_g, lse_e), f"replay {replay}: LSE differs from the eager forward"


@pytest.mark.parametrize("name", ["bwd_zigzag4k_4dev_gqa", "bwd_f32_zigzag1k_4dev"])
def test_backward_graph_replays_match_eager(gpu, name):
    import torch
    import ring_attention_blockwise_amd as ra
    from ring_attention_blockwise_amd import harness

    wl = ring_inputs.BACKWARD_WORKLOADS[name]
    dev = torch.device("cuda:0")
    share = harness.build_share(wl, 1, dev)
    copy_stream = torch.cuda.Stream()
    out, lse = harness.run_forward(share, copy_stream=copy_stream)
    d_out = harness.build_upstream(share)
    ws = torch.empty(ra.backward_workspace_size(share.ring_desc()), dtype=torch.uint8, device=dev)

    dk_e, dv_e = harness.new_kv_grads(share)
    dq_e = harness.run_backward(share, out, lse, d_out, dk_e, dv_e, copy_stream=copy_stream, workspace=ws)
    torch.cuda.synchronize()

    dk_g, dv_g = harness.new_kv_grads(share)
    dq_g = torch.empty_like(dq_e)
    rd = share.ring_desc()

    def call():
        ra.backward(rd, share.q, share.k_blocks, share.v_blocks, out, d_out, lse, dq_g, dk_g, dv_g, ws,
                    copy_stream=copy_stream)

    call()  # eager first: the library creates its ordering events outside capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for replay in range(3):
        dq_g.fill_(float("nan"))
        ws.fill_(7)
        for x in dk_g + dv_g:
            x.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dq_g, dq_e), f"replay {replay}: dQ differs from the eager backward"
        for j in range(wl.world):
            assert torch.equal(dk_g[j], dk_e[j]) and torch.equal(dv_g[j], dv_e[j]), f"replay {replay}, block {j}"
