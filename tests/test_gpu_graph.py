"""A whole-device forward (ring_attn_forward, two streams) captured into a
HIP graph and replayed gives the eager result bit for bit on every replay,
with eager work and synchronisation between the replays."""
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
