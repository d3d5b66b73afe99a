"""GPU: a decode step captured once in a HIP graph (torch.cuda.CUDAGraph over
the library's launches on the capturing stream; the step records no memset
or copy, only its kernels) replays to the eager step's result bit for bit,
every replay, with eager decode steps of other queries and budgets run
between the replays."""
import pytest
import torch

from synth import config_by_name

pytestmark = pytest.mark.gpu


def test_decode_step_graph_replays():
    import bit_plane_key_amd as b
    from bit_plane_key_amd import workloads as wl
    cfg = config_by_name("c2")
    print("building c2 cache", flush=True)
    cache = wl.build_cache(cfg)
    q = wl.queries(cfg)
    q_other = (q.float() * -0.5).to(torch.bfloat16)
    scale = wl.softmax_scale(cfg)
    k, budget = cfg.k, 88
    shape = (cfg.seqs, 1, cfg.heads, cfg.group)
    ws = torch.empty(b.workspace_bytes(cache, b.BPK_OP_DECODE, 0, 1, k), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((*shape, 128), dtype=torch.float32, device="cuda")
    idx = torch.empty((*shape, k), dtype=torch.int32, device="cuda")
    ref_idx = torch.empty_like(idx)
    ref_out = b.decode_step(cache, q, 0, 1, budget, k, scale, idx_out=ref_idx)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.decode_step(cache, q, 0, 1, budget, k, scale, out=out, idx_out=idx, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        b.decode_step(cache, q, 0, 1, budget, k, scale, out=out, idx_out=idx, ws=ws)
    for r in range(3):
        out.fill_(1.0)
        idx.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_idx), f"replay {r}: indices"
        assert torch.equal(out, ref_out), f"replay {r}: outputs"
        # eager steps between replays, on the graph's workspace too
        b.decode_step(cache, q_other, 0, 1, 64, k, scale, ws=ws)
        b.decode_step(cache, q_other, 0, 1, budget, k, scale)
        torch.cuda.synchronize()
