"""The absorbed decode step captured in a HIP graph (the way bench.py times
it) replays to the same bits as the eager launches, with the program's own
eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

from head_latent_attention_mla_amd import workloads as W

from test_gpu_parity import SCALE

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from head_latent_attention_mla_amd import mla as m
    return m


@pytest.mark.parametrize("kind", ["dense", "sparse"])
def test_decode_step_graph_replays_match_eager(mla, kind):
    w = W.Workload("graph", B=4, H=128, s_q=1, causal=False, T=700, seed=91, topk=128 if kind == "sparse" else None)
    inp = W.generate(w)
    q, w_uk, w_uv, cache = W.to_torch(inp)
    B, s_q, H = w.B, w.s_q, w.H
    N = B * s_q
    q_lat = torch.empty((B, s_q, H, 576), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, s_q, H, 128), dtype=torch.bfloat16, device="cuda")
    if kind == "sparse":
        sel, cnt = W.generate_selection(inp)
        sel_idx, sel_count = torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda()
        scan_len = int(sel.shape[1])
        ws = torch.empty(mla.sparse_workspace_bytes(B, s_q, H, scan_len), dtype=torch.uint8, device="cuda")
    else:
        scan_len = cache.max_seqlen
        ws = torch.empty(mla.decode_workspace_bytes(B, s_q, H, scan_len), dtype=torch.uint8, device="cuda")

    def step():
        mla.absorb_q(q.view(N, H, -1), w_uk, out=q_lat.view(N, H, -1))
        # bf16 split partials, as in the timed decode step
        if kind == "sparse":
            mla.sparse_decode_partial(q_lat, cache, sel_idx, sel_count, SCALE, workspace=ws, part_dtype=torch.bfloat16)
        else:
            mla.decode_partial(q_lat, cache, SCALE, False, workspace=ws, part_dtype=torch.bfloat16)
        mla.decode_combine_out(ws, w_uv, B, s_q, H, scan_len, out=out.view(N, H, -1), part_dtype=torch.bfloat16)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for r in range(4):
        out.zero_()
        ws.fill_(0xFF)                 # poison the workspace between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"
        # eager work on the same buffers between replays
        step()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"eager after replay {r}"
