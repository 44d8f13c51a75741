"""The decode step (scheduler, decode kernel, combine) captured as a HIP graph
and replayed: every replay must reproduce the eager result bit for bit.

The outputs are cleared by eager work between replays, and the replays are
interleaved with other eager kernels and host synchronisations, so a replay
that silently skipped or repeated work would show up as a mismatch.
"""
import pytest
import torch

from workloads import build_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (128, 2)])
def test_graph_replays_match_eager(mla, h_q, s_q):
    print(f"case graph h_q={h_q} s_q={s_q}", flush=True)
    seqlens = [1000, 65, 0, 300, 2049, 7]
    inp = build_inputs(seqlens, s_q, h_q, seed=4242)
    g = inp.to("cuda")
    parts = mla.num_parts(inp.batch, s_q, h_q, 1, mla.device_num_cus(torch.device("cuda", 0)))
    ws = torch.zeros((max(256, mla.workspace_bytes(inp.batch, s_q, h_q, parts)),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((inp.batch, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.batch, s_q, h_q), dtype=torch.float32, device="cuda")

    def step():
        meta = mla.metadata(g.seqlens, s_q, h_q, parts=parts)
        mla.splitkv(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal, meta, ws,
                    out, lse)
        mla.combine(g.seqlens, s_q, h_q, meta, ws, out, lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        out.zero_()
        lse.fill_(123.0)
        junk.mul_(1.0001)           # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: O differs from the eager step"
        assert torch.equal(lse, ref_l), f"replay {rep}: LSE differs from the eager step"


def test_graph_decode_step_with_append(mla):
    """append + scheduler + decode + combine captured as one graph: replays
    match the eager step bit for bit (the append is idempotent here, so the
    cache is the same before every replay)."""
    print("case graph append step", flush=True)
    s_q, h_q = 2, 128
    inp = build_inputs([700, 65, 3, 2049], s_q, h_q, seed=77)
    g = inp.to("cuda")
    new = torch.randn((inp.batch, s_q, 576), generator=torch.Generator().manual_seed(3)).to(
        torch.bfloat16).cuda()
    parts = mla.num_parts(inp.batch, s_q, h_q, 1, mla.device_num_cus(torch.device("cuda", 0)))
    ws = torch.zeros((max(256, mla.workspace_bytes(inp.batch, s_q, h_q, parts)),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((inp.batch, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.batch, s_q, h_q), dtype=torch.float32, device="cuda")

    def step():
        mla.kv_append(new, g.kcache, g.block_table, g.seqlens)
        meta = mla.metadata(g.seqlens, s_q, h_q, parts=parts)
        mla.splitkv(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal, meta, ws,
                    out, lse)
        mla.combine(g.seqlens, s_q, h_q, meta, ws, out, lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l, ref_k = out.clone(), lse.clone(), g.kcache.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), f"replay {rep}: O"
        assert torch.equal(lse, ref_l), f"replay {rep}: LSE"
        assert torch.equal(g.kcache.view(torch.int16), ref_k.view(torch.int16)), f"replay {rep}"
