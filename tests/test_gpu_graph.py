"""The decode step (scheduler, decode kernel, combine) captured as a HIP graph
and replayed: every replay must reproduce the eager result bit for bit, and
the replayed output is also checked against the fp64 oracle (max|dO| <=
1e-2 * max|O_ref|, |dLSE| <= 1e-3, empty rows exactly O = 0, LSE = -inf).

The outputs are cleared by eager work between replays, and the replays are
interleaved with other eager kernels and host synchronisations, so a replay
that silently skipped or repeated work would show up as a mismatch.
"""
import numpy as np
import pytest
import torch

from oracle import decode
from workloads import build_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _assert_oracle(out, lse, O_ref, L_ref, tag):
    O = out.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), f"{tag}: -inf rows differ"
    if np.any(~fin):
        assert np.all(L[~fin] == -np.inf) and np.all(O[~fin] == 0.0), f"{tag}: empty rows"
    tol_o = 1e-2 * float(np.max(np.abs(O_ref[fin])))
    err_o = float(np.max(np.abs(O - O_ref)))
    err_l = float(np.max(np.abs(L[fin] - L_ref[fin])))
    print(f"  {tag}: max|dO|={err_o:.3e} (tol {tol_o:.3e}) max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= 1e-3, tag


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
    # the last replay's output against the oracle
    O_ref, L_ref = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale,
                          inp.causal)
    _assert_oracle(out, lse, O_ref, L_ref, f"graph replay h{h_q} s{s_q} vs oracle")


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


def _replay_matches(step, outs, reps=3, keep=()):
    """Run step eagerly, capture it, then replay `reps` times with the outputs
    cleared and unrelated eager work in between: every replay must give the
    eager bits.  Tensors in `keep` (inputs the step also writes, such as the
    cache it appends to) are compared but not cleared."""
    outs = list(outs) + list(keep)
    keep_ids = {id(k) for k in keep}
    step()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
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
    for rep in range(reps):
        for o in outs:
            if id(o) not in keep_ids:
                o.view(torch.uint8).fill_(0x5a)
        junk.mul_(1.0001)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: output {i}"


def test_graph_fp8_step_with_append(mla):
    """FP8 cache: quantising append + scheduler + decode + combine in one graph."""
    from workloads import build_fp8_inputs
    print("case graph fp8 append step", flush=True)
    s_q, h_q = 2, 64
    inp = build_fp8_inputs([700, 65, 3, 2049, 0], s_q, h_q, seed=78)
    g = inp.to("cuda")
    new = torch.randn((inp.batch, s_q, 576), generator=torch.Generator().manual_seed(4)).to(
        torch.bfloat16).cuda()
    parts = mla.num_parts(inp.batch, s_q, h_q, 1, mla.device_num_cus(torch.device("cuda", 0)))
    ws = torch.zeros((max(256, mla.workspace_bytes(inp.batch, s_q, h_q, parts)),),
                     dtype=torch.uint8, device="cuda")
    meta = mla.metadata(g.seqlens, s_q, h_q, parts=parts)
    out = torch.empty((inp.batch, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.batch, s_q, h_q), dtype=torch.float32, device="cuda")

    def step():
        mla.kv_append_fp8(new, g.kcache, g.block_table, g.seqlens)
        mla.fwd_fp8(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal, meta=meta,
                    workspace=ws, out=out, lse=lse)

    _replay_matches(step, [out, lse], keep=[g.kcache])


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_graph_sparse_step(mla, kv):
    """Sparse mode: resolve + decode + combine captured and replayed."""
    from workloads import build_fp8_inputs, draw_topk_indices
    print(f"case graph sparse {kv}", flush=True)
    fp8 = kv == "fp8"
    lens = [900, 64, 1, 2500, 0, 300]
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, 1, 128, seed=79)
    g = inp.to("cuda")
    ix = draw_topk_indices(lens, 1, 128, False, torch.Generator().manual_seed(5),
                           pad_frac=0.1).cuda()
    topk = ix.shape[2]
    parts = mla.num_parts(inp.batch, 1, 128, 1, mla.device_num_cus(torch.device("cuda", 0)))
    meta = mla.sparse_metadata(inp.batch, 1, 128, topk, "cuda", parts=parts)
    ws = torch.zeros((mla.sparse_workspace_bytes(inp.batch, 1, 128, topk, parts),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((inp.batch, 1, 128, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.batch, 1, 128), dtype=torch.float32, device="cuda")
    fn = mla.sparse_fwd_fp8 if fp8 else mla.sparse_fwd

    def step():
        fn(g.q, g.kcache, g.block_table, g.seqlens, ix, inp.scale, False, meta=meta,
           workspace=ws, out=out, lse=lse)

    _replay_matches(step, [out, lse])


def test_graph_inline_plan(mla):
    """The two-launch decode (plan inside the decode kernel) captured and replayed;
    the plan it writes is compared too."""
    print("case graph inline plan", flush=True)
    s_q, h_q = 1, 128
    inp = build_inputs([1000, 65, 0, 300, 2049, 7], s_q, h_q, seed=80)
    g = inp.to("cuda")
    parts = mla.num_parts(inp.batch, s_q, h_q, 1, mla.device_num_cus(torch.device("cuda", 0)))
    meta = mla.metadata(g.seqlens, s_q, h_q, parts=parts)   # buffers the kernel's plan goes to
    ws = torch.zeros((max(256, mla.workspace_bytes(inp.batch, s_q, h_q, parts)),),
                     dtype=torch.uint8, device="cuda")
    out = torch.empty((inp.batch, s_q, h_q, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((inp.batch, s_q, h_q), dtype=torch.float32, device="cuda")

    def step():
        mla.fwd_inline_plan(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, meta=meta,
                            workspace=ws, out=out, lse=lse)

    _replay_matches(step, [out, lse, meta.tile_meta, meta.split_offsets])
