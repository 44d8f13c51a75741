"""Checked mode (MLA_DEBUG_SYNC=1 in the environment): every launch of the
library is followed by a wait on its stream, so a kernel fault would be
reported by the call that launched it.  These tests check that the mode
changes nothing but the waiting:

* the call returns only once its stream has drained (work queued ahead of
  it on the same stream included);
* outputs are bit-identical to the asynchronous mode for the dense decode
  (both cache formats), the sparse decode and the append;
* a stream under graph capture is not waited on: capture succeeds and the
  replays match the eager step bit for bit.
"""
import pytest
import torch

from workloads import build_fp8_inputs, build_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _busy(n=12):
    """Queue a few milliseconds of unrelated work on the current stream."""
    a = torch.randn((4096, 4096), device="cuda", dtype=torch.bfloat16)
    for _ in range(n):
        a = (a @ a).mul_(1e-3)
    return a


def test_checked_call_returns_after_its_stream_drains(mla, monkeypatch):
    print("case checked mode waits", flush=True)
    inp = build_inputs([3000, 700, 4096, 65], 1, 128, seed=811)
    g = inp.to("cuda")
    ref = mla.fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal)
    torch.cuda.synchronize()
    monkeypatch.setenv("MLA_DEBUG_SYNC", "1")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _busy()
        out, lse = mla.fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal)
        assert side.query(), "the checked call returned before its stream drained"
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(lse, ref[1])


@pytest.mark.parametrize("value", ["1", "yes"])
def test_checked_mode_same_bits(mla, monkeypatch, value):
    print(f"case checked mode bits MLA_DEBUG_SYNC={value}", flush=True)
    d = build_inputs([1000, 64, 3000, 1, 0, 2049], 2, 64, seed=812, extra_pool=2)
    f = build_fp8_inputs([900, 4000, 65, 0, 1300], 1, 128, seed=813, extra_pool=2)
    gd, gf = d.to("cuda"), f.to("cuda")
    idx = torch.randint(0, 1000, (d.batch, d.s_q, 128), generator=torch.Generator().manual_seed(5),
                        dtype=torch.int32).cuda()
    new = torch.randn((d.batch, d.s_q, 576), generator=torch.Generator().manual_seed(6)).to(
        torch.bfloat16).cuda()

    def run():
        kc = gd.kcache.clone()
        mla.kv_append(new, kc, gd.block_table, gd.seqlens)
        a = mla.fwd(gd.q, kc, gd.block_table, gd.seqlens, d.scale, d.causal)
        b = mla.fwd_fp8(gf.q, gf.kcache, gf.block_table, gf.seqlens, f.scale, f.causal)
        c = mla.sparse_fwd(gd.q, gd.kcache, gd.block_table, gd.seqlens, idx, d.scale)
        torch.cuda.synchronize()
        return [kc, *a, *b, *c]

    monkeypatch.delenv("MLA_DEBUG_SYNC", raising=False)
    ref = run()
    monkeypatch.setenv("MLA_DEBUG_SYNC", value)
    got = run()
    for i, (x, y) in enumerate(zip(got, ref)):    # bits: the cache holds NaN sentinels
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), \
            f"output {i} differs in checked mode"


def test_checked_mode_under_graph_capture(mla, monkeypatch):
    print("case checked mode graph capture", flush=True)
    s_q, h_q = 1, 128
    inp = build_inputs([1000, 65, 0, 300, 2049], s_q, h_q, seed=814)
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
    monkeypatch.setenv("MLA_DEBUG_SYNC", "1")
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
        lse.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {rep} differs"
