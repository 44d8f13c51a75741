"""Block-table entries that name no page of the pool (negative or >= the pool
size), and slots past the table's columns, on MI355X: the positions they
cover hold no key and are left out of the attention, in the dense and the
sparse mode alike.  Checked against the fp64 oracles, which take the same
reading, over the very same table.
"""
import numpy as np
import pytest
import torch

from oracle import decode, decode_fp8, decode_sparse, decode_sparse_fp8
from workloads import build_fp8_inputs, build_inputs, draw_topk_indices

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _check(out, lse, O_ref, L_ref, tag):
    O = out.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), tag
    tol = TOL_O * float(np.max(np.abs(O_ref[fin])))
    assert float(np.max(np.abs(O - O_ref))) <= tol, tag
    assert float(np.max(np.abs(L[fin] - L_ref[fin]))) <= TOL_LSE, tag


def _unmap(bt, n_pool):
    bt = bt.clone()
    bt[0, 1] = n_pool + 5
    bt[1, 0] = -3
    bt[2, 2] = 1 << 30
    return bt


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (32, 2), (64, 2)])
def test_dense_unmapped_pages_are_skipped(mla, kv, h_q, s_q):
    print(f"case unmapped dense {kv} h_q={h_q} s_q={s_q}", flush=True)
    fp8 = kv == "fp8"
    lens = [200, 130, 300]
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, s_q, h_q, seed=77, extra_pool=3)
    n_pool = int(inp.kcache.shape[0])
    bt = _unmap(inp.block_table, n_pool)
    g = inp.to("cuda")
    fwd = mla.fwd_fp8 if fp8 else mla.fwd
    out, lse = fwd(g.q, g.kcache, bt.cuda(), g.seqlens, inp.scale, inp.causal)
    torch.cuda.synchronize()
    ref = decode_fp8 if fp8 else decode
    O_ref, L_ref = ref(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, inp.causal)
    _check(out, lse, O_ref, L_ref, f"dense {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("h_q", [16, 128])
def test_dense_request_without_any_page(mla, kv, h_q):
    """Every slot of request 1 unmapped: its rows get O = 0, LSE = -inf; the
    other requests are unaffected."""
    print(f"case dense no page {kv} h_q={h_q}", flush=True)
    fp8 = kv == "fp8"
    inp = (build_fp8_inputs if fp8 else build_inputs)([200, 130, 300], 1, h_q, seed=80,
                                                       extra_pool=3)
    bt = inp.block_table.clone()
    bt[1, :] = -1
    g = inp.to("cuda")
    fwd = mla.fwd_fp8 if fp8 else mla.fwd
    out, lse = fwd(g.q, g.kcache, bt.cuda(), g.seqlens, inp.scale, inp.causal)
    torch.cuda.synchronize()
    assert torch.all(out[1] == 0)
    assert torch.all(torch.isneginf(lse[1]))
    ref = decode_fp8 if fp8 else decode
    O_ref, L_ref = ref(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, inp.causal)
    _check(out, lse, O_ref, L_ref, f"dense no page {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sparse_unmapped_pages_are_skipped(mla, kv):
    print(f"case unmapped sparse {kv}", flush=True)
    fp8 = kv == "fp8"
    lens = [200, 130, 300]
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, 1, 64, seed=78, extra_pool=3)
    n_pool = int(inp.kcache.shape[0])
    bt = _unmap(inp.block_table, n_pool)
    ix = draw_topk_indices(lens, 1, 96, False, torch.Generator().manual_seed(11))
    g = inp.to("cuda")
    fn = mla.sparse_fwd_fp8 if fp8 else mla.sparse_fwd
    out, lse = fn(g.q, g.kcache, bt.cuda(), g.seqlens, ix.cuda(), inp.scale, False)
    torch.cuda.synchronize()
    ref = decode_sparse_fp8 if fp8 else decode_sparse
    O_ref, L_ref = ref(inp.q, inp.kcache, bt, inp.seqlens, ix, inp.scale, False)
    _check(out, lse, O_ref, L_ref, f"sparse {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_skips_unmapped_pages(mla, kv):
    """The append writes nothing for new tokens whose page slot names no page
    of the pool; the whole cache equals the oracle's bit for bit."""
    from oracle import kv_append, kv_append_fp8
    print(f"case unmapped append {kv}", flush=True)
    fp8 = kv == "fp8"
    lens = [200, 130, 300]
    s_q = 4
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, s_q, 16, seed=79, extra_pool=3)
    n_pool = int(inp.kcache.shape[0])
    bt = inp.block_table.clone()
    bt[0, 3] = n_pool + 1         # the page of request 0's new tokens (positions 196..199)
    bt[2, 4] = -1                 # request 2's new tokens (296..299)
    new = torch.randn((3, s_q, 576), generator=torch.Generator().manual_seed(12)).to(torch.bfloat16)
    g = inp.to("cuda")
    fn = mla.kv_append_fp8 if fp8 else mla.kv_append
    fn(new.cuda(), g.kcache, bt.cuda(), g.seqlens)
    torch.cuda.synchronize()
    ref = (kv_append_fp8 if fp8 else kv_append)(inp.kcache, bt, inp.seqlens, new)
    ref = torch.as_tensor(ref)
    got = g.kcache.cpu()
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))


# Lengths that run past the table's columns (bt_stride): the positions beyond
# it hold no key in either mode, and the append writes nothing there.
def _short_table(inp, cols):
    return inp.block_table[:, :cols].contiguous()


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 2)])
def test_dense_slots_beyond_table_are_skipped(mla, kv, h_q, s_q):
    print(f"case dense beyond table {kv} h_q={h_q} s_q={s_q}", flush=True)
    fp8 = kv == "fp8"
    lens = [200, 130, 300]          # 4, 3 and 5 pages; the table keeps 3 columns
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, s_q, h_q, seed=81, extra_pool=3)
    bt = _short_table(inp, 3)
    g = inp.to("cuda")
    fwd = mla.fwd_fp8 if fp8 else mla.fwd
    out, lse = fwd(g.q, g.kcache, bt.cuda(), g.seqlens, inp.scale, inp.causal)
    torch.cuda.synchronize()
    ref = decode_fp8 if fp8 else decode
    O_ref, L_ref = ref(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, inp.causal)
    _check(out, lse, O_ref, L_ref, f"dense beyond table {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sparse_slots_beyond_table_are_skipped(mla, kv):
    print(f"case sparse beyond table {kv}", flush=True)
    fp8 = kv == "fp8"
    lens = [200, 130, 300]
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, 1, 64, seed=82, extra_pool=3)
    bt = _short_table(inp, 3)
    ix = draw_topk_indices(lens, 1, 128, False, torch.Generator().manual_seed(15))
    g = inp.to("cuda")
    fn = mla.sparse_fwd_fp8 if fp8 else mla.sparse_fwd
    out, lse = fn(g.q, g.kcache, bt.cuda(), g.seqlens, ix.cuda(), inp.scale, False)
    torch.cuda.synchronize()
    ref = decode_sparse_fp8 if fp8 else decode_sparse
    O_ref, L_ref = ref(inp.q, inp.kcache, bt, inp.seqlens, ix, inp.scale, False)
    _check(out, lse, O_ref, L_ref, f"sparse beyond table {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_skips_slots_beyond_table(mla, kv):
    from oracle import kv_append, kv_append_fp8
    print(f"case append beyond table {kv}", flush=True)
    fp8 = kv == "fp8"
    lens, s_q = [200, 130, 300], 4   # new tokens at slots 3, 2 and 4: two beyond 3 columns
    inp = (build_fp8_inputs if fp8 else build_inputs)(lens, s_q, 16, seed=83, extra_pool=3)
    bt = _short_table(inp, 3)
    new = torch.randn((3, s_q, 576), generator=torch.Generator().manual_seed(16)).to(torch.bfloat16)
    g = inp.to("cuda")
    fn = mla.kv_append_fp8 if fp8 else mla.kv_append
    fn(new.cuda(), g.kcache, bt.cuda(), g.seqlens)
    torch.cuda.synchronize()
    ref = torch.as_tensor((kv_append_fp8 if fp8 else kv_append)(inp.kcache, bt, inp.seqlens, new))
    assert torch.equal(g.kcache.cpu().view(torch.uint8), ref.view(torch.uint8))
    assert not torch.equal(ref.view(torch.uint8), inp.kcache.view(torch.uint8))   # request 1 wrote
