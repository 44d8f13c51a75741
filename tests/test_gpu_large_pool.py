"""Cache pools larger than 4 GiB on MI355X: page byte offsets beyond 2^31 and
2^32, for every entry point that reads or writes pages (dense and sparse
decode, both cache formats, the appends, the in-kernel plan).

The pages of a small seeded cache are copied to ids spread evenly over a
large all-zero pool on the GPU (in shuffled order, so the table order is not
the address order); the block table follows the move.  The decode is checked
against the fp64 oracle run on the small cache with the original ids, the
append by reading the moved pages back and comparing them bit for bit with
the oracle's append on the small cache.
"""
import numpy as np
import pytest
import torch

from oracle import decode, decode_fp8, decode_sparse, decode_sparse_fp8, kv_append, kv_append_fp8
from workloads import build_fp8_inputs, build_inputs, draw_topk_indices

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3
PAGE_BYTES = {"bf16": 64 * 576 * 2, "fp8": 41216}
# pool sizes that put 2^32 bytes near the middle of the pool (~8.6 GB each)
BIG_POOL = {"bf16": 116_510, "fp8": 208_414}


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
    err_o = float(np.max(np.abs(O - O_ref)))
    err_l = float(np.max(np.abs(L[fin] - L_ref[fin])))
    print(f"  {tag}: max|dO|={err_o:.3e} (tol {tol:.3e}) max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= tol, tag
    assert err_l <= TOL_LSE, tag


def _spread(inp, kv, seed):
    """The small cache moved into a large zero pool on the GPU; returns the
    pool, the moved block table (on the GPU) and the new id of every page."""
    n_small = int(inp.kcache.shape[0])
    nb = BIG_POOL[kv]
    step = nb // n_small
    g = torch.Generator().manual_seed(seed)
    new_id = torch.randperm(n_small, generator=g) * step + int(
        torch.randint(0, step, (1,), generator=g))
    hi = int(new_id.max()) * PAGE_BYTES[kv]
    lo = int(new_id.min()) * PAGE_BYTES[kv]
    assert lo < 2**31 and hi > 2**32 + 2**30, (lo, hi)
    big = torch.zeros((nb,) + tuple(inp.kcache.shape[1:]), dtype=inp.kcache.dtype,
                      device="cuda")
    big[new_id.cuda()] = inp.kcache.cuda()
    bt = new_id[inp.block_table.long()].to(torch.int32)
    return big, bt.cuda(), new_id


LENS = [700, 64, 1, 3000, 129, 0, 2050]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("h_q,s_q", [(16, 1), (128, 1), (64, 2)])
def test_dense_decode_large_pool(mla, kv, h_q, s_q):
    print(f"case large pool dense {kv} h_q={h_q} s_q={s_q}", flush=True)
    fp8 = kv == "fp8"
    inp = (build_fp8_inputs if fp8 else build_inputs)(LENS, s_q, h_q, seed=91 + h_q + s_q,
                                                      extra_pool=3)
    big, bt, _ = _spread(inp, kv, seed=5 + h_q)
    g = inp.to("cuda")
    fwd = mla.fwd_fp8 if fp8 else mla.fwd
    out, lse = fwd(g.q, big, bt, g.seqlens, inp.scale, inp.causal)
    torch.cuda.synchronize()
    ref = decode_fp8 if fp8 else decode
    O_ref, L_ref = ref(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    _check(out, lse, O_ref, L_ref, f"dense {kv}")
    del big


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_inline_plan_large_pool(mla, kv):
    print(f"case large pool inline plan {kv}", flush=True)
    fp8 = kv == "fp8"
    inp = (build_fp8_inputs if fp8 else build_inputs)(LENS, 1, 128, seed=97, extra_pool=3)
    big, bt, _ = _spread(inp, kv, seed=6)
    g = inp.to("cuda")
    out, lse = mla.fwd_inline_plan(g.q, big, bt, g.seqlens, inp.scale, fp8=fp8)
    torch.cuda.synchronize()
    ref = decode_fp8 if fp8 else decode
    O_ref, L_ref = ref(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    _check(out, lse, O_ref, L_ref, f"inline plan {kv}")
    del big


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sparse_decode_large_pool(mla, kv):
    print(f"case large pool sparse {kv}", flush=True)
    fp8 = kv == "fp8"
    inp = (build_fp8_inputs if fp8 else build_inputs)(LENS, 1, 128, seed=98, extra_pool=3)
    big, bt, _ = _spread(inp, kv, seed=7)
    ix = draw_topk_indices(LENS, 1, 256, False, torch.Generator().manual_seed(13))
    g = inp.to("cuda")
    fn = mla.sparse_fwd_fp8 if fp8 else mla.sparse_fwd
    out, lse = fn(g.q, big, bt, g.seqlens, ix.cuda(), inp.scale, False)
    torch.cuda.synchronize()
    ref = decode_sparse_fp8 if fp8 else decode_sparse
    O_ref, L_ref = ref(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, False)
    _check(out, lse, O_ref, L_ref, f"sparse {kv}")
    del big


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_append_large_pool(mla, kv):
    print(f"case large pool append {kv}", flush=True)
    fp8 = kv == "fp8"
    s_q = 5
    inp = (build_fp8_inputs if fp8 else build_inputs)(LENS, s_q, 16, seed=99, extra_pool=3)
    big, bt, new_id = _spread(inp, kv, seed=8)
    new = torch.randn((len(LENS), s_q, 576),
                      generator=torch.Generator().manual_seed(14)).to(torch.bfloat16)
    fn = mla.kv_append_fp8 if fp8 else mla.kv_append
    fn(new.cuda(), big, bt, inp.seqlens.cuda())
    torch.cuda.synchronize()
    ref = torch.as_tensor((kv_append_fp8 if fp8 else kv_append)(inp.kcache, inp.block_table,
                                                                inp.seqlens, new))
    got = big[new_id.cuda()].cpu()
    assert torch.equal(got.view(torch.uint8), ref.view(torch.uint8))
    # nothing was written outside the moved pages
    big[new_id.cuda()] = 0
    assert int(big.view(torch.uint8).count_nonzero()) == 0
    del big
