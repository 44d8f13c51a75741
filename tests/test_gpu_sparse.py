"""GPU parity of the sparse (selected-keys) mode, mla_decode_sparse_fwd,
against the fp64 oracle of oracle/mla_sparse_oracle.py (MI355X only).

Bar as for the dense path: max|O_gpu - O_ref| <= 1e-2 * max|O_ref| and
|LSE_gpu - LSE_ref| <= 1e-3 on rows with a counted entry; rows without one
must give exactly O = 0 and LSE = -inf.
"""
import math

import numpy as np
import pytest
import torch

from oracle import decode_sparse
from workloads import WORKLOADS, build_inputs, draw_topk_indices, make_inputs

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


def _say(msg):
    print(msg, flush=True)


def _run(mla, inp, indices, parts=None, causal=None):
    g = inp.to("cuda")
    causal = inp.causal if causal is None else causal
    out, lse = mla.sparse_fwd(g.q, g.kcache, g.block_table, g.seqlens, indices.cuda(), inp.scale,
                              causal, parts=parts)
    torch.cuda.synchronize()
    return out, lse


def _assert_parity(out, lse, O_ref, L_ref, reqs=None, tag=""):
    O = out.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    if reqs is not None:
        O, L, O_ref, L_ref = O[reqs], L[reqs], O_ref[reqs], L_ref[reqs]
    assert not np.any(np.isnan(O)), f"{tag}: NaN in O"
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), f"{tag}: -inf rows differ"
    if np.any(~fin):
        assert np.all(L[~fin] == -np.inf) and np.all(O[~fin] == 0.0), f"{tag}: empty rows"
    tol_o = TOL_O * float(np.max(np.abs(O_ref[fin]))) if np.any(fin) else 0.0
    err_o = float(np.max(np.abs(O - O_ref))) if O.size else 0.0
    err_l = float(np.max(np.abs(L[fin] - L_ref[fin]))) if np.any(fin) else 0.0
    _say(f"  {tag}: max|dO|={err_o:.3e} (tol {tol_o:.3e}) max|dLSE|={err_l:.3e}")
    assert err_o <= tol_o, f"{tag}: O error {err_o} > {tol_o}"
    assert err_l <= TOL_LSE, f"{tag}: LSE error {err_l}"


LENS = [1, 63, 64, 65, 300, 0, 2000, 129]


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
@pytest.mark.parametrize("s_q,topk", [(1, 32), (1, 96), (2, 64), (4, 256)])
@pytest.mark.parametrize("parts", [None, 5])
def test_sparse_small(mla, h_q, s_q, topk, parts):
    _say(f"case sparse h_q={h_q} s_q={s_q} topk={topk} parts={parts}")
    inp = build_inputs(LENS, s_q, h_q, seed=1100 + h_q + s_q + topk, extra_pool=5)
    g = torch.Generator().manual_seed(h_q * 7 + topk)
    ix = draw_topk_indices(LENS, s_q, topk, inp.causal, g, pad_frac=0.15)
    out, lse = _run(mla, inp, ix, parts)
    O_ref, L_ref = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale,
                                 inp.causal)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"sparse h{h_q} s{s_q} k{topk} P={parts}")


@pytest.mark.parametrize("h_q", [32, 128])   # 64-row tiles; the 128-row (row-wave) kernel
def test_sparse_edge_entries(mla, h_q):
    """Duplicates, padding, positions at/after the limit, future positions of
    an earlier token, an all-padding item and a zero-length request."""
    _say(f"case sparse edge entries h_q={h_q}")
    lens = [200, 0, 100, 70]
    inp = build_inputs(lens, 2, h_q, seed=1201, extra_pool=3)
    g = torch.Generator().manual_seed(12)
    ix = draw_topk_indices(lens, 2, 64, True, g)
    ix[0, 0, :4] = torch.tensor([5, 5, 5, 199], dtype=torch.int32)   # dup; 199 beyond token 0
    ix[0, 1, :3] = torch.tensor([199, 200, -5], dtype=torch.int32)
    ix[2, 0] = -1                                                      # nothing counts
    ix[3, 1, :2] = torch.tensor([10 ** 6, 69], dtype=torch.int32)
    out, lse = _run(mla, inp, ix)
    O_ref, L_ref = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale,
                                 True)
    assert np.all(L_ref[2, 0] == -np.inf) and np.all(L_ref[1] == -np.inf)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"sparse edges h{h_q}")


@pytest.mark.parametrize("h_q", [64, 128])
def test_sparse_all_visible_matches_dense(mla, h_q):
    """Selecting every visible position is the dense mode: the two GPU paths
    agree to the bar, and each agrees with its oracle."""
    _say(f"case sparse = dense h_q={h_q}")
    lens = [64, 96, 160, 20]
    inp = build_inputs(lens, 1, h_q, seed=1202, extra_pool=2)
    ix = torch.full((4, 1, 160), -1, dtype=torch.int32)
    for b, L in enumerate(lens):
        ix[b, 0, :L] = torch.arange(L, dtype=torch.int32)
    out_s, lse_s = _run(mla, inp, ix)
    g = inp.to("cuda")
    out_d, lse_d = mla.fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, False)
    torch.cuda.synchronize()
    O_d = out_d.float().cpu().numpy().astype(np.float64)
    L_d = lse_d.cpu().numpy().astype(np.float64)
    _assert_parity(out_s, lse_s, O_d, L_d, tag="sparse vs dense GPU")


def test_sparse_run_to_run_bitwise(mla):
    _say("case sparse determinism")
    lens = [3000, 500, 64]
    inp = build_inputs(lens, 1, 128, seed=1203, extra_pool=3)
    ix = draw_topk_indices(lens, 1, 512, False, torch.Generator().manual_seed(13), 0.1)
    a = _run(mla, inp, ix)
    b = _run(mla, inp, ix)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def test_sparse_full_workload(mla):
    """The sparse workload (64 x 2048 selected positions of 8K-32K contexts)
    in the benchmark's launch configuration; every request vs the oracle."""
    _say("case sparse full: generating inputs")
    inp = make_inputs("sparse")
    _say("case sparse full: decode on GPU")
    out, lse = _run(mla, inp, inp.indices)
    _say(f"case sparse full: oracle on all {inp.batch} requests")
    O_ref, L_ref = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.indices,
                                 inp.scale, inp.causal)
    _assert_parity(out, lse, O_ref, L_ref, tag="sparse full")
    assert not torch.isnan(out.float()).any().item()
    assert torch.isfinite(lse).all().item()


# ------------------------------------------------ sparse mode over FP8 pages

def _run_fp8(mla, inp, indices, parts=None, causal=None):
    g = inp.to("cuda")
    causal = inp.causal if causal is None else causal
    out, lse = mla.sparse_fwd_fp8(g.q, g.kcache, g.block_table, g.seqlens, indices.cuda(),
                                  inp.scale, causal, parts=parts)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
@pytest.mark.parametrize("s_q,topk", [(1, 32), (1, 96), (2, 64), (4, 256)])
@pytest.mark.parametrize("parts", [None, 5])
def test_sparse_fp8_small(mla, h_q, s_q, topk, parts):
    from oracle import decode_sparse_fp8
    from workloads import build_fp8_inputs
    _say(f"case sparse fp8 h_q={h_q} s_q={s_q} topk={topk} parts={parts}")
    inp = build_fp8_inputs(LENS, s_q, h_q, seed=1300 + h_q + s_q + topk, extra_pool=5)
    g = torch.Generator().manual_seed(h_q * 11 + topk)
    ix = draw_topk_indices(LENS, s_q, topk, inp.causal, g, pad_frac=0.15)
    out, lse = _run_fp8(mla, inp, ix, parts)
    O_ref, L_ref = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix,
                                     inp.scale, inp.causal)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"sparse fp8 h{h_q} s{s_q} k{topk} P={parts}")


@pytest.mark.parametrize("h_q", [32, 128])
def test_sparse_fp8_edge_entries(mla, h_q):
    """Duplicates, padding, positions at/after the limit, an all-padding item
    and a zero-length request, over FP8 pages."""
    from oracle import decode_sparse_fp8
    from workloads import build_fp8_inputs
    _say(f"case sparse fp8 edge entries h_q={h_q}")
    lens = [200, 0, 100, 70]
    inp = build_fp8_inputs(lens, 2, h_q, seed=1401, extra_pool=3)
    g = torch.Generator().manual_seed(14)
    ix = draw_topk_indices(lens, 2, 64, True, g)
    ix[0, 0, :4] = torch.tensor([5, 5, 5, 199], dtype=torch.int32)
    ix[0, 1, :3] = torch.tensor([199, 200, -5], dtype=torch.int32)
    ix[2, 0] = -1
    ix[3, 1, :2] = torch.tensor([10 ** 6, 69], dtype=torch.int32)
    out, lse = _run_fp8(mla, inp, ix)
    O_ref, L_ref = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix,
                                     inp.scale, True)
    assert np.all(L_ref[2, 0] == -np.inf) and np.all(L_ref[1] == -np.inf)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"sparse fp8 edges h{h_q}")


@pytest.mark.parametrize("h_q", [64, 128])
def test_sparse_fp8_all_visible_matches_dense_fp8(mla, h_q):
    """Selecting every visible position is the dense FP8 mode: the two GPU
    paths agree to the bar."""
    from workloads import build_fp8_inputs
    _say(f"case sparse fp8 = dense fp8 h_q={h_q}")
    lens = [64, 96, 160, 20]
    inp = build_fp8_inputs(lens, 1, h_q, seed=1402, extra_pool=2)
    ix = torch.full((4, 1, 160), -1, dtype=torch.int32)
    for b, L in enumerate(lens):
        ix[b, 0, :L] = torch.arange(L, dtype=torch.int32)
    out_s, lse_s = _run_fp8(mla, inp, ix)
    g = inp.to("cuda")
    out_d, lse_d = mla.fwd_fp8(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, False)
    torch.cuda.synchronize()
    _assert_parity(out_s, lse_s, out_d.float().cpu().numpy().astype(np.float64),
                   lse_d.cpu().numpy().astype(np.float64), tag="sparse fp8 vs dense fp8 GPU")


def test_sparse_fp8_run_to_run_bitwise(mla):
    from workloads import build_fp8_inputs
    _say("case sparse fp8 determinism")
    lens = [3000, 500, 64]
    inp = build_fp8_inputs(lens, 1, 128, seed=1403, extra_pool=3)
    ix = draw_topk_indices(lens, 1, 512, False, torch.Generator().manual_seed(15), 0.1)
    a = _run_fp8(mla, inp, ix)
    b = _run_fp8(mla, inp, ix)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])


def test_sparse_fp8_full_workload(mla):
    """The sparse workload over FP8 pages in the benchmark's launch
    configuration; every request vs the oracle."""
    from oracle import decode_sparse_fp8
    _say("case sparse fp8 full: generating inputs")
    inp = make_inputs("sparse", kv_format="fp8")
    _say("case sparse fp8 full: decode on GPU")
    out, lse = _run_fp8(mla, inp, inp.indices)
    _say(f"case sparse fp8 full: oracle on all {inp.batch} requests")
    O_ref, L_ref = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens,
                                     inp.indices, inp.scale, inp.causal)
    _assert_parity(out, lse, O_ref, L_ref, tag="sparse fp8 full")
    assert not torch.isnan(out.float()).any().item()
    assert torch.isfinite(lse).all().item()
