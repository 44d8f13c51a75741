"""Randomised GPU parity: seeded random shapes, lengths, part counts and
index lists for every decode entry point (bf16 and FP8 caches, dense and
sparse modes), each case checked against the fp64 oracle to the bar of the
other parity tests: max|O_gpu - O_ref| <= 1e-2 * max|O_ref|,
|LSE_gpu - LSE_ref| <= 1e-3, exact O = 0 / LSE = -inf on rows without a
visible key.  Lengths are drawn to hit page and half-page edges (0, 1, 31,
32, 33, 63, 64, 65, ...) as well as a spread of ordinary values.  The case
list is fixed by its seed, so a failure names a reproducible case.
"""
import numpy as np
import pytest
import torch

from oracle import decode, decode_fp8, decode_sparse, decode_sparse_fp8
from workloads import build_fp8_inputs, build_inputs, draw_topk_indices

pytestmark = pytest.mark.gpu

TOL_O = 1e-2
TOL_LSE = 1e-3
EDGE_LENS = [0, 1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 191, 192, 193]


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _case(seed):
    """(seqlens, s_q, h_q, parts, topk) of random case `seed`."""
    r = np.random.default_rng(10_000 + seed)
    batch = int(r.integers(1, 9))
    s_q = int(r.choice([1, 1, 1, 2, 3, 4, 8]))
    h_q = int(r.choice([16, 32, 64, 128]))
    lens = []
    for _ in range(batch):
        if r.random() < 0.5:
            lens.append(int(r.choice(EDGE_LENS)))
        else:
            lens.append(int(r.integers(1, 1500)))
    parts = None if r.random() < 0.5 else int(r.integers(1, 40))
    topk = int(r.choice([32, 64, 96, 160]))
    return lens, s_q, h_q, parts, topk


def _check(out, lse, O_ref, L_ref, tag):
    O = out.float().cpu().numpy().astype(np.float64)
    L = lse.cpu().numpy().astype(np.float64)
    assert not np.any(np.isnan(O)), f"{tag}: NaN in O"
    fin = np.isfinite(L_ref)
    assert np.array_equal(np.isfinite(L), fin), f"{tag}: -inf rows differ"
    if np.any(~fin):
        assert np.all(L[~fin] == -np.inf) and np.all(O[~fin] == 0.0), f"{tag}: empty rows"
    if np.any(fin):
        tol_o = TOL_O * float(np.max(np.abs(O_ref[fin])))
        err_o = float(np.max(np.abs(O - O_ref)))
        err_l = float(np.max(np.abs(L[fin] - L_ref[fin])))
        assert err_o <= tol_o, f"{tag}: O error {err_o} > {tol_o}"
        assert err_l <= TOL_LSE, f"{tag}: LSE error {err_l}"


@pytest.mark.parametrize("seed", range(48))
@pytest.mark.parametrize("mode", ["bf16", "fp8", "sparse", "sparse_fp8"])
def test_random_case(mla, mode, seed):
    lens, s_q, h_q, parts, topk = _case(seed)
    tag = f"{mode} seed={seed} lens={lens} s_q={s_q} h_q={h_q} parts={parts} topk={topk}"
    print(f"case {tag}", flush=True)
    fp8 = mode in ("fp8", "sparse_fp8")
    build = build_fp8_inputs if fp8 else build_inputs
    inp = build(lens, s_q, h_q, seed=20_000 + seed, extra_pool=3)
    g = inp.to("cuda")
    if mode.startswith("sparse"):
        ix = draw_topk_indices(lens, s_q, topk, inp.causal,
                               torch.Generator().manual_seed(30_000 + seed), pad_frac=0.2)
        fn = mla.sparse_fwd_fp8 if fp8 else mla.sparse_fwd
        out, lse = fn(g.q, g.kcache, g.block_table, g.seqlens, ix.cuda(), inp.scale, inp.causal,
                      parts=parts)
        ref = decode_sparse_fp8 if fp8 else decode_sparse
        O_ref, L_ref = ref(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale,
                           inp.causal)
    else:
        fn = mla.fwd_fp8 if fp8 else mla.fwd
        out, lse = fn(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                      parts=parts)
        ref = decode_fp8 if fp8 else decode
        O_ref, L_ref = ref(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale,
                           inp.causal)
    torch.cuda.synchronize()
    _check(out, lse, O_ref, L_ref, tag)
