"""Pins of the sparse-mode oracle (oracle/mla_sparse_oracle.py) against facts
fixed outside it:

* selecting every visible position, in order, is the dense definition: equal
  to the (separately pinned) dense oracle to fp64 rounding (the two evaluate
  the same sums in matrix products of different shapes);
* brute force with scalar Python loops on tiny inputs;
* entries that do not count (padding, positions beyond the visible limit,
  including the causal limit of each token) change nothing, bit for bit;
* the order of the list does not matter (to fp64 rounding);
* multiset semantics: one key listed n times gives O = V, LSE = s + ln n;
* no counted entry gives O = 0, LSE = -inf.
"""
import math

import numpy as np
import pytest
import torch

from oracle import counted_entries, decode, decode_sparse, decode_sparse_bruteforce
from workloads import build_inputs, draw_topk_indices


def _all_visible(seqlens, s_q, causal, topk):
    B = len(seqlens)
    ix = torch.full((B, s_q, topk), -1, dtype=torch.int32)
    for b, L in enumerate(seqlens):
        for t in range(s_q):
            vis = max(0, min(L, L - s_q + 1 + t)) if causal else L
            ix[b, t, :vis] = torch.arange(vis, dtype=torch.int32)
    return ix


@pytest.mark.parametrize("seqlens,s_q,causal", [([65, 130, 7], 1, False), ([70, 3, 200], 2, True),
                                                ([129, 64], 4, True)])
def test_all_visible_selection_is_dense(seqlens, s_q, causal):
    inp = build_inputs(seqlens, s_q, 8, seed=61)
    ix = _all_visible(seqlens, s_q, causal, max(seqlens) + 3)
    Os, Ls = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, causal)
    Od, Ld = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, causal)
    assert np.array_equal(np.isinf(Ls), np.isinf(Ld))
    assert np.allclose(Os, Od, rtol=0, atol=1e-12)
    assert np.allclose(Ls, Ld, rtol=0, atol=1e-12)


def test_bruteforce_agrees():
    inp = build_inputs([70, 9, 130], 2, 3, seed=62)
    g = torch.Generator().manual_seed(3)
    ix = draw_topk_indices([70, 9, 130], 2, 24, True, g, pad_frac=0.2)
    ix[0, 0, 0] = ix[0, 0, 1] = 5          # a duplicate
    Os, Ls = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, True)
    Ob, Lb = decode_sparse_bruteforce(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix,
                                      inp.scale, True)
    assert np.allclose(Os, Ob, rtol=1e-12, atol=1e-12)
    assert np.allclose(Ls, Lb, rtol=1e-12, atol=1e-12)


def test_non_counting_entries_change_nothing():
    inp = build_inputs([300, 80], 2, 4, seed=63)
    g = torch.Generator().manual_seed(4)
    ix = draw_topk_indices([300, 80], 2, 32, True, g)
    base = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, True)
    # append padding, positions at/after the limit, and token 0's causal limit
    extra = torch.tensor([-1, -7, 300, 301, 10 ** 6], dtype=torch.int32)
    ix2 = torch.cat([ix, extra.expand(2, 2, 5)], dim=2).contiguous()
    ix2[0, 0, -1] = 299    # token 0 of a 2-token request sees positions < 299
    ix2[1, 0, -1] = 79     # request 1: token 0 sees < 79
    got = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix2, inp.scale, True)
    assert np.array_equal(base[0], got[0]) and np.array_equal(base[1], got[1])
    assert list(counted_entries([3, -1, 9, 2], 9)) == [3, 2]


def test_order_does_not_matter():
    inp = build_inputs([500], 1, 4, seed=64)
    g = torch.Generator().manual_seed(5)
    ix = draw_topk_indices([500], 1, 64, False, g)
    a = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, False)
    ixp = ix[:, :, torch.randperm(64, generator=g)].contiguous()
    b = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ixp, inp.scale, False)
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-12) and np.allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_multiset_closed_form_and_empty():
    inp = build_inputs([100, 50], 1, 2, seed=65)
    ix = torch.full((2, 1, 8), -1, dtype=torch.int32)
    ix[0, 0, :3] = 42                       # one key listed three times
    O, L = decode_sparse(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, False)
    page = int(inp.block_table[0, 0])
    k = inp.kcache[page, 42, 0].double().numpy()
    for h in range(2):
        s = inp.scale * float(inp.q[0, 0, h].double().numpy() @ k)
        assert np.allclose(O[0, 0, h], k[:512], rtol=1e-14, atol=0)
        assert math.isclose(L[0, 0, h], s + math.log(3.0), rel_tol=0, abs_tol=1e-12)
    assert np.all(O[1] == 0.0) and np.all(L[1] == -np.inf)


# ------------------------------------------------ sparse mode over FP8 pages

def _fp8_case(seqlens, s_q, h_q, seed):
    from workloads import build_fp8_inputs
    return build_fp8_inputs(seqlens, s_q, h_q, seed=seed, extra_pool=3)


def test_fp8_all_visible_selection_is_fp8_dense():
    """Selecting every visible position is the (separately pinned) dense FP8
    oracle."""
    from oracle import decode_fp8, decode_sparse_fp8
    seqlens, s_q, causal = [70, 3, 150], 2, True
    inp = _fp8_case(seqlens, s_q, 4, seed=71)
    ix = _all_visible(seqlens, s_q, causal, max(seqlens) + 5)
    Os, Ls = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale,
                               causal)
    Od, Ld = decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, causal)
    assert np.array_equal(np.isinf(Ls), np.isinf(Ld))
    assert np.allclose(Os, Od, rtol=0, atol=1e-12)
    assert np.allclose(Ls, Ld, rtol=0, atol=1e-12)


def test_fp8_equals_bf16_sparse_over_dequantised_pages():
    """Every dequantised FP8 value is a bf16 value (at most 4 significant bits
    times a power of two), so the sparse mode over FP8 pages equals the bf16
    sparse oracle over a bf16 cache holding the dequantised rows, entry for
    entry — which pins the FP8 row addressing (page, row, the three fields)
    to the bf16 gathering."""
    from oracle import decode_sparse_fp8, dequant_page
    seqlens, s_q = [300, 65, 129], 1
    inp = _fp8_case(seqlens, s_q, 3, seed=72)
    pool8 = inp.kcache.view(torch.uint8).reshape(inp.kcache.shape[0], -1).numpy()
    K = np.stack([dequant_page(pool8[p]) for p in range(pool8.shape[0])])   # [pages, 64, 576]
    fin = np.isfinite(K)
    assert np.array_equal(torch.from_numpy(K[fin]).to(torch.bfloat16).double().numpy(), K[fin])
    kc16 = torch.from_numpy(K).to(torch.bfloat16).unsqueeze(2).contiguous()   # [pages, 64, 1, 576]
    g = torch.Generator().manual_seed(8)
    ix = draw_topk_indices(seqlens, s_q, 96, True, g, pad_frac=0.2)
    ix[0, 0, :3] = 17                       # a duplicate
    a = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, True)
    b = decode_sparse(inp.q, kc16, inp.block_table, inp.seqlens, ix, inp.scale, True)
    assert np.array_equal(np.isinf(a[1]), np.isinf(b[1]))
    assert np.allclose(a[0], b[0], rtol=0, atol=1e-13)
    assert np.allclose(a[1], b[1], rtol=0, atol=1e-13)


def test_fp8_non_counting_entries_change_nothing():
    from oracle import decode_sparse_fp8
    inp = _fp8_case([200, 90], 2, 2, seed=73)
    g = torch.Generator().manual_seed(9)
    ix = draw_topk_indices([200, 90], 2, 32, True, g)
    base = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix, inp.scale, True)
    extra = torch.tensor([-1, -3, 200, 10 ** 5], dtype=torch.int32)
    ix2 = torch.cat([ix, extra.expand(2, 2, 4)], dim=2).contiguous()
    ix2[1, 0, -1] = 89      # request 1, token 0 sees positions < 89
    got = decode_sparse_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, ix2, inp.scale, True)
    assert np.array_equal(base[0], got[0]) and np.array_equal(base[1], got[1])


def test_unmapped_pages_are_skipped():
    """Entries whose table slot holds a page id outside the pool count for
    nothing: the result equals the one with those entries removed from the
    list (bf16 and FP8 pages; brute force agrees)."""
    from oracle import decode_sparse_fp8
    from workloads import build_fp8_inputs
    for fp8 in (False, True):
        build = build_fp8_inputs if fp8 else build_inputs
        inp = build([200, 130], 1, 4, seed=74, extra_pool=3)
        n_pool = int(inp.kcache.shape[0])
        bt = inp.block_table.clone()
        bt[0, 1] = n_pool + 5          # positions 64..127 of request 0 unmapped
        bt[1, 0] = -3                  # positions 0..63 of request 1 unmapped
        g = torch.Generator().manual_seed(10)
        ix = draw_topk_indices([200, 130], 1, 64, False, g)
        keep = ix.clone()
        j0, j1 = keep[0, 0], keep[1, 0]
        j0[(j0 >= 64) & (j0 < 128)] = -1
        j1[(j1 >= 0) & (j1 < 64)] = -1
        ref = decode_sparse_fp8 if fp8 else decode_sparse
        a = ref(inp.q, inp.kcache, bt, inp.seqlens, ix, inp.scale, False)
        b = ref(inp.q, inp.kcache, inp.block_table, inp.seqlens, keep, inp.scale, False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
        if not fp8:
            c = decode_sparse_bruteforce(inp.q, inp.kcache, bt, inp.seqlens, ix, inp.scale, False)
            assert np.allclose(a[0], c[0], rtol=1e-12, atol=1e-12)
