"""Pins of the oracle's reading of table entries that hold no page.

A position whose table slot lies past the end of the request's row, or whose
slot names no page of the pool (negative, or at or beyond the pool size),
holds no key and is left out of the attention, as the sparse mode skips the
same entries.  The pages leave this caller error open; the pins tie the
reading to the plain dense definition on a request without the missing keys
(attention over a set of keys does not depend on where they sit), to the
scalar brute force, and to the empty-set closed form.
"""
import numpy as np
import pytest
import torch

from oracle import (decode, decode_bruteforce, decode_fp8, decode_sparse, gather_request_kv,
                    mapped_keys)
from workloads import build_fp8_inputs, build_inputs


def _req(O, L, b):
    return O[b], L[b]


@pytest.mark.parametrize("s_q,causal", [(1, False), (2, True), (3, False)])
def test_unmapped_page_equals_request_without_it(s_q, causal):
    """Request 0 (150 keys over pages p0, p1, p2) with p1 unmapped equals a
    request of 86 keys over pages (p0, p2): keys 0..63 of p0, then rows 0..21
    of p2.  The unmapped block lies before the causal boundary, so the
    visible counts line up token by token (149 - 64 = 85, 150 - 64 = 86)."""
    inp = build_inputs([150, 90], s_q, 16, seed=301, extra_pool=4, nan_tails=False)
    n_pool = int(inp.kcache.shape[0])
    bt = inp.block_table.clone()
    p0, p2 = int(bt[0, 0]), int(bt[0, 2])
    for bad in (-1, n_pool, n_pool + 7, 1 << 30):
        bt[0, 1] = bad
        O, L = decode(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, causal)
        bt2 = torch.tensor([[p0, p2, p2]], dtype=torch.int32)
        O2, L2 = decode(inp.q[:1], inp.kcache, bt2, torch.tensor([86], dtype=torch.int32),
                        inp.scale, causal)
        np.testing.assert_allclose(O[0], O2[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L[0], L2[0], rtol=0, atol=1e-12)
        # request 1 keeps all of its keys
        O3, L3 = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, causal)
        np.testing.assert_array_equal(O[1], O3[1])


def test_slots_past_the_row_are_dropped():
    """A 150-key request whose table row has 2 columns sees keys 0..127 only:
    the same as the request cut to 128 keys."""
    inp = build_inputs([150], 1, 16, seed=302, extra_pool=2, nan_tails=False)
    bt = inp.block_table[:, :2].contiguous()
    O, L = decode(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, False)
    O2, L2 = decode(inp.q, inp.kcache, bt, torch.tensor([128], dtype=torch.int32), inp.scale, False)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, L2, rtol=0, atol=1e-12)


def test_every_page_unmapped_is_empty():
    """No counted key: O = 0 and LSE = -inf (the empty-set closed form)."""
    inp = build_inputs([100, 64], 2, 16, seed=303, extra_pool=1, nan_tails=False)
    bt = torch.full_like(inp.block_table, -5)
    O, L = decode(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, True)
    assert np.all(O == 0.0)
    assert np.all(np.isneginf(L))


def test_zero_row_reading_would_differ():
    """Reading the unmapped page as 64 zero keys (score 0 each) moves the
    result: the pins above would catch that reading."""
    inp = build_inputs([150], 1, 16, seed=304, extra_pool=2, nan_tails=False)
    n_pool = int(inp.kcache.shape[0])
    bt = inp.block_table.clone()
    bt[0, 1] = -1
    O, L = decode(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, False)
    kc2 = torch.cat([inp.kcache, torch.zeros_like(inp.kcache[:1])]).contiguous()
    bt2 = bt.clone()
    bt2[0, 1] = n_pool
    Oz, Lz = decode(inp.q, kc2, bt2, inp.seqlens, inp.scale, False)
    assert float(np.max(np.abs(L - Lz))) > 1e-3


def test_bruteforce_agrees_with_unmapped_entries():
    """The vectorised oracle and the scalar brute force agree on a table with
    negative, out-of-pool and missing slots (causal, 2 tokens)."""
    inp = build_inputs([70, 130, 20], 2, 16, seed=305, extra_pool=2, nan_tails=False)
    n_pool = int(inp.kcache.shape[0])
    bt = inp.block_table.clone()
    bt[0, 0] = -2
    bt[1, 1] = n_pool + 3
    O, L = decode(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, True)
    Ob, Lb = decode_bruteforce(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, True)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-10)
    fin = np.isfinite(Lb)
    assert np.array_equal(np.isfinite(L), fin)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-10)


def test_dense_agrees_with_sparse_listing_every_position():
    """The sparse mode listing every position 0..L-1 counts exactly the keys
    that the dense mode counts, unmapped entries included."""
    inp = build_inputs([150, 90], 1, 16, seed=306, extra_pool=3, nan_tails=False)
    n_pool = int(inp.kcache.shape[0])
    bt = inp.block_table.clone()
    bt[0, 1] = n_pool + 1
    bt[1, 0] = -1
    ix = torch.full((2, 1, 160), -1, dtype=torch.int32)
    ix[0, 0, :150] = torch.arange(150)
    ix[1, 0, :90] = torch.arange(90)
    O, L = decode(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, False)
    Os, Ls = decode_sparse(inp.q, inp.kcache, bt, inp.seqlens, ix, inp.scale, False)
    np.testing.assert_allclose(O, Os, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Ls, rtol=0, atol=1e-12)


def test_mapped_keys_and_gather():
    bt = torch.tensor([[3, -1, 9], [0, 1, 2]], dtype=torch.int32)
    sl = torch.tensor([200, 100], dtype=torch.int32)
    m = mapped_keys(bt, sl, 0, 9)
    assert m.shape == (200,)
    assert m[:64].all() and not m[64:].any()        # slot 1 negative, slot 2 id 9 == pool size
    assert mapped_keys(bt, sl, 1, 9).all()
    kc = torch.ones((9, 64, 1, 576), dtype=torch.bfloat16)
    K = gather_request_kv(kc, bt, sl, 0)
    assert K.shape == (200, 576)
    assert np.all(K[:64] == 1.0) and np.all(K[64:] == 0.0)


def test_fp8_unmapped_page_equals_request_without_it():
    inp = build_fp8_inputs([150, 90], 1, 16, seed=307, extra_pool=3, nan_tails=False)
    n_pool = int(inp.kcache.shape[0])
    bt = inp.block_table.clone()
    p0, p2 = int(bt[0, 0]), int(bt[0, 2])
    bt[0, 1] = n_pool + 2
    O, L = decode_fp8(inp.q, inp.kcache, bt, inp.seqlens, inp.scale, False)
    bt2 = torch.tensor([[p0, p2]], dtype=torch.int32)
    O2, L2 = decode_fp8(inp.q[:1], inp.kcache, bt2, torch.tensor([86], dtype=torch.int32),
                        inp.scale, False)
    np.testing.assert_allclose(O[0], O2[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[0], L2[0], rtol=0, atol=1e-12)
