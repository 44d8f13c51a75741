"""The seeded input generator: determinism and the paged-cache layout contract."""
import torch

from workloads import WORKLOADS, algorithmic_counts, blocks_for, build_inputs, make_inputs


def test_same_seed_same_bytes():
    a = make_inputs("tiny")
    b = make_inputs("tiny")
    for x, y in ((a.q, b.q), (a.kcache, b.kcache), (a.block_table, b.block_table),
                 (a.seqlens, b.seqlens)):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y)


def test_layout_contract():
    inp = make_inputs("tiny")
    assert inp.q.shape == (2, 1, 16, 576) and inp.q.dtype == torch.bfloat16
    assert inp.kcache.shape == (9, 64, 1, 576)
    assert inp.seqlens.tolist() == [65, 130]
    pool = 8
    assert torch.isnan(inp.kcache[pool].float()).all()          # sentinel page
    used = []
    for b, L in enumerate(inp.seqlens.tolist()):
        n = blocks_for(L)
        pages = inp.block_table[b, :n].tolist()
        used += pages
        assert all(0 <= p < pool for p in pages)
        assert all(p == pool for p in inp.block_table[b, n:].tolist())
        last = inp.kcache[pages[-1]].float()
        tail = n * 64 - L
        assert torch.isnan(last[64 - tail:]).all()
        assert not torch.isnan(last[:64 - tail]).any()
    assert len(set(used)) == len(used)


def test_lognormal_lengths_in_range():
    w = WORKLOADS["ragged"]
    inp_sl = __import__("workloads").draw_seqlens(w.seqlen_kind, w.batch,
                                                  torch.Generator().manual_seed(w.seed))
    assert inp_sl.min() >= 1 and inp_sl.max() <= 32768 and inp_sl.shape == (132,)


def test_counts_formula():
    c = algorithmic_counts([4096] * 64, 1, 16)
    assert c["kv_bytes"] == 64 * 4096 * 1152
    assert c["flops"] == 2176 * 16 * 4096 * 64
    c2 = algorithmic_counts([10], 2, 1)
    assert c2["flops"] == 2176 * (9 + 10)


def test_build_inputs_q_scale():
    a = build_inputs([70], 1, 16, seed=3, q_scale=8.0)
    b = build_inputs([70], 1, 16, seed=3)
    assert torch.allclose(a.q.float(), (b.q.float() * 8).bfloat16().float(), atol=0.5)


def test_fp8_counts():
    c = algorithmic_counts([4096] * 64, 1, 16, "fp8")
    assert c["kv_bytes"] == 64 * 4096 * (512 + 128 + 4)
    b = algorithmic_counts([4096] * 64, 1, 16)
    assert c["flops"] == b["flops"] and b["kv_bytes"] == 64 * 4096 * 1152
