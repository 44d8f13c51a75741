"""The Python binding rejects tensors whose shapes disagree with each other
before anything is enqueued (the kernels trust these shapes, so a mismatch
that reached them would index outside the caller's buffers).

Each case passes one mismatched tensor and expects ValueError; the output
buffers carry a sentinel that must be untouched afterwards, so nothing ran.
"""
import pytest
import torch

from workloads import build_fp8_inputs, build_inputs, draw_topk_indices

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def case(mla):
    inp = build_inputs([100, 64, 1, 300], 1, 16, seed=61, extra_pool=2)
    g = inp.to("cuda")
    meta = mla.metadata(g.seqlens, 1, 16)
    ws = torch.zeros((mla.workspace_bytes(4, 1, 16, meta.num_parts),), dtype=torch.uint8,
                     device="cuda")
    torch.cuda.synchronize()
    return inp, g, meta, ws


def _sentinel(shape, dtype):
    return torch.full(shape, 3.0, dtype=dtype, device="cuda")


def _untouched(*ts):
    torch.cuda.synchronize()
    for t in ts:
        assert bool((t == 3.0).all().item()), "a kernel ran despite the rejected call"


def test_fwd_rejects_mismatched_batch_tensors(mla, case):
    inp, g, meta, ws = case
    out = _sentinel((4, 1, 16, 512), torch.bfloat16)
    lse = _sentinel((4, 1, 16), torch.float32)
    bad = {
        "seqlens": dict(seqlens=g.seqlens[:3].contiguous()),
        "block_table": dict(block_table=g.block_table[:2].contiguous()),
    }
    for tag, kw in bad.items():
        args = dict(q=g.q, kcache=g.kcache, block_table=g.block_table, seqlens=g.seqlens)
        args.update(kw)
        with pytest.raises(ValueError):
            mla.fwd(args["q"], args["kcache"], args["block_table"], args["seqlens"], inp.scale,
                    False, meta=meta, workspace=ws, out=out, lse=lse)
        _untouched(out, lse)


def test_fwd_rejects_wrong_output_shapes(mla, case):
    inp, g, meta, ws = case
    for oshape, lshape in (((4, 1, 16, 256), (4, 1, 16)), ((3, 1, 16, 512), (4, 1, 16)),
                           ((4, 1, 16, 512), (4, 16)), ((4, 1, 16, 512), (4, 2, 16))):
        out = _sentinel(oshape, torch.bfloat16)
        lse = _sentinel(lshape, torch.float32)
        with pytest.raises(ValueError):
            mla.fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, False, meta=meta,
                    workspace=ws, out=out, lse=lse)
        _untouched(out, lse)


def test_splitkv_rejects_metadata_of_another_shape(mla, case):
    inp, g, meta, ws = case
    out = _sentinel((4, 1, 16, 512), torch.bfloat16)
    lse = _sentinel((4, 1, 16), torch.float32)
    other_heads = mla.metadata(g.seqlens, 1, 32)
    other_batch = mla.metadata(g.seqlens[:3].contiguous(), 1, 16)
    Meta = mla.binding.Metadata
    short_tm = Meta(meta.tile_meta[:-1].contiguous(), meta.split_offsets, meta.num_parts, 1, 16)
    for m in (other_heads, other_batch, short_tm):
        with pytest.raises(ValueError):
            mla.splitkv(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, False, m, ws,
                        out, lse)
        _untouched(out, lse)


def test_combine_rejects_mismatched_shapes(mla, case):
    inp, g, meta, ws = case
    out = _sentinel((4, 1, 16, 512), torch.bfloat16)
    lse = _sentinel((4, 1, 16), torch.float32)
    with pytest.raises(ValueError):
        mla.combine(g.seqlens, 1, 32, meta, ws, out, lse)      # h_q of another shape
    with pytest.raises(ValueError):
        mla.combine(g.seqlens[:3].contiguous(), 1, 16, meta, ws, out, lse)
    _untouched(out, lse)


def test_kv_append_rejects_mismatched_batch(mla, case):
    inp, g, meta, ws = case
    kc = g.kcache.clone()
    new = torch.zeros((3, 1, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        mla.kv_append(new, kc, g.block_table, g.seqlens)
    torch.cuda.synchronize()
    assert torch.equal(kc.view(torch.int16), g.kcache.view(torch.int16))
    inp8 = build_fp8_inputs([100, 64, 1, 300], 1, 16, seed=62, extra_pool=2)
    g8 = inp8.to("cuda")
    kc8 = g8.kcache.clone()
    with pytest.raises(ValueError):
        mla.kv_append_fp8(new, kc8, g8.block_table, g8.seqlens)
    torch.cuda.synchronize()
    assert torch.equal(kc8, g8.kcache)


def test_sparse_rejects_metadata_of_dense_plan(mla):
    lens = [300, 100]
    inp = build_inputs(lens, 2, 16, seed=63, extra_pool=2)
    g = inp.to("cuda")
    ix = draw_topk_indices(lens, 2, 64, True, torch.Generator().manual_seed(3), 0.1).cuda()
    dense_meta = mla.metadata(g.seqlens, 2, 16)     # batch + 1 offsets, not batch*s_q + 1
    out = _sentinel((2, 2, 16, 512), torch.bfloat16)
    lse = _sentinel((2, 2, 16), torch.float32)
    with pytest.raises(ValueError):
        mla.sparse_fwd(g.q, g.kcache, g.block_table, g.seqlens, ix, inp.scale, True,
                       meta=dense_meta, out=out, lse=lse)
    _untouched(out, lse)
