"""The decode with its split plan derived inside the decode kernel
(mla_decode_fwd_inline_plan[_fp8]) on MI355X: the plan it writes equals the
scheduler kernel's (mla_decode_metadata) entry for entry, and its outputs
equal the three-launch path's bit for bit (same plan, same pieces, same
arithmetic), for bf16 and FP8 caches over seeded random and edge-case
length sets.  The three-launch path itself is checked against the oracle by
the other parity tests.
"""
import numpy as np
import pytest
import torch

from workloads import build_fp8_inputs, build_inputs, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _cases():
    out = [([65, 130], 1, 16, None), ([0], 1, 16, None), ([0, 0, 0], 2, 32, 7),
           ([1], 4, 64, 3), ([64] * 64, 1, 16, None), ([4096] * 3, 1, 128, None),
           ([5, 0, 1000, 63, 64, 65, 0, 129], 2, 128, 200), ([300] * 1024, 1, 16, None),
           ([1, 2, 3] * 341 + [7], 1, 32, 57), ([20000, 1], 8, 16, None)]
    r = np.random.default_rng(4242)
    for _ in range(14):
        B = int(r.integers(1, 300))
        lens = [int(x) for x in r.integers(0, 3000, size=B)]
        out.append((lens, int(r.choice([1, 2, 4])), int(r.choice([16, 32, 64, 128])),
                    None if r.random() < 0.5 else int(r.integers(1, 300))))
    return out


@pytest.mark.parametrize("idx", range(24))
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_inline_plan_matches_three_launches(mla, idx, kv):
    lens, s_q, h_q, parts = _cases()[idx]
    print(f"case inline plan {kv} idx={idx} B={len(lens)} s_q={s_q} h_q={h_q} parts={parts}",
          flush=True)
    build = build_fp8_inputs if kv == "fp8" else build_inputs
    inp = build(lens, s_q, h_q, seed=500 + idx, extra_pool=2)
    g = inp.to("cuda")
    fp8 = kv == "fp8"
    ref_meta = mla.metadata(g.seqlens, s_q, h_q, parts=parts)
    fwd = mla.fwd_fp8 if fp8 else mla.fwd
    o_ref, l_ref = fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                       meta=ref_meta)
    meta = mla.binding.Metadata(torch.full_like(ref_meta.tile_meta, -7),
                                torch.full_like(ref_meta.split_offsets, -7),
                                ref_meta.num_parts, s_q, h_q)
    o, l = mla.fwd_inline_plan(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                               meta=meta, fp8=fp8)
    torch.cuda.synchronize()
    assert torch.equal(meta.tile_meta.cpu(), ref_meta.tile_meta.cpu())
    assert torch.equal(meta.split_offsets.cpu(), ref_meta.split_offsets.cpu())
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))


@pytest.mark.parametrize("wl", ["membound", "ridge", "ragged", "draft"])
def test_inline_plan_full_workloads(mla, wl):
    """The benchmark workloads: the same plan and the same outputs as the
    three-launch path."""
    print(f"case inline plan full {wl}", flush=True)
    inp = make_inputs(wl)
    g = inp.to("cuda")
    ref_meta = mla.metadata(g.seqlens, inp.s_q, inp.h_q)
    o_ref, l_ref = mla.fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                           meta=ref_meta)
    meta = mla.binding.Metadata(torch.full_like(ref_meta.tile_meta, -7),
                                torch.full_like(ref_meta.split_offsets, -7),
                                ref_meta.num_parts, inp.s_q, inp.h_q)
    o, l = mla.fwd_inline_plan(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                               meta=meta)
    torch.cuda.synchronize()
    assert torch.equal(meta.tile_meta.cpu(), ref_meta.tile_meta.cpu())
    assert torch.equal(meta.split_offsets.cpu(), ref_meta.split_offsets.cpu())
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(l.view(torch.int32), l_ref.view(torch.int32))
