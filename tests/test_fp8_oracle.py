"""Pins of the FP8-cache oracle (oracle/mla_fp8_oracle.py) against facts fixed
outside it:

* the E4M3 code table against torch's float8_e4m3fn conversion (a library
  routine implementing the same OCP format), all 256 codes;
* the E4M3 round-to-nearest-even encoder against torch's cast, for every
  finite bf16 value in [-448, 448] and for random fp32 values;
* the quantiser's scale rule (a power of two, minimal) and its error bound
  (half a unit in the last place of E4M3);
* decode over an FP8 cache equal, bit for bit, to the bf16 oracle over a bf16
  cache built from the same bytes by torch alone (pins the page layout:
  offsets of codes, rope and scales, and the per-token scale);
* the FP8 append writing exactly the rows the bf16 append writes, with codes
  equal to torch's cast of x / scale.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import (E4M3_TABLE, FP8_PAGE_BYTES, FP8_ROPE_OFF, FP8_SCALE_OFF, decode,
                    decode_fp8, dequant_page, e4m3_encode, kv_append, kv_append_fp8,
                    quantize_row, quantize_scale)
from workloads import build_fp8_inputs, build_inputs


def test_e4m3_table_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(E4M3_TABLE))
    assert np.isnan(E4M3_TABLE[0x7F]) and np.isnan(E4M3_TABLE[0xFF])
    fin = ~np.isnan(ref)
    assert np.array_equal(ref[fin], E4M3_TABLE[fin])
    assert E4M3_TABLE[0x7E] == 448.0 and E4M3_TABLE[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_on_all_bf16():
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    v = bits.to(torch.float64)
    sel = torch.isfinite(v) & (v.abs() <= 448)
    vals = bits[sel]
    ref = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([e4m3_encode(x) for x in vals.to(torch.float64).numpy()], dtype=np.uint8)
    assert np.array_equal(ref, mine)


def test_e4m3_encode_matches_torch_on_random_fp32():
    g = torch.Generator().manual_seed(7)
    x = torch.randn(20000, generator=g) * torch.pow(2.0, torch.randint(-12, 8, (20000,), generator=g))
    x = x.clamp(-448, 448)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    mine = np.array([e4m3_encode(float(t)) for t in x.to(torch.float64)], dtype=np.uint8)
    assert np.array_equal(ref, mine)
    with pytest.raises(ValueError):
        e4m3_encode(449.0)


@pytest.mark.parametrize("amax", [1e-30, 2.0 ** -20, 0.3, 1.0, 3.2, 448.0, 449.0, 1e6, 7.5e30])
def test_quantize_scale_is_minimal_power_of_two(amax):
    s = quantize_scale(amax)
    m, e = math.frexp(s)
    assert m == 0.5                      # a power of two
    assert amax <= 448 * s
    assert amax > 448 * s / 2            # the next smaller power fails
    assert quantize_scale(0.0) == 1.0


def test_quantize_row_error_bound_and_range():
    g = torch.Generator().manual_seed(11)
    for trial in range(20):
        x = (torch.randn(576, generator=g) * 10.0 ** float(trial % 7 - 3)).to(torch.bfloat16)
        xf = x.to(torch.float64).numpy()
        codes, s, rope = quantize_row(xf)
        deq = E4M3_TABLE[codes] * s
        y = np.abs(xf[:512]) / s
        # half a unit in the last place: 2^-4 relative for normals, 2^-10 absolute below 2^-6
        bound = np.where(y >= 2.0 ** -6, y * 2.0 ** -4, 2.0 ** -10) * s
        assert np.all(np.abs(deq - xf[:512]) <= bound)
        vmax = np.max(np.abs(E4M3_TABLE[codes]))
        assert 224 <= vmax <= 448
        assert np.array_equal(rope, xf[512:])


def test_quantize_row_exact_for_representable_rows():
    g = torch.Generator().manual_seed(12)
    codes = torch.randint(0, 256, (512,), generator=g, dtype=torch.int64).to(torch.uint8)
    codes[codes == 0x7F] = 0x7E
    codes[codes == 0xFF] = 0xFE
    codes[0] = 0x7E                       # amax code 448 -> the scale is exactly 2^-3
    vals = E4M3_TABLE[codes.numpy()] * 2.0 ** -3
    row = np.concatenate([vals, np.zeros(64)])
    c2, s, _ = quantize_row(row)
    assert s == 2.0 ** -3
    assert np.array_equal(E4M3_TABLE[c2] * s, vals)


def _bf16_cache_from_fp8(pool: torch.Tensor) -> torch.Tensor:
    """The dequantized cache built with torch only (no oracle code)."""
    n = pool.shape[0]
    codes = pool[:, :FP8_ROPE_OFF].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
    scale = pool[:, FP8_SCALE_OFF:].contiguous().view(torch.float32)      # [n, 64]
    lat = codes.reshape(n, 64, 512) * scale[:, :, None]
    rope = pool[:, FP8_ROPE_OFF:FP8_SCALE_OFF].contiguous().view(torch.bfloat16).reshape(n, 64, 64)
    kc = torch.cat([lat.to(torch.bfloat16), rope], dim=2)
    return kc.reshape(n, 64, 1, 576)


@pytest.mark.parametrize("seqlens,s_q,h_q", [([65, 130], 1, 16), ([1, 64, 200], 2, 16),
                                               ([0, 97], 3, 4)])
def test_fp8_decode_equals_bf16_decode_of_dequantized_cache(seqlens, s_q, h_q):
    inp = build_fp8_inputs(seqlens, s_q, h_q, seed=21)
    kc16 = _bf16_cache_from_fp8(inp.kcache)
    # the pow2 scales make the dequantized values exact in bf16
    n = inp.kcache.shape[0]
    lat32 = inp.kcache[:, :FP8_ROPE_OFF].contiguous().view(torch.float8_e4m3fn).to(torch.float32)
    sc = inp.kcache[:, FP8_SCALE_OFF:].contiguous().view(torch.float32)
    exact = (lat32.reshape(n, 64, 512) * sc[:, :, None]).nan_to_num(0.0)
    assert torch.equal(kc16[:, :, 0, :512].to(torch.float32).nan_to_num(0.0), exact)
    O8, L8 = decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    O16, L16 = decode(inp.q, kc16, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    assert np.array_equal(O8, O16)
    assert np.array_equal(L8, L16)
    assert not np.any(np.isnan(O8))


def test_fp8_decode_sees_scale_and_rope():
    """A planted change in one visible row's scale or rope moves the result."""
    inp = build_fp8_inputs([40], 1, 4, seed=22)
    base = decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, False)
    page = int(inp.block_table[0, 0])
    for off in (FP8_SCALE_OFF + 4 * 5, FP8_ROPE_OFF + 2 * 64 * 5 + 1, 5 * 512 + 3):
        pool = inp.kcache.clone()
        pool[page, off] ^= 0x08
        O, L = decode_fp8(inp.q, pool, inp.block_table, inp.seqlens, inp.scale, False)
        assert not np.array_equal(L, base[1])
    # a row beyond the length is never read
    pool = inp.kcache.clone()
    pool[page, FP8_SCALE_OFF + 4 * 50] ^= 0x08
    O, L = decode_fp8(inp.q, pool, inp.block_table, inp.seqlens, inp.scale, False)
    assert np.array_equal(L, base[1]) and np.array_equal(O, base[0])


def test_fp8_append_matches_bf16_append_and_torch_cast():
    seqlens = [1, 63, 64, 65, 130, 2]
    s_q = 2
    inp8 = build_fp8_inputs(seqlens, s_q, 4, seed=23)
    inp16 = build_inputs(seqlens, s_q, 4, seed=23)
    g = torch.Generator().manual_seed(24)
    new = (torch.randn((len(seqlens), s_q, 576), generator=g) * 3).to(torch.bfloat16)
    new[1, 0, :512] = 0                      # all-zero latent: scale 1, codes 0
    out = torch.from_numpy(kv_append_fp8(inp8.kcache, inp8.block_table, inp8.seqlens, new))
    # rows written by the bf16 append (positions) = rows changed here
    kc16 = kv_append(inp16.kcache, inp16.block_table, inp16.seqlens, new)
    changed16 = (kc16.view(torch.int16) != inp16.kcache.view(torch.int16)).any(dim=-1)[:, :, 0]
    for b in range(len(seqlens)):
        for t in range(s_q):
            pos = seqlens[b] - s_q + t
            if pos < 0:
                continue
            page = int(inp8.block_table[b, pos // 64])
            r = pos % 64
            x = new[b, t].to(torch.float64)
            s = quantize_scale(float(x[:512].abs().max()))
            ref_codes = (x[:512] / s).to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
            assert torch.equal(out[page, r * 512:(r + 1) * 512], ref_codes)
            assert torch.equal(out[page, FP8_ROPE_OFF + 128 * r:FP8_ROPE_OFF + 128 * (r + 1)],
                               new[b, t, 512:].contiguous().view(torch.uint8))
            assert out[page, FP8_SCALE_OFF + 4 * r:FP8_SCALE_OFF + 4 * r + 4].view(
                torch.float32).item() == s
            assert bool(changed16[page, r])
    # nothing else changed
    diff = out != inp8.kcache
    pages, rows = [], []
    for p in range(out.shape[0]):
        d = diff[p]
        for r in range(64):
            if d[r * 512:(r + 1) * 512].any() or d[FP8_ROPE_OFF + 128 * r:FP8_ROPE_OFF + 128 * (r + 1)].any() \
                    or d[FP8_SCALE_OFF + 4 * r:FP8_SCALE_OFF + 4 * r + 4].any():
                pages.append(p)
                rows.append(r)
    got = set(zip(pages, rows))
    want = set((int(p), int(r)) for p, r in zip(*torch.nonzero(changed16, as_tuple=True)))
    assert got == want


def test_fp8_generator_layout():
    inp = build_fp8_inputs([65, 130], 1, 16, seed=25, pool=8)
    pool = inp.kcache
    assert pool.shape == (9, FP8_PAGE_BYTES) and pool.dtype == torch.uint8
    sent = pool[-1]
    assert bool((sent[:FP8_ROPE_OFF] == 0x7F).all())
    assert bool(sent[FP8_SCALE_OFF:].view(torch.float32).isnan().all())
    # valid rows: no NaN code, power-of-two scales in [2^-7, 2^-5]
    for b, L in enumerate([65, 130]):
        for j in range(L):
            pg = int(inp.block_table[b, j // 64])
            r = j % 64
            c = pool[pg, r * 512:(r + 1) * 512]
            assert not bool(((c & 0x7F) == 0x7F).any())
            s = pool[pg, FP8_SCALE_OFF + 4 * r:FP8_SCALE_OFF + 4 * r + 4].view(torch.float32).item()
            assert s in (2.0 ** -7, 2.0 ** -6, 2.0 ** -5)
    # tail rows of the last page are NaN
    pg = int(inp.block_table[0, 1])
    assert bool((pool[pg, 1 * 512:2 * 512] == 0x7F).all())
    K = dequant_page(pool[int(inp.block_table[0, 0])])
    assert K.shape == (64, 576) and not np.any(np.isnan(K))
