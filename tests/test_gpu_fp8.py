"""GPU parity of the FP8-cache path (mla_decode_*_fp8, mla_kv_append_fp8)
against the fp64 oracle of oracle/mla_fp8_oracle.py (MI355X only).

Decode: the same bar as the bf16 path — max|O_gpu - O_ref| <= 1e-2 *
max|O_ref|, |LSE_gpu - LSE_ref| <= 1e-3 on rows with a visible key, exact
O = 0 / LSE = -inf on rows without one.  The reference attends over the
exactly dequantized keys, so the bar measures only the kernel's own rounding
(bf16 products, fp32 sums, bf16 probabilities).  Append: the quantised cache
is compared bit for bit (codes, rope, scales), since both sides take every
rounding decision on exact values.
"""
import math

import numpy as np
import pytest
import torch

from oracle import decode_fp8, kv_append_fp8
from workloads import WORKLOADS, build_fp8_inputs, make_inputs

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


def _run(mla, inp, parts=None, dev="cuda"):
    assert inp.kv_format == "fp8"
    g = inp.to(dev)
    meta = mla.metadata(g.seqlens, inp.s_q, inp.h_q, parts=parts)
    out, lse = mla.fwd_fp8(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                           meta=meta)
    torch.cuda.synchronize()
    return out, lse, meta


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


def _ref(inp, requests=None, scale=None, causal=None):
    return decode_fp8(inp.q, inp.kcache, inp.block_table, inp.seqlens,
                      inp.scale if scale is None else scale,
                      inp.causal if causal is None else causal, requests=requests)


@pytest.mark.parametrize("parts", [None, 1, 2, 3])
def test_fp8_tiny_workload(mla, parts):
    _say(f"case fp8 tiny parts={parts}")
    inp = make_inputs("tiny", kv_format="fp8")
    out, lse, _ = _run(mla, inp, parts)
    O_ref, L_ref = _ref(inp)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"fp8 tiny P={parts}")


SMALL_LENS = [1, 63, 64, 65, 127, 128, 129, 300, 1000, 2, 0, 191]


@pytest.mark.parametrize("h_q", [16, 32, 64, 128])
@pytest.mark.parametrize("s_q", [1, 2])
@pytest.mark.parametrize("parts", [None, 5])
def test_fp8_small_shapes(mla, h_q, s_q, parts):
    _say(f"case fp8 small h_q={h_q} s_q={s_q} parts={parts}")
    inp = build_fp8_inputs(SMALL_LENS, s_q, h_q, seed=700 + h_q + s_q, extra_pool=7)
    out, lse, _ = _run(mla, inp, parts)
    O_ref, L_ref = _ref(inp)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"fp8 small h{h_q} s{s_q} P={parts}")


@pytest.mark.parametrize("h_q", [16, 128])
@pytest.mark.parametrize("s_q", [4, 8])
def test_fp8_draft_tokens(mla, h_q, s_q):
    _say(f"case fp8 draft h_q={h_q} s_q={s_q}")
    lens = [1, 3, 4, 63, 64, 65, 129, 300, 0, 7]
    inp = build_fp8_inputs(lens, s_q, h_q, seed=800 + h_q + s_q, extra_pool=5)
    out, lse, _ = _run(mla, inp, 5)
    O_ref, L_ref = _ref(inp)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"fp8 draft h{h_q} s{s_q}")


def test_fp8_prefill_chunk(mla):
    _say("case fp8 prefill chunk s_q=64 h_q=64")
    lens = [64, 65, 300, 3, 0]
    inp = build_fp8_inputs(lens, 64, 64, seed=871, extra_pool=3)
    out, lse, _ = _run(mla, inp, 3)
    O_ref, L_ref = _ref(inp)
    _assert_parity(out, lse, O_ref, L_ref, tag="fp8 prefill s64 h64")


@pytest.mark.parametrize("key", ["tiny", "membound", "ridge", "ragged", "long", "draft",
                                 "prefill"])
def test_fp8_full_workload(mla, key):
    """Full-size workload with an FP8 cache, in the benchmark's launch
    configuration; the oracle recomputes every request of the batch."""
    _say(f"case fp8 full {key}: generating inputs")
    inp = make_inputs(key, kv_format="fp8")
    _say(f"case fp8 full {key}: decode on GPU")
    out, lse, _ = _run(mla, inp)
    _say(f"case fp8 full {key}: oracle on all {inp.batch} requests")
    O_ref, L_ref = _ref(inp)
    _assert_parity(out, lse, O_ref, L_ref, tag=f"fp8 full {key}")
    assert not torch.isnan(out.float()).any().item()
    L = lse.cpu()
    for b, Lb in enumerate(inp.seqlens.tolist()):
        for t in range(inp.s_q):
            vis = Lb - inp.s_q + 1 + t if inp.causal else Lb
            if vis > 0:
                assert torch.isfinite(L[b, t]).all(), (key, b, t)
            else:
                assert (L[b, t] == -math.inf).all(), (key, b, t)


def test_fp8_run_to_run_and_page_permutation_bitwise(mla):
    _say("case fp8 determinism + page permutation")
    inp = build_fp8_inputs([1000, 129, 64, 4000], 2, 64, seed=9, extra_pool=11)
    a = _run(mla, inp)
    b = _run(mla, inp)
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1], b[1])
    npg = inp.kcache.shape[0]
    perm = torch.randperm(npg, generator=torch.Generator().manual_seed(1))
    newk = torch.empty_like(inp.kcache)
    newk[perm] = inp.kcache
    inp2 = type(inp)(inp.q, newk, perm[inp.block_table.long()].to(torch.int32), inp.seqlens,
                     inp.scale, inp.causal, inp.s_q, inp.h_q, "fp8")
    c = _run(mla, inp2)
    assert torch.equal(a[0].view(torch.int16), c[0].view(torch.int16))
    assert torch.equal(a[1], c[1])


def test_fp8_single_token_exact(mla):
    """L = 1: O equals the dequantized value row exactly (a code times a power
    of two is a bf16 value)."""
    _say("case fp8 single token")
    inp = build_fp8_inputs([1, 1, 1], 1, 128, seed=41, extra_pool=2)
    out, lse, _ = _run(mla, inp)
    for b in range(3):
        pg = inp.kcache[int(inp.block_table[b, 0])]
        codes = pg[:512].view(torch.float8_e4m3fn).to(torch.float32)
        s = pg[40960:40964].view(torch.float32)
        v = (codes * s).to(torch.bfloat16)
        assert torch.equal(out[b, 0].cpu().view(torch.int16),
                           v.expand(128, 512).contiguous().view(torch.int16))


def test_fp8_zero_scale_mean(mla):
    _say("case fp8 zero scale")
    inp = build_fp8_inputs([700, 64, 1], 1, 16, seed=31, extra_pool=2)
    g = inp.to("cuda")
    out, lse = mla.fwd_fp8(g.q, g.kcache, g.block_table, g.seqlens, 0.0, False)
    torch.cuda.synchronize()
    O_ref, L_ref = _ref(inp, scale=0.0, causal=False)
    _assert_parity(out, lse, O_ref, L_ref, tag="fp8 zero scale")


def test_fp8_nonpow2_scales(mla):
    """The decoder takes any finite scale: scales times 1.3 (not powers of
    two) and a spread of magnitudes."""
    _say("case fp8 non-power-of-two scales")
    inp = build_fp8_inputs([500, 77, 3000], 2, 32, seed=33, extra_pool=3)
    sc = inp.kcache[:-1, 40960:].contiguous().view(torch.float32)
    mult = torch.tensor([1.3, 0.77, 3.1, 0.011], dtype=torch.float32).repeat(16)
    sc = sc * mult[None, :]
    inp.kcache[:-1, 40960:] = sc.contiguous().view(torch.uint8)
    out, lse, _ = _run(mla, inp, 4)
    O_ref, L_ref = _ref(inp)
    _assert_parity(out, lse, O_ref, L_ref, tag="fp8 non-pow2 scales")


# ---- FP8 append -------------------------------------------------------------

def _new_rows(batch, s_q, seed):
    g = torch.Generator().manual_seed(seed)
    new = torch.randn((batch, s_q, 576), generator=g)
    mag = torch.pow(10.0, torch.randint(-30, 31, (batch, s_q, 1), generator=g).float())
    new = new * mag
    new[0, 0, :512] = 0.0                          # all-zero latent
    if batch > 1:
        new[1, 0, :512] = -0.0
        new[1, 0, 7] = 3.0e-39                     # bf16 subnormal, amax of its row
    if batch > 2:
        new[2, 0, :512] = torch.linspace(-448, 448, 512)   # ties in the E4M3 grid
    return new.to(torch.bfloat16)


@pytest.mark.parametrize("s_q", [1, 2, 5])
def test_fp8_kv_append_matches_oracle(mla, s_q):
    """The FP8 cache after the append equals the oracle's bit for bit, and
    decode over it matches the oracle's decode over the oracle's cache."""
    _say(f"case fp8 append s_q={s_q}")
    lens = [70, 63, 64, 65, 130, 0, 2, 1000, 1]
    inp = build_fp8_inputs(lens, s_q, 64, seed=900 + s_q, extra_pool=4)
    g = inp.to("cuda")
    new = _new_rows(inp.batch, s_q, 10 + s_q)
    mla.kv_append_fp8(new.cuda(), g.kcache, g.block_table, g.seqlens)
    torch.cuda.synchronize()
    ref = torch.from_numpy(kv_append_fp8(inp.kcache, inp.block_table, inp.seqlens, new))
    got = g.kcache.cpu()
    if not torch.equal(got, ref):
        bad = torch.nonzero(got != ref)
        raise AssertionError(f"append differs at {bad[:8].tolist()} "
                             f"got {got[tuple(bad[0])]} want {ref[tuple(bad[0])]}")
    # decode over the appended cache (scores of 1e30-scaled rows are huge;
    # decode with a unit-range copy of Q only where the rows are moderate)
    inp2 = type(inp)(inp.q, ref, inp.block_table, inp.seqlens, inp.scale, inp.causal,
                     inp.s_q, inp.h_q, "fp8")
    mags = new[:, :, :512].float().abs().amax(dim=-1)
    keep = [b for b in range(inp.batch) if bool((mags[b] < 1e3).all())]
    out, lse = mla.fwd_fp8(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal)
    torch.cuda.synchronize()
    O_ref, L_ref = decode_fp8(inp2.q, inp2.kcache, inp2.block_table, inp2.seqlens, inp.scale,
                              inp.causal, requests=keep)
    _assert_parity(out, lse, O_ref, L_ref, reqs=keep, tag=f"fp8 append s{s_q}")


def test_fp8_spiky_after_append(mla):
    """A planted key along q appended mid-sequence through the FP8 append:
    its score (~60) dominates and the running max jumps on a late page."""
    _say("case fp8 spiky via append")
    lens = [3000, 5000]
    inp = build_fp8_inputs(lens, 1, 16, seed=21, extra_pool=3, q_scale=8.0)
    planted = torch.zeros((2, 1, 576), dtype=torch.bfloat16)
    for b in range(2):
        qv = inp.q[b, 0, 0].double()
        c = 60.0 / (inp.scale * float(qv @ qv))
        planted[b, 0] = (c * qv).to(torch.bfloat16)
    # write the planted rows at positions 1500 / 4100: seqlens as seen by the
    # append are the positions + 1
    pos_lens = torch.tensor([1501, 4101], dtype=torch.int32)
    g = inp.to("cuda")
    mla.kv_append_fp8(planted.cuda(), g.kcache, g.block_table, pos_lens.cuda())
    torch.cuda.synchronize()
    ref = torch.from_numpy(kv_append_fp8(inp.kcache, inp.block_table, pos_lens, planted))
    assert torch.equal(g.kcache.cpu(), ref)
    inp2 = type(inp)(inp.q, ref, inp.block_table, inp.seqlens, inp.scale, False, 1, 16, "fp8")
    out, lse, _ = _run(mla, inp2)
    O_ref, L_ref = _ref(inp2)
    assert L_ref[0, 0, 0] > 50 and L_ref[1, 0, 0] > 50
    _assert_parity(out, lse, O_ref, L_ref, tag="fp8 spiky")
