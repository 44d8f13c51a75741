"""mla_decode_fwd_noalloc (the decode that allocates nothing: its plan and
partials live in the library's own device array) against mla_decode_fwd.

Two calls in a row through the raw C ABI, the second with a smaller input,
so that a plan or partial left in the shared array by the first call would
show up in the second.  Each output is checked against mla_decode_fwd's on
the same inputs with the same part count, to the parity bar (max|dO| <=
1e-2 * max|O_fwd|, |dLSE| <= 1e-3, empty rows exactly O = 0 / LSE = -inf) and
bit for bit (same kernels, same plan), and against the fp64 oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

from oracle import decode
from workloads import build_inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 72 << 20
PLAN_BYTES = 1024 * 8 * 4 + ((16384 + 1) * 4 + 255) // 256 * 256


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _noalloc_raw(mla, g, inp):
    out = torch.full((inp.batch, inp.s_q, inp.h_q, 512), 5.0, dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.full((inp.batch, inp.s_q, inp.h_q), 5.0, dtype=torch.float32, device="cuda")
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    st = mla.lib().mla_decode_fwd_noalloc(
        vp(g.q), vp(g.kcache), g.kcache.shape[0], vp(g.block_table), g.block_table.shape[1],
        vp(g.seqlens), inp.batch, inp.s_q, inp.h_q, 1, ctypes.c_float(inp.scale),
        int(inp.causal), vp(out), vp(lse),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, mla.status_string(st)
    return out, lse


def _parts_used(mla, inp):
    p = mla.num_parts(inp.batch, inp.s_q, inp.h_q, 1, mla.device_num_cus(torch.device("cuda")))
    p = min(p, 1024)
    while p > 1 and mla.workspace_bytes(inp.batch, inp.s_q, inp.h_q, p) > SCRATCH_BYTES - PLAN_BYTES:
        p //= 2
    return p


def _check(a_out, a_lse, b_out, b_lse, tag):
    A = a_out.float().cpu().numpy().astype(np.float64)
    B = b_out.float().cpu().numpy().astype(np.float64)
    la = a_lse.cpu().numpy().astype(np.float64)
    lb = b_lse.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lb)
    assert np.array_equal(np.isfinite(la), fin), tag
    assert np.all(la[~fin] == -np.inf) and np.all(A[~fin] == 0.0), tag
    err_o = float(np.max(np.abs(A - B)))
    tol_o = 1e-2 * float(np.max(np.abs(B[fin])))
    err_l = float(np.max(np.abs(la[fin] - lb[fin])))
    print(f"  {tag}: max|dO|={err_o:.3e} (tol {tol_o:.3e}) max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= tol_o and err_l <= 1e-3, tag


def test_noalloc_matches_fwd_on_two_calls(mla):
    cases = [
        # a 128-head batch whose requests split over several parts
        (build_inputs(np.random.default_rng(5).integers(1000, 6000, size=48).tolist(), 1, 128,
                      seed=1701, extra_pool=4), "large"),
        # then a smaller one: fewer requests, fewer rows, two causal tokens,
        # an empty request
        (build_inputs([300, 0, 65, 2049, 7], 2, 16, seed=1702, extra_pool=2), "small"),
    ]
    for inp, tag in cases:
        print(f"case noalloc {tag}: B={inp.batch} s_q={inp.s_q} h_q={inp.h_q}", flush=True)
        g = inp.to("cuda")
        out_n, lse_n = _noalloc_raw(mla, g, inp)
        meta = mla.metadata(g.seqlens, inp.s_q, inp.h_q, parts=_parts_used(mla, inp))
        out_f, lse_f = mla.fwd(g.q, g.kcache, g.block_table, g.seqlens, inp.scale, inp.causal,
                               meta=meta)
        torch.cuda.synchronize()
        _check(out_n, lse_n, out_f, lse_f, f"noalloc {tag} vs mla_decode_fwd")
        assert torch.equal(out_n.view(torch.int16), out_f.view(torch.int16)), tag
        assert torch.equal(lse_n, lse_f), tag
        O_ref, L_ref = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale,
                              inp.causal)
        _check(out_n, lse_n, torch.from_numpy(O_ref), torch.from_numpy(L_ref),
               f"noalloc {tag} vs oracle")


def test_noalloc_rejects_before_launch(mla):
    inp = build_inputs([100, 64], 1, 16, seed=1703, extra_pool=1)
    g = inp.to("cuda")
    out = torch.full((2, 1, 16, 512), 5.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((2, 1, 16), 5.0, dtype=torch.float32, device="cuda")
    vp = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    call = mla.lib().mla_decode_fwd_noalloc
    args = [vp(g.q), vp(g.kcache), g.kcache.shape[0], vp(g.block_table),
            g.block_table.shape[1], vp(g.seqlens), 2, 1, 16, 1, ctypes.c_float(inp.scale), 0,
            vp(out), vp(lse), stream]
    bad_batch = list(args)
    bad_batch[6] = 16385                 # above MLA_NOALLOC_MAX_BATCH
    assert call(*bad_batch) == -1
    bad_heads = list(args)
    bad_heads[8] = 48                    # unsupported h_q
    assert call(*bad_heads) == -2
    null_out = list(args)
    null_out[12] = None
    assert call(*null_out) == -1
    torch.cuda.synchronize()
    assert bool((out == 5.0).all().item()) and bool((lse == 5.0).all().item())
