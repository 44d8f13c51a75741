"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each check is chosen so that a plausible slip in the oracle (dropped scale,
wrong sign, wrong page/row index, rope dims leaking into V, an off-by-one in
the causal rule, a transposed operand) fails at least one of them:

* hand-derived closed forms (tests/golden/closed_form_cases.json),
* brute force with scalar Python loops on tiny inputs,
* block-table permutation invariance (bitwise),
* one-token sequences (O = V_0 exactly), equal scores (O = mean V, LSE = ln L),
* the absorbed-MQA form equal to per-head single-row attention,
* causal s_q=2 reducing to two s_q=1 problems,
* rope-dim shift (O unchanged, LSE shifted by scale*q_rope.r),
* convex hull of O and the LSE bounds,
* the split/merge identity of the log-sum-exp merge.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attend_rows, decode, decode_bruteforce, gather_request_kv,
                    lse_merge, visible_count)
import oracle.mla_decode_oracle as omod
from workloads import build_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_form_cases.json")


def _ev(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "inf": math.inf}))


def _golden_cases():
    with open(GOLDEN) as f:
        spec = json.load(f)
    return spec


def _build_case(case, d_k, bs):
    B, s_q, h_q = case["batch"], case["s_q"], case["h_q"]
    q = np.zeros((B, s_q, h_q, d_k))
    for b, t, h, d, v in case["q"]:
        q[b, t, h, d] = _ev(v)
    kc = np.zeros((case["num_pages"], bs, 1, d_k))
    for pg in case.get("nan_pages", []):
        kc[pg] = np.nan
    for pg, r0, r1, d, v in case.get("k_fill", []):
        kc[pg, r0:r1, 0, d] = _ev(v)
    for pg, r, d, v in case["k"]:
        kc[pg, r, 0, d] = _ev(v)
    bt = np.array(case["block_table"], dtype=np.int64)
    sl = np.array(case["seqlens"], dtype=np.int64)
    for pg, r0, r1 in case.get("nan_rows", []):
        kc[pg, r0:r1] = np.nan
    # rows beyond each request's length in its pages are never visible: NaN them
    for b in range(B):
        L = int(sl[b])
        for lp in range(bt.shape[1]):
            for r in range(bs):
                if lp * bs + r >= L:
                    kc[bt[b, lp], r] = np.nan
    return q, kc, bt, sl


@pytest.mark.parametrize("idx", range(len(_golden_cases()["cases"])))
def test_closed_form_golden(idx):
    spec = _golden_cases()
    case = spec["cases"][idx]
    q, kc, bt, sl = _build_case(case, spec["d_k"], spec["block_size"])
    O, LSE = decode(q, kc, bt, sl, _ev(case["scale"]), case["causal"])
    expO = np.zeros_like(O)
    for b, t, h, d, v in case["expect_O"]:
        expO[b, t, h, d] = _ev(v)
    expL = np.full_like(LSE, np.nan)
    for b, t, h, v in case["expect_LSE"]:
        expL[b, t, h] = _ev(v)
    assert not np.any(np.isnan(O)), case["name"]
    np.testing.assert_allclose(O, expO, rtol=0, atol=1e-13, err_msg=case["name"])
    assert np.all((LSE == expL) | (np.abs(LSE - expL) <= 1e-13)), (case["name"], LSE, expL)
    # the scalar-loop definition agrees too
    Ob, Lb = decode_bruteforce(q, kc, bt, sl, _ev(case["scale"]), case["causal"])
    np.testing.assert_allclose(Ob, expO, rtol=0, atol=1e-13)
    assert np.all((Lb == expL) | (np.abs(Lb - expL) <= 1e-13))


@pytest.mark.parametrize("seqlens,s_q,h_q", [
    ([1, 2, 63], 1, 2),
    ([64, 65], 1, 3),
    ([130, 7, 1], 2, 2),
    ([2, 66], 2, 1),
])
def test_bruteforce_agrees(seqlens, s_q, h_q):
    inp = build_inputs(seqlens, s_q, h_q, seed=7 + len(seqlens) + s_q, extra_pool=3)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    Ob, Lb = decode_bruteforce(inp.q, inp.kcache, inp.block_table, inp.seqlens,
                               inp.scale, inp.causal)
    fin = np.isfinite(Lb)
    assert np.array_equal(fin, np.isfinite(L))
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O, Ob, rtol=1e-11, atol=1e-12)


def test_block_table_permutation_invariance():
    inp = build_inputs([200, 64, 129], 1, 4, seed=11, extra_pool=5)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    g = torch.Generator().manual_seed(3)
    npages = inp.kcache.shape[0]
    perm = torch.randperm(npages, generator=g)            # new physical slot of page p
    newk = torch.empty_like(inp.kcache)
    newk[perm] = inp.kcache
    newbt = perm[inp.block_table.long()].to(torch.int32)
    O2, L2 = decode(inp.q, newk, newbt, inp.seqlens, inp.scale, inp.causal)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_single_token_is_v0():
    inp = build_inputs([1, 1], 1, 8, seed=5, extra_pool=2)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, inp.causal)
    for b in range(2):
        k0 = inp.kcache[int(inp.block_table[b, 0]), 0, 0].double().numpy()
        assert np.array_equal(O[b, 0], np.broadcast_to(k0[:512], (8, 512)))
        qd = inp.q[b, 0].double().numpy()
        np.testing.assert_allclose(L[b, 0], inp.scale * qd @ k0, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("mode", ["zero_q", "zero_scale"])
def test_equal_scores_mean(mode):
    inp = build_inputs([100, 37], 1, 4, seed=9, extra_pool=1)
    q = torch.zeros_like(inp.q) if mode == "zero_q" else inp.q
    scale = 0.0 if mode == "zero_scale" else inp.scale
    O, L = decode(q, inp.kcache, inp.block_table, inp.seqlens, scale, inp.causal)
    for b in range(2):
        K = gather_request_kv(inp.kcache, inp.block_table, inp.seqlens, b)
        mean = K[:, :512].mean(axis=0)
        np.testing.assert_allclose(O[b, 0], np.broadcast_to(mean, (4, 512)), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(L[b, 0], math.log(int(inp.seqlens[b])), rtol=1e-14)


def test_absorbed_form_equals_per_head():
    inp = build_inputs([150], 2, 8, seed=13, extra_pool=1)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, True)
    K = gather_request_kv(inp.kcache, inp.block_table, inp.seqlens, 0)
    Ln = int(inp.seqlens[0])
    for t in range(2):
        for h in range(8):
            qv = inp.q[0, t, h].double().numpy()
            nv = Ln - 2 + 1 + t
            s = inp.scale * (K[:nv] @ qv)
            m = s.max()
            w = np.exp(s - m)
            lse = m + math.log(w.sum())
            o = (w / w.sum()) @ K[:nv, :512]
            np.testing.assert_allclose(O[0, t, h], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(L[0, t, h], lse, rtol=1e-13)


def test_causal_reduces_to_single_token():
    inp = build_inputs([97], 2, 4, seed=17, extra_pool=1)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, True)
    # token 1 == s_q=1 problem with length L; token 0 == s_q=1 with length L-1
    for t, Lt in ((1, 97), (0, 96)):
        q1 = inp.q[:, t:t + 1].contiguous()
        O1, L1 = decode(q1, inp.kcache, inp.block_table, torch.tensor([Lt], dtype=torch.int32),
                        inp.scale, False)
        np.testing.assert_allclose(O[:, t], O1[:, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L[:, t], L1[:, 0], rtol=1e-14)


def test_rope_shift_changes_lse_only():
    inp = build_inputs([77, 140], 1, 4, seed=19, extra_pool=1, nan_tails=False)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, False)
    r = np.linspace(-0.5, 0.75, 64)
    k2 = inp.kcache.double().numpy().copy()
    k2[..., 512:] += r
    O2, L2 = decode(inp.q, k2, inp.block_table, inp.seqlens, inp.scale, False)
    np.testing.assert_allclose(O2, O, rtol=1e-10, atol=1e-12)
    shift = inp.scale * (inp.q[:, 0].double().numpy()[..., 512:] @ r)   # [B, h]
    np.testing.assert_allclose(L2[:, 0] - L[:, 0], shift, rtol=1e-10, atol=1e-11)


def test_convex_hull_and_lse_bounds():
    inp = build_inputs([300, 5], 1, 6, seed=23, extra_pool=1)
    O, L = decode(inp.q, inp.kcache, inp.block_table, inp.seqlens, inp.scale, False)
    for b in range(2):
        K = gather_request_kv(inp.kcache, inp.block_table, inp.seqlens, b)
        V = K[:, :512]
        assert np.all(O[b, 0] <= V.max(axis=0) + 1e-12)
        assert np.all(O[b, 0] >= V.min(axis=0) - 1e-12)
        s = inp.scale * (inp.q[b, 0].double().numpy() @ K.T)       # [h, L]
        assert np.all(L[b, 0] >= s.max(axis=1) - 1e-12)
        assert np.all(L[b, 0] <= s.max(axis=1) + math.log(K.shape[0]) + 1e-12)


@pytest.mark.parametrize("cuts", [(1,), (64,), (100, 130), (5, 6, 190)])
def test_split_merge_identity(cuts):
    inp = build_inputs([257], 1, 4, seed=29, extra_pool=1)
    K = gather_request_kv(inp.kcache, inp.block_table, inp.seqlens, 0)
    qrows = inp.q[0, 0].double().numpy()
    full_O, full_L = attend_rows(qrows, K, inp.scale, np.full(4, 257))
    edges = [0, *cuts, 257]
    parts = []
    for a, b in zip(edges[:-1], edges[1:]):
        parts.append(attend_rows(qrows, K[a:b], inp.scale, np.full(4, b - a)))
    O, L = lse_merge(parts)
    np.testing.assert_allclose(O, full_O, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L, full_L, rtol=1e-14)


def test_merge_with_empty_parts():
    O = np.ones((2, 512))
    L = np.array([0.5, -np.inf])
    empty = (np.zeros((2, 512)), np.array([-np.inf, -np.inf]))
    Om, Lm = lse_merge([(O, L), empty])
    np.testing.assert_allclose(Om[0], 1.0)
    assert Lm[0] == 0.5
    assert Lm[1] == -np.inf and np.all(Om[1] == 0)


def test_visible_count_rule():
    # s_q new tokens occupy the last s_q positions; token t sees L - s_q + 1 + t keys
    assert visible_count(10, 2, 0, True) == 9
    assert visible_count(10, 2, 1, True) == 10
    assert visible_count(1, 2, 0, True) == 0
    assert visible_count(10, 1, 0, True) == 10
    assert visible_count(10, 2, 0, False) == 10


def _golden_all_pass() -> bool:
    spec = _golden_cases()
    for case in spec["cases"]:
        q, kc, bt, sl = _build_case(case, spec["d_k"], spec["block_size"])
        with np.errstate(all="ignore"):
            O, LSE = omod.decode(q, kc, bt, sl, _ev(case["scale"]), case["causal"])
        expO = np.zeros_like(O)
        for b, t, h, d, v in case["expect_O"]:
            expO[b, t, h, d] = _ev(v)
        if np.any(np.isnan(O)) or np.max(np.abs(O - expO)) > 1e-9:
            return False
        for b, t, h, v in case["expect_LSE"]:
            e = _ev(v)
            got = LSE[b, t, h]
            if not (got == e or abs(got - e) <= 1e-9):
                return False
    return True


def test_planted_mistakes_are_caught(monkeypatch):
    """Plausible oracle slips, planted on the CPU, each fail the golden pins."""
    assert _golden_all_pass()
    orig_vis = omod.visible_count
    orig_attend = omod.attend_rows
    orig_gather = omod.gather_request_kv

    # 1. causal rule off by one
    monkeypatch.setattr(omod, "visible_count",
                        lambda L, s_q, t, causal: orig_vis(L, s_q, t, causal) - (1 if causal else 0))
    assert not _golden_all_pass()
    monkeypatch.setattr(omod, "visible_count", orig_vis)

    # 2. softmax scale dropped
    monkeypatch.setattr(omod, "attend_rows",
                        lambda qr, K, scale, nv, d_v=512: orig_attend(qr, K, 1.0, nv, d_v))
    assert not _golden_all_pass()
    # 3. values taken from the last 512 dims instead of the first 512
    def wrong_v(qr, K, scale, nv, d_v=512):
        Kv = np.concatenate([K[:, 64:], K[:, :64]], axis=1)
        O, L = orig_attend(qr, K, scale, nv, d_v)
        O2, _ = orig_attend(qr, K, scale, nv, d_v)
        # recompute O with the wrong value rows, same weights
        S = scale * (qr @ K.T)
        S = np.where(np.arange(K.shape[0])[None] < nv[:, None], S, -np.inf)
        with np.errstate(all="ignore"):
            P = np.exp(S - L[:, None])
        P = np.nan_to_num(P)
        return P @ Kv[:, :d_v], L
    monkeypatch.setattr(omod, "attend_rows", wrong_v)
    assert not _golden_all_pass()
    monkeypatch.setattr(omod, "attend_rows", orig_attend)

    # 4. page and row indices swapped in the gather
    def wrong_gather(kcache, block_table, seqlens, b):
        bt = np.asarray(block_table)
        L = int(np.asarray(seqlens)[b])
        kc = np.asarray(kcache, dtype=np.float64)
        rows = [kc[bt[b, j % bt.shape[1]], j // bt.shape[1], 0] for j in range(L)]
        return np.array(rows).reshape(L, -1)
    monkeypatch.setattr(omod, "gather_request_kv", wrong_gather)
    assert not _golden_all_pass()
    monkeypatch.setattr(omod, "gather_request_kv", orig_gather)
    assert _golden_all_pass()


# ---- paged-KV append (the cache write that precedes decode) ----------------

def _append_case(seed=7):
    from workloads import build_inputs
    inp = build_inputs([1, 63, 64, 65, 130, 0, 2], 3, 16, seed=seed, extra_pool=3)
    g = torch.Generator().manual_seed(seed + 1)
    new = torch.randn((inp.batch, 3, 576), generator=g).to(torch.bfloat16)
    return inp, new


def test_append_round_trip():
    """After the append, gathering each request through its block table gives
    the new rows at positions L-s_q .. L-1 (bit for bit) and every earlier
    row unchanged; a request shorter than s_q gets only its last L rows."""
    from oracle import gather_request_kv, kv_append
    inp, new = _append_case()
    kc2 = kv_append(inp.kcache, inp.block_table, inp.seqlens, new)
    for b, L in enumerate(inp.seqlens.tolist()):
        before = gather_request_kv(inp.kcache, inp.block_table, inp.seqlens, b)
        after = gather_request_kv(kc2, inp.block_table, inp.seqlens, b)
        k0 = max(0, L - 3)
        np.testing.assert_array_equal(after[:k0], before[:k0])
        for t in range(3):
            pos = L - 3 + t
            if pos >= 0:
                np.testing.assert_array_equal(after[pos], new[b, t].double().numpy())


def test_append_touches_only_new_rows():
    """Rows not owned by a request's new tokens (other pages, tails, the NaN
    sentinel page) are left exactly as they were."""
    from oracle import kv_append
    inp, new = _append_case(11)
    kc2 = kv_append(inp.kcache, inp.block_table, inp.seqlens, new)
    written = set()
    for b, L in enumerate(inp.seqlens.tolist()):
        for t in range(3):
            pos = L - 3 + t
            if pos >= 0:
                written.add((int(inp.block_table[b, pos // 64]), pos % 64))
    diff = ~torch.eq(kc2.view(torch.int16), inp.kcache.view(torch.int16)).all(dim=-1).squeeze(-1)
    changed = {(int(p), int(r)) for p, r in torch.nonzero(diff).tolist()}
    assert changed <= written


@pytest.mark.parametrize("cuts", [(64,), (100, 130), (5, 6, 190), (32, 64, 96, 128, 160, 192, 224)])
def test_bf16_partials_error_bound(cuts):
    """Split partials stored in bf16 (the decode's workspace format): merging
    bf16-rounded piece outputs moves the merged output by at most
    2^-8 * max_i |O_i| per element (bf16 keeps 8 significant bits, so
    round-to-nearest-even has relative error <= 2^-8; the merge weights are
    nonnegative and sum to one), and the
    LSE not at all; the bound is what the tolerance of the parity tests must
    absorb on top of the kernel's own rounding."""
    inp = build_inputs([257], 1, 8, seed=31, extra_pool=1)
    K = gather_request_kv(inp.kcache, inp.block_table, inp.seqlens, 0)
    qrows = inp.q[0, 0].double().numpy()
    edges = [0, *cuts, 257]
    parts = [attend_rows(qrows, K[a:b], inp.scale, np.full(8, b - a))
             for a, b in zip(edges[:-1], edges[1:])]
    exact_O, exact_L = lse_merge(parts)
    rounded = [(torch.from_numpy(O).to(torch.bfloat16).double().numpy(), L) for O, L in parts]
    O, L = lse_merge(rounded)
    bound = 2.0 ** -8 * np.max(np.stack([np.abs(p[0]) for p in parts]), axis=0)
    assert np.all(np.abs(O - exact_O) <= bound + 1e-15)
    np.testing.assert_array_equal(L, exact_L)
    # the bound is not vacuous: the rounding does move the merged output
    assert np.max(np.abs(O - exact_O)) > 2.0 ** -8 * np.max(np.abs(exact_O)) / 64
