"""fp64 CPU oracle of the sparse (selected-keys) mode of MLA paged decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Source.  The page "云上玩转DeepSeek系列之五：实测优化16%，体验FlashMLA加速
DeepSeek-V2-Lite推理" (ruibaoantu.com), section 四 (best practices), item 2
(monitoring and tuning), recommends FlashMLA's sparse attention mode for
sequences beyond 8K tokens; the page "深度剖析DeepSeek Infra开源全貌" and the
others give no algorithm for it.  This project's reading, the plainest one
that keeps everything else of the dense definition:

* For query token t of request b the caller supplies topk cache positions
  indices[b, t, 0:topk] (chosen by any top-k selector; the selection itself
  is not part of the mode).
* An entry counts iff 0 <= j < vis(b, t), the dense mode's visible limit
  (L_b - s_q + 1 + t when causal, else L_b), and its table slot j // 64 is
  inside the request's row with a page id in the pool; other entries
  (negative padding, positions beyond the limit, unmapped positions) are
  skipped.
* The attention of every head h of token t is the dense definition restricted
  to the counted entries, taken as a multiset (an entry listed twice counts
  twice):  s_i = scale * q . K_b[j_i],  LSE = ln sum_i exp(s_i),
  O = sum_i exp(s_i - LSE) K_b[j_i, :512];  no counted entry: O = 0,
  LSE = -inf.  Keys are gathered through the block table as in the dense
  mode (token j is row j % 64 of page block_table[b][j // 64]).
* Over an FP8 page pool (the same page names FP8 as its other throughput
  step) each selected row is dequantised exactly as the FP8 oracle does
  (latent = e4m3(code) * scale, rope as stored); nothing else changes.
"""
from __future__ import annotations

import math

import numpy as np

from .mla_decode_oracle import BLOCK_SIZE, D_V, _f64, _i64, attend_rows, visible_count


def counted_entries(indices_bt, vis: int, block_table_b=None, num_pages_pool=None) -> np.ndarray:
    """The entries of one token's index list that count (multiset, in order):
    0 <= j < vis and, when the request's table row and the pool size are
    given, a table slot j // 64 inside the row holding a page id in
    [0, num_pages_pool)."""
    ix = np.asarray(indices_bt, dtype=np.int64).reshape(-1)
    ix = ix[(ix >= 0) & (ix < vis)]
    if block_table_b is None:
        return ix
    bt = np.asarray(block_table_b, dtype=np.int64).reshape(-1)
    slot = ix // BLOCK_SIZE
    inrow = slot < bt.size
    page = np.where(inrow, bt[np.minimum(slot, bt.size - 1)], -1)
    return ix[inrow & (page >= 0) & (page < num_pages_pool)]


def _gather_rows(kcache, block_table_b, positions) -> np.ndarray:
    """K rows (fp64 [n, 576]) of the given logical positions of one request."""
    import torch
    pos = np.asarray(positions, dtype=np.int64)
    if pos.size == 0:
        return np.zeros((0, kcache.shape[-1]), dtype=np.float64)
    pages = np.asarray(block_table_b, dtype=np.int64)[pos // BLOCK_SIZE]
    rows = pos % BLOCK_SIZE
    if isinstance(kcache, torch.Tensor):
        sel = kcache[torch.as_tensor(pages), torch.as_tensor(rows), 0]
        return _f64(sel)
    return np.asarray(kcache[pages, rows, 0], dtype=np.float64)


def _gather_rows_fp8(pool, block_table_b, positions, cache: dict) -> np.ndarray:
    """Key rows (fp64 [n, 576], exact) of the given logical positions of one
    request in an FP8 page pool; dequantised pages are memoised in ``cache``."""
    from .mla_fp8_oracle import dequant_page, FP8_PAGE_BYTES
    pos = np.asarray(positions, dtype=np.int64)
    out = np.zeros((pos.size, 576), dtype=np.float64)
    if pos.size == 0:
        return out
    pool8 = pool.reshape(-1, FP8_PAGE_BYTES)
    bt = np.asarray(block_table_b, dtype=np.int64)
    for i, j in enumerate(pos):
        page = int(bt[j // BLOCK_SIZE])
        if page not in cache:
            cache[page] = dequant_page(pool8[page])
        out[i] = cache[page][j % BLOCK_SIZE]
    return out


def decode_sparse(q, kcache, block_table, seqlens, indices, scale: float, causal: bool,
                  requests=None):
    """fp64 reference of the sparse mode over a bf16 paged cache.

    q [B, s_q, h_q, 576]; kcache [pages, 64, 1, 576]; block_table [B, stride];
    seqlens [B]; indices int [B, s_q, topk].  Returns (O [B, s_q, h_q, 512],
    LSE [B, s_q, h_q]) in fp64; rows of requests not listed in ``requests``
    are NaN.
    """
    qf = _f64(q)
    B, s_q, h_q, dk = qf.shape
    sl = _i64(seqlens)
    bt = _i64(block_table)
    ix = _i64(indices)
    O = np.full((B, s_q, h_q, D_V), np.nan, dtype=np.float64)
    LSE = np.full((B, s_q, h_q), np.nan, dtype=np.float64)
    reqs = range(B) if requests is None else requests
    n_pool = int(kcache.shape[0])
    for b in reqs:
        L = int(sl[b])
        for t in range(s_q):
            ent = counted_entries(ix[b, t], visible_count(L, s_q, t, causal), bt[b], n_pool)
            K = _gather_rows(kcache, bt[b], ent)
            nvis = np.full((h_q,), K.shape[0], dtype=np.int64)
            Ob, lb = attend_rows(qf[b, t], K, scale, nvis)
            O[b, t] = Ob
            LSE[b, t] = lb
    return O, LSE


def decode_sparse_bruteforce(q, kcache, block_table, seqlens, indices, scale: float,
                             causal: bool):
    """The same definition with scalar Python loops (math.fsum, math.exp) and
    a per-entry validity test; tiny inputs only.  Used to pin decode_sparse."""
    qf = _f64(q).tolist()
    kf = _f64(kcache)
    bt = _i64(block_table).tolist()
    sl = [int(x) for x in _i64(seqlens)]
    ix = _i64(indices).tolist()
    B, s_q, h_q = len(qf), len(qf[0]), len(qf[0][0])
    O = np.zeros((B, s_q, h_q, D_V))
    LSE = np.zeros((B, s_q, h_q))
    for b in range(B):
        for t in range(s_q):
            vis = visible_count(sl[b], s_q, t, causal)
            rows = []
            for j in ix[b][t]:
                if not 0 <= j < vis or j // BLOCK_SIZE >= len(bt[b]):
                    continue
                page = bt[b][j // BLOCK_SIZE]
                if 0 <= page < kf.shape[0]:
                    rows.append(kf[page, j % BLOCK_SIZE, 0].tolist())
            for h in range(h_q):
                qv = qf[b][t][h]
                if not rows:
                    O[b, t, h] = 0.0
                    LSE[b, t, h] = -math.inf
                    continue
                sc = [scale * math.fsum(qv[d] * r[d] for d in range(len(qv))) for r in rows]
                m = max(sc)
                lse = m + math.log(math.fsum(math.exp(s - m) for s in sc))
                w = [math.exp(s - lse) for s in sc]
                O[b, t, h] = [math.fsum(w[i] * rows[i][d] for i in range(len(rows)))
                              for d in range(D_V)]
                LSE[b, t, h] = lse
    return O, LSE


def decode_sparse_fp8(q, pool, block_table, seqlens, indices, scale: float, causal: bool,
                      requests=None):
    """fp64 reference of the sparse mode over an FP8 page pool: the definition
    of ``decode_sparse`` with every selected key row dequantised exactly as in
    ``mla_fp8_oracle`` (latent = e4m3(code) * scale, rope as stored).

    pool uint8 [pages, 41216]; other arguments and the result as
    ``decode_sparse``."""
    from .mla_fp8_oracle import _u8
    qf = _f64(q)
    B, s_q, h_q, dk = qf.shape
    sl = _i64(seqlens)
    bt = _i64(block_table)
    ix = _i64(indices)
    pool8 = _u8(pool)
    O = np.full((B, s_q, h_q, D_V), np.nan, dtype=np.float64)
    LSE = np.full((B, s_q, h_q), np.nan, dtype=np.float64)
    cache: dict = {}
    from .mla_fp8_oracle import FP8_PAGE_BYTES
    n_pool = pool8.reshape(-1, FP8_PAGE_BYTES).shape[0]
    reqs = range(B) if requests is None else requests
    for b in reqs:
        L = int(sl[b])
        for t in range(s_q):
            ent = counted_entries(ix[b, t], visible_count(L, s_q, t, causal), bt[b], n_pool)
            K = _gather_rows_fp8(pool8, bt[b], ent, cache)
            nvis = np.full((h_q,), K.shape[0], dtype=np.int64)
            Ob, lb = attend_rows(qf[b, t], K, scale, nvis)
            O[b, t] = Ob
            LSE[b, t] = lb
    return O, LSE
