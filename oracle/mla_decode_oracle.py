"""Plain fp64 CPU oracle for MLA paged-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

What it computes (sources are the pages this project is built from):

* MLA: many query heads attend over a single shared latent KV head
  (page "深度剖析DeepSeek Infra开源全貌", jingzhunhuoke.net/55333.html,
  DAY1 FlashMLA, terminology paragraph on MLA).  Keys are 576 wide (512 latent
  + 64 rope); values are the first 512 dims of the same cache rows.
* The KV cache is paged in blocks of 64 tokens (same page, DAY1 feature ②);
  a request's logical token j lives in row j % 64 of physical page
  block_table[b][j // 64].
* The kernel is an exact, tiled rearrangement of ordinary softmax attention in
  the FlashAttention lineage (same page, DAY1 terminology paragraph on
  FlashMLA), computed as two products, scores then probabilities times values
  (same page, DAY1 feature ④, "Gemm1"/"Gemm2").  The exact result therefore
  has a plain definition, and this oracle is that definition in fp64:

      s_j  = scale * sum_d q_d K[j, d]                  (j visible)
      LSE  = log(sum_j exp(s_j))                       (natural log, fp64)
      O    = sum_j exp(s_j - LSE) * K[j, :512]

  with query row r = t*h_q + h of request b, and the visible set
  j < L_b - s_q + 1 + t when causal (the s_q newest tokens are already in the
  cache), else j < L_b.  An empty visible set gives O = 0, LSE = -inf.
* A position whose table slot j // 64 lies past the end of the request's
  table row, or whose slot names no page of the pool (a negative id or one
  at or beyond the pool size), holds no key: it is left out of the visible
  set.  The pages do not cover such a caller error; this project reads it as
  the sparse mode reads the same entries (skipped), so both modes agree and
  the result stays a softmax over real keys (``mapped_keys``).
* Variable lengths are balanced by splitting one request's keys over several
  workers and merging the pieces (same page, DAY1 feature ⑤, dynamic load for
  variable-length input); the merge by log-sum-exp (``lse_merge``) is exact.
* ``split_plan`` is the reference model of the split-KV work partition.  The
  pages only say that work is balanced dynamically; the precise plan is this
  project's own definition (stated in the function), and its parity is pinned
  by invariants (coverage exactly once, order, balance), not by the pages.

Precision: inputs are upcast exactly (bf16 -> fp64); all arithmetic is fp64.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK_SIZE = 64
D_K = 576
D_V = 512


def _f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (any float dtype, incl. bf16) or array."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu()
            if x.is_floating_point():
                x = x.to(torch.float64)
            return x.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _i64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().to(torch.int64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.int64)


def num_pages(seqlen: int, block_size: int = BLOCK_SIZE) -> int:
    return (int(seqlen) + block_size - 1) // block_size


def mapped_keys(block_table, seqlens, b: int, num_pool_pages: int) -> np.ndarray:
    """Which of request b's positions j < L_b hold a key (bool [L_b]): the
    table slot j // 64 lies inside the request's row and names a page id in
    [0, num_pool_pages)."""
    bt = _i64(block_table)
    L = int(_i64(seqlens)[b])
    slot = np.arange(L) // BLOCK_SIZE
    inrow = slot < bt.shape[1]
    page = np.where(inrow, bt[b, np.minimum(slot, bt.shape[1] - 1)], -1)
    return inrow & (page >= 0) & (page < num_pool_pages)


def gather_request_kv(kcache, block_table, seqlens, b: int) -> np.ndarray:
    """K_b[j, :] for j < L_b, gathered page by page (fp64, [L_b, 576]).

    Follows the paging of DAY1 feature ② (64-token pages) on the page cited in
    the module docstring: token j is row j % 64 of page block_table[b][j//64].
    Only the first ceil(L_b/64) table slots and only rows j < L_b are read;
    positions without a key (``mapped_keys``) come back as zero rows, which
    the attention leaves out.
    """
    kc = kcache if isinstance(kcache, np.ndarray) else None
    bt = _i64(block_table)
    L = int(_i64(seqlens)[b])
    bs = (kcache.shape[1])
    n = num_pages(L, bs)
    if n == 0:
        return np.zeros((0, kcache.shape[-1]), dtype=np.float64)
    n_pool = int(kcache.shape[0])
    slots = np.arange(n)
    pages = np.where(slots < bt.shape[1], bt[b, np.minimum(slots, bt.shape[1] - 1)], -1)
    ok = (pages >= 0) & (pages < n_pool)
    safe = np.where(ok, pages, 0)
    if kc is None:
        import torch
        rows = kcache[torch.as_tensor(safe)]           # [n, 64, 1, 576], still bf16
        K = _f64(rows).reshape(n, bs, -1)
    else:
        K = np.asarray(kc[safe], dtype=np.float64).reshape(n, bs, -1)
    K[~ok] = 0.0
    return K.reshape(n * bs, -1)[:L]


def counted_view(K: np.ndarray, counted: np.ndarray, nvis: np.ndarray):
    """The keys that count, in position order, and each row's visible count
    among them: the first nvis_c[r] rows of K[counted] are exactly the
    counted positions j < nvis[r]."""
    ccum = np.concatenate([[0], np.cumsum(counted.astype(np.int64))])
    return K[counted], ccum[np.minimum(nvis, K.shape[0])]


def kv_append(kcache, block_table, seqlens, new_kv) -> np.ndarray:
    """The cache after writing each request's s_q new key rows into their pages.

    Paging as above (64-token pages, token j in row j % 64 of page
    block_table[b][j // 64]); the lengths already count the new tokens, so new
    token t of request b is token L_b - s_q + t.  Positions before 0 (a
    request shorter than s_q) and positions whose page slot is outside the
    block table are not written.  Returns a new array (the input's dtype is
    kept, so bf16 rows are copied bit for bit); new_kv is [B, s_q, 576].
    """
    kc = kcache.clone() if hasattr(kcache, "clone") else np.array(kcache, copy=True)
    bt = _i64(block_table)
    sl = _i64(seqlens)
    B, s_q = int(new_kv.shape[0]), int(new_kv.shape[1])
    for b in range(B):
        for t in range(s_q):
            pos = int(sl[b]) - s_q + t
            if pos < 0 or pos // BLOCK_SIZE >= bt.shape[1]:
                continue
            page = int(bt[b, pos // BLOCK_SIZE])
            if page < 0 or page >= kc.shape[0]:
                continue
            kc[page, pos % BLOCK_SIZE, 0, :] = new_kv[b, t, :]
    return kc


def visible_count(L: int, s_q: int, t: int, causal: bool) -> int:
    """Number of keys query token t of a request of length L may see."""
    if not causal:
        return max(0, L)
    return max(0, min(L, L - s_q + 1 + t))


def attend_rows(qrows: np.ndarray, K: np.ndarray, scale: float, nvis: np.ndarray,
                d_v: int = D_V):
    """Softmax attention of each row of ``qrows`` over its first nvis[r] keys.

    qrows: [M, 576] fp64; K: [L, 576] fp64 (values = K[:, :d_v]).
    Returns O [M, d_v], LSE [M] (natural log).  One fp64 GEMM for the scores
    (the absorbed form: all M rows against the same latent keys).
    """
    M = qrows.shape[0]
    L = K.shape[0]
    O = np.zeros((M, d_v), dtype=np.float64)
    lse = np.full((M,), -np.inf, dtype=np.float64)
    if L == 0:
        return O, lse
    S = scale * (qrows @ K.T)                          # [M, L]
    col = np.arange(L)[None, :]
    vis = col < nvis[:, None]
    S = np.where(vis, S, -np.inf)
    has = nvis > 0
    if not np.any(has):
        return O, lse
    m = np.max(S[has], axis=1, keepdims=True)
    e = np.exp(S[has] - m)
    ssum = e.sum(axis=1, keepdims=True)
    lse[has] = (m + np.log(ssum))[:, 0]
    P = e / ssum
    O[has] = P @ K[:, :d_v]
    return O, lse


def decode(q, kcache, block_table, seqlens, scale: float, causal: bool,
           requests=None):
    """fp64 reference of paged MLA decode.

    q [B, s_q, h_q, 576], kcache [pages, 64, 1, 576], block_table [B, stride],
    seqlens [B].  Returns (O [B, s_q, h_q, 512], LSE [B, s_q, h_q]) in fp64;
    rows of requests not listed in ``requests`` are NaN.
    """
    qf = _f64(q)
    B, s_q, h_q, dk = qf.shape
    sl = _i64(seqlens)
    O = np.full((B, s_q, h_q, D_V), np.nan, dtype=np.float64)
    LSE = np.full((B, s_q, h_q), np.nan, dtype=np.float64)
    reqs = range(B) if requests is None else requests
    for b in reqs:
        L = int(sl[b])
        K = gather_request_kv(kcache, block_table, seqlens, b)
        qrows = qf[b].reshape(s_q * h_q, dk)
        nvis = np.array([visible_count(L, s_q, r // h_q, causal)
                         for r in range(s_q * h_q)], dtype=np.int64)
        Kc, nvis_c = counted_view(K, mapped_keys(block_table, seqlens, b, int(kcache.shape[0])), nvis)
        Ob, lb = attend_rows(qrows, Kc, scale, nvis_c)
        O[b] = Ob.reshape(s_q, h_q, D_V)
        LSE[b] = lb.reshape(s_q, h_q)
    return O, LSE


def decode_bruteforce(q, kcache, block_table, seqlens, scale: float, causal: bool):
    """The same definition with scalar Python loops (math.fsum, math.exp).

    No numpy arithmetic; for tiny inputs only.  Used to pin ``decode``.
    """
    qf = _f64(q).tolist()
    kf = _f64(kcache)
    bt = _i64(block_table).tolist()
    sl = [int(x) for x in _i64(seqlens)]
    B = len(qf)
    s_q = len(qf[0])
    h_q = len(qf[0][0])
    bs = kf.shape[1]
    kl = kf.tolist()
    O = [[[None] * h_q for _ in range(s_q)] for _ in range(B)]
    LSE = [[[None] * h_q for _ in range(s_q)] for _ in range(B)]
    for b in range(B):
        L = sl[b]
        for t in range(s_q):
            nv = visible_count(L, s_q, t, causal)
            for h in range(h_q):
                qv = qf[b][t][h]
                scores = []
                rows = []
                for j in range(nv):
                    if j // bs >= len(bt[b]) or not 0 <= bt[b][j // bs] < len(kl):
                        continue          # no page: no key at this position
                    row = kl[bt[b][j // bs]][j % bs][0]
                    rows.append(row)
                    scores.append(scale * math.fsum(qv[d] * row[d] for d in range(len(qv))))
                if not rows:
                    O[b][t][h] = [0.0] * D_V
                    LSE[b][t][h] = -math.inf
                    continue
                m = max(scores)
                denom = math.fsum(math.exp(s - m) for s in scores)
                lse = m + math.log(denom)
                w = [math.exp(s - lse) for s in scores]
                O[b][t][h] = [math.fsum(w[j] * rows[j][d] for j in range(len(rows)))
                              for d in range(D_V)]
                LSE[b][t][h] = lse
    return np.array(O, dtype=np.float64), np.array(LSE, dtype=np.float64)


def lse_merge(parts):
    """Exact merge of attention results over disjoint key subsets.

    parts: list of (O_i [..., d_v], LSE_i [...]) where O_i is the normalised
    output over key subset i and LSE_i its log-sum-exp.  Returns (O, LSE) of
    attention over the union:  LSE = log sum_i exp(LSE_i),
    O = sum_i exp(LSE_i - LSE) O_i.  Subsets with LSE_i = -inf contribute 0;
    if all are -inf the result is O = 0, LSE = -inf.
    (Split-KV balancing of variable lengths: page cited above, DAY1 ⑤.)
    """
    Os = [np.asarray(p[0], dtype=np.float64) for p in parts]
    Ls = [np.asarray(p[1], dtype=np.float64) for p in parts]
    Lst = np.stack(Ls)                                   # [n, ...]
    m = np.max(Lst, axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(Lst), np.exp(Lst - m_safe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    O = np.zeros_like(Os[0])
    for wi, Oi in zip(w, Os):
        coef = np.where(finite, wi / np.where(finite, tot, 1.0), 0.0)
        O = O + coef[..., None] * Oi
    return O, lse


# ---------------------------------------------------------------------------
# Split-KV work partition (reference model).
# ---------------------------------------------------------------------------

def fixed_cost_pages(rows_per_tile: int) -> int:
    """Per-request overhead, in page units, charged once per request.

    The overhead of starting a request (loading its query rows, writing its
    result) grows with the rows a workgroup carries: one page per 32 rows
    (none for 16 rows).
    """
    return rows_per_tile // 32


def rows_per_tile(s_q: int, h_q: int) -> int:
    """Query rows one workgroup carries: all of them, up to 128."""
    return min(s_q * h_q, 128)


def split_plan(seqlens, s_q: int, h_q: int, num_parts: int,
               block_size: int = BLOCK_SIZE):
    """Deterministic partition of all requests' pages over ``num_parts`` parts.

    Definition (integers only):
      n_b    = ceil(L_b / 64) pages;  c = fixed_cost_pages(rows_per_tile)
      cost_b = n_b + c if n_b > 0 else 0
      start_b = sum_{b' < b} cost_b';   C = sum_b cost_b
      q      = ceil(C / P)  (q = 1 if C = 0)
      Request b occupies units [start_b, start_b + cost_b): its first c units
      are overhead, page k is unit start_b + c + k.
      Boundary x (a unit position) maps to (b, k): the request whose units
      contain x and k = clamp(x - start_b - c, 0, n_b); x >= C maps to (B, 0).
      Part p covers [boundary(p*q), boundary((p+1)*q)) in (request, page)
      lexicographic order (part P-1 ends at (B, 0)).
      A boundary strictly inside request b's pages (0 < k < n_b) splits it.
      n_split_b = 1 + #{p >= 1 : start_b + c < p*q < start_b + c + n_b}.
      first_split(p) = (p - p0_b + 1) if part p begins strictly inside
      request b, else 0, where p0_b = floor((start_b + c) / q) + 1.
      split_offsets[0] = 0, split_offsets[b+1] = split_offsets[b]
                         + (n_split_b if n_split_b >= 2 else 0).

    Returns (tile_meta int32 [P, 8] = {begin_req, begin_page, end_req,
    end_page, first_split, 0, 0, 0}, split_offsets int32 [B+1]).
    """
    sl = [int(x) for x in _i64(seqlens)]
    B = len(sl)
    P = int(num_parts)
    c = fixed_cost_pages(rows_per_tile(s_q, h_q))
    n = [num_pages(L, block_size) if L > 0 else 0 for L in sl]
    cost = [n[b] + c if n[b] > 0 else 0 for b in range(B)]
    start = []
    acc = 0
    for b in range(B):
        start.append(acc)
        acc += cost[b]
    C = acc
    q = max(1, -(-C // P)) if C > 0 else 1

    def boundary(x: int):
        if x >= C:
            return (B, 0)
        for b in range(B):
            if cost[b] > 0 and start[b] <= x < start[b] + cost[b]:
                k = min(max(x - start[b] - c, 0), n[b])
                return (b, k)
        raise AssertionError("unreachable")

    tile_meta = np.zeros((P, 8), dtype=np.int32)
    for p in range(P):
        b0, k0 = boundary(p * q)
        b1, k1 = boundary((p + 1) * q) if p + 1 < P else (B, 0)
        first = 0
        if b0 < B and 0 < k0 < n[b0]:
            p0 = (start[b0] + c) // q + 1
            first = p - p0 + 1
        tile_meta[p, :5] = (b0, k0, b1, k1, first)
    split_offsets = np.zeros((B + 1,), dtype=np.int32)
    for b in range(B):
        ns = 1
        if n[b] > 0:
            lo = start[b] + c
            hi = lo + n[b]
            ns = 1 + ((hi - 1) // q - lo // q)
        split_offsets[b + 1] = split_offsets[b] + (ns if ns >= 2 else 0)
    return tile_meta, split_offsets


def plan_pieces(tile_meta, seqlens, block_size: int = BLOCK_SIZE):
    """Expand a partition into per-part lists of (request, first_page, end_page).

    Pieces of zero pages are dropped.  Used to check partitions.
    """
    sl = [int(x) for x in _i64(seqlens)]
    B = len(sl)
    n = [num_pages(L, block_size) for L in sl]
    out = []
    for row in np.asarray(tile_meta):
        b0, k0, b1, k1 = (int(v) for v in row[:4])
        pieces = []
        b = b0
        while b < B and (b < b1 or (b == b1 and k1 > 0)):
            lo = k0 if b == b0 else 0
            hi = k1 if b == b1 else n[b]
            if hi > lo:
                pieces.append((b, lo, hi))
            b += 1
        out.append(pieces)
    return out
