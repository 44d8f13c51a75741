"""Seeded synthetic inputs for MLA paged-KV decode.

This module only draws random numbers and lays them out in the paged-cache
format; it performs none of the attention arithmetic.  Both the fp64 oracle
(``oracle/``) and the HIP path consume exactly the bytes produced here.

Workload shapes follow the paged-KV decode setting of the page
"深度剖析DeepSeek Infra开源全貌" (jingzhunhuoke.net/55333.html), DAY1 FlashMLA,
feature ② (KV cache paged in 64-token blocks); head sizes (576-wide latent+rope
key, value = its first 512 dims, one shared KV head) are the MLA decode shape.

Recipe (per workload, generator ``torch.Generator('cpu').manual_seed(seed)``,
drawn in this order):
  1. seqlens (distribution per workload, below),
  2. a random permutation of the KV pool assigned, in order, to every
     request's logical blocks,
  3. Q ~ N(0,1) fp32 [B, s_q, h_q, 576] rounded to bf16 (round-to-nearest-even),
  4. KV pool ~ N(0,1) fp32 [pool, 64, 1, 576] rounded to bf16.
Then: one extra NaN-filled "sentinel" block is appended at index ``pool`` and
every unused block-table slot points at it; the rows of each request's last
block that lie beyond its length are overwritten with NaN.  Neither may ever
influence a result.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

BLOCK_SIZE = 64
D_K = 576
D_V = 512


@dataclass(frozen=True)
class Workload:
    key: str
    name: str
    batch: int
    s_q: int
    h_q: int
    seqlen_kind: str
    seed: int
    h_kv: int = 1
    extra_pool: int = 64
    fixed_pool: int | None = None
    topk: int = 0              # > 0: sparse mode, this many selected positions per token
    desc: str = field(default="", compare=False)

    @property
    def rows(self) -> int:
        return self.s_q * self.h_q


WORKLOADS: dict[str, Workload] = {
    "tiny": Workload("tiny", "tiny MLA decode", batch=2, s_q=1, h_q=16,
                     seqlen_kind="tiny", seed=1000, fixed_pool=8,
                     desc="B=2, s_q=1, h_q=16, seqlens {65,130}, pool of 8 blocks"),
    "membound": Workload("membound", "memory-bound decode", batch=64, s_q=1, h_q=16,
                         seqlen_kind="const4096", seed=1001, extra_pool=64,
                         desc="B=64, s_q=1, h_q=16, every seqlen 4096, pool 4096+64"),
    "ridge": Workload("ridge", "compute-near-ridge decode", batch=128, s_q=1, h_q=128,
                      seqlen_kind="uniform1024_8192", seed=1002, extra_pool=64,
                      desc="B=128, s_q=1, h_q=128, seqlens U[1024,8192]"),
    "ragged": Workload("ragged", "ragged 2-token speculative decode", batch=132, s_q=2,
                       h_q=128, seqlen_kind="lognormal", seed=1003, extra_pool=64,
                       desc="B=132, s_q=2 causal, h_q=128, seqlens "
                            "clamp(round(lognormal(7.5,1)),1,32768)"),
    "long": Workload("long", "long-context decode", batch=16, s_q=1, h_q=128,
                     seqlen_kind="alt16k_64k", seed=1004, fixed_pool=10496,
                     desc="B=16, s_q=1, h_q=128, seqlens alternating 16384/65536, "
                          "pool 10496 blocks"),
    # Beyond the five configurations above: decode of four draft tokens per
    # request (speculative decoding), causal among themselves.
    "draft": Workload("draft", "4-token draft decode", batch=32, s_q=4, h_q=128,
                      seqlen_kind="uniform2048_8192", seed=1005, extra_pool=64,
                      desc="B=32, s_q=4 causal, h_q=128, seqlens U[2048,8192]"),
    # A 64-token prefill chunk per request against the paged cache (the
    # chunk's tokens are already in the cache, causal among themselves).
    "prefill": Workload("prefill", "64-token chunked prefill", batch=8, s_q=64, h_q=128,
                        seqlen_kind="uniform2048_8192", seed=1006, extra_pool=64,
                        desc="B=8, s_q=64 causal, h_q=128, seqlens U[2048,8192]"),
    # Sparse mode on long contexts: each token attends over 2048 selected
    # positions of a 8K-32K context.
    "sparse": Workload("sparse", "top-2048 sparse long-context decode", batch=64, s_q=1,
                       h_q=128, seqlen_kind="uniform8192_32768", seed=1007, extra_pool=64,
                       topk=2048,
                       desc="B=64, s_q=1, h_q=128, seqlens U[8192,32768], 2048 selected "
                            "positions per token"),
}

# The order the workloads are listed in (index 0 is the small case).
WORKLOAD_ORDER = ["tiny", "membound", "ridge", "ragged", "long"]


def draw_seqlens(kind: str, batch: int, gen: torch.Generator) -> torch.Tensor:
    if kind == "tiny":
        return torch.tensor([65, 130], dtype=torch.int32)
    if kind == "const4096":
        return torch.full((batch,), 4096, dtype=torch.int32)
    if kind == "uniform1024_8192":
        return torch.randint(1024, 8193, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    if kind == "uniform8192_32768":
        return torch.randint(8192, 32769, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    if kind == "uniform2048_8192":
        return torch.randint(2048, 8193, (batch,), generator=gen, dtype=torch.int64).to(torch.int32)
    if kind == "lognormal":
        z = torch.randn((batch,), generator=gen, dtype=torch.float64)
        lens = torch.round(torch.exp(7.5 + 1.0 * z)).clamp(1, 32768)
        return lens.to(torch.int32)
    if kind == "alt16k_64k":
        return torch.tensor([16384 if b % 2 == 0 else 65536 for b in range(batch)],
                            dtype=torch.int32)
    raise ValueError(f"unknown seqlen kind {kind}")


def blocks_for(seqlen: int) -> int:
    """Number of 64-token pages a request of ``seqlen`` tokens occupies."""
    return (int(seqlen) + BLOCK_SIZE - 1) // BLOCK_SIZE


@dataclass
class DecodeInputs:
    q: torch.Tensor            # bf16 [B, s_q, h_q, 576]
    kcache: torch.Tensor       # bf16 [num_blocks, 64, 1, 576]  (last block = NaN sentinel)
    block_table: torch.Tensor  # int32 [B, bt_stride]
    seqlens: torch.Tensor      # int32 [B]
    scale: float
    causal: bool
    s_q: int
    h_q: int
    kv_format: str = "bf16"    # "bf16": kcache as above; "fp8": uint8 [num_blocks, 41216]
    indices: torch.Tensor | None = None   # sparse mode: int32 [B, s_q, topk], -1 = padding

    @property
    def batch(self) -> int:
        return int(self.seqlens.shape[0])

    def to(self, device) -> "DecodeInputs":
        return DecodeInputs(self.q.to(device), self.kcache.to(device),
                            self.block_table.to(device), self.seqlens.to(device),
                            self.scale, self.causal, self.s_q, self.h_q, self.kv_format,
                            None if self.indices is None else self.indices.to(device))


def build_inputs(seqlens, s_q: int, h_q: int, seed: int, pool: int | None = None,
                 extra_pool: int = 64, nan_tails: bool = True,
                 q_scale: float = 1.0, gen: torch.Generator | None = None) -> DecodeInputs:
    """Paged-cache inputs for explicit per-request lengths.

    ``pool`` defaults to (total pages + extra_pool).  Draw order: permutation,
    Q, KV pool (the seqlens are given).
    """
    seqlens = torch.as_tensor(seqlens, dtype=torch.int32).reshape(-1)
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    batch = int(seqlens.shape[0])
    nblk = [blocks_for(int(x)) for x in seqlens]
    total = sum(nblk)
    if pool is None:
        pool = total + extra_pool
    if pool < total:
        raise ValueError(f"pool {pool} smaller than the {total} pages needed")
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    bt_stride = max(1, max(nblk) if nblk else 1)
    sentinel = pool
    block_table = torch.full((batch, bt_stride), sentinel, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        block_table[b, :n] = perm[pos:pos + n]
        pos += n
    q = torch.randn((batch, s_q, h_q, D_K), generator=gen, dtype=torch.float32)
    if q_scale != 1.0:
        q = q * q_scale
    q = q.to(torch.bfloat16)
    kv = torch.empty((pool + 1, BLOCK_SIZE, 1, D_K), dtype=torch.bfloat16)
    # Draw the pool in slabs to bound the fp32 temporary.
    slab = 1024
    for s in range(0, pool, slab):
        e = min(pool, s + slab)
        kv[s:e] = torch.randn((e - s, BLOCK_SIZE, 1, D_K), generator=gen,
                              dtype=torch.float32).to(torch.bfloat16)
    kv[pool] = float("nan")
    if nan_tails:
        for b, n in enumerate(nblk):
            L = int(seqlens[b])
            tail = n * BLOCK_SIZE - L
            if n > 0 and tail > 0:
                kv[int(block_table[b, n - 1]), BLOCK_SIZE - tail:] = float("nan")
    return DecodeInputs(q=q, kcache=kv, block_table=block_table, seqlens=seqlens,
                        scale=D_K ** -0.5, causal=s_q > 1, s_q=s_q, h_q=h_q)


# FP8 cache page: codes uint8 [64][512] | rope bf16 [64][64] | scale fp32 [64]
FP8_LATENT = 512
FP8_CODES_OFF = 0
FP8_ROPE_OFF = BLOCK_SIZE * FP8_LATENT                        # 32768
FP8_SCALE_OFF = FP8_ROPE_OFF + BLOCK_SIZE * (D_K - FP8_LATENT) * 2   # 40960
FP8_PAGE_BYTES = FP8_SCALE_OFF + BLOCK_SIZE * 4               # 41216
FP8_NAN_CODE = 0x7F


def build_fp8_inputs(seqlens, s_q: int, h_q: int, seed: int, pool: int | None = None,
                     extra_pool: int = 64, nan_tails: bool = True,
                     q_scale: float = 1.0, gen: torch.Generator | None = None) -> DecodeInputs:
    """Paged FP8-cache inputs for explicit per-request lengths.

    Draw order: permutation, Q (as in ``build_inputs``), then per page slab:
    latent z ~ N(0,1) fp32 [64, 512] per page, per-token scale exponents
    e ~ U{-7,-6,-5}, rope ~ N(0,1) fp32 [64, 64].  Codes are torch's E4M3
    cast of clamp(64*z, -448, 448) and the scale is 2^e, so latent values are
    about N(0, 2^(e+6)) (the spread of quantised N(0,1) rows).  The sentinel
    page and the rows beyond each request's length are NaN in all three
    fields (code 0x7F, NaN rope, NaN scale).
    """
    seqlens = torch.as_tensor(seqlens, dtype=torch.int32).reshape(-1)
    if gen is None:
        gen = torch.Generator().manual_seed(seed)
    batch = int(seqlens.shape[0])
    nblk = [blocks_for(int(x)) for x in seqlens]
    total = sum(nblk)
    if pool is None:
        pool = total + extra_pool
    if pool < total:
        raise ValueError(f"pool {pool} smaller than the {total} pages needed")
    perm = torch.randperm(pool, generator=gen).to(torch.int32)
    bt_stride = max(1, max(nblk) if nblk else 1)
    block_table = torch.full((batch, bt_stride), pool, dtype=torch.int32)
    pos = 0
    for b, n in enumerate(nblk):
        block_table[b, :n] = perm[pos:pos + n]
        pos += n
    q = torch.randn((batch, s_q, h_q, D_K), generator=gen, dtype=torch.float32)
    if q_scale != 1.0:
        q = q * q_scale
    q = q.to(torch.bfloat16)
    kv = torch.empty((pool + 1, FP8_PAGE_BYTES), dtype=torch.uint8)
    slab = 512
    n_rope = D_K - FP8_LATENT
    for s in range(0, pool, slab):
        e = min(pool, s + slab)
        n = e - s
        z = torch.randn((n, BLOCK_SIZE, FP8_LATENT), generator=gen, dtype=torch.float32)
        ex = torch.randint(-7, -4, (n, BLOCK_SIZE), generator=gen, dtype=torch.int64)
        rope = torch.randn((n, BLOCK_SIZE, n_rope), generator=gen, dtype=torch.float32)
        codes = (64.0 * z).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
        kv[s:e, FP8_CODES_OFF:FP8_ROPE_OFF] = codes.reshape(n, -1)
        kv[s:e, FP8_ROPE_OFF:FP8_SCALE_OFF] = \
            rope.to(torch.bfloat16).contiguous().view(torch.uint8).reshape(n, -1)
        scl = torch.pow(2.0, ex.to(torch.float32))
        kv[s:e, FP8_SCALE_OFF:] = scl.contiguous().view(torch.uint8).reshape(n, -1)
    _fp8_nan_rows(kv, pool, 0, BLOCK_SIZE)
    if nan_tails:
        for b, n in enumerate(nblk):
            L = int(seqlens[b])
            tail = n * BLOCK_SIZE - L
            if n > 0 and tail > 0:
                _fp8_nan_rows(kv, int(block_table[b, n - 1]), BLOCK_SIZE - tail, BLOCK_SIZE)
    return DecodeInputs(q=q, kcache=kv, block_table=block_table, seqlens=seqlens,
                        scale=D_K ** -0.5, causal=s_q > 1, s_q=s_q, h_q=h_q,
                        kv_format="fp8")


def _fp8_nan_rows(kv: torch.Tensor, page: int, r0: int, r1: int) -> None:
    """Fill rows [r0, r1) of an FP8 page with NaN in codes, rope and scale."""
    pg = kv[page]
    pg[FP8_CODES_OFF + r0 * FP8_LATENT:FP8_CODES_OFF + r1 * FP8_LATENT] = FP8_NAN_CODE
    n_rope = D_K - FP8_LATENT
    nan_bf = torch.full(((r1 - r0) * n_rope,), float("nan"), dtype=torch.bfloat16)
    pg[FP8_ROPE_OFF + r0 * n_rope * 2:FP8_ROPE_OFF + r1 * n_rope * 2] = nan_bf.view(torch.uint8)
    nan_f = torch.full((r1 - r0,), float("nan"), dtype=torch.float32)
    pg[FP8_SCALE_OFF + 4 * r0:FP8_SCALE_OFF + 4 * r1] = nan_f.view(torch.uint8)


def draw_topk_indices(seqlens, s_q: int, topk: int, causal: bool, gen: torch.Generator,
                      pad_frac: float = 0.0) -> torch.Tensor:
    """Selected positions for the sparse mode, int32 [B, s_q, topk]: for token
    t of request b, `topk` distinct positions drawn uniformly among its
    visible ones (all of them, in random order, when fewer are visible); the
    remaining slots and a fraction `pad_frac` of the list are -1 (padding).
    Only random draws: no selection criterion is applied."""
    seqlens = [int(x) for x in seqlens]
    B = len(seqlens)
    out = torch.full((B, s_q, topk), -1, dtype=torch.int32)
    for b, L in enumerate(seqlens):
        for t in range(s_q):
            vis = max(0, min(L, L - s_q + 1 + t)) if causal else max(0, L)
            n = min(vis, topk)
            if n > 0:
                pick = torch.randperm(vis, generator=gen)[:n].to(torch.int32)
                out[b, t, :n] = pick
            if pad_frac > 0 and n > 0:
                drop = torch.rand((topk,), generator=gen) < pad_frac
                out[b, t][drop] = -1
            perm = torch.randperm(topk, generator=gen)
            out[b, t] = out[b, t][perm]
    return out


def make_inputs(key: str, nan_tails: bool = True, kv_format: str = "bf16") -> DecodeInputs:
    """The seeded inputs of one named workload (see WORKLOADS); kv_format
    "fp8" gives the same lengths, table and Q with an FP8 cache."""
    w = WORKLOADS[key]
    gen = torch.Generator().manual_seed(w.seed)
    seqlens = draw_seqlens(w.seqlen_kind, w.batch, gen)
    total = sum(blocks_for(int(x)) for x in seqlens)
    pool = w.fixed_pool if w.fixed_pool is not None else total + w.extra_pool
    if kv_format == "fp8":
        inp = build_fp8_inputs(seqlens, w.s_q, w.h_q, seed=w.seed, pool=pool,
                               nan_tails=nan_tails, gen=gen)
        if w.topk:
            inp.indices = draw_topk_indices(seqlens, w.s_q, w.topk, inp.causal, gen)
        return inp
    if kv_format != "bf16":
        raise ValueError(f"unknown kv_format {kv_format}")
    inp = build_inputs(seqlens, w.s_q, w.h_q, seed=w.seed, pool=pool,
                       nan_tails=nan_tails, gen=gen)
    if w.topk:
        inp.indices = draw_topk_indices(seqlens, w.s_q, w.topk, inp.causal, gen)
    return inp


# Cache bytes per token: a bf16 row, or an FP8 row (512 codes + 64 bf16 rope
# + one fp32 scale).
KV_BYTES_PER_TOKEN = {"bf16": D_K * 2, "fp8": FP8_LATENT + (D_K - FP8_LATENT) * 2 + 4}


def sparse_counts(indices, seqlens, s_q: int, h_q: int, causal: bool,
                  kv_format: str = "bf16") -> dict:
    """Bytes and flops of the sparse mode: each counted entry's KV row once
    (1152 B, or 644 B for an FP8 row) and its page-table slot (4 B), every
    index read (4 B), Q/O/LSE of every row, the lengths; 2*(576+512) flops per
    (row, counted entry)."""
    seqlens = torch.as_tensor(seqlens).to(torch.int64)
    ix = torch.as_tensor(indices).to(torch.int64)
    B, _, topk = ix.shape
    t = torch.arange(s_q).view(1, s_q)
    L = seqlens.view(B, 1)
    vis = (L - s_q + 1 + t).clamp(min=0) if causal else L.expand(B, s_q)
    vis = torch.minimum(vis, L)
    counted = int(((ix >= 0) & (ix < vis.unsqueeze(-1))).sum())
    M = s_q * h_q
    kv = counted * KV_BYTES_PER_TOKEN[kv_format]
    io = B * M * (D_K * 2 + D_V * 2 + 4)
    meta = counted * 4 + B * s_q * topk * 4 + B * 4
    return {"bytes": kv + io + meta, "kv_bytes": kv, "flops": 2 * (D_K + D_V) * h_q * counted,
            "counted": counted}


def algorithmic_counts(seqlens, s_q: int, h_q: int, kv_format: str = "bf16") -> dict:
    """Bytes and flops the method must move/compute (no padding, no partials).

    bytes = sum_b L_b*T (each KV row once per request; T = 1152 bytes per
            token for bf16 rows, 644 for FP8 rows)
            + B*M*(576*2 + 512*2 + 4) (Q in, O and LSE out)
            + sum_b ceil(L_b/64)*4 (block table) + B*4 (seqlens)
    flops = 2*(576+512) per visible (query row, key) pair; with s_q query
            tokens under the causal rule token t sees L-s_q+1+t keys.
    """
    seqlens = [int(x) for x in seqlens]
    M = s_q * h_q
    kv = sum(L * KV_BYTES_PER_TOKEN[kv_format] for L in seqlens)
    io = len(seqlens) * M * (D_K * 2 + D_V * 2 + 4)
    meta = sum(blocks_for(L) * 4 for L in seqlens) + len(seqlens) * 4
    pairs = 0
    for L in seqlens:
        for t in range(s_q):
            pairs += h_q * max(0, L - s_q + 1 + t)
    return {"bytes": kv + io + meta, "kv_bytes": kv, "flops": 2 * (D_K + D_V) * pairs}
