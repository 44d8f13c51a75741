"""fp64 CPU oracle of the FP8 paged KV cache variant of MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP library.

Source.  The page "云上玩转DeepSeek系列之五：实测优化16%，体验FlashMLA加速
DeepSeek-V2-Lite推理" (ruibaoantu.com), section 四 (best practices), item 2
(monitoring and tuning), names FP8 precision as a further throughput step; the
pages give no storage format.  The format below is this project's reading:
the plainest FP8 cache that keeps the attention of the bf16 path unchanged
except for how the 512 latent dims are stored.

Cache page (64 tokens, FP8_PAGE_BYTES = 41216 bytes, one uint8 row per page):

    [0, 32768)      codes  uint8 [64][512]  OCP 8-bit floating point E4M3
                                            codes of latent dims 0..511
    [32768, 40960)  rope   bf16  [64][64]   dims 512..575, kept in bf16
    [40960, 41216)  scale  fp32  [64]       per token; latent value of dim d
                                            is e4m3(code_d) * scale

E4M3 ("OCP FP8 E4M3", the OFP8 formats specification): sign bit 7, 4 exponent
bits (bias 7), 3 mantissa bits; exponent field 0 encodes subnormals
(m/8 * 2^-6); S.1111.111 is NaN; there are no infinities; the largest finite
magnitude is 448.

Quantiser (the write of one bf16 key row x[576], ``quantize_row``):
    amax  = max_d<512 |x_d|
    scale = the smallest power of two with amax <= 448 * scale  (1 if amax = 0)
    code_d = E4M3 round-to-nearest-even of x_d / scale   (the division by a
             power of two is exact and |x_d / scale| <= 448, so nothing
             saturates)
A power-of-two scale makes every decision exact and reproducible; the decoder
accepts any finite scale.

The attention itself is the definition of ``mla_decode_oracle.decode`` (see
there) applied to the dequantized keys: K[j, :512] = e4m3(code) * scale and
K[j, 512:] = rope, both exact in fp64.
"""
from __future__ import annotations

import math

import numpy as np

from .mla_decode_oracle import BLOCK_SIZE, D_K, D_V, _i64, attend_rows, counted_view, \
    mapped_keys, num_pages, visible_count

FP8_LATENT = 512
FP8_ROPE = D_K - FP8_LATENT                      # 64
FP8_CODES_OFF = 0
FP8_ROPE_OFF = BLOCK_SIZE * FP8_LATENT           # 32768
FP8_SCALE_OFF = FP8_ROPE_OFF + BLOCK_SIZE * FP8_ROPE * 2   # 40960
FP8_PAGE_BYTES = FP8_SCALE_OFF + BLOCK_SIZE * 4  # 41216
E4M3_MAX = 448.0


def _u8(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().cpu().contiguous().view(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.uint8)


# ---------------------------------------------------------------- E4M3 codes
def e4m3_decode(code: int) -> float:
    """Value of one E4M3 code, from the field definitions (NaN for S.1111.111)."""
    code = int(code) & 0xFF
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return s * math.ldexp(m / 8.0, -6)
    return s * math.ldexp(1.0 + m / 8.0, e - 7)


E4M3_TABLE = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(y: float) -> int:
    """E4M3 code of the nearest value to y, ties to even mantissa.

    Requires |y| <= 448 (the quantiser guarantees it).  The sign of y (also of
    -0.0 and of negative values that round to zero) is kept in bit 7.
    """
    y = float(y)
    if not abs(y) <= E4M3_MAX:
        raise ValueError(f"{y} outside the finite E4M3 range")
    sign = 0x80 if math.copysign(1.0, y) < 0 else 0
    a = abs(y)
    if a < math.ldexp(1.0, -6):
        # subnormal grid: multiples of 2^-9; n = 8 is the smallest normal,
        # whose code (exponent 1, mantissa 0) is also 8
        n = round(math.ldexp(a, 9))            # Python round: half to even
        return sign | n
    mant, exp = math.frexp(a)                  # a = mant * 2^exp, mant in [0.5, 1)
    E = exp - 1                                # a in [2^E, 2^(E+1))
    n = round(math.ldexp(a, 3 - E))            # in [8, 16], half to even
    if n == 16:
        E += 1
        n = 8
    return sign | ((E + 7) << 3) | (n - 8)


# ---------------------------------------------------------------- quantiser
def quantize_scale(amax: float) -> float:
    """Smallest power of two s with amax <= 448 * s (1.0 for amax == 0)."""
    if amax == 0.0:
        return 1.0
    _, exp = math.frexp(amax / E4M3_MAX)
    s = math.ldexp(1.0, exp)                   # >= amax/448, < 2*amax/448 (approx.)
    while s / 2.0 * E4M3_MAX >= amax:          # exact comparisons: powers of two
        s /= 2.0
    while s * E4M3_MAX < amax:
        s *= 2.0
    return s


def quantize_row(x) -> tuple[np.ndarray, float, np.ndarray]:
    """(codes uint8[512], scale, rope fp64[64]) of one 576-wide key row."""
    xf = np.asarray(x, dtype=np.float64).reshape(-1)
    lat = xf[:FP8_LATENT]
    amax = float(np.max(np.abs(lat))) if lat.size else 0.0
    s = quantize_scale(amax)
    codes = np.array([e4m3_encode(v / s) for v in lat], dtype=np.uint8)
    return codes, s, xf[FP8_LATENT:].copy()


# ---------------------------------------------------------------- page format
def page_fields(page_bytes: np.ndarray):
    """(codes uint8[64,512], rope fp64[64,64], scale fp64[64]) of one page."""
    pb = np.ascontiguousarray(page_bytes, dtype=np.uint8).reshape(-1)
    codes = pb[FP8_CODES_OFF:FP8_ROPE_OFF].reshape(BLOCK_SIZE, FP8_LATENT)
    rope_bits = pb[FP8_ROPE_OFF:FP8_SCALE_OFF].view("<u2").astype(np.uint32) << 16
    rope = rope_bits.view("<f4").astype(np.float64).reshape(BLOCK_SIZE, FP8_ROPE)
    scale = pb[FP8_SCALE_OFF:FP8_PAGE_BYTES].view("<f4").astype(np.float64)
    return codes, rope, scale


def dequant_page(page_bytes) -> np.ndarray:
    """Key rows of one page in fp64, [64, 576] (exact)."""
    codes, rope, scale = page_fields(_u8(page_bytes))
    K = np.empty((BLOCK_SIZE, D_K), dtype=np.float64)
    K[:, :FP8_LATENT] = E4M3_TABLE[codes] * scale[:, None]
    K[:, FP8_LATENT:] = rope
    return K


def gather_request_kv_fp8(pool, block_table, seqlens, b: int) -> np.ndarray:
    """K_b[j, :] for j < L_b (fp64 [L_b, 576]), paging as in the bf16 path:
    token j is row j % 64 of page block_table[b][j // 64]; positions without
    a page (slot past the row, id outside the pool) come back as zero rows,
    which the attention leaves out."""
    pool8 = _u8(pool).reshape(-1, FP8_PAGE_BYTES)
    bt = _i64(block_table)
    L = int(_i64(seqlens)[b])
    n = num_pages(L)
    if n == 0:
        return np.zeros((0, D_K), dtype=np.float64)
    blocks = []
    for slot in range(n):
        p = int(bt[b, slot]) if slot < bt.shape[1] else -1
        if 0 <= p < pool8.shape[0]:
            blocks.append(dequant_page(pool8[p]))
        else:
            blocks.append(np.zeros((BLOCK_SIZE, D_K), dtype=np.float64))
    return np.concatenate(blocks, axis=0)[:L]


def decode_fp8(q, pool, block_table, seqlens, scale: float, causal: bool, requests=None):
    """fp64 reference of paged MLA decode over an FP8 cache.

    q bf16 [B, s_q, h_q, 576]; pool uint8 [pages, 41216]; other arguments and
    the result as ``mla_decode_oracle.decode`` (rows of requests not listed in
    ``requests`` are NaN).
    """
    from .mla_decode_oracle import _f64
    qf = _f64(q)
    B, s_q, h_q, dk = qf.shape
    sl = _i64(seqlens)
    O = np.full((B, s_q, h_q, D_V), np.nan, dtype=np.float64)
    LSE = np.full((B, s_q, h_q), np.nan, dtype=np.float64)
    reqs = range(B) if requests is None else requests
    for b in reqs:
        L = int(sl[b])
        K = gather_request_kv_fp8(pool, block_table, seqlens, b)
        qrows = qf[b].reshape(s_q * h_q, dk)
        nvis = np.array([visible_count(L, s_q, r // h_q, causal)
                         for r in range(s_q * h_q)], dtype=np.int64)
        n_pool = _u8(pool).reshape(-1, FP8_PAGE_BYTES).shape[0]
        Kc, nvis_c = counted_view(K, mapped_keys(block_table, seqlens, b, n_pool), nvis)
        Ob, lb = attend_rows(qrows, Kc, scale, nvis_c)
        O[b] = Ob.reshape(s_q, h_q, D_V)
        LSE[b] = lb.reshape(s_q, h_q)
    return O, LSE


def kv_append_fp8(pool, block_table, seqlens, new_kv) -> np.ndarray:
    """The FP8 cache after writing each request's s_q new key rows.

    Positions as in ``mla_decode_oracle.kv_append`` (new token t of request b
    is token L_b - s_q + t; positions before 0, table slots beyond the table
    and page ids outside the pool are skipped).  Each written row is
    quantised by ``quantize_row``: its 512 codes, its scale (fp32, a power of
    two) and its 64 rope values (bf16, copied bit for bit).  Returns a new
    uint8 array [pages, 41216]; new_kv is bf16 [B, s_q, 576].
    """
    import torch
    out = np.array(_u8(pool), copy=True).reshape(-1, FP8_PAGE_BYTES)
    bt = _i64(block_table)
    sl = _i64(seqlens)
    nk = new_kv.detach().cpu() if isinstance(new_kv, torch.Tensor) else torch.as_tensor(new_kv)
    nk_bits = nk.contiguous().view(torch.int16).numpy().view("<u2")
    nk64 = nk.to(torch.float64).numpy()
    B, s_q = int(nk.shape[0]), int(nk.shape[1])
    for b in range(B):
        for t in range(s_q):
            pos = int(sl[b]) - s_q + t
            if pos < 0 or pos // BLOCK_SIZE >= bt.shape[1]:
                continue
            page = int(bt[b, pos // BLOCK_SIZE])
            if page < 0 or page >= out.shape[0]:
                continue
            r = pos % BLOCK_SIZE
            codes, s, _ = quantize_row(nk64[b, t])
            pg = out[page]
            pg[FP8_CODES_OFF + r * FP8_LATENT:FP8_CODES_OFF + (r + 1) * FP8_LATENT] = codes
            rope = nk_bits[b, t, FP8_LATENT:].astype("<u2")
            pg[FP8_ROPE_OFF + r * FP8_ROPE * 2:FP8_ROPE_OFF + (r + 1) * FP8_ROPE * 2] = \
                rope.view(np.uint8)
            pg[FP8_SCALE_OFF + 4 * r:FP8_SCALE_OFF + 4 * r + 4] = \
                np.array([s], dtype="<f4").view(np.uint8)
    return out
