"""The C ABI without a GPU: the library loads, exports every declared entry
point, and the host-only entry points and the argument validation (which
runs before anything is enqueued) behave as documented."""
import ctypes
import os
import re

import pytest

import mla_paged_kv_04_amd as mla
from mla_paged_kv_04_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for n in ("mla_decode_metadata", "mla_decode_fwd", "mla_decode_splitkv",
              "mla_decode_combine", "mla_decode_num_parts", "mla_decode_workspace_bytes",
              "mla_status_string", "mla_last_hip_error", "mla_device_num_cus"):
        assert n in names


def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(binding.LIB_PATH)
    for n in _declared():
        assert hasattr(h, n), n
    assert set(_declared()) <= set(binding._SIGNATURES)


def test_max_s_q_accepted():
    # the largest token count passes validation (fake pointers: a return
    # other than INVALID_ARG for s_q would need a launch, so only check the
    # host-only entry points)
    assert mla.num_parts(1, 128, 128, 1, 256) == 2         # 16384 rows: 128 row tiles of 128
    assert mla.workspace_bytes(1, 128, 16, 1) == 0
    with pytest.raises(Exception):
        mla.num_parts(1, 129, 16, 1, 256)


def test_num_parts():
    assert mla.num_parts(64, 1, 16, 1, 256) == 256
    assert mla.num_parts(128, 1, 128, 1, 256) == 256     # one 128-row tile
    assert mla.num_parts(132, 2, 128, 1, 256) == 128     # two 128-row tiles
    assert mla.num_parts(2, 1, 32, 1, 256) == 256
    assert mla.num_parts(2, 1, 16, 1, 1) == 1
    out = ctypes.c_int(0)
    L = mla.lib()
    assert L.mla_decode_num_parts(2, 1, 48, 1, 256, ctypes.byref(out)) == UNSUPPORTED
    assert L.mla_decode_num_parts(2, 129, 16, 1, 256, ctypes.byref(out)) == INVALID
    assert L.mla_decode_num_parts(2, 0, 16, 1, 256, ctypes.byref(out)) == INVALID
    assert mla.num_parts(2, 3, 16, 1, 256) == 256          # 48 rows: one 64-row tile
    assert mla.num_parts(2, 8, 128, 1, 256) == 32          # 1024 rows: eight 128-row tiles
    assert L.mla_decode_num_parts(2, 1, 16, 2, 256, ctypes.byref(out)) == INVALID
    assert L.mla_decode_num_parts(0, 1, 16, 1, 256, ctypes.byref(out)) == INVALID
    assert L.mla_decode_num_parts(2, 1, 16, 1, 0, ctypes.byref(out)) == INVALID
    assert L.mla_decode_num_parts(2, 1, 16, 1, 256, None) == INVALID


def test_workspace_bytes():
    assert mla.workspace_bytes(4, 1, 16, 1) == 0
    # bf16 O_part[slots][M][512] then fp32 LSE_part[slots][M], slots = 2 (parts - 1)
    b = mla.workspace_bytes(4, 1, 16, 256)
    assert b == -(-(2 * 255 * 16 * (512 * 2 + 4)) // 256) * 256
    assert mla.workspace_bytes(4, 2, 128, 64) >= 2 * 63 * 256 * (512 * 2 + 4)


def test_status_strings():
    for st in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert mla.status_string(st).startswith("MLA_")
    assert mla.status_string(12345) == "unknown status"


def _fwd_raw(fn="mla_decode_fwd", **kw):
    args = dict(q=16, kc=16, nblk=8, bt=16, bt_stride=2, sl=16, batch=2, s_q=1, h_q=16, h_kv=1,
                scale=0.04, causal=0, tm=16, so=16, parts=4, ws=256, ws_bytes=1 << 30,
                out=16, lse=16)
    args.update(kw)
    p = lambda v: ctypes.c_void_p(v) if v else None
    return getattr(mla.lib(), fn)(
        p(args["q"]), p(args["kc"]), args["nblk"], p(args["bt"]), args["bt_stride"], p(args["sl"]),
        args["batch"], args["s_q"], args["h_q"], args["h_kv"], args["scale"], args["causal"],
        p(args["tm"]), p(args["so"]), args["parts"], p(args["ws"]), args["ws_bytes"],
        p(args["out"]), p(args["lse"]), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=0), INVALID), (dict(kc=0), INVALID), (dict(bt=0), INVALID), (dict(sl=0), INVALID),
    (dict(tm=0), INVALID), (dict(so=0), INVALID), (dict(out=0), INVALID), (dict(lse=0), INVALID),
    (dict(q=8), INVALID), (dict(kc=4), INVALID), (dict(out=8), INVALID), (dict(lse=2), INVALID),
    (dict(ws=128), INVALID), (dict(ws=0), INVALID),
    (dict(batch=0), INVALID), (dict(s_q=129), INVALID), (dict(s_q=0), INVALID), (dict(h_kv=2), INVALID),
    (dict(h_q=48), UNSUPPORTED), (dict(h_q=8), UNSUPPORTED),
    (dict(parts=0), INVALID), (dict(nblk=0), INVALID), (dict(bt_stride=0), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(causal=2), INVALID), (dict(ws_bytes=1024), WORKSPACE),
])
@pytest.mark.parametrize("fn", ["mla_decode_fwd", "mla_decode_fwd_fp8"])
def test_fwd_rejects_before_launch(fn, kw, expect):
    # Pointers are fake (never dereferenced): validation returns before any launch.
    assert _fwd_raw(fn, **kw) == expect


def test_metadata_rejects_before_launch():
    L = mla.lib()
    p = ctypes.c_void_p
    assert L.mla_decode_metadata(p(16), 2, 1, 16, 1, 32, 4, p(16), p(16), None) == INVALID
    assert L.mla_decode_metadata(None, 2, 1, 16, 1, 64, 4, p(16), p(16), None) == INVALID
    assert L.mla_decode_metadata(p(16), 2, 1, 16, 1, 64, 0, p(16), p(16), None) == INVALID
    assert L.mla_decode_metadata(p(16), 2, 1, 64, 2, 64, 4, p(16), p(16), None) == INVALID
    assert L.mla_decode_metadata(p(18), 2, 1, 16, 1, 64, 4, p(16), p(16), None) == INVALID


def test_combine_rejects_before_launch():
    L = mla.lib()
    p = ctypes.c_void_p
    assert L.mla_decode_combine(p(16), 2, 1, 16, p(16), 4, p(256), 10, p(16), p(16), None) == WORKSPACE
    assert L.mla_decode_combine(None, 2, 1, 16, p(16), 4, p(256), 1 << 30, p(16), p(16), None) == INVALID


def test_kv_append_rejects_before_launch():
    L = mla.lib()
    p = ctypes.c_void_p
    ok = dict(nkv=p(16), kc=p(16), nblk=8, bt=p(16), bt_stride=2, sl=p(16), batch=2, s_q=1)

    def call(**kw):
        a = dict(ok, **kw)
        return L.mla_kv_append(a["nkv"], a["kc"], a["nblk"], a["bt"], a["bt_stride"], a["sl"],
                               a["batch"], a["s_q"], None)

    for kw in (dict(nkv=None), dict(kc=None), dict(bt=None), dict(sl=None), dict(nkv=p(8)),
               dict(kc=p(24)), dict(bt=p(2)), dict(sl=p(6)), dict(nblk=0), dict(bt_stride=0),
               dict(batch=0), dict(s_q=0), dict(s_q=129)):
        assert call(**kw) == INVALID, kw


def test_fp8_entry_points_reject_before_launch():
    L = mla.lib()
    p = ctypes.c_void_p
    ok = dict(nkv=p(16), kc=p(16), nblk=8, bt=p(16), bt_stride=2, sl=p(16), batch=2, s_q=1)
    for kw in (dict(nkv=None), dict(kc=p(8)), dict(batch=0), dict(s_q=129), dict(nblk=0)):
        a = dict(ok, **kw)
        assert L.mla_kv_append_fp8(a["nkv"], a["kc"], a["nblk"], a["bt"], a["bt_stride"],
                                   a["sl"], a["batch"], a["s_q"], None) == INVALID, kw
    # splitkv_fp8 with NULL events: same validation as the bf16 entry point
    args = [p(16), p(16), 8, p(16), 2, p(16), 2, 1, 16, 1, 0.04, 0, p(16), p(16), 4, p(256),
            1 << 30, p(16), p(16), None, None, None]
    bad = list(args)
    bad[8] = 48
    assert L.mla_decode_splitkv_fp8(*bad) == UNSUPPORTED
    bad = list(args)
    bad[1] = p(8)
    assert L.mla_decode_splitkv_fp8(*bad) == INVALID
    assert binding.FP8_PAGE_BYTES == 41216


@pytest.mark.parametrize("fn", ["mla_decode_sparse_fwd", "mla_decode_sparse_fwd_fp8"])
def test_sparse_entry_points_reject_before_launch(fn):
    """Shape, size and pointer checks of both sparse entry points run on the
    host before anything is enqueued (no GPU needed)."""
    L = mla.lib()
    p = ctypes.c_void_p
    # q, kcache, num_blocks, block_table, bt_stride, seqlens, batch, s_q, h_q, h_kv, scale,
    # causal, indices, topk, tile_meta, split_offsets, num_parts, workspace, bytes, out, lse,
    # start, stop, stream
    ok = [p(16), p(16), 8, p(16), 2, p(16), 2, 1, 16, 1, 0.04, 0, p(16), 64, p(16), p(16), 4,
          p(256), 1 << 30, p(16), p(16), None, None, None]
    f = getattr(L, fn)
    for idx, val, expect in ((13, 48, INVALID),          # topk not a multiple of 32
                             (13, 0, INVALID),
                             (13, (1 << 20) + 32, INVALID),
                             (12, None, INVALID),        # indices
                             (2, 0, INVALID),            # num_blocks
                             (2, (1 << 25) + 1, INVALID),
                             (8, 48, UNSUPPORTED),       # h_q
                             (17, p(128), INVALID),      # workspace alignment
                             (18, 1024, WORKSPACE)):     # workspace too small
        a = list(ok)
        a[idx] = val
        assert f(*a) == expect, (fn, idx, val)


@pytest.mark.parametrize("fn", ["mla_decode_fwd_inline_plan", "mla_decode_fwd_inline_plan_fp8"])
def test_inline_plan_rejects_before_launch(fn):
    """Host-side checks of the in-kernel-plan entry points: batches above
    1024 are unsupported (the three-launch path serves them)."""
    L = mla.lib()
    p = ctypes.c_void_p
    # q, kcache, num_blocks, block_table, bt_stride, seqlens, batch, s_q, h_q, h_kv, scale,
    # causal, tile_meta, split_offsets, num_parts, workspace, bytes, out, lse, start, stop,
    # stream
    ok = [p(16), p(16), 8, p(16), 2, p(16), 2, 1, 16, 1, 0.04, 0, p(16), p(16), 4, p(256),
          1 << 30, p(16), p(16), None, None, None]
    f = getattr(L, fn)
    for idx, val, expect in ((6, 1025, UNSUPPORTED), (6, 0, INVALID), (8, 48, UNSUPPORTED),
                             (2, 0, INVALID), (12, None, INVALID), (13, None, INVALID),
                             (15, p(128), INVALID), (16, 1024, WORKSPACE)):
        a = list(ok)
        a[idx] = val
        assert f(*a) == expect, (fn, idx, val)
