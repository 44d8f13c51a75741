"""Concurrent use of the library on MI355X: the entry points keep no device
state between calls (the caller owns every buffer), so decodes enqueued on
several streams at once, or from several host threads each with its own
stream, give the same bits as the same decodes run one after another.
Streams are created at the default priority.
"""
import threading

import pytest
import torch

from workloads import build_fp8_inputs, build_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_kv_04_amd as m
    m.lib()
    return m


def _cases():
    a = build_inputs([1000, 64, 3000, 1, 700, 4096, 129, 2000], 1, 16, seed=301, extra_pool=4)
    b = build_inputs([500, 2500, 3, 1800], 2, 128, seed=302, extra_pool=4)
    c = build_fp8_inputs([900, 4000, 65, 2100, 0, 1300], 1, 64, seed=303, extra_pool=4)
    return [(a.to("cuda"), a.scale, False), (b.to("cuda"), b.scale, False),
            (c.to("cuda"), c.scale, True)]


def _run(mla, g, scale, fp8):
    fwd = mla.fwd_fp8 if fp8 else mla.fwd
    return fwd(g.q, g.kcache, g.block_table, g.seqlens, scale, g.causal)


def test_concurrent_streams_bitwise(mla):
    print("case concurrent streams", flush=True)
    cases = _cases()
    ref = [_run(mla, *c) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    got = [[] for _ in cases]
    for _ in range(3):                      # interleave the enqueues over the streams
        for i, (c, s) in enumerate(zip(cases, streams)):
            with torch.cuda.stream(s):
                got[i].append(_run(mla, *c))
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for out, lse in got[i]:
            assert torch.equal(out, ref[i][0]), f"case {i}: O differs"
            assert torch.equal(lse, ref[i][1]), f"case {i}: LSE differs"


def test_host_threads_bitwise(mla):
    print("case host threads", flush=True)
    cases = _cases()
    ref = [_run(mla, *c) for c in cases]
    torch.cuda.synchronize()
    results = [None] * len(cases)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.default_stream())
            outs = []
            with torch.cuda.stream(s):
                for _ in range(4):
                    outs.append(_run(mla, *cases[i]))
            s.synchronize()
            results[i] = outs
        except Exception as e:   # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not errors, errors
    assert all(not t.is_alive() for t in threads)
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for out, lse in results[i]:
            assert torch.equal(out, ref[i][0]), f"thread {i}: O differs"
            assert torch.equal(lse, ref[i][1]), f"thread {i}: LSE differs"
