"""The decode entry points inside a captured HIP graph (torch.cuda.graph), and
calls on two streams at once.

The calls allocate nothing and issue no memset or synchronisation, so a
runtime can capture a decode step once and replay it.  Each case captures one
call, then replays it several times with eager work (clearing the output, new
query values copied into the captured input) and a synchronisation between
replays, and checks every replay bitwise against an eager call on the same
inputs.
"""
import pytest

import synth
from gpu_util import dev, empty, say, workspace

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu


def _replays(call, O, qbuf, qs):
    """Eager results for each query in qs, then the captured call replayed with each."""
    import torch
    eager = []
    for qv in qs:
        qbuf.copy_(qv)
        call()
        torch.cuda.synchronize()
        eager.append(O.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        for i, qv in enumerate(qs):
            O.zero_()
            qbuf.copy_(qv)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(O, eager[i]), (rep, i)
    say(f"  {3 * len(qs)} replays bitwise equal to the eager calls")


@pytest.mark.parametrize("shape", [
    # E, heads, r, b, L: single pass; many heads over a wide latent (two passes)
    (1024, 8, 512, 3, 700),
    (5120, 40, 2304, 2, 500),
], ids=["single_pass", "two_pass"])
def test_decode_attn_graph_replay(shape):
    import torch
    E, heads, r, b, L = shape
    d = 128
    say(f"case: qsvd_decode_attn in a graph E={E} heads={heads} r={r} b={b} L={L}")
    cs = synth.decode_case(E, heads, d, r, b, L, dtype="bf16", hadamard=128, seed=61 + r)
    C, Wk, Wv = dev(cs.C), dev(cs.Wu_k), dev(cs.Wu_v)
    qbuf = dev(cs.q).clone()
    qs = [dev(cs.q)]
    qs.append(torch.flip(qs[0], dims=[1]).contiguous())   # other query values: heads reversed
    O = empty((b, heads, d), torch.float32)
    nbytes = q.qsvd_decode_workspace_bytes(b, L, r, heads, d, q.BF16, 0)
    ws = workspace(nbytes)

    def call():
        q.qsvd_decode_attn(qbuf, q.BF16, C, q.BF16, None, 0, Wk, Wv, q.BF16, None, None, b, L, r, heads,
                           d, cs.softmax_scale, 0, O, q.F32, ws)

    _replays(call, O, qbuf, qs)


def test_decode_headwise_graph_replay():
    import torch
    b, L, heads, d, rk, rv = 2, 600, 8, 128, 64, 64
    say(f"case: qsvd_decode_attn_headwise in a graph b={b} L={L} heads={heads} RoPE")
    cs = synth.headwise_case(b, L, heads, d, rk, rv, seed=17)
    C, BK, BV = dev(cs.C), dev(cs.BK_t), dev(cs.BV)
    c, s = synth.rope_tables(L, d)
    rc, rs = dev(c), dev(s)
    qbuf = dev(cs.q).clone()
    qs = [dev(cs.q)]
    qs.append(torch.flip(qs[0], dims=[1]).contiguous())
    O = empty((b, heads, d), torch.float32)
    ws = workspace(q.qsvd_decode_headwise_workspace_bytes(b, L, heads, d, rk, rv, 0))

    def call():
        q.qsvd_decode_attn_headwise(qbuf, q.BF16, C, q.BF16, BK, BV, q.BF16, b, L, heads, d, rk, rv,
                                    cs.softmax_scale, rc, rs, 0, O, q.F32, ws)

    _replays(call, O, qbuf, qs)


def test_concurrent_streams_match_sequential():
    """Two streams (default priority), each with its own inputs, output and workspace, run decode
    steps concurrently; every result equals the same call run alone (the library keeps no
    per-call state outside the caller's buffers)."""
    import torch
    say("case: concurrent decode calls on two streams")
    cs = synth.decode_case(1024, 8, 128, 512, 3, 900, dtype="bf16", hadamard=128, seed=71)
    hc = synth.headwise_case(2, 700, 8, 128, 64, 64, seed=72)
    C, Wk, Wv, qv = dev(cs.C), dev(cs.Wu_k), dev(cs.Wu_v), dev(cs.q)
    Ch, BK, BV, qh = dev(hc.C), dev(hc.BK_t), dev(hc.BV), dev(hc.q)
    O1 = empty((3, 8, 128), torch.float32)
    O2 = empty((2, 8, 128), torch.float32)
    ws1 = workspace(q.qsvd_decode_workspace_bytes(3, 900, 512, 8, 128, q.BF16, 0))
    ws2 = workspace(q.qsvd_decode_headwise_workspace_bytes(2, 700, 8, 128, 64, 64, 0))

    def one():
        q.qsvd_decode_attn(qv, q.BF16, C, q.BF16, None, 0, Wk, Wv, q.BF16, None, None, 3, 900, 512, 8, 128,
                           cs.softmax_scale, 0, O1, q.F32, ws1)

    def two():
        q.qsvd_decode_attn_headwise(qh, q.BF16, Ch, q.BF16, BK, BV, q.BF16, 2, 700, 8, 128, 64, 64,
                                    hc.softmax_scale, None, None, 0, O2, q.F32, ws2)

    one()
    two()
    torch.cuda.synchronize()
    ref1, ref2 = O1.clone(), O2.clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rnd in range(4):
        O1.zero_()
        O2.zero_()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        for _ in range(3):
            with torch.cuda.stream(s1):
                one()
            with torch.cuda.stream(s2):
                two()
        torch.cuda.synchronize()
        assert torch.equal(O1, ref1) and torch.equal(O2, ref2), rnd
    say("  4 rounds of interleaved launches equal the sequential results")


def test_concurrent_host_threads_match_sequential():
    """Four host threads, each with its own stream, output and workspace, issue decode steps of
    different kinds at the same time (bf16 single pass, bf16 two passes, per-head latents, float32
    one launch).  ctypes drops the GIL around the calls, so the library's host side (validation,
    planning, the per-thread launch-attribute records) runs concurrently; every result equals the
    same call made alone."""
    import threading
    import torch
    say("case: concurrent decode calls from four host threads")
    c1 = synth.decode_case(1024, 8, 128, 512, 3, 900, dtype="bf16", hadamard=128, seed=81)
    c2 = synth.decode_case(5120, 40, 128, 2304, 1, 300, dtype="bf16", hadamard=128, seed=82)
    hc = synth.headwise_case(2, 700, 8, 128, 64, 64, seed=83)
    c4 = synth.decode_case(256, 4, 64, 96, 1, 512, dtype="f32", seed=84)
    calls = []

    def add_decode(cs, dt, b, L, r, heads, d):
        C, Wk, Wv, qv = dev(cs.C), dev(cs.Wu_k), dev(cs.Wu_v), dev(cs.q)
        O = empty((b, heads, d), torch.float32)
        ws = workspace(q.qsvd_decode_workspace_bytes(b, L, r, heads, d, dt, 0))
        calls.append((O, lambda s: q.qsvd_decode_attn(qv, dt, C, dt, None, 0, Wk, Wv, dt, None, None, b, L, r,
                                                      heads, d, cs.softmax_scale, 0, O, q.F32, ws,
                                                      stream=s)))

    add_decode(c1, q.BF16, 3, 900, 512, 8, 128)
    add_decode(c2, q.BF16, 1, 300, 2304, 40, 128)
    Ch, BK, BV, qh = dev(hc.C), dev(hc.BK_t), dev(hc.BV), dev(hc.q)
    Oh = empty((2, 8, 128), torch.float32)
    wsh = workspace(q.qsvd_decode_headwise_workspace_bytes(2, 700, 8, 128, 64, 64, 0))
    calls.append((Oh, lambda s: q.qsvd_decode_attn_headwise(qh, q.BF16, Ch, q.BF16, BK, BV, q.BF16, 2, 700, 8,
                                                            128, 64, 64, hc.softmax_scale, None, None, 0, Oh,
                                                            q.F32, wsh, stream=s)))
    add_decode(c4, q.F32, 1, 512, 96, 4, 64)
    refs = []
    for O, call in calls:
        call(None)
        torch.cuda.synchronize()
        refs.append(O.clone())
        O.zero_()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in calls]
    start = threading.Barrier(len(calls))
    errors = []

    def worker(i):
        try:
            start.wait()
            for _ in range(20):
                calls[i][1](streams[i].cuda_stream)
        except Exception as e:   # reported below, on the main thread
            errors.append((i, repr(e)))

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(len(calls))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (O, _) in enumerate(calls):
        assert torch.equal(O, refs[i]), i
    say("  20 calls per thread on four streams equal the sequential results")
