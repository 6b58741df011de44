"""The C-ABI library loads on the CPU, exports every declared symbol, and
rejects bad arguments on the host before any HIP call.  No kernel is launched:
every call below fails validation (or is a pure query)."""
import ctypes
import os
import re
import subprocess

import pytest

import rank_latent_attention_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsvd.h")

pytestmark = pytest.mark.skipif(not os.path.exists(q.library_path),
                                reason="libqsvd.so not built (run __graft_entry__.build())")

FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qsvd_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 10
    L = q.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", q.library_path], capture_output=True,
                         text=True).stdout
    exported = set(re.findall(r"\bT (qsvd_\w+)", out))
    assert set(names) <= exported
    assert set(q.EXPORTED) == set(names)


def test_status_strings():
    assert q.qsvd_status_string(0) == "QSVD_OK"
    for s in (-1, -2, -3, -4):
        assert q.qsvd_status_string(s).startswith("QSVD_ERR")


def st_quant(**kw):
    a = dict(inp=FAKE, in_dtype=q.F32, M=4, n=256, had=128, code=q.I8, group=0, codes=FAKE,
             scales=FAKE)
    a.update(kw)
    return q.lib().qsvd_quantize_latent(a["inp"], a["in_dtype"], a["M"], a["n"], a["had"],
                                        a["code"], a["group"], a["codes"], a["scales"], None)


def test_quantize_validation():
    assert st_quant(in_dtype=q.I8) == -1
    assert st_quant(code=q.BF16) == -1
    assert st_quant(had=64) == -2
    assert st_quant(group=64) == -2
    assert st_quant(n=100, had=0) == -1          # n % 8
    assert st_quant(n=264, had=128) == -1        # n % 128 with rotation
    assert st_quant(n=264, had=0, group=128) == -1
    assert st_quant(n=16384) == -1               # > 8192
    assert st_quant(M=-1) == -1
    assert st_quant(inp=None) == -1
    assert st_quant(codes=ctypes.c_void_p((1 << 20) + 8)) == -1   # misaligned
    assert "misaligned" in q.qsvd_last_error()
    assert st_quant(M=0, inp=None) == 0          # empty: no-op, no launch


def st_proj(**kw):
    a = dict(X=FAKE, xdt=q.I8, xs=FAKE, M=16, E=256, W=FAKE, wdt=q.I8, cs=None, r=64, C=FAKE,
             cdt=q.F32)
    a.update(kw)
    return q.lib().qsvd_project(a["X"], a["xdt"], a["xs"], a["M"], a["E"], a["W"], a["wdt"],
                                a["cs"], a["r"], a["C"], a["cdt"], None)


def test_project_validation():
    assert st_proj(xdt=q.F32, wdt=q.F32) == -2
    assert st_proj(wdt=q.BF16) == -2
    assert st_proj(cdt=q.I8) == -1
    assert st_proj(E=100) == -1
    assert st_proj(r=40) == -1
    assert st_proj(xs=None) == -1                # int8 needs per-token scales
    assert st_proj(xdt=q.BF16, wdt=q.BF16) == -1  # bf16 takes no x_scale
    assert st_proj(M=-5) == -1
    assert st_proj(C=None) == -1
    assert st_proj(M=0, X=None) == 0


def st_dec(**kw):
    a = dict(q_=FAKE, qdt=q.BF16, C=FAKE, cdt=q.BF16, cs=None, cg=0, Wk=FAKE, Wv=FAKE,
             wdt=q.BF16, wsk=None, wsv=None, b=2, L=100, r=256, heads=4, d=64, scale=0.125,
             splits=0, O=FAKE, odt=q.BF16, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return q.lib().qsvd_decode_attn(a["q_"], a["qdt"], a["C"], a["cdt"], a["cs"], a["cg"], a["Wk"],
                                    a["Wv"], a["wdt"], a["wsk"], a["wsv"], a["b"], a["L"], a["r"],
                                    a["heads"], a["d"], a["scale"], a["splits"], a["O"], a["odt"],
                                    a["ws"], a["wsb"], None)


def test_decode_validation():
    assert st_dec(b=0) == -1
    assert st_dec(b=65536) == -1                  # the batch fills a grid dimension
    assert st_dec(L=0) == -1
    assert st_dec(d=48) == -2
    for d in (16, 32, 256):                       # the boundary takes d in {64, 128}
        assert st_dec(d=d, heads=256 // d * 4 if d < 64 else 1, r=256) == -2, d
    assert st_dec(cdt=q.F32, qdt=q.F32, wdt=q.F32, odt=q.F32, d=32, heads=8) == -2
    assert st_dec(r=100) == -1                    # bf16 cache needs r % 32
    assert st_dec(r=4096) == -2                   # beyond the per-wavefront budget
    assert st_dec(cdt=q.I4, cs=FAKE, cg=128, r=96) == -1   # int4 needs r % 128
    assert st_dec(cdt=q.I4, cs=FAKE, cg=0) == -2
    assert st_dec(cdt=q.I4, cs=None, cg=128) == -1
    assert st_dec(cdt=q.I8, cs=FAKE, cg=128) == -2
    assert st_dec(cs=FAKE) == -1                  # bf16 cache takes no scales
    assert st_dec(qdt=q.F32) == -2
    assert st_dec(wdt=q.F32) == -2
    assert st_dec(wdt=q.I8) == -1                 # int8 W^u needs column scales
    assert st_dec(wsk=FAKE, wsv=FAKE) == -1       # bf16 W^u takes none
    odd = ctypes.c_void_p((1 << 20) + 4)          # 4-byte but not 16-byte aligned
    assert st_dec(wdt=q.I8, wsk=odd, wsv=FAKE) == -1   # W^u scales are read 16 bytes at a time
    assert st_dec(wdt=q.I8, wsk=FAKE, wsv=odd) == -1
    assert "misaligned" in q.qsvd_last_error()
    assert st_dec(cdt=q.F32, qdt=q.F32, wdt=q.F32, odt=q.BF16) == -2
    assert st_dec(scale=0.0) == -1
    assert st_dec(scale=float("nan")) == -1
    assert st_dec(splits=-1) == -1
    assert st_dec(O=None) == -1
    assert st_dec(ws=ctypes.c_void_p((1 << 20) + 4)) == -1
    need = q.qsvd_decode_workspace_bytes(2, 100, 256, 4, 64, q.BF16)
    assert need > 0
    assert st_dec(wsb=need - 1) == -3
    assert st_dec(ws=None) == -3
    assert "workspace" in q.qsvd_last_error()


def test_workspace_and_splits_plan():
    # the default split count fills the 256 compute units once
    assert q.qsvd_decode_default_splits(16, 8192, 1536, 32, 128, q.BF16) * 16 <= 256
    assert q.qsvd_decode_default_splits(8, 16384, 2304, 40, 128, q.BF16) == 10
    assert q.qsvd_decode_default_splits(1, 5, 256, 4, 64, q.BF16) == 1
    w1 = q.qsvd_decode_workspace_bytes(16, 8192, 1536, 32, 128, q.BF16, 1)
    w8 = q.qsvd_decode_workspace_bytes(16, 8192, 1536, 32, 128, q.BF16, 8)
    assert 0 < w1 < w8
    # partial state grows with the split count: heads * r * 2 bytes per split
    assert w8 - w1 >= 7 * 16 * 32 * 1536 * 2
    assert q.qsvd_decode_workspace_bytes(16, 8192, 1536, 32, 100, q.BF16) == 0   # invalid shape
    # explicit split counts are honoured up to one token per split
    assert q.qsvd_decode_workspace_bytes(1, 3, 256, 4, 64, q.BF16, 64) == \
        q.qsvd_decode_workspace_bytes(1, 3, 256, 4, 64, q.BF16, 3)
    # W8A4 shape (int4 cache): one workgroup per CU over 16 sequences
    assert q.qsvd_decode_default_splits(16, 8192, 768, 32, 128, q.I4) == 16
    # 13B shape: the two-pass plan holds the score array S[b][heads][L] (float32) and the
    # value pass's partials, and ignores an explicit split count
    w13 = q.qsvd_decode_workspace_bytes(8, 16384, 2304, 40, 128, q.BF16)
    assert w13 >= 8 * 40 * 16384 * 4 + 8 * 10 * 40 * 2304 * 2
    assert q.qsvd_decode_workspace_bytes(8, 16384, 2304, 40, 128, q.BF16, 3) == w13
    # per-head latents: the default is 4 splits at the 7B attention shape (512 workgroups)
    hw = q.qsvd_decode_headwise_workspace_bytes
    assert hw(16, 8192, 32, 128, 64, 64, 0) == hw(16, 8192, 32, 128, 64, 64, 4) > 0
    assert hw(16, 8192, 32, 128, 64, 64, 8) > hw(16, 8192, 32, 128, 64, 64, 4)


def test_timing_session_errors():
    L = q.lib()
    n = ctypes.c_int32(0)
    assert L.qsvd_timing_end(None, 0, ctypes.byref(n)) == -1
    assert L.qsvd_timing_begin(0) == -1


def st_exp(**kw):
    a = dict(q_=FAKE, qdt=q.BF16, C=FAKE, cdt=q.BF16, Wk=FAKE, Wv=FAKE, wdt=q.BF16, b=2, L=300,
             r=256, heads=4, d=128, scale=0.088, rc=None, rs=None, O=FAKE, odt=q.BF16, ws=FAKE,
             wsb=1 << 30)
    a.update(kw)
    return q.lib().qsvd_decode_attn_explicit(a["q_"], a["qdt"], a["C"], a["cdt"], a["Wk"], a["Wv"],
                                             a["wdt"], a["b"], a["L"], a["r"], a["heads"], a["d"],
                                             a["scale"], a["rc"], a["rs"], a["O"], a["odt"], a["ws"],
                                             a["wsb"], None)


def test_decode_explicit_validation():
    assert st_exp(b=0) == -1
    assert st_exp(L=0) == -1
    assert st_exp(d=64) == -2
    assert st_exp(r=96) == -1                     # r % 64
    assert st_exp(cdt=q.I8) == -2
    assert st_exp(wdt=q.I8) == -2
    assert st_exp(odt=q.I8) == -1
    assert st_exp(rc=FAKE) == -1                  # the two tables go together
    assert st_exp(scale=-1.0) == -1
    # more workgroups than one launch holds: rejected before any launch
    assert st_exp(b=1024, L=1 << 26, heads=256) == -1
    assert st_exp(Wv=None) == -1
    assert st_exp(rc=ctypes.c_void_p((1 << 20) + 4), rs=FAKE) == -1
    need = q.qsvd_decode_explicit_workspace_bytes(2, 300, 256, 4, 128)
    # per (sequence, 256-token tile, head): 132 float32
    assert need == 2 * 2 * 4 * 132 * 4
    assert st_exp(wsb=need - 1) == -3
    assert q.qsvd_decode_explicit_workspace_bytes(2, 300, 256, 4, 64) == 0


def st_hw(**kw):
    a = dict(q_=FAKE, qdt=q.BF16, C=FAKE, cdt=q.BF16, BK=FAKE, BV=FAKE, bdt=q.BF16, b=2, L=300,
             heads=6, d=128, rk=64, rv=32, scale=0.088, rc=None, rs=None, splits=0, O=FAKE,
             odt=q.BF16, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return q.lib().qsvd_decode_attn_headwise(a["q_"], a["qdt"], a["C"], a["cdt"], a["BK"], a["BV"],
                                             a["bdt"], a["b"], a["L"], a["heads"], a["d"], a["rk"],
                                             a["rv"], a["scale"], a["rc"], a["rs"], a["splits"],
                                             a["O"], a["odt"], a["ws"], a["wsb"], None)


def test_decode_headwise_validation():
    assert st_hw(b=0) == -1
    assert st_hw(L=0) == -1
    assert st_hw(heads=0) == -1
    assert st_hw(heads=257) == -1
    assert st_hw(d=64) == -2
    for rk, rv in ((16, 64), (48, 64), (160, 64), (64, 0), (64, 100)):
        assert st_hw(rk=rk, rv=rv) == -2, (rk, rv)
    assert st_hw(cdt=q.I8) == -2
    assert st_hw(bdt=q.F32) == -2
    assert st_hw(odt=q.I4) == -1
    assert st_hw(rs=FAKE) == -1                   # the two tables go together
    assert st_hw(scale=0.0) == -1
    assert st_hw(splits=-1) == -1
    assert st_hw(splits=1025) == -1
    assert st_hw(BK=None) == -1
    assert st_hw(O=ctypes.c_void_p((1 << 20) + 8)) == -1
    # default splits: 2 x 256 / (b x ceil(heads / 4)) = 128, clipped to the 10 tiles of L = 300
    need = q.qsvd_decode_headwise_workspace_bytes(2, 300, 6, 128, 64, 32, 0)
    assert need == 2 * 10 * 6 * (32 + 4) * 4
    assert q.qsvd_decode_headwise_workspace_bytes(2, 300, 6, 128, 64, 32, 3) == 2 * 3 * 6 * 36 * 4
    assert q.qsvd_decode_headwise_workspace_bytes(2, 300, 6, 64, 64, 32, 0) == 0
    assert st_hw(wsb=need - 1) == -3
    assert st_hw(ws=None) == -3


def test_latent_width_rule_matches_the_header():
    """The header's rule for the latent widths the MFMA paths accept: W the
    largest of 8..1 with r % (W g) == 0 (g = 32 / 64 / 128 columns for bf16 /
    int8 / int4 caches) and at most 384 columns per wavefront."""
    def accepted(r, g):
        for W in range(8, 0, -1):
            if r % (W * g) == 0:
                return r // W <= 384
        return False
    for r in range(32, 4097, 32):
        for dt, g in ((q.BF16, 32), (q.I8, 64), (q.I4, 128)):
            ok = q.qsvd_decode_workspace_bytes(2, 100, r, 8, 128, dt, 0) > 0
            assert ok == accepted(r, g), (r, dt)


def test_last_error_is_per_thread():
    """qsvd_last_error() is thread-local: threads that fail validation at the
    same time each read back their own message (ctypes drops the GIL around
    the calls, so they run concurrently in the library)."""
    import threading
    n, reps = 8, 200
    start = threading.Barrier(n)
    bad = []

    def worker(i):
        start.wait()
        for _ in range(reps):
            if st_dec(heads=300 + i) != -1:
                bad.append((i, "status"))
                return
            msg = q.qsvd_last_error()
            if f"heads = {300 + i}" not in msg:
                bad.append((i, msg))
                return

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(n)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not bad, bad[:3]
