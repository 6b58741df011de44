"""Guard bands around the decode workspace and output.

Every decode entry point receives a workspace and an output carved out of
one larger device buffer whose bytes outside the two regions hold a canary
pattern.  After each call the canaries must be intact (no write outside the
workspace size the library asked for, none outside O) and every element of
O must have been written (O starts as all-NaN bf16 / float32 bit patterns).
The calls run the single-pass stream (bf16, int8, int4 caches), the float32
path, the two-pass path for wide latents, the explicit rebuild and the
per-head latent path, on ragged shapes.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, say

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024      # canary bytes on each side (a multiple of 256)
CANARY = 0xA5


def _carve(nbytes):
    """A device buffer [GUARD | nbytes rounded up to 256 | GUARD] of canaries;
    returns (buffer, region view of nbytes)."""
    import torch
    n = (max(int(nbytes), 1) + 255) // 256 * 256
    buf = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + int(nbytes)]


def _check_guards(buf, nbytes, what):
    import torch
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    lo, hi = h[:GUARD], h[GUARD + int(nbytes):]
    bad_lo = np.flatnonzero(lo != CANARY)
    bad_hi = np.flatnonzero(hi != CANARY)
    assert bad_lo.size == 0, f"{what}: {bad_lo.size} bytes written before the region (first at -{GUARD - bad_lo[0]})"
    assert bad_hi.size == 0, f"{what}: {bad_hi.size} bytes written past the region (first at +{bad_hi[0]})"


def _output(b, heads, d, o_dtype):
    import torch
    esz = 4 if o_dtype == q.F32 else 2
    nbytes = b * heads * d * esz
    buf, reg = _carve(nbytes)
    reg.fill_(0xFF)        # NaN in both float32 and bf16
    tdt = torch.float32 if o_dtype == q.F32 else torch.bfloat16
    return buf, nbytes, reg.view(tdt).view(b, heads, d)


def _finish(wbuf, wbytes, obuf, obytes, O, what):
    _check_guards(wbuf, wbytes, f"{what} workspace")
    _check_guards(obuf, obytes, f"{what} output")
    got = O.float().cpu().numpy()
    assert np.all(np.isfinite(got)), f"{what}: {np.count_nonzero(~np.isfinite(got))} outputs not written"
    return got


SHARED = [
    # label, c_dtype, E, heads, d, r, b, L, splits
    ("f32", q.F32, 256, 4, 64, 96, 2, 77, 0),
    ("f32-many-splits", q.F32, 256, 4, 64, 96, 1, 300, 1000),
    ("bf16", q.BF16, 1024, 8, 128, 768, 3, 301, 0),
    ("bf16-7b", q.BF16, 4096, 32, 128, 1536, 2, 333, 0),
    ("bf16-splits", q.BF16, 1024, 16, 64, 512, 1, 1000, 7),
    ("int8", q.I8, 2048, 16, 128, 512, 2, 333, 0),
    ("int4", q.I4, 4096, 32, 128, 768, 2, 1000, 0),
    ("int4-splits", q.I4, 512, 4, 128, 128, 1, 5, 3),
    ("two-pass", q.BF16, 5120, 40, 128, 2304, 2, 500, 0),
    ("bf16-five-waves", q.BF16, 1024, 8, 128, 160, 2, 70, 0),
    ("bf16-one-wave", q.BF16, 1024, 8, 128, 352, 2, 70, 0),
    ("bf16-r3072", q.BF16, 4096, 32, 128, 3072, 1, 150, 0),
    ("int4-r3072", q.I4, 2048, 16, 128, 3072, 1, 150, 0),
]


@pytest.mark.parametrize("case", SHARED, ids=lambda c: c[0])
def test_decode_guard_bands(case):
    label, cdt, E, heads, d, r, b, L, splits = case
    say(f"case: guard bands, {label}: E={E} heads={heads} d={d} r={r} b={b} L={L} splits={splits}")
    g = np.random.default_rng(len(label) + L)
    if cdt in (q.F32, q.BF16):
        cs = synth.decode_case(E, heads, d, r, b, L, dtype="f32" if cdt == q.F32 else "bf16",
                               hadamard=128 if r % 128 == 0 else 0, seed=L)
        qv, C, Wk, Wv = dev(cs.q), dev(cs.C), dev(cs.Wu_k), dev(cs.Wu_v)
        qdt = wdt = cdt
        cscale, cgroup, wsk, wsv = None, 0, None, None
        ref = oracle.attend_explicit(*(oracle.bf16_decode(a) if cdt == q.BF16 else a
                                       for a in (cs.q, cs.C, cs.Wu_k, cs.Wu_v)),
                                     heads, d, cs.softmax_scale)
    else:
        bits = 4 if cdt == q.I4 else 8
        qmax = 7 if bits == 4 else 127
        codes = g.integers(-qmax, qmax + 1, size=(b, L, r)).astype(np.int8)
        scales = ((g.random((b, L, r // 128)) if bits == 4 else g.random((b, L))) * 0.05 + 0.01).astype(np.float32)
        Wk_q, Wk_s = synth.int8_columns(g.standard_normal((r, E)) / math.sqrt(r))
        Wv_q, Wv_s = synth.int8_columns(g.standard_normal((r, E)) / math.sqrt(r))
        qb = synth.to_bf16_bits(g.standard_normal((b, heads, d)))
        qv, Wk, Wv = dev(qb), dev(Wk_q), dev(Wv_q)
        C = dev(oracle.pack_int4(codes)) if bits == 4 else dev(codes)
        qdt, wdt = q.BF16, q.I8
        cscale, cgroup, wsk, wsv = dev(scales), (128 if bits == 4 else 0), dev(Wk_s), dev(Wv_s)
        ref = oracle.attend_explicit(oracle.bf16_decode(qb), oracle.dequant_rows(codes, scales, cgroup),
                                     oracle.dequant_cols(Wk_q, Wk_s), oracle.dequant_cols(Wv_q, Wv_s),
                                     heads, d, 1 / math.sqrt(d))
    scale = 1 / math.sqrt(d)
    odt = q.F32 if cdt == q.F32 else q.BF16
    need = q.qsvd_decode_workspace_bytes(b, L, r, heads, d, cdt, splits)
    assert need > 0
    for call in range(2):           # the second call reuses the dirtied workspace
        wbuf, ws = _carve(need)
        obuf, obytes, O = _output(b, heads, d, odt)
        q.qsvd_decode_attn(qv, qdt, C, cdt, cscale, cgroup, Wk, Wv, wdt, wsk, wsv, b, L, r, heads, d,
                           scale, splits, O, odt, ws, workspace_bytes=need)
        got = _finish(wbuf, need, obuf, obytes, O, label)
        err = oracle.rel_l2(got, ref)
        say(f"  call {call}: guards intact, rel-L2 {err:.2e}")
        assert err <= (1e-5 if cdt == q.F32 else 2e-2)


@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_explicit_guard_bands(rope):
    b, L, heads, r, d = 2, 333, 8, 512, 128
    say(f"case: guard bands, explicit rope={rope}")
    cs = synth.decode_case(heads * d, heads, d, r, b, L, dtype="bf16", hadamard=128, seed=17)
    rc = rs = None
    if rope:
        c, s = synth.rope_tables(L, d, 10000.0)
        rc, rs = dev(c), dev(s)
    need = q.qsvd_decode_explicit_workspace_bytes(b, L, r, heads, d)
    wbuf, ws = _carve(need)
    obuf, obytes, O = _output(b, heads, d, q.BF16)
    q.qsvd_decode_attn_explicit(dev(cs.q), q.BF16, dev(cs.C), q.BF16, dev(np.ascontiguousarray(cs.Wu_k.T)),
                                dev(np.ascontiguousarray(cs.Wu_v.T)), q.BF16, b, L, r, heads, d,
                                cs.softmax_scale, rc, rs, O, q.BF16, ws, workspace_bytes=need)
    _finish(wbuf, need, obuf, obytes, O, "explicit")


@pytest.mark.parametrize("splits", [0, 5])
def test_headwise_guard_bands(splits):
    b, L, heads, rk, rv = 2, 301, 6, 64, 32
    say(f"case: guard bands, headwise splits={splits}")
    cs = synth.headwise_case(b, L, heads, 128, rk, rv, seed=7)
    c, s = synth.rope_tables(L, 128, 10000.0)
    need = q.qsvd_decode_headwise_workspace_bytes(b, L, heads, 128, rk, rv, splits)
    wbuf, ws = _carve(need)
    obuf, obytes, O = _output(b, heads, 128, q.BF16)
    q.qsvd_decode_attn_headwise(dev(cs.q), q.BF16, dev(cs.C), q.BF16, dev(cs.BK_t), dev(cs.BV), q.BF16,
                                b, L, heads, 128, rk, rv, cs.softmax_scale, dev(c), dev(s), splits, O,
                                q.BF16, ws, workspace_bytes=need)
    _finish(wbuf, need, obuf, obytes, O, "headwise")
