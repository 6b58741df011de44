"""GPU parity for latent caches larger than 4 GiB (64-bit offsets in every
kernel that walks the cache: the single-pass and two-pass streams, the int4
stream, the per-head path and the explicit K/V path).

Each case decodes two sequences whose caches are the same periodic sequence
of rows: row t of the cache is base row t mod P, with P dividing L.  Every
base row then appears L / P times, so the softmax over the L cached tokens is
exactly the softmax over the P base rows (the common multiplicity cancels in
the normalisation), and the float64 oracle checks the result on the P base
rows alone.  The second sequence's rows lie past the first 4 GiB of the
cache; with the same query it must give bitwise the output of the first.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import decode, dev, empty, host, say, values, workspace

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu

TOL = 2e-2
GIB4 = 4 << 30


def _periodic(base_dev, reps, b):
    """[b][reps * P][...] cache whose every sequence repeats the P rows of base_dev."""
    import torch
    P = base_dev.shape[0]
    C = torch.empty((b, reps * P) + tuple(base_dev.shape[1:]), dtype=base_dev.dtype, device="cuda")
    for s in range(b):
        C[s].view((reps, P) + tuple(base_dev.shape[1:])).copy_(base_dev.unsqueeze(0).expand(
            (reps, P) + tuple(base_dev.shape[1:])))
    return C


def _free():
    import torch
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _check(O, ref, label):
    got = host(O)
    assert np.all(np.isfinite(got))
    assert np.array_equal(got[0], got[1]), f"{label}: the sequence past 4 GiB differs"
    err = oracle.rel_l2(got[0], ref)
    say(f"  {label}: rel-L2 {err:.2e}, sequences bitwise equal")
    assert err <= TOL


@pytest.mark.parametrize("shape", [
    # E, heads, r, P, reps: single-pass stream; the 13B-like many-head shape takes the two passes
    (1024, 8, 256, 1000, 4500),
    (5120, 40, 1792, 1000, 700),
], ids=["single_pass", "two_pass"])
def test_bf16_cache_over_4gib(shape):
    E, heads, r, P, reps = shape
    d, L = 128, P * reps
    assert 2 * L * r * 2 > GIB4
    say(f"case: bf16 cache over 4 GiB E={E} heads={heads} r={r} L={L} (period {P})")
    cs = synth.decode_case(E, heads, d, r, 1, P, dtype="bf16", hadamard=128, p=0.5, seed=501 + r)
    C = _periodic(dev(cs.C[0]), reps, 2)
    qv = dev(np.stack([cs.q[0], cs.q[0]]))
    O = decode(qv, q.BF16, C, q.BF16, dev(cs.Wu_k), dev(cs.Wu_v), q.BF16, 2, L, r, heads, d,
               cs.softmax_scale, o_dtype=q.F32)
    del C
    ref = oracle.attend_explicit(values(cs.q, "bf16"), values(cs.C, "bf16"), values(cs.Wu_k, "bf16"),
                                 values(cs.Wu_v, "bf16"), heads, d, cs.softmax_scale)[0]
    _check(O, ref, "bf16")
    _free()


def test_int4_cache_over_4gib():
    r, heads, d, P = 768, 32, 128, 1024
    E = heads * d
    reps = 5200
    L = P * reps
    assert 2 * L * (r // 2 + 4 * (r // 128)) > GIB4
    say(f"case: int4 cache over 4 GiB r={r} L={L} (period {P})")
    g = np.random.default_rng(77)
    codes = g.integers(-7, 8, size=(P, r)).astype(np.int8)
    scales = (g.random((P, r // 128)) * 0.05 + 0.01).astype(np.float32)
    Wk_q, Wk_s = synth.int8_columns(g.standard_normal((r, E)) / math.sqrt(r))
    Wv_q, Wv_s = synth.int8_columns(g.standard_normal((r, E)) / math.sqrt(r))
    qv = synth.to_bf16_bits(g.standard_normal((1, heads, d)) * 2.0)
    Cq = _periodic(dev(oracle.pack_int4(codes)), reps, 2)
    Cs = _periodic(dev(scales), reps, 2)
    O = decode(dev(np.concatenate([qv, qv])), q.BF16, Cq, q.I4, dev(Wk_q), dev(Wv_q), q.I8, 2, L, r,
               heads, d, 1 / math.sqrt(d), c_scales=Cs, c_group=128, wsk=dev(Wk_s), wsv=dev(Wv_s),
               o_dtype=q.F32)
    del Cq, Cs
    ref = oracle.attend_explicit(oracle.bf16_decode(qv), oracle.dequant_rows(codes[None], scales[None], 128),
                                 oracle.dequant_cols(Wk_q, Wk_s), oracle.dequant_cols(Wv_q, Wv_s), heads, d,
                                 1 / math.sqrt(d))[0]
    _check(O, ref, "int4")
    _free()


def test_headwise_cache_over_4gib():
    import torch
    heads, d, rk, rv, P, reps = 32, 128, 64, 64, 1000, 300
    L = P * reps
    assert 2 * L * heads * (rk + rv) * 2 > GIB4
    say(f"case: per-head latents over 4 GiB heads={heads} rk=rv={rk} L={L} (period {P})")
    cs = synth.headwise_case(1, P, heads, d, rk, rv, seed=909)
    C = _periodic(dev(cs.C[0]), reps, 2)
    qv = dev(np.concatenate([cs.q, cs.q]))
    BK, BV = dev(cs.BK_t), dev(cs.BV)
    ws = workspace(q.qsvd_decode_headwise_workspace_bytes(2, L, heads, d, rk, rv, 0))
    outs = {}
    for rope in (False, True):
        rc = rs = None
        if rope:
            c, s = synth.rope_tables(L, d)
            rc, rs = dev(c), dev(s)
        O = empty((2, heads, d), torch.float32)
        q.qsvd_decode_attn_headwise(qv, q.BF16, C, q.BF16, BK, BV, q.BF16, 2, L, heads, d, rk, rv,
                                    cs.softmax_scale, rc, rs, 0, O, q.F32, ws)
        torch.cuda.synchronize()
        outs[rope] = O
    del C
    # without rotary positions the periodic cache reduces to its P base rows
    Cb = values(cs.C, "bf16")
    BKo = np.ascontiguousarray(values(cs.BK_t, "bf16").transpose(0, 2, 1))
    ref = oracle.attend_headwise(values(cs.q, "bf16"), Cb[..., :rk], Cb[..., rk:], BKo,
                                 values(cs.BV, "bf16"), cs.softmax_scale, None)[0]
    _check(outs[False], ref, "per-head, no RoPE")
    # with rotary positions the rows are no longer interchangeable; the two
    # sequences (same cache, same positions) must still agree bitwise
    got = host(outs[True])
    assert np.all(np.isfinite(got)) and np.array_equal(got[0], got[1])
    say("  per-head, RoPE: sequences bitwise equal")
    _free()


def test_explicit_cache_over_4gib():
    """The explicit K/V path (no rotary positions) over a periodic cache past 4 GiB."""
    import torch
    E, heads, d, r, P, reps = 1024, 8, 128, 256, 1000, 4500
    L = P * reps
    assert 2 * L * r * 2 > GIB4
    say(f"case: explicit K/V over 4 GiB E={E} heads={heads} r={r} L={L} (period {P})")
    cs = synth.decode_case(E, heads, d, r, 1, P, dtype="bf16", hadamard=128, p=0.5, seed=733)
    C = _periodic(dev(cs.C[0]), reps, 2)
    qv = dev(np.stack([cs.q[0], cs.q[0]]))
    Wk_t = dev(np.ascontiguousarray(cs.Wu_k.T))
    Wv_t = dev(np.ascontiguousarray(cs.Wu_v.T))
    O = empty((2, heads, d), torch.float32)
    ws = workspace(q.qsvd_decode_explicit_workspace_bytes(2, L, r, heads, d))
    q.qsvd_decode_attn_explicit(qv, q.BF16, C, q.BF16, Wk_t, Wv_t, q.BF16, 2, L, r, heads, d,
                                cs.softmax_scale, None, None, O, q.F32, ws)
    torch.cuda.synchronize()
    del C
    ref = oracle.attend_explicit(values(cs.q, "bf16"), values(cs.C, "bf16"), values(cs.Wu_k, "bf16"),
                                 values(cs.Wu_v, "bf16"), heads, d, cs.softmax_scale)[0]
    _check(O, ref, "explicit")
    _free()
