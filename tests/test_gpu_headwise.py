"""GPU parity of qsvd_decode_attn_headwise (per-head latents, keys rebuilt on
chip, optional RoPE) against the float64 oracle attend_headwise.

Inputs are synth.headwise_case bf16 bit patterns; the oracle consumes their
exact values and computes its own RoPE angles in float64, while the kernel
receives the float32 cos / sin tables a runtime would hand it.  Tolerance:
relative L2 over the whole output, and of every (sequence, head) row in the
shape sweep, <= 2e-2 (bf16 inputs, float32 MFMA
accumulation, bf16 output; table rounding adds < 2^-24 relative per angle).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_rows, dev, empty, host, say, values, workspace

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu

TOL = 2e-2


def run_headwise(cs, rope=False, base=10000.0, splits=0, o_dtype=q.BF16):
    import torch
    rc = rs = None
    if rope:
        c, s = synth.rope_tables(cs.L, cs.d, base)
        rc, rs = dev(c), dev(s)
    O = empty((cs.b, cs.heads, cs.d), torch.bfloat16 if o_dtype == q.BF16 else torch.float32)
    nbytes = q.qsvd_decode_headwise_workspace_bytes(cs.b, cs.L, cs.heads, cs.d, cs.rk, cs.rv, splits)
    assert nbytes > 0
    ws = workspace(nbytes)
    q.qsvd_decode_attn_headwise(dev(cs.q), q.BF16, dev(cs.C), q.BF16, dev(cs.BK_t), dev(cs.BV), q.BF16,
                                cs.b, cs.L, cs.heads, cs.d, cs.rk, cs.rv, cs.softmax_scale, rc, rs,
                                splits, O, o_dtype, ws)
    torch.cuda.synchronize()
    return host(O)


def oracle_out(cs, rope, base=10000.0, seqs=None):
    sel = slice(None) if seqs is None else list(seqs)
    C = values(cs.C[sel], "bf16")
    BK = np.ascontiguousarray(values(cs.BK_t, "bf16").transpose(0, 2, 1))
    return oracle.attend_headwise(values(cs.q[sel], "bf16"), C[..., :cs.rk], C[..., cs.rk:], BK,
                                  values(cs.BV, "bf16"), cs.softmax_scale, base if rope else None)


SHAPES = [
    # b, L, heads, rk, rv
    (2, 300, 6, 64, 32),      # ragged last tile, a partial head group
    (1, 1, 4, 32, 32),        # a single cached latent
    (3, 1000, 8, 128, 128),   # 32 tiles, the widest ranks
    (1, 77, 32, 96, 64),      # 32 heads, three partial tiles
    (2, 513, 5, 32, 128),     # one token past 16 tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b{}L{}h{}rk{}rv{}".format(*s))
@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_headwise_matches_oracle(shape, rope):
    b, L, heads, rk, rv = shape
    say(f"case: headwise b={b} L={L} heads={heads} rk={rk} rv={rv} rope={rope}")
    cs = synth.headwise_case(b, L, heads, 128, rk, rv, seed=L + heads)
    got = run_headwise(cs, rope)
    check_rows(got, oracle_out(cs, rope), TOL, "headwise")


@pytest.mark.parametrize("splits", [1, 3, 40])
def test_headwise_split_count_invariance(splits):
    """Any split count (one split, uneven tile shares, more splits than tiles)
    gives the same attention as the default."""
    cs = synth.headwise_case(2, 1100, 8, 128, 64, 64, seed=3)
    say(f"case: headwise split invariance, splits={splits}")
    ref = run_headwise(cs, rope=True, o_dtype=q.F32)
    got = run_headwise(cs, rope=True, splits=splits, o_dtype=q.F32)
    assert oracle.rel_l2(got, ref) <= 1e-5
    assert oracle.rel_l2(got, oracle_out(cs, True)) <= TOL


def test_headwise_rope_relative_positions():
    """A small rotary base makes the rotation matter; the result follows the
    oracle and differs from the unrotated one."""
    cs = synth.headwise_case(1, 600, 4, 128, 64, 64, seed=21)
    plain = run_headwise(cs, rope=False)
    rot = run_headwise(cs, rope=True, base=500.0)
    assert oracle.rel_l2(rot, oracle_out(cs, True, base=500.0)) <= TOL
    assert oracle.rel_l2(rot, plain) > 5e-2


def test_headwise_full_size_sampled():
    """LLaVA-v1.5-7B attention shape with per-head latents (b = 16, L = 8192,
    32 heads x 128, rk = rv = 64) and RoPE: the whole batch in the launch
    configuration the bench times, two sequences against the oracle."""
    b, L, heads, rk, rv = 16, 8192, 32, 64, 64
    say(f"case: headwise full size b={b} L={L} heads={heads} rk={rk} rv={rv} RoPE")
    cs = synth.headwise_case(b, L, heads, 128, rk, rv, seed=7)
    got = run_headwise(cs, rope=True)
    assert np.all(np.isfinite(got))
    for s in (0, b - 1):
        ref = oracle_out(cs, True, seqs=[s])[0]
        err = oracle.rel_l2(got[s], ref)
        say(f"  sequence {s}: rel-L2 {err:.2e}")
        assert err <= TOL


EDGE_SHAPES = [
    # b, L, heads, rk, rv
    (1, 32, 1, 32, 32),       # one full tile, one head
    (2, 64, 3, 64, 96),       # two full tiles, no partial tile
    (1, 33, 4, 128, 32),      # one token past a tile
    (5, 700, 12, 32, 64),     # several head groups and sequences
]


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "b{}L{}h{}rk{}rv{}".format(*s))
def test_headwise_edges(shape):
    b, L, heads, rk, rv = shape
    say(f"case: headwise edge b={b} L={L} heads={heads} rk={rk} rv={rv}")
    cs = synth.headwise_case(b, L, heads, 128, rk, rv, seed=3 * L + heads)
    for rope in (False, True):
        got = run_headwise(cs, rope)
        err = oracle.rel_l2(got, oracle_out(cs, rope))
        say(f"  rope={rope}: rel-L2 {err:.2e}")
        assert err <= TOL


def test_headwise_longer_rope_tables():
    """Tables with more rows than cached tokens (a runtime's preallocated
    maximum length): only rows 0 .. L-1 matter, the result is unchanged."""
    import torch
    cs = synth.headwise_case(2, 150, 4, 128, 64, 64, seed=12)
    want = run_headwise(cs, rope=True, o_dtype=q.F32)
    c, s = synth.rope_tables(cs.L + 333, cs.d)
    O = empty((cs.b, cs.heads, cs.d), torch.float32)
    ws = workspace(q.qsvd_decode_headwise_workspace_bytes(cs.b, cs.L, cs.heads, cs.d, cs.rk, cs.rv, 0))
    q.qsvd_decode_attn_headwise(dev(cs.q), q.BF16, dev(cs.C), q.BF16, dev(cs.BK_t), dev(cs.BV), q.BF16,
                                cs.b, cs.L, cs.heads, cs.d, cs.rk, cs.rv, cs.softmax_scale, dev(c), dev(s),
                                0, O, q.F32, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(O), want)


@pytest.mark.parametrize("factor", [10.0, 60.0])
def test_headwise_sharpened_softmax(factor):
    """Peaked attention (a few tokens carry most of the weight) with RoPE and
    several splits: the online rescaling and the merge."""
    cs = synth.headwise_case(2, 900, 8, 128, 64, 64, seed=44)
    qs = np.ascontiguousarray(synth.to_bf16_bits(values(cs.q, "bf16") * factor))
    import dataclasses
    cs = dataclasses.replace(cs, q=qs)
    say(f"case: headwise sharpened x{factor}")
    for splits in (0, 5):
        got = run_headwise(cs, rope=True, splits=splits)
        err = oracle.rel_l2(got, oracle_out(cs, True))
        say(f"  splits={splits} rel-L2 {err:.2e}")
        assert err <= TOL
