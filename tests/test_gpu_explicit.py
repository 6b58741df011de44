"""GPU parity of qsvd_decode_attn_explicit (explicit on-chip K/V rebuild,
optional rotary positions) against the float64 oracle.

The oracle consumes the exact stored bf16 values; with RoPE it computes its
own angles in float64 (attend_explicit_rope), while the kernel receives the
float32 cos / sin tables a runtime would hand it.  Tolerance: relative L2
over the whole output, and of every (sequence, head) row, <= 2e-2 (bf16 inputs, float32 K/V accumulators, bf16
output; table rounding adds < 2^-24 relative per angle).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import check_rows, decode_case_on_gpu, dev, empty, host, say, values, workspace

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu

TOL = 2e-2


def run_explicit(cs, rope=False, o_dtype=q.BF16, base=10000.0):
    import torch
    Wk_t = dev(np.ascontiguousarray(cs.Wu_k.T))
    Wv_t = dev(np.ascontiguousarray(cs.Wu_v.T))
    rc = rs = None
    if rope:
        c, s = synth.rope_tables(cs.L, cs.d, base)
        rc, rs = dev(c), dev(s)
    O = empty((cs.b, cs.heads, cs.d), torch.bfloat16 if o_dtype == q.BF16 else torch.float32)
    ws = workspace(q.qsvd_decode_explicit_workspace_bytes(cs.b, cs.L, cs.r, cs.heads, cs.d))
    q.qsvd_decode_attn_explicit(dev(cs.q), q.BF16, dev(cs.C), q.BF16, Wk_t, Wv_t, q.BF16, cs.b,
                                cs.L, cs.r, cs.heads, cs.d, cs.softmax_scale, rc, rs, O, o_dtype, ws)
    torch.cuda.synchronize()
    return host(O)


def oracle_out(cs, rope, seqs=None, base=10000.0):
    sel = slice(None) if seqs is None else list(seqs)
    qq, C = values(cs.q, "bf16")[sel], values(cs.C, "bf16")[sel]
    Wk, Wv = values(cs.Wu_k, "bf16"), values(cs.Wu_v, "bf16")
    if rope:
        return oracle.attend_explicit_rope(qq, C, Wk, Wv, cs.heads, cs.d, cs.softmax_scale, base)
    return oracle.attend_explicit(qq, C, Wk, Wv, cs.heads, cs.d, cs.softmax_scale)


SHAPES = [
    # E, heads, r, b, L   (d = 128)
    (512, 4, 256, 2, 300),      # ragged last tile
    (1024, 8, 512, 1, 513),     # one token past two tiles
    (2048, 16, 1536, 1, 77),    # r of the 7B shape, one partial tile
    (512, 4, 128, 3, 1),        # a single cached latent
    (1024, 8, 256, 3, 2500),    # two groups of eight tiles per sequence, the last one partial
    (512, 4, 64, 2, 300),       # r = 64: a single 128-byte K stage
    (1024, 8, 192, 1, 513),     # r = 192: an odd number of K stages
    (4096, 32, 3072, 1, 100),   # r = 3072: the longest K loop of the tests
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "E{}h{}r{}b{}L{}".format(*s))
@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_explicit_matches_oracle(shape, rope):
    E, heads, r, b, L = shape
    say(f"case: explicit E={E} heads={heads} r={r} b={b} L={L} rope={rope}")
    cs = synth.decode_case(E, heads, 128, r, b, L, dtype="bf16", hadamard=128 if r % 128 == 0 else 0,
                           seed=E + L)
    got = run_explicit(cs, rope)
    check_rows(got, oracle_out(cs, rope), TOL, "explicit")


@pytest.mark.parametrize("L", [200, 1300, 4100], ids=lambda v: f"L{v}")
@pytest.mark.parametrize("factor", [30.0, 300.0])
@pytest.mark.parametrize("rope", [False, True], ids=["plain", "rope"])
def test_explicit_sharpened_softmax(L, factor, rope):
    """Peaked attention through the explicit rebuild: one, six and seventeen
    256-token tiles per sequence (a partial group of eight in the last case),
    so that a wrong per-tile maximum or log-sum-exp weight in the tile merge
    shows.  The configs' own generator gives near-uniform attention."""
    say(f"case: explicit sharpened x{factor} L={L} rope={rope}")
    cs = synth.decode_case(1024, 8, 128, 512, 2, L, dtype="bf16", hadamard=128, p=0.5, seed=79 + L)
    qv = synth.to_bf16_bits(synth.sharpen_query(values(cs.q, "bf16"), factor))
    cs.q = qv
    got = run_explicit(cs, rope)
    check_rows(got, oracle_out(cs, rope), TOL, f"x{factor}")


def test_explicit_equals_absorbed_path_without_rope():
    """Without rotation the explicit rebuild and the latent-space path compute
    the same attention (re-association only)."""
    cs = synth.decode_case(1024, 8, 128, 512, 2, 700, dtype="bf16", hadamard=128, seed=5)
    a = run_explicit(cs, rope=False, o_dtype=q.F32)
    b = decode_case_on_gpu(cs, o_dtype=q.F32)
    assert oracle.rel_l2(a, b) <= TOL


def test_explicit_rope_relative_positions():
    """A large rotary base makes every angle but theta_0's tiny; the output
    must still follow the oracle, and differ from the unrotated result."""
    cs = synth.decode_case(512, 4, 128, 256, 1, 600, dtype="bf16", hadamard=0, seed=21)
    plain = run_explicit(cs, rope=False)
    rot = run_explicit(cs, rope=True, base=500.0)
    assert oracle.rel_l2(rot, oracle_out(cs, True, base=500.0)) <= TOL
    assert oracle.rel_l2(rot, plain) > 5e-2


def test_explicit_full_size_7b_rope_sampled():
    """LLaVA-v1.5-7B shape (b = 16, L = 8192, r = 1536, 32 heads) with RoPE:
    the whole batch on the GPU, two sequences against the oracle."""
    cfg = synth.CONFIGS[1]
    say(f"case: explicit full size, {cfg.name}, RoPE")
    cs = synth.config_decode_case(cfg)
    got = run_explicit(cs, rope=True)
    assert np.all(np.isfinite(got))
    for s in (0, cs.b - 1):
        ref = oracle_out(cs, True, seqs=[s])[0]
        err = oracle.rel_l2(got[s], ref)
        say(f"  sequence {s}: rel-L2 {err:.2e}")
        assert err <= TOL
