"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each test runs the HIP path on the whole workload (default split count, bf16
output, one call over the whole batch) and checks sampled outputs against the
float64 oracle computed one by one, plus properties that hold at any size:

* decode of the LLaVA-v1.5-7B and -13B shapes (bf16 latent cache): sampled
  (sequence, head) outputs against the explicit-K/V oracle, every output
  finite, and the whole output independent of the split count;
* the W8A4 shape (int4 group-128 cache, int8 W^u): the GPU's own prefill chain
  (rotate + int8, int8 projection, rotate + int4) fills the cache; sampled
  sequences are bit-exact against the oracle chain, and decode of the whole
  batch is checked on sampled heads of those sequences;
* the 16384 x 4096 prefill: rotate + int8 of X, the projection to r = 1536
  that the bench times, the H2 requantisation and the K/V rebuild of a
  rank-2048 layer, each bit-exact on sampled rows (all four steps are row-wise,
  so the oracle of a row needs only that row).

Every input comes from synth/ and every expected value from oracle/.
Tolerance for decode outputs: relative L2 <= 2e-2 per (sequence, head) row
(bf16 absorbed query, probabilities, partials and output; each <= 2^-9).
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import decode, dev, empty, host, say, values

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _pairs(b, heads, n, seed):
    """n (sequence, head) pairs: both corners plus seeded picks."""
    g = np.random.default_rng(seed)
    pairs = {(0, 0), (b - 1, heads - 1)}
    while len(pairs) < n:
        pairs.add((int(g.integers(b)), int(g.integers(heads))))
    return sorted(pairs)


def _check_bf16_config(idx, n_pairs):
    cfg = synth.CONFIGS[idx]
    say(f"case: full-size decode, {cfg.name}")
    cs = synth.config_decode_case(cfg)
    assert cs.dtype == "bf16" and cs.b == cfg.b and cs.L == cfg.L
    qd, Cd, Wkd, Wvd = dev(cs.q), dev(cs.C), dev(cs.Wu_k), dev(cs.Wu_v)
    args = (qd, q.BF16, Cd, q.BF16, Wkd, Wvd, q.BF16, cs.b, cs.L, cs.r, cs.heads, cs.d,
            cs.softmax_scale)
    O = host(decode(*args))                       # default splits: the bench's launch
    assert np.all(np.isfinite(O))
    O7 = host(decode(*args, splits=7))
    err_split = oracle.rel_l2(O7, O)
    say(f"  default vs 7 splits: rel-L2 {err_split:.2e}")
    assert err_split <= TOL
    Wk, Wv = values(cs.Wu_k, "bf16"), values(cs.Wu_v, "bf16")
    by_seq = {}
    for s, h in _pairs(cs.b, cs.heads, n_pairs, seed=idx):
        by_seq.setdefault(s, []).append(h)
    worst = 0.0
    for s, hs in by_seq.items():
        ref = oracle.attend_explicit_heads(values(cs.q[s], "bf16"), values(cs.C[s], "bf16"),
                                           Wk, Wv, hs, cs.d, cs.softmax_scale)
        for i, h in enumerate(hs):
            err = oracle.rel_l2(O[s, h], ref[i])
            worst = max(worst, err)
            assert err <= TOL, (s, h, err)
    say(f"  {n_pairs} sampled heads: worst rel-L2 {worst:.2e}")


def test_decode_llava7b_bf16_full_size():
    _check_bf16_config(1, 12)


def test_decode_llava13b_bf16_full_size():
    _check_bf16_config(3, 8)


# ------------------------------------------------------------------ W8A4
def _rotate_quant(x_dev, in_dt, M, n, bits, group):
    import torch
    codes = empty((M, n if bits == 8 else n // 2), torch.int8 if bits == 8 else torch.uint8)
    scales = empty((M, n // group) if group else (M,), torch.float32)
    q.qsvd_quantize_latent(x_dev, in_dt, M, n, 128, q.I8 if bits == 8 else q.I4, group,
                           codes, scales)
    return codes, scales


def test_w8a4_chain_and_decode_full_size():
    import torch
    cfg = synth.CONFIGS[2]
    say(f"case: full-size W8A4 chain + decode, {cfg.name}")
    b, L, E, r, heads, d = cfg.b, cfg.L, cfg.E, cfg.r, cfg.heads, cfg.d
    inp = synth.quant_decode_inputs(cfg, range(b))
    w = inp.weights
    Xbits = [synth.to_bf16_bits(x) for x in inp.X]
    Xd = dev(np.concatenate(Xbits))               # [b*L][E] bf16, sequence-major
    M = b * L
    xq, xs = _rotate_quant(Xd, q.BF16, M, E, 8, 0)
    Cf = empty((M, r), torch.float32)
    q.qsvd_project(xq, q.I8, xs, M, E, dev(np.ascontiguousarray(w["Wd_q"].T)), q.I8,
                   dev(w["Wd_s"]), r, Cf, q.F32)
    cq, csc = _rotate_quant(Cf, q.F32, M, r, 4, 128)
    O = decode(dev(inp.q), q.BF16, cq, q.I4, dev(w["Wu_k_q"]), dev(w["Wu_v_q"]), q.I8,
               b, L, r, heads, d, inp.softmax_scale, c_scales=csc, c_group=128,
               wsk=dev(w["Wu_k_s"]), wsv=dev(w["Wu_v_s"]))
    O = host(O)
    assert np.all(np.isfinite(O))
    Wk = oracle.dequant_cols(w["Wu_k_q"], w["Wu_k_s"])
    Wv = oracle.dequant_cols(w["Wu_v_q"], w["Wu_v_s"])
    g = np.random.default_rng(2)
    for s in (0, b - 1):
        rows = slice(s * L, (s + 1) * L)
        c1, s1 = oracle.rotate_quantize(oracle.bf16_decode(Xbits[s]), 128, 8, 0)
        assert np.array_equal(xq[rows].cpu().numpy(), c1), s
        assert np.array_equal(xs[rows].cpu().numpy(), s1), s
        C = oracle.project_int8(c1, s1, w["Wd_q"], w["Wd_s"])
        assert np.array_equal(host(Cf[rows]), C), s
        c3, s3 = oracle.rotate_quantize(C, 128, 4, 128)
        assert np.array_equal(oracle.unpack_int4(cq[rows].cpu().numpy()), c3), s
        assert np.array_equal(csc[rows].cpu().numpy(), s3), s
        say(f"  sequence {s}: prefill chain bit-exact")
        hs = sorted({0, heads - 1, *map(int, g.integers(heads, size=4))})
        ref = oracle.attend_explicit_heads(oracle.bf16_decode(inp.q[s]),
                                           oracle.dequant_rows(c3, s3, 128), Wk, Wv, hs, d,
                                           inp.softmax_scale)
        for i, h in enumerate(hs):
            err = oracle.rel_l2(O[s, h], ref[i])
            assert err <= TOL, (s, h, err)
        say(f"  sequence {s}: heads {hs} within {TOL}")


# ------------------------------------------------------------------ prefill
def test_prefill_full_size_sampled_rows():
    import torch
    M, E, rp, rl = 4 * 4096, 4096, 1536, 2048
    say(f"case: full-size prefill M={M} E={E} (r={rp} projection, r={rl} chain layer)")
    X = synth.to_bf16_bits(synth.prefill_activations(M, E))
    rows = np.unique(np.concatenate([[0, 1, 63, 64, M - 1],
                                     np.random.default_rng(4).integers(M, size=27)]))
    xq, xs = _rotate_quant(dev(X), q.BF16, M, E, 8, 0)
    c1, s1 = oracle.rotate_quantize(oracle.bf16_decode(X[rows]), 128, 8, 0)
    del X
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(xq[ridx].cpu().numpy(), c1)
    assert np.array_equal(xs[ridx].cpu().numpy(), s1)
    say("  a1 rows bit-exact")
    # the projection the bench times
    Wd_q, Wd_s = synth.down_projection_int8(E, rp, 0.5, 0.5, 128, (100400,))
    Cp = empty((M, rp), torch.float32)
    q.qsvd_project(xq, q.I8, xs, M, E, dev(np.ascontiguousarray(Wd_q.T)), q.I8, dev(Wd_s), rp,
                   Cp, q.F32)
    assert np.array_equal(host(Cp[ridx]), oracle.project_int8(c1, s1, Wd_q, Wd_s))
    say("  a2 rows bit-exact (r = 1536)")
    del Cp
    # one rank-2048 layer of the chain: projection, H2 requantisation, K/V rebuild
    lay = synth.c4_layer(0, rl)
    Cl = empty((M, rl), torch.float32)
    q.qsvd_project(xq, q.I8, xs, M, E, dev(np.ascontiguousarray(lay["Wd_q"].T)), q.I8,
                   dev(lay["Wd_s"]), rl, Cl, q.F32)
    cq, csc = _rotate_quant(Cl, q.F32, M, rl, 8, 0)
    Wkv = np.concatenate([lay["Wu_k_q"], lay["Wu_v_q"]], axis=1)          # [r][2E]
    skv = np.concatenate([lay["Wu_k_s"], lay["Wu_v_s"]])
    KV = empty((M, 2 * E), torch.bfloat16)
    q.qsvd_project(cq, q.I8, csc, M, rl, dev(np.ascontiguousarray(Wkv.T)), q.I8, dev(skv),
                   2 * E, KV, q.BF16)
    C = oracle.project_int8(c1, s1, lay["Wd_q"], lay["Wd_s"])
    assert np.array_equal(host(Cl[ridx]), C)
    c3, s3 = oracle.rotate_quantize(C, 128, 8, 0)
    assert np.array_equal(cq[ridx].cpu().numpy(), c3)
    assert np.array_equal(csc[ridx].cpu().numpy(), s3)
    ref = oracle.bf16_round(oracle.project_int8(c3, s3, Wkv, skv))
    assert np.array_equal(host(KV[ridx]), ref)
    say(f"  r = {rl} layer: a2, a3, a4 rows bit-exact")


def test_prefill_w4a4_full_size_sampled_rows():
    """W4A4 at the 16384 x 4096 -> 1536 shape: X rotated by H1 and quantised to
    int4 per token (a1), the int4 x int4 projection (a2), sampled rows
    bit-exact against the oracle chain."""
    import torch
    M, E, r = 4 * 4096, 4096, 1536
    say(f"case: full-size W4A4 prefill M={M} E={E} r={r}")
    X = synth.to_bf16_bits(synth.prefill_activations(M, E))
    rows = np.unique(np.concatenate([[0, 1, M - 1], np.random.default_rng(6).integers(M, size=21)]))
    xq = empty((M, E // 2), torch.uint8)
    xs = empty((M,), torch.float32)
    q.qsvd_quantize_latent(dev(X), q.BF16, M, E, 128, q.I4, 0, xq, xs)
    c1, s1 = oracle.rotate_quantize(oracle.bf16_decode(X[rows]), 128, 4, 0)
    del X
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(oracle.unpack_int4(xq[ridx].cpu().numpy()), c1)
    assert np.array_equal(xs[ridx].cpu().numpy(), s1)
    lay = synth.c4_layer(0, r)
    Wd_q4, Wd_s4 = synth.int4_columns(oracle.dequant_cols(lay["Wd_q"], lay["Wd_s"]))
    Wp = empty((r, E // 2), torch.uint8)
    q.qsvd_pack_weight(dev(Wd_q4), q.I4, E, r, Wp)
    Cp = empty((M, r), torch.float32)
    q.qsvd_project(xq, q.I4, xs, M, E, Wp, q.I4, dev(Wd_s4), r, Cp, q.F32)
    assert np.array_equal(host(Cp[ridx]), oracle.project_int8(c1, s1, Wd_q4, Wd_s4))
    say("  a1 (int4) and a2 (W4A4) rows bit-exact")
