"""Pins of the float64 oracle against facts that the pages and mathematics fix.

CPU only.  Each test names the fact it pins; none of them re-types the
oracle's own formula.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- generator
def test_generator_orthonormal_and_descending():
    """P1: Haar factors are orthonormal; the spectrum is i^-p, descending."""
    lay = synth.make_layer(256, 96, 0.6, 0.5, (1000, 0), k=256)
    assert np.abs(lay.U.T @ lay.U - np.eye(256)).max() < 1e-13
    assert np.abs(lay.V.T @ lay.V - np.eye(256)).max() < 1e-13
    assert np.all(np.diff(lay.sigma) < 0)
    # the first r columns do not depend on how many are generated
    lay96 = synth.make_layer(256, 96, 0.6, 0.5, (1000, 0), k=96)
    assert np.abs(lay96.U - lay.U[:, :96]).max() < 1e-12


def test_joint_svd_recovers_known_spectrum():
    """P2: the library SVD of W_concat = U diag(sigma) V^T returns sigma_i = i^-0.6,
    and the oracle's beta-split factors rebuild the rank-r truncation."""
    E = 256
    lay = synth.make_layer(E, 96, 0.6, 0.5, (1000, 0), k=E)
    Wc = lay.W_concat()
    WQ, WK, WV = Wc[:, :E], Wc[:, E:2 * E], Wc[:, 2 * E:]
    Wd, Wu, S = oracle.joint_svd_factors(WQ, WK, WV, 96, 0.5)
    sig = np.arange(1, E + 1) ** -0.6
    assert np.max(np.abs(S[:E] - sig) / sig) < 1e-12
    # W^d W^u is sign-invariant; compare with the generator's own factors
    assert np.abs(Wd @ Wu - lay.Wd @ lay.Wu).max() < 1e-12
    assert Wd.shape == (E, 96) and Wu.shape == (96, 3 * E)
    # beta only moves singular values between the factors
    Wd3, Wu3, _ = oracle.joint_svd_factors(WQ, WK, WV, 96, 0.3)
    assert np.abs(Wd3 @ Wu3 - Wd @ Wu).max() < 1e-12
    col_norms = np.linalg.norm(Wd3, axis=0)
    assert np.allclose(col_norms, sig[:96] ** 0.3, rtol=1e-12)


# ------------------------------------------------------------- fact (a)
def _c0_inputs(r, L=64, seed=1000):
    E, heads, d = 256, 4, 64
    lay = synth.make_layer(E, r, 0.6, 0.5, (seed, 0), k=E)
    ch = synth.outlier_channels(E, 0.01, synth.rng(seed, 3))
    X = synth.activations(L + 1, E, ch, 20.0, synth.rng(seed, 10, 0))
    return lay, X, heads, d


def test_fact_a_full_rank_equals_original_attention():
    """P3, fact (a): at r = E and without quantisation the latent attention
    equals attention with the original W_Q, W_K, W_V (QSVD notes, 'Key design')."""
    E = 256
    lay, X, heads, d = _c0_inputs(E)
    Wc = lay.W_concat()
    ref = oracle.attend_original(X[:-1], X[-1], Wc[:, :E], Wc[:, E:2 * E], Wc[:, 2 * E:], heads, d)
    lat = oracle.attend_latent_from_x(X[:-1], X[-1], lay.Wd, lay.Wu, heads, d)
    assert oracle.rel_l2(lat, ref) < 1e-12
    # a truncated rank is a real approximation (the check has teeth)
    lay96, _, _, _ = _c0_inputs(96)
    lat96 = oracle.attend_latent_from_x(X[:-1], X[-1], lay96.Wd, lay96.Wu, heads, d)
    assert oracle.rel_l2(lat96, ref) > 1e-3


# ------------------------------------------------------------- fact (b)
def test_fact_b_rotations_leave_output_unchanged():
    """P4, fact (b): Y = (X H1^T)(H1 W^d H2^T)(H2 W^u) = X W^d W^u for orthogonal
    H1, H2 (QSVD notes, 'Key design'), and the latent attention is unchanged."""
    E, r, heads, d = 256, 128, 4, 64
    lay, X, _, _ = _c0_inputs(r)
    H1 = np.kron(np.eye(E // 128), oracle.sylvester_hadamard(128))
    H2 = oracle.sylvester_hadamard(128)
    assert np.abs(H1 @ H1.T - np.eye(E)).max() < 1e-13
    Y = (X @ H1.T) @ (H1 @ lay.Wd @ H2.T) @ (H2 @ lay.Wu)
    assert np.abs(Y - X @ lay.Wd @ lay.Wu).max() / np.abs(Y).max() < 1e-12
    C = X[:-1] @ lay.Wd
    Crot = (X[:-1] @ H1.T) @ (H1 @ lay.Wd @ H2.T)
    Wu_rot = H2 @ lay.Wu
    q = ((X[-1] @ lay.Wd) @ lay.Wu[:, :E]).reshape(1, heads, d)
    o1 = oracle.attend_explicit(q, C[None], lay.Wu_k, lay.Wu_v, heads, d, 1 / 8)
    o2 = oracle.attend_explicit(q, Crot[None], Wu_rot[:, E:2 * E], Wu_rot[:, 2 * E:], heads, d, 1 / 8)
    assert oracle.rel_l2(o2, o1) < 1e-12


# ------------------------------------------------------------- fact (c)
@pytest.mark.parametrize("beta", [0.3, 0.5, 0.7])
def test_fact_c_eckart_young(beta):
    """P5, fact (c): ||W_concat - W^d W^u||_F^2 equals the sum of the dropped
    sigma_i^2, for any beta (SVDQuant glossary, section 2.3)."""
    E = 256
    full = synth.make_layer(E, E, 0.6, beta, (1000, 0), k=E)
    Wc = full.W_concat()
    sig = full.sigma
    for r in (1, 96, 200, 255):
        lay = synth.make_layer(E, r, 0.6, beta, (1000, 0), k=E)
        res = np.sum((Wc - lay.Wd @ lay.Wu) ** 2)
        dropped = np.sum(sig[r:] ** 2)
        assert abs(res - dropped) / dropped < 1e-10
        assert abs(oracle.truncation_residual(Wc, r) - dropped) / dropped < 1e-10


# ------------------------------------------------------------- fact (d)
def test_fact_d_counts_and_page_ratios():
    """P6, fact (d): the latent cache holds r L values, the factors 4 r E
    parameters; the ratios reproduce the numbers the pages print."""
    g = json.load(open(os.path.join(GOLDEN, "page_ratios.json")))
    E, r, L = 4096, 1536, 8192
    cs = synth.decode_case(256, 4, 64, 96, 1, 16, seed=5)
    assert cs.C.shape == (1, 16, 96)                             # r * L per sequence
    assert oracle.joint_cache_count(L, r) == r * L
    assert oracle.joint_param_count(E, r) == 4 * r * E
    assert oracle.separate_param_count(E, r) == 6 * r * E
    assert oracle.separate_cache_count(L, r) == 2 * r * L
    assert oracle.full_kv_count(L, E) == 2 * L * E
    lay = synth.make_layer(256, 96, 0.6, 0.5, (3, 0))
    assert lay.Wd.size + lay.Wu.size == oracle.joint_param_count(256, 96)
    for pair in g["pairs"]:
        # R2 = r / 2E fixes r/E; then R1 must come out as printed
        rE = 2 * pair["R2"]
        assert abs(oracle.ratio_R1(1000, int(round(rE * 1000))) - pair["R1"]) < pair["tol"]
    # configs: 18.75 %, 9.38 %, 22.5 %
    assert oracle.ratio_R2(4096, 1536) == 0.1875
    assert round(oracle.ratio_R2(4096, 768) * 100, 2) == 9.38
    assert oracle.ratio_R2(5120, 2304) == 0.225
    # parameters shrink exactly when r < 0.75 E
    thr = g["compression_active_below"]["r_over_E"]
    assert oracle.ratio_R1(4096, int(thr * 4096)) == 1.0
    assert oracle.ratio_R1(4096, int(thr * 4096) - 1) < 1.0


# ------------------------------------------------------------- P7
def test_absorbed_equals_explicit():
    """P7: the latent-space (absorbed) order used on the GPU equals the explicit
    K/V reconstruction in float64."""
    cs = synth.decode_case(256, 4, 64, 96, 3, 200, seed=11)
    args = (cs.q, cs.C, cs.Wu_k, cs.Wu_v, cs.heads, cs.d, cs.softmax_scale)
    assert oracle.rel_l2(oracle.attend_absorbed(*args), oracle.attend_explicit(*args)) < 1e-12


# ------------------------------------------------------------- P8 FWHT
def test_fwht_sign_pattern_matches_library_hadamard():
    """P8: unit vectors map to the columns of the normalised Sylvester matrix;
    compared with scipy.linalg.hadamard and the popcount closed form."""
    I = np.eye(128)
    out = oracle.fwht_rows_f32(I)
    Hs = scipy.linalg.hadamard(128).astype(np.float64)
    assert np.array_equal(out, Hs * oracle.INV_SQRT128_F32)
    assert np.allclose(oracle.sylvester_hadamard(128) * math.sqrt(128), Hs)


def test_fwht_integer_inputs_exact():
    """P8: with small-integer inputs every stage sum is exact, so each output is
    the exact integer Hadamard product rounded once after the 1/sqrt(128) scale."""
    g = np.random.default_rng(0)
    x = g.integers(-1000, 1000, size=(5, 256)).astype(np.float64)
    Hs = scipy.linalg.hadamard(128).astype(np.float64)
    exact = np.concatenate([x[:, :128] @ Hs.T, x[:, 128:] @ Hs.T], axis=1)
    want = (exact.astype(np.float32) * np.float32(oracle.INV_SQRT128_F32)).astype(np.float64)
    assert np.array_equal(oracle.fwht_rows_f32(x), want)


def test_fwht_two_element_closed_form():
    """P8: a block holding only (a, b) at positions (0, 1) becomes
    fl32(fl32(a +- b) c) with + at even and - at odd positions."""
    a, b = np.float32(1.1), np.float32(-0.3)
    x = np.zeros(128)
    x[0], x[1] = a, b
    out = oracle.fwht_rows_f32(x)
    c = np.float32(oracle.INV_SQRT128_F32)
    assert np.all(out[0::2] == np.float64((a + b) * c))
    assert np.all(out[1::2] == np.float64((a - b) * c))


def test_fwht_orthogonal_and_float32_representable():
    """P8: applying the rotation twice is the identity (H H = I, up to float32
    rounding); outputs are float32 values; dense product within the f32 bound."""
    g = np.random.default_rng(1)
    x = oracle.fl32(g.standard_normal((7, 384)) * 10)
    y = oracle.fwht_rows_f32(x)
    assert np.array_equal(y, oracle.fl32(y))
    z = oracle.fwht_rows_f32(y)
    assert np.abs(z - x).max() < 1e-5 * np.abs(x).max()
    H = np.kron(np.eye(3), oracle.sylvester_hadamard(128))
    assert np.abs(y - x @ H.T).max() < 8 * 2 ** -24 * np.abs(x).sum(axis=1).max()


# ------------------------------------------------------------- P9 quantiser
def test_quantiser_golden_cases():
    """P9: hand-derived rows (zero row, spike, exact ties to even) and int4 packing."""
    g = json.load(open(os.path.join(GOLDEN, "quantiser_cases.json")))
    for case in g["cases"]:
        y = np.array(case["y"], dtype=np.float64)[None]
        codes, scales = oracle.quantize_rows(y, case["bits"], 0)
        assert codes[0].tolist() == case["codes"], case["name"]
        if "scale" in case:
            assert float(scales[0]) == case["scale"], case["name"]
        else:
            assert float(scales[0]) == float(np.float32(3.0) / np.float32(127.0))
        if "packed_hex" in case:
            packed = oracle.pack_int4(codes[0])
            assert [f"{v:02x}" for v in packed] == case["packed_hex"]
            assert np.array_equal(oracle.unpack_int4(packed), codes[0])


def _brute_code(v, s, qmax):
    # nearest code by exhaustive search, ties to the even code
    t = np.float32(np.float32(v) / np.float32(s))
    best = None
    for c in range(-qmax, qmax + 1):
        dist = abs(float(t) - c)
        if best is None or dist < best[0] - 1e-300 or (dist == best[0] and c % 2 == 0):
            best = (dist, c)
    return best[1]


@pytest.mark.parametrize("bits,group", [(8, 0), (4, 0), (4, 16)])
def test_quantiser_brute_force(bits, group):
    """P9: codes agree with an exhaustive nearest-code search in float32 arithmetic,
    and the reconstruction error is at most half a step."""
    qmax = 127 if bits == 8 else 7
    g = np.random.default_rng(bits * 100 + group)
    y = oracle.fl32(g.standard_normal((6, 32)) * np.array([1, 5, 0.01, 100, 1, 1])[:, None])
    y[4, 3] = 0.0
    codes, scales = oracle.quantize_rows(y, bits, group)
    gs = 32 if group == 0 else group
    for i in range(y.shape[0]):
        for j in range(32):
            s = scales[i] if group == 0 else scales[i, j // gs]
            amax = np.abs(y[i, (j // gs) * gs:(j // gs + 1) * gs]).max()
            assert s == np.float32(np.float32(amax) / np.float32(qmax))
            assert codes[i, j] == _brute_code(y[i, j], s, qmax)
            assert abs(y[i, j] - codes[i, j] * float(s)) <= 0.5 * float(s) * (1 + 1e-6)
    assert np.abs(codes).max() == qmax


def test_quantiser_groups_are_independent():
    """P9: per-group scales see only their own 128 elements."""
    y = np.zeros((1, 256))
    y[0, 5] = 7.0
    y[0, 200] = -0.5
    codes, scales = oracle.quantize_rows(y, 4, 128)
    assert codes[0, 5] == 7 and codes[0, 200] == -7
    assert scales[0, 0] == np.float32(1.0) and scales[0, 1] == np.float32(0.5) / np.float32(7.0)


# ------------------------------------------------------------- dequantisers
def test_dequant_rows_hand_built_groups():
    """Per-token-group scales touch only their own 128 columns and their own row
    (QSVD notes, 'Main results': W8A4 caches int4 latents with group scales).
    A scale broadcast along the wrong axis, or groups taken in the wrong order,
    changes a hand-derived value below."""
    codes = np.ones((2, 256), dtype=np.int8)
    codes[1, :] = -3
    codes[0, 130] = 5
    scales = np.array([[2.0, 0.5], [0.25, 8.0]], dtype=np.float32)
    got = oracle.dequant_rows(codes, scales, 128)
    assert got.shape == (2, 256)
    assert np.all(got[0, :128] == 2.0) and got[0, 129] == 0.5 and got[0, 130] == 2.5
    assert np.all(got[1, :128] == -0.75) and np.all(got[1, 128:] == -24.0)
    # per-token scales (group 0): row i scales by scales[i] only; 3 x 5 is not
    # square, so a transposed broadcast fails on shape or value
    c0 = np.arange(15, dtype=np.int8).reshape(3, 5) - 7
    s0 = np.array([1.0, 10.0, 100.0], dtype=np.float32)
    got0 = oracle.dequant_rows(c0, s0, 0)
    for i in range(3):
        for j in range(5):
            assert got0[i, j] == float(c0[i, j]) * float(s0[i])
    # batched leading axes, as the [b][L][r] caches use them
    c3 = np.random.default_rng(5).integers(-7, 8, size=(2, 3, 256)).astype(np.int8)
    s3 = np.random.default_rng(6).random((2, 3, 2)).astype(np.float32)
    got3 = oracle.dequant_rows(c3, s3, 128)
    for b in range(2):
        for t in range(3):
            for j in range(256):
                assert got3[b, t, j] == float(c3[b, t, j]) * float(s3[b, t, j // 128])


@pytest.mark.parametrize("bits,group", [(8, 0), (4, 0), (4, 128)])
def test_dequant_reconstructs_within_half_a_step(bits, group):
    """|dequant(quantise(y)) - y| <= s/2 in every group, through the int4
    packing where the cache uses it; checked with an element loop that does
    not call the dequantiser's broadcasting."""
    g = np.random.default_rng(40 + bits + group)
    y = oracle.fl32(g.standard_normal((4, 384)) * np.array([1.0, 30.0, 1e-3, 7.0])[:, None])
    y[2, 200:300] *= 1e4                      # one loud group next to quiet ones
    codes, scales = oracle.quantize_rows(y, bits, group)
    if bits == 4:
        codes = oracle.unpack_int4(oracle.pack_int4(codes))
    rec = oracle.dequant_rows(codes, scales, group)
    gs = 384 if group == 0 else group
    for i in range(4):
        for j in range(384):
            s = float(scales[i]) if group == 0 else float(scales[i, j // gs])
            assert rec[i, j] == float(codes[i, j]) * s
            assert abs(rec[i, j] - y[i, j]) <= 0.5 * s * (1 + 1e-6)
    # the quiet groups of row 2 keep their own (small) step
    if group == 128:
        assert scales[2, 0] < scales[2, 1] / 100


def test_dequant_cols_scales_columns_not_rows():
    """Per-output-column int8 weights (W8): W[k][n] = code[k][n] x scale[n]."""
    codes = np.array([[1, -2], [3, 4], [-5, 6]], dtype=np.int8)     # [K=3][N=2]
    scale = np.array([10.0, 0.5], dtype=np.float32)
    got = oracle.dequant_cols(codes, scale)
    assert got.tolist() == [[10.0, -1.0], [30.0, 2.0], [-50.0, 3.0]]


def test_project_real_brute_force():
    """The real-valued projection equals a triple-loop sum over k."""
    g = np.random.default_rng(8)
    x = g.standard_normal((3, 7))
    w = g.standard_normal((7, 5))
    got = oracle.project_real(x, w)
    assert got.shape == (3, 5)
    for m in range(3):
        for n in range(5):
            acc = 0.0
            for k in range(7):
                acc += x[m, k] * w[k, n]
            assert abs(got[m, n] - acc) <= 1e-14 * (1 + sum(abs(x[m, k] * w[k, n]) for k in range(7)))


# ------------------------------------------------------------- P10 GEMM
def test_int8_projection_exact_and_epilogue():
    """P10: int32 accumulators equal a brute-force integer product; the epilogue
    equals two float32 multiplies done in numpy float32 arithmetic."""
    g = np.random.default_rng(3)
    A = g.integers(-127, 128, size=(5, 300)).astype(np.int8)
    W = g.integers(-127, 128, size=(300, 7)).astype(np.int8)
    acc = oracle.project_int32(A, W)
    brute = [[sum(int(A[m, k]) * int(W[k, n]) for k in range(300)) for n in range(7)] for m in range(5)]
    assert acc.tolist() == brute
    sx = (g.random(5) * 0.01 + 1e-4).astype(np.float32)
    sw = (g.random(7) * 0.01 + 1e-4).astype(np.float32)
    c = oracle.project_int8(A, sx, W, sw)
    want = (np.array(brute, dtype=np.int64).astype(np.float32) * sx[:, None]) * sw[None, :]
    assert np.array_equal(c, want.astype(np.float64))
    # the largest int8 GEMM of the workloads stays exact in float64
    assert 4096 * 127 * 127 < 2 ** 53


# ------------------------------------------------------------- P11 attention
def test_attention_special_cases():
    """P11: L = 1 gives o_h = c W^u_v,h; q = 0 averages V; a dominant score picks
    its row; a shared latent component shifts scores without moving p."""
    E, heads, d, r = 256, 4, 64, 96
    cs = synth.decode_case(E, heads, d, r, 1, 50, seed=21)
    q, C, Wk, Wv = (np.asarray(a, np.float64) for a in (cs.q, cs.C, cs.Wu_k, cs.Wu_v))
    o1 = oracle.attend_explicit(q, C[:, :1], Wk, Wv, heads, d, 0.125)
    assert np.allclose(o1[0].reshape(-1), C[0, 0] @ Wv, rtol=1e-12, atol=1e-12)
    o0 = oracle.attend_explicit(np.zeros_like(q), C, Wk, Wv, heads, d, 0.125)
    assert np.allclose(o0[0].reshape(-1), (C[0] @ Wv).mean(axis=0), rtol=1e-12, atol=1e-12)
    # dominant score: make row 17 huge along head 2's key direction
    h = 2
    qt = Wk[:, h * d:(h + 1) * d] @ q[0, h]
    C2 = C.copy()
    C2[0, 17] += 1e4 * qt / np.linalg.norm(qt)
    o2 = oracle.attend_explicit(q, C2, Wk, Wv, heads, d, 0.125)
    assert np.allclose(o2[0, h], C2[0, 17] @ Wv[:, h * d:(h + 1) * d], rtol=1e-9)
    # shared component c0: o(c0 + D) = c0 W^u_v + o(D)
    c0 = np.random.default_rng(2).standard_normal(r)
    oa = oracle.attend_explicit(q, C, Wk, Wv, heads, d, 0.125)
    ob = oracle.attend_explicit(q, C + c0, Wk, Wv, heads, d, 0.125)
    assert np.allclose(ob[0].reshape(-1) - oa[0].reshape(-1), c0 @ Wv, rtol=1e-9, atol=1e-9)


def test_attention_over_a_repeated_cache():
    """P11: softmax attention depends on the cached rows only as a multiset with
    multiplicities; repeating every row k times leaves the output unchanged (the
    premise of the large-cache GPU tests), for the shared latent and the per-head
    form, while with rotary positions the repeats sit at new positions and the
    output changes."""
    E, heads, d, r, P, k = 256, 4, 64, 96, 7, 3
    cs = synth.decode_case(E, heads, d, r, 1, P, seed=23)
    q, C, Wk, Wv = (np.asarray(a, np.float64) for a in (cs.q, cs.C, cs.Wu_k, cs.Wu_v))
    Crep = np.tile(C, (1, k, 1))                      # row t = base row t mod P
    base = oracle.attend_explicit(q, C, Wk, Wv, heads, d, 0.125)
    assert np.allclose(oracle.attend_explicit(q, Crep, Wk, Wv, heads, d, 0.125), base, rtol=1e-12, atol=1e-14)
    hc = synth.headwise_case(1, P, 2, 128, 32, 32, seed=5)
    Cb = oracle.bf16_decode(hc.C)
    BK = np.ascontiguousarray(oracle.bf16_decode(hc.BK_t).transpose(0, 2, 1))
    BV, qh = oracle.bf16_decode(hc.BV), oracle.bf16_decode(hc.q)
    Cr = np.tile(Cb, (1, k, 1, 1))
    hb = oracle.attend_headwise(qh, Cb[..., :32], Cb[..., 32:], BK, BV, hc.softmax_scale, None)
    hr = oracle.attend_headwise(qh, Cr[..., :32], Cr[..., 32:], BK, BV, hc.softmax_scale, None)
    assert np.allclose(hr, hb, rtol=1e-12, atol=1e-14)
    rb = oracle.attend_headwise(qh, Cb[..., :32], Cb[..., 32:], BK, BV, hc.softmax_scale, 50.0)
    rr = oracle.attend_headwise(qh, Cr[..., :32], Cr[..., 32:], BK, BV, hc.softmax_scale, 50.0)
    assert not np.allclose(rr, rb, rtol=1e-6, atol=1e-8)


def test_attend_heads_subset_matches_full():
    cs = synth.decode_case(256, 4, 64, 96, 2, 40, seed=4)
    full = oracle.attend_explicit(cs.q, cs.C, cs.Wu_k, cs.Wu_v, 4, 64, cs.softmax_scale)
    part = oracle.attend_explicit_heads(cs.q[1], cs.C[1], cs.Wu_k, cs.Wu_v, [3, 1], 64, cs.softmax_scale)
    assert np.allclose(part, full[1, [3, 1]], rtol=1e-13, atol=1e-13)


def test_bf16_round_ties_and_decode():
    """bf16 rounding used when the oracle models a bf16 output: RNE on float32 bits."""
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert oracle.bf16_round(np.array([1 + 2 ** -8]))[0] == 1.0
    assert oracle.bf16_round(np.array([1 + 3 * 2 ** -8]))[0] == 1 + 2 ** -6
    assert oracle.bf16_decode(np.array([0x3F80, 0xBF80], dtype=np.uint16)).tolist() == [1.0, -1.0]


# ------------------------------------------------------------------ rotary positions
def test_rope_matches_complex_rotation_and_preserves_norm():
    """rope_rotate against the complex form: the pair (x[i], x[i + d/2]) is the
    complex number x[i] + j x[i + d/2] multiplied by e^{j pos theta_i}."""
    g = np.random.default_rng(11)
    d = 16
    x = g.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 4095])
    got = oracle.rope_rotate(x, pos, base=500.0)
    theta = 500.0 ** (-np.arange(d // 2) * 2.0 / d)
    z = (x[:, : d // 2] + 1j * x[:, d // 2:]) * np.exp(1j * pos[:, None] * theta[None, :])
    want = np.concatenate([z.real, z.imag], axis=1)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.array_equal(oracle.rope_rotate(x, np.zeros(5)), x)          # angle 0
    # two-dimensional case: the plain rotation matrix
    v = np.array([0.3, -1.7])
    a = 3.0                                                               # theta_0 = 1
    R = np.array([[math.cos(a), -math.sin(a)], [math.sin(a), math.cos(a)]])
    assert np.allclose(oracle.rope_rotate(v, 3), R @ v, atol=1e-15)


def test_rope_attention_relative_positions_and_l1():
    cs = synth.decode_case(256, 2, 128, 96, 2, 40, dtype="f32", seed=9)
    q, C = cs.q.astype(np.float64), cs.C.astype(np.float64)
    a = oracle.attend_explicit_rope(q, C, cs.Wu_k, cs.Wu_v, 2, 128, cs.softmax_scale)
    b = oracle.attend_explicit_rope(q, C, cs.Wu_k, cs.Wu_v, 2, 128, cs.softmax_scale, pos0=777)
    assert oracle.rel_l2(b, a) < 1e-11                 # only position differences enter
    plain = oracle.attend_explicit(q, C, cs.Wu_k, cs.Wu_v, 2, 128, cs.softmax_scale)
    assert oracle.rel_l2(a, plain) > 1e-3              # the rotation does change the result
    # L = 1: the only key and the query sit at the same position
    a1 = oracle.attend_explicit_rope(q, C[:, :1], cs.Wu_k, cs.Wu_v, 2, 128, cs.softmax_scale, pos0=5)
    p1 = oracle.attend_explicit(q, C[:, :1], cs.Wu_k, cs.Wu_v, 2, 128, cs.softmax_scale)
    assert oracle.rel_l2(a1, p1) < 1e-13


# ------------------------------------------------------------------ per-head latents
@pytest.mark.parametrize("base", [None, 10000.0])
def test_headwise_equals_block_diagonal_shared_latent(base):
    """Per-head latents are the shared-latent attention with the heads' latents
    concatenated and W^u block-diagonal: the two oracle paths must agree."""
    g = np.random.default_rng(31)
    b, L, heads, d, rk, rv = 2, 37, 3, 16, 5, 7
    q = g.standard_normal((b, heads, d))
    CK = g.standard_normal((b, L, heads, rk))
    CV = g.standard_normal((b, L, heads, rv))
    BK = g.standard_normal((heads, rk, d)) / math.sqrt(rk)
    BV = g.standard_normal((heads, rv, d)) / math.sqrt(rv)
    got = oracle.attend_headwise(q, CK, CV, BK, BV, 0.3, base)
    C = np.concatenate([CK.reshape(b, L, heads * rk), CV.reshape(b, L, heads * rv)], axis=2)
    Wk = np.zeros((heads * (rk + rv), heads * d))
    Wv = np.zeros_like(Wk)
    for h in range(heads):
        Wk[h * rk:(h + 1) * rk, h * d:(h + 1) * d] = BK[h]
        Wv[heads * rk + h * rv: heads * rk + (h + 1) * rv, h * d:(h + 1) * d] = BV[h]
    if base is None:
        want = oracle.attend_explicit(q, C, Wk, Wv, heads, d, 0.3)
    else:
        want = oracle.attend_explicit_rope(q, C, Wk, Wv, heads, d, 0.3, base)
    assert oracle.rel_l2(got, want) < 1e-12


def test_headwise_full_rank_identity_is_plain_attention():
    """rk = rv = d with B = I: keys and values are the latents themselves."""
    g = np.random.default_rng(32)
    b, L, heads, d = 1, 20, 2, 8
    q = g.standard_normal((b, heads, d))
    K = g.standard_normal((b, L, heads, d))
    V = g.standard_normal((b, L, heads, d))
    eye = np.stack([np.eye(d)] * heads)
    got = oracle.attend_headwise(q, K, V, eye, eye, 1 / math.sqrt(d))
    for h in range(heads):
        s = K[0, :, h] @ q[0, h] / math.sqrt(d)
        p = np.exp(s - s.max())
        p /= p.sum()
        assert np.allclose(got[0, h], p @ V[0, :, h], atol=1e-13)
