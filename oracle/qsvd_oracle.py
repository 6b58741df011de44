"""Float64 CPU oracle for the QSVD joint-QKV latent-attention inference path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It shares no code with the HIP
library (no kernels, headers, helpers or tables) and imports nothing from it;
the HIP path never calls it.

Sources (cited by page title and section):

[QSVD-notes]   "QSVD: Efficient Low-Rank Approximation for Unified Query-Key-Value
               Weight Compression", NeurIPS 2025 paper notes (zhaoyang97 Paper-Notes).
[QSVD-digest]  "QSVD: Efficient Low-rank Approximation for Unified Query-Key-Value
               Weight Compression in Low-Precision Vision-Language Models" (r9-hu
               paper digest).
[WSVD-digest]  "WSVD: Weighted Low-Rank Approximation for Fast and Efficient
               Execution of Low-Precision Vision-Language Models" (r9-hu digest).
[SVDQuant]     "SVDQuant 低秩残差量化算法" glossary entry (MindStudio docs).

Conventions (readings of points the pages leave open, listed in the design notes):
row-vector tokens X in R^{L x E}; Q = X W_Q; W_concat = [W_Q | W_K | W_V];
W^u split by column blocks in Q, K, V order; head h owns columns
[h d, (h+1) d); softmax scale 1/sqrt(d), no mask; no positional rotation except
in attend_explicit_rope (the explicit-reconstruction variant).

Floating point: everything is float64 except the explicitly emulated float32
rounding points of the encodings (Walsh-Hadamard rotation, absmax quantiser,
int8 GEMM epilogue).  fl32(a op b) for +, -, *, / is computed as the float64
result rounded to float32, which equals the correctly rounded float32
operation because 53 >= 2*24 + 2 (double rounding is innocuous).

Parity status per function is listed in each docstring ("pinned by").
"""
from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# Rounding helpers
# ----------------------------------------------------------------------------


def fl32(x) -> np.ndarray:
    """Round to the nearest float32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_decode(bits) -> np.ndarray:
    """bf16 storage bits (uint16) -> exact float64 value."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """Round float32 values to bf16 (ties to even); returns float64 values."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


# fl32(1/sqrt(128)); its bit pattern is 0x3DB504F3
INV_SQRT128_F32 = float(np.float32(1.0 / math.sqrt(128.0)))

# ----------------------------------------------------------------------------
# Rotation H: block-diagonal normalised Walsh-Hadamard, 128-wide blocks
# ----------------------------------------------------------------------------


def fwht_rows_f32(y, block: int = 128) -> np.ndarray:
    """Rotate each row by blockdiag(H_128): y' = y H^T (H symmetric, so = H y per block).

    [QSVD-notes] "Key design" (quantisation scheme: orthogonal H1 on X, H2 on
    C_qkv); [QSVD-digest] "Method, Step 3".  H_128[i][j] = (-1)^popcount(i & j)
    / sqrt(128) (Sylvester order).

    Float32 algorithm (pinned order): for stages h = 1, 2, 4, ..., 64, every
    pair (j, j + h) with (j & h) == 0 becomes (a + b, a - b), each rounded to
    float32; after the last stage every value is multiplied by fl32(1/sqrt(128))
    and rounded to float32.  Input values must be float32-representable.

    Pinned by: dense Sylvester matrix (exact arithmetic, tolerance), H H = I,
    unit vectors -> scaled columns, and two-element closed forms.
    """
    y = np.array(y, dtype=np.float64, copy=True)
    n = y.shape[-1]
    assert n % block == 0 and block & (block - 1) == 0
    lead = y.shape[:-1]
    v = y.reshape(-1, n // block, block)
    h = 1
    while h < block:
        w = v.reshape(v.shape[0], v.shape[1], block // (2 * h), 2, h)
        a = w[:, :, :, 0, :].copy()
        b = w[:, :, :, 1, :].copy()
        w[:, :, :, 0, :] = fl32(a + b)
        w[:, :, :, 1, :] = fl32(a - b)
        h *= 2
    v = fl32(v * (1.0 / math.sqrt(block) if block != 128 else INV_SQRT128_F32))
    return v.reshape(*lead, n)


def sylvester_hadamard(n: int) -> np.ndarray:
    """Dense normalised Sylvester-Hadamard matrix from its closed form
    H[i][j] = (-1)^popcount(i & j) / sqrt(n)."""
    i = np.arange(n)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0) / math.sqrt(n)


# ----------------------------------------------------------------------------
# Absmax quantiser (per token, or per token and 128-wide group)
# ----------------------------------------------------------------------------


def quantize_rows(y, bits: int, group: int = 0):
    """Symmetric absmax quantisation of float32 rows.

    [QSVD-notes] "Key design" and the W8A8 / W8A4 / W4A4 results table
    (per-token integer activations and cached latents); [QSVD-digest]
    "Method, Step 3".  The pages give no formulas; this is the plainest reading:

      qmax = 127 (8 bit) or 7 (4 bit)       (-128 / -8 are never produced)
      for every group (the whole row if group == 0, else `group` contiguous
      elements):  amax = max |y_i|;  s = fl32(amax / qmax);
                  code_i = clamp(rne(fl32(y_i / s)), -qmax, qmax);
                  amax == 0  ->  s = 0 and all codes 0.

    Returns (codes int8 [..][n], scales float32 [..] or [..][n/group]).
    Pinned by hand-built rows (zero row, single spike, exact ties), the
    |y - code s| <= s/2 bound, and brute force on tiny inputs.
    """
    qmax = {8: 127, 4: 7}[bits]
    y = np.asarray(y, dtype=np.float64)
    n = y.shape[-1]
    g = n if group == 0 else group
    assert n % g == 0
    v = y.reshape(*y.shape[:-1], n // g, g)
    amax = np.abs(v).max(axis=-1)
    s = fl32(amax / qmax)
    safe = np.where(s > 0, s, 1.0)
    q = np.rint(fl32(v / safe[..., None]))
    q = np.clip(q, -qmax, qmax)
    q = np.where((s > 0)[..., None], q, 0.0)
    codes = q.reshape(y.shape).astype(np.int8)
    scales = s.astype(np.float32)
    if group == 0:
        scales = scales[..., 0]
    return codes, scales


def pack_int4(codes) -> np.ndarray:
    """Two's-complement nibbles: element 2j -> low nibble of byte j, 2j+1 -> high."""
    c = np.asarray(codes, dtype=np.int16)
    assert c.shape[-1] % 2 == 0
    lo = c[..., 0::2] & 0xF
    hi = c[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_int4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant_rows(codes, scales, group: int = 0) -> np.ndarray:
    """code x scale per token (group == 0) or per token and `group`-wide column
    group (the W8A4 latent of [QSVD-notes] "Main results"); exact in float64.
    Pinned by hand-built rows (each group's scale touches only its own columns
    and row), the |dequant(quantise(y)) - y| <= s/2 bound through int4 packing,
    and an element loop on batched [b][L][r] codes."""
    c = np.asarray(codes, dtype=np.float64)
    s = np.asarray(scales, dtype=np.float64)
    if group == 0:
        return c * s[..., None]
    n = c.shape[-1]
    return (c.reshape(*c.shape[:-1], n // group, group) * s[..., None]).reshape(c.shape)


def dequant_cols(codes, col_scale) -> np.ndarray:
    """Per-output-column int8 weights: W[k][n] = code[k][n] x scale[n] (the W8
    weights of [QSVD-notes] "Main results").  Pinned by a hand-built non-square
    case whose values change if the scale runs along rows."""
    return np.asarray(codes, np.float64) * np.asarray(col_scale, np.float64)[None, :]


def rotate_quantize(x, hadamard_block: int, bits: int, group: int = 0):
    """Rows of x -> float32 -> optional block Walsh-Hadamard -> absmax codes.

    The shared input step of the X-side and latent-side quantisation
    ([QSVD-notes] "Key design": X H1^T before the int8 activation quantiser,
    C H2^T before the cached latent is quantised).
    """
    y = fl32(x)
    if hadamard_block:
        y = fwht_rows_f32(y, hadamard_block)
    return quantize_rows(y, bits, group)


# ----------------------------------------------------------------------------
# Shared down-projection C = X W^d (prefill)
# ----------------------------------------------------------------------------


def project_int8(x_codes, x_scale, w_codes, w_scale) -> np.ndarray:
    """C[m][n] = fl32(fl32(fl32(acc[m][n]) * x_scale[m]) * w_scale[n]),
    acc = sum_k x_codes[m][k] w_codes[k][n] (exact integer).

    [QSVD-notes] "Key design" (C_qkv = X W^d_qkv, computed once per token and
    cached); [QSVD-digest] "Key Contributions" (one shared down-projection
    gives a single pass over the input).  The integer product is formed with
    float64 BLAS: |acc| <= K * 127 * 127 < 2^53 for K < 5.5e8, so every
    summation order is exact.  Pinned by a brute-force integer product.
    """
    a = np.asarray(x_codes, np.float64)
    w = np.asarray(w_codes, np.float64)
    assert a.shape[-1] * 127 * 127 < 2 ** 53
    acc = a @ w
    c = fl32(fl32(acc) * np.asarray(x_scale, np.float64)[:, None])
    return fl32(c * np.asarray(w_scale, np.float64)[None, :])


def project_int32(x_codes, w_codes) -> np.ndarray:
    """Exact int32 accumulators of the int8 GEMM (for bit-exact checks)."""
    return (np.asarray(x_codes, np.float64) @ np.asarray(w_codes, np.float64)).astype(np.int64)


def project_real(x, w) -> np.ndarray:
    """Real-valued product for the bf16 / float32 projection (compared with a
    tolerance).  Pinned by a brute-force triple loop."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64)


# ----------------------------------------------------------------------------
# Joint QKV SVD (offline) and the method's counts
# ----------------------------------------------------------------------------


def joint_svd_factors(W_Q, W_K, W_V, r: int, beta: float):
    """[QSVD-notes] "Key design": concatenate W_Q, W_K, W_V (E x E each) into
    W_concat (E x 3E), take the rank-r SVD W_concat ~ U_r Sigma_r V_r^T, and
    split it into the shared down-projection W^d = U_r Sigma_r^beta (E x r)
    and the up-projections W^u = Sigma_r^(1-beta) V_r^T (r x 3E), whose column
    blocks are W^u_q, W^u_k, W^u_v ([QSVD-digest] "Method, Step 1"; the beta
    split from [QSVD-notes] "Key design" / [QSVD-digest] "Method, Step 3").

    Returns (W_d, W_u, sigma).  Singular-vector signs are LAPACK's.
    Pinned by Eckart-Young and by reproducing a known synthetic spectrum.
    """
    Wc = np.concatenate([W_Q, W_K, W_V], axis=1)
    U, S, Vt = np.linalg.svd(Wc, full_matrices=False)
    Wd = U[:, :r] * S[:r] ** beta
    Wu = (S[:r] ** (1.0 - beta))[:, None] * Vt[:r]
    return Wd, Wu, S


def truncation_residual(W, r: int) -> float:
    """||W - W_r||_F^2 with W_r the rank-r truncated SVD ([SVDQuant] section 2.3:
    the truncated SVD is the best rank-r approximation, and its residual energy
    is the sum of the dropped sigma_i^2)."""
    U, S, Vt = np.linalg.svd(W, full_matrices=False)
    Wr = (U[:, :r] * S[:r]) @ Vt[:r]
    return float(np.sum((W - Wr) ** 2))


def joint_param_count(E: int, r: int) -> int:
    """Shared W^d (E r) plus three up-projections (3 r E) = 4 r E ([QSVD-notes] "Key design")."""
    return E * r + 3 * r * E


def separate_param_count(E: int, r: int) -> int:
    """Separate per-matrix SVD of W_Q, W_K, W_V: 3 (E r + r E) = 6 r E ([QSVD-notes] "Key design")."""
    return 3 * (E * r + r * E)


def joint_cache_count(L: int, r: int) -> int:
    """Cached values per sequence and layer: one r-wide latent per token ([QSVD-notes] "Key design")."""
    return r * L


def separate_cache_count(L: int, r: int) -> int:
    """Separate K and V latents: 2 r L ([QSVD-digest] "Problem")."""
    return 2 * r * L


def full_kv_count(L: int, E: int) -> int:
    """Uncompressed K and V caches: 2 L E ([QSVD-digest] "Method, Step 1")."""
    return 2 * L * E


def ratio_R1(E: int, r: int) -> float:
    """Parameter ratio of the joint factors to W_Q, W_K, W_V: 4 r E / 3 E^2."""
    return joint_param_count(E, r) / (3 * E * E)


def ratio_R2(E: int, r: int, L: int = 1) -> float:
    """Cache ratio of the latent to the full K/V cache: r L / 2 L E."""
    return joint_cache_count(L, r) / full_kv_count(L, E)


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------


def _softmax(s: np.ndarray) -> np.ndarray:
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attend_explicit(q, C, Wu_k, Wu_v, heads: int, d: int, softmax_scale: float) -> np.ndarray:
    """Decode attention over a latent cache, with K and V materialised.

    [QSVD-notes] "Key design": only C_qkv = X W^d is cached; K and V are
    rebuilt on demand as K = C W^u_k, V = C W^u_v ([QSVD-digest] "Method,
    Step 1").  For every sequence b and head h:
        K_h = C_b W^u_k[:, h d:(h+1) d],  V_h = C_b W^u_v[:, h d:(h+1) d]
        s = softmax_scale * K_h q_{b,h};  p = softmax(s);  o_{b,h} = p^T V_h.
    q: [b][heads][d]; C: [b][L][r] (dequantised values); Wu_k, Wu_v: [r][E].
    Returns O [b][heads][d] (float64).
    Pinned by fact (a) (r = E equals attention with W_Q, W_K, W_V), by the
    special cases L = 1, q = 0, one dominant score, score shift invariance.
    """
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    Wk = np.asarray(Wu_k, np.float64)
    Wv = np.asarray(Wu_v, np.float64)
    b = q.shape[0]
    out = np.empty((b, heads, d))
    for s in range(b):
        K = C[s] @ Wk                       # [L][E]
        V = C[s] @ Wv
        for h in range(heads):
            cols = slice(h * d, (h + 1) * d)
            p = _softmax(softmax_scale * (K[:, cols] @ q[s, h]))
            out[s, h] = p @ V[:, cols]
    return out


def attend_explicit_heads(q, C, Wu_k, Wu_v, heads_idx, d: int, softmax_scale: float) -> np.ndarray:
    """attend_explicit for one sequence and a subset of heads (bounded CPU work).

    q: [heads][d]; C: [L][r].  Returns [len(heads_idx)][d]."""
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    out = []
    for h in heads_idx:
        cols = slice(h * d, (h + 1) * d)
        K = C @ np.asarray(Wu_k[:, cols], np.float64)
        V = C @ np.asarray(Wu_v[:, cols], np.float64)
        p = _softmax(softmax_scale * (K @ q[h]))
        out.append(p @ V)
    return np.stack(out)


def attend_absorbed(q, C, Wu_k, Wu_v, heads: int, d: int, softmax_scale: float) -> np.ndarray:
    """The same attention re-associated in the latent space (float64):
    q~_h = softmax_scale * W^u_k,h q_h (r-vector), s = C q~_h, p = softmax(s),
    O~_h = p^T C (r-vector), o_h = O~_h W^u_v,h.  Equal to attend_explicit in
    exact arithmetic by associativity; [WSVD-digest] "Method, 3.4" folds the
    value up-projection into the output side in the same way.
    Pinned against attend_explicit."""
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    Wk = np.asarray(Wu_k, np.float64)
    Wv = np.asarray(Wu_v, np.float64)
    b = q.shape[0]
    out = np.empty((b, heads, d))
    for s in range(b):
        for h in range(heads):
            cols = slice(h * d, (h + 1) * d)
            qt = softmax_scale * (Wk[:, cols] @ q[s, h])
            p = _softmax(C[s] @ qt)
            out[s, h] = (p @ C[s]) @ Wv[:, cols]
    return out


def attend_original(X_ctx, x_new, W_Q, W_K, W_V, heads: int, d: int) -> np.ndarray:
    """Uncompressed multi-head attention of one new token over its context:
    q = x_new W_Q, K = X_ctx W_K, V = X_ctx W_V, softmax(K_h q_h / sqrt d) V_h.
    Returns [heads][d].  The reference point of fact (a)."""
    q = np.asarray(x_new, np.float64) @ W_Q
    K = np.asarray(X_ctx, np.float64) @ W_K
    V = np.asarray(X_ctx, np.float64) @ W_V
    out = np.empty((heads, d))
    for h in range(heads):
        cols = slice(h * d, (h + 1) * d)
        p = _softmax((K[:, cols] @ q[cols]) / math.sqrt(d))
        out[h] = p @ V[:, cols]
    return out


def attend_latent_from_x(X_ctx, x_new, Wd, Wu, heads: int, d: int) -> np.ndarray:
    """Latent attention of the compressed layer, from activations:
    C = X_ctx W^d, q = (x_new W^d) W^u_q, then attend_explicit."""
    E = heads * d
    C = np.asarray(X_ctx, np.float64) @ Wd
    q = (np.asarray(x_new, np.float64) @ Wd) @ Wu[:, :E]
    return attend_explicit(q.reshape(1, heads, d), C[None], Wu[:, E:2 * E], Wu[:, 2 * E:],
                           heads, d, 1.0 / math.sqrt(d))[0]


# ----------------------------------------------------------------------------
# Rotary position embedding (explicit-reconstruction variant)
# ----------------------------------------------------------------------------


def rope_rotate(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of vectors x [..][d] at integer positions pos [..].

    [WSVD-digest] "Key Contributions" (and "Method, 3.4"): the fused decode
    kernel applies RoPE to the keys it reconstructs on chip.  The pages give
    no convention; the reading taken here is the split-half one of the LLaMA
    family the evaluated models use: with i = 0 .. d/2 - 1,
    theta_i = base^(-2 i / d) and angle a = pos * theta_i,
        x'[i]       = x[i] cos a - x[i + d/2] sin a
        x'[i + d/2] = x[i + d/2] cos a + x[i] sin a.
    Pinned by the complex form (x[i] + j x[i+d/2]) e^{j a}, norm
    preservation, and relative-position invariance of the attention below."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    a = np.asarray(pos, np.float64)[..., None] * theta
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def attend_explicit_rope(q, C, Wu_k, Wu_v, heads: int, d: int, softmax_scale: float,
                         base: float = 10000.0, pos0: int = 0) -> np.ndarray:
    """attend_explicit with rotary positions: cached latent t of every
    sequence is the token at position pos0 + t, the decode query is the token
    at position pos0 + L - 1 (its own latent is the last cached one).  Keys are
    rebuilt explicitly, K_h = C_b W^u_k,h, then rotated; the query is rotated;
    V_h = C_b W^u_v,h is not rotated:
        s_t = softmax_scale * rope(K_h[t], pos0 + t) . rope(q_h, pos0 + L - 1).
    Returns O [b][heads][d] (float64).  Pinned by pos0 invariance (only
    position differences enter) and, at L = 1, by attend_explicit."""
    q = np.asarray(q, np.float64)
    C = np.asarray(C, np.float64)
    Wk = np.asarray(Wu_k, np.float64)
    Wv = np.asarray(Wu_v, np.float64)
    b, L = q.shape[0], C.shape[1]
    kpos = pos0 + np.arange(L)
    out = np.empty((b, heads, d))
    for s in range(b):
        K = C[s] @ Wk
        V = C[s] @ Wv
        for h in range(heads):
            cols = slice(h * d, (h + 1) * d)
            kr = rope_rotate(K[:, cols], kpos, base)
            qr = rope_rotate(q[s, h], pos0 + L - 1, base)
            p = _softmax(softmax_scale * (kr @ qr))
            out[s, h] = p @ V[:, cols]
    return out


# ----------------------------------------------------------------------------
# Per-head latents (WSVD decode)
# ----------------------------------------------------------------------------


def attend_headwise(q, CK, CV, BK, BV, softmax_scale: float, base: float | None = None) -> np.ndarray:
    """Decode attention over per-head latents ([WSVD-digest] "Method, 3.1"
    per-head SVD W_Kh = A_Kh B_Kh with the per-head latent C_Kh = X A_Kh, and
    "Method, 3.4" the fused decode that rebuilds K_{h,t} = C_{Kh,t} B_{Kh}).
    With V the same way (C_Vh, B_Vh), for every sequence b and head h:
        K_h = CK[b, :, h] BK[h],  V_h = CV[b, :, h] BV[h],
        s = softmax_scale * rope(K_h[t], t) . rope(q_h, L - 1)   (no rotation if base is None),
        o_{b,h} = softmax(s)^T V_h.
    q [b][heads][d]; CK [b][L][heads][rk]; CV [b][L][heads][rv]; BK [heads][rk][d];
    BV [heads][rv][d].  Returns O [b][heads][d] (float64).
    Pinned by the block-diagonal form: the same attention through
    attend_explicit / attend_explicit_rope with the latents of all heads
    concatenated and W^u_k, W^u_v block-diagonal in the heads."""
    q = np.asarray(q, np.float64)
    CK = np.asarray(CK, np.float64)
    CV = np.asarray(CV, np.float64)
    BK = np.asarray(BK, np.float64)
    BV = np.asarray(BV, np.float64)
    b, L, heads = CK.shape[0], CK.shape[1], CK.shape[2]
    out = np.empty((b, heads, q.shape[2]))
    for s in range(b):
        for h in range(heads):
            K = CK[s, :, h] @ BK[h]
            V = CV[s, :, h] @ BV[h]
            qh = q[s, h]
            if base is not None:
                K = rope_rotate(K, np.arange(L), base)
                qh = rope_rotate(qh, L - 1, base)
            out[s, h] = _softmax(softmax_scale * (K @ qh)) @ V
    return out


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
