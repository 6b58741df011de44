/*
 * qsvd.h - C ABI of the QSVD joint-QKV latent-attention inference path (gfx950).
 *
 * The method (QSVD paper notes, NeurIPS 2025, "Key design"; QSVD digest,
 * "Method, Steps 1 and 3"): the Q, K and V projections of an attention layer
 * share one down-projection W^d (E x r).  Each token's latent
 * C_qkv = X W^d (width r) is computed once and cached instead of K and V;
 * K = C W^u_k and V = C W^u_v are rebuilt on demand.  Orthogonal rotations
 * smooth outliers before quantisation: Y = (X H1^T)(H1 W^d H2^T)(H2 W^u).
 *
 * Three calls carry the path:
 *   qsvd_quantize_latent  rotate rows by a block Walsh-Hadamard H and quantise
 *                         them (X by H1 before the projection, C by H2 before
 *                         it is cached);
 *   qsvd_project          the shared down-projection C = X W^d (and, with the
 *                         same semantics, the K/V reconstruction C [W^u_k|W^u_v]);
 *   qsvd_decode_attn      one decode step: attention of q over the L cached
 *                         latents, K and V never written to memory.
 *
 * Conventions for every call
 *   - Pointers to tensors are DEVICE pointers owned by the caller, 16-byte
 *     aligned, row-major, densely packed.  The library allocates nothing on
 *     these paths; scratch comes from the caller's workspace.
 *   - hip_stream is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous on that stream and never synchronise it.
 *   - Arguments are validated on the host before anything is launched.  On a
 *     validation failure the call returns a negative status, launches nothing
 *     and writes nothing; qsvd_last_error() describes the failure.  A launch
 *     error reported by the HIP runtime returns QSVD_ERR_DEVICE.
 *   - Thread-safe: the only mutable library state is thread-local (the last
 *     error text and an optional timing session).
 *   - bf16 is stored as raw 16-bit brain-float; int4 is packed two's-complement
 *     nibbles, element 2j in the low nibble of byte j and 2j+1 in the high one.
 *   - Rounding: float32 arithmetic rounds to nearest even, with no fused
 *     multiply-add in the rotation, the quantiser or the int8 GEMM epilogue;
 *     division is correctly rounded; float32 -> bf16 rounds to nearest even.
 */
#ifndef QSVD_H
#define QSVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* In C++ the enums below get int32_t as their fixed underlying type, so an
 * out-of-range value passed across the C ABI is a valid (and rejected)
 * argument rather than undefined behaviour; the size and passing convention
 * are those of the C enums (int). */
#ifdef __cplusplus
#define QSVD_ENUM_BASE : int32_t
#else
#define QSVD_ENUM_BASE
#endif

typedef enum qsvd_dtype QSVD_ENUM_BASE {
  QSVD_F32 = 0,   /* IEEE binary32 */
  QSVD_BF16 = 1,  /* bfloat16 */
  QSVD_I8 = 2,    /* int8 codes (symmetric, +-127) */
  QSVD_I4 = 3     /* packed int4 codes (symmetric, +-7) */
} qsvd_dtype_t;

typedef enum qsvd_status QSVD_ENUM_BASE {
  QSVD_OK = 0,
  QSVD_ERR_INVALID = -1,      /* bad shape, pointer, alignment or argument */
  QSVD_ERR_UNSUPPORTED = -2,  /* valid request this build does not implement */
  QSVD_ERR_WORKSPACE = -3,    /* workspace too small */
  QSVD_ERR_DEVICE = -4        /* the HIP runtime reported an error */
} qsvd_status_t;

/*
 * Rotate-and-quantise rows (QSVD paper notes, "Key design", quantisation
 * scheme: X is rotated by H1 before the int8 activation quantiser and the
 * latent C by H2 before it is cached; W8A8 / W8A4 in "Main results").
 *
 *   in      [M][n] rows, in_dtype F32 or BF16.
 *   hadamard_block  0: no rotation;  128: y = x blockdiag(H_128)^T with
 *           H_128[i][j] = (-1)^popcount(i&j) / sqrt(128), evaluated as a fast
 *           Walsh-Hadamard transform in float32 with the stage order
 *           h = 1, 2, 4, ..., 64 ((a, b) -> (a + b, a - b) for each pair
 *           (j, j + h), j & h == 0), then a multiply by float32(1/sqrt(128)).
 *   code_dtype  I8 (qmax 127) or I4 (qmax 7).
 *   group   0: one scale per row;  128: one scale per row and 128-column group.
 *   codes   I8: int8 [M][n];  I4: uint8 [M][n/2] packed.
 *   scales  float32 [M] (group 0) or [M][n/128] (group 128).
 *   Per group: amax = max|y|, s = float32(amax / qmax),
 *   code = clamp(round_half_even(float32(y / s)), -qmax, qmax); amax == 0
 *   gives s = 0 and zero codes.  M == 0 is a no-op.
 *   Constraints: n % 8 == 0; n % 128 == 0 when hadamard_block or group is
 *   128; n <= 8192.
 */
qsvd_status_t qsvd_quantize_latent(const void *in, qsvd_dtype_t in_dtype, int64_t M, int32_t n,
                                   int32_t hadamard_block, qsvd_dtype_t code_dtype, int32_t group,
                                   void *codes, float *scales, void *hip_stream);

/*
 * Shared down-projection C = X W^d (QSVD paper notes, "Key design": C_qkv is
 * computed once per token from one read of X; QSVD digest, "Key
 * Contributions").  The same call rebuilds K and V from quantised latents
 * ([K | V] = C [W^u_k | W^u_v]) when E is read as the latent width r and r
 * as the output width.
 *
 *   X          [M][E]  I8 codes with x_scale float32 [M]; or I4 codes packed
 *              two per byte ([M][E/2], element 2j in the low nibble of byte
 *              j, as qsvd_quantize_latent writes them) with x_scale [M]; or
 *              BF16 (x_scale NULL).
 *   W_packed   [r][E]  the weight W^d (E x r) stored transposed, i.e. each
 *              output column contiguous along E ([r][E/2] packed for I4);
 *              see qsvd_pack_weight.  w_dtype must equal x_dtype.
 *   col_scale  float32 [r] per-output-column weight scale, or NULL (= 1).
 *              Sigma_r^beta is folded into W^d before its quantisation.
 *   C          [M][r]  F32 or BF16.
 *   int8 and int4 (W4A4, QSVD paper notes "Main results"):
 *          acc = sum_k X[m][k] W[k][n] (exact int32);
 *          C[m][n] = float32(float32(float32(acc) * x_scale[m]) * col_scale[n]).
 *   bf16:  C[m][n] = (sum_k X[m][k] W[k][n]) * col_scale[n], float32 accumulation.
 *   Constraints: E % 64 == 0 (E % 128 == 0 for I4), r % 16 == 0, M >= 0
 *   (M == 0 is a no-op).
 */
qsvd_status_t qsvd_project(const void *X, qsvd_dtype_t x_dtype, const float *x_scale, int64_t M,
                           int32_t E, const void *W_packed, qsvd_dtype_t w_dtype,
                           const float *col_scale, int32_t r, void *C, qsvd_dtype_t c_dtype,
                           void *hip_stream);

/*
 * Transpose a weight [rows][cols] -> [cols][rows] (the W_packed layout of
 * qsvd_project).  dt: F32, BF16 or I8.  For I4, W holds int8 codes in
 * [-8, 7] (one per byte, [rows][cols], rows even) and packed receives
 * [cols][rows / 2] with codes k and k + 1 of a column in the low and high
 * nibble of one byte.  Offline, not on the hot path.
 */
qsvd_status_t qsvd_pack_weight(const void *W, qsvd_dtype_t dt, int32_t rows, int32_t cols,
                               void *packed, void *hip_stream);

/*
 * One decode step of latent attention (QSVD paper notes, "Key design": only
 * C_qkv is cached, K = C W^u_k and V = C W^u_v are rebuilt on demand; QSVD
 * digest, "Method, Step 1").  For every sequence b and head h:
 *
 *   K_h = C_b W^u_k[:, h d:(h+1) d],  V_h = C_b W^u_v[:, h d:(h+1) d]
 *   O[b][h] = softmax(softmax_scale * K_h q[b][h]) V_h
 *
 * The library evaluates it in the latent space (q~_h = softmax_scale W^u_k,h q_h,
 * scores C q~_h, O~_h = p^T C, O_h = O~_h W^u_v,h), streaming each sequence's
 * cache once for all heads in L-splits with an online softmax and a
 * log-sum-exp merge across splits (the WSVD digest, "Method, 3.4", describes
 * a fused flash-decoding kernel that folds the value up-projection into the
 * output side in the same way).
 *
 *   q        [b][heads][d]        F32 or BF16 (q_dtype)
 *   C        [b][L][r]            F32, BF16, I8 ([b][L][r] codes) or I4
 *                                 ([b][L][r/2] packed)
 *   c_scales I8: float32 [b][L];  I4: float32 [b][L][r/c_group];  else NULL
 *   c_group  I4: 128;  otherwise 0
 *   Wu_k, Wu_v  [r][E] (E = heads d), wu_dtype F32, BF16 or I8; for I8 the
 *            float32 per-column scales wu_scale_k / wu_scale_v [E], else NULL.
 *   O        [b][heads][d]        F32 or BF16 (o_dtype)
 *   splits   number of L-splits per sequence; 0 lets the library choose.
 *            BF16 caches with 33..64 heads and r = 256 k (7 <= k <= 9), whose
 *            per-head state would not fit one workgroup, run as two passes
 *            (all-head scores to the workspace, then the value product per
 *            256-column chunk); they choose their own chunking and ignore
 *            splits.
 *   workspace   device scratch of at least qsvd_decode_workspace_bytes(...)
 *            bytes (same b, L, r, heads, d, c_dtype and splits).
 *
 *   Supported combinations:
 *     F32  : q, C, W^u, O all F32 (float32 arithmetic throughout).
 *     BF16 : q, C, W^u BF16; O BF16 or F32 (bf16 MFMA, float32 accumulation).
 *     I4/I8: q BF16, W^u BF16 or I8; O BF16 or F32.
 *   Constraints: E == heads * d, heads <= 256, L >= 1, 1 <= b <= 65535;
 *   F32: 1 <= r <= 4096;  other caches: the latent columns are split over W
 *   wavefronts of r / W columns each, W the largest of 8, 7, ..., 1 with
 *   r % (W g) == 0 for the load granule g (BF16: 32 columns, I8: 64, I4: 128),
 *   and r / W must be at most 384 (so r <= 3072; e.g. 768, 1536, 2304 and
 *   3072 qualify for all three formats, 2560 not for I4).
 *   qsvd_decode_workspace_bytes returns 0 for a width that does not qualify.
 *   d is 64 or 128
 *   (QSVD_ERR_UNSUPPORTED otherwise).
 */
size_t qsvd_decode_workspace_bytes(int32_t b, int64_t L, int32_t r, int32_t heads, int32_t d,
                                   qsvd_dtype_t c_dtype, int32_t splits);

qsvd_status_t qsvd_decode_attn(const void *q, qsvd_dtype_t q_dtype, const void *C,
                               qsvd_dtype_t c_dtype, const float *c_scales, int32_t c_group,
                               const void *Wu_k, const void *Wu_v, qsvd_dtype_t wu_dtype,
                               const float *wu_scale_k, const float *wu_scale_v, int32_t b,
                               int64_t L, int32_t r, int32_t heads, int32_t d,
                               float softmax_scale, int32_t splits, void *O, qsvd_dtype_t o_dtype,
                               void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * qsvd_decode_attn_noalloc: qsvd_decode_attn without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc).  The call
 * allocates nothing: its scratch is a library-owned device array of 64 MiB
 * (one per GPU the library runs on, held until the process ends) that the
 * library locates with hipGetSymbolAddress once per device.  Arguments and
 * results are those of qsvd_decode_attn with the same kernels.
 *   Errors: as qsvd_decode_attn; QSVD_ERR_WORKSPACE when the shape needs more
 *   than 64 MiB of scratch (qsvd_decode_workspace_bytes tells how much; the
 *   7B, 13B and W8A4 decode shapes need at most about 40 MiB).
 *   Every call on one GPU uses that GPU's single scratch array: calls that
 *   overlap in time on one GPU (other streams, other threads) race and must
 *   be ordered by the caller.  Nothing in the array needs clearing between
 *   calls (each call writes every scratch value before reading it).
 */
qsvd_status_t qsvd_decode_attn_noalloc(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                       qsvd_dtype_t c_dtype, const float *c_scales, int32_t c_group,
                                       const void *Wu_k, const void *Wu_v, qsvd_dtype_t wu_dtype,
                                       const float *wu_scale_k, const float *wu_scale_v, int32_t b,
                                       int64_t L, int32_t r, int32_t heads, int32_t d,
                                       float softmax_scale, int32_t splits, void *O,
                                       qsvd_dtype_t o_dtype, void *hip_stream);

/*
 * qsvd_decode_attn_explicit: the same decode step with each head's keys and
 * values rebuilt explicitly on chip, K_h = C W^u_k,h and V_h = C W^u_v,h,
 * tile by tile (never written to memory), optionally with rotary position
 * embedding on the keys and the query.
 *
 * Passage: QSVD paper notes, "Key design" (K and V are reconstructed from the
 * cached latent on demand); WSVD digest, "Method, 3.4" and "Key
 * Contributions" (a fused flash-decoding pass reconstructs each head's keys
 * in registers, applies RoPE, and contracts with q without materialising K).
 * qsvd_decode_attn computes the same attention in the latent space (q folded
 * into W^u_k) and moves about 16x fewer MFMA operations; this entry point is
 * the literal reconstruction, and the form that stays valid with RoPE, which
 * breaks the query folding.
 *
 *   q          [b][heads][d] bf16; d must be 128.
 *   C          [b][L][r] bf16 latent cache; r a multiple of 64.
 *   Wk_packed, Wv_packed
 *              W^u_k and W^u_v TRANSPOSED, [E][r] bf16 each (qsvd_pack_weight of
 *              the [r][E] matrices), E = heads * d.
 *   rope_cos, rope_sin
 *              NULL (no rotation) or float32 tables [P][d/2] with P >= L:
 *              entry [t][i] is cos / sin of t * theta_i.  Cached latent t is
 *              the token at position t; the query sits at position L - 1 (its
 *              own latent is the last cached row).  Rotation pairs element i
 *              with element i + d/2:
 *                x'[i] = x[i] cos - x[i+d/2] sin,  x'[i+d/2] = x[i+d/2] cos + x[i] sin.
 *              V is not rotated.
 *   O          [b][heads][d], o_dtype BF16 or F32.
 *   workspace  qsvd_decode_explicit_workspace_bytes(b, L, r, heads, d) bytes
 *              (per (sequence, 256-token tile, head): max, sum and the
 *              unnormalised 128-wide output, float32).
 * Errors: QSVD_ERR_UNSUPPORTED for dtypes other than bf16 or d != 128,
 * QSVD_ERR_INVALID for bad shapes / pointers / a lone RoPE table,
 * QSVD_ERR_WORKSPACE for a short workspace.  Nothing is launched on error.
 */
size_t qsvd_decode_explicit_workspace_bytes(int32_t b, int64_t L, int32_t r, int32_t heads,
                                            int32_t d);

qsvd_status_t qsvd_decode_attn_explicit(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                        qsvd_dtype_t c_dtype, const void *Wk_packed,
                                        const void *Wv_packed, qsvd_dtype_t wu_dtype, int32_t b,
                                        int64_t L, int32_t r, int32_t heads, int32_t d,
                                        float softmax_scale, const float *rope_cos,
                                        const float *rope_sin, void *O, qsvd_dtype_t o_dtype,
                                        void *workspace, size_t workspace_bytes,
                                        void *hip_stream);

/*
 * qsvd_decode_attn_headwise: decode over per-head latents.  Each head h has
 * its own factors W_Kh = A_Kh B_Kh and W_Vh = A_Vh B_Vh, and the cache holds
 * the per-head latents C_Kh = X A_Kh (rk values per token) and C_Vh = X A_Vh
 * (rv values).  For every sequence and head:
 *   K_h = C_Kh B_Kh (rebuilt tile by tile on chip, never written out),
 *   s_t = softmax_scale * rope(K_h[t], t) . rope(q_h, L - 1),
 *   o_h = (softmax(s)^T C_Vh) B_Vh   (B_Vh applied once, after the softmax).
 *
 * Passage: WSVD digest, "Method, 3.1" (per-head low-rank factors and
 * per-head latent caches) and "Method, 3.4" (the fused flash-decoding pass:
 * latent tiles streamed on chip, K rebuilt in registers with RoPE, B_Vh
 * folded into the output side).
 *
 *   q          [b][heads][d] bf16; d must be 128.
 *   C          [b][L][heads][rk + rv] bf16: per token and head, the key latent
 *              (rk values) followed by the value latent (rv values).
 *   BK_t       [heads][d][rk] bf16: B_Kh transposed (contiguous along the latent).
 *   BV         [heads][rv][d] bf16: B_Vh as is.
 *   rk, rv     each 32, 64, 96 or 128.
 *   rope_cos, rope_sin
 *              NULL (no rotation) or float32 tables [P][d/2], P >= L, with the
 *              same meaning and rotation as in qsvd_decode_attn_explicit
 *              (cached token t at position t, the query at L - 1).  Rotations
 *              are composed: a 32-token tile starting at t0 reads row t0 and
 *              the rows 0 .. 31, so row t must be the rotation by t * theta_i
 *              (angles linear in the position, as in RoPE with any base or a
 *              linearly scaled theta).
 *   splits     L-splits per sequence (0: a default that fills the device;
 *              at most 1024, clipped to the number of 32-token tiles).
 *   O          [b][heads][d], o_dtype BF16 or F32.
 *   workspace  qsvd_decode_headwise_workspace_bytes(...) bytes, 16-byte aligned
 *              (per (sequence, split, head): running max, sum and the
 *              rv-wide unnormalised softmax(s)^T C_Vh, float32).
 * All pointers are device memory owned by the caller and 16-byte aligned.
 * Errors: QSVD_ERR_UNSUPPORTED for dtypes other than bf16, d != 128 or a rank
 * outside {32, 64, 96, 128}; QSVD_ERR_INVALID for bad shapes / pointers / a
 * lone RoPE table; QSVD_ERR_WORKSPACE for a short workspace.  Nothing is
 * launched on error; the workspace size query returns 0 for invalid shapes.
 */
size_t qsvd_decode_headwise_workspace_bytes(int32_t b, int64_t L, int32_t heads, int32_t d,
                                            int32_t rk, int32_t rv, int32_t splits);

qsvd_status_t qsvd_decode_attn_headwise(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                        qsvd_dtype_t c_dtype, const void *BK_t, const void *BV,
                                        qsvd_dtype_t b_dtype, int32_t b, int64_t L, int32_t heads,
                                        int32_t d, int32_t rk, int32_t rv, float softmax_scale,
                                        const float *rope_cos, const float *rope_sin,
                                        int32_t splits, void *O, qsvd_dtype_t o_dtype,
                                        void *workspace, size_t workspace_bytes,
                                        void *hip_stream);

/* The split count qsvd_decode_attn uses when called with splits == 0. */
int32_t qsvd_decode_default_splits(int32_t b, int64_t L, int32_t r, int32_t heads, int32_t d,
                                   qsvd_dtype_t c_dtype);

/* Static text for a status code. */
const char *qsvd_status_string(qsvd_status_t s);

/* Detail of the last failing call on this thread ("" if none). */
const char *qsvd_last_error(void);

/*
 * Optional per-kernel timing on the calling thread.  Between
 * qsvd_timing_begin and qsvd_timing_end the library records one HIP event on
 * the launch stream just before every kernel it launches from this thread (a
 * launch boundary).  A launch's time is the span from its boundary to the
 * next boundary on the same stream, or to a closing event qsvd_timing_end
 * records on that stream, so the times of a stream's launches add up to the
 * session's span on it (idle gaps between launches are counted in the launch
 * before the gap).  qsvd_timing_end waits for the closing events and returns,
 * per kernel name, the launch count and the summed time.  max_launches bounds
 * the session (extra launches are not timed).
 */
typedef struct qsvd_kernel_time {
  char name[32];
  int32_t launches;
  double total_ms;
} qsvd_kernel_time_t;

qsvd_status_t qsvd_timing_begin(int32_t max_launches);
qsvd_status_t qsvd_timing_end(qsvd_kernel_time_t *out, int32_t max_out, int32_t *n_out);

#ifdef __cplusplus
}
#endif

#endif /* QSVD_H */
