// Internal declarations shared by the host API and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "qsvd.h"

namespace qsvd {

// ---------------------------------------------------------------- timing
// Marks a kernel launch for the timing session of this thread: when a session
// is active, the constructor records the launch-boundary event on the launch
// stream (the launch follows it; see qsvd_timing_begin).
class LaunchTimer {
 public:
  LaunchTimer(const char *name, hipStream_t stream);
  LaunchTimer(const LaunchTimer &) = delete;
  LaunchTimer &operator=(const LaunchTimer &) = delete;
};

// Allow `kernel` (a __global__ function's address) `bytes` of dynamic LDS on
// the current device.  The attribute belongs to the function on each device
// and persists, so the runtime call is made once per (kernel, device, larger
// size) on each thread; later launches find it in a thread-local record.
hipError_t set_dynamic_lds(const void *kernel, size_t bytes);

// ---------------------------------------------------------------- launchers
// Each returns the HIP error of its launches (hipSuccess on success).  All
// shapes are validated by the caller.

hipError_t launch_rotate_quant(const void *in, bool in_bf16, int64_t M, int n, bool hadamard,
                               bool int4, bool grouped, void *codes, float *scales,
                               hipStream_t s);

// in_kind: operand format of A and B (bf16, int8 codes, packed int4 codes)
enum : int { kGemmBF16 = 0, kGemmI8 = 1, kGemmI4 = 2 };
hipError_t launch_gemm(const void *A, const float *a_scale, int in_kind, int64_t M, int K,
                       const void *Bt, const float *col_scale, int N, void *C, bool c_bf16,
                       hipStream_t s);

// transpose int8 codes [rows][cols] into packed int4 [cols][rows / 2]
hipError_t launch_pack_int4(const void *W, int rows, int cols, void *out, hipStream_t s);

hipError_t launch_transpose(const void *W, int elem_bytes, int rows, int cols, void *out,
                            hipStream_t s);

struct ExplicitArgs {
  const void *q;        // [b][heads][128] bf16
  const void *C;        // [b][L][r] bf16
  const void *Wk_t;     // [E][r] bf16 (W^u_k transposed)
  const void *Wv_t;     // [E][r] bf16 (W^u_v transposed)
  const float *rope_cos, *rope_sin;   // [>= L][64] each, or both NULL
  int b;
  int64_t L;
  int r, heads;
  float softmax_scale;
  void *O;
  int o_dtype;
  void *workspace;
};

size_t explicit_workspace_bytes(int b, int64_t L, int heads);
hipError_t launch_decode_explicit(const ExplicitArgs &a, hipStream_t s);

struct HeadwiseArgs {
  const void *q;        // [b][heads][128] bf16
  const void *C;        // [b][L][heads][rk + rv] bf16
  const void *BK_t;     // [heads][128][rk] bf16 (B_Kh transposed)
  const void *BV;       // [heads][rv][128] bf16
  const float *rope_cos, *rope_sin;   // [>= L][64] each, or both NULL
  int b;
  int64_t L;
  int heads, rk, rv, splits;
  float softmax_scale;
  void *O;
  int o_dtype;
  void *workspace;
};

// Splits per sequence of a per-head-latent decode (splits = 0: default).
int headwise_splits(int b, int64_t L, int heads, int splits);
size_t headwise_workspace_bytes(int b, int64_t L, int heads, int rv, int splits);
hipError_t launch_decode_headwise(const HeadwiseArgs &a, hipStream_t s);

struct DecodeArgs {
  const void *q;
  int q_dtype;
  const void *C;
  int c_dtype;
  const float *c_scales;
  int c_group;
  const void *Wu_k;
  const void *Wu_v;
  int wu_dtype;
  const float *wu_scale_k;
  const float *wu_scale_v;
  int b;
  int64_t L;
  int r;
  int heads;
  int d;
  float softmax_scale;
  int splits;
  void *O;
  int o_dtype;
  void *workspace;
};

// Two-pass decode for wide latents with many heads (bf16 caches): a score pass
// writes S[b][heads][Lp] and per-chunk maxima; a value pass writes the split
// partials in the single pass's layout for the shared merge.
struct WideArgs {
  const void *C;          // [b][L][r] bf16
  const uint16_t *qt;     // absorbed queries [b][heads][r]
  float *S;               // [b][heads][Lp]
  float *m1;              // [b][nchunk1][heads]
  uint16_t *opart;        // [b][splits][r / 64][heads][64]
  float *ml;              // [b][splits][heads][2]
  int64_t L, Lp, chunk1, chunk3;
  int b, r, heads, nchunk1, splits;
};

struct WidePlanInfo {
  int64_t chunk1;   // tokens per score-pass workgroup (multiple of 32)
  int64_t chunk3;   // tokens per value-pass split (multiple of 32)
  int64_t Lp;       // L rounded up to 32
  int nchunk1, splits, rw;
  size_t s_bytes, m1_bytes;
};

bool wide_applies(int r, int heads, int c_dtype, int head_groups);
void wide_plan(int b, int64_t L, int r, int heads, WidePlanInfo *w);
hipError_t launch_wide_scores(const WideArgs &a, hipStream_t s);
hipError_t launch_wide_values(const WideArgs &a, hipStream_t s);

// Shape of the MFMA stream kernel: W wavefronts of RW = 32 NKB latent columns
// each (r = W RW), NHB 16-head blocks per workgroup, T tokens per tile.
struct MfmaShape {
  int W, NKB, NHB, T, D;   // D: token tiles of loads in flight (quantised 64-token tiles)
};

// True when the MFMA stream kernel supports latent width r for the cache
// dtype (bf16 / int8 / int4); fills *out (if non-NULL) with its shape.
bool mfma_shape(int r, int heads, int c_dtype, MfmaShape *out);

// Workspace layout of one decode call.
struct DecodePlan {
  MfmaShape shape;   // MFMA stream kernel shape (mfma only)
  int splits;        // L-splits per sequence
  int64_t chunk;     // tokens per split (multiple of the token tile)
  int head_groups;   // workgroups per (sequence, split) along heads
  int group_heads;   // heads per head group
  bool mfma;         // bf16 / quantised MFMA stream kernel (else float32 kernel)
  bool fused;        // float32 path in one launch (small problems, library-chosen splits)
  bool wide;         // two-pass decode (score pass + value pass) instead of the stream kernel
  WidePlanInfo wp;   // its chunking (wide only)
  int rw;            // columns per partial block of the split partials
  int merge_rows;    // latent rows per merge workgroup (MFMA paths)
  int jc;            // merge chunks along r (chunk shares summed by the finalize)
  size_t qt_bytes;   // absorbed queries
  size_t part_bytes; // per-split partial state
  size_t total;
};

DecodePlan plan_decode(int b, int64_t L, int r, int heads, int d, int c_dtype, int splits);

hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &p, hipStream_t s);

// Argument validation and launch of one qsvd_decode_attn step.  With need
// non-NULL it receives the workspace size of the plan; workspace == NULL with
// workspace_bytes == 0 then validates and sizes without launching.
qsvd_status_t decode_attn_checked(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                  qsvd_dtype_t c_dtype, const float *c_scales, int32_t c_group,
                                  const void *Wu_k, const void *Wu_v, qsvd_dtype_t wu_dtype,
                                  const float *wu_scale_k, const float *wu_scale_v, int32_t b,
                                  int64_t L, int32_t r, int32_t heads, int32_t d,
                                  float softmax_scale, int32_t splits, void *O, qsvd_dtype_t o_dtype,
                                  void *workspace, size_t workspace_bytes, void *hip_stream,
                                  size_t *need);

// Record a failure message for qsvd_last_error and return s.
qsvd_status_t report(qsvd_status_t s, const char *fmt, ...);

}  // namespace qsvd
