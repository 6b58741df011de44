// Host side of the C ABI: argument validation (before any HIP call), dispatch
// to the kernel launchers, error mapping and the optional timing session.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "qsvd_internal.h"

namespace {

thread_local std::string g_last_error;

qsvd_status_t fail(qsvd_status_t s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

qsvd_status_t ok() {
  g_last_error.clear();
  return QSVD_OK;
}

qsvd_status_t device_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(QSVD_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

const char *dtype_name(int dt) {
  switch (dt) {
    case QSVD_F32: return "F32";
    case QSVD_BF16: return "BF16";
    case QSVD_I8: return "I8";
    case QSVD_I4: return "I4";
    default: return "?";
  }
}

// ---------------------------------------------------------------- timing session
// One event is recorded on the launch stream just before each timed launch
// (a launch boundary).  A launch's time is the span from its boundary to the
// next boundary on the same stream (or to the closing event qsvd_timing_end
// records there), so the launch times of a stream add up to the whole span of
// the session on it, idle gaps included, and each launch costs one marker.
struct TimingRecord {
  const char *name;
  hipEvent_t start;
  hipStream_t stream;
};

struct TimingSession {
  bool active = false;
  int max_launches = 0;
  std::vector<hipEvent_t> pool;
  std::vector<TimingRecord> records;
};

thread_local TimingSession g_timing;

}  // namespace

namespace qsvd {

LaunchTimer::LaunchTimer(const char *name, hipStream_t stream) {
  TimingSession &t = g_timing;
  if (!t.active || static_cast<int>(t.records.size()) >= t.max_launches) return;
  TimingRecord rec{name, t.pool[t.records.size()], stream};
  if (hipEventRecord(rec.start, stream) != hipSuccess) return;
  t.records.push_back(rec);
}

hipError_t set_dynamic_lds(const void *kernel, size_t bytes) {
  struct Entry {
    const void *fn;
    int device;
    size_t bytes;
  };
  thread_local std::vector<Entry> done;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return e;
  Entry *hit = nullptr;
  for (Entry &x : done)
    if (x.fn == kernel && x.device == device) hit = &x;
  if (hit && hit->bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e != hipSuccess) return e;
  if (hit)
    hit->bytes = bytes;
  else
    done.push_back(Entry{kernel, device, bytes});
  return hipSuccess;
}

qsvd_status_t report(qsvd_status_t s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

}  // namespace qsvd

extern "C" {

const char *qsvd_status_string(qsvd_status_t s) {
  switch (s) {
    case QSVD_OK: return "QSVD_OK";
    case QSVD_ERR_INVALID: return "QSVD_ERR_INVALID: invalid argument";
    case QSVD_ERR_UNSUPPORTED: return "QSVD_ERR_UNSUPPORTED: unsupported combination";
    case QSVD_ERR_WORKSPACE: return "QSVD_ERR_WORKSPACE: workspace too small";
    case QSVD_ERR_DEVICE: return "QSVD_ERR_DEVICE: HIP runtime error";
    default: return "QSVD: unknown status";
  }
}

const char *qsvd_last_error(void) { return g_last_error.c_str(); }

qsvd_status_t qsvd_quantize_latent(const void *in, qsvd_dtype_t in_dtype, int64_t M, int32_t n,
                                   int32_t hadamard_block, qsvd_dtype_t code_dtype, int32_t group,
                                   void *codes, float *scales, void *hip_stream) {
  if (in_dtype != QSVD_F32 && in_dtype != QSVD_BF16)
    return fail(QSVD_ERR_INVALID, "quantize_latent: in_dtype %s (F32 or BF16)", dtype_name(in_dtype));
  if (code_dtype != QSVD_I8 && code_dtype != QSVD_I4)
    return fail(QSVD_ERR_INVALID, "quantize_latent: code_dtype %s (I8 or I4)", dtype_name(code_dtype));
  if (hadamard_block != 0 && hadamard_block != 128)
    return fail(QSVD_ERR_UNSUPPORTED, "quantize_latent: hadamard_block %d (0 or 128)", hadamard_block);
  if (group != 0 && group != 128)
    return fail(QSVD_ERR_UNSUPPORTED, "quantize_latent: group %d (0 or 128)", group);
  if (M < 0) return fail(QSVD_ERR_INVALID, "quantize_latent: M = %lld < 0", (long long)M);
  if (n <= 0 || n % 8 != 0 || n > 8192)
    return fail(QSVD_ERR_INVALID, "quantize_latent: n = %d (positive, multiple of 8, <= 8192)", n);
  if ((hadamard_block || group) && n % 128 != 0)
    return fail(QSVD_ERR_INVALID, "quantize_latent: n = %d must be a multiple of 128", n);
  if (M > (int64_t)0x7FFFFFFF * 4)
    return fail(QSVD_ERR_INVALID, "quantize_latent: M = %lld too large", (long long)M);
  if (M == 0) return ok();
  if (!in || !codes || !scales) return fail(QSVD_ERR_INVALID, "quantize_latent: NULL pointer");
  if (!aligned16(in) || !aligned16(codes) || !aligned4(scales))
    return fail(QSVD_ERR_INVALID, "quantize_latent: misaligned pointer");
  const hipError_t e = qsvd::launch_rotate_quant(
      in, in_dtype == QSVD_BF16, M, n, hadamard_block == 128, code_dtype == QSVD_I4, group == 128,
      codes, scales, static_cast<hipStream_t>(hip_stream));
  return device_status(e, "quantize_latent");
}

qsvd_status_t qsvd_project(const void *X, qsvd_dtype_t x_dtype, const float *x_scale, int64_t M,
                           int32_t E, const void *W_packed, qsvd_dtype_t w_dtype,
                           const float *col_scale, int32_t r, void *C, qsvd_dtype_t c_dtype,
                           void *hip_stream) {
  if (x_dtype != QSVD_I8 && x_dtype != QSVD_I4 && x_dtype != QSVD_BF16)
    return fail(QSVD_ERR_UNSUPPORTED, "project: x_dtype %s (I8, I4 or BF16)", dtype_name(x_dtype));
  if (w_dtype != x_dtype)
    return fail(QSVD_ERR_UNSUPPORTED, "project: w_dtype %s must equal x_dtype %s",
                dtype_name(w_dtype), dtype_name(x_dtype));
  if (c_dtype != QSVD_F32 && c_dtype != QSVD_BF16)
    return fail(QSVD_ERR_INVALID, "project: c_dtype %s (F32 or BF16)", dtype_name(c_dtype));
  if (M < 0) return fail(QSVD_ERR_INVALID, "project: M = %lld < 0", (long long)M);
  if (E <= 0 || E % 64 != 0)
    return fail(QSVD_ERR_INVALID, "project: E = %d (positive multiple of 64)", E);
  if (r <= 0 || r % 16 != 0)
    return fail(QSVD_ERR_INVALID, "project: r = %d (positive multiple of 16)", r);
  if (x_dtype == QSVD_I4 && E % 128 != 0)
    return fail(QSVD_ERR_INVALID, "project: int4 operands need E %% 128 == 0 (E = %d)", E);
  if ((x_dtype == QSVD_I8 || x_dtype == QSVD_I4) && !x_scale)
    return fail(QSVD_ERR_INVALID, "project: integer X needs x_scale");
  if (x_dtype == QSVD_BF16 && x_scale)
    return fail(QSVD_ERR_INVALID, "project: bf16 X takes no x_scale");
  if (M == 0) return ok();
  if (!X || !W_packed || !C) return fail(QSVD_ERR_INVALID, "project: NULL pointer");
  if (!aligned16(X) || !aligned16(W_packed) || !aligned16(C) ||
      (x_scale && !aligned4(x_scale)) || (col_scale && !aligned4(col_scale)))
    return fail(QSVD_ERR_INVALID, "project: misaligned pointer");
  const int64_t tiles = ((M + 127) / 128) * ((r + 127) / 128);
  if (tiles > 0x7FFFFFFF) return fail(QSVD_ERR_INVALID, "project: problem too large");
  const int kind = x_dtype == QSVD_I4 ? qsvd::kGemmI4 : (x_dtype == QSVD_I8 ? qsvd::kGemmI8 : qsvd::kGemmBF16);
  const hipError_t e = qsvd::launch_gemm(X, x_scale, kind, M, E, W_packed, col_scale,
                                         r, C, c_dtype == QSVD_BF16,
                                         static_cast<hipStream_t>(hip_stream));
  return device_status(e, "project");
}

qsvd_status_t qsvd_pack_weight(const void *W, qsvd_dtype_t dt, int32_t rows, int32_t cols,
                               void *packed, void *hip_stream) {
  int esz;
  switch (dt) {
    case QSVD_F32: esz = 4; break;
    case QSVD_BF16: esz = 2; break;
    case QSVD_I8: esz = 1; break;
    case QSVD_I4: esz = 0; break;
    default: return fail(QSVD_ERR_INVALID, "pack_weight: dtype %s", dtype_name(dt));
  }
  if (rows < 0 || cols < 0) return fail(QSVD_ERR_INVALID, "pack_weight: negative shape");
  if (dt == QSVD_I4 && rows % 2 != 0)
    return fail(QSVD_ERR_INVALID, "pack_weight: I4 needs an even row count (rows = %d)", rows);
  if (rows == 0 || cols == 0) return ok();
  if (!W || !packed) return fail(QSVD_ERR_INVALID, "pack_weight: NULL pointer");
  if (dt == QSVD_I4)
    return device_status(qsvd::launch_pack_int4(W, rows, cols, packed,
                                                static_cast<hipStream_t>(hip_stream)),
                         "pack_weight");
  return device_status(qsvd::launch_transpose(W, esz, rows, cols, packed,
                                              static_cast<hipStream_t>(hip_stream)),
                       "pack_weight");
}

static qsvd_status_t validate_decode_shape(int32_t b, int64_t L, int32_t r, int32_t heads,
                                           int32_t d, qsvd_dtype_t c_dtype, int32_t splits) {
  // b <= 65535: the absorb, merge and float32 stream launches put the batch in a grid dimension
  if (b < 1 || b > 65535) return fail(QSVD_ERR_INVALID, "decode: b = %d (1..65535)", b);
  if (L < 1) return fail(QSVD_ERR_INVALID, "decode: L = %lld < 1", (long long)L);
  if (heads < 1 || heads > 256) return fail(QSVD_ERR_INVALID, "decode: heads = %d (1..256)", heads);
  if (d != 64 && d != 128) return fail(QSVD_ERR_UNSUPPORTED, "decode: d = %d (64 or 128)", d);
  if (splits < 0) return fail(QSVD_ERR_INVALID, "decode: splits = %d < 0", splits);
  if (c_dtype == QSVD_F32) {
    if (r < 1 || r > 4096) return fail(QSVD_ERR_UNSUPPORTED, "decode: F32 cache needs 1 <= r <= 4096");
  } else if (c_dtype == QSVD_BF16 || c_dtype == QSVD_I8 || c_dtype == QSVD_I4) {
    if (r < 32 || r % 32 != 0)
      return fail(QSVD_ERR_INVALID, "decode: r = %d must be a positive multiple of 32", r);
    if (c_dtype == QSVD_I4 && r % 128 != 0)
      return fail(QSVD_ERR_INVALID, "decode: int4 cache needs r %% 128 == 0 (r = %d)", r);
    if (!qsvd::mfma_shape(r, heads, c_dtype, nullptr))
      return fail(QSVD_ERR_UNSUPPORTED,
                  "decode: r = %d has no stream-kernel shape (r = W * 32 * k, W <= 8, k <= 12)", r);
  } else {
    return fail(QSVD_ERR_INVALID, "decode: c_dtype %s", dtype_name(c_dtype));
  }
  if (L > (int64_t(1) << 40) / b)   // b * L <= 2^40, without overflow
    return fail(QSVD_ERR_INVALID, "decode: b * L too large");
  return QSVD_OK;
}

size_t qsvd_decode_workspace_bytes(int32_t b, int64_t L, int32_t r, int32_t heads, int32_t d,
                                   qsvd_dtype_t c_dtype, int32_t splits) {
  if (validate_decode_shape(b, L, r, heads, d, c_dtype, splits) != QSVD_OK) return 0;
  return qsvd::plan_decode(b, L, r, heads, d, c_dtype, splits).total;
}

int32_t qsvd_decode_default_splits(int32_t b, int64_t L, int32_t r, int32_t heads, int32_t d,
                                   qsvd_dtype_t c_dtype) {
  if (validate_decode_shape(b, L, r, heads, d, c_dtype, 0) != QSVD_OK) return 0;
  return qsvd::plan_decode(b, L, r, heads, d, c_dtype, 0).splits;
}

static qsvd_status_t validate_explicit_shape(int32_t b, int64_t L, int32_t r, int32_t heads,
                                             int32_t d) {
  if (b < 1) return fail(QSVD_ERR_INVALID, "decode_explicit: b = %d < 1", b);
  if (L < 1) return fail(QSVD_ERR_INVALID, "decode_explicit: L = %lld < 1", (long long)L);
  if (heads < 1 || heads > 256) return fail(QSVD_ERR_INVALID, "decode_explicit: heads = %d (1..256)", heads);
  if (d != 128) return fail(QSVD_ERR_UNSUPPORTED, "decode_explicit: d = %d (128)", d);
  if (r < 64 || r % 64 != 0 || r > 16384)
    return fail(QSVD_ERR_INVALID, "decode_explicit: r = %d (a multiple of 64, 64..16384)", r);
  if (L > (int64_t(1) << 36) / b)   // b * L <= 2^36, without overflow
    return fail(QSVD_ERR_INVALID, "decode_explicit: b * L too large");
  // one workgroup per (sequence, 256-token tile, head), tiles padded to groups
  // of 8 (a 1-D launch)
  const int64_t groups = ((L + 255) / 256 + 7) / 8;
  if (static_cast<int64_t>(b) * heads * groups * 8 > 0x7FFFFFFF)
    return fail(QSVD_ERR_INVALID, "decode_explicit: b * heads * L / 256 too large for one launch");
  return QSVD_OK;
}

size_t qsvd_decode_explicit_workspace_bytes(int32_t b, int64_t L, int32_t r, int32_t heads,
                                            int32_t d) {
  if (validate_explicit_shape(b, L, r, heads, d) != QSVD_OK) return 0;
  return qsvd::explicit_workspace_bytes(b, L, heads);
}

qsvd_status_t qsvd_decode_attn_explicit(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                        qsvd_dtype_t c_dtype, const void *Wk_packed,
                                        const void *Wv_packed, qsvd_dtype_t wu_dtype, int32_t b,
                                        int64_t L, int32_t r, int32_t heads, int32_t d,
                                        float softmax_scale, const float *rope_cos,
                                        const float *rope_sin, void *O, qsvd_dtype_t o_dtype,
                                        void *workspace, size_t workspace_bytes,
                                        void *hip_stream) {
  qsvd_status_t st = validate_explicit_shape(b, L, r, heads, d);
  if (st != QSVD_OK) return st;
  if (q_dtype != QSVD_BF16 || c_dtype != QSVD_BF16 || wu_dtype != QSVD_BF16)
    return fail(QSVD_ERR_UNSUPPORTED, "decode_explicit: q, C and W^u must be BF16");
  if (o_dtype != QSVD_BF16 && o_dtype != QSVD_F32)
    return fail(QSVD_ERR_INVALID, "decode_explicit: o_dtype %s", dtype_name(o_dtype));
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(QSVD_ERR_INVALID, "decode_explicit: softmax_scale must be positive and finite");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(QSVD_ERR_INVALID, "decode_explicit: rope_cos and rope_sin go together");
  if (!q || !C || !Wk_packed || !Wv_packed || !O)
    return fail(QSVD_ERR_INVALID, "decode_explicit: NULL pointer");
  if (!aligned16(q) || !aligned16(C) || !aligned16(Wk_packed) || !aligned16(Wv_packed) ||
      !aligned16(O) || (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) ||
      (workspace && !aligned16(workspace)))
    return fail(QSVD_ERR_INVALID, "decode_explicit: misaligned pointer");
  const size_t need = qsvd::explicit_workspace_bytes(b, L, heads);
  if (!workspace || workspace_bytes < need)
    return fail(QSVD_ERR_WORKSPACE, "decode_explicit: workspace %zu bytes, need %zu",
                workspace_bytes, need);
  qsvd::ExplicitArgs a{};
  a.q = q;
  a.C = C;
  a.Wk_t = Wk_packed;
  a.Wv_t = Wv_packed;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.b = b;
  a.L = L;
  a.r = r;
  a.heads = heads;
  a.softmax_scale = softmax_scale;
  a.O = O;
  a.o_dtype = o_dtype;
  a.workspace = workspace;
  return device_status(qsvd::launch_decode_explicit(a, static_cast<hipStream_t>(hip_stream)),
                       "decode_attn_explicit");
}

static qsvd_status_t validate_headwise_shape(int32_t b, int64_t L, int32_t heads, int32_t d,
                                             int32_t rk, int32_t rv, int32_t splits) {
  if (b < 1) return fail(QSVD_ERR_INVALID, "decode_headwise: b = %d < 1", b);
  if (L < 1) return fail(QSVD_ERR_INVALID, "decode_headwise: L = %lld < 1", (long long)L);
  if (heads < 1 || heads > 256)
    return fail(QSVD_ERR_INVALID, "decode_headwise: heads = %d (1..256)", heads);
  if (d != 128) return fail(QSVD_ERR_UNSUPPORTED, "decode_headwise: d = %d (128)", d);
  if (rk < 32 || rk > 128 || rk % 32 != 0 || rv < 32 || rv > 128 || rv % 32 != 0)
    return fail(QSVD_ERR_UNSUPPORTED, "decode_headwise: rk = %d, rv = %d (each 32, 64, 96 or 128)",
                rk, rv);
  if (splits < 0 || splits > 1024)
    return fail(QSVD_ERR_INVALID, "decode_headwise: splits = %d (0..1024)", splits);
  if (L > (int64_t(1) << 36) / b)   // b * L <= 2^36, without overflow
    return fail(QSVD_ERR_INVALID, "decode_headwise: b * L too large");
  const int64_t grid = static_cast<int64_t>(b) * qsvd::headwise_splits(b, L, heads, splits) *
                       ((heads + 3) / 4);
  if (grid >= (int64_t(1) << 31)) return fail(QSVD_ERR_INVALID, "decode_headwise: b too large");
  return QSVD_OK;
}

size_t qsvd_decode_headwise_workspace_bytes(int32_t b, int64_t L, int32_t heads, int32_t d,
                                            int32_t rk, int32_t rv, int32_t splits) {
  if (validate_headwise_shape(b, L, heads, d, rk, rv, splits) != QSVD_OK) return 0;
  return qsvd::headwise_workspace_bytes(b, L, heads, rv, splits);
}

qsvd_status_t qsvd_decode_attn_headwise(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                        qsvd_dtype_t c_dtype, const void *BK_t, const void *BV,
                                        qsvd_dtype_t b_dtype, int32_t b, int64_t L, int32_t heads,
                                        int32_t d, int32_t rk, int32_t rv, float softmax_scale,
                                        const float *rope_cos, const float *rope_sin,
                                        int32_t splits, void *O, qsvd_dtype_t o_dtype,
                                        void *workspace, size_t workspace_bytes,
                                        void *hip_stream) {
  qsvd_status_t st = validate_headwise_shape(b, L, heads, d, rk, rv, splits);
  if (st != QSVD_OK) return st;
  if (q_dtype != QSVD_BF16 || c_dtype != QSVD_BF16 || b_dtype != QSVD_BF16)
    return fail(QSVD_ERR_UNSUPPORTED, "decode_headwise: q, C and B_K / B_V must be BF16");
  if (o_dtype != QSVD_BF16 && o_dtype != QSVD_F32)
    return fail(QSVD_ERR_INVALID, "decode_headwise: o_dtype %s", dtype_name(o_dtype));
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(QSVD_ERR_INVALID, "decode_headwise: softmax_scale must be positive and finite");
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(QSVD_ERR_INVALID, "decode_headwise: rope_cos and rope_sin go together");
  if (!q || !C || !BK_t || !BV || !O) return fail(QSVD_ERR_INVALID, "decode_headwise: NULL pointer");
  if (!aligned16(q) || !aligned16(C) || !aligned16(BK_t) || !aligned16(BV) || !aligned16(O) ||
      (rope_cos && (!aligned16(rope_cos) || !aligned16(rope_sin))) ||
      (workspace && !aligned16(workspace)))
    return fail(QSVD_ERR_INVALID, "decode_headwise: misaligned pointer");
  const size_t need = qsvd::headwise_workspace_bytes(b, L, heads, rv, splits);
  if (!workspace || workspace_bytes < need)
    return fail(QSVD_ERR_WORKSPACE, "decode_headwise: workspace %zu bytes, need %zu",
                workspace_bytes, need);
  qsvd::HeadwiseArgs a{};
  a.q = q;
  a.C = C;
  a.BK_t = BK_t;
  a.BV = BV;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.b = b;
  a.L = L;
  a.heads = heads;
  a.rk = rk;
  a.rv = rv;
  a.splits = splits;
  a.softmax_scale = softmax_scale;
  a.O = O;
  a.o_dtype = o_dtype;
  a.workspace = workspace;
  return device_status(qsvd::launch_decode_headwise(a, static_cast<hipStream_t>(hip_stream)),
                       "decode_attn_headwise");
}

qsvd_status_t qsvd_decode_attn(const void *q, qsvd_dtype_t q_dtype, const void *C,
                               qsvd_dtype_t c_dtype, const float *c_scales, int32_t c_group,
                               const void *Wu_k, const void *Wu_v, qsvd_dtype_t wu_dtype,
                               const float *wu_scale_k, const float *wu_scale_v, int32_t b,
                               int64_t L, int32_t r, int32_t heads, int32_t d,
                               float softmax_scale, int32_t splits, void *O, qsvd_dtype_t o_dtype,
                               void *workspace, size_t workspace_bytes, void *hip_stream) {
  return qsvd::decode_attn_checked(q, q_dtype, C, c_dtype, c_scales, c_group, Wu_k, Wu_v, wu_dtype,
                                   wu_scale_k, wu_scale_v, b, L, r, heads, d, softmax_scale, splits,
                                   O, o_dtype, workspace, workspace_bytes, hip_stream, nullptr);
}


qsvd_status_t qsvd_timing_begin(int32_t max_launches) {
  TimingSession &t = g_timing;
  if (t.active) return fail(QSVD_ERR_INVALID, "timing_begin: a session is already active");
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(QSVD_ERR_INVALID, "timing_begin: max_launches = %d", max_launches);
  t.pool.resize(static_cast<size_t>(max_launches));
  for (auto &ev : t.pool) {
    const hipError_t e = hipEventCreate(&ev);
    if (e != hipSuccess) return device_status(e, "timing_begin");
  }
  t.records.clear();
  t.records.reserve(max_launches);
  t.max_launches = max_launches;
  t.active = true;
  return ok();
}

qsvd_status_t qsvd_timing_end(qsvd_kernel_time_t *out, int32_t max_out, int32_t *n_out) {
  TimingSession &t = g_timing;
  if (!t.active) return fail(QSVD_ERR_INVALID, "timing_end: no active session");
  t.active = false;
  hipError_t err = hipSuccess;
  // closing boundary on every stream that has timed launches
  std::vector<std::pair<hipStream_t, hipEvent_t>> closing;
  for (const auto &rec : t.records) {
    bool seen = false;
    for (auto &c : closing) seen = seen || c.first == rec.stream;
    if (seen) continue;
    hipEvent_t ev = nullptr;
    err = hipEventCreate(&ev);
    if (err == hipSuccess) err = hipEventRecord(ev, rec.stream);
    if (err == hipSuccess) err = hipEventSynchronize(ev);
    if (ev) closing.push_back({rec.stream, ev});
    if (err != hipSuccess) break;
  }
  std::vector<qsvd_kernel_time_t> agg;
  const size_t n_rec = t.records.size();
  for (size_t i = 0; i < n_rec && err == hipSuccess; ++i) {
    const TimingRecord &rec = t.records[i];
    hipEvent_t end = nullptr;
    for (size_t j = i + 1; j < n_rec && !end; ++j)
      if (t.records[j].stream == rec.stream) end = t.records[j].start;
    for (auto &c : closing)
      if (!end && c.first == rec.stream) end = c.second;
    float ms = 0.f;
    err = hipEventElapsedTime(&ms, rec.start, end);
    if (err != hipSuccess) break;
    qsvd_kernel_time_t *slot = nullptr;
    for (auto &a : agg)
      if (std::strncmp(a.name, rec.name, sizeof(a.name)) == 0) slot = &a;
    if (!slot) {
      qsvd_kernel_time_t k{};
      std::strncpy(k.name, rec.name, sizeof(k.name) - 1);
      agg.push_back(k);
      slot = &agg.back();
    }
    slot->launches += 1;
    slot->total_ms += ms;
  }
  for (auto &c : closing) (void)hipEventDestroy(c.second);
  for (auto &ev : t.pool) (void)hipEventDestroy(ev);
  t.pool.clear();
  t.records.clear();
  if (err != hipSuccess) return device_status(err, "timing_end");
  const int n = static_cast<int>(agg.size());
  if (n_out) *n_out = n;
  for (int i = 0; i < n && i < max_out && out; ++i) out[i] = agg[i];
  return ok();
}

}  // extern "C"

namespace qsvd {

qsvd_status_t decode_attn_checked(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                  qsvd_dtype_t c_dtype, const float *c_scales, int32_t c_group,
                                  const void *Wu_k, const void *Wu_v, qsvd_dtype_t wu_dtype,
                                  const float *wu_scale_k, const float *wu_scale_v, int32_t b,
                                  int64_t L, int32_t r, int32_t heads, int32_t d,
                                  float softmax_scale, int32_t splits, void *O, qsvd_dtype_t o_dtype,
                                  void *workspace, size_t workspace_bytes, void *hip_stream,
                                  size_t *need) {
  qsvd_status_t st = validate_decode_shape(b, L, r, heads, d, c_dtype, splits);
  if (st != QSVD_OK) return st;
  if (c_dtype == QSVD_F32) {
    if (q_dtype != QSVD_F32 || wu_dtype != QSVD_F32 || o_dtype != QSVD_F32)
      return fail(QSVD_ERR_UNSUPPORTED, "decode: F32 cache needs F32 q, W^u and O");
  } else {
    if (q_dtype != QSVD_BF16)
      return fail(QSVD_ERR_UNSUPPORTED, "decode: %s cache needs BF16 q", dtype_name(c_dtype));
    if (wu_dtype != QSVD_BF16 && wu_dtype != QSVD_I8)
      return fail(QSVD_ERR_UNSUPPORTED, "decode: W^u dtype %s (BF16 or I8)", dtype_name(wu_dtype));
    if (o_dtype != QSVD_BF16 && o_dtype != QSVD_F32)
      return fail(QSVD_ERR_INVALID, "decode: o_dtype %s", dtype_name(o_dtype));
  }
  if (c_dtype == QSVD_I4) {
    if (c_group != 128) return fail(QSVD_ERR_UNSUPPORTED, "decode: int4 cache needs c_group 128");
    if (!c_scales) return fail(QSVD_ERR_INVALID, "decode: int4 cache needs c_scales");
  } else if (c_dtype == QSVD_I8) {
    if (c_group != 0) return fail(QSVD_ERR_UNSUPPORTED, "decode: int8 cache is per token (c_group 0)");
    if (!c_scales) return fail(QSVD_ERR_INVALID, "decode: int8 cache needs c_scales");
  } else {
    if (c_scales || c_group != 0)
      return fail(QSVD_ERR_INVALID, "decode: %s cache takes no scales", dtype_name(c_dtype));
  }
  if (wu_dtype == QSVD_I8) {
    if (!wu_scale_k || !wu_scale_v)
      return fail(QSVD_ERR_INVALID, "decode: int8 W^u needs wu_scale_k and wu_scale_v");
  } else if (wu_scale_k || wu_scale_v) {
    return fail(QSVD_ERR_INVALID, "decode: %s W^u takes no scales", dtype_name(wu_dtype));
  }
  if (!(softmax_scale > 0.f) || !(softmax_scale < 1e30f))
    return fail(QSVD_ERR_INVALID, "decode: softmax_scale must be positive and finite");
  if (!q || !C || !Wu_k || !Wu_v || !O) return fail(QSVD_ERR_INVALID, "decode: NULL pointer");
  if (!aligned16(q) || !aligned16(C) || !aligned16(Wu_k) || !aligned16(Wu_v) || !aligned16(O) ||
      (c_scales && !aligned4(c_scales)) || (wu_scale_k && !aligned16(wu_scale_k)) ||
      (wu_scale_v && !aligned16(wu_scale_v)) || (workspace && !aligned16(workspace)))
    return fail(QSVD_ERR_INVALID, "decode: misaligned pointer");
  const DecodePlan plan = plan_decode(b, L, r, heads, d, c_dtype, splits);
  if (need) {
    *need = plan.total;
    if (!workspace && workspace_bytes == 0) return ok();
  }
  if (!workspace || workspace_bytes < plan.total)
    return fail(QSVD_ERR_WORKSPACE, "decode: workspace %zu bytes, need %zu", workspace_bytes,
                plan.total);
  DecodeArgs a{};
  a.q = q;
  a.q_dtype = q_dtype;
  a.C = C;
  a.c_dtype = c_dtype;
  a.c_scales = c_scales;
  a.c_group = c_group;
  a.Wu_k = Wu_k;
  a.Wu_v = Wu_v;
  a.wu_dtype = wu_dtype;
  a.wu_scale_k = wu_scale_k;
  a.wu_scale_v = wu_scale_v;
  a.b = b;
  a.L = L;
  a.r = r;
  a.heads = heads;
  a.d = d;
  a.softmax_scale = softmax_scale;
  a.splits = splits;
  a.O = O;
  a.o_dtype = o_dtype;
  a.workspace = workspace;
  return device_status(launch_decode(a, plan, static_cast<hipStream_t>(hip_stream)),
                       "decode_attn");
}

}  // namespace qsvd
