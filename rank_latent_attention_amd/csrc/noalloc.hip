// qsvd_decode_attn_noalloc: the decode step of qsvd_decode_attn with its
// scratch (absorbed queries, split partials, merge shares) in a file-scope
// device array instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops that
// forbid allocation).  The kernels are the ones qsvd_decode_attn launches.
#include <mutex>

#include "qsvd_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB on every device the library runs on
constexpr int kMaxDevices = 64;

// One copy per device, resident until the process ends.  In host code the
// name is only a handle for hipGetSymbolAddress: kernels receive the device
// address that call returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace qsvd {

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
static qsvd_status_t scratch_address(void **out) {
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return report(QSVD_ERR_DEVICE, "decode_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (device < 0 || device >= kMaxDevices)
    return report(QSVD_ERR_UNSUPPORTED, "decode_noalloc: device %d (at most %d devices)", device, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[device]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return report(QSVD_ERR_DEVICE, "decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_ptr[device] = p;
  }
  *out = g_scratch_ptr[device];
  return QSVD_OK;
}

}  // namespace qsvd

qsvd_status_t qsvd_decode_attn_noalloc(const void *q, qsvd_dtype_t q_dtype, const void *C,
                                       qsvd_dtype_t c_dtype, const float *c_scales, int32_t c_group,
                                       const void *Wu_k, const void *Wu_v, qsvd_dtype_t wu_dtype,
                                       const float *wu_scale_k, const float *wu_scale_v, int32_t b,
                                       int64_t L, int32_t r, int32_t heads, int32_t d,
                                       float softmax_scale, int32_t splits, void *O,
                                       qsvd_dtype_t o_dtype, void *hip_stream) {
  // validate every argument and size the plan without launching
  size_t need = 0;
  qsvd_status_t st = qsvd::decode_attn_checked(q, q_dtype, C, c_dtype, c_scales, c_group, Wu_k, Wu_v,
                                               wu_dtype, wu_scale_k, wu_scale_v, b, L, r, heads, d,
                                               softmax_scale, splits, O, o_dtype, nullptr, 0,
                                               hip_stream, &need);
  if (st != QSVD_OK) return st;
  if (need > kScratchBytes)
    return qsvd::report(QSVD_ERR_WORKSPACE,
                        "decode_noalloc: this shape needs %zu bytes of scratch; the static scratch holds %zu "
                        "(use qsvd_decode_attn with a workspace)",
                        need, kScratchBytes);
  void *ws = nullptr;
  st = qsvd::scratch_address(&ws);
  if (st != QSVD_OK) return st;
  return qsvd::decode_attn_checked(q, q_dtype, C, c_dtype, c_scales, c_group, Wu_k, Wu_v, wu_dtype,
                                   wu_scale_k, wu_scale_v, b, L, r, heads, d, softmax_scale, splits, O,
                                   o_dtype, ws, kScratchBytes, hip_stream, nullptr);
}
