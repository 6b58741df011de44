// Fused block Walsh-Hadamard rotation + absmax quantiser (gfx950).
//
// QSVD paper notes (NeurIPS 2025), "Key design", quantisation scheme: the
// input X is rotated by an orthogonal H1 and the cached latent C by H2 before
// low-bit quantisation, which spreads channel outliers; the W8A8 / W8A4 rows
// of "Main results" quantise activations and latents per token.
//
// One wavefront owns one row.  Lane l holds 8 consecutive elements of every
// 512-element chunk, so a 128-wide Hadamard block lives in 16 lanes: stages
// h = 1, 2, 4 pair registers inside a lane, stages h = 8 .. 64 pair lane l with
// lane l ^ (h / 8).  The absmax is a wavefront (per token) or 16-lane (per
// 128-group) max reduction.  Float arithmetic is compiled without
// contraction, so every sum, difference, product and quotient is one IEEE
// float32 operation rounded to nearest even.
#include "device_common.h"
#include "qsvd_internal.h"

namespace qsvd {
namespace {

constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // float32(1/sqrt(128)), bits 0x3DB504F3

enum : int { kHadamard = 1, kInt4 = 2, kGrouped = 4 };

template <typename InT>
__device__ __forceinline__ void load8(const InT *p, float v[8]);

template <>
__device__ __forceinline__ void load8<float>(const float *p, float v[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float v[8]) {
  const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(a[i] << 16);
    v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
  }
}

// In-place float32 Walsh-Hadamard of one 128-block spread over 16 lanes.
__device__ __forceinline__ void fwht128(float v[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        const float a = v[i], b = v[i + h];
        v[i] = a + b;
        v[i + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __shfl_xor(v[i], m, kWave);
      v[i] = upper ? (p - v[i]) : (v[i] + p);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = v[i] * kInvSqrt128;
}

__device__ __forceinline__ int quant1(float y, float s, float qmax) {
  if (!(s > 0.f)) return 0;
  float c = rintf(y / s);
  c = fminf(fmaxf(c, -qmax), qmax);
  return static_cast<int>(c);
}

template <typename InT, int NCH>
__global__ __launch_bounds__(256) void rotate_quant_kernel(const InT *__restrict__ in, int64_t M,
                                                           int n, int flags,
                                                           uint8_t *__restrict__ codes,
                                                           float *__restrict__ scales) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform per wavefront; no workgroup barrier follows
  const bool int4 = (flags & kInt4) != 0;
  const bool grouped = (flags & kGrouped) != 0;
  const float qmax = int4 ? 7.f : 127.f;

  float v[NCH][8];
  const InT *src = in + row * static_cast<int64_t>(n);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = c * 512 + lane * 8;
    if (base < n) {
      load8<InT>(src + base, v[c]);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[c][i] = 0.f;
    }
  }
  if (flags & kHadamard) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (c * 512 < n) fwht128(v[c], lane);  // uniform: n % 128 == 0
    }
  }

  float s_row = 0.f;
  if (!grouped) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    amax = group_max<kWave>(amax);
    s_row = amax / qmax;
    if (lane == 0) scales[row] = s_row;
  }

  const int ngroups = n >> 7;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int base = c * 512 + lane * 8;
    float s = s_row;
    if (grouped) {
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
      amax = group_max<16>(amax);
      s = amax / qmax;
      if (base < n && (lane & 15) == 0) scales[row * ngroups + (base >> 7)] = s;
    }
    if (base >= n) continue;
    int q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quant1(v[c][i], s, qmax);
    if (int4) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= static_cast<uint32_t>(q[i] & 0xF) << (4 * i);
      *reinterpret_cast<uint32_t *>(codes + row * static_cast<int64_t>(n / 2) + base / 2) = w;
    } else {
      u32x2 w = {0u, 0u};
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i >> 2] |= static_cast<uint32_t>(q[i] & 0xFF) << (8 * (i & 3));
      *reinterpret_cast<u32x2 *>(codes + row * static_cast<int64_t>(n) + base) = w;
    }
  }
}

template <typename InT>
hipError_t dispatch(const InT *in, int64_t M, int n, int flags, uint8_t *codes, float *scales,
                    hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((M + 3) / 4)), block(256);
  const int nch = (n + 511) / 512;
  if (nch <= 1)
    rotate_quant_kernel<InT, 1><<<grid, block, 0, s>>>(in, M, n, flags, codes, scales);
  else if (nch <= 2)
    rotate_quant_kernel<InT, 2><<<grid, block, 0, s>>>(in, M, n, flags, codes, scales);
  else if (nch <= 4)
    rotate_quant_kernel<InT, 4><<<grid, block, 0, s>>>(in, M, n, flags, codes, scales);
  else if (nch <= 8)
    rotate_quant_kernel<InT, 8><<<grid, block, 0, s>>>(in, M, n, flags, codes, scales);
  else
    rotate_quant_kernel<InT, 16><<<grid, block, 0, s>>>(in, M, n, flags, codes, scales);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rotate_quant(const void *in, bool in_bf16, int64_t M, int n, bool hadamard,
                               bool int4, bool grouped, void *codes, float *scales,
                               hipStream_t s) {
  if (M == 0) return hipSuccess;
  LaunchTimer t("rotate_quant", s);
  const int flags = (hadamard ? kHadamard : 0) | (int4 ? kInt4 : 0) | (grouped ? kGrouped : 0);
  if (in_bf16)
    return dispatch(static_cast<const uint16_t *>(in), M, n, flags, static_cast<uint8_t *>(codes),
                    scales, s);
  return dispatch(static_cast<const float *>(in), M, n, flags, static_cast<uint8_t *>(codes),
                  scales, s);
}

}  // namespace qsvd
