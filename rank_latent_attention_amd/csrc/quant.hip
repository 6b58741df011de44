// Fused block Walsh-Hadamard rotation + absmax quantiser (gfx950).
//
// QSVD paper notes (NeurIPS 2025), "Key design", quantisation scheme: the
// input X is rotated by an orthogonal H1 and the cached latent C by H2 before
// low-bit quantisation, which spreads channel outliers; the W8A8 / W8A4 rows
// of "Main results" quantise activations and latents per token.
//
// One wavefront owns one row.  A 128-element Hadamard block is spread over 4
// consecutive lanes: the block's 16-byte chunks (8 bf16 or 4 float32 values
// each) are dealt round-robin, chunk c to lane c % 4, so lane q holds chunks
// q, q+4, q+8, ...  Butterfly stages inside a chunk and between a lane's
// chunks run in registers; the two stages between chunk neighbours (chunk
// bit 0 and 1) pair lanes l ^ 1 and l ^ 2 through DPP quad permutes.  One
// pass of the wavefront covers 16 blocks (2048 values); longer rows take
// several passes.  The absmax is a wavefront max (per token) or a 4-lane max
// (per 128-group).  Float arithmetic is compiled without contraction, so
// every sum, difference, product and quotient is one IEEE float32 operation
// rounded to nearest even, and the stages run in the order h = 1, 2, .., 64
// whatever register or lane holds the pair.
#include "device_common.h"
#include "qsvd_internal.h"

namespace qsvd {
namespace {

constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;  // float32(1/sqrt(128)), bits 0x3DB504F3

enum : int { kHadamard = 1, kInt4 = 2, kGrouped = 4 };

// 16-byte chunk -> EPC float values
template <typename InT>
struct Chunk;

template <>
struct Chunk<float> {
  static constexpr int EPC = 4;
  __device__ static void load(const float *p, float v[4]) {
    const f32x4 a = *reinterpret_cast<const f32x4 *>(p);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  }
};

template <>
struct Chunk<uint16_t> {
  static constexpr int EPC = 8;
  __device__ static void load(const uint16_t *p, float v[8]) {
    const u32x4 a = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
};

// value of the lane at xor distance 1 or 2 inside the quad
template <int X>
__device__ __forceinline__ float quad_xor(float v) {
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;   // quad_perm [1,0,3,2] / [2,3,0,1]
  return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), ctrl, 0xF, 0xF, false));
}

// code = rne(fl32(y / s)) for s > 0, else 0; |code| <= qmax without a clamp
// because s = fl32(amax / qmax) makes |y / s| < qmax + 1/2 (the clamp is kept
// on this rarely used path only).
__device__ __forceinline__ float quant_div(float y, float s, float qmax) {
  if (!(s > 0.f)) return 0.f;
  return fminf(fmaxf(rintf(y / s), -qmax), qmax);
}

// The same quotient from the correctly rounded reciprocal r = fl32(1 / s):
// q = fl32(y r) is within one ulp of y / s, the residual y - q s is exact
// through an FMA, and one correction q + (y - q s) r rounds to fl32(y / s)
// (Markstein's correction theorem, binary32, round to nearest) as long as
// nothing underflows, which s >= 2^-64 and |y / s| <= 128 rule out for every
// quotient that rounds to a nonzero code.
__device__ __forceinline__ float quant_rcp(float y, float s, float r) {
  const float q = y * r;
  const float rem = fmaf(-s, q, y);
  return rintf(fmaf(rem, r, q));
}

// NP passes of 2048 values; v[p][t][i] = value i of chunk q + 4 t of block
// 16 p + lane / 4, where q = lane % 4
template <typename InT, int NP, bool HAD, bool INT4, bool GROUPED>
__global__ __launch_bounds__(256) void rotate_quant_kernel(const InT *__restrict__ in, int64_t M,
                                                           int n, uint8_t *__restrict__ codes,
                                                           float *__restrict__ scales) {
  constexpr int EPC = Chunk<InT>::EPC;
  constexpr int T = 128 / (4 * EPC);               // chunks of a block per lane
  constexpr float qmax = INT4 ? 7.f : 127.f;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= M) return;  // uniform per wavefront; no workgroup barrier follows
  const int q = lane & 3;

  // element offset of chunk (p, t) of this lane; valid when < n
  auto elem = [&](int p, int t) { return (16 * p + (lane >> 2)) * 128 + (q + 4 * t) * EPC; };

  float v[NP][T][EPC];
  const InT *src = in + row * static_cast<int64_t>(n);
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int e = elem(p, t);
      if (e < n) {
        Chunk<InT>::load(src + e, v[p][t]);
      } else {
#pragma unroll
        for (int i = 0; i < EPC; ++i) v[p][t][i] = 0.f;
      }
    }

  if constexpr (HAD) {   // n % 128 == 0: every chunk of a touched block is valid
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      if (p * 2048 >= n) break;
      // h = 1 .. EPC/2: inside a chunk
#pragma unroll
      for (int h = 1; h < EPC; h <<= 1)
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
          for (int i = 0; i < EPC; ++i)
            if ((i & h) == 0) {
              const float a = v[p][t][i], b = v[p][t][i + h];
              v[p][t][i] = a + b;
              v[p][t][i + h] = a - b;
            }
      // h = EPC, 2 EPC: chunk bits 0 and 1, across the quad.  The lower lane
      // of a pair gets other + own = own + other, the upper lane other + (-own)
      // = other - own; both are the single rounded sum or difference.
      const uint32_t flip1 = (q & 1) ? 0x80000000u : 0u, flip2 = (q & 2) ? 0x80000000u : 0u;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < EPC; ++i)
          v[p][t][i] = quad_xor<1>(v[p][t][i]) + __uint_as_float(__float_as_uint(v[p][t][i]) ^ flip1);
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < EPC; ++i)
          v[p][t][i] = quad_xor<2>(v[p][t][i]) + __uint_as_float(__float_as_uint(v[p][t][i]) ^ flip2);
      // h = 4 EPC .. 64: between this lane's chunks
#pragma unroll
      for (int ht = 1; ht < T; ht <<= 1)
#pragma unroll
        for (int t = 0; t < T; ++t)
          if ((t & ht) == 0)
#pragma unroll
            for (int i = 0; i < EPC; ++i) {
              const float a = v[p][t][i], b = v[p][t + ht][i];
              v[p][t][i] = a + b;
              v[p][t + ht][i] = a - b;
            }
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < EPC; ++i) v[p][t][i] = v[p][t][i] * kInvSqrt128;
    }
  }

  float s_row = 0.f;
  if constexpr (!GROUPED) {
    float amax = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < EPC; ++i) amax = fmaxf(amax, fabsf(v[p][t][i]));
    amax = group_max<kWave>(amax);
    s_row = amax / qmax;
    if (lane == 0) scales[row] = s_row;
  }

  const int ngroups = n >> 7;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (p * 2048 >= n) break;
    float s = s_row;
    if constexpr (GROUPED) {   // n % 128 == 0; the block of this lane is 16 p + lane / 4
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < EPC; ++i) amax = fmaxf(amax, fabsf(v[p][t][i]));
      amax = fmaxf(amax, quad_xor<1>(amax));
      amax = fmaxf(amax, quad_xor<2>(amax));
      s = amax / qmax;
      const int blk = 16 * p + (lane >> 2);
      if (blk < ngroups && q == 0) scales[row * ngroups + blk] = s;
    }
    const float r = 1.f / s;
    const bool fast = __builtin_amdgcn_ballot_w64(!(s >= 0x1p-64f)) == 0;   // uniform
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int e = elem(p, t);
      if (e >= n) continue;
      int c[EPC];
      if (fast) {
#pragma unroll
        for (int i = 0; i < EPC; ++i) c[i] = static_cast<int>(quant_rcp(v[p][t][i], s, r));
      } else {
#pragma unroll
        for (int i = 0; i < EPC; ++i) c[i] = static_cast<int>(quant_div(v[p][t][i], s, qmax));
      }
      if constexpr (INT4) {
        uint32_t w = 0;
#pragma unroll
        for (int i = 0; i < EPC; ++i) w |= static_cast<uint32_t>(c[i] & 0xF) << (4 * i);
        uint8_t *dst = codes + row * static_cast<int64_t>(n / 2) + e / 2;
        if constexpr (EPC == 8) *reinterpret_cast<uint32_t *>(dst) = w;
        else *reinterpret_cast<uint16_t *>(dst) = static_cast<uint16_t>(w);
      } else {
        uint8_t *dst = codes + row * static_cast<int64_t>(n) + e;
        if constexpr (EPC == 8) {
          u32x2 w = {0u, 0u};
#pragma unroll
          for (int i = 0; i < 8; ++i) w[i >> 2] |= static_cast<uint32_t>(c[i] & 0xFF) << (8 * (i & 3));
          *reinterpret_cast<u32x2 *>(dst) = w;
        } else {
          uint32_t w = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) w |= static_cast<uint32_t>(c[i] & 0xFF) << (8 * i);
          *reinterpret_cast<uint32_t *>(dst) = w;
        }
      }
    }
  }
}

template <typename InT, bool HAD, bool INT4, bool GROUPED>
void dispatch_np(const InT *in, int64_t M, int n, uint8_t *codes, float *scales, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((M + 3) / 4)), block(256);
  switch ((n + 2047) / 2048) {
    case 1: rotate_quant_kernel<InT, 1, HAD, INT4, GROUPED><<<grid, block, 0, s>>>(in, M, n, codes, scales); break;
    case 2: rotate_quant_kernel<InT, 2, HAD, INT4, GROUPED><<<grid, block, 0, s>>>(in, M, n, codes, scales); break;
    case 3: rotate_quant_kernel<InT, 3, HAD, INT4, GROUPED><<<grid, block, 0, s>>>(in, M, n, codes, scales); break;
    default: rotate_quant_kernel<InT, 4, HAD, INT4, GROUPED><<<grid, block, 0, s>>>(in, M, n, codes, scales); break;
  }
}

template <typename InT>
hipError_t dispatch(const InT *in, int64_t M, int n, int flags, uint8_t *codes, float *scales,
                    hipStream_t s) {
  switch (flags) {
    case 0: dispatch_np<InT, false, false, false>(in, M, n, codes, scales, s); break;
    case kHadamard: dispatch_np<InT, true, false, false>(in, M, n, codes, scales, s); break;
    case kInt4: dispatch_np<InT, false, true, false>(in, M, n, codes, scales, s); break;
    case kHadamard | kInt4: dispatch_np<InT, true, true, false>(in, M, n, codes, scales, s); break;
    case kGrouped: dispatch_np<InT, false, false, true>(in, M, n, codes, scales, s); break;
    case kHadamard | kGrouped: dispatch_np<InT, true, false, true>(in, M, n, codes, scales, s); break;
    case kInt4 | kGrouped: dispatch_np<InT, false, true, true>(in, M, n, codes, scales, s); break;
    default: dispatch_np<InT, true, true, true>(in, M, n, codes, scales, s); break;
  }
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
