// MFMA GEMM for the shared down-projection C = X W^d (gfx950).
//
// QSVD paper notes (NeurIPS 2025), "Key design": one down-projection shared
// by Q, K and V produces the latent C_qkv = X W^d that is cached; the QSVD
// digest ("Key Contributions") notes that it reads X once.  With W8A8 the
// product is an int8 x int8 contraction with per-token and per-column scales.
//
// C[M][N] = A[M][K] * B[K][N] with B stored transposed (Bt[N][K]) so both
// operands are contiguous along K, the layout MFMA operands want.  One
// workgroup (4 wavefronts) computes a 128 x 128 tile; each wavefront owns
// 64 x 64 = 2 x 2 MFMA 32x32 blocks.  A K-step is 64 bytes of each operand row
// (64 int8 or 32 bf16), staged through double-buffered LDS.
//   int8: v_mfma_i32_32x32x32_i8, exact int32 accumulation; epilogue
//         float32(float32(float32(acc) * a_scale[m]) * col_scale[n]).
//   bf16: v_mfma_f32_32x32x16_bf16, float32 accumulation; * col_scale[n].
// The blockIdx -> tile map keeps the row blocks of one XCD contiguous so an
// A tile is fetched into a single XCD's L2.
#include "device_common.h"
#include "qsvd_internal.h"

namespace qsvd {
namespace {

constexpr int BM = 128, BN = 128, BKB = 64;  // tile rows, cols, K bytes per step
constexpr int LDS_STRIDE = BKB + 16;         // padded row stride in LDS (bytes)

template <bool INT8, bool OUT_BF16>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t *__restrict__ A,
                                                   const float *__restrict__ a_scale, int64_t M,
                                                   int K, const uint8_t *__restrict__ Bt,
                                                   const float *__restrict__ col_scale, int N,
                                                   void *__restrict__ Cout) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][BM * LDS_STRIDE];

  const int esize = INT8 ? 1 : 2;
  const int64_t kbytes = static_cast<int64_t>(K) * esize;
  const int nbn = (N + BN - 1) / BN;

  // XCD-aware tile order: workgroup id i runs on XCD i % 8.
  const int total = gridDim.x;
  const int id = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = id % 8, local = id / 8;
  const int tile = xcd * per + min(xcd, rem) + local;
  const int64_t m0 = static_cast<int64_t>(tile / nbn) * BM;
  const int n0 = (tile % nbn) * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: thread t moves rows t/4 and t/4 + 64, 16-byte chunk t%4
  const int lrow = tid >> 2, lchunk = (tid & 3) * 16;
  u32x4 ra[2], rb[2];
  auto gload = [&](int64_t kb0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t m = m0 + lrow + h * 64;
      const int n = n0 + lrow + h * 64;
      ra[h] = (m < M) ? *reinterpret_cast<const u32x4 *>(A + m * kbytes + kb0 + lchunk)
                      : u32x4{0u, 0u, 0u, 0u};
      rb[h] = (n < N) ? *reinterpret_cast<const u32x4 *>(Bt + static_cast<int64_t>(n) * kbytes +
                                                          kb0 + lchunk)
                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      *reinterpret_cast<u32x4 *>(&lds[buf][0][(lrow + h * 64) * LDS_STRIDE + lchunk]) = ra[h];
      *reinterpret_cast<u32x4 *>(&lds[buf][1][(lrow + h * 64) * LDS_STRIDE + lchunk]) = rb[h];
    }
  };

  using Acc = typename std::conditional<INT8, i32x16, f32x16>::type;
  Acc acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int nk = static_cast<int>(kbytes / BKB);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(static_cast<int64_t>(kt + 1) * BKB);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // two 32-byte MFMA K-steps per 64-byte stage
      const int koff = ks * 32 + (lane >> 5) * 16;
      u32x4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const u32x4 *>(
            &lds[buf][0][(wm * 64 + i * 32 + (lane & 31)) * LDS_STRIDE + koff]);
        bf[i] = *reinterpret_cast<const u32x4 *>(
            &lds[buf][1][(wn * 64 + i * 32 + (lane & 31)) * LDS_STRIDE + koff]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (INT8) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(i32x4, af[i]), __builtin_bit_cast(i32x4, bf[j]), acc[i][j], 0,
                0, 0);
          } else {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bf[j]), acc[i][j],
                0, 0, 0);
          }
        }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 accumulator layout: element e of lane l is
  // row 8*(e/4) + 4*(l/32) + e%4, column l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= N) continue;
      const float cs = col_scale ? col_scale[n] : 1.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
        if (m >= M) continue;
        float v;
        if constexpr (INT8) {
          v = static_cast<float>(acc[i][j][e]);
          v = v * a_scale[m];
          v = v * cs;
        } else {
          v = acc[i][j][e] * cs;
        }
        if constexpr (OUT_BF16)
          static_cast<uint16_t *>(Cout)[m * N + n] = f32_to_bf16(v);
        else
          static_cast<float *>(Cout)[m * N + n] = v;
      }
    }
}

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ in, int rows,
                                                        int cols, T *__restrict__ out) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int r = r0 + ty + k, c = c0 + tx;
    if (r < rows && c < cols) tile[ty + k][tx] = in[static_cast<int64_t>(r) * cols + c];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 32; k += 8) {
    const int c = c0 + ty + k, r = r0 + tx;
    if (r < rows && c < cols) out[static_cast<int64_t>(c) * rows + r] = tile[tx][ty + k];
  }
}

}  // namespace

hipError_t launch_gemm(const void *A, const float *a_scale, bool int8, int64_t M, int K,
                       const void *Bt, const float *col_scale, int N, void *C, bool c_bf16,
                       hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid(static_cast<unsigned>(tiles)), block(256);
  const auto *a = static_cast<const uint8_t *>(A);
  const auto *b = static_cast<const uint8_t *>(Bt);
  LaunchTimer t(int8 ? "gemm_i8" : "gemm_bf16", s);
  if (int8) {
    if (c_bf16)
      gemm_kernel<true, true><<<grid, block, 0, s>>>(a, a_scale, M, K, b, col_scale, N, C);
    else
      gemm_kernel<true, false><<<grid, block, 0, s>>>(a, a_scale, M, K, b, col_scale, N, C);
  } else {
    if (c_bf16)
      gemm_kernel<false, true><<<grid, block, 0, s>>>(a, a_scale, M, K, b, col_scale, N, C);
    else
      gemm_kernel<false, false><<<grid, block, 0, s>>>(a, a_scale, M, K, b, col_scale, N, C);
  }
  return hipGetLastError();
}

hipError_t launch_transpose(const void *W, int elem_bytes, int rows, int cols, void *out,
                            hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const dim3 grid((cols + 31) / 32, (rows + 31) / 32), block(256);
  LaunchTimer t("transpose", s);
  switch (elem_bytes) {
    case 1:
      transpose_kernel<uint8_t><<<grid, block, 0, s>>>(static_cast<const uint8_t *>(W), rows,
                                                       cols, static_cast<uint8_t *>(out));
      break;
    case 2:
      transpose_kernel<uint16_t><<<grid, block, 0, s>>>(static_cast<const uint16_t *>(W), rows,
                                                        cols, static_cast<uint16_t *>(out));
      break;
    default:
      transpose_kernel<uint32_t><<<grid, block, 0, s>>>(static_cast<const uint32_t *>(W), rows,
                                                        cols, static_cast<uint32_t *>(out));
      break;
  }
  return hipGetLastError();
}

}  // namespace qsvd
