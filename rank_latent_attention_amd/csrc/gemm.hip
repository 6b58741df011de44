// MFMA GEMM for the shared down-projection C = X W^d (gfx950).
//
// QSVD paper notes (NeurIPS 2025), "Key design": one down-projection shared
// by Q, K and V produces the latent C_qkv = X W^d that is cached; the QSVD
// digest ("Key Contributions") notes that it reads X once.  With W8A8 the
// product is an int8 x int8 contraction with per-token and per-column scales.
//
// C[M][N] = A[M][K] * B[K][N] with B stored transposed (Bt[N][K]) so both
// operands are contiguous along K, the layout MFMA operands want.
//   int8: v_mfma_i32_32x32x32_i8, exact int32 accumulation; epilogue
//         float32(float32(float32(acc) * a_scale[m]) * col_scale[n]).
//   bf16: v_mfma_f32_32x32x16_bf16, float32 accumulation; * col_scale[n].
//
// Data path.  A workgroup computes a BM x BN tile with WM x WN wavefronts
// (two per SIMD), each owning (BM/WM) x (BN/WN) in 32 x 32 MFMA blocks.  A K
// stage is 128 bytes of every operand row (one cache line), moved from global
// memory straight into LDS by buffer_load ... lds (no VGPR staging, no LDS
// store instructions); two LDS slots, the next stage in flight while the
// current one is multiplied.  In LDS, the 16-byte chunk c of row r sits at
// position c ^ g(r) of its 128-byte row, which makes the MFMA operand reads
// (32 consecutive rows, one chunk) free of bank conflicts.  The epilogue
// transposes each 32 x 32 block through LDS so that every lane writes four
// consecutive outputs of a row.  The blockIdx -> tile map keeps the row
// blocks of one XCD contiguous so an A tile is fetched into a single XCD's L2.
#include "device_common.h"
#include "dma_pipe.h"
#include "qsvd_internal.h"

#include <climits>
#include <cstdint>
#include <type_traits>

namespace qsvd {
namespace {

using dma::BK;
using dma::kRowsPerDma;
using dma::lds_ptr;
using dma::rsrc_rows;
using dma::swz;
using dma::wait_all_loads;

constexpr int kComputeUnits = 256;       // gfx950: 8 XCDs x 32 CUs
constexpr int kEpiStride = 36;           // epilogue block row stride (32-bit words)

template <bool INT8, bool OUT_BF16, int BM, int BN, int WM, int WN, bool INT4>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_kernel(const uint8_t *__restrict__ A, const float *__restrict__ a_scale, int64_t M, int K,
                 const uint8_t *__restrict__ Bt, const float *__restrict__ col_scale, int N,
                 void *__restrict__ Cout) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;            // wavefront tile
  constexpr int MB = TM / 32, NB = TN / 32;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wavefront tile");
  constexpr int SLOT = (BM + BN) * BK;
  constexpr int BLK_A = BM / kRowsPerDma;
  constexpr int BLK = (BM + BN) / kRowsPerDma;
  static_assert(BLK % NW == 0, "DMA blocks split evenly over the wavefronts");
  constexpr int LPW = BLK / NW;                        // DMA instructions per wavefront per stage
  static_assert(1024 + NW * 32 * kEpiStride * 4 <= 2 * SLOT, "epilogue fits in the slots");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  static_assert(INT8 || !INT4, "int4 operands are integer codes");
  const int64_t kbytes = INT4 ? static_cast<int64_t>(K) / 2 : static_cast<int64_t>(K) * (INT8 ? 1 : 2);
  const int nbn = (N + BN - 1) / BN;
  const int total = gridDim.x, id = blockIdx.x;
  const int per = total / 8, rem = total % 8;
  const int xcd = id % 8, local = id / 8;
  const int tile = xcd * per + min(xcd, rem) + local;
  const int64_t m0 = static_cast<int64_t>(tile / nbn) * BM;
  const int n0 = (tile % nbn) * BN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // rows past M (N) read as zero through the buffer range check
  const __amdgpu_buffer_rsrc_t ra = rsrc_rows(A + m0 * kbytes, (M - m0) * kbytes);
  const __amdgpu_buffer_rsrc_t rb = rsrc_rows(Bt + static_cast<int64_t>(n0) * kbytes,
                                              (static_cast<int64_t>(N) - n0) * kbytes);
  // A DMA instruction fills 8 LDS rows; lane l writes 16 bytes at l * 16, i.e.
  // row l / 8, position l % 8, so it fetches chunk (l % 8) ^ swz(row).  The
  // rows of this wavefront's blocks are wave * 8 + l / 8 modulo 16.
  const uint32_t lane_off = dma::lane_offset(lane, wave, kbytes);

  // epilogue operands fetched up front
  float my_as = 0.f;
  if constexpr (INT8) {
    if (tid < BM && m0 + tid < M) my_as = a_scale[m0 + tid];
  }
  float csr[NB][4];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int n = n0 + wn * TN + j * 32 + (lane & 7) * 4 + c;
      csr[j][c] = (col_scale && n < N) ? col_scale[n] : 1.f;
    }

  // DMA instruction i (0 <= i < LPW) of a stage: LDS block wave + NW * i
  auto issue_one = [&](int i, int stage, int slot) {
    const uint32_t kb = static_cast<uint32_t>(stage) * BK;
    uint8_t *base = lds + slot * SLOT;
    const int blk = wave + NW * i;
    if (blk < BLK_A) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, lds_ptr(base + blk * 1024), 16,
          lane_off + static_cast<uint32_t>(blk * kRowsPerDma * kbytes) + kb, 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rb, lds_ptr(base + blk * 1024), 16,
          lane_off + static_cast<uint32_t>((blk - BLK_A) * kRowsPerDma * kbytes) + kb, 0, 0, 0);
    }
  };

  using Acc = typename std::conditional<INT8, i32x16, f32x16>::type;
  Acc acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  // operand fragments: row (lane & 31) of a 32-row block, chunk 2 * ks + lane / 32
  const int fr = lane & 31;
  const int fsw = swz(fr);
  // One stage: per 32-byte K step, the operand reads, a share of the next
  // stage's DMA instructions, then the MFMAs; the scheduling groups interleave
  // the DMA issue with the MFMAs so neither waits for the other.
  constexpr int KSTEPS = BK / 32;
  constexpr int PER = (LPW + KSTEPS - 1) / KSTEPS;     // DMA instructions per K step
  auto compute = [&](int slot, int ksteps, int nstage, int nslot) {
    const uint8_t *base = lds + slot * SLOT;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      // a short last stage skips its tail steps and the DMA shares issued
      // there, which only repeat the last stage into a slot that is not read
      if (ks >= ksteps) break;
      const int pos = ((ks * 2 + (lane >> 5)) ^ fsw) * 16;
      u32x4 af[MB], bfr[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *reinterpret_cast<const u32x4 *>(base + (wm * TM + i * 32 + fr) * BK + pos);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bfr[j] = *reinterpret_cast<const u32x4 *>(base + (BM + wn * TN + j * 32 + fr) * BK + pos);
#pragma unroll
      for (int q = 0; q < PER; ++q)
        if (ks * PER + q < LPW) issue_one(ks * PER + q, nstage, nslot);
      if constexpr (INT4) {
        // 16 bytes = 32 int4 codes.  Masking a nibble into the high half of
        // its byte gives the int8 value 16 * code, exactly: the odd elements
        // (high nibbles) and the even ones (shifted up) form two int8
        // operands; A and B pair them the same way, so the sum over K is
        // unchanged and the int32 accumulator holds 256 * sum exactly.
        u32x4 blo[NB];
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            blo[j][e] = (bfr[j][e] << 4) & 0xF0F0F0F0u;
            bfr[j][e] &= 0xF0F0F0F0u;
          }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          u32x4 alo, ahi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            alo[e] = (af[i][e] << 4) & 0xF0F0F0F0u;
            ahi[e] = af[i][e] & 0xF0F0F0F0u;
          }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(i32x4, alo), __builtin_bit_cast(i32x4, blo[j]), acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                __builtin_bit_cast(i32x4, ahi), __builtin_bit_cast(i32x4, bfr[j]), acc[i][j], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            if constexpr (INT8)
              acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                  __builtin_bit_cast(i32x4, af[i]), __builtin_bit_cast(i32x4, bfr[j]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
          }
      }
      __builtin_amdgcn_sched_group_barrier(0x100, MB + NB, 0);   // LDS operand reads
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);       // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // 1 DMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB * (INT4 ? 2 : 1), 0);   // the remaining MFMAs
    }
  };

  // K is a multiple of 64 bytes; a last stage of 64 bytes runs two K steps
  // (its upper half holds the next row's bytes and is not used)
  const int nk = static_cast<int>((kbytes + BK - 1) / BK);
  const int last_steps = (kbytes % BK == 0) ? BK / 32 : static_cast<int>(kbytes % BK) / 32;
#pragma unroll
  for (int i = 0; i < LPW; ++i) issue_one(i, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed for every wavefront and everyone is done reading
    // the other slot, which takes stage kt + 1 during this stage's MFMAs (past
    // the end, a repeat of the last stage into a slot that is not read again)
    wait_all_loads();
    __builtin_amdgcn_s_barrier();
    compute(kt & 1, kt == nk - 1 ? last_steps : BK / 32, min(kt + 1, nk - 1), (kt + 1) & 1);
  }
  wait_all_loads();
  __builtin_amdgcn_s_barrier();

  // Epilogue: row scales to LDS; each wavefront writes a 32 x 32 accumulator
  // block into its own LDS area (element e of lane l is row 8*(e/4) +
  // 4*(l/32) + e%4, column l%32) and reads it back as 4 consecutive columns
  // of one row per lane.
  float *las = reinterpret_cast<float *>(lds);
  if constexpr (INT8) {
    if (tid < BM) las[tid] = my_as;
  }
  __syncthreads();
  uint32_t *blk = reinterpret_cast<uint32_t *>(lds + 1024 + wave * (32 * kEpiStride * 4));
  const int rr = lane >> 3, cc = (lane & 7) * 4;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // (a bit cast of a vector element would read element 0 with this
        // compiler; convert through a scalar)
        uint32_t bits;
        if constexpr (INT8) bits = static_cast<uint32_t>(static_cast<int>(acc[i][j][e]));
        else bits = __float_as_uint(static_cast<float>(acc[i][j][e]));
        blk[(8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)) * kEpiStride + (lane & 31)] = bits;
      }
      __builtin_amdgcn_wave_barrier();
      const int n = n0 + wn * TN + j * 32 + cc;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = q * 8 + rr;
        const u32x4 w = *reinterpret_cast<const u32x4 *>(blk + r * kEpiStride + cc);
        const int lrow = wm * TM + i * 32 + r;
        const int64_t m = m0 + lrow;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t wc = w[c];
          if constexpr (INT8) {
            // int4: the accumulator is 256 * the integer sum (a multiple of 256)
            v[c] = static_cast<float>(INT4 ? (static_cast<int>(wc) >> 8) : static_cast<int>(wc));
            v[c] = v[c] * las[lrow];
            v[c] = v[c] * csr[j][c];
          } else {
            v[c] = __uint_as_float(wc) * csr[j][c];
          }
        }
        if (m < M && n < N) {
          if constexpr (OUT_BF16) {
            u32x2 o = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(Cout) + m * N + n) = o;
          } else {
            *reinterpret_cast<f32x4 *>(static_cast<float *>(Cout) + m * N + n) = {v[0], v[1], v[2], v[3]};
          }
        }
      }
      __builtin_amdgcn_wave_barrier();
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

template <bool INT8, bool OUT_BF16, int BM, int BN, int WM, int WN, bool INT4>
hipError_t run_gemm(const uint8_t *a, const float *a_scale, int64_t M, int K, const uint8_t *b,
                    const float *col_scale, int N, void *C, hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  constexpr size_t lds = static_cast<size_t>(2) * (BM + BN) * BK;
  auto kern = gemm_kernel<INT8, OUT_BF16, BM, BN, WM, WN, INT4>;
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<dim3(static_cast<unsigned>(tiles)), dim3(64 * WM * WN), lds, s>>>(a, a_scale, M, K, b,
                                                                          col_scale, N, C);
  return hipGetLastError();
}

template <bool INT8, bool OUT_BF16, bool INT4 = false>
hipError_t run_gemm_shape(const uint8_t *a, const float *a_scale, int64_t M, int K,
                          const uint8_t *b, const float *col_scale, int N, void *C,
                          hipStream_t s) {
  // Tile choice: a launch takes ceil(tiles / concurrent) rounds, each about
  // as long as one tile's area per compute unit; pick the least rounds x area
  // (x workgroups per CU), the larger tile on ties.  16384 x 1536 -> 256 x 384
  // (256 tiles, one round); 16384 x 512 -> 128 x 256; 16384 x 8192 -> 256 x 256.
  struct Cand { int bm, bn, per_cu; };
  static constexpr Cand cands[] = {{256, 384, 1}, {256, 256, 1}, {128, 256, 1}, {128, 128, 2}};
  int best = INT4 ? 1 : 0;
  int64_t best_cost = INT64_MAX;
  // (int4 unpacking needs registers the 256 x 384 accumulators leave no room for)
  for (int i = INT4 ? 1 : 0; i < 4; ++i) {
    const int64_t tiles = ((M + cands[i].bm - 1) / cands[i].bm) * ((N + cands[i].bn - 1) / cands[i].bn);
    const int64_t slots = static_cast<int64_t>(kComputeUnits) * cands[i].per_cu;
    const int64_t cost = ((tiles + slots - 1) / slots) * cands[i].bm * cands[i].bn * cands[i].per_cu;
    if (cost < best_cost) { best_cost = cost; best = i; }
  }
  switch (best) {
    case 0:
      if constexpr (!INT4) return run_gemm<INT8, OUT_BF16, 256, 384, 2, 4, false>(a, a_scale, M, K, b, col_scale, N, C, s);
      [[fallthrough]];
    case 1: return run_gemm<INT8, OUT_BF16, 256, 256, 2, 4, INT4>(a, a_scale, M, K, b, col_scale, N, C, s);
    case 2: return run_gemm<INT8, OUT_BF16, 128, 256, 2, 4, INT4>(a, a_scale, M, K, b, col_scale, N, C, s);
    default: return run_gemm<INT8, OUT_BF16, 128, 128, 2, 2, INT4>(a, a_scale, M, K, b, col_scale, N, C, s);
  }
}

}  // namespace

hipError_t launch_gemm(const void *A, const float *a_scale, int in_kind, int64_t M, int K,
                       const void *Bt, const float *col_scale, int N, void *C, bool c_bf16,
                       hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const auto *a = static_cast<const uint8_t *>(A);
  const auto *b = static_cast<const uint8_t *>(Bt);
  LaunchTimer t(in_kind == kGemmI4 ? "gemm_i4" : (in_kind == kGemmI8 ? "gemm_i8" : "gemm_bf16"), s);
  if (in_kind == kGemmI4) {
    if (c_bf16) return run_gemm_shape<true, true, true>(a, a_scale, M, K, b, col_scale, N, C, s);
    return run_gemm_shape<true, false, true>(a, a_scale, M, K, b, col_scale, N, C, s);
  }
  if (in_kind == kGemmI8) {
    if (c_bf16) return run_gemm_shape<true, true>(a, a_scale, M, K, b, col_scale, N, C, s);
    return run_gemm_shape<true, false>(a, a_scale, M, K, b, col_scale, N, C, s);
  }
  if (c_bf16) return run_gemm_shape<false, true>(a, a_scale, M, K, b, col_scale, N, C, s);
  return run_gemm_shape<false, false>(a, a_scale, M, K, b, col_scale, N, C, s);
}

// packed[c][k / 2] = code[k][c] (low nibble) | code[k + 1][c] << 4, from int8 codes [rows][cols]
__global__ __launch_bounds__(256) void pack_int4_transpose_kernel(const int8_t *__restrict__ in,
                                                                  int rows, int cols,
                                                                  uint8_t *__restrict__ out) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int half = rows / 2;
  if (i >= static_cast<int64_t>(cols) * half) return;
  const int c = static_cast<int>(i / half), k2 = static_cast<int>(i % half);
  const int lo = in[static_cast<int64_t>(2 * k2) * cols + c] & 0xF;
  const int hi = in[static_cast<int64_t>(2 * k2 + 1) * cols + c] & 0xF;
  out[i] = static_cast<uint8_t>(lo | (hi << 4));
}

hipError_t launch_pack_int4(const void *W, int rows, int cols, void *out, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  const int64_t n = static_cast<int64_t>(cols) * (rows / 2);
  LaunchTimer t("pack_int4", s);
  pack_int4_transpose_kernel<<<dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s>>>(
      static_cast<const int8_t *>(W), rows, cols, static_cast<uint8_t *>(out));
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
