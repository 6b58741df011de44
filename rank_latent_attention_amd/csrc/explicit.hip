// Decode with explicit on-chip K/V reconstruction, optional rotary positions (gfx950).
//
// QSVD paper notes (NeurIPS 2025), "Key design": only the latent C = X W^d is
// cached, and K = C W^u_k, V = C W^u_v are rebuilt when needed.  The WSVD
// digest ("Method, 3.4" and "Key Contributions") describes the fused
// flash-decoding pass that reconstructs keys tile by tile in registers,
// applies RoPE and contracts with q without writing K to memory.  This file is
// that literal form; the library's main decode path re-associates the same
// sums in the latent space instead (q absorbed into W^u_k), which moves 16x
// fewer MFMA operations, and is the one held to the HBM roofline.
//
// One workgroup (8 wavefronts, two per SIMD) owns 256 tokens of one sequence
// and one head h.  Its main loop is a 256 x 256 x r GEMM: A = the bf16 latent
// rows of the tile, B = the 128 rows of W^u_k,h^T and the 128 rows of
// W^u_v,h^T (weights pre-packed K-contiguous, [E][r]), streamed global ->
// LDS by DMA in 128-byte K stages (dma_pipe.h) into v_mfma_f32_32x32x16_bf16.
// Wavefronts (wm, wn) hold rows 128 wm .. and columns 64 wn .. of [K_h | V_h]
// in float32 accumulators.  Epilogue:
//   1. the key wavefronts write K_h^T (float32) to LDS;
//   2. every token's score s_t = rope(K_h[t], t) . rope(q_h, L - 1) * scale
//      (rotation by the caller's cos / sin tables; none without tables);
//   3. the softmax of the tile (max m, sum l of 2^(s - m), in log2 units);
//   4. the value wavefronts contract p with their V_h accumulators;
//   5. (m, l, sum_t p_t V_h[t]) go to the workspace.
// explicit_merge_kernel combines the tiles of each (sequence, head) by their
// log-sum-exp weights into O.
#include "device_common.h"
#include "dma_pipe.h"
#include "qsvd_internal.h"

#include <algorithm>

#include <cmath>
#include <cstdint>

namespace qsvd {
namespace {

using dma::BK;
using dma::kRowsPerDma;
using dma::lds_ptr;
using dma::rsrc_rows;
using dma::swz;
using dma::wait_all_loads;

constexpr float kLog2eX = 1.4426950408889634f;
constexpr int kD = 128;                    // head dimension of this variant
constexpr int kTok = 256;                  // tokens per workgroup
constexpr int kTG = 8;                     // tiles per group of the XCD-aware order
constexpr int kBN = 2 * kD;                // [K_h | V_h] columns
constexpr int kSlot = (kTok + kBN) * BK;   // one LDS stage (64 KB)
constexpr int kKtStride = kTok + 4;        // K^T row stride (floats)
constexpr int kKtBytes = kD * kKtStride * 4;
constexpr int kQrOff = kKtBytes > 2 * kSlot ? kKtBytes : 2 * kSlot;  // rotated query [128]
constexpr int kPsOff = kQrOff + kD * 4;    // partial scores [2][256], then p [256]
constexpr int kRedOff = kPsOff + 2 * kTok * 4;   // reductions: [2][128] + [8]
constexpr int kLdsBytes = kRedOff + 2 * kD * 4 + 64;
constexpr int kPartFloats = 4 + kD;        // (m, l, -, -, O[128]) per (sequence, tile, head)

template <bool ROPE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void explicit_attn_kernel(const uint16_t *__restrict__ q, const uint8_t *__restrict__ C,
                          const uint8_t *__restrict__ Wk_t, const uint8_t *__restrict__ Wv_t,
                          const float *__restrict__ rope_cos, const float *__restrict__ rope_sin,
                          int64_t L, int r, int heads, float scale_log2,
                          float *__restrict__ part) {
  constexpr int WM = 2, WN = 4, NW = WM * WN;
  constexpr int TM = kTok / WM, TN = kBN / WN;   // 128 x 64 per wavefront
  constexpr int MB = TM / 32, NB = TN / 32;
  constexpr int BLK_A = kTok / kRowsPerDma;      // 32 DMA blocks of latent rows
  constexpr int BLK_K = kD / kRowsPerDma;        // 16 blocks of W^u_k rows, then 16 of W^u_v
  constexpr int BLK = (kTok + kBN) / kRowsPerDma;
  constexpr int LPW = BLK / NW;                  // 8 DMA instructions per wavefront per stage
  constexpr int KSTEPS = BK / 32;
  constexpr int PER = LPW / KSTEPS;
  static_assert(LPW % KSTEPS == 0, "DMA shares");
  extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];

  const int64_t ntiles = (L + kTok - 1) / kTok;
  int h;
  int64_t tile, seq;
  if (heads % 8 == 0) {
    // XCD x (workgroup id mod 8) owns heads x * heads / 8 ..; its concurrent
    // workgroups cover those heads for one group of kTG tiles, which all XCDs
    // work on at the same time: each XCD's L2 keeps its heads' W^u rows, and
    // the group's latent rows come from HBM about once for all eight XCDs.
    const int hpx = heads / 8;
    const int64_t id = blockIdx.x, local = id / 8;
    const int64_t ngroups = (ntiles + kTG - 1) / kTG;
    const int64_t rest = local / hpx, rest2 = rest / kTG;
    h = static_cast<int>(id % 8) * hpx + static_cast<int>(local % hpx);
    tile = (rest2 % ngroups) * kTG + rest % kTG;
    seq = rest2 / ngroups;
    if (tile >= ntiles) return;   // padding of the last tile group (the whole workgroup)
  } else {
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total / 8, rem = total % 8, xcd = id % 8, local = id / 8;
    const int64_t task = xcd * per + min(xcd, rem) + local;   // the heads of one tile share an XCD's L2
    h = static_cast<int>(task % heads);
    tile = (task / heads) % ntiles;
    seq = task / (static_cast<int64_t>(heads) * ntiles);
  }
  const int64_t t0 = tile * kTok;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int64_t kbytes = static_cast<int64_t>(r) * 2;

  float *qr = reinterpret_cast<float *>(lds + kQrOff);
  float *ps = reinterpret_cast<float *>(lds + kPsOff);
  float *red = reinterpret_cast<float *>(lds + kRedOff);

  // rotated, scaled query (outside the DMA slots; read after the main loop)
  if (tid < kD / 2) {
    const uint16_t *qh = q + (seq * heads + h) * kD;
    const float x0 = bf16_to_f32(qh[tid]), x1 = bf16_to_f32(qh[tid + kD / 2]);
    float y0 = x0, y1 = x1;
    if constexpr (ROPE) {
      const float c = rope_cos[(L - 1) * (kD / 2) + tid], s = rope_sin[(L - 1) * (kD / 2) + tid];
      y0 = x0 * c - x1 * s;
      y1 = x1 * c + x0 * s;
    }
    qr[tid] = y0 * scale_log2;
    qr[tid + kD / 2] = y1 * scale_log2;
  }

  // ---- main loop: [K_h | V_h] for the 256 tokens
  const __amdgpu_buffer_rsrc_t ra = rsrc_rows(C + (seq * L + t0) * kbytes, (L - t0) * kbytes);
  const __amdgpu_buffer_rsrc_t rbk = rsrc_rows(Wk_t + h * kD * kbytes, kD * kbytes);
  const __amdgpu_buffer_rsrc_t rbv = rsrc_rows(Wv_t + h * kD * kbytes, kD * kbytes);
  const uint32_t lane_off = dma::lane_offset(lane, wave, kbytes);
  auto issue_one = [&](int i, int stage, int slot) {
    const uint32_t kb = static_cast<uint32_t>(stage) * BK;
    uint8_t *base = lds + slot * kSlot;
    const int blk = wave + NW * i;
    if (blk < BLK_A) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, lds_ptr(base + blk * 1024), 16,
          lane_off + static_cast<uint32_t>(blk * kRowsPerDma * kbytes) + kb, 0, 0, 0);
    } else if (blk < BLK_A + BLK_K) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rbk, lds_ptr(base + blk * 1024), 16,
          lane_off + static_cast<uint32_t>((blk - BLK_A) * kRowsPerDma * kbytes) + kb, 0, 0, 0);
    } else {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rbv, lds_ptr(base + blk * 1024), 16,
          lane_off + static_cast<uint32_t>((blk - BLK_A - BLK_K) * kRowsPerDma * kbytes) + kb, 0, 0, 0);
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int fr = lane & 31;
  const int fsw = swz(fr);
  auto compute = [&](int slot, int nstage, int nslot) {
    const uint8_t *base = lds + slot * kSlot;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int pos = ((ks * 2 + (lane >> 5)) ^ fsw) * 16;
      u32x4 af[MB], bfr[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = *reinterpret_cast<const u32x4 *>(base + (wm * TM + i * 32 + fr) * BK + pos);
#pragma unroll
      for (int j = 0; j < NB; ++j)
        bfr[j] = *reinterpret_cast<const u32x4 *>(base + (kTok + wn * TN + j * 32 + fr) * BK + pos);
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) issue_one(ks * PER + q2, nstage, nslot);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, af[i]), __builtin_bit_cast(bf16x8, bfr[j]), acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, MB + NB, 0);   // LDS operand reads
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);       // 2 MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);       // 1 DMA
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB, 0);
    }
  };

  // r % 64 == 0: whole 128-byte stages
  const int nk = static_cast<int>(kbytes / BK);
#pragma unroll
  for (int i = 0; i < LPW; ++i) issue_one(i, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed for every wavefront, nobody reads the other slot any
    // more; it takes stage kt + 1 (past the end, a repeat never read)
    wait_all_loads();
    __builtin_amdgcn_s_barrier();
    compute(kt & 1, min(kt + 1, nk - 1), (kt + 1) & 1);
  }
  wait_all_loads();
  __syncthreads();

  // ---- 1. K^T to LDS.  Accumulator element e of lane l: row 8 (e / 4) +
  // 4 (l / 32) + e % 4 of the 32-row block, column l % 32.
  // (The rotary rows of this thread's token are requested first, so they
  // arrive while the keys go to LDS.)
  f32x4 rcs[ROPE ? 8 : 1], rsn[ROPE ? 8 : 1];
  if constexpr (ROPE) {
    const int64_t pos = t0 + (tid & (kTok - 1));
    const int64_t prow = (pos < L ? pos : L - 1) * (kD / 2);
#pragma unroll
    for (int i4 = 0; i4 < 8; ++i4) {
      const int i0 = (tid >> 8) * 32 + 4 * i4;
      rcs[i4] = *reinterpret_cast<const f32x4 *>(rope_cos + prow + i0);
      rsn[i4] = *reinterpret_cast<const f32x4 *>(rope_sin + prow + i0);
    }
  }
  float *kt = reinterpret_cast<float *>(lds);
  if (wn < 2) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          const int c = wn * TN + j * 32 + (lane & 31);
          const int t = wm * TM + i * 32 + 8 * e4 + 4 * (lane >> 5);
          *reinterpret_cast<f32x4 *>(kt + c * kKtStride + t) =
              f32x4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
        }
  }
  __syncthreads();

  // ---- 2. scores: thread (token tid % 256, dimension pairs half * 32 ..)
  {
    const int t = tid & (kTok - 1), half = tid >> 8;
    const int64_t pos = t0 + t;
    float s = 0.f;
    if constexpr (ROPE) {
#pragma unroll
      for (int i4 = 0; i4 < 8; ++i4) {
        const int i0 = half * 32 + 4 * i4;
        const f32x4 cs = rcs[i4];
        const f32x4 sn = rsn[i4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = i0 + u;
          const float k0 = kt[i * kKtStride + t], k1 = kt[(i + kD / 2) * kKtStride + t];
          const float r0 = k0 * cs[u] - k1 * sn[u];
          const float r1 = k1 * cs[u] + k0 * sn[u];
          s = fmaf(r0, qr[i], s);
          s = fmaf(r1, qr[i + kD / 2], s);
        }
      }
    } else {
#pragma unroll 8
      for (int i = half * 32; i < half * 32 + 32; ++i) {
        s = fmaf(kt[i * kKtStride + t], qr[i], s);
        s = fmaf(kt[(i + kD / 2) * kKtStride + t], qr[i + kD / 2], s);
      }
    }
    ps[half * kTok + t] = s;
  }
  __syncthreads();

  // ---- 3. softmax of the tile (log2 units), threads 0..255
  float pt = 0.f;
  if (tid < kTok) {
    float s = ps[tid] + ps[kTok + tid];
    if (t0 + tid >= L) s = -INFINITY;
    float mx = s;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, kWave));
    if (lane == 0) red[2 * kD + wave] = mx;
    pt = s;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(red[2 * kD], red[2 * kD + 1]), fmaxf(red[2 * kD + 2], red[2 * kD + 3]));
  if (tid < kTok) {
    pt = (pt == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(pt - M);
    float sum = pt;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, kWave);
    if (lane == 0) red[2 * kD + 4 + wave] = sum;
    ps[tid] = pt;   // same index as this thread's own read above
  }
  __syncthreads();

  // ---- 4. value wavefronts: sum_t p_t V_h[t]
  float *obuf = red;   // [2][128]
  if (wn >= 2) {
    float o[NB] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = ps[wm * TM + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3)];
#pragma unroll
        for (int j = 0; j < NB; ++j) o[j] = fmaf(p, acc[i][j][e], o[j]);
      }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      o[j] += __shfl_xor(o[j], 32, kWave);
      if (lane < 32) obuf[wm * kD + (wn - 2) * TN + j * 32 + lane] = o[j];
    }
  }
  __syncthreads();

  // ---- 5. the tile's partial state
  float *dst = part + ((seq * ntiles + tile) * heads + h) * kPartFloats;
  if (tid < kD) dst[4 + tid] = obuf[tid] + obuf[kD + tid];
  if (tid == 0) {
    dst[0] = M;
    dst[1] = red[2 * kD + 4] + red[2 * kD + 5] + red[2 * kD + 6] + red[2 * kD + 7];
    dst[2] = 0.f;
    dst[3] = 0.f;
  }
}

// One wavefront per (sequence, head): O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i.
template <typename OT>
__global__ __launch_bounds__(256) void explicit_merge_kernel(const float *__restrict__ part,
                                                             OT *__restrict__ O, int b, int heads,
                                                             int64_t ntiles) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= b * heads) return;   // uniform per wavefront; no barrier follows
  const int seq = w / heads, h = w % heads;
  // Tiles are read TB at a time with unconditional loads (an index past the
  // last tile rereads it and is not used), so each batch is one memory round
  // trip; the sums still run over the tiles in order.
  constexpr int TB = 8;
  auto src_of = [&](int64_t i) {
    return part + ((seq * ntiles + std::min<int64_t>(i, ntiles - 1)) * heads + h) * kPartFloats;
  };
  float M = -INFINITY;
  for (int64_t i0 = 0; i0 < ntiles; i0 += TB) {
    float mv[TB];
#pragma unroll
    for (int k = 0; k < TB; ++k) mv[k] = src_of(i0 + k)[0];
#pragma unroll
    for (int k = 0; k < TB; ++k)
      if (i0 + k < ntiles) M = fmaxf(M, mv[k]);
  }
  float den = 0.f, o0 = 0.f, o1 = 0.f;
  for (int64_t i0 = 0; i0 < ntiles; i0 += TB) {
    float mv[TB], lv[TB], a0[TB], a1[TB];
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      const float *src = src_of(i0 + k);
      mv[k] = src[0];
      lv[k] = src[1];
      a0[k] = src[4 + lane];
      a1[k] = src[4 + 64 + lane];
    }
#pragma unroll
    for (int k = 0; k < TB; ++k) {
      if (i0 + k < ntiles) {
        const float wgt = __builtin_amdgcn_exp2f(mv[k] - M);
        den = fmaf(wgt, lv[k], den);
        o0 = fmaf(wgt, a0[k], o0);
        o1 = fmaf(wgt, a1[k], o1);
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  OT *out = O + (static_cast<int64_t>(seq) * heads + h) * kD;
  if constexpr (sizeof(OT) == 2) {
    out[lane] = f32_to_bf16(o0 * inv);
    out[64 + lane] = f32_to_bf16(o1 * inv);
  } else {
    out[lane] = o0 * inv;
    out[64 + lane] = o1 * inv;
  }
}

}  // namespace

size_t explicit_workspace_bytes(int b, int64_t L, int heads) {
  const int64_t ntiles = (L + kTok - 1) / kTok;
  return static_cast<size_t>(b) * ntiles * heads * kPartFloats * sizeof(float);
}

hipError_t launch_decode_explicit(const ExplicitArgs &a, hipStream_t s) {
  const int64_t ntiles = (a.L + kTok - 1) / kTok;
  const int64_t total = a.heads % 8 == 0
                            ? static_cast<int64_t>(a.b) * a.heads * ((ntiles + kTG - 1) / kTG) * kTG
                            : static_cast<int64_t>(a.b) * ntiles * a.heads;
  float *part = static_cast<float *>(a.workspace);
  const float scale_log2 = a.softmax_scale * kLog2eX;
  {
    LaunchTimer t("explicit_attn", s);
    auto kern = a.rope_cos ? explicit_attn_kernel<true> : explicit_attn_kernel<false>;
    hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), kLdsBytes);
    if (e != hipSuccess) return e;
    kern<<<dim3(static_cast<unsigned>(total)), dim3(512), kLdsBytes, s>>>(
        static_cast<const uint16_t *>(a.q), static_cast<const uint8_t *>(a.C),
        static_cast<const uint8_t *>(a.Wk_t), static_cast<const uint8_t *>(a.Wv_t), a.rope_cos,
        a.rope_sin, a.L, a.r, a.heads, scale_log2, part);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  LaunchTimer t("explicit_merge", s);
  const dim3 grid(static_cast<unsigned>((a.b * a.heads + 3) / 4)), block(256);
  if (a.o_dtype == QSVD_BF16)
    explicit_merge_kernel<uint16_t><<<grid, block, 0, s>>>(part, static_cast<uint16_t *>(a.O), a.b,
                                                           a.heads, ntiles);
  else
    explicit_merge_kernel<float><<<grid, block, 0, s>>>(part, static_cast<float *>(a.O), a.b, a.heads,
                                                        ntiles);
  return hipGetLastError();
}

}  // namespace qsvd
