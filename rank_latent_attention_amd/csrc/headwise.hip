// Decode over per-head latents (WSVD), keys rebuilt on chip, optional RoPE (gfx950).
//
// WSVD digest, "Method, 3.1": every head has its own low-rank factors,
// W_Kh = A_Kh B_Kh, and caches its own latent C_Kh = X A_Kh (r values per
// token and head instead of one shared R-wide latent), and the same for V.
// "Method, 3.4": the fused flash-decoding kernel streams C_Kh tiles, rebuilds
// K_{h,t} = C_{Kh,t} B_Kh in registers, applies RoPE, contracts with q_h, and
// fuses B_Vh into the output side instead of rebuilding V.
//
// Cache layout: C[b][L][heads][rk + rv] bf16, each head's key latent followed
// by its value latent, so one token's row holds every head.  Weights: B_Kh
// transposed, BK_t[heads][128][rk] (contiguous along the latent), and
// BV[heads][rv][128].
//
// headwise_stream_kernel: workgroup (sequence, split, 4 heads), one wavefront
// per head; past the staging of the RoPE rows the wavefronts share nothing.  A
// wavefront keeps its head's B_Kh fragments in registers for the whole split
// and, per 32-token tile:
//   1. 16-byte buffer loads of the tile's key and value latents of its head,
//      one or two tiles ahead (rows past L read as zero and are masked);
//   2. K (32 x 128) = C_K (32 x rk) B_Kh with v_mfma_f32_16x16x32_bf16, the
//      latent rows straight from the load registers as the A operand;
//   3. RoPE: dimension i pairs with i + 64, both in the same lane (column
//      blocks nb and nb + 4).  Rotations compose, so the query is turned back
//      to the tile start once per tile (table row t0) and then by each token's
//      offset inside the tile (rows 0 .. 31, read once), with f16 dot2 products;
//   4. scores (16-lane DPP sums), the online softmax of the split (log2 units);
//   5. O~ += p^T C_V: each lane accumulates its own tokens' value columns
//      (rescaled only when the running max moves); p moves from the score
//      lanes to the value lanes through 128 bytes of the wavefront's LDS.
// The lanes' O~ shares are summed once per split; (m, l, O~) go to the
// workspace.  headwise_merge_kernel combines the splits by their log-sum-exp
// weights and applies B_Vh.
#include "device_common.h"
#include "qsvd_internal.h"

#include <cmath>
#include <cstdint>

namespace qsvd {
namespace {

constexpr float kLog2eH = 1.4426950408889634f;
constexpr int kHd = 128;         // head dimension of this path
constexpr int kHT = 32;          // tokens per tile
constexpr int kHeadsPerWg = 4;   // one wavefront per head
constexpr int kHwCUs = 256;

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// sum over each aligned group of 16 lanes (xor 1, xor 2, mirror in 8, mirror in 16)
__device__ __forceinline__ float sum16(float v) {
  v = dpp_add<0xB1>(v);
  v = dpp_add<0x4E>(v);
  v = dpp_add<0x141>(v);
  v = dpp_add<0x140>(v);
  return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t hw_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}

struct HeadwiseParams {
  const uint16_t *q;
  const uint8_t *C;
  const uint16_t *BK_t;
  const float *rope_cos, *rope_sin;
  float *part;
  int64_t L;
  int heads, S;
  float scale_log2;
};

// Launch shape of one (rk, rv, RoPE) instance.  Registers a wavefront needs
// (B_Kh fragments, two tile buffers, K accumulators, O~ shares, the rotated
// query, addresses) decide between two wavefronts per SIMD (<= 256) and one
// (<= 512).  The in-tile RoPE rows (32 packed cos / sin pairs a lane) sit in
// LDS when that buys the second wavefront, else in registers; a lone
// wavefront keeps two tiles in flight (three buffers) when its registers allow.
template <int KBK, int KBV, bool ROPE>
struct HwShape {
  static constexpr int kBase = 32 * KBK + 16 * (KBK + KBV) + 8 * KBV + 104;
  static constexpr bool kRowsInLds = ROPE && kBase + 32 > 256 && kBase + 8 <= 256;
  static constexpr int kOcc = kBase + (ROPE ? (kRowsInLds ? 8 : 32) : 0) <= 256 ? 2 : 1;
  static constexpr int kBufs = kOcc == 1 && kBase + (ROPE ? 32 : 0) + 8 * (KBK + KBV) <= 440 ? 3 : 2;
};

// Head dimension held by lane li in column block nb of K: lane li owns
// dimensions 4 li .. 4 li + 3 (blocks 0-3) and 64 + 4 li .. 64 + 4 li + 3
// (blocks 4-7), so a RoPE pair (i, i + 64) sits in one lane and the lane's
// cos / sin values of a position are one 16-byte load.
__device__ __forceinline__ int hw_dim(int nb, int li) { return (nb >> 2) * 64 + 4 * li + (nb & 3); }

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Four (cos, sin) pairs of one table row as f16 pairs (round to nearest even).
__device__ __forceinline__ u32x4 rope_pairs(const float *c, const float *s) {
  const f32x4 cv = *reinterpret_cast<const f32x4 *>(c), sv = *reinterpret_cast<const f32x4 *>(s);
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{cv[j], sv[j]}, h16x2));
  return out;
}

template <int KBK, int KBV, bool ROPE>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(HwShape<KBK, KBV, ROPE>::kOcc, HwShape<KBK, KBV, ROPE>::kOcc)))
void headwise_stream_kernel(HeadwiseParams p) {
  constexpr int RK = 32 * KBK, RV = 32 * KBV, NC = KBK + KBV;
  constexpr int NB = kHd / 16;   // 16-column blocks of K
  constexpr int NBUF = HwShape<KBK, KBV, ROPE>::kBufs;
  constexpr bool RT_LDS = HwShape<KBK, KBV, ROPE>::kRowsInLds;
  __shared__ float pbuf[kHeadsPerWg][kHT];
  // RoPE rows 0 .. 31, the in-tile rotations, as f16 (cos, sin) pairs; shared by the heads
  __shared__ u32x4 rt[RT_LDS ? kHT : 1][16];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int G = (p.heads + kHeadsPerWg - 1) / kHeadsPerWg;
  int task;
  {
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total / 8, rem = total % 8, xcd = id % 8, local = id / 8;
    task = xcd * per + min(xcd, rem) + local;
  }
  const int grp = task % G;
  const int split = (task / G) % p.S;
  const int64_t seq = task / (G * p.S);
  const int h = grp * kHeadsPerWg + wave;
  if constexpr (RT_LDS) {
    for (int i = threadIdx.x; i < kHT * 16; i += blockDim.x) {
      const int row = i / 16, c4 = i % 16;
      const int64_t r = row < p.L ? row : p.L - 1;   // rows past L: never used unmasked
      rt[row][c4] = rope_pairs(p.rope_cos + r * (kHd / 2) + 4 * c4, p.rope_sin + r * (kHd / 2) + 4 * c4);
    }
    __syncthreads();   // the only barrier: before any wavefront leaves
  }
  if (h >= p.heads) return;   // past this point the wavefronts share nothing

  const int64_t L = p.L;
  const int64_t tiles_all = (L + kHT - 1) / kHT;
  const int ntiles = split < tiles_all ? static_cast<int>((tiles_all - split + p.S - 1) / p.S) : 0;
  const int64_t row_bytes = static_cast<int64_t>(p.heads) * (RK + RV) * 2;
  const uint32_t head_off = static_cast<uint32_t>(h * (RK + RV) * 2);
  auto tile_t0 = [&](int it) { return (static_cast<int64_t>(split) + static_cast<int64_t>(it) * p.S) * kHT; };

  // tile registers: [buffer][16-token half][chunk]; chunk c < KBK holds key
  // columns 32 c + 8 lg .. +8, chunk KBK + v value columns 32 v + 8 lg .. +8, of
  // token 16 half + li
  u32x4 tl[NBUF][2][NC];
  auto load_tile = [&](auto BUF, int it) {
    constexpr int bf = decltype(BUF)::value;
    const int64_t t0 = tile_t0(it);
    const __amdgpu_buffer_rsrc_t rc = hw_rsrc(p.C + (seq * L + t0) * row_bytes, (L - t0) * row_bytes);
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t ro = static_cast<uint32_t>((16 * hf + li) * row_bytes) + head_off;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = c < KBK ? 32 * c + 8 * lg : RK + 32 * (c - KBK) + 8 * lg;
        tl[bf][hf][c] = __builtin_amdgcn_raw_buffer_load_b128(rc, ro + col * 2, 0, 0);
      }
    }
  };
  if (ntiles > 0) {
    load_tile(std::integral_constant<int, 0>{}, 0);
    if constexpr (NBUF == 3) load_tile(std::integral_constant<int, 1>{}, min(1, ntiles - 1));
  }

  // B_Kh fragments (B operand: column hw_dim(nb, li), latent rows 32 kb + 8 lg .. +8)
  bf16x8 bk[NB][KBK];
  const uint16_t *bkh = p.BK_t + static_cast<int64_t>(h) * kHd * RK;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int kb = 0; kb < KBK; ++kb)
      bk[nb][kb] = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const u32x4 *>(bkh + hw_dim(nb, li) * RK + 32 * kb + 8 * lg));

  // rotated query scaled by softmax_scale log2(e), this lane's dimensions
  float qr[NB];
  {
    const uint16_t *qh = p.q + (seq * p.heads + h) * kHd;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * li + j;
      const float x0 = bf16_to_f32(qh[i]), x1 = bf16_to_f32(qh[i + kHd / 2]);
      float y0 = x0, y1 = x1;
      if constexpr (ROPE) {
        const float c = p.rope_cos[(L - 1) * (kHd / 2) + i], s = p.rope_sin[(L - 1) * (kHd / 2) + i];
        y0 = fmaf(x0, c, -(x1 * s));
        y1 = fmaf(x1, c, x0 * s);
      }
      qr[j] = y0 * p.scale_log2;
      qr[j + 4] = y1 * p.scale_log2;
    }
  }
  // in-tile RoPE rows in registers: offset o = 16 hf + 4 lg + e of this lane's tokens
  u32x4 ocs[2][4];
  if constexpr (ROPE && !RT_LDS) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t o = 16 * hf + 4 * lg + e;
        const int64_t off = (o < L ? o : L - 1) * (kHd / 2) + 4 * li;
        ocs[hf][e] = rope_pairs(p.rope_cos + off, p.rope_sin + off);
      }
  }

  // RoPE table row of the tile about to be processed (one tile ahead)
  f32x4 rcos = {0.f, 0.f, 0.f, 0.f}, rsin = {0.f, 0.f, 0.f, 0.f};
  if constexpr (ROPE) {
    if (ntiles > 0) {
      const int64_t off0 = tile_t0(0) * (kHd / 2) + 4 * li;
      rcos = *reinterpret_cast<const f32x4 *>(p.rope_cos + off0);
      rsin = *reinterpret_cast<const f32x4 *>(p.rope_sin + off0);
    }
  }
  float m = -INFINITY, l = 0.f;
  float ov[KBV][8];   // this lane's tokens' value columns 32 v + 8 lg + c, summed over tiles
#pragma unroll
  for (int v = 0; v < KBV; ++v)
#pragma unroll
    for (int c = 0; c < 8; ++c) ov[v][c] = 0.f;

  auto body = [&](auto BUF, int it) {
    constexpr int bf = decltype(BUF)::value;
    const int64_t t0 = tile_t0(it);
    // RoPE: rot(K_t, t) . rot(q, L - 1) = K_t . R(-o) y with y = R(-t0) rot(q, L - 1)
    // for token t = t0 + o; rotations by position compose (angles are t theta_i),
    // so a tile reads table row t0 besides the in-tile rows 0 .. 31 held all along
    // (y0, y1) and (y1, -y0) as f16 pairs: R(-o) y is then two dot2 products
    // with the f16 (cos, sin) pair of the offset
    h16x2 ya[4], yb[4];
    if constexpr (ROPE) {
      // table row t0, loaded one tile ahead
      const f32x4 c0 = rcos, s0 = rsin;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float y0 = fmaf(qr[j], c0[j], qr[j + 4] * s0[j]);
        const float y1 = fmaf(qr[j + 4], c0[j], -(qr[j] * s0[j]));
        ya[j] = __builtin_convertvector(f32x2{y0, y1}, h16x2);
        yb[j] = __builtin_convertvector(f32x2{y1, -y0}, h16x2);
      }
      // the next tile's row, requested before the tile prefetch below: vector
      // loads complete in order, so a row requested after the prefetch and used
      // at the start of the next tile would make that tile wait for the
      // prefetch as well
      const int64_t offn = tile_t0(min(it + 1, ntiles - 1)) * (kHd / 2) + 4 * li;
      rcos = *reinterpret_cast<const f32x4 *>(p.rope_cos + offn);
      rsin = *reinterpret_cast<const f32x4 *>(p.rope_sin + offn);
    }
    // tile it + NBUF - 1 into the buffer freed by tile it - 1 (past the end: a
    // repeat of the last tile, never used)
    load_tile(std::integral_constant<int, (bf + NBUF - 1) % NBUF>{}, min(it + NBUF - 1, ntiles - 1));

    float sc[2][4];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // K = C_K B_Kh; element e of lane: token 16 hf + 4 lg + e, dimension hw_dim(nb, li)
      f32x4 kacc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBK; ++kb)
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, tl[bf][hf][kb]), bk[nb][kb], a,
                                                      0, 0, 0);
        kacc[nb] = a;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float s = 0.f;
        if constexpr (ROPE) {
          // rotation by the in-tile offset o = 16 hf + 4 lg + e
          u32x4 cs;
          if constexpr (RT_LDS)
            cs = rt[16 * hf + 4 * lg + e][li];
          else
            cs = ocs[hf][e];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t csw = cs[j];   // a named scalar: bit_cast of a vector element reads element 0
            const h16x2 csj = __builtin_bit_cast(h16x2, csw);
            const float z0 = __builtin_amdgcn_fdot2(ya[j], csj, 0.f, false);   // y0 c + y1 s
            const float z1 = __builtin_amdgcn_fdot2(yb[j], csj, 0.f, false);   // y1 c - y0 s
            s = fmaf(kacc[j][e], z0, s);
            s = fmaf(kacc[j + 4][e], z1, s);
          }
        } else {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s = fmaf(kacc[nb][e], qr[nb], s);
        }
        sc[hf][e] = sum16(s);
      }
    }
    if (t0 + kHT > L) {   // the partial last tile: tokens past L drop out
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (t0 + 16 * hf + 4 * lg + e >= L) sc[hf][e] = -INFINITY;
    }

    // ---- online softmax over the 32 tokens (each score sits in 16 lanes)
    float mx = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, sc[hf][e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float m_new = fmaxf(m, mx);   // finite: the first token of a tile is < L
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    float psum = 0.f;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pe = __builtin_amdgcn_exp2f(sc[hf][e] - m_new);   // 0 for masked tokens
        sc[hf][e] = pe;
        psum += pe;
      }
    psum += __shfl_xor(psum, 16, kWave);
    psum += __shfl_xor(psum, 32, kWave);
    l = fmaf(l, alpha, psum);
    m = m_new;

    // ---- p to the value lanes: lane li owns tokens li and 16 + li
    if (li == 0) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int e = 0; e < 4; ++e) pbuf[wave][16 * hf + 4 * lg + e] = sc[hf][e];
    }
    __builtin_amdgcn_wave_barrier();
    const float p0 = pbuf[wave][li], p1 = pbuf[wave][16 + li];
    __builtin_amdgcn_wave_barrier();

    // ---- O~ = alpha O~ + p^T C_V over this lane's two tokens
    if (alpha < 1.f) {   // the running max moved (uniform over the wavefront)
#pragma unroll
      for (int v = 0; v < KBV; ++v)
#pragma unroll
        for (int c = 0; c < 8; ++c) ov[v][c] *= alpha;
    }
#pragma unroll
    for (int v = 0; v < KBV; ++v) {
      const u32x4 w0 = tl[bf][0][KBK + v], w1 = tl[bf][1][KBK + v];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        ov[v][2 * c] = fmaf(p1, __uint_as_float(w1[c] << 16), fmaf(p0, __uint_as_float(w0[c] << 16), ov[v][2 * c]));
        ov[v][2 * c + 1] = fmaf(p1, __uint_as_float(w1[c] & 0xFFFF0000u),
                                fmaf(p0, __uint_as_float(w0[c] & 0xFFFF0000u), ov[v][2 * c + 1]));
      }
    }
  };

  for (int it = 0; it < ntiles; it += NBUF) {
    body(std::integral_constant<int, 0>{}, it);
    if (it + 1 < ntiles) body(std::integral_constant<int, 1>{}, it + 1);
    if constexpr (NBUF == 3)
      if (it + 2 < ntiles) body(std::integral_constant<int, 2 % NBUF>{}, it + 2);
  }

  // ---- the split's partial state: O~ summed over the 16 lanes (tokens) of each group
  float *dst = p.part + ((seq * p.S + split) * p.heads + h) * (RV + 4);
#pragma unroll
  for (int v = 0; v < KBV; ++v)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float t = sum16(ov[v][c]);
      if (li == 0) dst[4 + 32 * v + 8 * lg + c] = t;
    }
  if (lane == 0) {
    dst[0] = m;
    dst[1] = l;
    dst[2] = 0.f;
    dst[3] = 0.f;
  }
}

// One wavefront per (sequence, head): O~ = sum_s 2^(m_s - M) O~_s / sum_s 2^(m_s - M) l_s,
// then O = O~ B_Vh.  Splits are spread over the lanes for the max and the
// denominator; lane c then sums column c of O~ over the splits.
template <typename OT, int RV>
__global__ __launch_bounds__(256) void headwise_merge_kernel(const float *__restrict__ part,
                                                             const uint16_t *__restrict__ BV,
                                                             OT *__restrict__ O, int b, int heads, int S) {
  constexpr int PW = RV + 4;
  constexpr int SB = 8;                            // splits whose loads are issued together
  constexpr int CPL = (RV + kWave - 1) / kWave;    // O~ columns per lane
  __shared__ float om[4][RV];
  const int wl = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + wl;
  if (w >= b * heads) return;   // uniform per wavefront; the LDS use below is wave-local
  const int seq = w / heads, h = w % heads;
  const float *base = part + (static_cast<int64_t>(seq) * S * heads + h) * PW;
  const int64_t sstride = static_cast<int64_t>(heads) * PW;
  // One round of loads: (m, l) and the O~ row of the first SB splits (split
  // indices past S reread the last split and are not used), and B_Vh as
  // column pairs (lane: output columns 2 lane, 2 lane + 1 of every row).
  float mv[SB], lv[SB], pr[SB][CPL];
#pragma unroll
  for (int k = 0; k < SB; ++k) {
    const float *src = base + min(k, S - 1) * sstride;
    mv[k] = src[0];
    lv[k] = src[1];
#pragma unroll
    for (int c = 0; c < CPL; ++c) pr[k][c] = src[4 + min(lane + kWave * c, RV - 1)];
  }
  const uint32_t *bv = reinterpret_cast<const uint32_t *>(BV + static_cast<int64_t>(h) * RV * kHd);
  uint32_t wv[RV];
#pragma unroll
  for (int c = 0; c < RV; ++c) wv[c] = bv[c * (kHd / 2) + lane];
  // log-sum-exp weights 2^(m_s - M) (every lane holds every split's (m, l))
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < SB; ++k)
    if (k < S) M = fmaxf(M, mv[k]);
  for (int s = SB; s < S; ++s) M = fmaxf(M, base[s * sstride]);
  float den = 0.f, acc[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
#pragma unroll
  for (int k = 0; k < SB; ++k) {
    if (k < S) {
      const float wgt = mv[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv[k] - M);
      den = fmaf(wgt, lv[k], den);
#pragma unroll
      for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wgt, pr[k][c], acc[c]);
    }
  }
  for (int s = SB; s < S; ++s) {
    const float *src = base + s * sstride;
    const float ms = src[0];
    const float wgt = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    den = fmaf(wgt, src[1], den);
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = fmaf(wgt, src[4 + min(lane + kWave * c, RV - 1)], acc[c]);
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int c = 0; c < CPL; ++c)
    if (lane + kWave * c < RV) om[wl][lane + kWave * c] = acc[c] * inv;
  __builtin_amdgcn_wave_barrier();
  // o_h = O~_h B_Vh
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int c = 0; c < RV; ++c) {
    const float oc = om[wl][c];
    a0 = fmaf(oc, __uint_as_float(wv[c] << 16), a0);
    a1 = fmaf(oc, __uint_as_float(wv[c] & 0xFFFF0000u), a1);
  }
  OT *out = O + (static_cast<int64_t>(seq) * heads + h) * kHd + 2 * lane;
  if constexpr (sizeof(OT) == 2) {
    *reinterpret_cast<uint32_t *>(out) = pack_bf16x2(a0, a1);
  } else {
    *reinterpret_cast<float2 *>(out) = float2{a0, a1};
  }
}

template <typename OT>
hipError_t launch_hw_merge(const float *part, const void *BV, void *O, int b, int heads, int S, int rv,
                           hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((b * heads + 3) / 4)), block(256);
  const uint16_t *bv = static_cast<const uint16_t *>(BV);
  OT *o = static_cast<OT *>(O);
  switch (rv) {
    case 32: headwise_merge_kernel<OT, 32><<<grid, block, 0, s>>>(part, bv, o, b, heads, S); break;
    case 64: headwise_merge_kernel<OT, 64><<<grid, block, 0, s>>>(part, bv, o, b, heads, S); break;
    case 96: headwise_merge_kernel<OT, 96><<<grid, block, 0, s>>>(part, bv, o, b, heads, S); break;
    default: headwise_merge_kernel<OT, 128><<<grid, block, 0, s>>>(part, bv, o, b, heads, S); break;
  }
  return hipGetLastError();
}

template <int KBK, int KBV>
hipError_t launch_hw_t(const HeadwiseParams &hp, bool rope, int grid, hipStream_t s) {
  if (rope)
    headwise_stream_kernel<KBK, KBV, true><<<dim3(grid), dim3(256), 0, s>>>(hp);
  else
    headwise_stream_kernel<KBK, KBV, false><<<dim3(grid), dim3(256), 0, s>>>(hp);
  return hipGetLastError();
}

template <int KBK>
hipError_t launch_hw_k(const HeadwiseParams &hp, int rv, bool rope, int grid, hipStream_t s) {
  switch (rv) {
    case 32: return launch_hw_t<KBK, 1>(hp, rope, grid, s);
    case 64: return launch_hw_t<KBK, 2>(hp, rope, grid, s);
    case 96: return launch_hw_t<KBK, 3>(hp, rope, grid, s);
    default: return launch_hw_t<KBK, 4>(hp, rope, grid, s);
  }
}

}  // namespace

int headwise_splits(int b, int64_t L, int heads, int splits) {
  const int64_t tiles = (L + kHT - 1) / kHT;
  const int64_t groups = static_cast<int64_t>(b) * ((heads + kHeadsPerWg - 1) / kHeadsPerWg);
  int64_t S = splits > 0 ? splits : std::max<int64_t>(1, kHwCUs * 2 / std::max<int64_t>(groups, 1));
  S = std::min<int64_t>(std::min<int64_t>(S, tiles), 1024);
  return static_cast<int>(std::max<int64_t>(S, 1));
}

size_t headwise_workspace_bytes(int b, int64_t L, int heads, int rv, int splits) {
  const int S = headwise_splits(b, L, heads, splits);
  return static_cast<size_t>(b) * S * heads * (rv + 4) * sizeof(float);
}

hipError_t launch_decode_headwise(const HeadwiseArgs &a, hipStream_t s) {
  const int S = headwise_splits(a.b, a.L, a.heads, a.splits);
  const int G = (a.heads + kHeadsPerWg - 1) / kHeadsPerWg;
  const int grid = a.b * S * G;
  HeadwiseParams hp{};
  hp.q = static_cast<const uint16_t *>(a.q);
  hp.C = static_cast<const uint8_t *>(a.C);
  hp.BK_t = static_cast<const uint16_t *>(a.BK_t);
  hp.rope_cos = a.rope_cos;
  hp.rope_sin = a.rope_sin;
  hp.part = static_cast<float *>(a.workspace);
  hp.L = a.L;
  hp.heads = a.heads;
  hp.S = S;
  hp.scale_log2 = a.softmax_scale * kLog2eH;
  hipError_t e;
  {
    LaunchTimer t("headwise_stream", s);
    const bool rope = a.rope_cos != nullptr;
    switch (a.rk) {
      case 32: e = launch_hw_k<1>(hp, a.rv, rope, grid, s); break;
      case 64: e = launch_hw_k<2>(hp, a.rv, rope, grid, s); break;
      case 96: e = launch_hw_k<3>(hp, a.rv, rope, grid, s); break;
      default: e = launch_hw_k<4>(hp, a.rv, rope, grid, s); break;
    }
    if (e != hipSuccess) return e;
  }
  LaunchTimer t("headwise_merge", s);
  if (a.o_dtype == QSVD_BF16) return launch_hw_merge<uint16_t>(hp.part, a.BV, a.O, a.b, a.heads, S, a.rv, s);
  return launch_hw_merge<float>(hp.part, a.BV, a.O, a.b, a.heads, S, a.rv, s);
}

}  // namespace qsvd
