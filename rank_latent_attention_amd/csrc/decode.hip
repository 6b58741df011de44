// Split-L flash decoding over the shared QKV latent cache (gfx950).
//
// QSVD paper notes (NeurIPS 2025), "Key design": only C_qkv = X W^d (r values
// per token) is cached; K = C W^u_k and V = C W^u_v are rebuilt on demand.
// The WSVD digest ("Problem") shows why this must be streamed carefully: a
// kernel that reloads the shared latent once per head moves L*R bytes per head
// and loses to plain flash decoding.  Here every workgroup reads its slice of
// C once for all the heads it owns, and the attention runs in the latent
// space, which is the same function by associativity:
//
//   decode_absorb   q~[b][h][:] = (softmax_scale * log2 e) * W^u_k,h q[b][h]
//   decode_stream   per (sequence, L-split, head group): for each token tile
//                   S = C_tile q~^T (scores of all heads), online softmax,
//                   O~ <- O~ * alpha + P^T C_tile; writes (m, l, O~ / l)
//   decode_merge    per (head, 128-row chunk of r): log-sum-exp merge of the
//                   splits and the chunk's share of O~ W^u_v,h
//   decode_finalize sum of the chunk shares -> O
//
// The WSVD digest ("Method, 3.4") folds the value up-projection into the
// output side in the same way; K and V never exist in memory.
//
// MFMA stream kernel layout (bf16 / int4 / int8 caches).  A workgroup has W
// wavefronts; wavefront w owns latent columns [w*rw, (w+1)*rw) of every token
// (rw = r / W).  Per tile of T tokens:
//   1. the wavefront moves its C slice (T x rw) from HBM through registers
//      (128-bit loads, next tile prefetched) into a wavefront-private LDS
//      region, dequantising int4/int8 codes to bf16 on the way;
//   2. partial scores over its columns: v_mfma_f32_16x16x32_bf16 with the
//      C rows as A and the absorbed queries (kept in registers) as B;
//   3. partial scores are summed across wavefronts through LDS; the owners of
//      each head do the online-softmax bookkeeping and write P (bf16);
//   4. O~ (heads x rw, float32, in registers) is rescaled and accumulates
//      P^T C_tile with C read transposed from LDS (16x16x32 for T = 32,
//      16x16x16 for T = 16).
#include "device_common.h"
#include "qsvd_internal.h"

#include <cmath>

namespace qsvd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNumCU = 256;  // MI355X compute units
constexpr int kMergeRows = 128;
constexpr int kMaxSplits = 1024;

enum CType : int { CT_BF16 = 0, CT_I4 = 1, CT_I8 = 2 };

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void compiler_fence() { __atomic_signal_fence(__ATOMIC_SEQ_CST); }

// ------------------------------------------------------------------ absorb
// q~[b][h][j] = scale * sum_i Wk[j][h d + i] * q[b][h][i].  One workgroup owns
// 16 rows j of one head; 16 lanes split the d-wide row segment.
template <typename QT, typename WT, typename OT, int EPP>
__global__ __launch_bounds__(256) void absorb_kernel(const QT *__restrict__ q,
                                                     const WT *__restrict__ Wk,
                                                     const float *__restrict__ wscale,
                                                     OT *__restrict__ qt, int b, int r, int heads,
                                                     int d, float scale) {
  constexpr int BB = 32;          // sequences staged in LDS per pass
  __shared__ float qs[BB * 256];  // [BB][d], d <= 256
  const int h = blockIdx.y;
  const int E = heads * d;
  const int jj = threadIdx.x >> 4, part = threadIdx.x & 15;
  const int j = blockIdx.x * 16 + jj;
  const bool valid = j < r;
  float w[EPP];
#pragma unroll
  for (int e = 0; e < EPP; ++e) {
    const int col = h * d + part * EPP + e;
    float v = 0.f;
    if (valid) {
      if constexpr (sizeof(WT) == 2)
        v = bf16_to_f32(Wk[static_cast<int64_t>(j) * E + col]);
      else
        v = static_cast<float>(Wk[static_cast<int64_t>(j) * E + col]);
    }
    w[e] = v;
  }
  for (int b0 = 0; b0 < b; b0 += BB) {
    const int nbb = min(BB, b - b0);
    __syncthreads();
    for (int idx = threadIdx.x; idx < nbb * d; idx += blockDim.x) {
      const int bb = b0 + idx / d, i = idx % d;
      float v;
      if constexpr (sizeof(QT) == 2)
        v = bf16_to_f32(q[(static_cast<int64_t>(bb) * heads + h) * d + i]);
      else
        v = q[(static_cast<int64_t>(bb) * heads + h) * d + i];
      if (wscale) v = v * wscale[h * d + i];
      qs[idx] = v;
    }
    __syncthreads();
    for (int bi = 0; bi < nbb; ++bi) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < EPP; ++e) acc = fmaf(w[e], qs[bi * d + part * EPP + e], acc);
      acc = group_sum<16>(acc);
      if (valid && part == 0) {
        const int64_t o = (static_cast<int64_t>(b0 + bi) * heads + h) * r + j;
        if constexpr (sizeof(OT) == 2)
          qt[o] = f32_to_bf16(acc * scale);
        else
          qt[o] = acc * scale;
      }
    }
  }
}

// MFMA form for bf16 queries (d % 32 == 0): per head, Q~_h[b][j] = q_h[b][:] . W^u_k[j][h d:(h+1) d]
// is a [16 sequences x d] x [d x 16 rows] product per v_mfma_f32_16x16x32_bf16
// chain.  Workgroup = (64 rows j, head h, 16 sequences); wavefront = 16 rows.
// int8 W^u_k codes convert exactly to bf16; their column scales multiply q.
template <typename WT>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t *__restrict__ q,
                                                          const WT *__restrict__ Wk,
                                                          const float *__restrict__ wscale,
                                                          uint16_t *__restrict__ qt, int b, int r,
                                                          int heads, int d, float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, b0 = blockIdx.z * 16;
  const int j0 = blockIdx.x * 64 + wave * 16;
  const int64_t E = static_cast<int64_t>(heads) * d;
  const int bb = b0 + (lane & 15);
  const int j = j0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < d; k0 += 32) {
    const int i = k0 + kq;
    u32x4 av = {0u, 0u, 0u, 0u}, bv = {0u, 0u, 0u, 0u};
    if (bb < b) {
      av = *reinterpret_cast<const u32x4 *>(q + (static_cast<int64_t>(bb) * heads + h) * d + i);
      if (wscale) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __uint_as_float(av[e] << 16) * wscale[h * d + i + 2 * e];
          const float hi = __uint_as_float(av[e] & 0xFFFF0000u) * wscale[h * d + i + 2 * e + 1];
          av[e] = pack_bf16x2(lo, hi);
        }
      }
    }
    if (j < r) {
      if constexpr (sizeof(WT) == 2) {
        bv = *reinterpret_cast<const u32x4 *>(Wk + static_cast<int64_t>(j) * E + h * d + i);
      } else {
        const u32x2 c = *reinterpret_cast<const u32x2 *>(Wk + static_cast<int64_t>(j) * E + h * d + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t word = c[e >> 1];
          const int sh = 16 * (e & 1);
          const int c0 = static_cast<int>(word << (24 - sh)) >> 24;
          const int c1 = static_cast<int>(word << (16 - sh)) >> 24;
          bv[e] = pack_bf16x2(static_cast<float>(c0), static_cast<float>(c1));
        }
      }
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                  __builtin_bit_cast(bf16x8, bv), acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bo = b0 + 4 * (lane >> 4) + e;
    if (bo < b && j < r) qt[(static_cast<int64_t>(bo) * heads + h) * r + j] = f32_to_bf16(acc[e] * scale);
  }
}

// ------------------------------------------------------------------ float32 stream
// One workgroup per (split, head, sequence); four wavefronts take every fourth
// token of the split, each with its own online-softmax state, combined at the end.
template <int MAXJ>
__global__ __launch_bounds__(256) void stream_f32_kernel(const float *__restrict__ C,
                                                         const float *__restrict__ qt,
                                                         float *__restrict__ opart,
                                                         float *__restrict__ ml, int64_t L, int r,
                                                         int heads, int S, int64_t chunk) {
  extern __shared__ float sm[];  // qs[r] | wo[4][r] | wm[4] | wl[4]
  float *qs = sm;
  float *wo = sm + r;
  float *wm = wo + 4 * r;
  float *wl = wm + 4;
  const int split = blockIdx.x, h = blockIdx.y, seq = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int j = threadIdx.x; j < r; j += blockDim.x)
    qs[j] = qt[(static_cast<int64_t>(seq) * heads + h) * r + j];
  __syncthreads();
  float qv[MAXJ], o[MAXJ];
#pragma unroll
  for (int k = 0; k < MAXJ; ++k) {
    const int j = lane + 64 * k;
    qv[k] = (j < r) ? qs[j] : 0.f;
    o[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int64_t t0 = split * chunk;
  const int64_t t1 = min(L, t0 + chunk);
  for (int64_t t = t0 + wave; t < t1; t += 4) {
    const float *row = C + (static_cast<int64_t>(seq) * L + t) * r;
    float c[MAXJ];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < MAXJ; ++k) {
      const int j = lane + 64 * k;
      c[k] = (j < r) ? row[j] : 0.f;
      s = fmaf(c[k], qv[k], s);
    }
    s = group_sum<64>(s);
    const float mn = fmaxf(m, s);
    const float alpha = exp2f(m - mn);
    const float p = exp2f(s - mn);
    l = fmaf(l, alpha, p);
#pragma unroll
    for (int k = 0; k < MAXJ; ++k) o[k] = fmaf(o[k], alpha, p * c[k]);
    m = mn;
  }
#pragma unroll
  for (int k = 0; k < MAXJ; ++k) {
    const int j = lane + 64 * k;
    if (j < r) wo[wave * r + j] = o[k];
  }
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = l;
  }
  __syncthreads();
  float M = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
  float f[4], Lt = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[w] = (M == -INFINITY) ? 0.f : exp2f(wm[w] - M);
    Lt = fmaf(wl[w], f[w], Lt);
  }
  const int64_t pidx = (static_cast<int64_t>(seq) * S + split) * heads + h;
  for (int j = threadIdx.x; j < r; j += blockDim.x) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) acc = fmaf(wo[w * r + j], f[w], acc);
    opart[pidx * r + j] = (Lt > 0.f) ? acc / Lt : 0.f;
  }
  if (threadIdx.x == 0) {
    ml[2 * pidx] = M;
    ml[2 * pidx + 1] = Lt;
  }
}

// ------------------------------------------------------------------ MFMA stream
struct StreamParams {
  const uint8_t *C;
  const float *c_scales;
  const uint16_t *qt;  // bf16 [b][heads][r]
  uint16_t *opart;     // bf16 [b][S][heads][r]
  float *ml;           // [b][S][heads][2]
  int64_t L;
  int r;
  int heads;
  int S;
  int64_t chunk;
  int G;            // head groups
  int group_heads;  // heads per group (last may be smaller)
  int nb;           // 16-column blocks per wavefront
  int ntasks;
};

template <int CT>
struct CacheTraits;
template <>
struct CacheTraits<CT_BF16> {
  static constexpr int kElemsPerUnit = 8;  // 16 bytes
  static constexpr int kUnitBytes = 16;
};
template <>
struct CacheTraits<CT_I4> {
  static constexpr int kElemsPerUnit = 16;  // 8 bytes
  static constexpr int kUnitBytes = 8;
};
template <>
struct CacheTraits<CT_I8> {
  static constexpr int kElemsPerUnit = 16;  // 16 bytes
  static constexpr int kUnitBytes = 16;
};

__host__ __device__ constexpr int lds_row_stride(int rw) { return rw * 2 + 16; }

__host__ __device__ constexpr size_t stream_lds_bytes(int W, int T, int rw, int HGP) {
  return static_cast<size_t>(W) * T * lds_row_stride(rw) +            // C tiles
         static_cast<size_t>(W) * (T / 16) * (HGP / 16) * 64 * 16 +  // partial scores
         static_cast<size_t>(HGP / 16) * 64 * (T / 4) * 2 +          // P
         static_cast<size_t>(HGP) * 4 * 3;                           // alpha, m, l
}

template <int CT, int HGP, int MAXNB, int T>
__global__ __launch_bounds__(512) void stream_mfma_kernel(StreamParams p) {
  using Tr = CacheTraits<CT>;
  constexpr int NHB = HGP / 16;
  constexpr int NTB = T / 16;
  constexpr int KPL = T / 4;          // tokens per lane in the O~ MFMA operand
  constexpr int MAXKB = MAXNB / 2;    // 32-column score K-blocks
  constexpr int MAXU = (T * MAXNB * 16 / Tr::kElemsPerUnit + 63) / 64;  // load units per lane
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = blockDim.x >> 6;
  const int nthreads = blockDim.x;
  const int nb = p.nb, rw = nb * 16, nkb = nb / 2;
  const int RS = lds_row_stride(rw);
  const int r = p.r;

  // XCD-aware task order: workgroup i runs on XCD i % 8; give each XCD a
  // contiguous run of tasks so the head groups of one (sequence, split) share
  // an L2.
  int task;
  {
    const int total = gridDim.x, id = blockIdx.x;
    const int per = total / 8, rem = total % 8, xcd = id % 8, local = id / 8;
    task = xcd * per + min(xcd, rem) + local;
  }
  const int grp = task % p.G;
  const int pair = task / p.G;
  const int split = pair % p.S;
  const int seq = pair / p.S;
  const int h0 = grp * p.group_heads;
  const int hg = min(p.group_heads, p.heads - h0);
  // Split s owns token tiles s, s + S, s + 2S, ...: at any moment the
  // workgroups of one sequence read neighbouring tiles, so the whole GPU
  // streams a few contiguous regions instead of S far-apart ones.
  const int64_t t_end = p.L;
  const int64_t tiles_all = (p.L + T - 1) / T;
  const int ntiles = split < tiles_all ? static_cast<int>((tiles_all - split + p.S - 1) / p.S) : 0;
  const int j0w = wave * rw;

  uint8_t *ct = smem + static_cast<size_t>(wave) * T * RS;
  float *spart = reinterpret_cast<float *>(smem + static_cast<size_t>(W) * T * RS);
  uint16_t *pl = reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(spart) +
                                              static_cast<size_t>(W) * NTB * NHB * 64 * 16);
  float *alpha_s = reinterpret_cast<float *>(pl + NHB * 64 * KPL);
  float *m_s = alpha_s + HGP;
  float *l_s = m_s + HGP;

  // absorbed queries as the B operand of the score MFMA: lane holds
  // q~[h = hb*16 + lane%16][j = kb*32 + (lane/16)*8 .. +8]
  bf16x8 qf[NHB][MAXKB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int kb = 0; kb < MAXKB; ++kb) {
      const int h = hb * 16 + (lane & 15);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (kb < nkb && h < hg) {
        const int j = j0w + kb * 32 + (lane >> 4) * 8;
        v = *reinterpret_cast<const u32x4 *>(
            p.qt + (static_cast<int64_t>(seq) * p.heads + h0 + h) * r + j);
      }
      qf[hb][kb] = __builtin_bit_cast(bf16x8, v);
    }

  f32x4 oacc[NHB][MAXNB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int jb = 0; jb < MAXNB; ++jb) oacc[hb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = tid; i < HGP; i += nthreads) {
    m_s[i] = -INFINITY;
    l_s[i] = 0.f;
  }
  __syncthreads();

  const int units_per_row = rw / Tr::kElemsPerUnit;
  const int nunits = T * units_per_row;

  // ---- tile staging
  u32x4 buf[MAXU];
  float bscale[MAXU];
  // Every lane loads unconditionally: rows past the end of the sequence re-read
  // its last row (their scores are masked to -inf, so P is 0 for them) and
  // units past the slice re-read its last unit (never stored).
  auto load_tile = [&](int64_t tile_t0) {
#pragma unroll
    for (int k = 0; k < MAXU; ++k) {
      const int u = min(lane + 64 * k, nunits - 1);
      const int row = u / units_per_row, col = u % units_per_row;
      const int64_t t = min(tile_t0 + row, t_end - 1);
      const int64_t tok = static_cast<int64_t>(seq) * p.L + t;
      const int j = j0w + col * Tr::kElemsPerUnit;
      if constexpr (CT == CT_BF16) {
        buf[k] = *reinterpret_cast<const u32x4 *>(p.C + (tok * r + j) * 2);
      } else if constexpr (CT == CT_I4) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(p.C + (tok * r + j) / 2);
        buf[k] = u32x4{v.x, v.y, 0u, 0u};
        bscale[k] = p.c_scales[tok * (r / 128) + j / 128];
      } else {
        buf[k] = *reinterpret_cast<const u32x4 *>(p.C + tok * r + j);
        bscale[k] = p.c_scales[tok];
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int k = 0; k < MAXU; ++k) {
      const int u = lane + 64 * k;
      if (u < nunits) {
        const int row = u / units_per_row, col = u % units_per_row;
        uint8_t *dst = ct + row * RS + col * Tr::kElemsPerUnit * 2;
        if constexpr (CT == CT_BF16) {
          *reinterpret_cast<u32x4 *>(dst) = buf[k];
        } else {
          uint32_t out[8];
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            int c0, c1;
            if constexpr (CT == CT_I4) {
              const uint32_t word = buf[k][e >> 3];
              c0 = static_cast<int>(word << (28 - 4 * (e & 7))) >> 28;
              c1 = static_cast<int>(word << (24 - 4 * (e & 7))) >> 28;
            } else {
              const uint32_t word = buf[k][e >> 2];
              c0 = static_cast<int>(word << (24 - 8 * (e & 3))) >> 24;
              c1 = static_cast<int>(word << (16 - 8 * (e & 3))) >> 24;
            }
            out[e >> 1] = pack_bf16x2(static_cast<float>(c0) * bscale[k],
                                      static_cast<float>(c1) * bscale[k]);
          }
          *reinterpret_cast<u32x4 *>(dst) = u32x4{out[0], out[1], out[2], out[3]};
          *reinterpret_cast<u32x4 *>(dst + 16) = u32x4{out[4], out[5], out[6], out[7]};
        }
      }
    }
  };

  const int64_t tile_stride = static_cast<int64_t>(p.S) * T;
  if (ntiles > 0) load_tile(static_cast<int64_t>(split) * T);
  for (int it = 0; it < ntiles; ++it) {
    const int64_t tile_t0 = (static_cast<int64_t>(split) + static_cast<int64_t>(it) * p.S) * T;
    store_tile();
    if (it + 1 < ntiles) load_tile(tile_t0 + tile_stride);
    compiler_fence();

    // ---- partial scores over this wavefront's columns
    f32x4 sacc[NTB][NHB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sacc[tb][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < MAXKB; ++kb) {
      if (kb < nkb) {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(
              ct + (tb * 16 + (lane & 15)) * RS + kb * 64 + (lane >> 4) * 16);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
            sacc[tb][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, a), qf[hb][kb], sacc[tb][hb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        *reinterpret_cast<f32x4 *>(spart + (((wave * NTB + tb) * NHB + hb) * 64 + lane) * 4) =
            sacc[tb][hb];
    __syncthreads();

    // ---- cross-wavefront sum + online softmax; T/2 lanes per head, 2 tokens each
    for (int tau = tid; tau < HGP * (T / 2); tau += nthreads) {
      const int h = tau / (T / 2), u = tau % (T / 2), t0 = 2 * u;
      const int tb = t0 >> 4, hb = h >> 4;
      const int ln = 16 * ((t0 & 15) >> 2) + (h & 15);
      const int i0 = t0 & 3;
      float s0 = 0.f, s1 = 0.f;
      for (int w = 0; w < W; ++w) {
        const float *src = spart + (((w * NTB + tb) * NHB + hb) * 64 + ln) * 4 + i0;
        s0 += src[0];
        s1 += src[1];
      }
      if (tile_t0 + t0 >= t_end) s0 = -INFINITY;
      if (tile_t0 + t0 + 1 >= t_end) s1 = -INFINITY;
      const float mx = group_max<T / 2>(fmaxf(s0, s1));
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = exp2f(m_old - m_new);
      const uint16_t p0 = f32_to_bf16(exp2f(s0 - m_new));
      const uint16_t p1 = f32_to_bf16(exp2f(s1 - m_new));
      const float psum = group_sum<T / 2>(bf16_to_f32(p0) + bf16_to_f32(p1));
      if (u == 0) {
        const float l_old = l_s[h];
        m_s[h] = m_new;
        l_s[h] = fmaf(l_old, alpha, psum);
        alpha_s[h] = alpha;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int t = t0 + e;
        const int g = (t & 15) >> 2, kk = (t >> 4) * 4 + (t & 3);
        pl[(hb * 64 + g * 16 + (h & 15)) * KPL + kk] = e ? p1 : p0;
      }
    }
    __syncthreads();

    // ---- O~ = O~ * alpha + P^T C_tile
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = alpha_s[hb * 16 + 4 * (lane >> 4) + i];
#pragma unroll
      for (int jb = 0; jb < MAXNB; ++jb)
        if (jb < nb)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[hb][jb][i] *= al[i];
    }
    if constexpr (T == 32) {
      bf16x8 pa[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        pa[hb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                pl + (hb * 64 + lane) * KPL));
#pragma unroll
      for (int jb = 0; jb < MAXNB; ++jb) {
        if (jb < nb) {
          const uint16_t *col = reinterpret_cast<const uint16_t *>(ct) + jb * 16 + (lane & 15);
          const int rs2 = RS / 2;
          const int g4 = 4 * (lane >> 4);
          uint32_t w[4];
#pragma unroll
          for (int kk = 0; kk < 8; kk += 2) {
            const int ta = (kk >> 2) * 16 + g4 + (kk & 3);
            w[kk >> 1] = static_cast<uint32_t>(col[ta * rs2]) |
                         (static_cast<uint32_t>(col[(ta + 1) * rs2]) << 16);
          }
          const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
            oacc[hb][jb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[hb], bv, oacc[hb][jb], 0, 0, 0);
        }
      }
    } else {
      bf16x4 pa[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        pa[hb] = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(
                                                pl + (hb * 64 + lane) * KPL));
#pragma unroll
      for (int jb = 0; jb < MAXNB; ++jb) {
        if (jb < nb) {
          const uint16_t *col = reinterpret_cast<const uint16_t *>(ct) + jb * 16 + (lane & 15);
          const int rs2 = RS / 2;
          const int g4 = 4 * (lane >> 4);
          const uint32_t w0 = static_cast<uint32_t>(col[g4 * rs2]) |
                              (static_cast<uint32_t>(col[(g4 + 1) * rs2]) << 16);
          const uint32_t w1 = static_cast<uint32_t>(col[(g4 + 2) * rs2]) |
                              (static_cast<uint32_t>(col[(g4 + 3) * rs2]) << 16);
          const bf16x4 bv = __builtin_bit_cast(bf16x4, u32x2{w0, w1});
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
            oacc[hb][jb] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa[hb], bv, oacc[hb][jb], 0, 0, 0);
        }
      }
    }
    compiler_fence();
  }
  __syncthreads();

  // ---- partial state: O~ / l (bf16) and (m, l)
  const int64_t pbase = (static_cast<int64_t>(seq) * p.S + split) * p.heads + h0;
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = hb * 16 + 4 * (lane >> 4) + i;
      if (h < hg) {
        const float l = l_s[h];
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int jb = 0; jb < MAXNB; ++jb)
          if (jb < nb)
            p.opart[(pbase + h) * r + j0w + jb * 16 + (lane & 15)] =
                f32_to_bf16(oacc[hb][jb][i] * inv);
      }
    }
  for (int h = tid; h < hg; h += nthreads) {
    p.ml[2 * (pbase + h)] = m_s[h];
    p.ml[2 * (pbase + h) + 1] = l_s[h];
  }
}

// ------------------------------------------------------------------ merge
// Workgroup (chunk jc of 128 latent rows, head h, 16 sequences):
//   1. log-sum-exp weights of every split (one wavefront per sequence),
//   2. merged O~ rows of the chunk (16 B partial loads),
//   3. the chunk's share of O~ W^u_v,h in float32 -> opj[jc][b][h][d].
// W^u_v is read once per (chunk, head): the whole grid reads it once.
template <typename PT, typename WT>
__global__ __launch_bounds__(256) void merge_kernel(const PT *__restrict__ opart,
                                                    const float *__restrict__ ml,
                                                    const WT *__restrict__ Wv,
                                                    const float *__restrict__ wscale,
                                                    float *__restrict__ opj, int b, int r,
                                                    int heads, int d, int S) {
  constexpr int BB = 16;
  extern __shared__ float msm[];
  float *wts = msm;                  // [BB][S]
  float *mv = msm + BB * S;          // [BB][kMergeRows]
  const int jc = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * BB;
  const int nbb = min(BB, b - b0);
  const int64_t E = static_cast<int64_t>(heads) * d;
  const int j0 = jc * kMergeRows;
  const int rows = min(kMergeRows, r - j0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int bi = wave; bi < nbb; bi += 4) {
    const int64_t base = static_cast<int64_t>(b0 + bi) * S * heads + h;
    float mx = -INFINITY;
    for (int s = lane; s < S; s += 64) mx = fmaxf(mx, ml[2 * (base + static_cast<int64_t>(s) * heads)]);
    mx = group_max<64>(mx);
    float den = 0.f;
    for (int s = lane; s < S; s += 64) {
      const int64_t o = base + static_cast<int64_t>(s) * heads;
      const float w = (mx == -INFINITY) ? 0.f : exp2f(ml[2 * o] - mx) * ml[2 * o + 1];
      wts[bi * S + s] = w;
      den += w;
    }
    den = group_sum<64>(den);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int s = lane; s < S; s += 64) wts[bi * S + s] *= inv;
  }
  __syncthreads();

  if constexpr (sizeof(PT) == 2) {
    // r % 32 == 0 on this path: 8 consecutive rows per thread, 16-byte loads
    const int bi = tid >> 4, jj0 = (tid & 15) * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (bi < nbb && jj0 < rows) {
      const int64_t base = static_cast<int64_t>(b0 + bi) * S * heads + h;
      for (int s = 0; s < S; ++s) {
        const float w = wts[bi * S + s];
        if (w != 0.f) {
          const u32x4 v = *reinterpret_cast<const u32x4 *>(
              opart + (base + static_cast<int64_t>(s) * heads) * r + j0 + jj0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] = fmaf(w, __uint_as_float(v[e] << 16), acc[2 * e]);
            acc[2 * e + 1] = fmaf(w, __uint_as_float(v[e] & 0xFFFF0000u), acc[2 * e + 1]);
          }
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) mv[bi * kMergeRows + jj0 + e] = acc[e];
  } else {
    for (int idx = tid; idx < BB * kMergeRows; idx += blockDim.x) {
      const int bi = idx / kMergeRows, jj = idx % kMergeRows;
      float acc = 0.f;
      if (bi < nbb && jj < rows) {
        const int64_t base = static_cast<int64_t>(b0 + bi) * S * heads + h;
        for (int s = 0; s < S; ++s) {
          const float w = wts[bi * S + s];
          if (w != 0.f) acc = fmaf(w, opart[(base + static_cast<int64_t>(s) * heads) * r + j0 + jj], acc);
        }
      }
      mv[idx] = acc;
    }
  }
  __syncthreads();

  // thread -> column i of the head, sequences g, g + groups, ...
  const int groups = max(1, 256 / d);
  const int i = tid % d, g = tid / d;
  if (g < groups && i < d) {
    float acc[BB];
#pragma unroll
    for (int k = 0; k < BB; ++k) acc[k] = 0.f;
    const WT *wcol = Wv + static_cast<int64_t>(j0) * E + h * d + i;
    int jj = 0;
    for (; jj + 4 <= rows; jj += 4) {
      float w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if constexpr (sizeof(WT) == 2)
          w[u] = bf16_to_f32(wcol[(jj + u) * E]);
        else
          w[u] = static_cast<float>(wcol[(jj + u) * E]);
      }
#pragma unroll
      for (int k = 0; k < BB; ++k) {
        const int bi = g + k * groups;
        if (bi < nbb) {
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[k] = fmaf(mv[bi * kMergeRows + jj + u], w[u], acc[k]);
        }
      }
    }
    for (; jj < rows; ++jj) {
      float w;
      if constexpr (sizeof(WT) == 2)
        w = bf16_to_f32(wcol[jj * E]);
      else
        w = static_cast<float>(wcol[jj * E]);
#pragma unroll
      for (int k = 0; k < BB; ++k) {
        const int bi = g + k * groups;
        if (bi < nbb) acc[k] = fmaf(mv[bi * kMergeRows + jj], w, acc[k]);
      }
    }
    const float sc = wscale ? wscale[h * d + i] : 1.f;
#pragma unroll
    for (int k = 0; k < BB; ++k) {
      const int bi = g + k * groups;
      if (bi < nbb)
        opj[((static_cast<int64_t>(jc) * b + b0 + bi) * heads + h) * d + i] = acc[k] * sc;
    }
  }
}

template <typename OT>
__global__ __launch_bounds__(256) void finalize_kernel(const float *__restrict__ opj,
                                                       OT *__restrict__ O, int64_t n, int JC) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float acc = 0.f;
  for (int jc = 0; jc < JC; ++jc) acc += opj[static_cast<int64_t>(jc) * n + i];
  if constexpr (sizeof(OT) == 2)
    O[i] = f32_to_bf16(acc);
  else
    O[i] = acc;
}

// ------------------------------------------------------------------ dispatch helpers
struct MfmaShape {
  int W, nb, HGP, MAXNB, T;
};

// Register budget (256 VGPRs per lane at two wavefronts per SIMD): 32-head
// groups up to 8 column blocks per wavefront, 16-head groups up to 18.
MfmaShape mfma_shape(int r, int heads) {
  MfmaShape s{};
  s.W = 1;
  for (int w : {8, 4, 2, 1})
    if (r % (32 * w) == 0) {
      s.W = w;
      break;
    }
  s.nb = r / s.W / 16;
  s.HGP = (heads > 16 && s.nb <= 8) ? 32 : 16;
  s.MAXNB = 0;
  const int cands32[] = {4, 8};
  const int cands16[] = {4, 8, 12, 18};
  if (s.HGP == 32) {
    for (int c : cands32)
      if (s.nb <= c) {
        s.MAXNB = c;
        break;
      }
  } else {
    for (int c : cands16)
      if (s.nb <= c) {
        s.MAXNB = c;
        break;
      }
  }
  s.T = (s.MAXNB <= 12) ? 32 : 16;
  return s;
}

template <int CT, int HGP, int MAXNB, int T>
hipError_t launch_stream_t(const StreamParams &sp, int W, size_t lds, hipStream_t s) {
  auto kern = stream_mfma_kernel<CT, HGP, MAXNB, T>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<dim3(sp.ntasks), dim3(W * 64), lds, s>>>(sp);
  return hipGetLastError();
}

template <int CT>
hipError_t launch_stream_ct(const StreamParams &sp, const MfmaShape &sh, hipStream_t s) {
  const size_t lds = stream_lds_bytes(sh.W, sh.T, sh.nb * 16, sh.HGP);
  if (sh.HGP == 32) {
    if (sh.MAXNB == 4) return launch_stream_t<CT, 32, 4, 32>(sp, sh.W, lds, s);
    return launch_stream_t<CT, 32, 8, 32>(sp, sh.W, lds, s);
  }
  switch (sh.MAXNB) {
    case 4: return launch_stream_t<CT, 16, 4, 32>(sp, sh.W, lds, s);
    case 8: return launch_stream_t<CT, 16, 8, 32>(sp, sh.W, lds, s);
    case 12: return launch_stream_t<CT, 16, 12, 32>(sp, sh.W, lds, s);
    default: return launch_stream_t<CT, 16, 18, 16>(sp, sh.W, lds, s);
  }
}

template <typename QT, typename WT, typename OT, int EPP>
hipError_t run_absorb(dim3 grid, hipStream_t s, const QT *q, const WT *w, const DecodeArgs &a,
                      OT *qt, float scale) {
  absorb_kernel<QT, WT, OT, EPP>
      <<<grid, dim3(256), 0, s>>>(q, w, a.wu_scale_k, qt, a.b, a.r, a.heads, a.d, scale);
  return hipGetLastError();
}

template <int MJ>
hipError_t run_stream_f32(dim3 grid, size_t lds, hipStream_t s, const float *C, const float *q,
                          float *op, float *ml, const DecodeArgs &a, const DecodePlan &p) {
  auto kern = stream_f32_kernel<MJ>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<grid, dim3(256), lds, s>>>(C, q, op, ml, a.L, a.r, a.heads, p.splits, p.chunk);
  return hipGetLastError();
}

template <typename QT, typename WT, typename OT>
hipError_t launch_absorb_t(const DecodeArgs &a, OT *qt, hipStream_t s) {
  const dim3 grid((a.r + 15) / 16, a.heads);
  const float scale = a.softmax_scale * kLog2e;
  const auto *q = static_cast<const QT *>(a.q);
  const auto *w = static_cast<const WT *>(a.Wu_k);
  const int epp = a.d / 16;
  switch (epp) {
    case 1: return run_absorb<QT, WT, OT, 1>(grid, s, q, w, a, qt, scale);
    case 2: return run_absorb<QT, WT, OT, 2>(grid, s, q, w, a, qt, scale);
    case 4: return run_absorb<QT, WT, OT, 4>(grid, s, q, w, a, qt, scale);
    case 8: return run_absorb<QT, WT, OT, 8>(grid, s, q, w, a, qt, scale);
    default: return run_absorb<QT, WT, OT, 16>(grid, s, q, w, a, qt, scale);
  }
}

template <typename PT, typename WT>
hipError_t launch_merge_t(const DecodeArgs &a, const DecodePlan &p, const PT *opart,
                          const float *ml, float *opj, hipStream_t s) {
  const int JC = (a.r + kMergeRows - 1) / kMergeRows;
  const size_t lds = (static_cast<size_t>(16) * p.splits + 16 * kMergeRows) * sizeof(float);
  auto kern = merge_kernel<PT, WT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<dim3(JC, a.heads, (a.b + 15) / 16), dim3(256), lds, s>>>(
      opart, ml, static_cast<const WT *>(a.Wu_v), a.wu_scale_v, opj, a.b, a.r, a.heads, a.d,
      p.splits);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_absorb_mfma(const DecodeArgs &a, uint16_t *qt, hipStream_t s) {
  const dim3 grid((a.r + 63) / 64, a.heads, (a.b + 15) / 16);
  absorb_mfma_kernel<WT><<<grid, dim3(256), 0, s>>>(
      static_cast<const uint16_t *>(a.q), static_cast<const WT *>(a.Wu_k), a.wu_scale_k, qt, a.b,
      a.r, a.heads, a.d, a.softmax_scale * kLog2e);
  return hipGetLastError();
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

DecodePlan plan_decode(int b, int64_t L, int r, int heads, int d, int c_dtype, int splits) {
  DecodePlan p{};
  p.mfma = c_dtype != QSVD_F32;
  int64_t tile = 32;
  if (p.mfma) {
    const MfmaShape sh = mfma_shape(r, heads);
    tile = sh.T;
    const int G = (heads + sh.HGP - 1) / sh.HGP;
    p.head_groups = G;
    p.group_heads = (heads + G - 1) / G;
  } else {
    p.head_groups = heads;
    p.group_heads = 1;
  }
  int64_t S;
  if (p.mfma) {
    // token tiles are dealt round-robin to the splits; no split is left empty
    const int64_t tiles_all = (L + tile - 1) / tile;
    if (splits > 0) {
      S = splits;
    } else {
      const int64_t per = static_cast<int64_t>(b) * p.head_groups;
      S = std::max<int64_t>(1, kNumCU / std::max<int64_t>(per, 1));
    }
    S = std::min<int64_t>(std::min<int64_t>(S, tiles_all), kMaxSplits);
    p.chunk = 0;
    p.splits = static_cast<int>(S);
  } else {
    const int64_t max_splits = std::min<int64_t>(kMaxSplits, L);
    if (splits > 0) {
      S = std::min<int64_t>(splits, max_splits);
      p.chunk = (L + S - 1) / S;
    } else {
      const int64_t per = static_cast<int64_t>(b) * p.head_groups;
      S = std::max<int64_t>(1, kNumCU / std::max<int64_t>(per, 1));
      S = std::max<int64_t>(1, std::min<int64_t>(S, (L + 63) / 64));
      S = std::min<int64_t>(S, max_splits);
      p.chunk = (L + S - 1) / S;
    }
    p.splits = static_cast<int>((L + p.chunk - 1) / p.chunk);
  }
  const size_t esz = p.mfma ? 2 : 4;
  p.qt_bytes = align256(static_cast<size_t>(b) * heads * r * esz);
  const size_t opart = align256(static_cast<size_t>(b) * p.splits * heads * r * esz);
  const size_t ml = align256(static_cast<size_t>(b) * p.splits * heads * 2 * sizeof(float));
  const int JC = (r + kMergeRows - 1) / kMergeRows;
  const size_t opj = align256(static_cast<size_t>(JC) * b * heads * d * sizeof(float));
  p.part_bytes = opart + ml + opj;
  p.total = p.qt_bytes + p.part_bytes;
  return p;
}

hipError_t launch_decode(const DecodeArgs &a, const DecodePlan &p, hipStream_t s) {
  uint8_t *ws = static_cast<uint8_t *>(a.workspace);
  const size_t esz = p.mfma ? 2 : 4;
  void *qt = ws;
  void *opart = ws + p.qt_bytes;
  const size_t opart_bytes = align256(static_cast<size_t>(a.b) * p.splits * a.heads * a.r * esz);
  float *ml = reinterpret_cast<float *>(ws + p.qt_bytes + opart_bytes);
  const size_t ml_bytes = align256(static_cast<size_t>(a.b) * p.splits * a.heads * 2 * sizeof(float));
  float *opj = reinterpret_cast<float *>(ws + p.qt_bytes + opart_bytes + ml_bytes);
  hipError_t e;

  // ---- absorb
  {
    LaunchTimer t("decode_absorb", s);
    if (!p.mfma) {
      e = launch_absorb_t<float, float, float>(a, static_cast<float *>(qt), s);
    } else if (a.d % 32 == 0) {
      if (a.wu_dtype == QSVD_I8)
        e = launch_absorb_mfma<int8_t>(a, static_cast<uint16_t *>(qt), s);
      else
        e = launch_absorb_mfma<uint16_t>(a, static_cast<uint16_t *>(qt), s);
    } else if (a.wu_dtype == QSVD_I8) {
      e = launch_absorb_t<uint16_t, int8_t, uint16_t>(a, static_cast<uint16_t *>(qt), s);
    } else {
      e = launch_absorb_t<uint16_t, uint16_t, uint16_t>(a, static_cast<uint16_t *>(qt), s);
    }
    if (e != hipSuccess) return e;
  }

  // ---- stream
  {
    LaunchTimer t("decode_stream", s);
    if (!p.mfma) {
      const int maxj = (a.r + 63) / 64;
      const dim3 grid(p.splits, a.heads, a.b);
      const size_t lds = static_cast<size_t>(a.r) * 5 * sizeof(float) + 8 * sizeof(float);
      const auto *C = static_cast<const float *>(a.C);
      const auto *q = static_cast<const float *>(qt);
      auto *op = static_cast<float *>(opart);
      if (maxj <= 2) e = run_stream_f32<2>(grid, lds, s, C, q, op, ml, a, p);
      else if (maxj <= 4) e = run_stream_f32<4>(grid, lds, s, C, q, op, ml, a, p);
      else if (maxj <= 8) e = run_stream_f32<8>(grid, lds, s, C, q, op, ml, a, p);
      else if (maxj <= 16) e = run_stream_f32<16>(grid, lds, s, C, q, op, ml, a, p);
      else e = run_stream_f32<64>(grid, lds, s, C, q, op, ml, a, p);
    } else {
      const MfmaShape sh = mfma_shape(a.r, a.heads);
      StreamParams sp{};
      sp.C = static_cast<const uint8_t *>(a.C);
      sp.c_scales = a.c_scales;
      sp.qt = static_cast<const uint16_t *>(qt);
      sp.opart = static_cast<uint16_t *>(opart);
      sp.ml = ml;
      sp.L = a.L;
      sp.r = a.r;
      sp.heads = a.heads;
      sp.S = p.splits;
      sp.chunk = p.chunk;
      sp.G = p.head_groups;
      sp.group_heads = p.group_heads;
      sp.nb = sh.nb;
      sp.ntasks = a.b * p.splits * p.head_groups;
      switch (a.c_dtype) {
        case QSVD_BF16: e = launch_stream_ct<CT_BF16>(sp, sh, s); break;
        case QSVD_I4: e = launch_stream_ct<CT_I4>(sp, sh, s); break;
        default: e = launch_stream_ct<CT_I8>(sp, sh, s); break;
      }
    }
    if (e != hipSuccess) return e;
  }

  // ---- merge
  {
    LaunchTimer t("decode_merge", s);
    if (!p.mfma)
      e = launch_merge_t<float, float>(a, p, static_cast<const float *>(opart), ml, opj, s);
    else if (a.wu_dtype == QSVD_I8)
      e = launch_merge_t<uint16_t, int8_t>(a, p, static_cast<const uint16_t *>(opart), ml, opj, s);
    else
      e = launch_merge_t<uint16_t, uint16_t>(a, p, static_cast<const uint16_t *>(opart), ml, opj,
                                             s);
    if (e != hipSuccess) return e;
  }

  // ---- finalize
  {
    LaunchTimer t("decode_finalize", s);
    const int64_t n = static_cast<int64_t>(a.b) * a.heads * a.d;
    const int JC = (a.r + kMergeRows - 1) / kMergeRows;
    const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
    if (a.o_dtype == QSVD_BF16)
      finalize_kernel<uint16_t><<<grid, block, 0, s>>>(opj, static_cast<uint16_t *>(a.O), n, JC);
    else
      finalize_kernel<float><<<grid, block, 0, s>>>(opj, static_cast<float *>(a.O), n, JC);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace qsvd
