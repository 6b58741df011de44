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
//   decode_merge    per (head, 128-row chunk of r, 16 sequences): log-sum-exp
//                   merge of the splits and the chunk's share of O~ W^u_v,h
//   decode_finalize sum of the chunk shares -> O
//
// The WSVD digest ("Method, 3.4") folds the value up-projection into the
// output side in the same way; K and V never exist in memory.
//
// MFMA stream kernel (bf16 / int8 / int4 caches).  A workgroup has W
// wavefronts; wavefront w owns RW = 32 * NKB latent columns of every token.
// Per tile of 32 tokens:
//   1. the tile's C slice arrives in registers (16-byte loads issued one tile
//      ahead) laid out as the A operand of v_mfma_f32_16x16x32_bf16: lane l
//      holds 8 columns of token l % 16.  Codes of quantised caches are
//      dequantised to bf16 here;
//   2. partial scores over the wavefront's columns: A = C rows, B = absorbed
//      queries (kept in registers for the whole split);
//   3. the same registers go to a wavefront-private LDS tile (row-major), and
//      the loads of the next tile are issued;
//   4. partial scores are summed across wavefronts through LDS; one pass over
//      (head, token pair) does the online-softmax bookkeeping and writes P as
//      the A operand of the value product;
//   5. O~ (heads x RW, float32 accumulators) is rescaled and accumulates
//      P^T C_tile, the C operand read token-major out of LDS with the gfx950
//      transposing load ds_read_b64_tr_b16.
// Two workgroup barriers per tile; the loads of tile i+1 are in flight during
// steps 4-5 of tile i and step 1 of tile i+1 waits for them.
#include "device_common.h"
#include "qsvd_internal.h"

#include <cmath>
#include <cstdlib>
#include <type_traits>

namespace qsvd {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kNumCU = 256;  // MI355X compute units
constexpr int kMergeRows = 128;
constexpr int kMaxSplits = 1024;

enum CType : int { CT_BF16 = 0, CT_I4 = 1, CT_I8 = 2 };

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

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

// MFMA form for bf16 queries (d = 32 DK): per head, Q~_h[b][j] = q_h[b][:] . W^u_k[j][h d:(h+1) d]
// is computed transposed, [16 rows x d] x [d x 16 sequences], DK
// v_mfma_f32_16x16x32_bf16 steps.  Workgroup = (64 rows j, head h, 16 sequences); wavefront = 16 rows.
// All operand loads are issued before the first product.  int8 W^u_k codes
// convert exactly to bf16; their column scales multiply q.
template <typename WT, int DK>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(const uint16_t *__restrict__ q,
                                                          const WT *__restrict__ Wk,
                                                          const float *__restrict__ wscale,
                                                          uint16_t *__restrict__ qt, int b, int r,
                                                          int heads, float scale) {
  constexpr int d = 32 * DK;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.y, b0 = blockIdx.z * 16;
  const int j0 = blockIdx.x * 64 + wave * 16;
  const int64_t E = static_cast<int64_t>(heads) * d;
  const int bb = b0 + (lane & 15);
  const int j = j0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  u32x4 av[DK], bv[DK];
#pragma unroll
  for (int k = 0; k < DK; ++k) {
    const int i = 32 * k + kq;
    av[k] = u32x4{0u, 0u, 0u, 0u};
    bv[k] = u32x4{0u, 0u, 0u, 0u};
    if (bb < b) av[k] = *reinterpret_cast<const u32x4 *>(q + (static_cast<int64_t>(bb) * heads + h) * d + i);
    if (j < r) {
      if constexpr (sizeof(WT) == 2) {
        bv[k] = *reinterpret_cast<const u32x4 *>(Wk + static_cast<int64_t>(j) * E + h * d + i);
      } else {
        const u32x2 c = *reinterpret_cast<const u32x2 *>(Wk + static_cast<int64_t>(j) * E + h * d + i);
        bv[k] = u32x4{c.x, c.y, 0u, 0u};
      }
    }
  }
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < DK; ++k) {
    const int i = 32 * k + kq;
    u32x4 a = av[k], w = bv[k];
    if (wscale) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(a[e] << 16) * wscale[h * d + i + 2 * e];
        const float hi = __uint_as_float(a[e] & 0xFFFF0000u) * wscale[h * d + i + 2 * e + 1];
        a[e] = pack_bf16x2(lo, hi);
      }
    }
    if constexpr (sizeof(WT) == 1) {
#pragma unroll
      for (int e = 3; e >= 0; --e) {
        const uint32_t word = w[e >> 1];
        const int sh = 16 * (e & 1);
        w[e] = pack_bf16x2(static_cast<float>(static_cast<int>(word << (24 - sh)) >> 24),
                           static_cast<float>(static_cast<int>(word << (16 - sh)) >> 24));
      }
    }
    // transposed product: rows j of W^u_k as A, sequences as B, so that a
    // lane ends with 4 consecutive rows j0 + 4 g + (0..3) of sequence b0 + i
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                  __builtin_bit_cast(bf16x8, a), acc, 0, 0, 0);
  }
  const int jo = j0 + 4 * (lane >> 4);
  if (bb < b && jo < r)  // r % 16 == 0: the 4 rows are all valid
    *reinterpret_cast<u32x2 *>(qt + (static_cast<int64_t>(bb) * heads + h) * r + jo) =
        u32x2{pack_bf16x2(acc[0] * scale, acc[1] * scale), pack_bf16x2(acc[2] * scale, acc[3] * scale)};
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
  int G;            // head groups
  int group_heads;  // heads per group (the last group may have fewer)
  int ntasks;
};

// Cache element formats.  A 16-byte load carries EPL elements; they feed KPL
// consecutive 32-wide K blocks of the score product.
template <int CT>
struct CacheTraits;
template <>
struct CacheTraits<CT_BF16> {
  static constexpr int EPL = 8;
  __device__ static int64_t byte_offset(int64_t elem) { return elem * 2; }
};
template <>
struct CacheTraits<CT_I8> {
  static constexpr int EPL = 16;
  __device__ static int64_t byte_offset(int64_t elem) { return elem; }
};
template <>
struct CacheTraits<CT_I4> {
  static constexpr int EPL = 32;
  __device__ static int64_t byte_offset(int64_t elem) { return elem / 2; }
};

__host__ __device__ constexpr int ct_row_stride(int nkb) { return nkb * 64 + 16; }
// partial scores of one wavefront: [NHB * 16 heads][T + 4] float32 (head-major,
// padded so that the 16 heads of one store land in distinct LDS banks)
__host__ __device__ constexpr int sp_row(int T) { return T + 4; }

// LDS bytes of the stream kernel: wavefront C tiles | partial scores | P | alpha, m, l.
__host__ __device__ constexpr size_t stream_lds_bytes(int W, int NHB, int NKB, int T) {
  return static_cast<size_t>(W) * T * ct_row_stride(NKB) +
         static_cast<size_t>(W) * NHB * 16 * sp_row(T) * 4 + static_cast<size_t>(NHB) * 64 * T / 2 +
         static_cast<size_t>(NHB) * 16 * 4 * 3;
}

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t *p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(
          reinterpret_cast<__attribute__((address_space(3))) uint8_t *>(
              reinterpret_cast<uintptr_t>(p))));
  return __builtin_bit_cast(bf16x4, v);
}

// bf16 pair of two float32 values, hardware round-to-nearest-even conversion.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// bf16 pair of two dequantised codes c * s (float32 product, round to nearest even).
__device__ __forceinline__ uint32_t dq_pair(int c0, int c1, float s) {
  return cvt_bf16x2(static_cast<float>(c0) * s, static_cast<float>(c1) * s);
}

// Reductions over aligned groups of N = 8 or 16 lanes with DPP lane swaps
// (xor 1, xor 2, mirror within 8, mirror within 16).
template <int CTRL, bool MAX>
__device__ __forceinline__ float dpp_step(float x) {
  const float y = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
  return MAX ? fmaxf(x, y) : x + y;
}

template <int N, bool MAX>
__device__ __forceinline__ float dpp_reduce(float v) {
  v = dpp_step<0xB1, MAX>(v);   // quad_perm [1,0,3,2]
  v = dpp_step<0x4E, MAX>(v);   // quad_perm [2,3,0,1]
  v = dpp_step<0x141, MAX>(v);  // row_half_mirror
  if constexpr (N >= 16) v = dpp_step<0x140, MAX>(v);  // row_mirror
  if constexpr (N == 32) {      // the neighbouring 16-lane row
    const float y = __shfl_xor(v, 16, 64);
    v = MAX ? fmaxf(v, y) : v + y;
  }
  return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}

// Template parameters: cache format CT, NHB 16-head blocks per workgroup, NKB
// 32-column K blocks per wavefront (RW = 32 NKB columns), T tokens per tile
// (16, 32, or 64 for quantised caches, whose codes stage in few registers),
// D tiles of loads in flight (1 or 2; register staging).  The
// wavefront count W = blockDim.x / 64 <= 8 satisfies r = W * RW.
template <int CT, int NHB, int NKB, int T, int D>
__global__ __launch_bounds__(512) void stream_mfma_kernel(StreamParams p) {
  using Tr = CacheTraits<CT>;
  constexpr int EPL = Tr::EPL;
  constexpr int KPL = EPL / 8;          // K blocks per 16-byte load
  constexpr int NLD = NKB / KPL;        // loads per 16-token row block
  constexpr int NTB = T / 16;           // 16-token row blocks per tile
  constexpr int NJB = NKB * 2;          // 16-column blocks of O~
  constexpr int RW = NKB * 32;          // columns per wavefront
  constexpr int RS = ct_row_stride(NKB);
  constexpr int PPL = T == 16 ? 4 : 8;  // tokens per lane in a value product operand
  constexpr int NKS = T == 16 ? 1 : T / 32;   // 32-token K steps of the value product
  constexpr int SPR = sp_row(T);
  constexpr int HGP = NHB * 16;
  constexpr int MAXW = 8;
  static_assert(NKB % KPL == 0, "wavefront columns must be whole 16-byte loads");
  static_assert(T == 16 || T == 32 || T == 64, "tile");
  static_assert(D == 1 || D == 2, "prefetch depth");
  static_assert(HGP * RW * 2 <= T * RS, "the output rows are staged in the wavefront's C tile");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int W = blockDim.x >> 6;
  const int nthreads = blockDim.x;
  const int r = p.r;
  const int li = lane & 15, lg = lane >> 4;

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
  // Split s owns token tiles s, s + S, s + 2S, ...: the workgroups of one
  // sequence read neighbouring tiles at any moment.
  const int64_t L = p.L;
  const int64_t tiles_all = (L + T - 1) / T;
  const int ntiles = split < tiles_all ? static_cast<int>((tiles_all - split + p.S - 1) / p.S) : 0;
  const int j0w = wave * RW;

  uint8_t *ct = smem + static_cast<size_t>(wave) * T * RS;
  float *spart = reinterpret_cast<float *>(smem + static_cast<size_t>(W) * T * RS);
  uint16_t *pl = reinterpret_cast<uint16_t *>(spart + static_cast<size_t>(W) * HGP * SPR);
  float *alpha_s = reinterpret_cast<float *>(pl + NHB * 64 * (T / 4));
  float *m_s = alpha_s + HGP;
  float *l_s = m_s + HGP;

  // ---- tile loads through buffer resources based at the tile's first row:
  // rows at or past the end of the sequence fall outside the resource and
  // read as zero (their scores are masked to -inf below, so their P is 0).
  const int64_t row_bytes = Tr::byte_offset(r);
  const uint32_t voff0 = static_cast<uint32_t>(li * row_bytes + Tr::byte_offset(j0w + EPL * lg));
  u32x4 stage[D][NTB][NLD];
  float sscale[D][NTB][NLD];
  auto load_rows = [&](auto BUF, int64_t t0, int tb) {
    constexpr int bf = decltype(BUF)::value;
    const int64_t row0 = static_cast<int64_t>(seq) * L + t0;
    const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(p.C + row0 * row_bytes, (L - t0) * row_bytes);
    const uint32_t vo = voff0 + static_cast<uint32_t>(tb * 16 * row_bytes);
#pragma unroll
    for (int ld = 0; ld < NLD; ++ld)
      stage[bf][tb][ld] = __builtin_amdgcn_raw_buffer_load_b128(rc, vo + ld * Tr::byte_offset(32 * KPL), 0, 0);
    if constexpr (CT == CT_I8) {
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.c_scales + row0, (L - t0) * 4);
      const float sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (tb * 16 + li) * 4, 0, 0));
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) sscale[bf][tb][ld] = sc;
    }
    if constexpr (CT == CT_I4) {
      const int groups = r / 128;
      const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(p.c_scales + row0 * groups, (L - t0) * groups * 4);
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld)
        sscale[bf][tb][ld] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rs, ((tb * 16 + li) * groups + (j0w + 128 * ld) / 128) * 4, 0, 0));
    }
  };
  auto tile_start = [&](int it) { return (static_cast<int64_t>(split) + static_cast<int64_t>(it) * p.S) * T; };

  // the first D tiles are requested before anything else
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb)
    if (ntiles > 0) load_rows(std::integral_constant<int, 0>{}, tile_start(0), tb);
  if constexpr (D == 2) {
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
      if (ntiles > 1) load_rows(std::integral_constant<int, D - 1>{}, tile_start(1), tb);
  }

  // Absorbed queries as the B operand of the score product.  K block
  // kb = KPL * ld + s of lane group g covers columns
  // j0w + 32 KPL ld + EPL g + 8 s + (0..7): the order in which the 16-byte
  // cache loads deliver them.
  bf16x8 qf[NHB][NKB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int h = hb * 16 + li;
      const int ld = kb / KPL, s = kb % KPL;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < hg) {
        const int j = j0w + 32 * KPL * ld + EPL * lg + 8 * s;
        v = *reinterpret_cast<const u32x4 *>(p.qt + (static_cast<int64_t>(seq) * p.heads + h0 + h) * r + j);
      }
      qf[hb][kb] = __builtin_bit_cast(bf16x8, v);
    }

  // O~ transposed: oacc[hb][jb] holds columns 16 jb + 4 g + (0..3) of head 16 hb + i
  f32x4 oacc[NHB][NJB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) oacc[hb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = tid; i < HGP; i += nthreads) {
    m_s[i] = -INFINITY;
    l_s[i] = 0.f;
  }
  __syncthreads();

  auto body = [&](auto BUF, int it) {
    constexpr int bf = decltype(BUF)::value;
    const int64_t tile_t0 = tile_start(it);
    const bool more = it + D < ntiles;
    const int64_t next_t0 = tile_start(it + D);

    // ---- 1-3. per 16-token row block: bf16 A operands, partial scores over
    // this wavefront's columns, the rows to LDS, then the loads D tiles ahead
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      u32x4 cv[NKB];
#pragma unroll
      for (int ld = 0; ld < NLD; ++ld) {
        if constexpr (CT == CT_BF16) {
          cv[ld] = stage[bf][tb][ld];
        } else if constexpr (CT == CT_I8) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            uint32_t o[4];
#pragma unroll
            for (int w2 = 0; w2 < 2; ++w2) {
              const uint32_t word = stage[bf][tb][ld][2 * s + w2];
              o[2 * w2] = dq_pair(static_cast<int>(word << 24) >> 24,
                                  static_cast<int>(word << 16) >> 24, sscale[bf][tb][ld]);
              o[2 * w2 + 1] = dq_pair(static_cast<int>(word << 8) >> 24,
                                      static_cast<int>(word) >> 24, sscale[bf][tb][ld]);
            }
            cv[2 * ld + s] = u32x4{o[0], o[1], o[2], o[3]};
          }
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const uint32_t word = stage[bf][tb][ld][s];
            uint32_t o[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              o[e] = dq_pair(static_cast<int>(word << (28 - 8 * e)) >> 28,
                             static_cast<int>(word << (24 - 8 * e)) >> 28, sscale[bf][tb][ld]);
            cv[4 * ld + s] = u32x4{o[0], o[1], o[2], o[3]};
          }
        }
      }
      f32x4 sacc[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
          sacc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, cv[kb]), qf[hb][kb], sacc[hb], 0, 0, 0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int ld = kb / KPL, s = kb % KPL;
        const int jl = 32 * KPL * ld + EPL * lg + 8 * s;
        *reinterpret_cast<u32x4 *>(ct + (tb * 16 + li) * RS + jl * 2) = cv[kb];
      }
      if (more) load_rows(BUF, next_t0, tb);
      // partial scores, head-major: lane holds tokens 16 tb + 4 g + (0..3) of head 16 hb + i
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        *reinterpret_cast<f32x4 *>(spart + (wave * HGP + hb * 16 + li) * SPR + tb * 16 + 4 * lg) = sacc[hb];
    }
    lds_barrier();   // the next tile's loads stay in flight

    // ---- 4. cross-wavefront sum + online softmax; T/2 lanes per head, 2 tokens each
    for (int item = tid; item < HGP * (T / 2); item += nthreads) {
      const int h = item / (T / 2), u = item % (T / 2), t0 = 2 * u;
      float s0 = 0.f, s1 = 0.f;
      // all MAXW reads in flight: rows past W re-read row W-1 and add nothing
      float2 v[MAXW];
#pragma unroll
      for (int w = 0; w < MAXW; ++w)
        v[w] = *reinterpret_cast<const float2 *>(spart + (min(w, W - 1) * HGP + h) * SPR + t0);
#pragma unroll
      for (int w = 0; w < MAXW; ++w) {
        s0 += (w < W) ? v[w].x : 0.f;
        s1 += (w < W) ? v[w].y : 0.f;
      }
      if (tile_t0 + t0 >= L) s0 = -INFINITY;
      if (tile_t0 + t0 + 1 >= L) s1 = -INFINITY;
      const float mx = dpp_reduce<T / 2, true>(fmaxf(s0, s1));
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
      const uint32_t pp = cvt_bf16x2(__builtin_amdgcn_exp2f(s0 - m_new), __builtin_amdgcn_exp2f(s1 - m_new));
      const float psum = dpp_reduce<T / 2, false>(__uint_as_float(pp << 16) + __uint_as_float(pp & 0xFFFF0000u));
      if (u == 0) {
        m_s[h] = m_new;
        l_s[h] = fmaf(l_s[h], alpha, psum);
        alpha_s[h] = alpha;
      }
      // P as the B operand of the value product: K step t / 32 (T >= 32), lane
      // 16 ((t % 32) / PPL) + h % 16, element t % PPL
      const int ks = T == 16 ? 0 : t0 >> 5, tk = T == 16 ? t0 : t0 & 31;
      uint16_t *pdst = pl + ((ks * NHB + (h >> 4)) * 64 + 16 * (tk / PPL) + (h & 15)) * PPL + (tk % PPL);
      *reinterpret_cast<uint32_t *>(pdst) = pp;
    }
    lds_barrier();

    // ---- 5. O~^T = O~^T * alpha + C_tile^T P^T (the rescale is skipped by a
    // wavefront whose heads all kept their running maximum)
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const float al = alpha_s[hb * 16 + li];
      if (__builtin_amdgcn_ballot_w64(al != 1.f) != 0) {
#pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
#pragma unroll
          for (int e = 0; e < 4; ++e) oacc[hb][jb][e] *= al;
      }
    }
    // A operand: column 16 jb + lane % 16, tokens PPL g + (0..PPL-1), by
    // transposing 8-byte reads of 4 tokens each (lane i of a 16-lane group
    // supplies row i / 4 and columns 4 (i % 4) .. +3 of a 4 x 16 block).
    if constexpr (T >= 32) {
#pragma unroll
     for (int ks = 0; ks < NKS; ++ks) {
      // K step ks: tokens 32 ks + PPL g + (0..PPL-1)
      const uint8_t *trb = ct + (32 * ks + PPL * lg + (li >> 2)) * RS + (4 * (li & 3)) * 2;
      bf16x8 pb[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        pb[hb] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(pl + ((ks * NHB + hb) * 64 + lane) * PPL));
      // column blocks in groups of VB: all transposing reads of a group are
      // issued before its products
      constexpr int VB = (NJB % 4 == 0) ? 4 : ((NJB % 3 == 0) ? 3 : 2);
      static_assert(NJB % VB == 0, "column groups");
#pragma unroll
      for (int jg = 0; jg < NJB; jg += VB) {
        bf16x4 lo[VB], hi[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k) {
          lo[k] = lds_read_tr16(trb + (jg + k) * 32);
          hi[k] = lds_read_tr16(trb + 4 * RS + (jg + k) * 32);
        }
#pragma unroll
        for (int k = 0; k < VB; ++k) {
          const bf16x8 av = __builtin_shufflevector(lo[k], hi[k], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
            oacc[hb][jg + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[hb], oacc[hb][jg + k], 0, 0, 0);
        }
      }
     }
    } else {
      const uint8_t *trb = ct + (PPL * lg + (li >> 2)) * RS + (4 * (li & 3)) * 2;
      bf16x4 pb[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        pb[hb] = __builtin_bit_cast(bf16x4, *reinterpret_cast<const u32x2 *>(pl + (hb * 64 + lane) * PPL));
      constexpr int VB = (NJB % 4 == 0) ? 4 : ((NJB % 3 == 0) ? 3 : 2);
      static_assert(NJB % VB == 0, "column groups");
#pragma unroll
      for (int jg = 0; jg < NJB; jg += VB) {
        bf16x4 av[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k) av[k] = lds_read_tr16(trb + (jg + k) * 32);
#pragma unroll
        for (int k = 0; k < VB; ++k)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
            oacc[hb][jg + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[k], pb[hb], oacc[hb][jg + k], 0, 0, 0);
      }
    }
  };

  for (int it = 0; it < ntiles; it += D) {
    body(std::integral_constant<int, 0>{}, it);
    if constexpr (D == 2) {
      if (it + 1 < ntiles) body(std::integral_constant<int, 1>{}, it + 1);
    }
  }
  __syncthreads();

  // ---- partial state: O~ / l in bf16, one contiguous block per wavefront
  // ([sequence][split][wavefront][head][RW]), staged in the wavefront's LDS
  // tile so that the stores are 16-byte and contiguous; and (m, l)
  const int64_t pbase = (static_cast<int64_t>(seq) * p.S + split) * p.heads + h0;
  {
    uint16_t *ot = reinterpret_cast<uint16_t *>(ct);  // [HGP][RW]
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int h = hb * 16 + li;
      const float l = l_s[h];
      const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
        *reinterpret_cast<u32x2 *>(ot + h * RW + jb * 16 + 4 * lg) =
            u32x2{cvt_bf16x2(oacc[hb][jb][0] * inv, oacc[hb][jb][1] * inv),
                  cvt_bf16x2(oacc[hb][jb][2] * inv, oacc[hb][jb][3] * inv)};
    }
    // same-wavefront LDS write -> read, ordered by the LDS queue; the partials
    // stream out with non-temporal stores (written once, read once by the merge)
    uint16_t *dst = p.opart + ((static_cast<int64_t>(seq) * p.S + split) * W + wave) *
                                  static_cast<int64_t>(p.heads) * RW + static_cast<int64_t>(h0) * RW;
    for (int u = lane; u < hg * RW / 8; u += 64)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(ot + u * 8), reinterpret_cast<u32x4 *>(dst + u * 8));
  }
  for (int h = tid; h < hg; h += nthreads) {
    p.ml[2 * (pbase + h)] = m_s[h];
    p.ml[2 * (pbase + h) + 1] = l_s[h];
  }
}

// ------------------------------------------------------------------ MFMA merge
// Workgroup (chunk jc of kMergeRows latent rows, head h, 16 sequences).  All
// global loads are issued up front (one memory round trip):
//   - the chunk of W^u_v,h (kMergeRows x d) into registers (int8 codes are
//     exact in bf16; their column scales multiply the result);
//   - (m, l) of every split (thread = sequence tid / 16, splits tid % 16 + 16 k);
//   - the partial O~ rows of up to kMergeBatch splits (thread = sequence
//     tid / 16, rows 8 (tid % 16) .. +8).
// Then: log-sum-exp weights (16-lane DPP reductions), the merged O~ rows as
// the A operand of v_mfma_f32_16x16x32_bf16 (M = 16 sequences, K = latent
// rows) in LDS, the W chunk to LDS, and O~ W^u_v,h with the B operand read by
// transposing LDS loads -> opj[jc][b][h][:] (float32), summed over the chunks
// by decode_finalize.  W^u_v is read once per (chunk, head, 16 sequences).
constexpr int kMergeBatch = 16;

template <typename WT>
__global__ __launch_bounds__(256) void merge_mfma_kernel(const uint16_t *__restrict__ opart,
                                                         const float *__restrict__ ml,
                                                         const WT *__restrict__ Wv,
                                                         const float *__restrict__ wscale,
                                                         float *__restrict__ opj, int b, int r,
                                                         int heads, int d, int S, int RW) {
  constexpr int BB = 16;
  constexpr int MAXU = kMergeRows * 256 / 8 / 256;  // 8-column W units per thread (d <= 256)
  constexpr int MAXSL = 4;                          // splits per thread held in registers (S <= 64)
  extern __shared__ __attribute__((aligned(16))) uint8_t msm[];
  const int WRS = d * 2 + 16;                                       // W chunk row stride (bytes)
  uint8_t *wl = msm;                                                // [kMergeRows][WRS]
  u32x4 *aop = reinterpret_cast<u32x4 *>(msm + kMergeRows * WRS);   // [kMergeRows/32][64]
  float *wts = reinterpret_cast<float *>(aop + (kMergeRows / 32) * 64);  // [BB][S]
  const int jc = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * BB;
  const int nbb = min(BB, b - b0);
  const int64_t E = static_cast<int64_t>(heads) * d;
  const int j0 = jc * kMergeRows;
  const int rows = min(kMergeRows, r - j0);  // multiple of 32
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int units = d / 8;                   // 8-column units per row
  const int bi = tid >> 4, sl = tid & 15, jj0 = sl * 8;
  const int bseq = b0 + min(bi, nbb - 1);
  const bool rvalid = bi < nbb && jj0 < rows;

  // ---- all loads
  u32x4 wreg[MAXU];
#pragma unroll
  for (int k = 0; k < MAXU; ++k) {
    const int u = tid + 256 * k;
    wreg[k] = u32x4{0u, 0u, 0u, 0u};
    if (u < rows * units) {
      const int row = u / units, c8 = (u % units) * 8;
      const WT *src = Wv + static_cast<int64_t>(j0 + row) * E + static_cast<int64_t>(h) * d + c8;
      if constexpr (sizeof(WT) == 2) {
        wreg[k] = *reinterpret_cast<const u32x4 *>(src);
      } else {
        const u32x2 c = *reinterpret_cast<const u32x2 *>(src);
        wreg[k] = u32x4{c.x, c.y, 0u, 0u};
      }
    }
  }
  const int64_t mlbase = static_cast<int64_t>(bseq) * S * heads + h;
  float2 mlv[MAXSL];
#pragma unroll
  for (int k = 0; k < MAXSL; ++k) {
    const int s = sl + 16 * k;
    mlv[k] = (s < S) ? *reinterpret_cast<const float2 *>(ml + 2 * (mlbase + static_cast<int64_t>(s) * heads))
                     : float2{-INFINITY, 0.f};
  }
  // partial rows of (sequence, split, head): wavefront-blocked layout
  // [sequence][split][r / RW][head][RW]; consecutive splits are heads * r apart
  const int jrow = j0 + min(jj0, rows - 8);
  const uint16_t *psrc = opart + (static_cast<int64_t>(bseq) * S * (r / RW) + jrow / RW) * heads * RW +
                         static_cast<int64_t>(h) * RW + jrow % RW;
  const int64_t sstride = static_cast<int64_t>(heads) * r;
  u32x4 pv[kMergeBatch];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    pv[k] = u32x4{0u, 0u, 0u, 0u};
    if (rvalid && k < S) pv[k] = *reinterpret_cast<const u32x4 *>(psrc + k * sstride);
  }

  // ---- split weights: w_s = 2^(m_s - M) l_s / sum
  {
    float mx = -INFINITY;
#pragma unroll
    for (int k = 0; k < MAXSL; ++k) mx = fmaxf(mx, mlv[k].x);
    for (int s = sl + 16 * MAXSL; s < S; s += 16)
      mx = fmaxf(mx, ml[2 * (mlbase + static_cast<int64_t>(s) * heads)]);
    mx = dpp_reduce<16, true>(mx);
    float den = 0.f;
#pragma unroll
    for (int k = 0; k < MAXSL; ++k) {
      const int s = sl + 16 * k;
      const float w = (mx == -INFINITY || s >= S) ? 0.f : __builtin_amdgcn_exp2f(mlv[k].x - mx) * mlv[k].y;
      if (s < S) wts[bi * S + s] = w;
      den += w;
    }
    for (int s = sl + 16 * MAXSL; s < S; s += 16) {
      const int64_t o = mlbase + static_cast<int64_t>(s) * heads;
      const float w = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[2 * o] - mx) * ml[2 * o + 1];
      wts[bi * S + s] = w;
      den += w;
    }
    den = dpp_reduce<16, false>(den);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int s = sl; s < S; s += 16) wts[bi * S + s] *= inv;
  }

  // ---- W registers -> LDS (bf16)
#pragma unroll
  for (int k = 0; k < MAXU; ++k) {
    const int u = tid + 256 * k;
    if (u < rows * units) {
      const int row = u / units, c8 = (u % units) * 8;
      u32x4 v = wreg[k];
      if constexpr (sizeof(WT) == 1) {
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          const uint32_t word = v[e >> 1];
          const int sh = 16 * (e & 1);
          v[e] = cvt_bf16x2(static_cast<float>(static_cast<int>(word << (24 - sh)) >> 24),
                            static_cast<float>(static_cast<int>(word << (16 - sh)) >> 24));
        }
      }
      *reinterpret_cast<u32x4 *>(wl + row * WRS + c8 * 2) = v;
    }
  }
  __syncthreads();

  // ---- merged O~ rows
  {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float w = (k < S) ? wts[bi * S + k] : 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = fmaf(w, __uint_as_float(pv[k][e] << 16), acc[2 * e]);
        acc[2 * e + 1] = fmaf(w, __uint_as_float(pv[k][e] & 0xFFFF0000u), acc[2 * e + 1]);
      }
    }
    for (int s0 = kMergeBatch; s0 < S; s0 += kMergeBatch) {
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        pv[k] = u32x4{0u, 0u, 0u, 0u};
        if (rvalid && s0 + k < S) pv[k] = *reinterpret_cast<const u32x4 *>(psrc + (s0 + k) * sstride);
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const float w = (s0 + k < S) ? wts[bi * S + s0 + k] : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] = fmaf(w, __uint_as_float(pv[k][e] << 16), acc[2 * e]);
          acc[2 * e + 1] = fmaf(w, __uint_as_float(pv[k][e] & 0xFFFF0000u), acc[2 * e + 1]);
        }
      }
    }
    if (!rvalid) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    }
    // A operand of K block jj0 / 32: lane 16 ((jj0 / 8) % 4) + sequence
    aop[(jj0 >> 5) * 64 + 16 * ((jj0 >> 3) & 3) + bi] =
        u32x4{cvt_bf16x2(acc[0], acc[1]), cvt_bf16x2(acc[2], acc[3]),
              cvt_bf16x2(acc[4], acc[5]), cvt_bf16x2(acc[6], acc[7])};
  }
  __syncthreads();

  // ---- O~ W^u_v,h: wavefront w takes 16-column blocks w, w + 4, ...
  const int li = lane & 15, lg = lane >> 4;
  const int nkb = rows / 32;
  for (int nb = wave; nb < d / 16; nb += 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const uint8_t *trb = wl + (8 * lg + (li >> 2)) * WRS + (nb * 16 + 4 * (li & 3)) * 2;
    for (int kb = 0; kb < nkb; ++kb) {
      const bf16x4 lo = lds_read_tr16(trb + (32 * kb) * WRS);
      const bf16x4 hi = lds_read_tr16(trb + (32 * kb + 4) * WRS);
      const bf16x8 bv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, aop[kb * 64 + lane]), bv,
                                                    acc, 0, 0, 0);
    }
    const int col = nb * 16 + li;
    const float sc = wscale ? wscale[static_cast<int64_t>(h) * d + col] : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bo = 4 * lg + e;
      if (bo < nbb) opj[((static_cast<int64_t>(jc) * b + b0 + bo) * heads + h) * d + col] = acc[e] * sc;
    }
  }
}

// ------------------------------------------------------------------ merge
// Workgroup (chunk jc of 128 latent rows, head h, 16 sequences):
//   1. log-sum-exp weights of every split (one wavefront per sequence),
//   2. merged O~ rows of the chunk (16 B partial loads),
//   3. the chunk's share of O~ W^u_v,h in float32 -> opj[jc][b][h][d].
// W^u_v is read once per (chunk, head): the whole grid reads it once.
template <typename PT, typename WT>
__global__ __launch_bounds__(256) void merge_f32_kernel(const PT *__restrict__ opart,
                                                    const float *__restrict__ ml,
                                                    const WT *__restrict__ Wv,
                                                    const float *__restrict__ wscale,
                                                    float *__restrict__ opj, int b, int r,
                                                    int heads, int d, int S) {
  constexpr int BB = 16;
  extern __shared__ float fsm[];
  float *wts = fsm;                  // [BB][S]
  float *mv = fsm + BB * S;          // [BB][kMergeRows]
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

// O = sum over the JC chunk shares, 4 consecutive outputs per thread, the
// loads of all chunks issued before the sum (n % 4 == 0).
template <typename OT>
__global__ __launch_bounds__(256) void finalize_kernel(const float *__restrict__ opj,
                                                       OT *__restrict__ O, int64_t n, int JC) {
  constexpr int MAXJC = 32;
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 v[MAXJC];
#pragma unroll
  for (int c = 0; c < MAXJC; ++c)
    if (c < JC) v[c] = *reinterpret_cast<const f32x4 *>(opj + c * n + i);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < MAXJC; ++c)
    if (c < JC) acc += v[c];
  for (int c = MAXJC; c < JC; ++c) acc += *reinterpret_cast<const f32x4 *>(opj + c * n + i);
  if constexpr (sizeof(OT) == 2) {
    *reinterpret_cast<u32x2 *>(O + i) = u32x2{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
  } else {
    *reinterpret_cast<f32x4 *>(O + i) = acc;
  }
}

// ------------------------------------------------------------------ dispatch helpers
constexpr size_t kMaxLds = 160 * 1024;

// K blocks per 16-byte cache load for a cache dtype.
int kpl_of(int c_dtype) { return c_dtype == QSVD_I4 ? 4 : (c_dtype == QSVD_I8 ? 2 : 1); }

template <int CT, int NHB, int NKB, int T, int D>
hipError_t launch_stream_t(const StreamParams &sp, int W, hipStream_t s) {
  auto kern = stream_mfma_kernel<CT, NHB, NKB, T, D>;
  const size_t lds = stream_lds_bytes(W, NHB, NKB, T);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<dim3(sp.ntasks), dim3(W * 64), lds, s>>>(sp);
  return hipGetLastError();
}

template <int CT, int NHB, int NKB>
hipError_t launch_stream_tile(const StreamParams &sp, const MfmaShape &sh, hipStream_t s) {
  if constexpr (CT != CT_BF16 && NKB <= 8) {
    if (sh.T == 64) return launch_stream_t<CT, NHB, NKB, 64, 1>(sp, sh.W, s);
  }
  if constexpr (NHB == 2) {
    return launch_stream_t<CT, NHB, NKB, 32, 1>(sp, sh.W, s);  // mfma_shape pairs NHB = 2 with T >= 32
  } else {
    if (sh.T == 32) return launch_stream_t<CT, NHB, NKB, 32, 1>(sp, sh.W, s);
    return launch_stream_t<CT, NHB, NKB, 16, 2>(sp, sh.W, s);
  }
}

template <int CT, int NKB>
hipError_t launch_stream_nhb(const StreamParams &sp, const MfmaShape &sh, hipStream_t s) {
  if constexpr (NKB <= 6) {
    if (sh.NHB == 2) return launch_stream_tile<CT, 2, NKB>(sp, sh, s);
  }
  return launch_stream_tile<CT, 1, NKB>(sp, sh, s);
}

template <int CT>
hipError_t launch_stream_ct(const StreamParams &sp, const MfmaShape &sh, hipStream_t s) {
  if constexpr (CT == CT_BF16) {
    switch (sh.NKB) {
      case 1: return launch_stream_nhb<CT, 1>(sp, sh, s);
      case 2: return launch_stream_nhb<CT, 2>(sp, sh, s);
      case 3: return launch_stream_nhb<CT, 3>(sp, sh, s);
      case 4: return launch_stream_nhb<CT, 4>(sp, sh, s);
      case 5: return launch_stream_nhb<CT, 5>(sp, sh, s);
      case 6: return launch_stream_nhb<CT, 6>(sp, sh, s);
      case 7: return launch_stream_nhb<CT, 7>(sp, sh, s);
      case 8: return launch_stream_nhb<CT, 8>(sp, sh, s);
      case 9: return launch_stream_nhb<CT, 9>(sp, sh, s);
      case 10: return launch_stream_nhb<CT, 10>(sp, sh, s);
      case 11: return launch_stream_nhb<CT, 11>(sp, sh, s);
      default: return launch_stream_nhb<CT, 12>(sp, sh, s);
    }
  } else if constexpr (CT == CT_I8) {
    switch (sh.NKB) {
      case 2: return launch_stream_nhb<CT, 2>(sp, sh, s);
      case 4: return launch_stream_nhb<CT, 4>(sp, sh, s);
      case 6: return launch_stream_nhb<CT, 6>(sp, sh, s);
      case 8: return launch_stream_nhb<CT, 8>(sp, sh, s);
      case 10: return launch_stream_nhb<CT, 10>(sp, sh, s);
      default: return launch_stream_nhb<CT, 12>(sp, sh, s);
    }
  } else {
    switch (sh.NKB) {
      case 4: return launch_stream_nhb<CT, 4>(sp, sh, s);
      case 8: return launch_stream_nhb<CT, 8>(sp, sh, s);
      default: return launch_stream_nhb<CT, 12>(sp, sh, s);
    }
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

hipError_t launch_merge_f32(const DecodeArgs &a, const DecodePlan &p, const float *opart,
                            const float *ml, float *opj, hipStream_t s) {
  const int JC = (a.r + kMergeRows - 1) / kMergeRows;
  const size_t lds = (static_cast<size_t>(16) * p.splits + 16 * kMergeRows) * sizeof(float);
  auto kern = merge_f32_kernel<float, float>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<dim3(JC, a.heads, (a.b + 15) / 16), dim3(256), lds, s>>>(
      opart, ml, static_cast<const float *>(a.Wu_v), a.wu_scale_v, opj, a.b, a.r, a.heads, a.d,
      p.splits);
  return hipGetLastError();
}

size_t merge_mfma_lds(int d, int S) {
  return static_cast<size_t>(kMergeRows) * (d * 2 + 16) + (kMergeRows / 32) * 64 * 16 +
         static_cast<size_t>(16) * S * sizeof(float);
}

template <typename WT>
hipError_t launch_merge_mfma(const DecodeArgs &a, const DecodePlan &p, const uint16_t *opart,
                             const float *ml, float *opj, hipStream_t s) {
  const int JC = (a.r + kMergeRows - 1) / kMergeRows;
  const size_t lds = merge_mfma_lds(a.d, p.splits);
  auto kern = merge_mfma_kernel<WT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  kern<<<dim3(JC, a.heads, (a.b + 15) / 16), dim3(256), lds, s>>>(
      opart, ml, static_cast<const WT *>(a.Wu_v), a.wu_scale_v, opj, a.b, a.r, a.heads, a.d,
      p.splits, p.rw);
  return hipGetLastError();
}

template <typename WT, int DK>
hipError_t launch_absorb_mfma_t(const DecodeArgs &a, uint16_t *qt, hipStream_t s) {
  const dim3 grid((a.r + 63) / 64, a.heads, (a.b + 15) / 16);
  absorb_mfma_kernel<WT, DK><<<grid, dim3(256), 0, s>>>(
      static_cast<const uint16_t *>(a.q), static_cast<const WT *>(a.Wu_k), a.wu_scale_k, qt, a.b,
      a.r, a.heads, a.softmax_scale * kLog2e);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_absorb_mfma(const DecodeArgs &a, uint16_t *qt, hipStream_t s) {
  switch (a.d) {
    case 32: return launch_absorb_mfma_t<WT, 1>(a, qt, s);
    case 64: return launch_absorb_mfma_t<WT, 2>(a, qt, s);
    case 128: return launch_absorb_mfma_t<WT, 4>(a, qt, s);
    default: return launch_absorb_mfma_t<WT, 8>(a, qt, s);
  }
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

// Shape of the MFMA stream kernel for a latent width r and cache dtype: the
// largest wavefront count W <= 8 that gives every wavefront a whole number of
// 16-byte loads per row (RW = r / W a multiple of 32 * KPL) with at most 12 K
// blocks; two 16-head blocks per workgroup when at most 6 K blocks (register
// budget), and 32-token tiles when they fit in LDS and registers (<= 10 K
// blocks).
bool mfma_shape(int r, int heads, int c_dtype, MfmaShape *out) {
  const int kpl = kpl_of(c_dtype);
  for (int W = 8; W >= 1; --W) {
    if (r % (W * 32 * kpl) != 0) continue;
    const int nkb = r / (32 * W);
    if (nkb > 12) return false;
    MfmaShape s{};
    s.W = W;
    s.NKB = nkb;
    s.NHB = (heads > 16 && nkb <= 6 && stream_lds_bytes(W, 2, nkb, 32) <= kMaxLds) ? 2 : 1;
    s.T = (nkb <= 10 && stream_lds_bytes(W, s.NHB, nkb, 32) <= kMaxLds) ? 32 : 16;
    // quantised codes stage in few registers: a 64-token tile halves the
    // per-token share of the barriers and the softmax where LDS holds it
    if (c_dtype != QSVD_BF16 && s.T == 32 && nkb <= 8 && stream_lds_bytes(W, s.NHB, nkb, 64) <= kMaxLds)
      s.T = 64;
    // tuning override of the tile (32: one tile of loads in flight, 16: two)
    static const int tile_env = [] {
      const char *e = std::getenv("QSVD_STREAM_TILE");
      return e ? std::atoi(e) : 0;
    }();
    if (tile_env == 16 && s.NHB == 1) s.T = 16;
    if (tile_env == 32 && nkb <= 10 && stream_lds_bytes(W, s.NHB, nkb, 32) <= kMaxLds) s.T = 32;
    if (stream_lds_bytes(W, s.NHB, nkb, s.T) > kMaxLds) return false;
    if (out) *out = s;
    return true;
  }
  return false;
}

DecodePlan plan_decode(int b, int64_t L, int r, int heads, int d, int c_dtype, int splits) {
  DecodePlan p{};
  p.mfma = c_dtype != QSVD_F32;
  int64_t S;
  if (p.mfma) {
    MfmaShape sh{};
    mfma_shape(r, heads, c_dtype, &sh);  // validated by the caller
    p.shape = sh;
    const int G = (heads + 16 * sh.NHB - 1) / (16 * sh.NHB);
    p.head_groups = G;
    p.group_heads = (heads + G - 1) / G;
    // token tiles are dealt round-robin to the splits; no split is left empty
    const int64_t tiles_all = (L + sh.T - 1) / sh.T;
    if (splits > 0) {
      S = splits;
    } else {
      const int64_t per = static_cast<int64_t>(b) * p.head_groups;
      S = std::max<int64_t>(1, kNumCU / std::max<int64_t>(per, 1));
    }
    S = std::min<int64_t>(std::min<int64_t>(S, tiles_all), kMaxSplits);
    p.chunk = 0;
    p.splits = static_cast<int>(S);
    p.rw = r / sh.W;
    // many heads over a wide latent: two passes that each read the cache once
    // beat a single pass whose head groups read it three or more times
    if (wide_applies(r, heads, c_dtype, G)) {
      p.wide = true;
      wide_plan(b, L, r, heads, &p.wp);
      p.splits = p.wp.splits;
      p.rw = p.wp.rw;
    }
  } else {
    p.head_groups = heads;
    p.group_heads = 1;
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
  if (p.wide) p.part_bytes += align256(p.wp.s_bytes) + align256(p.wp.m1_bytes);
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

  // ---- stream (two passes for wide latents with many heads)
  if (p.wide) {
    uint8_t *wbase = reinterpret_cast<uint8_t *>(opj) +
                     align256(static_cast<size_t>((a.r + kMergeRows - 1) / kMergeRows) * a.b * a.heads * a.d * sizeof(float));
    WideArgs wa{};
    wa.C = a.C;
    wa.qt = static_cast<const uint16_t *>(qt);
    wa.S = reinterpret_cast<float *>(wbase);
    wa.m1 = reinterpret_cast<float *>(wbase + align256(p.wp.s_bytes));
    wa.opart = static_cast<uint16_t *>(opart);
    wa.ml = ml;
    wa.L = a.L;
    wa.Lp = p.wp.Lp;
    wa.chunk1 = p.wp.chunk1;
    wa.chunk3 = p.wp.chunk3;
    wa.b = a.b;
    wa.r = a.r;
    wa.heads = a.heads;
    wa.nchunk1 = p.wp.nchunk1;
    wa.splits = p.splits;
    e = launch_wide_scores(wa, s);
    if (e != hipSuccess) return e;
    e = launch_wide_values(wa, s);
    if (e != hipSuccess) return e;
  } else {
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
      const MfmaShape &sh = p.shape;
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
      sp.G = p.head_groups;
      sp.group_heads = p.group_heads;
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
      e = launch_merge_f32(a, p, static_cast<const float *>(opart), ml, opj, s);
    else if (a.wu_dtype == QSVD_I8)
      e = launch_merge_mfma<int8_t>(a, p, static_cast<const uint16_t *>(opart), ml, opj, s);
    else
      e = launch_merge_mfma<uint16_t>(a, p, static_cast<const uint16_t *>(opart), ml, opj, s);
    if (e != hipSuccess) return e;
  }

  // ---- finalize
  {
    LaunchTimer t("decode_finalize", s);
    const int64_t n = static_cast<int64_t>(a.b) * a.heads * a.d;
    const int JC = (a.r + kMergeRows - 1) / kMergeRows;
    const dim3 grid(static_cast<unsigned>((n / 4 + 255) / 256)), block(256);
    if (a.o_dtype == QSVD_BF16)
      finalize_kernel<uint16_t><<<grid, block, 0, s>>>(opj, static_cast<uint16_t *>(a.O), n, JC);
    else
      finalize_kernel<float><<<grid, block, 0, s>>>(opj, static_cast<float *>(a.O), n, JC);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace qsvd
