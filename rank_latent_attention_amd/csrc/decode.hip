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
// The stream kernel's running softmax maximum moves only when a tile's
// maximum exceeds it by more than this (log2 units): p stays below 2^8.
constexpr float kRescaleSlack = 8.f;

enum CType : int { CT_BF16 = 0, CT_I4 = 1, CT_I8 = 2 };

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads past the end return zero
// without a branch (and without touching memory).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}


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
  // branch-free operand loads: sequences past b and rows past r lie outside
  // the resources (based at the workgroup's first sequence and row) and read
  // as zero, so every load is in flight before the first wait
  const int jb0 = blockIdx.x * 64;
  const __amdgpu_buffer_rsrc_t rq =
      buffer_rsrc(q + static_cast<int64_t>(b0) * heads * d, static_cast<int64_t>(min(16, b - b0)) * heads * d * 2);
  const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(Wk + static_cast<int64_t>(jb0) * E,
                                                static_cast<int64_t>(min(64, r - jb0)) * E * sizeof(WT));
  const uint32_t qoff = static_cast<uint32_t>((((lane & 15) * heads + h) * d + kq) * 2);
  const uint32_t woff = static_cast<uint32_t>(((j - jb0) * E + h * d + kq) * sizeof(WT));
  u32x4 av[DK], bv[DK];
#pragma unroll
  for (int k = 0; k < DK; ++k) {
    av[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + 64 * k, 0, 0));
    if constexpr (sizeof(WT) == 2) {
      bv[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, woff + 64 * k, 0, 0));
    } else {
      const u32x2 c = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rw, woff + 32 * k, 0, 0));
      bv[k] = u32x4{c.x, c.y, 0u, 0u};
    }
  }
  // int8 W^u_k: the column scales of this lane's q elements, requested with
  // the operands (one memory round trip for the whole workgroup)
  f32x4 sv[DK][2];
  if constexpr (sizeof(WT) == 1) {
#pragma unroll
    for (int k = 0; k < DK; ++k) {
      sv[k][0] = *reinterpret_cast<const f32x4 *>(wscale + h * d + 32 * k + kq);
      sv[k][1] = *reinterpret_cast<const f32x4 *>(wscale + h * d + 32 * k + kq + 4);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // every operand load is issued before the products
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < DK; ++k) {
    u32x4 a = av[k], w = bv[k];
    // int8 W^u_k: q times the column scales, carried as a bf16 pair
    // (head + tail, about 16 significant bits) so that the product keeps
    // the precision of q itself
    u32x4 a_tail = {0u, 0u, 0u, 0u};
    if constexpr (sizeof(WT) == 1) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = __uint_as_float(a[e] << 16) * sv[k][e >> 1][2 * (e & 1)];
        const float hi = __uint_as_float(a[e] & 0xFFFF0000u) * sv[k][e >> 1][2 * (e & 1) + 1];
        a[e] = pack_bf16x2(lo, hi);
        a_tail[e] = pack_bf16x2(lo - __uint_as_float(a[e] << 16), hi - __uint_as_float(a[e] & 0xFFFF0000u));
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
    if constexpr (sizeof(WT) == 1)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                    __builtin_bit_cast(bf16x8, a_tail), acc, 0, 0, 0);
  }
  const int jo = j0 + 4 * (lane >> 4);
  if (bb < b && jo < r)  // r % 16 == 0: the 4 rows are all valid
    *reinterpret_cast<u32x2 *>(qt + (static_cast<int64_t>(bb) * heads + h) * r + jo) =
        u32x2{pack_bf16x2(acc[0] * scale, acc[1] * scale), pack_bf16x2(acc[2] * scale, acc[3] * scale)};
}

// Reductions over aligned groups of N = 8, 16 or 32 lanes: DPP lane swaps
// (xor 1, xor 2, mirror within 8, mirror within 16), then for 32 one swap of
// neighbouring 16-lane rows.
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
  // the wavefront's tokens t0 + wave, t0 + wave + 4, ... in batches of TB
  // whose rows are requested together (rows past t1 are clamped and skipped)
  constexpr int TB = 4;
  for (int64_t tb = t0 + wave; tb < t1; tb += 4 * TB) {
    float c[TB][MAXJ];
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      const int64_t t = min(tb + 4 * u, t1 - 1);
      const float *row = C + (static_cast<int64_t>(seq) * L + t) * r;
#pragma unroll
      for (int k = 0; k < MAXJ; ++k) {
        const int j = lane + 64 * k;
        c[u][k] = (j < r) ? row[j] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < TB; ++u) {
      if (tb + 4 * u >= t1) break;
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < MAXJ; ++k) s = fmaf(c[u][k], qv[k], s);
      s = dpp_reduce<32, false>(s);
      s += __shfl_xor(s, 32, 64);
      const float mn = fmaxf(m, s);
      const float alpha = exp2f(m - mn);
      const float p = exp2f(s - mn);
      l = fmaf(l, alpha, p);
#pragma unroll
      for (int k = 0; k < MAXJ; ++k) o[k] = fmaf(o[k], alpha, p * c[u][k]);
      m = mn;
    }
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

// ------------------------------------------------------------------ float32, one launch
// Small float32 problems take the whole step in one launch (the four launches
// of the split path cost more than the work).  Workgroup (head h, sequence),
// 16 wavefronts:
//   1. q~ = scale log2e W^u_k,h q_h: wavefront w computes latent rows w,
//      w + 16, ... (one 64-lane dot product each, every row requested first),
//   2. wavefront w streams tokens w, w + 16, ... with its own online softmax,
//      four tokens at a time (one per 16-lane group), TBW per batch,
//   3. the 16 states are combined in LDS by log-sum-exp weights (fixed order),
//   4. O = (O~ / l) W^u_v,h: thread (column c, row group g) sums the rows
//      g, g + G, ..., and the G row groups are summed in LDS.
constexpr int kFusedWaves = 16;

template <int MAXJ>
__global__ __launch_bounds__(64 * kFusedWaves) void decode_f32_fused_kernel(
    const float *__restrict__ q, const float *__restrict__ C, const float *__restrict__ Wk,
    const float *__restrict__ Wv, float *__restrict__ O, int64_t L, int r, int heads, int d,
    float scale) {
  constexpr int NW = kFusedWaves, NT = 64 * NW;
  constexpr int RPW = (64 * MAXJ + NW - 1) / NW;   // latent rows per wavefront in step 1
  constexpr int CPL = 4 * MAXJ;                    // latent columns per lane (16 lanes per token)
  constexpr int TPG = 64 / CPL;                    // tokens per 16-lane group and batch
  constexpr int TBW = 4 * TPG;                     // tokens per wavefront and batch
  constexpr int KU = (64 * MAXJ + 7) / 8;          // W^u_v rows per thread in step 4 (NT / d >= 8)
  extern __shared__ float fs[];
  float *qs = fs;               // [r] q~
  float *wo = qs + r;           // [NW][r] per-wavefront O~
  float *wm = wo + NW * r;      // [NW] running maxima
  float *wl = wm + NW;          // [NW] running sums
  float *ot = wl + NW;          // [r] O~ / l
  float *red = ot + r;          // [NT] projection shares
  const int h = blockIdx.x, seq = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t E = static_cast<int64_t>(heads) * d;
  const float *Cs = C + static_cast<int64_t>(seq) * L * r;

  // Loads whose addresses do not depend on q~ go first: the W^u_k,h rows
  // (step 1) and this wavefront's first TB token rows (step 2); this thread's
  // W^u_v,h rows (step 4) are requested before the combine.  They go through buffer
  // resources: rows past the end (tokens past L, latent rows past r) read as
  // zero, the row offsets are wave-uniform scalar offsets, and no load sits
  // behind a branch, so all of them are in flight together.  Columns past r
  // or d read neighbouring values, which meet a zero query element (steps 1
  // and 2) or are never stored.
  const float *qh = q + (static_cast<int64_t>(seq) * heads + h) * d;
  const float q0 = qh[min(lane, d - 1)], q1 = qh[min(lane + 64, d - 1)];
  const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(Wk + static_cast<int64_t>(h) * d, (r * E - h * d) * 4);
  const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(Wv + static_cast<int64_t>(h) * d, (r * E - h * d) * 4);
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(Cs, L * r * 4);
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform, for scalar offsets
  float w0[RPW], w1[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const int so = static_cast<int>((wave_s + NW * i) * E * 4);
    w0[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, lane * 4, so, 0));
    w1[i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rk, lane * 4 + 256, so, 0));
  }
  // Step 2's layout: the wavefront takes four tokens at a time, one per
  // 16-lane group; lane li of group grp holds columns li, li + 16, ... of its
  // token (16 consecutive values per group and load).  Batch i0 of this
  // wavefront: group grp takes tokens wave + NW (i0 + 4 u + grp), u < TPG.
  const int grp = lane >> 4, li = lane & 15;
  float c[TPG][CPL];
  auto load_rows = [&](int64_t i0) {
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      const int64_t tok = wave + NW * (i0 + 4 * u + grp);
      const int vo = static_cast<int>(std::min<int64_t>(tok, L) * r + li) * 4;   // rows at L read zero
#pragma unroll
      for (int k = 0; k < CPL; ++k)
        c[u][k] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rc, vo + 64 * k, 0, 0));
    }
  };
  load_rows(0);

  // ---- 1. absorbed query
  {
    const float qa = lane < d ? q0 : 0.f, qb = lane + 64 < d ? q1 : 0.f;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      float v = fmaf(w1[i], qb, w0[i] * qa);
      v = dpp_reduce<32, false>(v);
      v += __shfl_xor(v, 32, 64);
      const int k = wave + NW * i;
      if (lane == 0 && k < r) qs[k] = v * scale;
    }
  }
  __syncthreads();

  // ---- 2. this wavefront's tokens, TBW per batch: 16-lane dot products (four
  // tokens per DPP reduction), the batch maximum over all four groups, one
  // rescale of (O~, l), then p C per group; the groups' partial O~ and l are
  // added at the end (they share the running maximum)
  float qv[CPL], o[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int j = li + 16 * k;
    qv[k] = j < r ? qs[j] : 0.f;   // columns past r add nothing to the scores
    o[k] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int64_t i0 = 0; wave + NW * i0 < L; i0 += TBW) {
    if (i0 != 0) load_rows(i0);
    float sc[TPG];
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < CPL; ++k) v = fmaf(c[u][k], qv[k], v);
      v = dpp_reduce<16, false>(v);
      sc[u] = wave + NW * (i0 + 4 * u + grp) < L ? v : -INFINITY;
    }
    float mn = m;
#pragma unroll
    for (int u = 0; u < TPG; ++u) mn = fmaxf(mn, sc[u]);
    mn = fmaxf(mn, __shfl_xor(mn, 16, 64));
    mn = fmaxf(mn, __shfl_xor(mn, 32, 64));   // finite: the batch's first token is inside L
    const float alpha = exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[k] *= alpha;
#pragma unroll
    for (int u = 0; u < TPG; ++u) {
      const float pe = exp2f(sc[u] - mn);   // 0 for tokens past L
      l += pe;
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[k] = fmaf(pe, c[u][k], o[k]);
    }
    m = mn;
  }
  // the four groups' shares (fixed order: xor 16, then xor 32)
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    o[k] += __shfl_xor(o[k], 16, 64);
    o[k] += __shfl_xor(o[k], 32, 64);
  }
  if (grp == 0) {
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int j = li + 16 * k;
      if (j < r) wo[wave * r + j] = o[k];
    }
  }
  if (lane == 0) {
    wm[wave] = m;
    wl[wave] = l;
  }
  // this thread's W^u_v,h rows g, g + G, ... (rows past r read as zero)
  const int G = NT / d, cc = tid % d, g = tid / d;
  float wv[KU];
#pragma unroll
  for (int u = 0; u < KU; ++u)
    wv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, static_cast<int>((g * E + cc) * 4),
                                                                 static_cast<int>(G * u * E * 4), 0));
  __syncthreads();

  // ---- 3. combine the wavefronts (L >= 1: the maximum is finite)
  {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w]);
    float f[NW], lt = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      f[w] = exp2f(wm[w] - M);   // 0 for a wavefront without tokens
      lt = fmaf(wl[w], f[w], lt);
    }
    const float inv = 1.f / lt;
    for (int j = tid; j < r; j += NT) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc = fmaf(wo[w * r + j], f[w], acc);
      ot[j] = acc * inv;
    }
  }
  __syncthreads();

  // ---- 4. output projection: thread (column cc, rows g, g + G, ...), the G
  // row groups summed through LDS in a fixed order
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < KU; ++u)
    if (g + G * u < r) acc = fmaf(ot[g + G * u], wv[u], acc);
  red[tid] = acc;
  __syncthreads();
  if (tid < d) {
    float v = 0.f;
    for (int gg = 0; gg < G; ++gg) v += red[gg * d + tid];
    O[(static_cast<int64_t>(seq) * heads + h) * d + tid] = v;
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

// Scale groups of one wavefront's columns: int4 caches carry one scale per
// 128-column group (NKB / 4 groups per wavefront, whose columns are whole
// groups); int8 caches one scale per token.
__host__ __device__ constexpr int stream_groups(bool int4, int NKB) { return int4 ? NKB / 4 : 1; }

// Quantised 64-token tiles: depths (tiles of loads in flight) whose staging
// registers fit beside O~ and Q~ without spilling (checked in the gfx950
// assembly of each instantiation).
__host__ __device__ constexpr bool stream_depth_fits(bool int4, int NHB, int NKB, int D) {
  return D == 1 || (D == 2 && (int4 ? NKB <= 4 : NKB * NHB <= 4)) || (D == 3 && int4 && NKB <= 4 && NHB == 1);
}

// LDS bytes of the stream kernel: wavefront C tiles | partial scores | P |
// alpha, m, l | (quantised caches) each wavefront's scales of the tile.
__host__ __device__ constexpr size_t stream_lds_bytes(int W, int NHB, int NKB, int T, int c_kind = 0) {
  return static_cast<size_t>(W) * T * ct_row_stride(NKB) +
         static_cast<size_t>(W) * NHB * 16 * sp_row(T) * 4 + static_cast<size_t>(NHB) * 64 * T / 2 +
         static_cast<size_t>(NHB) * 16 * 4 * 3 +
         (c_kind == 0 ? 0 : static_cast<size_t>(W) * stream_groups(c_kind == 1, NKB) * T * 4);
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

// Exact integer codes as bf16 MFMA operands, offset by a constant so that the
// conversion is a few bit operations per code (the scales are applied to the
// products instead, see stream_mfma_kernel).
//
// int4: the bf16 bit pattern 0x4300 | m is the value 128 + m for a 7-bit m,
// and m = n ^ 8 maps the two's-complement nibble n of a code c to c + 8, so
// 0x4300 | (n ^ 8) is exactly 136 + c.  One dword holds codes n0..n7 (n0 in
// the lowest nibble); the four output dwords hold the pairs (n0, n4),
// (n1, n5), (n2, n6), (n3, n7), i.e. K position p carries code
// kI4Perm[p] of the group of eight.
constexpr float kI4Offset = 136.f;
constexpr float kI8Offset = 128.f;
__device__ __forceinline__ u32x4 i4_codes_bf16(uint32_t w) {
  // (n ^ 8) | 0x4300 == n ^ 0x4308 for a nibble n: one and-xor per pair
  const uint32_t m = 0x000F000Fu, e = 0x43084308u;
  return u32x4{(w & m) ^ e, ((w >> 4) & m) ^ e, ((w >> 8) & m) ^ e, ((w >> 12) & m) ^ e};
}
// int8: c ^ 0x80 is the unsigned byte c + 128, converted exactly by
// v_cvt_f32_ubyteN; bf16 keeps the upper half of an integer below 256 exactly.
__device__ __forceinline__ u32x2 i8_codes_bf16(uint32_t w) {
  const uint32_t x = w ^ 0x80808080u;
  const float f0 = static_cast<float>(x & 0xFFu), f1 = static_cast<float>((x >> 8) & 0xFFu);
  const float f2 = static_cast<float>((x >> 16) & 0xFFu), f3 = static_cast<float>(x >> 24);
  return u32x2{__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
               __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u)};
}
// The int4 K order applied to eight consecutive bf16 values (q0..q7 in
// v[0..3] as pairs): (q0, q4), (q1, q5), (q2, q6), (q3, q7).
__device__ __forceinline__ u32x4 i4_order(u32x4 v) {
  return u32x4{__builtin_amdgcn_perm(v[2], v[0], 0x05040100u), __builtin_amdgcn_perm(v[2], v[0], 0x07060302u),
               __builtin_amdgcn_perm(v[3], v[1], 0x05040100u), __builtin_amdgcn_perm(v[3], v[1], 0x07060302u)};
}
// Column (within its group of eight) held at K position p of the int4 order.
__device__ __forceinline__ int i4_column(int p) { return (p >> 1) + 4 * (p & 1); }

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
  static_assert(D >= 1 && D <= 4, "prefetch depth");
  // output staging rows: RW + 8 elements apart, so the 16 heads of one store
  // instruction fall in different LDS banks
  constexpr int OSTR = RW + 8;
  static_assert(HGP * OSTR * 2 <= T * RS, "the output rows are staged in the wavefront's C tile");
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
  // quantised caches: this wavefront's scales of the tile, [group][token]
  float *ssc = l_s + HGP + static_cast<size_t>(wave) * stream_groups(CT == CT_I4, NKB) * T;

  // ---- tile loads through buffer resources based at the tile's first row:
  // rows at or past the end of the sequence fall outside the resource and
  // read as zero (their scores are masked to -inf below, so their P is 0).
  const int64_t row_bytes = Tr::byte_offset(r);
  const uint32_t voff0 = static_cast<uint32_t>(li * row_bytes + Tr::byte_offset(j0w + EPL * lg));
  u32x4 stage[D][NTB][NLD];
  float sscale[D][NTB][NLD];
  // Branch-free: a tile past the split's last one (valid == false) is loaded
  // through an empty resource, which returns zeros without touching memory,
  // so the code path (and the compiler's waits for the loads) is the same
  // for every tile.
  auto load_rows = [&](auto BUF, int64_t t0_in, int tb, bool valid) {
    constexpr int bf = decltype(BUF)::value;
    const int64_t t0 = valid ? t0_in : L;
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


  // The first D tiles are requested at once (buffer k holds tiles k, k + D,
  // k + 2 D, ...).  Quantised caches request the absorbed queries first:
  // vector loads complete in order, and queries requested after the tiles
  // would make the offset sums below wait for the tiles as well.
  auto prefetch = [&](auto BUF) {
    constexpr int k = decltype(BUF)::value;
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) load_rows(BUF, tile_start(k), tb, ntiles > k);
  };
  auto prefetch_all = [&]() {
    prefetch(std::integral_constant<int, 0>{});
    if constexpr (D > 1) prefetch(std::integral_constant<int, 1>{});
    if constexpr (D > 2) prefetch(std::integral_constant<int, 2>{});
    if constexpr (D > 3) prefetch(std::integral_constant<int, 3>{});
  };
  if constexpr (CT == CT_BF16) {
    prefetch_all();
    __builtin_amdgcn_sched_barrier(0);
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
      const int j = j0w + 32 * KPL * ld + EPL * lg + 8 * s;
      u32x4 v = {0u, 0u, 0u, 0u};
      if constexpr (CT == CT_BF16) {
        if (h < hg) v = *reinterpret_cast<const u32x4 *>(p.qt + (static_cast<int64_t>(seq) * p.heads + h0 + h) * r + j);
      } else {
        // padded heads (h >= hg) read a real head's row: their scores and
        // value columns are computed and never written (a branch-free load
        // keeps the compiler's waits exact before the offset sums)
        v = *reinterpret_cast<const u32x4 *>(p.qt + (static_cast<int64_t>(seq) * p.heads + h0 + min(h, hg - 1)) * r + j);
      }
      qf[hb][kb] = __builtin_bit_cast(bf16x8, v);
    }
  if constexpr (CT != CT_BF16) {
    prefetch_all();
    // (nothing that reads the queries may be scheduled above the prefetch)
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (CT == CT_I4) {   // the K order of the int4 code operands
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
        qf[hb][kb] = __builtin_bit_cast(bf16x8, i4_order(__builtin_bit_cast(u32x4, qf[hb][kb])));
  }

  // Quantised caches: the score and value products run on the exact codes
  // plus a constant offset (136 for int4, 128 for int8) and the scales are
  // applied to the results.  For a wavefront and scale group g:
  //   partial score  s_t = scale_{t,g} (-off sum_j q~_j + sum_j (off + c_tj) q~_j)
  //   value product  O~_j = sum_t P'_t (off + c_tj) - off sum_t P'_t,
  //                  P'_t = bf16(p_t scale_{t,g})
  // koff holds off * sum_j q~_j (a product of ones with the Q~ operands) and
  // psum the running sum of the P' this lane contributes (rescaled with O~).
  constexpr int NG = stream_groups(CT == CT_I4, NKB);
  constexpr float kOff = CT == CT_I4 ? kI4Offset : kI8Offset;
  constexpr int KPG = NKB / NG;       // K blocks per scale group
  float koff[NG][NHB];
  f32x4 psum[NG][NHB];   // sum_t P'_t of head 16 hb + i (all four elements), from MFMAs
  if constexpr (CT != CT_BF16) {
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = g * KPG; kb < (g + 1) * KPG; ++kb)
          a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, qf[hb][kb], a, 0, 0, 0);
        koff[g][hb] = kOff * a[0];
        psum[g][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  }
  const bf16x8 ones8 = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const bf16x4 ones4 = __builtin_bit_cast(bf16x4, u32x2{0x3F803F80u, 0x3F803F80u});

  // O~ transposed: oacc[hb][jb] holds columns 16 jb + 4 g + (0..3) of head 16 hb + i
  // (K positions of the int4 order for int4 caches)
  f32x4 oacc[NHB][NJB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) oacc[hb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int i = tid; i < HGP; i += nthreads) {
    m_s[i] = -INFINITY;
    l_s[i] = 0.f;
  }
  lds_barrier();   // the first tiles' loads stay in flight

  auto body = [&](auto BUF, int it) {
    constexpr int bf = decltype(BUF)::value;
    const int64_t tile_t0 = tile_start(it);
    // tokens of this tile inside the sequence (wave-uniform)
    const int tile_valid = static_cast<int>(std::min<int64_t>(L - tile_t0, T));
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
            const u32x2 a = i8_codes_bf16(stage[bf][tb][ld][2 * s]);
            const u32x2 c = i8_codes_bf16(stage[bf][tb][ld][2 * s + 1]);
            cv[2 * ld + s] = u32x4{a.x, a.y, c.x, c.y};
          }
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) cv[4 * ld + s] = i4_codes_bf16(stage[bf][tb][ld][s]);
        }
      }
      if constexpr (CT != CT_BF16) {
        // the scales of token 16 tb + li (one per group) for the folds below;
        // same-wavefront LDS write -> read, ordered by the LDS queue
        if (lg == 0) {
#pragma unroll
          for (int g = 0; g < NG; ++g) ssc[g * T + tb * 16 + li] = sscale[bf][tb][g * (NLD / NG)];
        }
      }
      // quantised caches start each group's sum at -off sum_j q~_j, so that
      // the products leave sum_j c_tj q~_j (no subtraction per element)
      f32x4 sacc[NG][NHB];
#pragma unroll
      for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          if constexpr (CT != CT_BF16) {
            const float k0 = -koff[g][hb];
            sacc[g][hb] = f32x4{k0, k0, k0, k0};
          } else {
            sacc[g][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
          sacc[kb / KPG][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, cv[kb]), qf[hb][kb], sacc[kb / KPG][hb], 0, 0, 0);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int ld = kb / KPL, s = kb % KPL;
        const int jl = 32 * KPL * ld + EPL * lg + 8 * s;
        *reinterpret_cast<u32x4 *>(ct + (tb * 16 + li) * RS + jl * 2) = cv[kb];
      }
      load_rows(BUF, next_t0, tb, more);
      // partial scores, head-major: lane holds tokens 16 tb + 4 g + (0..3) of head 16 hb + i
      f32x4 part[NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) part[hb] = sacc[0][hb];
      if constexpr (CT != CT_BF16) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const f32x4 s4 = *reinterpret_cast<const f32x4 *>(ssc + g * T + tb * 16 + 4 * lg);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = sacc[g][hb][e] * s4[e];
              part[hb][e] = g == 0 ? v : part[hb][e] + v;
            }
        }
      }
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        *reinterpret_cast<f32x4 *>(spart + (wave * HGP + hb * 16 + li) * SPR + tb * 16 + 4 * lg) = part[hb];
    }
    lds_barrier();   // the next tile's loads stay in flight

    // ---- 4. cross-wavefront sum + online softmax: 8 lanes per head, TPI =
    // T / 8 consecutive tokens each (the max and the sum are per-lane over
    // the tokens, then 3 DPP steps over the head's 8 lanes)
    {
      constexpr int TPI = T / 8;
      for (int item = tid; item < HGP * 8; item += nthreads) {
        const int h = item >> 3, u = item & 7, t0 = u * TPI;
        const float m_old = m_s[h];
        // rows past W are not read (wave-uniform bound, constant row offsets)
        const float *sph = spart + h * SPR + t0;
        float sc[TPI];
#pragma unroll
        for (int w = 0; w < MAXW; ++w) {
          if (w < W) {
            float v[TPI];
            if constexpr (TPI == 8) {
              const f32x4 a = *reinterpret_cast<const f32x4 *>(sph + w * (HGP * SPR));
              const f32x4 c = *reinterpret_cast<const f32x4 *>(sph + w * (HGP * SPR) + 4);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v[e] = a[e];
                v[4 + e] = c[e];
              }
            } else if constexpr (TPI == 4) {
              const f32x4 a = *reinterpret_cast<const f32x4 *>(sph + w * (HGP * SPR));
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = a[e];
            } else {
              const float2 a = *reinterpret_cast<const float2 *>(sph + w * (HGP * SPR));
              v[0] = a.x;
              v[1] = a.y;
            }
#pragma unroll
            for (int e = 0; e < TPI; ++e) sc[e] = w == 0 ? v[e] : sc[e] + v[e];
          }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < TPI; ++e) {
          if (t0 + e >= tile_valid) sc[e] = -INFINITY;
          mx = fmaxf(mx, sc[e]);
        }
        mx = dpp_reduce<8, true>(mx);
        // lazy running maximum: kept until the tile's maximum exceeds it by
        // more than kRescaleSlack (log2 units), so p <= 2^kRescaleSlack and O~
        // is rescaled only on such tiles; the result is the same function
        const float m_new = mx > m_old + kRescaleSlack ? mx : m_old;
        const float alpha = __builtin_amdgcn_exp2f(m_old - m_new);
        uint32_t pp[TPI / 2];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < TPI / 2; ++e) {
          pp[e] = cvt_bf16x2(__builtin_amdgcn_exp2f(sc[2 * e] - m_new), __builtin_amdgcn_exp2f(sc[2 * e + 1] - m_new));
          ps += __uint_as_float(pp[e] << 16) + __uint_as_float(pp[e] & 0xFFFF0000u);
        }
        ps = dpp_reduce<8, false>(ps);
        if (u == 0) {
          m_s[h] = m_new;
          l_s[h] = fmaf(l_s[h], alpha, ps);
          alpha_s[h] = alpha;
        }
        // P as the B operand of the value product: K step t / 32 (T >= 32), lane
        // 16 ((t % 32) / PPL) + h % 16, element t % PPL (TPI <= PPL, aligned)
        const int ks = T == 16 ? 0 : t0 >> 5, tk = T == 16 ? t0 : t0 & 31;
        uint16_t *pdst = pl + ((ks * NHB + (h >> 4)) * 64 + 16 * (tk / PPL) + (h & 15)) * PPL + (tk % PPL);
        if constexpr (TPI == 8)
          *reinterpret_cast<u32x4 *>(pdst) = u32x4{pp[0], pp[1], pp[2], pp[3]};
        else if constexpr (TPI == 4)
          *reinterpret_cast<u32x2 *>(pdst) = u32x2{pp[0], pp[1]};
        else
          *reinterpret_cast<uint32_t *>(pdst) = pp[0];
      }
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
        if constexpr (CT != CT_BF16) {
#pragma unroll
          for (int g = 0; g < NG; ++g) psum[g][hb][0] *= al;
        }
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
      // P of this lane's tokens (head 16 hb + li); quantised caches scale it
      // per group: P'_g = bf16(p scale_{t,g})
      bf16x8 pq[NG][NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const u32x4 pv = *reinterpret_cast<const u32x4 *>(pl + ((ks * NHB + hb) * 64 + lane) * PPL);
        if constexpr (CT == CT_BF16) {
          pq[0][hb] = __builtin_bit_cast(bf16x8, pv);
        } else {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const f32x4 sa = *reinterpret_cast<const f32x4 *>(ssc + g * T + 32 * ks + PPL * lg);
            const f32x4 sb = *reinterpret_cast<const f32x4 *>(ssc + g * T + 32 * ks + PPL * lg + 4);
            u32x4 q;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float s_lo = i < 2 ? sa[2 * i] : sb[2 * i - 4];
              const float s_hi = i < 2 ? sa[2 * i + 1] : sb[2 * i - 3];
              q[i] = cvt_bf16x2(__uint_as_float(pv[i] << 16) * s_lo, __uint_as_float(pv[i] & 0xFFFF0000u) * s_hi);
            }
            pq[g][hb] = __builtin_bit_cast(bf16x8, q);
            // sum over the tokens of the P' the products use (ones as A)
            psum[g][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pq[g][hb], psum[g][hb], 0, 0, 0);
          }
        }
      }
      // column blocks in groups of VB: all transposing reads of a group are
      // issued before its products (a group never straddles two scale groups)
      constexpr int VB = (NJB % 4 == 0) ? 4 : ((NJB % 3 == 0) ? 3 : 2);
      static_assert(NJB % VB == 0 && (NJB / NG) % VB == 0, "column groups");
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
            oacc[hb][jg + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pq[jg / (NJB / NG)][hb],
                                                                      oacc[hb][jg + k], 0, 0, 0);
        }
      }
     }
    } else {
      const uint8_t *trb = ct + (PPL * lg + (li >> 2)) * RS + (4 * (li & 3)) * 2;
      bf16x4 pq[NG][NHB];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        const u32x2 pv = *reinterpret_cast<const u32x2 *>(pl + (hb * 64 + lane) * PPL);
        if constexpr (CT == CT_BF16) {
          pq[0][hb] = __builtin_bit_cast(bf16x4, pv);
        } else {
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            const f32x4 sa = *reinterpret_cast<const f32x4 *>(ssc + g * T + PPL * lg);
            u32x2 q;
#pragma unroll
            for (int i = 0; i < 2; ++i)
              q[i] = cvt_bf16x2(__uint_as_float(pv[i] << 16) * sa[2 * i],
                                __uint_as_float(pv[i] & 0xFFFF0000u) * sa[2 * i + 1]);
            pq[g][hb] = __builtin_bit_cast(bf16x4, q);
            psum[g][hb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pq[g][hb], psum[g][hb], 0, 0, 0);
          }
        }
      }
      constexpr int VB = (NJB % 4 == 0) ? 4 : ((NJB % 3 == 0) ? 3 : 2);
      static_assert(NJB % VB == 0 && (NJB / NG) % VB == 0, "column groups");
#pragma unroll
      for (int jg = 0; jg < NJB; jg += VB) {
        bf16x4 av[VB];
#pragma unroll
        for (int k = 0; k < VB; ++k) av[k] = lds_read_tr16(trb + (jg + k) * 32);
#pragma unroll
        for (int k = 0; k < VB; ++k)
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
            oacc[hb][jg + k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[k], pq[jg / (NJB / NG)][hb],
                                                                        oacc[hb][jg + k], 0, 0, 0);
      }
    }
  };

  for (int it = 0; it < ntiles; it += D) {
    body(std::integral_constant<int, 0>{}, it);
    if constexpr (D > 1) {
      if (it + 1 < ntiles) body(std::integral_constant<int, 1>{}, it + 1);
    }
    if constexpr (D > 2) {
      if (it + 2 < ntiles) body(std::integral_constant<int, 2>{}, it + 2);
    }
    if constexpr (D > 3) {
      if (it + 3 < ntiles) body(std::integral_constant<int, 3>{}, it + 3);
    }
  }
  lds_barrier();   // every wavefront is done with the C tiles the epilogue reuses

  // ---- partial state: O~ / l in bf16, one contiguous block per wavefront
  // ([sequence][split][wavefront][head][RW]), staged in the wavefront's LDS
  // tile so that the stores are 16-byte and contiguous; and (m, l)
  const int64_t pbase = (static_cast<int64_t>(seq) * p.S + split) * p.heads + h0;
  {
    uint16_t *ot = reinterpret_cast<uint16_t *>(ct);  // [HGP][OSTR]
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int h = hb * 16 + li;
      const float l = l_s[h];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      float corr[NG];   // quantised caches: off * sum_t P'_t over the four lanes of head h
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        corr[g] = 0.f;
        if constexpr (CT != CT_BF16) corr[g] = kOff * psum[g][hb][0];
      }
#pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        f32x4 o = oacc[hb][jb];
        if constexpr (CT != CT_BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (o[e] - corr[jb / (NJB / NG)]) * inv;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] *= inv;
        }
        if constexpr (CT == CT_I4) {
          // K positions 16 jb + 4 g + e of the int4 order back to columns
          uint16_t *row = ot + h * OSTR + jb * 16 + 8 * (lg >> 1);
          const int p0 = 4 * (lg & 1);
          const uint32_t a = cvt_bf16x2(o[0], o[1]), c = cvt_bf16x2(o[2], o[3]);
          row[i4_column(p0)] = static_cast<uint16_t>(a);
          row[i4_column(p0 + 1)] = static_cast<uint16_t>(a >> 16);
          row[i4_column(p0 + 2)] = static_cast<uint16_t>(c);
          row[i4_column(p0 + 3)] = static_cast<uint16_t>(c >> 16);
        } else {
          *reinterpret_cast<u32x2 *>(ot + h * OSTR + jb * 16 + 4 * lg) =
              u32x2{cvt_bf16x2(o[0], o[1]), cvt_bf16x2(o[2], o[3])};
        }
      }
    }
    // same-wavefront LDS write -> read, ordered by the LDS queue; the partials
    // stream out with non-temporal stores (written once, read once by the merge)
    uint16_t *dst = p.opart + ((static_cast<int64_t>(seq) * p.S + split) * W + wave) *
                                  static_cast<int64_t>(p.heads) * RW + static_cast<int64_t>(h0) * RW;
    for (int u = lane; u < hg * RW / 8; u += 64)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4 *>(ot + (u / (RW / 8)) * OSTR + (u % (RW / 8)) * 8),
                                  reinterpret_cast<u32x4 *>(dst + u * 8));
  }
  for (int h = tid; h < hg; h += nthreads) {
    p.ml[2 * (pbase + h)] = m_s[h];
    p.ml[2 * (pbase + h) + 1] = l_s[h];
  }
}

// ------------------------------------------------------------------ MFMA merge
// Workgroup (chunk jc of MR latent rows, head h, 16 sequences), 512 threads;
// the host picks MR so that the grid is (about) one round of the compute
// units.  All global loads are issued up front (one memory round trip):
//   - the chunk of W^u_v,h (MR x d) into registers (int8 codes are exact in
//     bf16; their column scales multiply the result);
//   - (m, l) of every split (threads 0..255: sequence tid / 16, splits
//     tid % 16 + 16 k);
//   - the partial O~ rows of up to kMergeBatch splits (thread = sequence
//     tid / (MR / 8), rows 8 (tid % (MR / 8)) .. +8).
// Then: log-sum-exp weights (16-lane DPP reductions), the merged O~ rows as
// the A operand of v_mfma_f32_16x16x32_bf16 (M = 16 sequences, K = latent
// rows) in LDS, the W chunk to LDS, and O~ W^u_v,h with the B operand read by
// transposing LDS loads -> opj[jc][b][h][:] (float32), summed over the chunks
// by decode_finalize.  W^u_v is read once per (chunk, head, 16 sequences).
constexpr int kMergeBatch = 16;
constexpr int kMergeThreads = 512;

template <typename WT, int MR>
__global__ __launch_bounds__(kMergeThreads) void merge_mfma_kernel(const uint16_t *__restrict__ opart,
                                                                   const float *__restrict__ ml,
                                                                   const WT *__restrict__ Wv,
                                                                   const float *__restrict__ wscale,
                                                                   float *__restrict__ opj, int b, int r,
                                                                   int heads, int d, int S, int RW) {
  constexpr int BB = 16;
  constexpr int NT = kMergeThreads;
  constexpr int OCT = MR / 8;                       // 8-row groups of the chunk
  constexpr int MAXU = (MR * 16 + NT - 1) / NT;     // 8-column W units per thread (d <= 128)
  constexpr int MAXSL = 4;                          // splits per thread held in registers
  static_assert(MR % 32 == 0 && BB * OCT <= NT, "merge chunk");
  extern __shared__ __attribute__((aligned(16))) uint8_t msm[];
  const int WRS = d * 2 + 16;                                  // W chunk row stride (bytes)
  uint8_t *wl = msm;                                           // [MR][WRS]
  u32x4 *aop = reinterpret_cast<u32x4 *>(msm + MR * WRS);      // [MR/32][64]
  float *wts = reinterpret_cast<float *>(aop + (MR / 32) * 64);  // [BB][S]
  const int jc = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * BB;
  const int nbb = min(BB, b - b0);
  const int64_t E = static_cast<int64_t>(heads) * d;
  const int j0 = jc * MR;
  const int rows = min(MR, r - j0);  // multiple of 32
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int units = d / 8;           // 8-column units per row
  // partial-row role
  const int pbi = tid / OCT, poc = tid % OCT, jj0 = poc * 8;
  const bool rvalid = pbi < nbb && jj0 < rows;
  const int pseq = b0 + min(pbi, nbb - 1);
  // split-weight role (threads 0..255)
  const int wbi = (tid >> 4) & 15, sl = tid & 15;
  const int wseq = b0 + min(wbi, nbb - 1);

  // ---- all loads
  u32x4 wreg[MAXU];
#pragma unroll
  for (int k = 0; k < MAXU; ++k) {
    const int u = tid + NT * k;
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
  const int64_t mlbase = static_cast<int64_t>(wseq) * S * heads + h;
  float2 mlv[MAXSL];
#pragma unroll
  for (int k = 0; k < MAXSL; ++k) {
    const int s = sl + 16 * k;
    mlv[k] = (tid < 256 && s < S) ? *reinterpret_cast<const float2 *>(ml + 2 * (mlbase + static_cast<int64_t>(s) * heads))
                                  : float2{-INFINITY, 0.f};
  }
  // partial rows of (sequence, split, head): wavefront-blocked layout
  // [sequence][split][r / RW][head][RW]; consecutive splits are heads * r apart
  const int jrow = j0 + min(jj0, rows - 8);
  const uint16_t *psrc = opart + (static_cast<int64_t>(pseq) * S * (r / RW) + jrow / RW) * heads * RW +
                         static_cast<int64_t>(h) * RW + jrow % RW;
  const int64_t sstride = static_cast<int64_t>(heads) * r;
  // int8 W^u_v: the column scale of this lane's output column in the
  // product below (column block = wavefront, d <= 128), requested now
  float sc0 = 1.f;
  if constexpr (sizeof(WT) == 1)
    if (wave < d / 16) sc0 = wscale[static_cast<int64_t>(h) * d + wave * 16 + (lane & 15)];
  u32x4 pv[kMergeBatch];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    pv[k] = u32x4{0u, 0u, 0u, 0u};
    if (rvalid && k < S) pv[k] = *reinterpret_cast<const u32x4 *>(psrc + k * sstride);
  }

  // ---- split weights: w_s = 2^(m_s - M) l_s / sum (threads 0..255; the
  // 16 lanes of a sequence are one DPP row)
  if (tid < 256) {
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
      if (s < S) wts[wbi * S + s] = w;
      den += w;
    }
    for (int s = sl + 16 * MAXSL; s < S; s += 16) {
      const int64_t o = mlbase + static_cast<int64_t>(s) * heads;
      const float w = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ml[2 * o] - mx) * ml[2 * o + 1];
      wts[wbi * S + s] = w;
      den += w;
    }
    den = dpp_reduce<16, false>(den);
    const float inv = den > 0.f ? 1.f / den : 0.f;
    for (int s = sl; s < S; s += 16) wts[wbi * S + s] *= inv;
  }

  // ---- W registers -> LDS (bf16)
#pragma unroll
  for (int k = 0; k < MAXU; ++k) {
    const int u = tid + NT * k;
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
  if (pbi < BB) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float w = (k < S) ? wts[min(pbi, nbb - 1) * S + k] : 0.f;
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
        const float w = (s0 + k < S) ? wts[min(pbi, nbb - 1) * S + s0 + k] : 0.f;
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
    aop[(jj0 >> 5) * 64 + 16 * ((jj0 >> 3) & 3) + pbi] =
        u32x4{cvt_bf16x2(acc[0], acc[1]), cvt_bf16x2(acc[2], acc[3]),
              cvt_bf16x2(acc[4], acc[5]), cvt_bf16x2(acc[6], acc[7])};
  }
  __syncthreads();

  // ---- O~ W^u_v,h: wavefront w takes 16-column blocks w, w + 8, ...
  const int li = lane & 15, lg = lane >> 4;
  const int nkb = rows / 32;
  for (int nb = wave; nb < d / 16; nb += NT / 64) {
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
    float sc = sc0;
    if constexpr (sizeof(WT) == 1)
      if (nb != wave) sc = wscale[static_cast<int64_t>(h) * d + col];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bo = 4 * lg + e;
      if (bo < nbb) opj[((static_cast<int64_t>(jc) * b + b0 + bo) * heads + h) * d + col] = acc[e] * sc;
    }
  }
}

// ------------------------------------------------------------------ merge (float32 path)
// Workgroup (chunk jc of kMergeRows latent rows, head h, 16 sequences):
//   1. log-sum-exp weights of every split (one wavefront per sequence),
//   2. merged O~ rows of the chunk,
//   3. the chunk's share of O~ W^u_v,h in float32 -> opj[jc][b][h][d].
// Every thread requests its share of the W^u_v chunk first (batches of 16
// independent loads, staged in LDS), and the partial rows of a batch of
// splits together, so no thread walks W or the splits one load at a time.
// W^u_v is read once per (chunk, head): the whole grid reads it once.
constexpr int kMergeF32Batch = 8;

__global__ __launch_bounds__(256) void merge_f32_kernel(const float *__restrict__ opart,
                                                        const float *__restrict__ ml,
                                                        const float *__restrict__ Wv,
                                                        const float *__restrict__ wscale,
                                                        float *__restrict__ opj, int b, int r,
                                                        int heads, int d, int S) {
  constexpr int BB = 16, NT = 256, WB = 16;
  extern __shared__ float fsm[];
  float *wts = fsm;                  // [BB][S]
  float *mv = wts + BB * S;          // [BB][kMergeRows]
  float *wl = mv + BB * kMergeRows;  // [kMergeRows][d]
  const int jc = blockIdx.x, h = blockIdx.y, b0 = blockIdx.z * BB;
  const int nbb = min(BB, b - b0);
  const int64_t E = static_cast<int64_t>(heads) * d;
  const int j0 = jc * kMergeRows;
  const int rows = min(kMergeRows, r - j0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = rows * d;   // W chunk elements, row-major [row][column]

  // ---- W chunk: first batch requested now, stored after the weights
  auto w_at = [&](int idx) {
    const int e = min(idx, nw - 1);
    return Wv + static_cast<int64_t>(j0 + e / d) * E + static_cast<int64_t>(h) * d + e % d;
  };
  float wv[WB];
#pragma unroll
  for (int k = 0; k < WB; ++k) wv[k] = *w_at(tid + NT * k);

  // ---- split weights w_s = 2^(m_s - M) l_s / sum
  for (int bi = wave; bi < nbb; bi += NT / 64) {
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
#pragma unroll
  for (int k = 0; k < WB; ++k)
    if (tid + NT * k < nw) wl[tid + NT * k] = wv[k];
  for (int k0 = WB * NT; k0 < nw; k0 += WB * NT) {
#pragma unroll
    for (int k = 0; k < WB; ++k) wv[k] = *w_at(k0 + tid + NT * k);
#pragma unroll
    for (int k = 0; k < WB; ++k)
      if (k0 + tid + NT * k < nw) wl[k0 + tid + NT * k] = wv[k];
  }
  __syncthreads();

  // ---- merged O~ rows: batches of splits whose partial rows load together
  for (int idx = tid; idx < BB * kMergeRows; idx += NT) {
    const int bi = idx / kMergeRows, jj = idx % kMergeRows;
    float acc = 0.f;
    if (bi < nbb && jj < rows) {
      const int64_t base = static_cast<int64_t>(b0 + bi) * S * heads + h;
      for (int s0 = 0; s0 < S; s0 += kMergeF32Batch) {
        float v[kMergeF32Batch];
#pragma unroll
        for (int k = 0; k < kMergeF32Batch; ++k)
          v[k] = opart[(base + static_cast<int64_t>(min(s0 + k, S - 1)) * heads) * r + j0 + jj];
#pragma unroll
        for (int k = 0; k < kMergeF32Batch; ++k)
          if (s0 + k < S) acc = fmaf(wts[bi * S + s0 + k], v[k], acc);
      }
    }
    mv[idx] = acc;
  }
  __syncthreads();

  // ---- thread -> column i of the head and rows rg, rg + RG, ... of the
  // chunk for every sequence; the RG row groups are summed through LDS
  // (fixed order) after a barrier.  The shares reuse the W chunk's LDS.
  const int RG = NT / d;             // 2 (d = 128) or 4 (d = 64)
  const int i = tid % d, rg = tid / d;
  float acc[BB];
#pragma unroll
  for (int k = 0; k < BB; ++k) acc[k] = 0.f;
  for (int jj = rg; jj < rows; jj += RG) {
    const float w = wl[jj * d + i];
    if (nbb == BB) {
#pragma unroll
      for (int k = 0; k < BB; ++k) acc[k] = fmaf(mv[k * kMergeRows + jj], w, acc[k]);
    } else {
      for (int k = 0; k < nbb; ++k) acc[k] = fmaf(mv[k * kMergeRows + jj], w, acc[k]);
    }
  }
  __syncthreads();                   // every thread is done with the W chunk
  float *red = wl;                   // [RG][BB][d]
#pragma unroll
  for (int k = 0; k < BB; ++k)
    if (k < nbb) red[(rg * BB + k) * d + i] = acc[k];
  __syncthreads();
  const float sc = wscale ? wscale[h * d + i] : 1.f;
  for (int k = rg; k < nbb; k += RG) {
    float v = 0.f;
    for (int g = 0; g < RG; ++g) v += red[(g * BB + k) * d + i];
    opj[((static_cast<int64_t>(jc) * b + b0 + k) * heads + h) * d + i] = v * sc;
  }
}

// O = sum over the JC chunk shares, 4 consecutive outputs per thread
// (n % 4 == 0).  The loads of the first MAXJC chunks are unconditional (a
// chunk index past JC rereads the last chunk and is not summed), so all of
// them are in flight before the first wait.
template <typename OT, int MAXJC>
__global__ __launch_bounds__(256) void finalize_kernel(const float *__restrict__ opj,
                                                       OT *__restrict__ O, int64_t n, int JC) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 v[MAXJC];
#pragma unroll
  for (int c = 0; c < MAXJC; ++c) v[c] = *reinterpret_cast<const f32x4 *>(opj + min(c, JC - 1) * n + i);
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
  const size_t lds = stream_lds_bytes(W, NHB, NKB, T, CT == CT_BF16 ? 0 : (CT == CT_I4 ? 1 : 2));
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<dim3(sp.ntasks), dim3(W * 64), lds, s>>>(sp);
  return hipGetLastError();
}

template <int CT, int NHB, int NKB>
hipError_t launch_stream_tile(const StreamParams &sp, const MfmaShape &sh, hipStream_t s) {
  if constexpr (CT != CT_BF16 && NKB <= 8) {
    if (sh.T == 64) {
      if constexpr (stream_depth_fits(CT == CT_I4, NHB, NKB, 3))
        if (sh.D == 3) return launch_stream_t<CT, NHB, NKB, 64, 3>(sp, sh.W, s);
      if constexpr (stream_depth_fits(CT == CT_I4, NHB, NKB, 2))
        if (sh.D >= 2) return launch_stream_t<CT, NHB, NKB, 64, 2>(sp, sh.W, s);
      return launch_stream_t<CT, NHB, NKB, 64, 1>(sp, sh.W, s);
    }
  }
  if constexpr (NHB == 2) {
    return launch_stream_t<CT, NHB, NKB, 32, 1>(sp, sh.W, s);  // mfma_shape pairs NHB = 2 with T >= 32
  } else {
    if (sh.T == 32) return launch_stream_t<CT, NHB, NKB, 32, 1>(sp, sh.W, s);
    if (sh.D == 1) return launch_stream_t<CT, NHB, NKB, 16, 1>(sp, sh.W, s);
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
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), lds);
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
  // d is 64 or 128 (validated by the caller): 16 lanes take d / 16 elements each
  if (a.d == 64) return run_absorb<QT, WT, OT, 4>(grid, s, q, w, a, qt, scale);
  return run_absorb<QT, WT, OT, 8>(grid, s, q, w, a, qt, scale);
}

hipError_t launch_merge_f32(const DecodeArgs &a, const DecodePlan &p, const float *opart,
                            const float *ml, float *opj, hipStream_t s) {
  const int JC = (a.r + kMergeRows - 1) / kMergeRows;
  const size_t lds = (static_cast<size_t>(16) * p.splits + 16 * kMergeRows +
                      static_cast<size_t>(kMergeRows) * a.d) * sizeof(float);
  auto kern = merge_f32_kernel;
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<dim3(JC, a.heads, (a.b + 15) / 16), dim3(256), lds, s>>>(
      opart, ml, static_cast<const float *>(a.Wu_v), a.wu_scale_v, opj, a.b, a.r, a.heads, a.d,
      p.splits);
  return hipGetLastError();
}

size_t merge_mfma_lds(int MR, int d, int S) {
  return static_cast<size_t>(MR) * (d * 2 + 16) + static_cast<size_t>(MR / 32) * 64 * 16 +
         static_cast<size_t>(16) * S * sizeof(float);
}

template <typename WT, int MR>
hipError_t launch_merge_mfma_t(const DecodeArgs &a, const DecodePlan &p, const uint16_t *opart,
                               const float *ml, float *opj, hipStream_t s) {
  const size_t lds = merge_mfma_lds(MR, a.d, p.splits);
  auto kern = merge_mfma_kernel<WT, MR>;
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<dim3(p.jc, a.heads, (a.b + 15) / 16), dim3(kMergeThreads), lds, s>>>(
      opart, ml, static_cast<const WT *>(a.Wu_v), a.wu_scale_v, opj, a.b, a.r, a.heads, a.d,
      p.splits, p.rw);
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_merge_mfma(const DecodeArgs &a, const DecodePlan &p, const uint16_t *opart,
                             const float *ml, float *opj, hipStream_t s) {
  switch (p.merge_rows) {
    case 32: return launch_merge_mfma_t<WT, 32>(a, p, opart, ml, opj, s);
    case 64: return launch_merge_mfma_t<WT, 64>(a, p, opart, ml, opj, s);
    case 96: return launch_merge_mfma_t<WT, 96>(a, p, opart, ml, opj, s);
    case 128: return launch_merge_mfma_t<WT, 128>(a, p, opart, ml, opj, s);
    case 192: return launch_merge_mfma_t<WT, 192>(a, p, opart, ml, opj, s);
    default: return launch_merge_mfma_t<WT, 256>(a, p, opart, ml, opj, s);
  }
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
  // d is 64 or 128 (validated by the caller)
  if (a.d == 64) return launch_absorb_mfma_t<WT, 2>(a, qt, s);
  return launch_absorb_mfma_t<WT, 4>(a, qt, s);
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
    const int kind = c_dtype == QSVD_BF16 ? 0 : (c_dtype == QSVD_I4 ? 1 : 2);
    s.NHB = (heads > 16 && nkb <= 6 && stream_lds_bytes(W, 2, nkb, 32, kind) <= kMaxLds) ? 2 : 1;
    s.T = (nkb <= 10 && stream_lds_bytes(W, s.NHB, nkb, 32, kind) <= kMaxLds) ? 32 : 16;
    // quantised codes stage in few registers: a 64-token tile halves the
    // per-token share of the barriers and the softmax where LDS holds it
    if (c_dtype != QSVD_BF16 && s.T == 32 && nkb <= 8 && stream_lds_bytes(W, s.NHB, nkb, 64, kind) <= kMaxLds)
      s.T = 64;
    // tuning override of the tile (32: one tile of loads in flight, 16: two)
    static const int tile_env = [] {
      const char *e = std::getenv("QSVD_STREAM_TILE");
      return e ? std::atoi(e) : 0;
    }();
    if (tile_env == 16 && s.NHB == 1) s.T = 16;
    if (tile_env == 32 && nkb <= 10 && stream_lds_bytes(W, s.NHB, nkb, 32, kind) <= kMaxLds) s.T = 32;
    // tiles of loads in flight: two for 16-token tiles, else one.  Quantised
    // 64-token tiles could stage two, but the second adds register pressure
    // and no speed (W8A4 shape: 36.6 vs 36.8 us int4, 38.9 vs 39.1 us int8);
    // tuning override QSVD_STREAM_DEPTH = 1..3
    s.D = (s.T == 16) ? 2 : 1;
    static const int depth_env = [] {
      const char *e = std::getenv("QSVD_STREAM_DEPTH");
      return e ? std::atoi(e) : 0;
    }();
    if (s.T == 64 && depth_env >= 1 && depth_env <= 3 && stream_depth_fits(kind == 1, s.NHB, nkb, depth_env))
      s.D = depth_env;
    if (s.T == 16 && depth_env == 1) s.D = 1;
    if (stream_lds_bytes(W, s.NHB, nkb, s.T, kind) > kMaxLds) return false;
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
    static const bool no_wide = [] {
      const char *e = std::getenv("QSVD_NO_WIDE");   // tuning override: single pass only
      return e && std::atoi(e) == 1;
    }();
    if (!no_wide && wide_applies(r, heads, c_dtype, G)) {
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
      S = std::max<int64_t>(1, std::min<int64_t>(S, (L + 15) / 16));
      S = std::min<int64_t>(S, max_splits);
      p.chunk = (L + S - 1) / S;
    }
    p.splits = static_cast<int>((L + p.chunk - 1) / p.chunk);
    // small problems in one launch: at most 64 tokens per wavefront and one
    // round of workgroups; a caller's explicit split count keeps the split path
    p.fused = splits == 0 && r <= 256 && L <= 64 * kFusedWaves &&
              static_cast<int64_t>(b) * heads <= kNumCU;
  }
  // merge chunk: the fewest rounds of workgroups over the compute units, then
  // the most workgroups (smallest chunk) within that many rounds
  if (p.mfma) {
    const int64_t groups = static_cast<int64_t>(heads) * ((b + 15) / 16);
    int best = 256;
    int64_t best_rounds = INT64_MAX;
    for (int mr : {256, 192, 128, 96, 64, 32}) {
      const int64_t jc = (r + mr - 1) / mr;
      const int64_t rounds = (jc * groups + kNumCU - 1) / kNumCU;
      if (rounds <= best_rounds) {
        best_rounds = rounds;
        best = mr;
      }
    }
    p.merge_rows = best;
  } else {
    p.merge_rows = kMergeRows;
  }
  p.jc = (r + p.merge_rows - 1) / p.merge_rows;
  const size_t esz = p.mfma ? 2 : 4;
  p.qt_bytes = align256(static_cast<size_t>(b) * heads * r * esz);
  const size_t opart = align256(static_cast<size_t>(b) * p.splits * heads * r * esz);
  const size_t ml = align256(static_cast<size_t>(b) * p.splits * heads * 2 * sizeof(float));
  const size_t opj = align256(static_cast<size_t>(p.jc) * b * heads * d * sizeof(float));
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

  if (p.fused) {
    LaunchTimer t("decode_fused", s);
    const int maxj = (a.r + 63) / 64;
    const size_t lds = (static_cast<size_t>(a.r) * (kFusedWaves + 2) + 2 * kFusedWaves + 64 * kFusedWaves) *
                       sizeof(float);
    const dim3 grid(a.heads, a.b), block(64 * kFusedWaves);
    const auto *q = static_cast<const float *>(a.q);
    const auto *C = static_cast<const float *>(a.C);
    const auto *Wk = static_cast<const float *>(a.Wu_k);
    const auto *Wv = static_cast<const float *>(a.Wu_v);
    auto *O = static_cast<float *>(a.O);
    const float scale = a.softmax_scale * kLog2e;
    switch (maxj) {
      case 1: decode_f32_fused_kernel<1><<<grid, block, lds, s>>>(q, C, Wk, Wv, O, a.L, a.r, a.heads, a.d, scale); break;
      case 2: decode_f32_fused_kernel<2><<<grid, block, lds, s>>>(q, C, Wk, Wv, O, a.L, a.r, a.heads, a.d, scale); break;
      case 3: decode_f32_fused_kernel<3><<<grid, block, lds, s>>>(q, C, Wk, Wv, O, a.L, a.r, a.heads, a.d, scale); break;
      default: decode_f32_fused_kernel<4><<<grid, block, lds, s>>>(q, C, Wk, Wv, O, a.L, a.r, a.heads, a.d, scale); break;
    }
    return hipGetLastError();
  }

  // ---- absorb
  {
    LaunchTimer t("decode_absorb", s);
    if (!p.mfma) {
      e = launch_absorb_t<float, float, float>(a, static_cast<float *>(qt), s);
    } else if (a.wu_dtype == QSVD_I8) {
      e = launch_absorb_mfma<int8_t>(a, static_cast<uint16_t *>(qt), s);
    } else {
      e = launch_absorb_mfma<uint16_t>(a, static_cast<uint16_t *>(qt), s);
    }
    if (e != hipSuccess) return e;
  }

  // ---- stream (two passes for wide latents with many heads)
  if (p.wide) {
    uint8_t *wbase = reinterpret_cast<uint8_t *>(opj) +
                     align256(static_cast<size_t>(p.jc) * a.b * a.heads * a.d * sizeof(float));
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
    const int JC = p.jc;
    const dim3 grid(static_cast<unsigned>((n / 4 + 255) / 256)), block(256);
    auto run = [&](auto OTV, auto MJ) {
      using OT = decltype(OTV);
      finalize_kernel<OT, decltype(MJ)::value><<<grid, block, 0, s>>>(opj, static_cast<OT *>(a.O), n, JC);
    };
    auto pick = [&](auto OTV) {
      if (JC <= 8) run(OTV, std::integral_constant<int, 8>{});
      else if (JC <= 16) run(OTV, std::integral_constant<int, 16>{});
      else run(OTV, std::integral_constant<int, 32>{});
    };
    if (a.o_dtype == QSVD_BF16) pick(uint16_t{});
    else pick(float{});
    e = hipGetLastError();
  }
  return e;
}

}  // namespace qsvd
