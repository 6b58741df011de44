// Two-pass decode for wide latents with many heads (bf16 caches, gfx950).
//
// QSVD paper notes, "Key design": K = C W^u_k and V = C W^u_v are rebuilt from
// the cached latent on demand; the WSVD digest ("Method, 3.4") folds the
// value up-projection into the output side.  The single-pass stream kernel
// keeps, per workgroup, the absorbed queries Q~ and the running O~ of every
// head it owns in registers.  At r = 2304 with 40 heads (LLaVA-v1.5-13B) that
// state is about 550 KB, more than a compute unit holds, so the single pass
// splits the heads into three workgroups that each stream the cache.  Here the
// two halves of the work run as two passes that each read the cache once:
//
//   wide_scores_kernel  per (sequence, chunk of tokens): S = C Q~^T for every
//                       head (scores in log2 units, Q~ pre-scaled), written to
//                       the workspace as S[b][heads][Lp], plus the chunk's
//                       maximum per head.  Only Q~ is resident.
//   wide_values_kernel  per (sequence, split, 256-column chunk of r):
//                       p = 2^(S - m_split), O~ = p^T C over the split's
//                       tokens for every head and the chunk's columns, and
//                       l = sum p.  Only a 256-column slice of O~ is resident.
//
// The value pass writes (O~ / l, m, l) in the single pass's partial layout, so
// the log-sum-exp merge and the W^u_v projection that follow are shared.
#include "device_common.h"
#include "qsvd_internal.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

namespace qsvd {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWideW = 8;        // wavefronts of the score pass; r = 8 * 32 * NKB
constexpr int kWideT = 32;       // tokens per tile (both passes)
constexpr int kWideCW = 256;     // columns per value-pass workgroup
constexpr int kWideVW = 4;       // wavefronts of the value pass (64 columns each)
constexpr int kWideCUs = 256;

template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false)));
}
// maximum over each aligned group of 32 lanes
__device__ __forceinline__ float max32(float v) {
  v = dpp_max<0xB1>(v);
  v = dpp_max<0x4E>(v);
  v = dpp_max<0x141>(v);
  v = dpp_max<0x140>(v);
  return fmaxf(v, __shfl_xor(v, 16, kWave));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const void *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}

__device__ __forceinline__ int xcd_task() {
  const int total = gridDim.x, id = blockIdx.x;
  const int per = total / 8, rem = total % 8, xcd = id % 8, local = id / 8;
  return xcd * per + min(xcd, rem) + local;
}

__device__ __forceinline__ bf16x4 wide_read_tr16(const uint8_t *p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16 *)(
          reinterpret_cast<__attribute__((address_space(3))) uint8_t *>(reinterpret_cast<uintptr_t>(p))));
  return __builtin_bit_cast(bf16x4, v);
}

// ------------------------------------------------------------------ score pass
// Workgroup (sequence, chunk of C1 tokens), 8 wavefronts; wavefront w owns
// latent columns 32 NKB w .. +32 NKB.  Per 32-token tile: each wavefront's
// partial scores S_w = C[:, cols_w] Q~[:, cols_w]^T (v_mfma_f32_16x16x32_bf16,
// the cache rows straight from the load registers as the A operand, Q~ held
// as the B operand for the whole chunk) go to LDS; the workgroup sums the 8
// partials, writes S and keeps the running maximum of each head.
template <int NH, int NKB>
__global__ __launch_bounds__(512) void wide_scores_kernel(WideArgs p) {
  constexpr int HS = NH * 16, SPR = kWideT + 4, RW = 32 * NKB;
  extern __shared__ __attribute__((aligned(16))) float spart[];   // [8][HS][SPR]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int task = xcd_task();
  const int chunk = task % p.nchunk1;
  const int64_t seq = task / p.nchunk1;
  const int64_t L = p.L;
  const int64_t t_begin = static_cast<int64_t>(chunk) * p.chunk1;
  const int64_t t_end = std::min<int64_t>(t_begin + p.chunk1, L);
  const int ntiles = t_begin < t_end ? static_cast<int>((t_end - t_begin + kWideT - 1) / kWideT) : 0;
  const int64_t row_bytes = static_cast<int64_t>(p.r) * 2;
  const int j0w = wave * RW;
  const uint8_t *C = static_cast<const uint8_t *>(p.C);

  // tile registers: [16-token block][K block]: token 16 tb + li, columns
  // j0w + 32 kb + 8 lg .. +8; a block's rows of the next tile are requested
  // as soon as its products have read them
  u32x4 stage[2][NKB];
  // (branch-free: past the chunk's last tile the resource is empty, which
  // reads zeros without memory traffic and keeps the compiler's waits exact)
  auto load_rows = [&](int it, int tb, bool valid) {
    const int64_t t0 = valid ? t_begin + static_cast<int64_t>(it) * kWideT : t_end;
    const __amdgpu_buffer_rsrc_t rc = wide_rsrc(C + (seq * L + t0) * row_bytes, (t_end - t0) * row_bytes);
    const uint32_t vo = static_cast<uint32_t>((16 * tb + li) * row_bytes + (j0w + 8 * lg) * 2);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) stage[tb][kb] = __builtin_amdgcn_raw_buffer_load_b128(rc, vo + 64 * kb, 0, 0);
  };
  load_rows(0, 0, ntiles > 0);
  load_rows(0, 1, ntiles > 0);

  // absorbed queries as the B operand: head 16 hb + li, columns j0w + 32 kb + 8 lg .. +8
  bf16x8 qf[NH][NKB];
  const uint16_t *qt = static_cast<const uint16_t *>(p.qt);
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int h = hb * 16 + li;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (h < p.heads) v = *reinterpret_cast<const u32x4 *>(qt + (seq * p.heads + h) * p.r + j0w + 32 * kb + 8 * lg);
      qf[hb][kb] = __builtin_bit_cast(bf16x8, v);
    }

  // the (head, token) items of the cross-wavefront sum: item tid + 512 k is
  // head tid / 32 + 16 k, token tid % 32 (32 lanes per head)
  float mrun[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) mrun[k] = -INFINITY;
  float *S = p.S;

  for (int it = 0; it < ntiles; ++it) {
    const int64_t t0 = t_begin + static_cast<int64_t>(it) * kWideT;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      f32x4 sacc[NH];
#pragma unroll
      for (int hb = 0; hb < NH; ++hb) sacc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hb = 0; hb < NH; ++hb)
          sacc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, stage[tb][kb]),
                                                             qf[hb][kb], sacc[hb], 0, 0, 0);
      load_rows(it + 1, tb, it + 1 < ntiles);
      // lane holds tokens 16 tb + 4 lg + (0..3) of head 16 hb + li
#pragma unroll
      for (int hb = 0; hb < NH; ++hb)
        *reinterpret_cast<f32x4 *>(spart + (wave * HS + hb * 16 + li) * SPR + tb * 16 + 4 * lg) = sacc[hb];
    }
    lds_barrier();   // the next tile's loads stay in flight
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const int h = (tid >> 5) + 16 * k, t = tid & 31;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWideW; ++w) s += spart[(w * HS + h) * SPR + t];
      const int64_t tok = t0 + t;
      if (h < p.heads && tok < t_end) {
        __builtin_nontemporal_store(s, &S[(seq * p.heads + h) * p.Lp + tok]);   // streamed out, read by the value pass
        mrun[k] = fmaxf(mrun[k], s);
      }
    }
    lds_barrier();
  }

#pragma unroll
  for (int k = 0; k < NH; ++k) {
    const int h = (tid >> 5) + 16 * k;
    const float m = max32(mrun[k]);
    if ((tid & 31) == 0 && h < p.heads) p.m1[(seq * p.nchunk1 + chunk) * p.heads + h] = m;
  }
}

// ------------------------------------------------------------------ value pass
// Workgroup (sequence, split, 256-column chunk cc), 4 wavefronts of 64
// columns each.  The split's maximum per head comes from the score pass's
// chunk maxima.  A 32-token tile (32 rows x 512 bytes) moves from memory
// straight into an LDS buffer by buffer_load ... lds, one tile ahead of
// the one in use; in LDS the 16-byte chunk c of row R sits at c ^ vsw(R), so
// the 4 rows of a transposing read fall in distinct banks.  The probabilities
// p = 2^(S - m) of a tile are formed once per workgroup, one tile ahead
// (wavefront w: tokens 8 w .. 8 w + 7 of every head), as bf16 MFMA operand
// fragments in LDS.  Each wavefront forms O~^T[cols][heads] += C_tile^T P^T
// with v_mfma_f32_16x16x32_bf16: A = C^T from gfx950's transposing LDS reads,
// B = P^T from the fragments.
__device__ __forceinline__ int vsw(int row) { return 2 * (row & 3); }

// workgroups of the value pass per compute unit (its register budget)
constexpr int wide_values_per_cu(int nh) { return nh <= 3 ? 3 : 2; }
// LDS tile buffers: the tile in use and the one in flight.  The loop waits for
// every outstanding vector-memory operation (vmcnt 0) before it reads a tile
// that arrived by LDS DMA: the compiler does not track those loads, and a
// wait that counted the instructions issued after the DMA would silently
// release early if code generation split or merged one of them.  A third
// buffer would add nothing under that wait.
constexpr int wide_values_bufs(int) { return 2; }

template <int NH>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(wide_values_per_cu(NH), wide_values_per_cu(NH))))
void wide_values_kernel(WideArgs p) {
  constexpr int RB = kWideCW * 2;               // bytes of a tile row
  constexpr int TB = kWideT * RB;               // bytes of a tile
  constexpr int NJB = kWideCW / kWideVW / 16;   // 16-column blocks per wavefront
  constexpr int NBUF = wide_values_bufs(NH);
  constexpr int PB = NH * 64 * 16;              // bytes of a tile's p fragments
  // s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima): every load
  // issued so far, the DMA of the tile about to be read included, has landed
  constexpr int kWaitImm = 0x0070 | 0x0F00;
  static_assert(NBUF == 2, "the full vmcnt wait leaves nothing for a third buffer to overlap");
  __shared__ __attribute__((aligned(1024))) uint8_t ct[NBUF][TB];
  __shared__ __attribute__((aligned(16))) uint8_t pf[2][PB];
  __shared__ float lred[kWideVW][NH * 16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int ncc = p.r / kWideCW;
  const int task = xcd_task();
  const int cc = task % ncc;
  const int split = (task / ncc) % p.splits;
  const int64_t seq = task / (ncc * p.splits);
  const int64_t L = p.L;
  const int64_t t_begin = static_cast<int64_t>(split) * p.chunk3;
  const int64_t t_end = std::min<int64_t>(t_begin + p.chunk3, L);
  const int ntiles = t_begin < t_end ? static_cast<int>((t_end - t_begin + kWideT - 1) / kWideT) : 0;
  const int64_t row_bytes = static_cast<int64_t>(p.r) * 2;
  const uint8_t *C = static_cast<const uint8_t *>(p.C);

  // the split's reference maximum for this lane's heads 16 hb + li: the
  // maximum over the score-pass chunks the split overlaps (an upper bound of
  // the split's own maximum, which the merge's rescaling accepts)
  float mh[NH];
  {
    const int c0 = static_cast<int>(t_begin / p.chunk1);
    const int c1 = std::min(static_cast<int>((t_end + p.chunk1 - 1) / p.chunk1), p.nchunk1);
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int h = hb * 16 + li;
      float m = -INFINITY;
      if (h < p.heads)
        for (int c = c0; c < c1; ++c) m = fmaxf(m, p.m1[(seq * p.nchunk1 + c) * p.heads + h]);
      mh[hb] = m;
    }
  }

  // DMA of tile it into buffer buf: wavefront w fills rows 8 w .. 8 w + 7, two
  // rows per instruction (lane l: row 2 m + l / 32, LDS chunk l % 32)
  auto dma_tile = [&](int it, int buf) {
    const int64_t t0 = t_begin + static_cast<int64_t>(it) * kWideT;
    const __amdgpu_buffer_rsrc_t rc = wide_rsrc(C + (seq * L + t0) * row_bytes, (t_end - t0) * row_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wave * 4 + i;
      const int row = 2 * m + (lane >> 5);
      const uint32_t vo = static_cast<uint32_t>(row * row_bytes + cc * RB + (((lane & 31) ^ vsw(row)) * 16));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rc, (__attribute__((address_space(3))) void *)(&ct[buf][2 * m * RB]), 16, vo, 0, 0, 0);
    }
  };
  // scores of this lane's heads 16 hb + li and tokens t0 + 8 wave + 2 lg + (0, 1)
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  auto load_scores = [&](int it, f32x2 (&dst)[NH]) {
    const int64_t t0 = t_begin + static_cast<int64_t>(it) * kWideT;
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int h = min(hb * 16 + li, p.heads - 1);   // padded heads read a real row, unused
      dst[hb] = *reinterpret_cast<const f32x2 *>(p.S + (seq * p.heads + h) * p.Lp + t0 + 8 * wave + 2 * lg);
    }
  };
  // p of tile it from its scores into fragment buffer pbuf: the fragment of
  // lane (li, g) of head block hb holds tokens 8 g .. 8 g + 7 of head 16 hb + li
  float lsum[NH];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) lsum[hb] = 0.f;
  auto make_p = [&](int it, const f32x2 (&sv)[NH], int pbuf, bool count) {
    const int64_t t0 = t_begin + static_cast<int64_t>(it) * kWideT;
    const int64_t tk = t0 + 8 * wave + 2 * lg;
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) {
      const int h = hb * 16 + li;
      float p0 = __builtin_amdgcn_exp2f(sv[hb][0] - mh[hb]);
      float p1 = __builtin_amdgcn_exp2f(sv[hb][1] - mh[hb]);
      if (h >= p.heads || tk >= t_end) p0 = 0.f;   // tokens past the split drop out
      if (h >= p.heads || tk + 1 >= t_end) p1 = 0.f;
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{p0, p1}, bf16x2));
      *reinterpret_cast<uint32_t *>(&pf[pbuf][(hb * 64 + wave * 16 + li) * 16 + 4 * lg]) = pk;
      // l sums the same bf16 probabilities the product uses
      if (count) lsum[hb] += __uint_as_float(pk << 16) + __uint_as_float(pk & 0xFFFF0000u);
    }
  };

  f32x4 oacc[NH][NJB];
#pragma unroll
  for (int hb = 0; hb < NH; ++hb)
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) oacc[hb][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Order of the loads: scores 0 (used at once), DMA 0, scores 1, then in
  // iteration k the scores of tile k + 2 and the DMA of tile k + 1 (past the
  // end: repeats of the last tile into a buffer that is not read again).
  f32x2 snext[NH];
  if (ntiles > 0) {
    f32x2 s0[NH];
    load_scores(0, s0);
    make_p(0, s0, 0, true);
    __builtin_amdgcn_sched_barrier(0);
    dma_tile(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load_scores(min(1, ntiles - 1), snext);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it % NBUF;
    f32x2 scur[NH];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) scur[hb] = snext[hb];
    // tile it and p(it) are in LDS for every wavefront; every wavefront is
    // done with tile it - 1 and p(it - 1)
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(kWaitImm);
    lds_barrier();   // also completes this wavefront's p fragment writes first
    __builtin_amdgcn_sched_barrier(0);
    load_scores(min(it + 2, ntiles - 1), snext);
    dma_tile(min(it + NBUF - 1, ntiles - 1), (it + NBUF - 1) % NBUF);
    __builtin_amdgcn_sched_barrier(0);
    // p of the next tile (a repeat past the end: written, not read, not counted)
    make_p(min(it + 1, ntiles - 1), scur, (it + 1) & 1, it + 1 < ntiles);

    bf16x8 pb[NH];
#pragma unroll
    for (int hb = 0; hb < NH; ++hb) pb[hb] = *reinterpret_cast<const bf16x8 *>(&pf[it & 1][(hb * 64 + lane) * 16]);

    // A = C^T: column 16 jb + li of this wavefront, tokens 8 lg + (0..7): lane
    // li reads 8 bytes of row 8 lg + li / 4 (+ 4) at column 4 (li % 4)
    const int rlo = 8 * lg + (li >> 2);
    const uint8_t *rowp = &ct[buf][rlo * RB];
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb) {
      const int ob = wave * (kWideCW / kWideVW) * 2 + jb * 32 + 8 * (li & 3);   // byte within the row
      const int pos = (((ob >> 4) ^ vsw(rlo)) << 4) | (ob & 15);
      const bf16x4 lo = wide_read_tr16(rowp + pos);
      const bf16x4 hi = wide_read_tr16(rowp + 4 * RB + pos);   // rows + 4 share the swizzle
      const bf16x8 av = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int hb = 0; hb < NH; ++hb)
        oacc[hb][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[hb], oacc[hb][jb], 0, 0, 0);
    }
  }
  // the repeated DMAs past the end land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0070);

  // l per head: the 4 lane groups and the 4 wavefronts hold disjoint tokens
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    float l = lsum[hb];
    l += __shfl_xor(l, 16, kWave);
    l += __shfl_xor(l, 32, kWave);
    if (lg == 0) lred[wave][hb * 16 + li] = l;
  }
  __syncthreads();
  const int nsplit = p.splits;
  const int rw = kWideCW / kWideVW;
  const int cg = cc * kWideVW + wave;   // 64-column group of r
#pragma unroll
  for (int hb = 0; hb < NH; ++hb) {
    const int h = hb * 16 + li;
    const float l = (lred[0][hb * 16 + li] + lred[1][hb * 16 + li]) + (lred[2][hb * 16 + li] + lred[3][hb * 16 + li]);
    if (h >= p.heads) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    // oacc[hb][jb] element e: column 16 jb + 4 lg + e of the wavefront's group, head h
    uint16_t *dst = p.opart + (((seq * nsplit + split) * (p.r / rw) + cg) * p.heads + h) * rw;
#pragma unroll
    for (int jb = 0; jb < NJB; ++jb)
      *reinterpret_cast<u32x2 *>(dst + jb * 16 + 4 * lg) =
          u32x2{pack_bf16x2(oacc[hb][jb][0] * inv, oacc[hb][jb][1] * inv),
                pack_bf16x2(oacc[hb][jb][2] * inv, oacc[hb][jb][3] * inv)};
    if (cc == 0 && wave == 0 && lg == 0) {
      p.ml[2 * ((seq * nsplit + split) * p.heads + h)] = mh[hb];
      p.ml[2 * ((seq * nsplit + split) * p.heads + h) + 1] = l;
    }
  }
}

template <int NH, int NKB>
hipError_t launch_scores_t(const WideArgs &a, hipStream_t s) {
  auto kern = wide_scores_kernel<NH, NKB>;
  const size_t lds = static_cast<size_t>(kWideW) * NH * 16 * (kWideT + 4) * sizeof(float);
  hipError_t e = set_dynamic_lds(reinterpret_cast<const void *>(kern), lds);
  if (e != hipSuccess) return e;
  kern<<<dim3(static_cast<unsigned>(a.b * a.nchunk1)), dim3(64 * kWideW), lds, s>>>(a);
  return hipGetLastError();
}

template <int NH>
hipError_t launch_scores_nh(const WideArgs &a, int nkb, hipStream_t s) {
  switch (nkb) {
    case 7: return launch_scores_t<NH, 7>(a, s);
    case 8: return launch_scores_t<NH, 8>(a, s);
    default: return launch_scores_t<NH, 9>(a, s);
  }
}

}  // namespace

// Two passes when the single pass would split the heads into three or more
// workgroups: bf16 cache, r = 8 * 32 * NKB with 7 <= NKB <= 9 (up to r = 2304)
// and 33..64 heads (3 or 4 blocks of 16; Q~ of all heads fits the registers).
bool wide_applies(int r, int heads, int c_dtype, int head_groups) {
  if (c_dtype != QSVD_BF16 || head_groups < 3) return false;
  if (r % (kWideW * 32) != 0 || r % kWideCW != 0) return false;
  const int nkb = r / (kWideW * 32);
  return nkb >= 7 && nkb <= 9 && heads > 32 && heads <= 64;
}

void wide_plan(int b, int64_t L, int r, int heads, WidePlanInfo *w) {
  const int64_t tiles = (L + kWideT - 1) / kWideT;
  // score pass: one workgroup per compute unit
  int64_t nchunk = std::max<int64_t>(1, (kWideCUs + b - 1) / b);
  nchunk = std::min<int64_t>(nchunk, tiles);
  const int64_t chunk1 = ((tiles + nchunk - 1) / nchunk) * kWideT;
  nchunk = (L + chunk1 - 1) / chunk1;
  // value pass: as many splits as one round of workgroups holds, each a whole
  // number of tiles
  const int64_t slots = static_cast<int64_t>(kWideCUs) * wide_values_per_cu((heads + 15) / 16);
  int64_t splits = std::max<int64_t>(1, slots / (static_cast<int64_t>(b) * (r / kWideCW)));
  splits = std::min<int64_t>(std::min<int64_t>(splits, tiles), 1024);
  const int64_t chunk3 = ((tiles + splits - 1) / splits) * kWideT;
  w->chunk1 = chunk1;
  w->nchunk1 = static_cast<int>(nchunk);
  w->chunk3 = chunk3;
  w->splits = static_cast<int>((L + chunk3 - 1) / chunk3);
  w->Lp = ((L + kWideT - 1) / kWideT) * kWideT;
  w->s_bytes = static_cast<size_t>(b) * heads * w->Lp * sizeof(float);
  w->m1_bytes = static_cast<size_t>(b) * w->nchunk1 * heads * sizeof(float);
  w->rw = kWideCW / kWideVW;
}

hipError_t launch_wide_scores(const WideArgs &a, hipStream_t s) {
  const int nh = (a.heads + 15) / 16, nkb = a.r / (kWideW * 32);
  LaunchTimer t("decode_scores", s);
  return nh == 3 ? launch_scores_nh<3>(a, nkb, s) : launch_scores_nh<4>(a, nkb, s);
}

hipError_t launch_wide_values(const WideArgs &a, hipStream_t s) {
  const int nh = (a.heads + 15) / 16;
  const unsigned grid = static_cast<unsigned>(a.b * a.splits * (a.r / kWideCW));
  LaunchTimer t("decode_values", s);
  if (nh == 3)
    wide_values_kernel<3><<<dim3(grid), dim3(64 * kWideVW), 0, s>>>(a);
  else
    wide_values_kernel<4><<<dim3(grid), dim3(64 * kWideVW), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qsvd
