// Global -> LDS operand staging shared by the MFMA kernels that stream two
// K-contiguous operands (gfx950).
//
// A K stage is BK = 128 bytes of every operand row (one cache line).  One
// buffer_load_dwordx4 ... lds moves 64 lanes x 16 bytes = 8 rows of a stage
// straight into LDS: lane l writes at l * 16, so it fetches row l / 8 and the
// chunk that belongs at position l % 8 of that row.  In LDS the 16-byte chunk
// c of row r sits at position c ^ swz(r), which keeps the MFMA operand reads
// (32 consecutive rows, one chunk per half-wavefront) free of bank conflicts.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qsvd {
namespace dma {

constexpr int BK = 128;                  // K bytes per stage (128 int8 or 64 bf16)
constexpr int kRowsPerDma = 1024 / BK;   // rows filled by one DMA instruction

// buffer resource over [base, base + bytes); reads past the end return zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_rows(const uint8_t *base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), static_cast<short>(0),
                                           static_cast<int>(n), 0x00020000);
}

__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(uint8_t *p) {
  return (__attribute__((address_space(3))) void *)(p);
}

// s_waitcnt vmcnt(0) lgkmcnt(0): every DMA of this wavefront has landed in
// LDS and its LDS reads have returned.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0070); }

// position of 16-byte chunk c of LDS row r is c ^ swz(r): distinct for any 8
// consecutive rows (128-byte bank window) and, with the row parity, for any 16
// consecutive rows (256-byte window)
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// byte offset, inside a DMA block, of the chunk lane l fetches, for a wavefront
// whose blocks start at rows wave * kRowsPerDma (mod 16) of the slot
__device__ __forceinline__ uint32_t lane_offset(int lane, int wave, int64_t row_bytes) {
  const int lr = lane >> 3;
  return static_cast<uint32_t>(lr * row_bytes + (((lane & 7) ^ swz(wave * kRowsPerDma + lr)) * 16));
}

}  // namespace dma
}  // namespace qsvd
