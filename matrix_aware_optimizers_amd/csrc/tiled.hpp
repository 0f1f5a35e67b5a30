// Tiled bf16 layout of the Newton-Schulz workspaces.
//
// A matrix of R x C logical elements is stored padded to Rp x Cp (both
// multiples of 256, the pad zero) as 32 x 32 blocks of 2 KB, block (I, J) at
// element (I * Cp / 32 + J) * 1024. Inside a block row r holds 32 elements
// (64 bytes) as four 16-byte chunks, logical chunk c at position
// c ^ t32_swz(r). Two reads of the same storage come out as whole 1 KB runs:
// the 256 x 32 slice of a 256-row band (K-contiguous operand) is 8 blocks of a
// block column, and the 32 x 256 slice of a K x N operand is 8 consecutive
// blocks of a block row. The chunk permutation is the one the contraction
// kernel uses for its LDS tiles, so a slice is copied into LDS unchanged.
#pragma once

#include "common.hpp"

namespace mao {

__host__ __device__ __forceinline__ int t32_swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// Element offset of logical (i, k) in a tiled matrix with padded width cp.
__host__ __device__ __forceinline__ int64_t t32_off(int64_t i, int64_t k, int64_t cp) {
  return ((((i >> 5) * (cp >> 5)) + (k >> 5)) << 10) + ((i & 31) << 5) +
         ((int64_t)((((int)(k >> 3) & 3) ^ t32_swz((int)(i & 31)))) << 3) + (k & 7);
}

inline int64_t t32_pad(int64_t n) { return round_up(n, 256); }

}  // namespace mao
