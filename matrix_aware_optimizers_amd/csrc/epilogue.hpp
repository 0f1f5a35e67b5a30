// Epilogue of a 256 x 256 fp32 accumulator tile (4 wavefronts in 2 x 2, each
// 128 x 128 as 4 x 4 blocks of v_mfma_f32_32x32 results), shared by the
// streamed bf16 kernel and the fp32 rank-k update kernel.
//
// D = alpha * acc + beta * C0, rows scaled by row_scale, written to D and/or
// its transpose Dt (the SYRK mirror when D == Dt on a symmetric result).
//
// Staged epilogue (staged_epilogue): the tile goes through LDS in two halves
// of 128 rows, as four 32-row bands of 256 floats (one 32 KB buffer each).
// Row pass: each thread finishes 8
// consecutive columns of a row -- C0 read and D written in 16- (bf16) or
// 32-byte (fp32) pieces, one whole row per 32 lanes -- and, when a transposed
// copy is due, puts the finished values back. Column pass: 16 lanes cover 128
// consecutive rows of one column and write them as one row of Dt. Columns
// are XOR-permuted in groups of 8 by the row (bits 3-4 from row bits 3-4, bit
// 5 from row bit 2 and the band), so accumulator writes are conflict-free and
// column reads meet at most two-way. A diagonal SYRK tile writes D on and
// below the diagonal and the mirror strictly above it. With CHECKED, rows
// past M and columns past N are skipped (edge tiles). C0, D and Dt may each be
// tiled (tiled.hpp); a run of 8 columns starting at a multiple of 8 is one
// contiguous chunk in either layout. A diagonal term dadd is added to D[i][i]
// for i < M (never to the zero pad of a tiled D).
//
// Direct epilogues (direct_epilogue_*): for the cases that need no LDS --
// tiled bf16 results without a transposed copy or row scale, and interior
// tiles of row-major fp32 results without C0 -- each lane's values go out
// from the accumulators after a 4 x 4 transpose across groups of four lanes.
#pragma once

#include "common.hpp"
#include "tiled.hpp"

namespace mao {

__device__ __forceinline__ float c0_load(const void* C0, bool f32, int64_t off) {
  return f32 ? ((const float*)C0)[off] : bf16_to_f32(((const bf16_t*)C0)[off]);
}

__device__ __forceinline__ void d_store(void* D, bool f32, int64_t off, float v) {
  if (f32)
    ((float*)D)[off] = v;
  else
    ((bf16_t*)D)[off] = f32_to_bf16(v);
}

__device__ __forceinline__ int epi_swz(int rb, int band) {
  return ((((rb) >> 3) & 3) << 3) | (((((rb) >> 2) ^ (band)) & 1) << 5);
}

__device__ __forceinline__ void store8_any(void* P, bool f32, int64_t off, const float* v) {
  if (f32) {
    float* dp = (float*)P + off;
    *(float4*)dp = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(dp + 4) = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    pk.z = pack_bf16x2(v[4], v[5]);
    pk.w = pack_bf16x2(v[6], v[7]);
    *(uint4*)((bf16_t*)P + off) = pk;
  }
}

struct EpiArgs {
  int m0, n0, M, N;
  float alpha, beta;
  const void* C0;
  int64_t ldc0;
  bool c32;
  const float* rs;
  void* D;
  int64_t ldd;
  bool d32;
  void* Tt;
  int64_t ldt;
  bool diag;
  // tiled storage (tiled.hpp): the ld fields are then padded widths
  bool c_t32 = false, d_t32 = false, t_t32 = false;
  float dadd = 0.f;  // added to D[i][i], i < M
};

// LB: staging addresses from eight per-lane bases (fewer live registers in the
// tiled kernels); otherwise computed per element. HC0: the tile has a C0 term.
// Without one the row pass issues no loads, so nothing waits on the memory
// counter there: the counter covers loads and stores alike and retires them
// in order, so a wait for a C0 load also waits for every store issued before
// it.
template <bool CHECKED, bool LB = false, bool HC0 = true>
__device__ __forceinline__ void staged_epilogue_impl(const f32x16_t (&acc)[4][4], float* b0, float* b1,
                                                float* b2, float* b3, const EpiArgs& e) {
  constexpr int TB = 256;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  // Staging address of acc[I][j][v]: row rb = 8 g + 4 h + i (g = v / 4,
  // i = v % 4), column (wn 128 + 32 j + r32) ^ epi_swz(rb, I). The swizzle
  // flips column bits 3-4 by g and bit 5 by (h ^ I) & 1, so the address is
  // one of eight per-lane bases (parity p = (j ^ I) & 1, group g) plus a
  // compile-time offset: no per-element address arithmetic.
  int lb[2][4];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      lb[p][g] = 4 * h * TB + wn * 128 + (r32 ^ (g << 3)) + (((p ^ h) & 1) << 5);
#define MAO_BAND(I, ST)                                                                   \
  _Pragma("unroll") for (int j = 0; j < 4; ++j)                                           \
  _Pragma("unroll") for (int v = 0; v < 16; ++v) {                                        \
    if constexpr (LB) {                                                                   \
      (ST)[lb[(j ^ (I)) & 1][v >> 2] + (8 * (v >> 2) + (v & 3)) * TB + (j >> 1) * 64] =    \
          acc[I][j][v];                                                                   \
    } else {                                                                              \
      const int rb_ = 8 * (v >> 2) + 4 * h + (v & 3);                                     \
      const int col_ = (wn * 128 + j * 32 + r32) ^ epi_swz(rb_, I);                       \
      (ST)[rb_ * TB + col_] = acc[I][j][v];                                               \
    }                                                                                     \
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
      MAO_BAND(0, b0)
      MAO_BAND(1, b1)
      MAO_BAND(2, b2)
      MAO_BAND(3, b3)
    }
    __syncthreads();
    if constexpr (!HC0) {
      // no C0: per group of four rows, the eight LDS reads are issued before
      // any row is finished, so their latency is paid once per group
      const int c8 = (threadIdx.x & 31) * 8;
      const int64_t gcol = e.n0 + c8;
      const bool cfull = !CHECKED || gcol + 8 <= e.N;
#pragma unroll 1
      for (int it0 = 0; it0 < 16; it0 += 4) {
        float4 xs[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = (it0 + u) * 8 + (threadIdx.x >> 5);
          const int band = row >> 5, rb = row & 31;
          const float* bp = band == 0 ? b0 : band == 1 ? b1 : band == 2 ? b2 : b3;
          const float* src = bp + rb * TB + (c8 ^ epi_swz(rb, band));
          xs[u][0] = *(const float4*)src;
          xs[u][1] = *(const float4*)(src + 4);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = (it0 + u) * 8 + (threadIdx.x >> 5);
          const int band = row >> 5, rb = row & 31;
          const int64_t grow = e.m0 + half * 128 + row;
          if (CHECKED && (grow >= e.M || gcol >= e.N)) continue;
          float v[8] = {xs[u][0].x, xs[u][0].y, xs[u][0].z, xs[u][0].w,
                        xs[u][1].x, xs[u][1].y, xs[u][1].z, xs[u][1].w};
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] *= e.alpha;
          if (e.dadd != 0.f && grow < e.M) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (grow == gcol + q) v[q] += e.dadd;
          }
          if (e.rs) {
            const float sc = e.rs[grow];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= sc;
          }
          if (e.D) {
            const int64_t off = e.d_t32 ? t32_off(grow, gcol, e.ldd) : grow * e.ldd + gcol;
            if (cfull && (!e.diag || grow >= gcol + 7)) {
              store8_any(e.D, e.d32, off, v);
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q)
                if ((!CHECKED || gcol + q < e.N) && (!e.diag || grow >= gcol + q))
                  d_store(e.D, e.d32, off + q, v[q]);
            }
          }
          if (e.Tt) {
            float* dst = (band == 0 ? b0 : band == 1 ? b1 : band == 2 ? b2 : b3) + rb * TB +
                         (c8 ^ epi_swz(rb, band));
            *(float4*)dst = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
          }
        }
      }
    } else {
      const int c8 = (threadIdx.x & 31) * 8;
      const int64_t gcol = e.n0 + c8;
      const bool cfull = !CHECKED || gcol + 8 <= e.N;
      // four rows at a time: their C0 pieces are all requested before any is
      // used, so the memory latency is paid once per group, not per row
      for (int it0 = 0; it0 < 16; it0 += 4) {
        float cv[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int64_t grow = e.m0 + half * 128 + (it0 + u) * 8 + (threadIdx.x >> 5);
#pragma unroll
          for (int q = 0; q < 8; ++q) cv[u][q] = 0.f;
          if (!HC0 || !e.C0 || (CHECKED && (grow >= e.M || gcol >= e.N))) continue;
          const int64_t off = e.c_t32 ? t32_off(grow, gcol, e.ldc0) : grow * e.ldc0 + gcol;
          if (cfull && e.c32) {
            const float* cp = (const float*)e.C0 + off;
            const float4 y0 = *(const float4*)cp, y1 = *(const float4*)(cp + 4);
            cv[u][0] = y0.x; cv[u][1] = y0.y; cv[u][2] = y0.z; cv[u][3] = y0.w;
            cv[u][4] = y1.x; cv[u][5] = y1.y; cv[u][6] = y1.z; cv[u][7] = y1.w;
          } else if (cfull) {
            const uint4 y = *(const uint4*)((const bf16_t*)e.C0 + off);
            const uint32_t w[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              cv[u][2 * q] = bf16_to_f32((bf16_t)(w[q] & 0xffff));
              cv[u][2 * q + 1] = bf16_to_f32((bf16_t)(w[q] >> 16));
            }
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (gcol + q < e.N) cv[u][q] = c0_load(e.C0, e.c32, off + q);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = (it0 + u) * 8 + (threadIdx.x >> 5);
          const int band = row >> 5, rb = row & 31;
          float* bp = band == 0 ? b0 : band == 1 ? b1 : band == 2 ? b2 : b3;
          float* src = bp + rb * TB + (c8 ^ epi_swz(rb, band));
          const int64_t grow = e.m0 + half * 128 + row;
          if (CHECKED && (grow >= e.M || gcol >= e.N)) continue;
          const float4 x0 = *(const float4*)src, x1 = *(const float4*)(src + 4);
          float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = e.alpha * v[q] + ((HC0 && e.C0) ? e.beta * cv[u][q] : 0.f);
          if (e.dadd != 0.f && grow < e.M) {
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (grow == gcol + q) v[q] += e.dadd;
          }
          if (e.rs) {
            const float sc = e.rs[grow];
#pragma unroll
            for (int q = 0; q < 8; ++q) v[q] *= sc;
          }
          if (e.D) {
            const int64_t off = e.d_t32 ? t32_off(grow, gcol, e.ldd) : grow * e.ldd + gcol;
            if (cfull && (!e.diag || grow >= gcol + 7)) {
              store8_any(e.D, e.d32, off, v);
            } else {
#pragma unroll
              for (int q = 0; q < 8; ++q)
                if ((!CHECKED || gcol + q < e.N) && (!e.diag || grow >= gcol + q))
                  d_store(e.D, e.d32, off + q, v[q]);
            }
          }
          if (e.Tt) {
            *(float4*)src = make_float4(v[0], v[1], v[2], v[3]);
            *(float4*)(src + 4) = make_float4(v[4], v[5], v[6], v[7]);
          }
        }
      }
    }
    if (e.Tt) {
      __syncthreads();
      const int rgrp = threadIdx.x & 15;
      const int band = rgrp >> 2, rb0 = (rgrp & 3) * 8;
      const float* bp = band == 0 ? b0 : band == 1 ? b1 : band == 2 ? b2 : b3;
      const int64_t grow = e.m0 + half * 128 + rgrp * 8;
      const bool rfull = !CHECKED || grow + 8 <= e.M;
      for (int it = 0; it < 16; ++it) {
        const int c = it * 16 + (threadIdx.x >> 4);
        const int64_t gc = e.n0 + c;
        if (CHECKED && (gc >= e.N || grow >= e.M)) continue;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) v[q] = bp[(rb0 + q) * TB + (c ^ epi_swz(rb0 + q, band))];
        const int64_t off = e.t_t32 ? t32_off(gc, grow, e.ldt) : gc * e.ldt + grow;
        if (rfull && (!e.diag || grow > gc)) {
          store8_any(e.Tt, e.d32, off, v);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if ((!CHECKED || grow + q < e.M) && (!e.diag || grow + q > gc))
              d_store(e.Tt, e.d32, off + q, v[q]);
        }
      }
    }
    __syncthreads();
  }
#undef MAO_BAND
}

// Four lanes 4k + q (q = 0..3) each hold x[0..3], rows r..r+3 of column
// 4k + q; afterwards lane 4k + q holds row r + q, columns 4k..4k+3. Two
// butterfly steps over quad-permuting DPP moves (lane bit 0, then bit 1),
// each lane sending the two values whose element index differs from its own
// lane index in that bit.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ void quad_transpose(float& x0, float& x1, float& x2, float& x3, bool b1,
                                               bool b2) {
  // lane bit 0: elements 1, 3 (bit clear) or 0, 2 (bit set) come from lane ^ 1
  const float r0 = dpp_xor1(b1 ? x0 : x1), r1 = dpp_xor1(b1 ? x2 : x3);
  const float n0 = b1 ? r0 : x0, n1 = b1 ? x1 : r0, n2 = b1 ? r1 : x2, n3 = b1 ? x3 : r1;
  // lane bit 1: elements 2, 3 (bit clear) or 0, 1 (bit set) come from lane ^ 2
  const float s0 = dpp_xor2(b2 ? n0 : n2), s1 = dpp_xor2(b2 ? n1 : n3);
  x0 = b2 ? s0 : n0;
  x1 = b2 ? s1 : n1;
  x2 = b2 ? n2 : s0;
  x3 = b2 ? n3 : s1;
}

// alpha * v, or v itself when the product's alpha is one (UNIT): the
// direct epilogues are bound by instruction issue, and the multiply costs
// about an eighth of their time.
template <bool UNIT>
__device__ __forceinline__ float scale_by(float v, float alpha) {
  return UNIT ? v : v * alpha;
}

// Epilogue of a tile whose bf16 D is tiled (tiled.hpp) and has no C0, row
// scale, diagonal term or transposed copy: D = alpha * acc straight from the
// accumulators, no LDS. A 32 x 32 MFMA result gives lane (h, c) rows
// 8 g + 4 h + i (i = 0..3) of column c; after a quad transpose lane
// (h, 4 k + q) holds row 8 g + 4 h + q, columns 4 k..4 k + 3, which it
// writes as 8 bytes. One store instruction of a wavefront then covers rows
// 8 g..8 g + 7 of a block, 512 contiguous bytes.
template <bool UNIT>
__device__ __forceinline__ void direct_epilogue_t32(const f32x16_t (&acc)[4][4], int m0, int n0,
                                                    float alpha, bf16_t* D, int64_t ldd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int q = r32 & 3, k = r32 >> 2;
  const bool qb1 = (q & 1) != 0, qb2 = (q & 2) != 0;
  const int64_t cpb = ldd >> 5;  // blocks per block row
  bf16_t* base = D + ((((int64_t)(m0 >> 5) + wm * 4) * cpb + (n0 >> 5) + wn * 4) << 10);
  int inner[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 8 * g + 4 * h + q;
    inner[g] = r * 32 + (((k >> 1) ^ t32_swz(r)) << 3) + 4 * (k & 1);
  }
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16_t* blk = base + (((int64_t)I * cpb + j) << 10);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x0 = scale_by<UNIT>(acc[I][j][4 * g], alpha), x1 = scale_by<UNIT>(acc[I][j][4 * g + 1], alpha);
        float x2 = scale_by<UNIT>(acc[I][j][4 * g + 2], alpha), x3 = scale_by<UNIT>(acc[I][j][4 * g + 3], alpha);
        quad_transpose(x0, x1, x2, x3, qb1, qb2);
        uint2 pk;
        pk.x = pack_bf16x2(x0, x1);
        pk.y = pack_bf16x2(x2, x3);
        *(uint2*)(blk + inner[g]) = pk;
      }
      // keep the scheduler from hoisting the next block's accumulator reads
      // (their registers would spill)
      __builtin_amdgcn_sched_barrier(0);
    }
}

// The same for a tile of a symmetric product computed on the lower tile
// triangle (tm >= tn) of a tiled bf16 D: D = alpha * acc (+ beta * C0, + dadd
// on the diagonal below row M), written in place and mirrored. Before the
// quad transpose lane (h, c) holds rows 8 g + 4 h + i of column c, which are
// four consecutive columns of row c of the mirror block: the mirror is
// written from there as 8 bytes, and C0 is read there too (C0 is a symmetric
// tiled matrix, so its mirrored entries are its own). On a diagonal tile the
// blocks above the diagonal come from the mirror only, and a diagonal 32 x 32
// block takes its lower part (diagonal included) from D and its strict upper
// part from the mirror, element by element.
template <bool HC0, bool UNIT>
__device__ __forceinline__ void direct_epilogue_t32_syrk(const f32x16_t (&acc)[4][4], int m0, int n0,
                                                         bool diag, float alpha, const bf16_t* C0,
                                                         int64_t ldc0, float beta, float dadd, int M,
                                                         bf16_t* D, int64_t ldd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int q = r32 & 3, k = r32 >> 2;
  const bool qb1 = (q & 1) != 0, qb2 = (q & 2) != 0;
  if (diag && wm < wn) return;  // every block of this quarter lies above the diagonal
  const int64_t cpb = ldd >> 5, cpc = ldc0 >> 5;
  int inner[4], innm[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int r = 8 * g + 4 * h + q;
    inner[g] = r * 32 + (((k >> 1) ^ t32_swz(r)) << 3) + 4 * (k & 1);
    innm[g] = r32 * 32 + ((g ^ t32_swz(r32)) << 3) + 4 * h;
  }
  const int bi0 = (m0 >> 5) + wm * 4, bj0 = (n0 >> 5) + wn * 4;
  // C0 of a row of four blocks is requested one row ahead (two buffers)
  uint2 cb[2][4][4];
  auto load_row = [&](int I, uint2 (&dst)[4][4]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16_t* blk = C0 + ((((int64_t)bj0 + j) * cpc + bi0 + I) << 10);
#pragma unroll
      for (int g = 0; g < 4; ++g) dst[j][g] = *(const uint2*)(blk + innm[g]);
    }
  };
  if constexpr (HC0) load_row(0, cb[0]);
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    if constexpr (HC0) {
      if (I < 3) load_row(I + 1, cb[(I + 1) & 1]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int BI = wm * 4 + I, BJ = wn * 4 + j;  // block within the tile
      if (diag && BI < BJ) continue;
      const bool dblk = diag && BI == BJ;
      bf16_t* dp = D + ((((int64_t)bi0 + I) * cpb + bj0 + j) << 10);
      bf16_t* mp = D + ((((int64_t)bj0 + j) * cpb + bi0 + I) << 10);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x0 = scale_by<UNIT>(acc[I][j][4 * g], alpha), x1 = scale_by<UNIT>(acc[I][j][4 * g + 1], alpha);
        float x2 = scale_by<UNIT>(acc[I][j][4 * g + 2], alpha), x3 = scale_by<UNIT>(acc[I][j][4 * g + 3], alpha);
        if constexpr (HC0) {
          const uint2 c = cb[I & 1][j][g];
          x0 += beta * bf16_to_f32((bf16_t)(c.x & 0xffff));
          x1 += beta * bf16_to_f32((bf16_t)(c.x >> 16));
          x2 += beta * bf16_to_f32((bf16_t)(c.y & 0xffff));
          x3 += beta * bf16_to_f32((bf16_t)(c.y >> 16));
        }
        // mirror: row r32 of block (BJ, BI), columns 8 g + 4 h .. + 3
        if (!dblk) {
          uint2 pk;
          pk.x = pack_bf16x2(x0, x1);
          pk.y = pack_bf16x2(x2, x3);
          *(uint2*)(mp + innm[g]) = pk;
        } else {
          const int c0 = 8 * g + 4 * h;
          const float xs[4] = {x0, x1, x2, x3};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (c0 + i > r32) mp[innm[g] + i] = f32_to_bf16(xs[i]);
        }
        quad_transpose(x0, x1, x2, x3, qb1, qb2);
        if (!dblk) {
          uint2 pk;
          pk.x = pack_bf16x2(x0, x1);
          pk.y = pack_bf16x2(x2, x3);
          *(uint2*)(dp + inner[g]) = pk;
        } else {
          // row r of the diagonal block, columns 4 k + e: the lower part
          const int r = 8 * g + 4 * h + q;
          const bool in_m = m0 + BI * 32 + r < M;
          float xs[4] = {x0, x1, x2, x3};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (r == 4 * k + e && in_m) xs[e] += dadd;
            if (r >= 4 * k + e) dp[inner[g] + e] = f32_to_bf16(xs[e]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Interior tile of a row-major fp32 result without C0 or row scale:
// D = alpha * acc and/or its transposed copy Dt, straight from the
// accumulators in 16-byte pieces (D after the quad transpose, Dt before it:
// column c of a block is row c of Dt). With `diag` the tile is a diagonal
// tile of a symmetric product and Dt is D's mirror (the same matrix): the
// blocks above the diagonal come from the mirror only, and a diagonal block
// takes its lower part from D and its strict upper part from the mirror.
__device__ __forceinline__ void direct_epilogue_f32(const f32x16_t (&acc)[4][4], int m0, int n0,
                                                    bool diag, float alpha, float* D, int64_t ldd,
                                                    float* Dt, int64_t ldt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  const int q = r32 & 3, k = r32 >> 2;
  const bool qb1 = (q & 1) != 0, qb2 = (q & 2) != 0;
  if (diag && wm < wn) return;
  // this wavefront's 128 x 128 quarter: D rows from rb, columns from cb
  const int64_t rb = m0 + wm * 128, cb = n0 + wn * 128;
  float* dq = D ? D + (rb + 4 * h + q) * ldd + cb + 4 * k : nullptr;  // + (32 I + 8 g) ldd + 32 j
  float* tq = Dt ? Dt + (cb + r32) * ldt + rb + 4 * h : nullptr;       // + 32 j ldt + 32 I + 8 g
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int BI = wm * 4 + I, BJ = wn * 4 + j;
      if (diag && BI < BJ) continue;
      const bool dblk = diag && BI == BJ;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x0 = acc[I][j][4 * g] * alpha, x1 = acc[I][j][4 * g + 1] * alpha;
        float x2 = acc[I][j][4 * g + 2] * alpha, x3 = acc[I][j][4 * g + 3] * alpha;
        if (tq) {
          float* t = tq + 32 * j * ldt + 32 * I + 8 * g;
          if (!dblk) {
            *(float4*)t = make_float4(x0, x1, x2, x3);
          } else {
            // strict upper part: row r32 of the block, columns 8 g + 4 h + i
            const int c0 = 8 * g + 4 * h;
            if (c0 + 0 > r32) t[0] = x0;
            if (c0 + 1 > r32) t[1] = x1;
            if (c0 + 2 > r32) t[2] = x2;
            if (c0 + 3 > r32) t[3] = x3;
          }
        }
        if (dq) {
          quad_transpose(x0, x1, x2, x3, qb1, qb2);
          float* d = dq + (32 * I + 8 * g) * ldd + 32 * j;
          if (!dblk) {
            *(float4*)d = make_float4(x0, x1, x2, x3);
          } else {
            const int r = 8 * g + 4 * h + q;
            if (r >= 4 * k + 0) d[0] = x0;
            if (r >= 4 * k + 1) d[1] = x1;
            if (r >= 4 * k + 2) d[2] = x2;
            if (r >= 4 * k + 3) d[3] = x3;
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}

template <bool CHECKED, bool LB = false>
__device__ __forceinline__ void staged_epilogue(const f32x16_t (&acc)[4][4], float* b0, float* b1,
                                                float* b2, float* b3, const EpiArgs& e) {
  // the tiled kernels (LB) take a C0-free copy; the others keep one general
  // copy, which their register budget allows
  if (!LB || e.C0)
    staged_epilogue_impl<CHECKED, LB, true>(acc, b0, b1, b2, b3, e);
  else
    staged_epilogue_impl<CHECKED, LB, false>(acc, b0, b1, b2, b3, e);
}

}  // namespace mao
