// fp32 rank-k updates, k <= 64: D = alpha * A B^T + beta * C0 with A: M x k,
// B: N x k. These are the QR's trailing-matrix and explicit-Q updates
// (S -= W Zf^T, E -= W Zo^T), which stream the whole M x N result once per
// 64-column panel: the work is the C0 read and the D write, so the kernel is
// built around moving them in full rows.
//
// Workgroup tile 256 x 256, 4 wavefronts in 2 x 2, each 128 x 128 as 4 x 4
// blocks of v_mfma_f32_32x32x2f32. Both operand tiles (256 x k each) are
// loaded once into LDS (rows padded to 68 floats, so the 16-byte reads of 16
// consecutive rows hit distinct banks), zero-filled past k and past the
// matrix edge. Lane half h multiplies k = 32 h .. 32 h + 31 of both operands.
// The result leaves through the staged epilogue (epilogue.hpp), whose four
// 32-row bands reuse the two operand buffers.
#include "epilogue.hpp"
#include "gemm.hpp"

namespace mao {

namespace {

constexpr int TB = 256;
constexpr int KMAX = 64;
constexpr int LDK = KMAX + 4;

__device__ __forceinline__ float4 load_row4(const float* row, int k, int K) {
  if (k + 4 <= K) return *(const float4*)(row + k);
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (k + e < K) ? row[k + e] : 0.f;
  return make_float4(v[0], v[1], v[2], v[3]);
}

__global__ __launch_bounds__(256) void gemm_f32_rank_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) float As[TB * LDK];
  __shared__ __attribute__((aligned(16))) float Bs[TB * LDK];

  int pi, local;
  xcd_tile(args, blockIdx.x, pi, local);
  const GemmProblem& P = args.p[pi];
  const int b = local / P.tiles_per_batch;
  if (P.pred != nullptr && P.pred[b * P.spred] == 0) return;
  local -= b * P.tiles_per_batch;
  int tm, tn;
  {
    constexpr int G = 8;
    const int per_group = G * P.tiles_n;
    const int grp = local / per_group;
    const int first_m = grp * G;
    const int gsz = min(G, P.tiles_m - first_m);
    const int in = local - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
  }
  const int m0 = tm * TB, n0 = tn * TB;
  const int M = P.M, N = P.N, K = P.K;
  const float* A = (const float*)P.A + (int64_t)b * P.sA;
  const float* B = (const float*)P.B + (int64_t)b * P.sB;

  // operand tiles: thread -> chunk (t % 16) of rows t / 16 + 16 i
  {
    const int ch = (threadIdx.x & 15) * 4, r0 = threadIdx.x >> 4;
    float4 va[16], vb[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r0 + 16 * i;
      const int gm = m0 + row, gn = n0 + row;
      va[i] = gm < M ? load_row4(A + (int64_t)gm * P.lda, ch, K) : make_float4(0.f, 0.f, 0.f, 0.f);
      vb[i] = gn < N ? load_row4(B + (int64_t)gn * P.ldb, ch, K) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = r0 + 16 * i;
      *(float4*)&As[row * LDK + ch] = va[i];
      *(float4*)&Bs[row * LDK + ch] = vb[i];
    }
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const float* pa = As + (wm * 128 + r32) * LDK + 32 * h;
  const float* pb = Bs + (wn * 128 + r32) * LDK + 32 * h;
#pragma unroll 1
  for (int c = 0; c < 8; ++c) {
    if (4 * c >= K) break;  // both lane halves past k (uniform)
    float4 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const float4*)(pa + i * 32 * LDK + 4 * c);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j] = *(const float4*)(pb + j * 32 * LDK + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float av = e == 0 ? fa[i].x : e == 1 ? fa[i].y : e == 2 ? fa[i].z : fa[i].w;
          const float bv = e == 0 ? fb[j].x : e == 1 ? fb[j].y : e == 2 ? fb[j].z : fb[j].w;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[i][j], 0, 0, 0);
        }
  }
  __syncthreads();

  const bool d32 = (P.flags & GF_D_F32) != 0;
  const bool c32 = (P.flags & GF_C0_F32) != 0;
  const int dsz = d32 ? 4 : 2, csz = c32 ? 4 : 2;
  EpiArgs ea;
  ea.m0 = m0;
  ea.n0 = n0;
  ea.M = M;
  ea.N = N;
  ea.alpha = P.alpha;
  ea.beta = P.beta;
  ea.C0 = P.C0 ? (const void*)((const char*)P.C0 + (int64_t)b * P.sC0 * csz) : nullptr;
  ea.ldc0 = P.ldc0;
  ea.c32 = c32;
  ea.rs = P.row_scale ? P.row_scale + b * P.srs : nullptr;
  ea.D = P.D ? (void*)((char*)P.D + (int64_t)b * P.sD * dsz) : nullptr;
  ea.ldd = P.ldd;
  ea.d32 = d32;
  ea.Tt = P.Dt ? (void*)((char*)P.Dt + (int64_t)b * P.sDt * dsz) : nullptr;
  ea.ldt = P.lddt;
  ea.diag = false;
  float* b0 = As;
  float* b1 = As + 32 * TB;
  float* b2 = Bs;
  float* b3 = Bs + 32 * TB;
  if (m0 + TB <= M && n0 + TB <= N)
    staged_epilogue<false>(acc, b0, b1, b2, b3, ea);
  else
    staged_epilogue<true>(acc, b0, b1, b2, b3, ea);
}

// 128 x 128 tiles for the updates without a transposed copy: 70 KB of LDS,
// so two workgroups share a CU and one's MFMAs run under the other's memory
// traffic. Each lane requests its 64 C0 values before the operand tiles, so
// the C0 latency is paid under the tile loads and the MFMAs; the result is
// written straight from the accumulators (32 consecutive columns of a row
// per half-wavefront).
constexpr int TS = 128;

__global__ __launch_bounds__(256, 2) void gemm_f32_rank128_kernel(GemmArgs args) {
  __shared__ __attribute__((aligned(16))) float As[TS * LDK];
  __shared__ __attribute__((aligned(16))) float Bs[TS * LDK];

  int pi, local;
  xcd_tile(args, blockIdx.x, pi, local);
  const GemmProblem& P = args.p[pi];
  const int b = local / P.tiles_per_batch;
  if (P.pred != nullptr && P.pred[b * P.spred] == 0) return;
  local -= b * P.tiles_per_batch;
  int tm, tn;
  {
    constexpr int G = 8;
    const int per_group = G * P.tiles_n;
    const int grp = local / per_group;
    const int first_m = grp * G;
    const int gsz = min(G, P.tiles_m - first_m);
    const int in = local - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
  }
  const int m0 = tm * TS, n0 = tn * TS;
  const int M = P.M, N = P.N, K = P.K;
  const float* A = (const float*)P.A + (int64_t)b * P.sA;
  const float* B = (const float*)P.B + (int64_t)b * P.sB;
  const bool d32 = (P.flags & GF_D_F32) != 0;
  const bool c32 = (P.flags & GF_C0_F32) != 0;
  const int dsz = d32 ? 4 : 2, csz = c32 ? 4 : 2;
  const void* C0 = P.C0 ? (const void*)((const char*)P.C0 + (int64_t)b * P.sC0 * csz) : nullptr;
  void* D = P.D ? (void*)((char*)P.D + (int64_t)b * P.sD * dsz) : nullptr;
  const float* rs = P.row_scale ? P.row_scale + b * P.srs : nullptr;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;
  // element (i, j, v) of this lane: row m0 + 64 wm + 32 i + 8 (v / 4) + 4 h + v % 4,
  // column n0 + 64 wn + 32 j + r32
  float cv[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        cv[i][j][v] = (C0 && row < M && col < N) ? c0_load(C0, c32, (int64_t)row * P.ldc0 + col) : 0.f;
      }
    }

  {
    const int ch = (threadIdx.x & 15) * 4, r0 = threadIdx.x >> 4;
    float4 va[8], vb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i;
      const int gm = m0 + row, gn = n0 + row;
      va[i] = gm < M ? load_row4(A + (int64_t)gm * P.lda, ch, K) : make_float4(0.f, 0.f, 0.f, 0.f);
      vb[i] = gn < N ? load_row4(B + (int64_t)gn * P.ldb, ch, K) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = r0 + 16 * i;
      *(float4*)&As[row * LDK + ch] = va[i];
      *(float4*)&Bs[row * LDK + ch] = vb[i];
    }
  }
  __syncthreads();

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const float* pa = As + (wm * 64 + r32) * LDK + 32 * h;
  const float* pb = Bs + (wn * 64 + r32) * LDK + 32 * h;
#pragma unroll 1
  for (int c = 0; c < 8; ++c) {
    if (4 * c >= K) break;  // both lane halves past k (uniform)
    float4 fa[2], fb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) fa[i] = *(const float4*)(pa + i * 32 * LDK + 4 * c);
#pragma unroll
    for (int j = 0; j < 2; ++j) fb[j] = *(const float4*)(pb + j * 32 * LDK + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float av = e == 0 ? fa[i].x : e == 1 ? fa[i].y : e == 2 ? fa[i].z : fa[i].w;
          const float bv = e == 0 ? fb[j].x : e == 1 ? fb[j].y : e == 2 ? fb[j].z : fb[j].w;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc[i][j], 0, 0, 0);
        }
  }

  if (!D) return;
  const float alpha = P.alpha, beta = P.beta;
  if (d32 && m0 + TS <= M && n0 + TS <= N && P.ldd % 4 == 0) {
    // A full fp32 tile goes through LDS (rows 0-63 over As, 64-127 over Bs,
    // both free once the products are done) and leaves in 16-byte pieces: a
    // quarter of the store instructions of the per-element stores below, which
    // the CU's store drain paces. Same values, stored in a different order.
    __syncthreads();
    constexpr int LT = 132;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int lc = 64 * wn + 32 * j + r32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int lr = 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
          float x = alpha * acc[i][j][v] + (C0 ? beta * cv[i][j][v] : 0.f);
          if (rs) x *= rs[m0 + lr];
          float* dst = lr < 64 ? As + lr * LT + lc : Bs + (lr - 64) * LT + lc;
          *dst = x;
        }
      }
    __syncthreads();
    const int c4 = (threadIdx.x & 31) * 4;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int lr = it * 8 + (threadIdx.x >> 5);
      const float* src = lr < 64 ? As + lr * LT + c4 : Bs + (lr - 64) * LT + c4;
      *(float4*)((float*)D + (int64_t)(m0 + lr) * P.ldd + n0 + c4) = *(const float4*)src;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        if (row >= M || col >= N) continue;
        float x = alpha * acc[i][j][v] + (C0 ? beta * cv[i][j][v] : 0.f);
        if (rs) x *= rs[row];
        d_store(D, d32, (int64_t)row * P.ldd + col, x);
      }
    }
}

}  // namespace

mao_status launch_gemm_f32_rank128(GemmArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_f32_rank128_kernel, dim3(args.total_tiles), dim3(256), 0, stream, args);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status launch_gemm_f32_rank(GemmArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL(gemm_f32_rank_kernel, dim3(args.total_tiles), dim3(256), 0, stream, args);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

}  // namespace mao
