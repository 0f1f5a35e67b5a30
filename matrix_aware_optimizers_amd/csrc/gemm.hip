// NT contraction on CDNA4 matrix cores.
//
// D[i][j] = alpha * sum_k A[i][k] * B[j][k] + beta * C0[i][j]
//
// Both operands are K-contiguous (row-major M x K and N x K), which is the
// layout every contraction of the optimizer steps is arranged into (the
// Newton-Schulz Grams X X^T and A A, the product B X through the transposed
// copy of X that the previous product writes, and the SOAP / FOAM rotations
// through transposed copies of the bases). One launch covers up to
// kMaxProblems problems, each a strided batch, so a whole layer's (or a whole
// expert bank's) Newton-Schulz stage is one dispatch.
//
// Tiling: 256 threads = 4 wavefronts in 2 x 2; a workgroup tile is BM x BN,
// each wavefront owns (BM/2) x (BN/2) as 32 x 32 MFMA blocks. A K-slice of the
// tile is 128 bytes per row (64 bf16 or 32 fp32), staged global -> registers
// -> LDS with double buffering (the next slice is fetched into registers while
// the current one feeds the MFMAs). LDS rows are padded to 144 bytes so the
// 16-byte reads of 32 consecutive rows spread over the banks. Each lane reads
// one contiguous half of a row (64 bytes); the K order inside a slice is
// permuted consistently for both operands, which leaves the sum unchanged.
//
// Epilogue: alpha/beta blend with C0 (bf16 or fp32), optional row scale,
// store of D and/or its transpose Dt (bf16 or fp32). In SYRK mode only tiles
// on or below the diagonal run and each writes its mirror image too; the
// diagonal tiles write each off-diagonal pair once, so the result is exactly
// symmetric.
//
// Tile order: workgroups are dealt round-robin to the 8 XCDs, so consecutive
// block ids are remapped to consecutive tiles on the same XCD (its L2), and
// tiles are rastered in groups of 8 tile-rows so that neighbours share
// operand panels.
#include "gemm.hpp"

#include <algorithm>
#include <utility>

namespace mao {

namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;  // K bytes per tile row per slice
constexpr int kLdsRow = 144;    // padded LDS row stride (bytes)

template <typename T> struct InCfg;
template <> struct InCfg<bf16_t> { static constexpr int EPC = 8; };
template <> struct InCfg<float> { static constexpr int EPC = 4; };

template <typename T>
__device__ __forceinline__ uint4 load_chunk(const T* row, int k, int K) {
  constexpr int EPC = InCfg<T>::EPC;
  if (k + EPC <= K) return *(const uint4*)(row + k);
  union {
    uint4 v;
    T e[EPC];
  } u;
  u.v = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < EPC; ++i)
    if (k + i < K) u.e[i] = row[k + i];
  return u.v;
}

__device__ __forceinline__ float c0_at(const void* C0, bool f32, int64_t off) {
  return f32 ? ((const float*)C0)[off] : bf16_to_f32(((const bf16_t*)C0)[off]);
}

__device__ __forceinline__ void store_at(void* D, bool f32, int64_t off, float v) {
  if (f32)
    ((float*)D)[off] = v;
  else
    ((bf16_t*)D)[off] = f32_to_bf16(v);
}

template <typename TIn, int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_nt_kernel(GemmArgs args) {
  constexpr int EPC = InCfg<TIn>::EPC;
  constexpr int BK = kRowBytes / (int)sizeof(TIn);
  constexpr int CA = BM * 8 / kThreads;
  constexpr int CB = BN * 8 / kThreads;
  constexpr int FM = BM / 64, FN = BN / 64;
  constexpr int kStage = (BM + BN) * kLdsRow;
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kStage];

  // ---- which tile ------------------------------------------------------
  int pi, local;
  xcd_tile(args, blockIdx.x, pi, local);
  const GemmProblem& P = args.p[pi];
  const int b = local / P.tiles_per_batch;
  if (P.pred != nullptr && P.pred[b * P.spred] == 0) return;
  local -= b * P.tiles_per_batch;
  int tm, tn;
  const bool syrk = (P.flags & GF_SYRK) != 0;
  if (syrk) {
    tm = (int)((sqrtf(8.f * (float)local + 1.f) - 1.f) * 0.5f);
    while (tm > 0 && tm * (tm + 1) / 2 > local) --tm;
    while ((tm + 1) * (tm + 2) / 2 <= local) ++tm;
    tn = local - tm * (tm + 1) / 2;
  } else {
    constexpr int G = 8;
    const int per_group = G * P.tiles_n;
    const int grp = local / per_group;
    const int first_m = grp * G;
    const int gsz = min(G, P.tiles_m - first_m);
    const int in = local - grp * per_group;
    tm = first_m + in % gsz;
    tn = in / gsz;
  }
  const int m0 = tm * BM, n0 = tn * BN;
  const int M = P.M, N = P.N, K = P.K;
  const int dsz = (P.flags & GF_D_F32) ? 4 : 2, csz = (P.flags & GF_C0_F32) ? 4 : 2;
  const OpPtrs ops = problem_operands(P, b, (int)sizeof(TIn), csz, dsz);
  const TIn* A = (const TIn*)ops.A;
  const TIn* B = (const TIn*)ops.B;
  const int64_t lda = P.lda, ldb = P.ldb;

  // Two register sets in flight: while slice k is multiplied out of LDS, the
  // slices k+1 and k+2 are on their way from memory.
  uint4 ra0[CA], rb0[CB], ra1[CA], rb1[CB];
  auto gload = [&](uint4* ra, uint4* rb, int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int c = 0; c < CA; ++c) {
      const int q = threadIdx.x + c * kThreads;
      const int row = q >> 3, ch = q & 7;
      const int gm = m0 + row;
      ra[c] = (gm < M) ? load_chunk<TIn>(A + (int64_t)gm * lda, k0 + ch * EPC, K)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int q = threadIdx.x + c * kThreads;
      const int row = q >> 3, ch = q & 7;
      const int gn = n0 + row;
      rb[c] = (gn < N) ? load_chunk<TIn>(B + (int64_t)gn * ldb, k0 + ch * EPC, K)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](const uint4* ra, const uint4* rb, int stage) __attribute__((always_inline)) {
    unsigned char* base = lds + stage * kStage;
#pragma unroll
    for (int c = 0; c < CA; ++c) {
      const int q = threadIdx.x + c * kThreads;
      *(uint4*)(base + (q >> 3) * kLdsRow + (q & 7) * 16) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < CB; ++c) {
      const int q = threadIdx.x + c * kThreads;
      *(uint4*)(base + (BM + (q >> 3)) * kLdsRow + (q & 7) * 16) = rb[c];
    }
  };

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  auto compute = [&](int stage) {
    const unsigned char* base = lds + stage * kStage;
    const unsigned char* pa = base + (wm * (BM / 2) + r32) * kLdsRow + h * 64;
    const unsigned char* pb = base + (BM + wn * (BN / 2) + r32) * kLdsRow + h * 64;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = *(const uint4*)(pa + i * 32 * kLdsRow + c * 16);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[j] = *(const uint4*)(pb + j * 32 * kLdsRow + c * 16);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (sizeof(TIn) == 2) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, af[i]), __builtin_bit_cast(bf16x8_t, bfr[j]),
                acc[i][j], 0, 0, 0);
          } else {
            const uint32_t* a4 = (const uint32_t*)&af[i];
            const uint32_t* b4 = (const uint32_t*)&bfr[j];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                  __uint_as_float(a4[e]), __uint_as_float(b4[e]), acc[i][j], 0, 0, 0);
          }
        }
      }
    }
  };

  const int nk = (K + BK - 1) / BK;
  if (nk > 0) {
    gload(ra0, rb0, 0);
    if (nk > 1) gload(ra1, rb1, BK);
    lstore(ra0, rb0, 0);
    __syncthreads();
    // invariant at the top of iteration kt: LDS stage kt&1 holds slice kt,
    // set (kt&1 ? 0 : 1) holds slice kt+1 (in flight)
    for (int kt = 0; kt < nk; kt += 2) {
      if (kt + 2 < nk) gload(ra0, rb0, (kt + 2) * BK);
      compute(0);
      if (kt + 1 < nk) lstore(ra1, rb1, 1);
      __syncthreads();
      if (kt + 1 >= nk) break;
      if (kt + 3 < nk) gload(ra1, rb1, (kt + 3) * BK);
      compute(1);
      if (kt + 2 < nk) lstore(ra0, rb0, 0);
      __syncthreads();
    }
  }

  // ---- epilogue: one 64-row slab of the tile at a time through LDS --------
  const bool diag = syrk && (tm == tn);
  const bool d32 = (P.flags & GF_D_F32) != 0;
  const bool c32 = (P.flags & GF_C0_F32) != 0;
  void* D = ops.D;
  void* Tt = syrk ? D : ops.Dt;
  const int64_t ldt = syrk ? P.ldd : P.lddt;
  const void* C0 = ops.C0;
  const float alpha = P.alpha, beta = P.beta;
  const float* rs = P.row_scale ? P.row_scale + b * P.srs : nullptr;

  constexpr int SLD = BN + 1;  // padded slab row (floats)
  float* slab = (float*)lds;
  constexpr int CPR = BN / 4;         // 4-wide chunks per slab row
  constexpr int RPI = kThreads / CPR; // slab rows per pass of the block
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int sr = wm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        const int sc = wn * (BN / 2) + j * 32 + r32;
        slab[sr * SLD + sc] = acc[i][j][v];
      }
    __syncthreads();
    // direct: D[r][c] = alpha acc + beta C0, row-scaled; final values kept in LDS
    const int c4 = (threadIdx.x % CPR) * 4;
    const int gcol = n0 + c4;
    for (int sr = threadIdx.x / CPR; sr < 64; sr += RPI) {
      const int grow = m0 + (sr >> 5) * (BM / 2) + i * 32 + (sr & 31);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = alpha * slab[sr * SLD + c4 + e];
      if (grow < M) {
        const bool full = gcol + 3 < N;
        if (C0) {
          const int64_t off = (int64_t)grow * P.ldc0 + gcol;
          if (full && c32) {
            const float4 c = *(const float4*)((const float*)C0 + off);
            v[0] += beta * c.x; v[1] += beta * c.y; v[2] += beta * c.z; v[3] += beta * c.w;
          } else if (full) {
            const uint2 c = *(const uint2*)((const bf16_t*)C0 + off);
            v[0] += beta * bf16_to_f32((bf16_t)(c.x & 0xffff));
            v[1] += beta * bf16_to_f32((bf16_t)(c.x >> 16));
            v[2] += beta * bf16_to_f32((bf16_t)(c.y & 0xffff));
            v[3] += beta * bf16_to_f32((bf16_t)(c.y >> 16));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gcol + e < N) v[e] += beta * c0_at(C0, c32, off + e);
          }
        }
        if (rs) {
          const float sc = rs[grow];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= sc;
        }
        if (D) {
          const int64_t off = (int64_t)grow * P.ldd + gcol;
          if (full && !diag) {
            if (d32) {
              *(float4*)((float*)D + off) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              uint2 pk;
              pk.x = pack_bf16x2(v[0], v[1]);
              pk.y = pack_bf16x2(v[2], v[3]);
              *(uint2*)((bf16_t*)D + off) = pk;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (gcol + e < N && (!diag || grow >= gcol + e)) store_at(D, d32, off + e, v[e]);
          }
        }
      }
      if (Tt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) slab[sr * SLD + c4 + e] = v[e];
      }
    }
    if (Tt) {
      __syncthreads();
      // transposed: Tt[c][r .. r+3] from four consecutive slab rows
      const int sr4 = (threadIdx.x & 15) * 4;
      const int grow = m0 + (sr4 >> 5) * (BM / 2) + i * 32 + (sr4 & 31);
      for (int sc = threadIdx.x >> 4; sc < BN; sc += kThreads / 16) {
        const int gc = n0 + sc;
        if (gc >= N || grow >= M) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = slab[(sr4 + e) * SLD + sc];
        const int64_t off = (int64_t)gc * ldt + grow;
        if (!diag && grow + 3 < M) {
          if (d32) {
            *(float4*)((float*)Tt + off) = make_float4(v[0], v[1], v[2], v[3]);
          } else {
            uint2 pk;
            pk.x = pack_bf16x2(v[0], v[1]);
            pk.y = pack_bf16x2(v[2], v[3]);
            *(uint2*)((bf16_t*)Tt + off) = pk;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (grow + e < M && (!diag || grow + e > gc)) store_at(Tt, d32, off + e, v[e]);
        }
      }
    }
  }
}

template <typename TIn, int BM, int BN>
mao_status launch_cfg(GemmArgs& args, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_nt_kernel<TIn, BM, BN>), dim3(args.total_tiles), dim3(kThreads), 0,
                     stream, args);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

// Pointer-table fill: the pointers travel as kernel arguments, a chunk per
// launch (under 2 KB of arguments).
constexpr int kFillChunk = 240;
struct PtrFill {
  const void** dst;
  int n;
  const void* p[kFillChunk];
};

__global__ __launch_bounds__(256) void ptr_fill_kernel(PtrFill a) {
  for (int i = threadIdx.x; i < a.n; i += blockDim.x) a.dst[i] = a.p[i];
}

int count_tiles(GemmProblem* probs, int nprob, int bm) {
  int64_t total = 0;
  for (int i = 0; i < nprob; ++i) {
    GemmProblem& p = probs[i];
    if (p.M <= 0 || p.N <= 0 || p.batch <= 0) continue;
    const int64_t tmi = ceil_div(p.M, bm), tni = ceil_div(p.N, bm);
    total += (int64_t)p.batch * ((p.flags & GF_SYRK) ? tmi * (tmi + 1) / 2 : tmi * tni);
  }
  return (int)total;
}

}  // namespace

mao_status write_pointer_table(const void** dst, const void* const* src, int n, hipStream_t s) {
  for (int i = 0; i < n; i += kFillChunk) {
    PtrFill a;
    a.dst = dst + i;
    a.n = std::min(kFillChunk, n - i);
    for (int k = 0; k < a.n; ++k) a.p[k] = src[i + k];
    hipLaunchKernelGGL(ptr_fill_kernel, dim3(1), dim3(256), 0, s, a);
    MAO_LAUNCH_CHECK();
  }
  return MAO_OK;
}

mao_status launch_gemm(int in_dtype, GemmProblem* probs, int nprob, hipStream_t stream, int tag) {
  // contractions outside Newton-Schulz and the QR are timed apart by input
  // type, so that each is measured against its own peak
  if (tag == TAG_OTHER && in_dtype == MAO_BF16) tag = TAG_OTHER_BF16;
  if (nprob <= 0) return MAO_OK;
  if (nprob > kMaxProblems) {
    set_error("launch_gemm: %d problems > %d", nprob, kMaxProblems);
    return MAO_E_UNSUPPORTED;
  }
  // A K x N operand B is read only by the 256 x 256 bf16 kernel; a launch
  // takes one B layout for all its problems.
  int nkm = 0;
  for (int i = 0; i < nprob; ++i) nkm += (probs[i].flags & GF_B_KMAJOR) ? 1 : 0;
  if (nkm != 0) {
    bool ok = nkm == nprob && in_dtype == MAO_BF16;
    for (int i = 0; i < nprob; ++i) ok = ok && !(probs[i].flags & GF_SYRK);
    if (!ok) {
      set_error("launch_gemm: a K x N operand B needs bf16 inputs, no SYRK, and the same layout "
                "for every problem of the launch");
      return MAO_E_UNSUPPORTED;
    }
  }
  // Tiled operands are read only by the 256 x 256 bf16 kernel, all problems
  // of the launch alike; a tiled D there is written pad included, so it takes
  // no row scale and no separate transposed copy.
  int nt = 0, ntio = 0;
  for (int i = 0; i < nprob; ++i) {
    nt += (probs[i].flags & GF_T32) ? 1 : 0;
    ntio += ((probs[i].flags & (GF_D_T32 | GF_C0_T32)) || probs[i].dadd != 0.f) ? 1 : 0;
  }
  if (nt != 0 || ntio != 0) {
    bool ok = nt == nprob && in_dtype == MAO_BF16;
    for (int i = 0; i < nprob; ++i) {
      const GemmProblem& p = probs[i];
      ok = ok && !p.row_scale && !((p.flags & GF_D_T32) && p.Dt && !(p.flags & GF_SYRK));
      ok = ok && p.lda % 256 == 0 && p.ldb % 256 == 0;
      ok = ok && (!(p.flags & GF_D_T32) || p.ldd % 256 == 0) && (!(p.flags & GF_C0_T32) || p.ldc0 % 256 == 0);
    }
    if (!ok) {
      set_error("launch_gemm: tiled operands (and a diagonal term) need bf16 inputs, the same "
                "layout for every problem, padded widths that are multiples of 256, and no row "
                "scale or separate Dt with a tiled D");
      return MAO_E_UNSUPPORTED;
    }
  }
  // Pointer-table batches run on the direct and 128 / 64 kernels only, never
  // with tiled operands.
  int ntab = 0;
  for (int i = 0; i < nprob; ++i) ntab += probs[i].ptab ? 1 : 0;
  if (ntab != 0 && (nt != 0 || ntio != 0)) {
    set_error("launch_gemm: a pointer-table batch takes no tiled operands");
    return MAO_E_UNSUPPORTED;
  }
  // fp32 rank-k updates (k <= 64, the QR updates) stream their result once:
  // the 256 x 256 rank kernel moves it in whole rows.
  bool rank = in_dtype == MAO_F32 && nkm == 0 && ntab == 0;
  for (int i = 0; i < nprob; ++i) rank = rank && probs[i].K <= 64 && !(probs[i].flags & GF_SYRK);
  rank = rank && count_tiles(probs, nprob, 256) >= 16;
  // without a transposed copy the 128 x 128 rank kernel (two per CU) serves
  bool rank128 = rank;
  for (int i = 0; i < nprob; ++i) rank128 = rank128 && probs[i].Dt == nullptr;
  // Results at most 64 columns wide (the QR's skinny projections) keep 64 x 64
  // tiles however many there are: a 128-wide tile would compute half zeros.
  bool skinny = true;
  for (int i = 0; i < nprob; ++i) skinny = skinny && probs[i].N <= 64;
  const bool big = in_dtype == MAO_BF16 ? (nkm != 0 || nt != 0 || count_tiles(probs, nprob, 256) >= 128)
                                         : (!skinny && count_tiles(probs, nprob, 256) >= 128);
  const int bm = rank128 ? 128
                 : (rank || big) ? 256
                 : (!skinny && count_tiles(probs, nprob, 128) >= 512) ? 128 : 64;
  // Longest K first: the last tiles to start are the short ones.
  int order[kMaxProblems];
  for (int i = 0; i < nprob; ++i) order[i] = i;
  for (int i = 1; i < nprob; ++i)
    for (int j = i; j > 0 && probs[order[j]].K > probs[order[j - 1]].K; --j) std::swap(order[j], order[j - 1]);
  GemmArgs args = {};
  int n = 0, total = 0;
  for (int i = 0; i < nprob; ++i) {
    GemmProblem p = probs[order[i]];
    if (p.M <= 0 || p.N <= 0 || p.batch <= 0) continue;
    p.tiles_m = (int)ceil_div(p.M, bm);
    p.tiles_n = (int)ceil_div(p.N, bm);
    p.tiles_per_batch = (p.flags & GF_SYRK) ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
    p.tile_begin = total;
    total += p.batch * p.tiles_per_batch;
    args.p[n++] = p;
  }
  if (n == 0) return MAO_OK;
  args.nprob = n;
  args.total_tiles = total;
  void* ev = nullptr;
  const bool timed = timing_on();
  if (timed) timing_record_begin(stream, &ev);
  mao_status st;
  if (rank128)
    st = launch_gemm_f32_rank128(args, stream);
  else if (rank)
    st = launch_gemm_f32_rank(args, stream);
  else if (in_dtype == MAO_BF16)
    st = bm == 256 ? launch_gemm_bf16_direct(args, stream)
         : bm == 128 ? launch_cfg<bf16_t, 128, 128>(args, stream) : launch_cfg<bf16_t, 64, 64>(args, stream);
  else
    st = bm == 256 ? launch_gemm_f32_direct(args, stream)
         : bm == 128 ? launch_cfg<float, 128, 128>(args, stream) : launch_cfg<float, 64, 64>(args, stream);
  if (timed) {
    // a launch gated by a device-side flag may skip its jobs: its flops
    // (counted as if every job ran) are kept apart
    double flops = 0.0;
    bool gated = false;
    for (int i = 0; i < n; ++i) {
      const GemmProblem& p = args.p[i];
      const double mnk = (double)p.M * p.N * p.K * p.batch;
      flops += (p.flags & GF_SYRK) ? mnk : 2.0 * mnk;
      gated = gated || p.pred != nullptr;
    }
    timing_record_end(stream, ev, gated ? TAG_GATED : tag, flops);
  }
  return st;
}

}  // namespace mao
