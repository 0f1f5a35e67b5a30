// NT contraction D = alpha * A B^T + beta * C0 on MFMA (gfx950), grouped over
// up to kMaxProblems problems (each a strided batch) in one launch.
#pragma once

#include "common.hpp"

namespace mao {

enum GemmFlags : int {
  GF_SYRK = 1,     // square symmetric result: lower-triangular tiles only, mirrored
  GF_D_F32 = 2,    // D / Dt stored fp32 (else bf16)
  GF_C0_F32 = 4,   // C0 stored fp32 (else bf16)
  GF_B_KMAJOR = 8, // B stored K x N (row-major, ldb >= N): D = alpha A B (bf16 only)
  // Tiled operands (tiled.hpp; bf16, 256 x 256 kernel only): A, and B in the
  // orientation GF_B_KMAJOR names, are tiled with lda / ldb their padded
  // widths; every tile, K included, lies inside the zero-padded storage.
  GF_T32 = 16,
  GF_D_T32 = 32,   // D (and the SYRK mirror) written tiled, ldd its padded width
  GF_C0_T32 = 64,  // C0 read tiled, ldc0 its padded width
};

constexpr int kMaxProblems = 8;

struct GemmProblem {
  const void* A;     // M x K, row-major, lda (elements of the input dtype)
  const void* B;     // N x K, row-major, ldb
  const void* C0;    // M x N or nullptr
  void* D;           // M x N or nullptr
  void* Dt;          // N x M (transposed copy of D) or nullptr
  const float* row_scale;  // D row i multiplied by row_scale[i] (or nullptr)
  const int* pred;   // skip the problem when *pred == 0 (or nullptr)
  // Pointer-table batch (or nullptr): entry b's A, B, C0, D, Dt are
  // ptab[5 b .. 5 b + 4] (device memory; a null C0 / D / Dt is absent), in
  // place of the base pointers and batch strides above.
  const void* const* ptab;
  int64_t srs, spred;  // batch strides of row_scale and pred (elements; 0: shared)
  int64_t lda, ldb, ldc0, ldd, lddt;
  int64_t sA, sB, sC0, sD, sDt;  // batch strides (elements)
  float alpha, beta;
  float dadd;        // added to D[i][i] (tiled launches only; 0 otherwise)
  int M, N, K, batch;
  int flags;
  // filled by the launcher
  int tiles_m, tiles_n, tiles_per_batch, tile_begin;
};

struct GemmArgs {
  GemmProblem p[kMaxProblems];
  int nprob;
  int total_tiles;
};

// Tile of workgroup `bid`: problem `pi`, tile `local` within it (batch-major).
// Workgroups reach the 8 XCDs round-robin (bid % 8). Each problem's tiles are
// cut into 8 contiguous runs, one per XCD, so that every XCD gets the same
// share of every problem (balanced when the problems of a launch differ in K)
// and a run of neighbouring tiles that share operand panels in its L2; an XCD
// walks its runs problem by problem. Run lengths follow the round-robin deal of
// the concatenated tile list, which makes the map a bijection onto the tiles.
__device__ __forceinline__ void xcd_tile(const GemmArgs& a, int bid, int& pi, int& local) {
  const int x = bid & 7;
  int idx = bid >> 3, off = 0;
  pi = 0;
  local = 0;
  for (int q = 0; q < a.nprob; ++q) {
    const int n = a.p[q].batch * a.p[q].tiles_per_batch;
    const int base = n >> 3, r = n & 7, o = off & 7;
    const int mine = base + ((((x - o) & 7) < r) ? 1 : 0);
    if (idx < mine) {
      int extra = 0;
      for (int xx = 0; xx < x; ++xx) extra += (((xx - o) & 7) < r) ? 1 : 0;
      pi = q;
      local = x * base + extra + idx;
      return;
    }
    idx -= mine;
    off += n;
  }
}

// Operands of batch entry b (byte pointers): from the problem's pointer table,
// else base + b * stride. isz / csz / dsz: element sizes of A and B, C0, D.
struct OpPtrs {
  const char* A;
  const char* B;
  const char* C0;
  char* D;
  char* Dt;
};
__device__ __forceinline__ OpPtrs problem_operands(const GemmProblem& P, int b, int isz, int csz,
                                                   int dsz) {
  OpPtrs o;
  if (P.ptab != nullptr) {
    const void* const* e = P.ptab + 5 * (int64_t)b;
    o.A = (const char*)e[0];
    o.B = (const char*)e[1];
    o.C0 = (const char*)e[2];
    o.D = (char*)e[3];
    o.Dt = (char*)e[4];
    return o;
  }
  o.A = (const char*)P.A + (int64_t)b * P.sA * isz;
  o.B = (const char*)P.B + (int64_t)b * P.sB * isz;
  o.C0 = P.C0 ? (const char*)P.C0 + (int64_t)b * P.sC0 * csz : nullptr;
  o.D = P.D ? (char*)P.D + (int64_t)b * P.sD * dsz : nullptr;
  o.Dt = P.Dt ? (char*)P.Dt + (int64_t)b * P.sDt * dsz : nullptr;
  return o;
}

// Writes n pointers (host values) to the device table dst, in launches of
// kernel arguments (no host-to-device copy, nothing allocated).
mao_status write_pointer_table(const void** dst, const void* const* src, int n, hipStream_t s);

// What a launch computes, for the optional event timing (instrumentation).
enum GemmTag : int { TAG_NS_GRAM = 0, TAG_NS_SQUARE = 1, TAG_NS_APPLY = 2, TAG_OTHER = 3,
                     TAG_QR = 4, TAG_OTHER_BF16 = 5, TAG_QR_PROJ = 6, TAG_QR_FUSED = 7,
                     TAG_QR_PANEL = 8, TAG_GATED = 9, TAG_ELEMWISE = 10, TAG_COUNT = 11 };

// Enqueue one grouped launch. in_dtype: MAO_BF16 or MAO_F32. All problems of
// a launch share the input dtype. Host-side shape checks are the caller's.
mao_status launch_gemm(int in_dtype, GemmProblem* probs, int nprob, hipStream_t stream,
                       int tag = TAG_OTHER);

// bf16 path for large problems: 256 x 256 tiles, operands streamed into a
// four-stage LDS ring (gemm_direct.hip). Same semantics as gemm_nt_kernel.
mao_status launch_gemm_bf16_direct(GemmArgs& args, hipStream_t stream);
// The same kernel on fp32 operands (N x K B only, row-major), 16 K elements
// per slice on v_mfma_f32_32x32x2f32.
mao_status launch_gemm_f32_direct(GemmArgs& args, hipStream_t stream);

// fp32 rank-k updates, k <= 64, 256 x 256 tiles (gemm_f32_rank.hip).
mao_status launch_gemm_f32_rank(GemmArgs& args, hipStream_t stream);
// The same with 128 x 128 tiles, two workgroups per CU; no transposed copy.
mao_status launch_gemm_f32_rank128(GemmArgs& args, hipStream_t stream);

// Instrumentation: when enabled, every contraction launch is bracketed by HIP
// events on its stream, with its algorithmic flop count (symmetric products
// at half cost), and the Muon step's memory-bound passes under
// TAG_ELEMWISE with their algorithmic bytes in place of flops. Off by
// default.
bool timing_on();
void timing_record_begin(hipStream_t s, void** start);
void timing_record_end(hipStream_t s, void* start, int tag, double flops);

// Convenience for a single problem.
inline GemmProblem gemm_problem(int M, int N, int K, float alpha, const void* A, int64_t lda,
                                const void* B, int64_t ldb, float beta, const void* C0,
                                int64_t ldc0, void* D, int64_t ldd, int flags) {
  GemmProblem p = {};
  p.A = A; p.B = B; p.C0 = C0; p.D = D; p.Dt = nullptr;
  p.row_scale = nullptr; p.pred = nullptr; p.ptab = nullptr;
  p.lda = lda; p.ldb = ldb; p.ldc0 = ldc0; p.ldd = ldd; p.lddt = 0;
  p.alpha = alpha; p.beta = beta;
  p.M = M; p.N = N; p.K = K; p.batch = 1;
  p.flags = flags;
  return p;
}

}  // namespace mao
