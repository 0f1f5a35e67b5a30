// Symmetric eigendecomposition by parallel block Jacobi: FOAM's refresh by a
// full eigendecomposition of its factor ("Factored One-sided Adam-Moment for
// Practical and Scalable SOAP" review, section 1: the basis is the
// eigenvectors of R, recomputed periodically; section 3 counts the
// eigendecompositions FOAM saves).
//
// The solver is warm-started: it diagonalises D = Q^T F Q, the factor in the
// current basis (which FOAM's refresh criterion has just computed), and
// rotates Q's columns, so a basis that is already close needs few sweeps.
//
// Layout: D is padded to kp = round_up(n, 128) (zero rows and columns, which
// no rotation ever mixes in) and cut into 64-wide blocks; the nblk = kp / 64
// blocks are paired round-robin (block 0 fixed, the others rotating), so one
// sweep is nblk - 1 rounds of nblk / 2 disjoint pairs. Per round:
//
//   pair kernel   one workgroup per pair loads the 128 x 128 subproblem
//                 D[I, I] (I = the pair's two blocks) into LDS and diagonalises
//                 it by cyclic Jacobi rotations (64 disjoint rotations per
//                 parallel step, 127 steps per inner sweep, until a sweep
//                 rotates nothing), accumulating the 128 x 128 orthogonal J
//                 with J^T D[I, I] J diagonal;
//   apply kernel  every off-diagonal pair block D[I_P, I_Q] <- J_P^T D[I_P, I_Q]
//                 J_Q (two 128 x 128 x 128 fp32 MFMA products in one
//                 workgroup, written with its mirror so D stays exactly
//                 symmetric) and every 128-row strip of Q: Q[:, I_P] <- Q[:, I_P]
//                 J_P.
//
// Each J leaves the pair kernel polished by one Newton-Schulz step J <- J (3I
// - J^T J) / 2 (the fp32 rotations that built it leave it off orthogonality
// by far more than rounding). After each sweep the off-diagonal ratio
// ||D - diag D||_F / ||D||_F is reduced on the device; a job whose sweep
// rotated nothing, whose ratio reached the fp32 floor 8 u sqrt(kp), or whose
// ratio a sweep no longer halved is marked converged and every later kernel
// of that job returns at once (no host synchronisation). Finally the eigenvalues
// (diag D) are sorted descending (ties by index) and Q's columns gathered in
// that order, also transposed into E.
//
// Rotation: for the pair (i, j) with a = D_ii, d = D_jj, b = D_ij, zeta =
// (d - a) / 2b, t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), c = 1 /
// sqrt(1 + t^2), s = c t; columns i, j become c x_i - s x_j and s x_i + c x_j,
// which zeroes D_ij and moves a, d to a - t b, d + t b. A pair is left alone
// when |b| <= max(4 u max_k |D_kk|, 4 u sqrt(|a d|)) over its subproblem
// (u = 2^-24): below that b is rounding.
#include "eigh.hpp"

#include "gemm.hpp"

#include <algorithm>
#include <cmath>

namespace mao {

namespace {

constexpr int EB = 64;     // block width
constexpr int PB = 128;    // pair (two blocks)
constexpr int LDX = 129;   // LDS row stride of 128 x 128 tiles (conflict-free columns)
constexpr int kInnerMaxSweeps = 4;  // inexact inner solves: the outer sweeps converge regardless
constexpr int kTableJobs = 16;

struct EW {
  char* base;
  int64_t stride;  // bytes between jobs
  int64_t offD, offQ, offJ, offPart, offCtrl, offIdx, offEv, offX2;
  int n, kp, ldp, nblk;
  const int* pred;
  int64_t spred;
  float* info;
};

struct JobP {
  float* D;
  float* Q;
  float* J;
  double* part;
  int* ctrl;  // [0] converged, [1] rotated this sweep, [2] sweeps run, [3] last ratio
  int* idx;
  float* ev;  // eigenvalues in sorted order
  float* X2;  // kp x ldp: the sorted basis transposed (E before its polish)
};

__device__ __forceinline__ JobP job_ptrs(const EW& w, int j) {
  char* b = w.base + (int64_t)j * w.stride;
  return JobP{(float*)(b + w.offD), (float*)(b + w.offQ), (float*)(b + w.offJ),
              (double*)(b + w.offPart), (int*)(b + w.offCtrl), (int*)(b + w.offIdx),
              (float*)(b + w.offEv), (float*)(b + w.offX2)};
}

__device__ __forceinline__ bool job_off(const EW& w, int j) {
  return w.pred != nullptr && w.pred[j * w.spred] == 0;
}

// block at position pos of round r (block 0 stays, the others rotate)
__device__ __forceinline__ int rr_block(int pos, int r, int nblk) {
  return pos == 0 ? 0 : 1 + (pos - 1 + r) % (nblk - 1);
}

// global index of local index x (0..127) of pair P in round r
struct PairMap {
  int b1, b2;
  __device__ __forceinline__ int g(int x) const { return x < EB ? b1 * EB + x : b2 * EB + (x - EB); }
};

__device__ __forceinline__ PairMap pair_map(int P, int r, int nblk) {
  return PairMap{rr_block(P, r, nblk), rr_block(nblk - 1 - P, r, nblk)};
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// ---------------------------------------------------------------------------
// init: D (symmetric part, padded), Q (padded with identity), control words
// ---------------------------------------------------------------------------

struct InitTable {
  const float* D[kTableJobs];
  int64_t ldD[kTableJobs];
  const float* Q[kTableJobs];
  int64_t ldQ[kTableJobs];
  int j0;
};

__global__ __launch_bounds__(256) void eigh_init_kernel(EW w, InitTable t) {
  const int q = blockIdx.y, j = t.j0 + q;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  __shared__ float a[64][65], bt[64][65];
  const int tiles = w.kp / 64;
  const int n = w.n;
  const float* D = t.D[q];
  const float* Q = t.Q[q];
  const int64_t ldD = t.ldD[q], ldQ = t.ldQ[q];
  if (blockIdx.x == 0 && threadIdx.x < 8) p.ctrl[threadIdx.x] = 0;
  for (int tile = blockIdx.x; tile < tiles * tiles; tile += gridDim.x) {
    const int r0 = (tile / tiles) * 64, c0 = (tile % tiles) * 64;
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int i = e >> 6, k = e & 63;
      const int r = r0 + i, c = c0 + k;
      a[i][k] = (r < n && c < n) ? D[(int64_t)r * ldD + c] : 0.f;
      // the mirrored tile, read row-wise: bt[i][k] = D[c0 + i][r0 + k]
      const int rr = c0 + i, cc = r0 + k;
      bt[i][k] = (rr < n && cc < n) ? D[(int64_t)rr * ldD + cc] : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int i = e >> 6, k = e & 63;
      const int r = r0 + i, c = c0 + k;
      p.D[(int64_t)r * w.ldp + c] = 0.5f * (a[i][k] + bt[k][i]);
      float qv;
      if (r < n && c < n)
        qv = Q[(int64_t)r * ldQ + c];
      else
        qv = (r == c) ? 1.f : 0.f;
      p.Q[(int64_t)r * w.ldp + c] = qv;
    }
  }
}

// ---------------------------------------------------------------------------
// 128 x 128 x 128 fp32 MFMA products out of LDS
// ---------------------------------------------------------------------------

// The waves of a workgroup tile the 128 x 128 result WM x WN; each wave owns
// (128 / WM) x (128 / WN) as TM x TN 32 x 32 MFMA blocks.
template <int WM, int WN>
struct MM {
  static constexpr int TM = 128 / WM / 32, TN = 128 / WN / 32;
  typedef f32x16_t Acc[TM][TN];

  // out[x][c] = sum_k a(k, x) B[k][c] with a(k, x) = A[x][k] (ROWS) or A[k][x]
  template <bool ROWS>
  static __device__ __forceinline__ void run(const float* A, const float* B, Acc& acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int h = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][jj][v] = 0.f;
#pragma unroll 4
    for (int kk = 0; kk < PB / 2; ++kk) {
      const int k = 2 * kk + h;
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int x = wm * (128 / WM) + i * 32 + r32;
        a[i] = ROWS ? A[x * LDX + k] : A[k * LDX + x];
      }
#pragma unroll
      for (int jj = 0; jj < TN; ++jj) b[jj] = B[k * LDX + wn * (128 / WN) + jj * 32 + r32];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
          acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[jj], acc[i][jj], 0, 0, 0);
    }
  }

  // element (row, col) held by accumulator register v of block (i, jj)
  static __device__ __forceinline__ void at(int i, int jj, int v, int& row, int& col) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave / WN, wn = wave % WN;
    row = wm * (128 / WM) + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    col = wn * (128 / WN) + jj * 32 + (lane & 31);
  }

  static __device__ __forceinline__ void to_lds(const Acc& acc, float* out) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN; ++jj)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          int row, col;
          at(i, jj, v, row, col);
          out[row * LDX + col] = acc[i][jj][v];
        }
  }
};

// a dense 128 x 128 block (ld 128) into LDS, 16-byte loads
template <int NT>
__device__ __forceinline__ void load_j(const float* Jsrc, float* dst) {
  for (int e = threadIdx.x; e < PB * PB / 4; e += NT) {
    const float4 v = *(const float4*)(Jsrc + 4 * e);
    float* d = dst + (e >> 5) * LDX + (e & 31) * 4;
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
  }
}

// ---------------------------------------------------------------------------
// pair kernel: diagonalise the 128 x 128 subproblem of each pair
// ---------------------------------------------------------------------------

constexpr int kPairThreads = 1024;  // 16 waves: LDS latency of the rotation steps hidden
typedef MM<4, 4> MMP;

__global__ __launch_bounds__(kPairThreads) void eigh_pair_kernel(EW w, int r) {
  const int j = blockIdx.y;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  if (p.ctrl[0] != 0) return;
  __shared__ float A[PB * LDX];
  __shared__ float Jm[PB * LDX];
  __shared__ int pi_[64], pj_[64];
  __shared__ float pc_[64], ps_[64], pt_[64];
  __shared__ int rot_flag;

  const int tid = threadIdx.x;
  const PairMap pm = pair_map(blockIdx.x, r, w.nblk);
  for (int e = tid; e < PB * PB / 4; e += kPairThreads) {
    const int x = e >> 5, y = (e & 31) * 4;
    const float4 v = *(const float4*)(p.D + (int64_t)pm.g(x) * w.ldp + pm.g(y));
    float* a = A + x * LDX + y;
    a[0] = v.x;
    a[1] = v.y;
    a[2] = v.z;
    a[3] = v.w;
    float* jr = Jm + x * LDX + y;
#pragma unroll
    for (int u = 0; u < 4; ++u) jr[u] = (x == y + u) ? 1.f : 0.f;
  }
  // Rounding that the fp32 products leave in an entry of D follows the
  // magnitudes in its rows and columns: a rotation is skipped below 4 u of
  // the subproblem's largest diagonal entry as well as below 4 u of
  // sqrt(|a d|).
  __shared__ float red[16];
  {
    __syncthreads();
    float v = tid < PB ? fabsf(A[tid * (LDX + 1)]) : 0.f;
    v = wave_max(v);
    if ((tid & 63) == 0) red[tid >> 6] = v;
    __syncthreads();
  }
  float scale = 0.f;
#pragma unroll
  for (int u = 0; u < kPairThreads / 64; ++u) scale = fmaxf(scale, red[u]);
  const float tau_abs = 4.f * 0x1p-24f * scale;
  // the quads (P, Q <= P) and J column pairs this thread updates, fixed for
  // every step (they name pair slots, not indices)
  constexpr int kQuads = 64 * 65 / 2;
  constexpr int kMyQuads = (kQuads + kPairThreads - 1) / kPairThreads;
  int myP[kMyQuads], myQ[kMyQuads];
#pragma unroll
  for (int u = 0; u < kMyQuads; ++u) {
    const int q = tid + u * kPairThreads;
    int P = -1, Q = 0;
    if (q < kQuads) {
      P = (int)((sqrtf(8.f * (float)q + 1.f) - 1.f) * 0.5f);
      while (P * (P + 1) / 2 > q) --P;
      while ((P + 1) * (P + 2) / 2 <= q) ++P;
      Q = q - P * (P + 1) / 2;
    }
    myP[u] = P;
    myQ[u] = Q;
  }
  const int jq = tid & 63;  // J column pair; rows (tid >> 6) + 16 i
  __syncthreads();

  bool rotated_any = false;
  for (int sw = 0; sw < kInnerMaxSweeps; ++sw) {
    if (tid == 0) rot_flag = 0;
    __syncthreads();
    for (int step = 0; step < PB - 1; ++step) {
      if (tid < 64) {
        const int q = tid;
        const int i = q == 0 ? 0 : 1 + (q - 1 + step) % (PB - 1);
        const int k = 1 + (PB - 2 - q + step) % (PB - 1);  // position 127 - q
        const float a = A[i * LDX + i], d = A[k * LDX + k], b = A[i * LDX + k];
        float c = 1.f, s = 0.f, t = 0.f;
        if (fabsf(b) > fmaxf(tau_abs, 0x1p-22f * sqrtf(fabsf(a * d)))) {
          const float zeta = (d - a) / (2.f * b);
          t = fabsf(zeta) > 1e15f ? 0.5f / zeta
                                  : copysignf(1.f, zeta) / (fabsf(zeta) + sqrtf(1.f + zeta * zeta));
          c = 1.f / sqrtf(1.f + t * t);
          s = c * t;
          rot_flag = 1;
        }
        pi_[q] = i;
        pj_[q] = k;
        pc_[q] = c;
        ps_[q] = s;
        pt_[q] = t;
      }
      __syncthreads();
      // D[I, I] <- R^T D R, one 2 x 2 quad of rows {i_P, j_P} x columns
      // {i_Q, j_Q} per (P, Q) with Q <= P, written with its mirror
#pragma unroll
      for (int u = 0; u < kMyQuads; ++u) {
        const int P = myP[u], Q = myQ[u];
        if (P < 0) continue;
        const int iP = pi_[P], jP = pj_[P];
        const float sP = ps_[P];
        if (P == Q) {
          if (sP != 0.f) {
            const float t = pt_[P];
            const float b = A[iP * LDX + jP];
            A[iP * LDX + iP] -= t * b;
            A[jP * LDX + jP] += t * b;
            A[iP * LDX + jP] = 0.f;
            A[jP * LDX + iP] = 0.f;
          }
          continue;
        }
        const float sQ = ps_[Q];
        if (sP == 0.f && sQ == 0.f) continue;
        const int iQ = pi_[Q], jQ = pj_[Q];
        const float cP = pc_[P], cQ = pc_[Q];
        const float m00 = A[iP * LDX + iQ], m01 = A[iP * LDX + jQ];
        const float m10 = A[jP * LDX + iQ], m11 = A[jP * LDX + jQ];
        const float l00 = cP * m00 - sP * m10, l01 = cP * m01 - sP * m11;
        const float l10 = sP * m00 + cP * m10, l11 = sP * m01 + cP * m11;
        const float n00 = cQ * l00 - sQ * l01, n01 = sQ * l00 + cQ * l01;
        const float n10 = cQ * l10 - sQ * l11, n11 = sQ * l10 + cQ * l11;
        A[iP * LDX + iQ] = n00;
        A[iP * LDX + jQ] = n01;
        A[jP * LDX + iQ] = n10;
        A[jP * LDX + jQ] = n11;
        A[iQ * LDX + iP] = n00;
        A[jQ * LDX + iP] = n01;
        A[iQ * LDX + jP] = n10;
        A[jQ * LDX + jP] = n11;
      }
      // J <- J R
      {
        const float sQ = ps_[jq];
        if (sQ != 0.f) {
          const float cQ = pc_[jq];
          const int iQ = pi_[jq], jQ = pj_[jq];
#pragma unroll
          for (int u0 = 0; u0 < PB; u0 += kPairThreads / 64) {
            const int u = u0 + (tid >> 6);
            const float x0 = Jm[u * LDX + iQ], x1 = Jm[u * LDX + jQ];
            Jm[u * LDX + iQ] = cQ * x0 - sQ * x1;
            Jm[u * LDX + jQ] = sQ * x0 + cQ * x1;
          }
        }
      }
      __syncthreads();
    }
    const int flag = rot_flag;
    __syncthreads();
    if (!flag) break;
    rotated_any = true;
  }
  if (rotated_any && tid == 0) atomicOr(p.ctrl + 1, 1);
  // J from hundreds of fp32 rotations drifts from orthogonality (each
  // rotation's rounding nudges the column norms the same way); one
  // Newton-Schulz step J <- J (3I - J^T J) / 2 squares that error away. The
  // rotated block in LDS belongs to the unpolished J, so the block is
  // recomputed from the original as J^T D[I, I] J with the polished J: every
  // part of D then moves by the same orthogonal map.
  MMP::Acc acc;
  MMP::run<false>(Jm, Jm, acc);  // J^T J
  __syncthreads();
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    int row, col;
    MMP::at(0, 0, v, row, col);
    A[row * LDX + col] = (row == col ? 1.5f : 0.f) - 0.5f * acc[0][0][v];
  }
  __syncthreads();
  MMP::run<true>(Jm, A, acc);  // J (3I - J^T J) / 2
  __syncthreads();
  float* Jout = p.J + (int64_t)blockIdx.x * PB * PB;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    int row, col;
    MMP::at(0, 0, v, row, col);
    Jout[row * PB + col] = acc[0][0][v];
    Jm[row * LDX + col] = acc[0][0][v];
  }
  for (int e = tid; e < PB * PB / 4; e += kPairThreads) {
    const int x = e >> 5, y = (e & 31) * 4;
    const float4 v = *(const float4*)(p.D + (int64_t)pm.g(x) * w.ldp + pm.g(y));
    float* a = A + x * LDX + y;
    a[0] = v.x;
    a[1] = v.y;
    a[2] = v.z;
    a[3] = v.w;
  }
  __syncthreads();
  MMP::run<false>(A, Jm, acc);  // D J (D symmetric)
  __syncthreads();
  MMP::to_lds(acc, A);
  __syncthreads();
  MMP::run<false>(Jm, A, acc);  // J^T D J
  __syncthreads();
  MMP::to_lds(acc, A);
  __syncthreads();
  for (int e = tid; e < PB * PB / 4; e += kPairThreads) {
    const int x = e >> 5, y = (e & 31) * 4;
    float4 v;
    v.x = 0.5f * (A[x * LDX + y] + A[y * LDX + x]);
    v.y = 0.5f * (A[x * LDX + y + 1] + A[(y + 1) * LDX + x]);
    v.z = 0.5f * (A[x * LDX + y + 2] + A[(y + 2) * LDX + x]);
    v.w = 0.5f * (A[x * LDX + y + 3] + A[(y + 3) * LDX + x]);
    *(float4*)(p.D + (int64_t)pm.g(x) * w.ldp + pm.g(y)) = v;
  }
}

// ---------------------------------------------------------------------------
// apply kernel: off-diagonal pair blocks of D, and strips of Q
// ---------------------------------------------------------------------------

constexpr int kApplyThreads = 512;
typedef MM<4, 2> MMA;

__global__ __launch_bounds__(kApplyThreads) void eigh_apply_kernel(EW w, int r) {
  const int j = blockIdx.y;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  if (p.ctrl[0] != 0) return;
  __shared__ float X[PB * LDX];
  __shared__ float Jb[PB * LDX];
  const int npairs = w.nblk / 2;
  const int nD = npairs * (npairs - 1) / 2;
  const int bid = blockIdx.x;
  const int64_t ldp = w.ldp;
  const int tid = threadIdx.x;
  MMA::Acc acc;
  if (bid < nD) {
    // (P, Qp) with P < Qp: bid = Qp (Qp - 1) / 2 + P
    int Qp = (int)((1.f + sqrtf(1.f + 8.f * (float)bid)) * 0.5f);
    while (Qp * (Qp - 1) / 2 > bid) --Qp;
    while ((Qp + 1) * Qp / 2 <= bid) ++Qp;
    const int P = bid - Qp * (Qp - 1) / 2;
    const PairMap mp = pair_map(P, r, w.nblk), mq = pair_map(Qp, r, w.nblk);
    // X[k][x] = D[I_Q k][I_P x] = D[I_P x][I_Q k] (D symmetric)
    for (int e = tid; e < PB * PB / 4; e += kApplyThreads) {
      const int k = e >> 5, x = (e & 31) * 4;
      const float4 v = *(const float4*)(p.D + (int64_t)mq.g(k) * ldp + mp.g(x));
      float* d = X + k * LDX + x;
      d[0] = v.x;
      d[1] = v.y;
      d[2] = v.z;
      d[3] = v.w;
    }
    load_j<kApplyThreads>(p.J + (int64_t)Qp * PB * PB, Jb);
    __syncthreads();
    MMA::run<false>(X, Jb, acc);  // T = D[I_P, I_Q] J_Q
    __syncthreads();
    MMA::to_lds(acc, X);
    load_j<kApplyThreads>(p.J + (int64_t)P * PB * PB, Jb);
    __syncthreads();
    MMA::run<false>(Jb, X, acc);  // J_P^T T
    __syncthreads();
    MMA::to_lds(acc, X);
    __syncthreads();
    for (int e = tid; e < PB * PB / 4; e += kApplyThreads) {
      const int x = e >> 5, c = (e & 31) * 4;
      const float* s0 = X + x * LDX + c;
      *(float4*)(p.D + (int64_t)mp.g(x) * ldp + mq.g(c)) = make_float4(s0[0], s0[1], s0[2], s0[3]);
    }
    for (int e = tid; e < PB * PB / 4; e += kApplyThreads) {
      const int c = e >> 5, x = (e & 31) * 4;
      *(float4*)(p.D + (int64_t)mq.g(c) * ldp + mp.g(x)) =
          make_float4(X[x * LDX + c], X[(x + 1) * LDX + c], X[(x + 2) * LDX + c],
                      X[(x + 3) * LDX + c]);
    }
  } else {
    const int b2 = bid - nD;
    const int ub = b2 / npairs, P = b2 % npairs;
    const int64_t u0 = (int64_t)ub * PB;
    const PairMap mp = pair_map(P, r, w.nblk);
    // X[k][x] = Q[u0 + x][I_P k]
    for (int e = tid; e < PB * PB / 4; e += kApplyThreads) {
      const int x = e >> 5, k = (e & 31) * 4;
      const float4 v = *(const float4*)(p.Q + (u0 + x) * ldp + mp.g(k));
      X[k * LDX + x] = v.x;
      X[(k + 1) * LDX + x] = v.y;
      X[(k + 2) * LDX + x] = v.z;
      X[(k + 3) * LDX + x] = v.w;
    }
    load_j<kApplyThreads>(p.J + (int64_t)P * PB * PB, Jb);
    __syncthreads();
    MMA::run<false>(X, Jb, acc);  // Q[strip, I_P] J_P
    __syncthreads();
    MMA::to_lds(acc, X);
    __syncthreads();
    for (int e = tid; e < PB * PB / 4; e += kApplyThreads) {
      const int x = e >> 5, c = (e & 31) * 4;
      const float* s0 = X + x * LDX + c;
      *(float4*)(p.Q + (u0 + x) * ldp + mp.g(c)) = make_float4(s0[0], s0[1], s0[2], s0[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// convergence: off-diagonal ratio after a sweep
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void eigh_conv_partial_kernel(EW w) {
  const int j = blockIdx.y;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  if (p.ctrl[0] != 0) return;
  __shared__ double red[8];
  const int rb = blockIdx.x;
  double off = 0.0, tot = 0.0;
  for (int e = threadIdx.x; e < 64 * w.kp; e += 256) {
    const int i = rb * 64 + e / w.kp, c = e % w.kp;
    const double v = (double)p.D[(int64_t)i * w.ldp + c];
    tot += v * v;
    if (i != c) off += v * v;
  }
  off = block_sum_d(off, red);
  tot = block_sum_d(tot, red);
  if (threadIdx.x == 0) {
    p.part[2 * rb] = off;
    p.part[2 * rb + 1] = tot;
  }
}

__global__ __launch_bounds__(64) void eigh_conv_final_kernel(EW w, int sweep) {
  const int j = blockIdx.x;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  float* info = w.info ? w.info + (int64_t)j * (kEighMaxSweeps + 1) : nullptr;
  if (p.ctrl[0] != 0) {
    if (info && threadIdx.x == 0) info[sweep] = 0.f;
    return;
  }
  const int nrb = w.kp / 64;
  double off = 0.0, tot = 0.0;
  for (int i = threadIdx.x; i < nrb; i += 64) {
    off += p.part[2 * i];
    tot += p.part[2 * i + 1];
  }
  off = wave_sum_d(off);
  tot = wave_sum_d(tot);
  if (threadIdx.x == 0) {
    const double rho = tot > 0.0 ? sqrt(off / tot) : 0.0;
    const bool rotated = p.ctrl[1] != 0;
    const float prev = __int_as_float(p.ctrl[3]);
    p.ctrl[2] = sweep + 1;
    // converged: nothing rotated, the ratio is at the fp32 floor
    // (8 u sqrt(kp)), or a sweep no longer halved it
    const double floor32 = 8.0 * 0x1p-24 * sqrt((double)w.kp);
    if (!rotated || rho <= floor32 || (sweep > 0 && rho > 0.5 * (double)prev)) p.ctrl[0] = 1;
    p.ctrl[1] = 0;
    p.ctrl[3] = __float_as_int((float)rho);
    if (info) {
      info[sweep] = (float)rho;
      info[kEighMaxSweeps] = (float)(sweep + 1);
    }
  }
}

// ---------------------------------------------------------------------------
// order: eigenvalues descending (ties by index), padding last
// ---------------------------------------------------------------------------

constexpr int kSortMax = 16384;

__global__ __launch_bounds__(1024) void eigh_sort_kernel(EW w) {
  const int j = blockIdx.x;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  __shared__ float key[kSortMax];
  __shared__ int ix[kSortMax];
  int N2 = 1;
  while (N2 < w.kp) N2 <<= 1;
  for (int i = threadIdx.x; i < N2; i += 1024) {
    key[i] = i < w.n ? p.D[(int64_t)i * w.ldp + i] : -INFINITY;
    ix[i] = i;
  }
  __syncthreads();
  // a precedes b: larger key, or equal keys and smaller index
  auto prec = [&](int a, int b) { return key[a] > key[b] || (key[a] == key[b] && ix[a] < ix[b]); };
  for (int k = 2; k <= N2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = threadIdx.x; i < N2; i += 1024) {
        const int l = i ^ jj;
        if (l > i) {
          const bool asc = (i & k) == 0;
          if (asc ? prec(l, i) : prec(i, l)) {
            const float tk = key[i];
            key[i] = key[l];
            key[l] = tk;
            const int ti = ix[i];
            ix[i] = ix[l];
            ix[l] = ti;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = threadIdx.x; i < w.n; i += 1024) {
    p.idx[i] = ix[i];
    p.ev[i] = key[i];
  }
}

// ---------------------------------------------------------------------------
// gather: Q_out[:, c] = Q[:, idx[c]], E_out = Q_out^T, eigenvalues
// ---------------------------------------------------------------------------

struct EvalTable {
  float* evals[kTableJobs];
  int j0;
};

// Qs = Q[:, idx] (row-major, into the D area, free once sorted) and Es =
// Qs^T (into X2); the sorted eigenvalues to the caller.
__global__ __launch_bounds__(256) void eigh_gather_kernel(EW w, EvalTable t) {
  const int q = blockIdx.y, j = t.j0 + q;
  if (job_off(w, j)) return;
  JobP p = job_ptrs(w, j);
  __shared__ float T[64][65];
  __shared__ int cols[64];
  const int n = w.n, tiles = (n + 63) / 64;
  float* ev = t.evals[q];
  for (int tile = blockIdx.x; tile < tiles * tiles; tile += gridDim.x) {
    const int r0 = (tile / tiles) * 64, c0 = (tile % tiles) * 64;
    __syncthreads();
    if (threadIdx.x < 64) cols[threadIdx.x] = c0 + threadIdx.x < n ? p.idx[c0 + threadIdx.x] : 0;
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int i = e >> 6, k = e & 63;
      const int r = r0 + i;
      T[i][k] = (r < n && c0 + k < n) ? p.Q[(int64_t)r * w.ldp + cols[k]] : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int i = e >> 6, k = e & 63;
      if (r0 + i < n && c0 + k < n) p.D[(int64_t)(r0 + i) * w.ldp + c0 + k] = T[i][k];
    }
    for (int e = threadIdx.x; e < 64 * 64; e += 256) {
      const int k = e >> 6, i = e & 63;
      if (r0 + i < n && c0 + k < n) p.X2[(int64_t)(c0 + k) * w.ldp + r0 + i] = T[i][k];
    }
    if (ev && r0 == 0 && threadIdx.x < 64 && c0 + threadIdx.x < n)
      ev[c0 + threadIdx.x] = p.ev[c0 + threadIdx.x];
  }
}

struct Offsets {
  int64_t D, Q, J, part, ctrl, idx, ev, X2, total;
};

Offsets eigh_offsets(int n) {
  const int64_t kp = round_up(n, PB), ldp = kp + 4;
  Carver c(nullptr);
  Offsets o;
  o.D = 0;
  c.take<float>((size_t)(kp * ldp));
  o.Q = (int64_t)align_up(c.used, 256);
  c.take<float>((size_t)(kp * ldp));
  o.J = (int64_t)align_up(c.used, 256);
  c.take<float>((size_t)(kp / 2 / EB) * PB * PB);
  o.part = (int64_t)align_up(c.used, 256);
  c.take<double>((size_t)(kp / EB) * 2);
  o.ctrl = (int64_t)align_up(c.used, 256);
  c.take<int>(8);
  o.idx = (int64_t)align_up(c.used, 256);
  c.take<int>((size_t)kp);
  o.ev = (int64_t)align_up(c.used, 256);
  c.take<float>((size_t)kp);
  o.X2 = (int64_t)align_up(c.used, 256);
  c.take<float>((size_t)(kp * ldp));
  o.total = (int64_t)c.used;
  return o;
}

}  // namespace

size_t eigh_work_stride(int n) { return align_up((size_t)eigh_offsets(n).total, 256); }

mao_status eigh_batched(const EighBatch& b, hipStream_t stream) {
  const int n = b.n, nj = b.njob;
  if (nj <= 0) return MAO_OK;
  if (n < 1 || n > kEighMaxN) {
    set_error("eigendecomposition of size %d outside 1..%d", n, kEighMaxN);
    return MAO_E_UNSUPPORTED;
  }
  const Offsets o = eigh_offsets(n);
  EW w;
  w.base = b.work;
  w.stride = (int64_t)eigh_work_stride(n);
  w.offD = o.D;
  w.offQ = o.Q;
  w.offJ = o.J;
  w.offPart = o.part;
  w.offCtrl = o.ctrl;
  w.offIdx = o.idx;
  w.offEv = o.ev;
  w.offX2 = o.X2;
  w.n = n;
  w.kp = (int)round_up(n, PB);
  w.ldp = w.kp + 4;
  w.nblk = w.kp / EB;
  w.pred = b.pred;
  w.spred = b.spred;
  w.info = b.info;

  const int ptiles = (w.kp / 64) * (w.kp / 64);
  for (int c0 = 0; c0 < nj; c0 += kTableJobs) {
    const int cn = std::min(kTableJobs, nj - c0);
    InitTable t;
    for (int q = 0; q < kTableJobs; ++q) {
      const bool has = q < cn;
      t.D[q] = has ? b.jobs[c0 + q].D : nullptr;
      t.ldD[q] = has ? b.jobs[c0 + q].ldD : 0;
      t.Q[q] = has ? b.jobs[c0 + q].Q : nullptr;
      t.ldQ[q] = has ? b.jobs[c0 + q].ldQ : 0;
    }
    t.j0 = c0;
    hipLaunchKernelGGL(eigh_init_kernel, dim3(std::min(ptiles, 1024), cn), dim3(256), 0, stream,
                       w, t);
    MAO_LAUNCH_CHECK();
  }
  const int npairs = w.nblk / 2;
  const int nD = npairs * (npairs - 1) / 2;
  const int nQ = (int)ceil_div(n, PB) * npairs;
  for (int sweep = 0; sweep < kEighMaxSweeps; ++sweep) {
    for (int r = 0; r < w.nblk - 1; ++r) {
      hipLaunchKernelGGL(eigh_pair_kernel, dim3(npairs, nj), dim3(kPairThreads), 0, stream, w, r);
      hipLaunchKernelGGL(eigh_apply_kernel, dim3(nD + nQ, nj), dim3(kApplyThreads), 0, stream, w,
                         r);
    }
    hipLaunchKernelGGL(eigh_conv_partial_kernel, dim3(w.kp / 64, nj), dim3(256), 0, stream, w);
    hipLaunchKernelGGL(eigh_conv_final_kernel, dim3(nj), dim3(64), 0, stream, w, sweep);
    MAO_LAUNCH_CHECK();
  }
  hipLaunchKernelGGL(eigh_sort_kernel, dim3(nj), dim3(1024), 0, stream, w);
  MAO_LAUNCH_CHECK();
  const int otiles = (int)(ceil_div(n, 64) * ceil_div(n, 64));
  for (int c0 = 0; c0 < nj; c0 += kTableJobs) {
    const int cn = std::min(kTableJobs, nj - c0);
    EvalTable t;
    for (int q = 0; q < kTableJobs; ++q) t.evals[q] = q < cn ? b.jobs[c0 + q].evals : nullptr;
    t.j0 = c0;
    hipLaunchKernelGGL(eigh_gather_kernel, dim3(std::min(otiles, 1024), cn), dim3(256), 0,
                       stream, w, t);
    MAO_LAUNCH_CHECK();
  }
  // Orthogonality polish of the sorted basis, one Newton-Schulz step on its
  // transpose Y = Qs^T (rows = eigenvectors): C = Y Y^T (= Qs^T Qs, into the
  // Q area), Y' = 1.5 Y - 0.5 C Y, written as E (D of the product) and as Q
  // (its transposed store). The product reads Qs as its N x K operand (rows
  // of Qs are columns of Y).
  const int64_t sf = w.stride / (int64_t)sizeof(float);
  float* base = (float*)b.work;
  float* Qs = base + o.D / (int64_t)sizeof(float);
  float* Cc = base + o.Q / (int64_t)sizeof(float);
  float* Es = base + o.X2 / (int64_t)sizeof(float);
  GemmProblem sy = gemm_problem(n, n, n, 1.f, Es, w.ldp, Es, w.ldp, 0.f, nullptr, 0, Cc, w.ldp,
                                GF_SYRK | GF_D_F32);
  sy.batch = nj;
  sy.sA = sy.sB = sy.sD = sf;
  sy.pred = b.pred;
  sy.spred = b.spred;
  MAO_TRY(launch_gemm(MAO_F32, &sy, 1, stream));
  for (int c0 = 0; c0 < nj; c0 += kMaxProblems) {
    const int cn = std::min(kMaxProblems, nj - c0);
    GemmProblem pr[kMaxProblems];
    for (int q = 0; q < cn; ++q) {
      const int j = c0 + q;
      const EighJob& jb = b.jobs[j];
      pr[q] = gemm_problem(n, n, n, -0.5f, Cc + j * sf, w.ldp, Qs + j * sf, w.ldp, 1.5f,
                           Es + j * sf, w.ldp, jb.E, jb.ldE, GF_D_F32 | GF_C0_F32);
      pr[q].Dt = jb.Q;
      pr[q].lddt = jb.ldQ;
      pr[q].pred = b.pred ? b.pred + j * b.spred : nullptr;
    }
    MAO_TRY(launch_gemm(MAO_F32, pr, cn, stream));
  }
  return MAO_OK;
}

}  // namespace mao
