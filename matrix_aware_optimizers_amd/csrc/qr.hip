// Blocked Householder QR with explicit Q for the eigenbasis refresh
// ("SOAP, Muon, and Beyond", section 3-2 (4): per-step QR of the
// power-iteration product).
//
// Storage: the matrix P to factor is held column-major, i.e. as row-major S
// with S[j][i] = P[i][j], so every column of P -- and every Householder vector
// -- is a contiguous row. The explicit factor comes out the same way,
// E = Q^T row-major, plus an optional row-major copy of Q.
//
// Algorithm (right-looking, compact-WY blocks of kQrNB = 64 columns):
//   for each panel [j0, j0+nb):
//     1. panel kernel: Householder vectors of the panel columns (LAPACK's
//        convention: beta = -sign(alpha) ||x||, tau = (beta - alpha)/beta,
//        v = [1; x_tail / (alpha - beta)], tau = 0 when the tail is zero),
//        the triangular T of H_1 ... H_nb = I - V T V^T (from V^T V with
//        T[0:j, j] = -tau_j T[0:j, 0:j] V[:, 0:j]^T v_j), and the products
//        Zf = V T^T, Zo = V T;
//     2. trailing columns c: s_c <- s_c - Zf (V^T s_c) as two MFMA products
//        W = S_trail V^T, S_trail -= W Zf^T.
//   then Q = H_1 H_2 ... (backward accumulation from E = I, each block
//   e_c <- e_c - Zo (V^T e_c) on the rows / columns >= j0), and finally
//   column j of Q is multiplied by sign(beta_j) so that diag(R) >= 0.
//
// The panel kernel is a cooperative grid of ceil(len/256) workgroups; each
// owns 256 positions of the panel's columns in LDS, and the column-by-column
// dependency is carried by one grid barrier per column (partial sums of the
// tail norm and of the dot products with the remaining panel columns, summed
// by every workgroup in the same order). Barrier waits are bounded: on a time
// out the kernel raises a flag and stops waiting, so it always exits.
#include "qr.hpp"

#include "elementwise.hpp"
#include "gemm.hpp"

#include <algorithm>
#include <vector>

namespace mao {

namespace {

constexpr int NB = kQrNB;
constexpr int TPB = kQrThreads;
constexpr int LDX = TPB + 1;  // padded LDS row

struct PanelArgs {
  const float* S;
  int64_t ldS;
  int n, j0, nb;
  float* V;  // nb x len, ld ldV
  int64_t ldV;
  float* Zf;  // len x NB
  float* Zo;  // len x NB
  float* sign;
  float* part;  // 2 x G x 64
  float* dg;    // 2 x 64
  float* gram;  // G x 4096
  float* T;     // 4096
  unsigned* counter;
  int* err;
  const int* pred;
  const int* pred2;  // run only when *pred2 != 0 (the fast panel gave up)
};

__device__ void grid_barrier(unsigned* counter, unsigned target, int* err) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(counter, 1u);
    unsigned spins = 0;
    while (__hip_atomic_load(counter, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target) {
      if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
      if (++spins > (1u << 24)) {
        atomicExch(err, 1);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  __syncthreads();
  __threadfence();
}

// Up to kQrMaxJobs same-size panels per launch: job jb owns workgroups
// [jb G, (jb + 1) G); its barriers count only its own workgroups.
constexpr int kQrMaxJobs = 16;
struct PanelBatch {
  PanelArgs a[kQrMaxJobs];
  int njob;
};

__global__ __launch_bounds__(TPB) void qr_panel_kernel(PanelBatch B) {
  const int G = gridDim.x / B.njob, jb = blockIdx.x / G;
  const PanelArgs& a = B.a[jb];
  if (a.pred != nullptr && *a.pred == 0) return;
  if (a.pred2 != nullptr && *a.pred2 == 0) return;
  __shared__ float X[NB][LDX];
  __shared__ float red[NB][LDX];
  __shared__ float Tl[NB][NB + 1];
  __shared__ float qs[4][NB];
  __shared__ float tot[NB], dgv[NB], taus[NB], betas[NB];

  const int t = threadIdx.x, g = blockIdx.x - jb * G;
  const int n = a.n, j0 = a.j0, nb = a.nb;
  const int r = j0 + g * TPB + t;
  const bool valid = r < n;

  for (int k0 = 0; k0 < NB; k0 += 16) {
    float xv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      xv[u] = (valid && k0 + u < nb) ? a.S[(int64_t)(j0 + k0 + u) * a.ldS + r] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) X[k0 + u][t] = xv[u];
  }
  __syncthreads();

  unsigned bar = 0;
  for (int jj = 0; jj < nb; ++jj) {
    const int j = j0 + jj;
    const float xa = X[jj][t];
    const bool below = valid && r > j;
    const bool pivot = valid && r == j;
    for (int k = jj; k < nb; ++k) red[k][t] = below ? xa * X[k][t] : 0.f;
    float* dgb = a.dg + (jj & 1) * NB;
    if (pivot)
      for (int k = jj; k < nb; ++k) dgb[k] = X[k][t];
    __syncthreads();
    {
      const int v = t & 63, q = t >> 6;
      float s = 0.f;
      if (v >= jj && v < nb)
        for (int i = 0; i < 64; ++i) s += red[v][q * 64 + i];
      qs[q][v] = s;
    }
    __syncthreads();
    float* pb = a.part + (size_t)(jj & 1) * G * NB;
    if (t < NB) pb[g * NB + t] = qs[0][t] + qs[1][t] + qs[2][t] + qs[3][t];
    grid_barrier(a.counter, ++bar * (unsigned)G, a.err);
    {
      // every thread sums a quarter of the workgroups' partials of one value
      // (independent loads in flight together), then a fixed-order combine
      const int v = t & 63, q = t >> 6;
      float s = 0.f;
      if (v >= jj && v < nb) {
#pragma unroll 8
        for (int gg = q; gg < G; gg += 4) s += pb[gg * NB + v];
      }
      qs[q][v] = s;
      if (t < NB) dgv[t] = (t >= jj && t < nb) ? dgb[t] : 0.f;
    }
    __syncthreads();
    if (t < NB) tot[t] = qs[0][t] + qs[1][t] + qs[2][t] + qs[3][t];
    __syncthreads();
    const float alpha = dgv[jj], sig2 = tot[jj];
    float beta, tau, scal;
    if (sig2 == 0.f) {
      tau = 0.f;
      beta = alpha;
      scal = 0.f;
    } else {
      const float nrm = sqrtf(alpha * alpha + sig2);
      beta = alpha >= 0.f ? -nrm : nrm;
      tau = (beta - alpha) / beta;
      scal = 1.f / (alpha - beta);
    }
    for (int k = jj + 1; k < nb; ++k) {
      const float coef = tau * (dgv[k] + scal * tot[k]);
      if (below)
        X[k][t] -= coef * scal * xa;
      else if (pivot)
        X[k][t] -= coef;
    }
    X[jj][t] = below ? scal * xa : (pivot ? 1.f : 0.f);
    if (t == 0) {
      taus[jj] = tau;
      betas[jj] = beta;
    }
    __syncthreads();
  }

  // V panel out (nb x len)
  if (valid)
    for (int k = 0; k < nb; ++k) a.V[(int64_t)k * a.ldV + (r - j0)] = X[k][t];

  // partial Gram V^T V (strictly upper part)
  for (int e = t; e < NB * NB; e += TPB) {
    const int i = e >> 6, k = e & 63;
    float s = 0.f;
    if (i < k && k < nb)
      for (int u = 0; u < TPB; ++u) s += X[i][u] * X[k][u];
    a.gram[(size_t)g * NB * NB + e] = s;
  }
  grid_barrier(a.counter, ++bar * (unsigned)G, a.err);

  if (g == 0) {
    for (int e = t; e < NB * NB; e += TPB) {
      float s = 0.f;
      const int i = e >> 6, k = e & 63;
      if (i < k && k < nb) {
#pragma unroll 8
        for (int gg = 0; gg < G; ++gg) s += a.gram[(size_t)gg * NB * NB + e];
      }
      red[i][k] = s;
    }
    for (int e = t; e < NB * NB; e += TPB) {
      const int i = e >> 6, k = e & 63;
      Tl[i][k] = (i == k && i < nb) ? taus[i] : 0.f;
    }
    __syncthreads();
    for (int j = 1; j < nb; ++j) {
      if (t < j) {
        float s = 0.f;
        for (int l = t; l < j; ++l) s += Tl[t][l] * red[l][j];
        Tl[t][j] = -taus[j] * s;
      }
      __syncthreads();
    }
    for (int e = t; e < NB * NB; e += TPB) a.T[e] = Tl[e >> 6][e & 63];
    if (t < nb) a.sign[j0 + t] = betas[t] < 0.f ? -1.f : 1.f;
  }
  grid_barrier(a.counter, ++bar * (unsigned)G, a.err);

  for (int e = t; e < NB * NB; e += TPB) Tl[e >> 6][e & 63] = a.T[e];
  __syncthreads();
  if (valid) {
    float* zf = a.Zf + (int64_t)(r - j0) * NB;
    float* zo = a.Zo + (int64_t)(r - j0) * NB;
    float vr[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) vr[i] = (i < nb) ? X[i][t] : 0.f;
    for (int c = 0; c < NB; ++c) {
      float sf[4] = {0.f, 0.f, 0.f, 0.f}, so[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        sf[i & 3] = fmaf(vr[i], Tl[c][i], sf[i & 3]);
        so[i & 3] = fmaf(vr[i], Tl[i][c], so[i & 3]);
      }
      zf[c] = (sf[0] + sf[1]) + (sf[2] + sf[3]);
      zo[c] = (so[0] + so[1]) + (so[2] + so[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Fast panel: the same outputs (V, T, signs, V T^T, V T) from seven grid
// synchronisations instead of one per column.
//
// 1. Shifted CholeskyQR3 in fp64 arithmetic on the fp32 panel A (len x nb):
//    three passes of Gram G = Y^T Y (fp64 sums of exact fp64 products),
//    Cholesky G (+ s I on the first pass) = R^T R, Y <- Y R^{-1}; the first
//    pass's shift s = 11 (len nb + nb (nb+1)) 2^-53 tr(G) makes the
//    factorisation well defined for any numerically full-rank panel, the two
//    plain passes restore orthogonality. Q = the third pass's Y.
// 2. Householder representation rebuilt from Q: with D = diag(d), d = +-1,
//    the first nb columns of H = I - Y T Y^T equal Q D, so [I; 0] - Q D =
//    Y (T Y1^T) is an LU factorisation (Y unit lower trapezoidal, Y1 its top
//    block). It is computed without pivoting, choosing d_j = sign of the
//    eliminated diagonal entry of -Q1 so that every pivot is 1 + |.| >= 1;
//    then T = U Y1^{-T}, the rows of Y below the top block are -q D U^{-1},
//    and R~ = D R, so column j of Q gets the sign d_j.
// Any breakdown -- a zero or non-finite Cholesky pivot, or a third-pass Gram
// diagonal away from 1 -- is decided identically by every workgroup, which
// then all return; the per-column Householder panel runs instead (a flag).
constexpr int NU = NB * (NB + 1) / 2;   // packed upper-triangular entries
constexpr int LDG = NB + 2;             // fp64 LDS row: 16-byte aligned rows, 2 banks apart
constexpr int LDT = NB + 4;             // fp32 LDS row of T (16-byte aligned)

struct CholArgs {
  const float* S;
  int64_t ldS;
  int n, j0, nb;
  float* V;
  int64_t ldV;
  float* Zf;
  float* Zo;
  float* sign;
  float* T;        // 4096 floats: T, broadcast to every workgroup
  double* part;    // G x NU per-workgroup Gram partials
  double* gram;    // NU reduced Gram entries
  double* bcast;   // U (NB x NB) then d (NB)
  unsigned* counter;
  int* err;
  const int* pred;
  int* fail;       // set to 1 when the panel falls back to the Householder kernel
};

__device__ __forceinline__ int upk(int i, int k) { return i * NB - (i * (i - 1)) / 2 + (k - i); }

// Lane l's value of v, in every lane (l a compile-time constant here).
__device__ __forceinline__ double lane_d(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

struct CholBatch {
  CholArgs a[kQrMaxJobs];
  int njob;
};
static_assert(sizeof(CholBatch) <= 4096 && sizeof(PanelBatch) <= 4096, "kernel argument size");

__global__ __launch_bounds__(TPB) void qr_panel_chol_kernel(CholBatch B) {
  const int G = gridDim.x / B.njob, jb = blockIdx.x / G;
  const CholArgs& a = B.a[jb];
  if (a.pred != nullptr && *a.pred == 0) return;
  __shared__ float X[NB][LDX];      // current Y (fp32), later V
  __shared__ __attribute__((aligned(16))) double Gs[NB][LDG];  // Gram / LU work
  __shared__ __attribute__((aligned(16))) double Rt[NB][LDG];  // Cholesky factor R (row k = R[k][.]); later U
  __shared__ __attribute__((aligned(16))) float Tl[NB][LDT];
  __shared__ double dinv[NB];
  __shared__ float dsg[NB];
  __shared__ double red64[TPB];
  __shared__ int bad;

  const int t = threadIdx.x, g = blockIdx.x - jb * G;
  const int n = a.n, j0 = a.j0, nb = a.nb, len = n - j0;
  const int r = j0 + g * TPB + t;
  const bool valid = r < n;
  const int li = g * TPB + t;  // row of the panel

  for (int k0 = 0; k0 < NB; k0 += 16) {
    float xv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      xv[u] = (valid && k0 + u < nb) ? a.S[(int64_t)(j0 + k0 + u) * a.ldS + r] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) X[k0 + u][t] = xv[u];
  }
  if (t == 0) bad = 0;

  unsigned bar = 0;
  double y[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) y[k] = 0.0;

#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    __syncthreads();
    // ---- partial Gram of this workgroup's rows: 36 upper 8 x 8 blocks x 7 row chunks
    {
      double acc[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int w = 0; w < 8; ++w) acc[u][w] = 0.0;
      const int blk = t % 36, chunk = t / 36;
      int bi = 0, rem = blk;
      while (rem >= 8 - bi) {
        rem -= 8 - bi;
        ++bi;
      }
      const int bk = bi + rem;
      if (chunk < 7) {
        const int r0 = chunk * 37, r1 = min(TPB, r0 + 37);
        for (int q = r0; q < r1; ++q) {
          double va[8], vb[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            va[u] = (double)X[bi * 8 + u][q];
            vb[u] = (double)X[bk * 8 + u][q];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int w = 0; w < 8; ++w) acc[u][w] = fma(va[u], vb[w], acc[u][w]);
        }
      }
      for (int c = 0; c < 7; ++c) {
        __syncthreads();
        if (chunk == c) {
#pragma unroll
          for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
              const int i = bi * 8 + u, k = bk * 8 + w;
              if (i <= k) Gs[i][k] = (c == 0 ? 0.0 : Gs[i][k]) + acc[u][w];
            }
        }
      }
      __syncthreads();
      for (int idx = t; idx < NB * NB; idx += TPB) {
        const int i = idx / NB, k = idx % NB;
        if (i <= k) a.part[(size_t)g * NU + upk(i, k)] = Gs[i][k];
      }
    }
    grid_barrier(a.counter, ++bar * (unsigned)G, a.err);
    // ---- reduce the partials: workgroup g owns a contiguous range of entries;
    // `sub` threads share an entry, each summing every sub-th partial (loads
    // in flight together), then one of them adds the sub sums in order.
    {
      const int per = (NU + G - 1) / G;
      const int e0 = g * per, e1 = min(NU, e0 + per);
      const int sub = max(1, min(16, TPB / per));
      const int slots = (TPB / sub) * sub;
      for (int base = e0; base < e1; base += TPB / sub) {
        const int e = base + t / sub, q = t % sub;
        double sum = 0.0;
        if (t < slots && e < e1) {
          int gg = q;
          for (; gg + 3 * sub < G; gg += 4 * sub) {
            const double v0 = a.part[(size_t)gg * NU + e];
            const double v1 = a.part[(size_t)(gg + sub) * NU + e];
            const double v2 = a.part[(size_t)(gg + 2 * sub) * NU + e];
            const double v3 = a.part[(size_t)(gg + 3 * sub) * NU + e];
            sum += v0;
            sum += v1;
            sum += v2;
            sum += v3;
          }
          for (; gg < G; gg += sub) sum += a.part[(size_t)gg * NU + e];
        }
        __syncthreads();
        red64[t] = sum;
        __syncthreads();
        if (t < slots && q == 0 && e < e1) {
          double tot = 0.0;
          for (int u = 0; u < sub; ++u) tot += red64[t + u];
          a.gram[e] = tot;
        }
        __syncthreads();
      }
    }
    grid_barrier(a.counter, ++bar * (unsigned)G, a.err);
    // ---- Gram into LDS (symmetric), identity on the padded columns, shift
    {
      double gv[NB * NB / TPB];
#pragma unroll
      for (int u = 0; u < NB * NB / TPB; ++u) {
        const int idx = t + u * TPB, i = idx >> 6, k = idx & 63;
        gv[u] = (i < nb && k < nb) ? a.gram[i <= k ? upk(i, k) : upk(k, i)] : (i == k ? 1.0 : 0.0);
      }
#pragma unroll
      for (int u = 0; u < NB * NB / TPB; ++u) {
        const int idx = t + u * TPB;
        Gs[idx >> 6][idx & 63] = gv[u];
      }
    }
    __syncthreads();
    if (pass == 2) {
      // the second pass left Q nearly orthonormal: its Gram diagonal is ~1
      if (t < nb && !(fabs(Gs[t][t] - 1.0) < 1e-3)) bad = 1;
    }
    if (pass == 0 && t == 0) {
      double tr = 0.0;
      for (int k = 0; k < nb; ++k) tr += Gs[k][k];
      const double sh = 11.0 * ((double)len * nb + (double)nb * (nb + 1)) * 0x1p-53 * tr;
      for (int k = 0; k < nb; ++k) Gs[k][k] += sh;
    }
    // ---- Cholesky G = R^T R, row k of R into Rt[k][.], by the first
    // wavefront alone: lane j keeps column j of G in registers, the pivot
    // comes from lane k by readlane and row k of R goes round through LDS
    // (one wavefront's LDS accesses complete in order), so the 64 steps need
    // no workgroup barrier.
    __syncthreads();
    if (t < NB) {
      const int j = t;
      double gc[NB];
#pragma unroll
      for (int i = 0; i < NB; ++i) gc[i] = Gs[i][j];
      bool badl = false;
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const double piv = lane_d(gc[k], k);
        badl = badl || !(piv > 1e-300) || !(piv < 1e300);
        const double rkk = sqrt(fmax(piv, 1e-300));
        const double rkj = (j == k) ? rkk : gc[k] / rkk;
        if (j >= k) Rt[k][j] = rkj;
        dinv[j] = rkj;  // row k of R, shared (dinv is rewritten below)
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = k + 1; i < NB; ++i) gc[i] = fma(-dinv[i], rkj, gc[i]);
        // keep the updates at this step (the compiler would otherwise sink
        // each one to the step that reads it, keeping every R entry live)
#pragma unroll
        for (int i = k + 1; i < NB; ++i) asm volatile("" : "+v"(gc[i]));
        __builtin_amdgcn_wave_barrier();
      }
      dinv[j] = 1.0 / Rt[j][j];  // own write above
      if (j == 0 && badl) bad = 1;
    }
    __syncthreads();
    if (bad) {
      if (g == 0 && t == 0) *a.fail = 1;
      return;  // every workgroup decided alike
    }
    // ---- Y <- Y R^{-1} for this thread's row (forward substitution). Row
    // k + 1 of R is requested while row k is applied (rc / rn), and the
    // updates are pinned to their step, so the LDS latency is hidden.
#pragma unroll
    for (int k = 0; k < NB; ++k) y[k] = (double)X[k][t];
    {
      double rc[NB];
#pragma unroll
      for (int j = 1; j < NB; ++j) rc[j] = Rt[0][j];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        double rn[NB];
#pragma unroll
        for (int j = k + 2; j < NB; ++j) rn[j] = Rt[k + 1][j];
        y[k] *= dinv[k];
#pragma unroll
        for (int j = k + 1; j < NB; ++j) y[j] = fma(-y[k], rc[j], y[j]);
#pragma unroll
        for (int j = k + 1; j < NB; ++j) asm volatile("" : "+v"(y[j]));
#pragma unroll
        for (int j = k + 2; j < NB; ++j) rc[j] = rn[j];
      }
    }
    if (pass < 2) {
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NB; ++k) X[k][t] = (float)y[k];
    }
  }

  // ---- reconstruction: LU of -Q1 (top nb x nb block) with sign choice, T
  __syncthreads();
  if (g == 0) {
    // LU and T by the first wavefront. Lane i keeps row i of Z = -Q1 in
    // registers (zero outside nb x nb, which leaves the nb x nb factors
    // unchanged); the pivot row comes from lane j by readlane and L
    // overwrites Z below the diagonal. Lane i then turns its row into U
    // (signs d_c) and solves its row of T = U L^{-T} in place, reading L[j][l]
    // from lane j. No workgroup barrier inside.
    if (t < NB) {
      const int i = t;
      double w[NB];
      double udiag = 1.0;
#pragma unroll
      for (int c = 0; c < NB; ++c) w[c] = (i < nb && c < nb) ? -y[c] : 0.0;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const double zjj = lane_d(w[j], j);
        const double dj = zjj >= 0.0 ? 1.0 : -1.0;
        const double ujj = 1.0 + dj * zjj;
        if (i == 0 && j < nb) {
          dsg[j] = (float)dj;
          Rt[j][j] = ujj;  // U diagonal (Rt reused for U, stored U[i][c] at Rt[i][c])
        }
        if (i == j) udiag = ujj;
        const double lij = (i > j) ? dj * w[j] / ujj : 0.0;  // L[i][j]
        if (i > j) w[j] = lij;
#pragma unroll
        for (int cc = j + 1; cc < NB; ++cc) w[cc] = fma(-lij, lane_d(w[cc], j), w[cc]);
#pragma unroll
        for (int cc = j + 1; cc < NB; ++cc) asm volatile("" : "+v"(w[cc]));
      }
      __builtin_amdgcn_wave_barrier();
      // L to Gs (rows of Y's top block), U (strictly upper) to Rt, U row in w
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        if (c < i) {
          Gs[i][c] = w[c];
        } else if (c == i) {
          w[c] = (i < nb) ? udiag : 0.0;
        } else {
          const double u = (c < nb) ? (double)dsg[c] * w[c] : 0.0;
          if (i < nb && c < nb) Rt[i][c] = u;
          w[c] = u;
        }
      }
      // t_ij = U_ij - sum_{i <= l < j} t_il L_jl, l ascending
#pragma unroll
      for (int l = 0; l < NB; ++l) {
        const double m = (l >= i) ? w[l] : 0.0;
#pragma unroll
        for (int j = l + 1; j < NB; ++j) w[j] = fma(-m, lane_d(w[l], j), w[j]);
#pragma unroll
        for (int j = l + 1; j < NB; ++j) asm volatile("" : "+v"(w[j]));
      }
#pragma unroll
      for (int j = 0; j < NB; ++j) a.T[i * NB + j] = (i < nb && j >= i && j < nb) ? (float)w[j] : 0.f;
    }
    __syncthreads();
    for (int e = t; e < nb * nb; e += TPB) {
      const int i = e / nb, c = e % nb;
      a.bcast[i * NB + c] = (i <= c) ? Rt[i][c] : 0.0;
    }
    if (t < nb) {
      a.bcast[NB * NB + t] = (double)dsg[t];
      a.sign[j0 + t] = dsg[t];
    }
  }
  grid_barrier(a.counter, ++bar * (unsigned)G, a.err);
  if (g != 0) {
    for (int e = t; e < nb * nb; e += TPB) Rt[e / nb][e % nb] = a.bcast[(e / nb) * NB + e % nb];
    if (t < nb) dsg[t] = (float)a.bcast[NB * NB + t];
  }
  for (int e = t; e < NB * NB; e += TPB) Tl[e >> 6][e & 63] = a.T[e];
  if (t < NB) dinv[t] = (t < nb) ? 1.0 / Rt[t][t] : 1.0;  // U diagonal reciprocals
  __syncthreads();

  // ---- rows of Y: top block from L, the rest -q D U^{-1}
  if (li < nb) {
    for (int k = 0; k < NB; ++k) X[k][t] = (k < li) ? (float)Gs[li][k] : (k == li ? 1.f : 0.f);
  } else {
    double z[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) z[k] = (k < nb) ? -(double)dsg[k] * y[k] : 0.0;
    // z <- z U^{-1}, with the same one-row-ahead requests as the solve
    // above; a last, narrower panel keeps the columns past nb at zero
    if (nb == NB) {
      double uc[NB];
#pragma unroll
      for (int j = 1; j < NB; ++j) uc[j] = Rt[0][j];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        double un[NB];
#pragma unroll
        for (int j = k + 2; j < NB; ++j) un[j] = Rt[k + 1][j];
        z[k] = z[k] * dinv[k];
#pragma unroll
        for (int j = k + 1; j < NB; ++j) z[j] = fma(-z[k], uc[j], z[j]);
#pragma unroll
        for (int j = k + 1; j < NB; ++j) asm volatile("" : "+v"(z[j]));
#pragma unroll
        for (int j = k + 2; j < NB; ++j) uc[j] = un[j];
      }
    } else {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        if (k < nb) {
          z[k] = z[k] * dinv[k];
#pragma unroll
          for (int j = k + 1; j < NB; ++j)
            if (j < nb) z[j] = fma(-z[k], Rt[k][j], z[j]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) X[k][t] = valid ? (float)z[k] : 0.f;
  }
  // T^T beside T (in the fp64 Gram space, free once every row of Y is
  // built), so that both products read 16-byte rows
  __syncthreads();
  float* Tt = (float*)&Gs[0][0];
  for (int e = t; e < NB * NB; e += TPB) Tt[(e & 63) * LDT + (e >> 6)] = Tl[e >> 6][e & 63];
  __syncthreads();
  if (valid) {
    for (int k = 0; k < nb; ++k) a.V[(int64_t)k * a.ldV + li] = X[k][t];
    float* zf = a.Zf + (int64_t)li * NB;
    float* zo = a.Zo + (int64_t)li * NB;
    float vr[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) vr[i] = (i < nb) ? X[i][t] : 0.f;
    for (int c = 0; c < NB; ++c) {
      float sf[4] = {0.f, 0.f, 0.f, 0.f}, so[4] = {0.f, 0.f, 0.f, 0.f};
      const float4* tf = (const float4*)&Tl[c][0];
      const float4* to = (const float4*)&Tt[c * LDT];
#pragma unroll
      for (int i4 = 0; i4 < NB / 4; ++i4) {
        const float4 f = tf[i4], o = to[i4];
        sf[0] = fmaf(vr[4 * i4 + 0], f.x, sf[0]);
        sf[1] = fmaf(vr[4 * i4 + 1], f.y, sf[1]);
        sf[2] = fmaf(vr[4 * i4 + 2], f.z, sf[2]);
        sf[3] = fmaf(vr[4 * i4 + 3], f.w, sf[3]);
        so[0] = fmaf(vr[4 * i4 + 0], o.x, so[0]);
        so[1] = fmaf(vr[4 * i4 + 1], o.y, so[1]);
        so[2] = fmaf(vr[4 * i4 + 2], o.z, so[2]);
        so[3] = fmaf(vr[4 * i4 + 3], o.w, so[3]);
      }
      zf[c] = (sf[0] + sf[1]) + (sf[2] + sf[3]);
      zo[c] = (so[0] + so[1]) + (so[2] + so[3]);
    }
  }
}

__global__ void zero_u32_kernel(unsigned* p, int n, int* err) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
  if (threadIdx.x == 0) *err = 0;
}

// Skinny products W = A B^T (M x nb, K long -- the V^T projections of the
// trailing matrix and of E) have too few output tiles to occupy the chip, so
// K is cut into up to KSPLIT chunks (one grouped launch, partial products into
// `parts`) and the partials are summed in a fixed order.
constexpr int KSPLIT = 4;

__global__ __launch_bounds__(256) void sum_parts_kernel(float* out, const float* parts,
                                                        int64_t part_stride, int nparts,
                                                        int64_t count, int64_t job_stride,
                                                        const int* pred, int64_t spred) {
  const int jb = blockIdx.y;
  if (pred != nullptr && pred[jb * spred] == 0) return;
  out += jb * job_stride;
  parts += jb * job_stride;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256) {
    float s = parts[i];
    for (int q = 1; q < nparts; ++q) s += parts[q * part_stride + i];
    out[i] = s;
  }
}

// W_j = A_j B_j^T for njob jobs at strides sA, sB (elements); W and its split-K
// partials at stride sW per job.
mao_status skinny_product(int M, int nb, int K, const float* A, int64_t lda, int64_t sA,
                          const float* B, int64_t ldb, int64_t sB, float* W, float* parts,
                          int64_t sW, int njob, const int* pred, int64_t spred,
                          hipStream_t stream) {
  const int chunk = (int)round_up((K + KSPLIT - 1) / KSPLIT, 64);
  const int nparts = (K + chunk - 1) / chunk;
  if (nparts <= 1 || M < 1024) {
    GemmProblem p1 = gemm_problem(M, nb, K, 1.f, A, lda, B, ldb, 0.f, nullptr, 0, W, NB, GF_D_F32);
    p1.batch = njob;
    p1.sA = sA;
    p1.sB = sB;
    p1.sD = sW;
    p1.pred = pred;
    p1.spred = spred;
    return launch_gemm(MAO_F32, &p1, 1, stream, TAG_QR);
  }
  GemmProblem pr[KSPLIT];
  const int64_t stride = (int64_t)M * NB;
  for (int q = 0; q < nparts; ++q) {
    const int k0 = q * chunk, kc = std::min(chunk, K - k0);
    pr[q] = gemm_problem(M, nb, kc, 1.f, A + k0, lda, B + k0, ldb, 0.f, nullptr, 0,
                         parts + q * stride, NB, GF_D_F32);
    pr[q].batch = njob;
    pr[q].sA = sA;
    pr[q].sB = sB;
    pr[q].sD = sW;
    pr[q].pred = pred;
    pr[q].spred = spred;
  }
  MAO_TRY(launch_gemm(MAO_F32, pr, nparts, stream, TAG_QR));
  const int64_t count = (int64_t)M * NB;
  const int blocks = (int)std::min<int64_t>(1024, (count + 255) / 256);
  hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks, njob), dim3(256), 0, stream, W, parts, stride,
                     nparts, count, sW, pred, spred);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

int panels(int n) { return (n + NB - 1) / NB; }
int max_groups(int n) { return (n + TPB - 1) / TPB; }

int64_t vstore_floats(int n) {
  int64_t tot = 0;
  for (int p = 0; p < panels(n); ++p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    tot += round_up((int64_t)nb * round_up(len, 8), 64);
  }
  return tot;
}

int64_t zo_floats(int n) {
  int64_t tot = 0;
  for (int p = 0; p < panels(n); ++p) {
    const int len = n - p * NB;
    tot += round_up((int64_t)len * NB, 64);
  }
  return tot;
}

}  // namespace

QrWork carve_qr_work(Carver& c, int n) {
  QrWork w;
  const int G = max_groups(n);
  w.vstore = c.take<float>(vstore_floats(n));
  w.zo = c.take<float>(zo_floats(n));
  w.zf = c.take<float>((size_t)n * NB);
  w.wbuf = c.take<float>((size_t)n * NB);
  w.wparts = c.take<float>((size_t)KSPLIT * n * NB);
  w.sign = c.take<float>(n);
  w.part = c.take<float>((size_t)2 * G * NB);
  w.dg = c.take<float>(2 * NB);
  w.gram = c.take<float>((size_t)G * NB * NB);
  w.T = c.take<float>(NB * NB);
  w.counters = c.take<unsigned>(2 * panels(n));
  w.err = c.take<int>(1);
  w.fail = c.take<int>(panels(n));
  w.part64 = c.take<double>((size_t)G * NU);
  w.gram64 = c.take<double>(NU);
  w.bcast = c.take<double>(NB * NB + NB);
  return w;
}

size_t qr_work_bytes(int n) {
  Carver c(nullptr);
  carve_qr_work(c, n);
  return c.used + 256;
}

size_t qr_work_stride(int n) { return align_up(qr_work_bytes(n), 256); }

namespace {

// Jobs whose panel grids fit on the device together (one workgroup per CU
// for the panel kernels' LDS footprint), capped by the launch table.
int jobs_per_launch(int G) {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, b1 = 0, b2 = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b1, qr_panel_chol_kernel, TPB, 0) != hipSuccess) b1 = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b2, qr_panel_kernel, TPB, 0) != hipSuccess) b2 = 1;
    cached[dev] = std::max(1, cus * std::max(1, std::min(b1, b2)));
  }
  return std::max(1, std::min(kQrMaxJobs, cached[dev] / std::max(G, 1)));
}

}  // namespace

mao_status qr_core_batched(const QrBatch& b, hipStream_t stream) {
  const int n = b.n, nj = b.njob;
  if (nj <= 0) return MAO_OK;
  const int np = panels(n);
  const size_t wst = qr_work_stride(n);
  const int64_t wsf = (int64_t)(wst / sizeof(float));  // job stride of work, in floats
  std::vector<QrWork> w(nj);
  for (int j = 0; j < nj; ++j) {
    Carver c(b.work + (size_t)j * wst);
    w[j] = carve_qr_work(c, n);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, w[j].counters, 2 * np, w[j].err);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, (unsigned*)w[j].fail, np, w[j].err);
  }
  MAO_LAUNCH_CHECK();
  auto job_pred = [&](int j) -> const int* { return b.pred ? b.pred + j * b.spred : nullptr; };

  // offsets of the packed panels (the same in every job's workspace)
  int64_t voff = 0, zoff = 0;
  std::vector<int64_t> vo(np), zo(np);
  for (int p = 0; p < np; ++p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    vo[p] = voff;
    zo[p] = zoff;
    voff += round_up((int64_t)nb * round_up(len, 8), 64);
    zoff += round_up((int64_t)len * NB, 64);
  }

  const int G = max_groups(n);
  const int per = jobs_per_launch(G);
  for (int p = 0; p < np; ++p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    const int Gp = (len + TPB - 1) / TPB;
    for (int c0 = 0; c0 < nj; c0 += per) {
      const int cn = std::min(per, nj - c0);
      CholBatch cb;
      PanelBatch pb;
      cb.njob = pb.njob = cn;
      for (int q = 0; q < cn; ++q) {
        const int j = c0 + q;
        QrWork& wj = w[j];
        PanelArgs& a = pb.a[q];
        a.S = b.S + j * b.sS;
        a.ldS = b.ldS;
        a.n = n;
        a.j0 = j0;
        a.nb = nb;
        a.V = wj.vstore + vo[p];
        a.ldV = round_up(len, 8);
        a.Zf = wj.zf;
        a.Zo = wj.zo + zo[p];
        a.sign = wj.sign;
        a.part = wj.part;
        a.dg = wj.dg;
        a.gram = wj.gram;
        a.T = wj.T;
        a.counter = wj.counters + p;
        a.err = wj.err;
        a.pred = job_pred(j);
        a.pred2 = wj.fail + p;
        CholArgs& ca = cb.a[q];
        ca.S = a.S;
        ca.ldS = a.ldS;
        ca.n = n;
        ca.j0 = j0;
        ca.nb = nb;
        ca.V = a.V;
        ca.ldV = a.ldV;
        ca.Zf = a.Zf;
        ca.Zo = a.Zo;
        ca.sign = wj.sign;
        ca.T = wj.T;
        ca.part = wj.part64;
        ca.gram = wj.gram64;
        ca.bcast = wj.bcast;
        ca.counter = wj.counters + np + p;
        ca.err = wj.err;
        ca.pred = a.pred;
        ca.fail = wj.fail + p;
      }
      void* cargs[] = {&cb};
      MAO_HIP_CHECK(hipLaunchCooperativeKernel((const void*)qr_panel_chol_kernel, dim3(Gp * cn),
                                               dim3(TPB), cargs, 0, stream));
      void* kargs[] = {&pb};
      MAO_HIP_CHECK(hipLaunchCooperativeKernel((const void*)qr_panel_kernel, dim3(Gp * cn),
                                               dim3(TPB), kargs, 0, stream));
    }
    const int mt = n - j0 - nb;
    if (mt > 0) {
      float* Strail = b.S + (int64_t)(j0 + nb) * b.ldS + j0;
      // W = S_trail V^T   (mt x nb)
      MAO_TRY(skinny_product(mt, nb, len, Strail, b.ldS, b.sS, w[0].vstore + vo[p], round_up(len, 8),
                             wsf, w[0].wbuf, w[0].wparts, wsf, nj, b.pred, b.spred, stream));
      // S_trail -= W Zf^T  (mt x len)
      GemmProblem p2 = gemm_problem(mt, len, nb, -1.f, w[0].wbuf, NB, w[0].zf, NB, 1.f, Strail,
                                    b.ldS, Strail, b.ldS, GF_D_F32 | GF_C0_F32);
      p2.batch = nj;
      p2.sA = p2.sB = wsf;
      p2.sC0 = p2.sD = b.sS;
      p2.pred = b.pred;
      p2.spred = b.spred;
      MAO_TRY(launch_gemm(MAO_F32, &p2, 1, stream, TAG_QR));
    }
  }

  // explicit Q: E = Q^T, backward accumulation
  for (int j = 0; j < nj; ++j)
    MAO_TRY(fill_identity(view(b.E + j * b.sE, b.ldE), n, job_pred(j), stream));
  for (int p = np - 1; p >= 0; --p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    float* Esub = b.E + (int64_t)j0 * b.ldE + j0;
    MAO_TRY(skinny_product(len, nb, len, Esub, b.ldE, b.sE, w[0].vstore + vo[p], round_up(len, 8),
                           wsf, w[0].wbuf, w[0].wparts, wsf, nj, b.pred, b.spred, stream));
    GemmProblem p2 = gemm_problem(len, len, nb, -1.f, w[0].wbuf, NB, w[0].zo + zo[p], NB, 1.f,
                                  Esub, b.ldE, Esub, b.ldE, GF_D_F32 | GF_C0_F32);
    p2.batch = nj;
    p2.sA = p2.sB = wsf;
    p2.sC0 = p2.sD = b.sE;
    p2.pred = b.pred;
    p2.spred = b.spred;
    if (p != 0) {
      MAO_TRY(launch_gemm(MAO_F32, &p2, 1, stream, TAG_QR));
      continue;
    }
    // last block: column signs, and each job's Q written as the transposed copy
    p2.row_scale = w[0].sign;
    p2.srs = wsf;
    bool anyq = false;
    for (int j = 0; j < nj; ++j) anyq = anyq || (b.Q && b.Q[j]);
    if (!anyq) {
      MAO_TRY(launch_gemm(MAO_F32, &p2, 1, stream, TAG_QR));
      continue;
    }
    for (int c0 = 0; c0 < nj; c0 += kMaxProblems) {
      const int cn = std::min(kMaxProblems, nj - c0);
      GemmProblem pq[kMaxProblems];
      for (int q = 0; q < cn; ++q) {
        const int j = c0 + q;
        pq[q] = p2;
        pq[q].batch = 1;
        pq[q].A = w[j].wbuf;
        pq[q].B = w[j].zo + zo[p];
        pq[q].C0 = pq[q].D = Esub + j * b.sE;
        pq[q].row_scale = w[j].sign;
        pq[q].pred = job_pred(j);
        pq[q].spred = 0;
        if (b.Q && b.Q[j]) {
          pq[q].Dt = b.Q[j];
          pq[q].lddt = b.ldQ[j];
        }
      }
      MAO_TRY(launch_gemm(MAO_F32, pq, cn, stream, TAG_QR));
    }
  }
  return MAO_OK;
}

mao_status qr_core(float* S, int64_t ldS, int n, float* E, int64_t ldE, float* Qout, int64_t ldQ,
                   QrWork& w, const int* pred, hipStream_t stream) {
  QrBatch b;
  b.n = n;
  b.njob = 1;
  b.S = S;
  b.ldS = ldS;
  b.E = E;
  b.ldE = ldE;
  float* qs[1] = {Qout};
  int64_t lq[1] = {ldQ};
  b.Q = qs;
  b.ldQ = lq;
  b.pred = pred;
  b.work = (char*)w.vstore;  // the first block carved by carve_qr_work
  return qr_core_batched(b, stream);
}

}  // namespace mao
