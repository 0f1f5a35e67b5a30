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
// out the kernel raises a flag and stops waiting, so it always exits, and the
// flag NaN-poisons that job's basis at the end of the QR.
#include "qr.hpp"

#include "elementwise.hpp"
#include "gemm.hpp"

#include <algorithm>
#include <atomic>
#include <vector>

namespace mao {

namespace {

constexpr int NB = kQrNB;
typedef __attribute__((ext_vector_type(4))) double f64x4_t;
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
  int g0, G;         // the segment's first workgroup in the launch; workgroups per job
  int cnt;           // jobs in the segment (consecutive jobs of one size)
  int64_t wst, sS, spred;  // job strides: workspace (bytes), S (floats), pred (ints)
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

// Up to kQrMaxJobs segments per launch, of any sizes. A segment is cnt
// consecutive jobs of one size whose buffers sit at fixed strides; it owns
// workgroups [g0, g0 + cnt G) (G = ceil(len / 256) for its panel), job i of
// it the i-th run of G, and a job's barriers count only its own workgroups.
constexpr int kQrMaxJobs = 16;
struct PanelBatch {
  PanelArgs a[kQrMaxJobs];
  int njob;
};

// a workspace pointer of job 0 moved off bytes on (never null)
template <typename T>
__device__ __forceinline__ T* at_bytes(T* p, int64_t off) {
  return (T*)((char*)p + off);
}

// The segment of this workgroup, its job in the segment (*jl) and its index
// in that job's workgroups (*g).
template <typename Args>
__device__ __forceinline__ int seg_of(const Args* a, int njob, int* jl, int* g) {
  int sg = 0;
  while (sg + 1 < njob && (int)blockIdx.x >= a[sg + 1].g0) ++sg;
  const int rel = (int)blockIdx.x - a[sg].g0;
  *jl = rel / a[sg].G;
  *g = rel - *jl * a[sg].G;
  return sg;
}

__global__ __launch_bounds__(TPB) void qr_panel_kernel(PanelBatch B) {
  int jl, g;
  const PanelArgs& a = B.a[seg_of(B.a, B.njob, &jl, &g)];
  // job jl's buffers: workspace pointers ob bytes on, S so floats on (offsets
  // applied at each use, so the pointers stay reloadable kernel arguments)
  const int64_t ob = jl * a.wst, so = jl * a.sS;
  const int* const pred = a.pred ? a.pred + jl * a.spred : nullptr;
  const int G = a.G;
  if (pred != nullptr && *pred == 0) return;
  if (a.pred2 != nullptr && *at_bytes(a.pred2, ob) == 0) return;
  __shared__ float X[NB][LDX];
  __shared__ float red[NB][LDX];
  __shared__ float Tl[NB][NB + 1];
  __shared__ float qs[4][NB];
  __shared__ float tot[NB], dgv[NB], taus[NB], betas[NB];

  const int t = threadIdx.x;
  const int n = a.n, j0 = a.j0, nb = a.nb;
  const int r = j0 + g * TPB + t;
  const bool valid = r < n;

  for (int k0 = 0; k0 < NB; k0 += 16) {
    float xv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      xv[u] = (valid && k0 + u < nb) ? (a.S + so)[(int64_t)(j0 + k0 + u) * a.ldS + r] : 0.f;
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
    float* dgb = at_bytes(a.dg, ob) + (jj & 1) * NB;
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
    float* pb = at_bytes(a.part, ob) + (size_t)(jj & 1) * G * NB;
    if (t < NB) pb[g * NB + t] = qs[0][t] + qs[1][t] + qs[2][t] + qs[3][t];
    grid_barrier(at_bytes(a.counter, ob), ++bar * (unsigned)G, at_bytes(a.err, ob));
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
    for (int k = 0; k < nb; ++k) at_bytes(a.V, ob)[(int64_t)k * a.ldV + (r - j0)] = X[k][t];

  // partial Gram V^T V (strictly upper part)
  for (int e = t; e < NB * NB; e += TPB) {
    const int i = e >> 6, k = e & 63;
    float s = 0.f;
    if (i < k && k < nb)
      for (int u = 0; u < TPB; ++u) s += X[i][u] * X[k][u];
    at_bytes(a.gram, ob)[(size_t)g * NB * NB + e] = s;
  }
  grid_barrier(at_bytes(a.counter, ob), ++bar * (unsigned)G, at_bytes(a.err, ob));

  if (g == 0) {
    for (int e = t; e < NB * NB; e += TPB) {
      float s = 0.f;
      const int i = e >> 6, k = e & 63;
      if (i < k && k < nb) {
#pragma unroll 8
        for (int gg = 0; gg < G; ++gg) s += at_bytes(a.gram, ob)[(size_t)gg * NB * NB + e];
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
    for (int e = t; e < NB * NB; e += TPB) at_bytes(a.T, ob)[e] = Tl[e >> 6][e & 63];
    if (t < nb) at_bytes(a.sign, ob)[j0 + t] = betas[t] < 0.f ? -1.f : 1.f;
  }
  grid_barrier(at_bytes(a.counter, ob), ++bar * (unsigned)G, at_bytes(a.err, ob));

  for (int e = t; e < NB * NB; e += TPB) Tl[e >> 6][e & 63] = at_bytes(a.T, ob)[e];
  __syncthreads();
  if (valid) {
    float* zf = at_bytes(a.Zf, ob) + (int64_t)(r - j0) * NB;
    float* zo = at_bytes(a.Zo, ob) + (int64_t)(r - j0) * NB;
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
  int no_fallback; // test hook: a breakdown raises the job's time-out flag instead
  int g0, G;       // the segment's first workgroup in the launch; workgroups per job
  int cnt;         // jobs in the segment
  int64_t wst, sS, spred;  // job strides: workspace (bytes), S (floats), pred (ints)
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
  int jl, g;
  const CholArgs& a = B.a[seg_of(B.a, B.njob, &jl, &g)];
  // job jl's buffers: workspace pointers ob bytes on, S so floats on (offsets
  // applied at each use, so the pointers stay reloadable kernel arguments)
  const int64_t ob = jl * a.wst, so = jl * a.sS;
  const int* const pred = a.pred ? a.pred + jl * a.spred : nullptr;
  const int G = a.G;
  if (pred != nullptr && *pred == 0) return;
  __shared__ float X[NB][LDX];      // current Y (fp32), later V
  __shared__ __attribute__((aligned(16))) double Gs[NB][LDG];  // Gram / LU work
  __shared__ __attribute__((aligned(16))) double Rt[NB][LDG];  // Cholesky factor R (row k = R[k][.]); later U
  __shared__ __attribute__((aligned(16))) float Tl[NB][LDT];
  __shared__ double dinv[NB];
  __shared__ float dsg[NB];
  __shared__ double red64[TPB];
  __shared__ int bad;

  const int t = threadIdx.x;
  const int n = a.n, j0 = a.j0, nb = a.nb, len = n - j0;
  const int r = j0 + g * TPB + t;
  const bool valid = r < n;
  const int li = g * TPB + t;  // row of the panel

  for (int k0 = 0; k0 < NB; k0 += 16) {
    float xv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u)
      xv[u] = (valid && k0 + u < nb) ? (a.S + so)[(int64_t)(j0 + k0 + u) * a.ldS + r] : 0.f;
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
    // ---- partial Gram of this workgroup's rows on fp64 MFMA (products of
    // fp32 values are exact in fp64): the 10 upper 16 x 16 blocks (I <= J)
    // of X^T X over the 256 rows, 4 rows per step, blocks dealt to the
    // wavefronts in turn
    {
      const int wv = t >> 6, ln = t & 63;
      for (int blk = wv; blk < 10; blk += 4) {
        int I = 0, rem = blk;
        while (rem >= 4 - I) {
          rem -= 4 - I;
          ++I;
        }
        const int J = I + rem;
        f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
        const float* xa = &X[16 * I + (ln & 15)][ln >> 4];
        const float* xb = &X[16 * J + (ln & 15)][ln >> 4];
#pragma unroll 8
        for (int kk = 0; kk < TPB / 4; ++kk)
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64((double)xa[4 * kk], (double)xb[4 * kk], acc, 0,
                                                     0, 0);
        // A[i][k] comes from lane i + 16 k, B[k][j] from lane j + 16 k, and
        // lane ln's v-th result is G[16 I + 4 v + ln / 16][16 J + ln % 16]
        // (the fp64 16 x 16 layout, checked on the GPU)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int gi = 16 * I + 4 * v + (ln >> 4), gk = 16 * J + (ln & 15);
          if (gi <= gk) at_bytes(a.part, ob)[(size_t)g * NU + upk(gi, gk)] = acc[v];
        }
      }
    }
    grid_barrier(at_bytes(a.counter, ob), ++bar * (unsigned)G, at_bytes(a.err, ob));
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
            const double v0 = at_bytes(a.part, ob)[(size_t)gg * NU + e];
            const double v1 = at_bytes(a.part, ob)[(size_t)(gg + sub) * NU + e];
            const double v2 = at_bytes(a.part, ob)[(size_t)(gg + 2 * sub) * NU + e];
            const double v3 = at_bytes(a.part, ob)[(size_t)(gg + 3 * sub) * NU + e];
            sum += v0;
            sum += v1;
            sum += v2;
            sum += v3;
          }
          for (; gg < G; gg += sub) sum += at_bytes(a.part, ob)[(size_t)gg * NU + e];
        }
        __syncthreads();
        red64[t] = sum;
        __syncthreads();
        if (t < slots && q == 0 && e < e1) {
          double tot = 0.0;
          for (int u = 0; u < sub; ++u) tot += red64[t + u];
          at_bytes(a.gram, ob)[e] = tot;
        }
        __syncthreads();
      }
    }
    grid_barrier(at_bytes(a.counter, ob), ++bar * (unsigned)G, at_bytes(a.err, ob));
    // ---- Gram into LDS (symmetric), identity on the padded columns, shift
    {
      double gv[NB * NB / TPB];
#pragma unroll
      for (int u = 0; u < NB * NB / TPB; ++u) {
        const int idx = t + u * TPB, i = idx >> 6, k = idx & 63;
        gv[u] = (i < nb && k < nb) ? at_bytes(a.gram, ob)[i <= k ? upk(i, k) : upk(k, i)] : (i == k ? 1.0 : 0.0);
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
    // wavefront alone: lane j keeps column j of G in registers and computes
    // R[k][j]; the pivot and the row's other entries come from their lanes
    // by readlane, so the 64 steps touch LDS only to store R.
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
        // G[i][j] -= R[k][i] R[k][j], R[k][i] from lane i
#pragma unroll
        for (int i = k + 1; i < NB; ++i) gc[i] = fma(-lane_d(rkj, i), rkj, gc[i]);
        // keep the updates at this step (the compiler would otherwise sink
        // each one to the step that reads it, keeping every R entry live)
#pragma unroll
        for (int i = k + 1; i < NB; ++i) asm volatile("" : "+v"(gc[i]));
      }
      dinv[j] = 1.0 / Rt[j][j];  // own write above
      if (j == 0 && badl) bad = 1;
    }
    __syncthreads();
    if (bad) {
      if (g == 0 && t == 0) {
        *at_bytes(a.fail, ob) = 1;
        // test hook: no fallback -- the job's barriers give up, its basis is NaN
        if (a.no_fallback) atomicExch(at_bytes(a.err, ob), 1);
      }
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
      for (int j = 0; j < NB; ++j) at_bytes(a.T, ob)[i * NB + j] = (i < nb && j >= i && j < nb) ? (float)w[j] : 0.f;
    }
    __syncthreads();
    for (int e = t; e < nb * nb; e += TPB) {
      const int i = e / nb, c = e % nb;
      at_bytes(a.bcast, ob)[i * NB + c] = (i <= c) ? Rt[i][c] : 0.0;
    }
    if (t < nb) {
      at_bytes(a.bcast, ob)[NB * NB + t] = (double)dsg[t];
      at_bytes(a.sign, ob)[j0 + t] = dsg[t];
    }
  }
  grid_barrier(at_bytes(a.counter, ob), ++bar * (unsigned)G, at_bytes(a.err, ob));
  if (g != 0) {
    for (int e = t; e < nb * nb; e += TPB) Rt[e / nb][e % nb] = at_bytes(a.bcast, ob)[(e / nb) * NB + e % nb];
    if (t < nb) dsg[t] = (float)at_bytes(a.bcast, ob)[NB * NB + t];
  }
  for (int e = t; e < NB * NB; e += TPB) Tl[e >> 6][e & 63] = at_bytes(a.T, ob)[e];
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
    for (int k = 0; k < nb; ++k) at_bytes(a.V, ob)[(int64_t)k * a.ldV + li] = X[k][t];
    float* zf = at_bytes(a.Zf, ob) + (int64_t)li * NB;
    float* zo = at_bytes(a.Zo, ob) + (int64_t)li * NB;
    float vr[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) vr[i] = (i < nb) ? X[i][t] : 0.f;
    // four columns at a time, so that each row leaves in 16-byte pieces
    // (each column summed as four interleaved partial sums)
    for (int c4 = 0; c4 < NB; c4 += 4) {
      float sf[4][4], so[4][4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int q = 0; q < 4; ++q) sf[cc][q] = so[cc][q] = 0.f;
#pragma unroll
      for (int i4 = 0; i4 < NB / 4; ++i4) {
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const float4 f = ((const float4*)&Tl[c4 + cc][0])[i4];
          const float4 o = ((const float4*)&Tt[(c4 + cc) * LDT])[i4];
          sf[cc][0] = fmaf(vr[4 * i4 + 0], f.x, sf[cc][0]);
          sf[cc][1] = fmaf(vr[4 * i4 + 1], f.y, sf[cc][1]);
          sf[cc][2] = fmaf(vr[4 * i4 + 2], f.z, sf[cc][2]);
          sf[cc][3] = fmaf(vr[4 * i4 + 3], f.w, sf[cc][3]);
          so[cc][0] = fmaf(vr[4 * i4 + 0], o.x, so[cc][0]);
          so[cc][1] = fmaf(vr[4 * i4 + 1], o.y, so[cc][1]);
          so[cc][2] = fmaf(vr[4 * i4 + 2], o.z, so[cc][2]);
          so[cc][3] = fmaf(vr[4 * i4 + 3], o.w, so[cc][3]);
        }
      }
      float rf[4], ro[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        rf[cc] = (sf[cc][0] + sf[cc][1]) + (sf[cc][2] + sf[cc][3]);
        ro[cc] = (so[cc][0] + so[cc][1]) + (so[cc][2] + so[cc][3]);
      }
      *(float4*)(zf + c4) = make_float4(rf[0], rf[1], rf[2], rf[3]);
      *(float4*)(zo + c4) = make_float4(ro[0], ro[1], ro[2], ro[3]);
    }
  }
}

__global__ void zero_u32_kernel(unsigned* p, int n, int* err, int err_init) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
  if (threadIdx.x == 0) *err = err_init;
}

// A grid barrier that timed out (its flag raised) leaves the panels, and so
// the basis, undefined. Every job whose flag is up gets E and its row-major Q
// (when written) set to NaN, so that the step's update and weights come out
// NaN instead of silently wrong. One launch covers up to kPoisonJobs jobs
// (blockIdx.y); jobs with a zero predicate or a clear flag return at once.
constexpr int kPoisonJobs = 32;
struct PoisonArgs {
  const int* err;      // job j's flag at err + j * err_stride
  int64_t err_stride;  // ints
  float* E;            // job j at E + j * sE
  int64_t ldE, sE;
  float* Q[kPoisonJobs];
  int64_t ldQ[kPoisonJobs];
  const int* pred;
  int64_t spred;
  int n, j0;           // n x n matrices; first job of this launch
};

__global__ __launch_bounds__(256) void qr_poison_kernel(PoisonArgs a) {
  const int q = blockIdx.y, j = a.j0 + q;
  if (a.pred != nullptr && a.pred[j * a.spred] == 0) return;
  if (__hip_atomic_load(a.err + j * a.err_stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0)
    return;
  const float nan = __builtin_nanf("");
  const int64_t total = (int64_t)a.n * a.n;
  float* E = a.E + j * a.sE;
  float* Q = a.Q[q];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / a.n, c = i - r * a.n;
    E[r * a.ldE + c] = nan;
    if (Q != nullptr) Q[r * a.ldQ[q] + c] = nan;
  }
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
    return launch_gemm(MAO_F32, &p1, 1, stream, TAG_QR_PROJ);
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
  MAO_TRY(launch_gemm(MAO_F32, pr, nparts, stream, TAG_QR_PROJ));
  const int64_t count = (int64_t)M * NB;
  const int blocks = (int)std::min<int64_t>(1024, (count + 255) / 256);
  hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks, njob), dim3(256), 0, stream, W, parts, stride,
                     nparts, count, sW, pred, spred);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

int panels(int n) { return (n + NB - 1) / NB; }

// Column splits of a fused panel update over an M x L block: enough
// workgroups to give every CU about two, while each split keeps at least four
// 64-column chunks.
// Column ranges per strip of a fused pass. Every workgroup walks its chunks
// one after another, so a pass takes (rounds of resident workgroups) x
// (chunks per workgroup + about 3 for loading W and writing Wn); the split
// count minimising that is taken (at least 4 chunks per range).
int fused_splits(int M, int L, int njob) {
  const int strips = (M + NB - 1) / NB, chunks = (L + NB - 1) / NB;
  const int64_t slots = qr_fused_slots();
  int best = 1;
  int64_t best_t = INT64_MAX;
  for (int sp = 1; sp <= kQrFusedMaxSplits; ++sp) {
    if (sp > 1 && chunks / sp < 4) break;
    const int64_t wg = (int64_t)njob * strips * sp;
    const int64_t t = ((wg + slots - 1) / slots) * ((chunks + sp - 1) / sp + 3);
    if (t < best_t) {
      best_t = t;
      best = sp;
    }
  }
  return best;
}
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
  w.zf2 = c.take<float>((size_t)n * NB);
  w.wbuf = c.take<float>((size_t)n * NB);
  // split-K partials of the projections, or two regions of fused-update slices
  w.wparts = c.take<float>((size_t)std::max(KSPLIT, 2 * kQrFusedMaxSplits) * n * NB);
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
  w.zsp = c.take<bf16_t>((size_t)3 * n * NB);
  w.vsp = c.take<bf16_t>((size_t)3 * NB * round_up(n, 8));
  return w;
}

size_t qr_work_bytes(int n) {
  Carver c(nullptr);
  carve_qr_work(c, n);
  return c.used + 256;
}

size_t qr_work_stride(int n) { return align_up(qr_work_bytes(n), 256); }

namespace {

// Workgroups of the panel kernels that fit on the device at once (one per CU
// for their LDS footprint): the most one cooperative panel launch may hold.
// The per-device figure is cached; threads that race on the first call both
// compute the same value, and the atomic store/load keeps that race defined.
int panel_slots() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int slots = cached[dev].load(std::memory_order_relaxed);
  if (slots == 0) {
    int cus = 0, b1 = 0, b2 = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b1, qr_panel_chol_kernel, TPB, 0) != hipSuccess) b1 = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b2, qr_panel_kernel, TPB, 0) != hipSuccess) b2 = 1;
    slots = std::max(1, cus * std::max(1, std::min(b1, b2)));
    cached[dev].store(slots, std::memory_order_relaxed);
  }
  return slots;
}

}  // namespace

namespace {

// One size group of a refresh: its jobs, workspaces and the state the
// factorisation carries from panel to panel.
struct QrRun {
  const QrBatch* b = nullptr;
  int n = 0, nj = 0, np = 0;
  size_t wst = 0;
  int64_t wsf = 0, wsl = 0;  // job stride of the workspace and slice stride of W, in floats
  std::vector<QrWork> w;
  std::vector<int64_t> vo, zo;  // offsets of the packed panels (the same in every job)
  float* wprev = nullptr;       // W_{p-1}, as sprev slices
  int sprev = 1;
  float* wnext = nullptr;

  const int* job_pred(int j) const { return b->pred ? b->pred + j * b->spred : nullptr; }
  int prec() const { return b->fact_bf16x3 ? kQrBf16x3 : kQrBf16x6; }

  mao_status setup(const QrBatch& batch, hipStream_t stream) {
    b = &batch;
    n = batch.n;
    nj = batch.njob;
    np = panels(n);
    wst = qr_work_stride(n);
    wsf = (int64_t)(wst / sizeof(float));
    wsl = (int64_t)n * NB;
    w.resize(nj);
    for (int j = 0; j < nj; ++j) {
      Carver c(batch.work + (size_t)j * wst);
      w[j] = carve_qr_work(c, n);
      const int err0 = batch.abort_barriers ? 1 : 0;
      hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, w[j].counters, 2 * np, w[j].err, err0);
      hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, (unsigned*)w[j].fail, np, w[j].err, err0);
    }
    MAO_LAUNCH_CHECK();
    int64_t voff = 0, zoff = 0;
    vo.resize(np);
    zo.resize(np);
    for (int p = 0; p < np; ++p) {
      const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
      vo[p] = voff;
      zo[p] = zoff;
      voff += round_up((int64_t)nb * round_up(len, 8), 64);
      zoff += round_up((int64_t)len * NB, 64);
    }
    wprev = w[0].wbuf;
    sprev = 1;
    wnext = w[0].wparts;
    return MAO_OK;
  }

  float* zf_of(int p) const { return (p & 1) ? w[0].zf2 : w[0].zf; }

  // the split operands of this group's fused passes: Z parts zpart apart at
  // row pitch 64, vector parts vpart apart at row pitch ldvp
  int64_t zpart() const { return (int64_t)n * NB; }
  int64_t ldvp() const { return round_up(n, 8); }
  int64_t vpart() const { return (int64_t)NB * ldvp(); }
  int64_t wsb() const { return (int64_t)(wst / sizeof(bf16_t)); }  // job stride, in bf16
  int parts(int prec) const { return prec == kQrBf16x6 ? 3 : 2; }

  // Z (zrows x 64, columns >= znb zero) and/or V (vrows x vcols at ldv) of
  // every job into their bf16 parts
  mao_status presplit(const float* Z, int zrows, int znb, const float* V, int64_t ldv, int vrows,
                      int vcols, int prec, hipStream_t stream) const {
    QrSplitArgs sa;
    sa.Z = Z;
    sa.sZ = wsf;
    sa.zrows = Z ? zrows : 0;
    sa.znb = znb;
    sa.Zp = w[0].zsp;
    sa.sZp = wsb();
    sa.zpart = zpart();
    sa.V = V;
    sa.ldV = ldv;
    sa.sV = wsf;
    sa.vrows = V ? vrows : 0;
    sa.vcols = vcols;
    sa.Vp = w[0].vsp;
    sa.sVp = wsb();
    sa.vpart = vpart();
    sa.ldVp = ldvp();
    sa.parts = parts(prec);
    sa.pred = b->pred;
    sa.spred = b->spred;
    return qr_presplit(sa, nj, stream);
  }

  // the fused-pass arguments that point at the split operands (Z from row
  // zrow0 of its parts, Vn from column vcol0 of its parts)
  void split_args(QrFusedArgs& f, int zrow0, int vcol0) const {
    f.Zp = w[0].zsp + (int64_t)zrow0 * NB;
    f.sZp = wsb();
    f.zpart = zpart();
    f.Vp = w[0].vsp + vcol0;
    f.ldVp = ldvp();
    f.sVp = wsb();
    f.vpart = vpart();
  }

  // Factorisation with one panel of look-ahead. W_{p-1} is the projection of
  // panel p-1's trailing rows onto its vectors. Before panel p is factored,
  // only its own rows take panel p-1's update; the rest of the trailing rows
  // take it afterwards in one fused pass that also projects them onto panel
  // p's vectors (W_p). Only columns >= j0 are updated: the R block left of
  // them is never read again (the basis comes from the vectors alone). V T^T
  // of consecutive panels alternate between zf and zf2; W alternates between
  // the two slice regions of wparts (wbuf for the first panel's plain
  // projection).
  mao_status before_panel(int p, hipStream_t stream) {
    if (p == 0 || p >= np) return MAO_OK;
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    // V T^T of panel p-1 (len + NB rows) split once for this step's two passes
    MAO_TRY(presplit(zf_of(p - 1), len + NB, NB, nullptr, 0, 0, 0, prec(), stream));
    // panel p's rows take panel p-1's update (one 64-column chunk per workgroup)
    QrFusedArgs fa;
    fa.C = b->S + (int64_t)j0 * b->ldS + j0;
    fa.ldC = b->ldS;
    fa.sC = b->sS;
    fa.W = wprev;
    fa.sW = wsf;
    fa.wslices_in = sprev;
    fa.wslice = wsl;
    split_args(fa, NB, 0);  // V T^T rows of the columns >= j0
    fa.M = nb;
    fa.L = len;
    fa.nb = NB;  // panel p-1 is a full panel
    fa.nbn = 0;
    fa.splits = (len + NB - 1) / NB;
    fa.prec = prec();
    fa.pred = b->pred;
    fa.spred = b->spred;
    return qr_fused_update(fa, nj, stream);
  }

  // The arguments of job j's panel p for both panel kernels.
  void panel_args(int p, int j, PanelArgs& a, CholArgs& ca) const {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    const QrWork& wj = w[j];
    a.S = b->S + j * b->sS;
    a.ldS = b->ldS;
    a.n = n;
    a.j0 = j0;
    a.nb = nb;
    a.V = wj.vstore + vo[p];
    a.ldV = round_up(len, 8);
    a.Zf = (p & 1) ? wj.zf2 : wj.zf;
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
    a.G = (len + TPB - 1) / TPB;
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
    ca.no_fallback = b->no_fallback ? 1 : 0;
    ca.G = a.G;
  }

  mao_status after_panel(int p, hipStream_t stream) {
    if (p >= np) return MAO_OK;
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    const int mt = n - j0 - nb;
    if (mt <= 0) return MAO_OK;
    float* Strail = b->S + (int64_t)(j0 + nb) * b->ldS + j0;
    if (p == 0) {
      // W_0 = S_trail V_0^T   (mt x nb)
      return skinny_product(mt, nb, len, Strail, b->ldS, b->sS, w[0].vstore + vo[p],
                            round_up(len, 8), wsf, w[0].wbuf, w[0].wparts, wsf, nj, b->pred,
                            b->spred, stream);
    }
    // the rest of the trailing rows: panel p-1's update, then W_p = S_trail V_p^T
    MAO_TRY(presplit(nullptr, 0, 0, w[0].vstore + vo[p], round_up(len, 8), nb, len, prec(), stream));
    QrFusedArgs fc;
    fc.C = Strail;
    fc.ldC = b->ldS;
    fc.sC = b->sS;
    fc.W = wprev + (int64_t)nb * NB;  // W_{p-1} rows of S rows >= j0 + nb
    fc.sW = wsf;
    fc.wslices_in = sprev;
    fc.wslice = wsl;
    split_args(fc, NB, 0);
    fc.Wn = wnext;
    fc.sWn = wsf;
    fc.M = mt;
    fc.L = len;
    fc.nb = NB;
    fc.nbn = nb;
    fc.splits = fused_splits(mt, len, nj);
    fc.prec = prec();
    fc.pred = b->pred;
    fc.spred = b->spred;
    MAO_TRY(qr_fused_update(fc, nj, stream));
    wprev = wnext;
    sprev = fc.splits;
    wnext = wnext == w[0].wparts ? w[0].wparts + kQrFusedMaxSplits * wsl : w[0].wparts;
    return MAO_OK;
  }

  mao_status finish(hipStream_t stream);
};

// Panel launches of one panel index over the jobs of every size group: each
// launch takes jobs while their workgroups fit the device at once (the panel
// kernels need all of them resident), as segments of consecutive jobs of one
// group, while the segment table has room.
mao_status launch_panels(const std::vector<const QrRun*>& runs, int p, hipStream_t stream) {
  const int slots = panel_slots();
  size_t r = 0;
  int j = 0;
  while (r < runs.size()) {
    CholBatch cb;
    PanelBatch pb;
    int ng = 0, cn = 0;
    while (r < runs.size() && cn < kQrMaxJobs) {
      const QrRun& run = *runs[r];
      PanelArgs a;
      CholArgs ca;
      run.panel_args(p, j, a, ca);
      int cnt = std::min(run.nj - j, (slots - ng) / a.G);
      if (cnt <= 0) {
        if (cn > 0) break;
        cnt = 1;
      }
      a.g0 = ca.g0 = ng;
      a.cnt = ca.cnt = cnt;
      a.wst = ca.wst = (int64_t)run.wst;
      a.sS = ca.sS = run.b->sS;
      a.spred = ca.spred = run.b->spred;
      ng += cnt * a.G;
      pb.a[cn] = a;
      cb.a[cn] = ca;
      ++cn;
      j += cnt;
      if (j == run.nj) {
        ++r;
        j = 0;
      }
    }
    cb.njob = pb.njob = cn;
    void* ev = nullptr;
    const bool timed = timing_on();
    if (timed) timing_record_begin(stream, &ev);
    void* cargs[] = {&cb};
    MAO_HIP_CHECK(hipLaunchCooperativeKernel((const void*)qr_panel_chol_kernel, dim3(ng),
                                             dim3(TPB), cargs, 0, stream));
    void* kargs[] = {&pb};
    MAO_HIP_CHECK(hipLaunchCooperativeKernel((const void*)qr_panel_kernel, dim3(ng), dim3(TPB),
                                             kargs, 0, stream));
    if (timed) timing_record_end(stream, ev, TAG_QR_PANEL, 0.0);
  }
  return MAO_OK;
}

}  // namespace

mao_status qr_core_multi(const QrBatch* batches, int ngroups, hipStream_t stream) {
  std::vector<QrRun> runs;
  runs.reserve(ngroups);
  int np = 0;
  for (int g = 0; g < ngroups; ++g) {
    if (batches[g].njob <= 0) continue;
    runs.emplace_back();
    MAO_TRY(runs.back().setup(batches[g], stream));
    np = std::max(np, runs.back().np);
  }
  // panel index by panel index over every size: the panels of all groups
  // share launches (the groups are independent; each keeps its own order)
  std::vector<const QrRun*> live;
  for (int p = 0; p < np; ++p) {
    live.clear();
    for (QrRun& r : runs) {
      if (p >= r.np) continue;
      MAO_TRY(r.before_panel(p, stream));
      live.push_back(&r);
    }
    MAO_TRY(launch_panels(live, p, stream));
    for (QrRun& r : runs) MAO_TRY(r.after_panel(p, stream));
  }
  for (QrRun& r : runs) MAO_TRY(r.finish(stream));
  return MAO_OK;
}

mao_status qr_core_batched(const QrBatch& b, hipStream_t stream) {
  return qr_core_multi(&b, 1, stream);
}

namespace {

mao_status QrRun::finish(hipStream_t stream) {
  const QrBatch& bb = *b;
  // explicit Q: E = Q^T, backward accumulation. The last panel's projection
  // is a plain product (into wbuf); every later one comes out of the previous
  // panel's fused update as partial slices, in two regions of wparts used in
  // turn.
  for (int j = 0; j < nj; ++j)
    MAO_TRY(fill_identity(view(bb.E + j * bb.sE, bb.ldE), n, job_pred(j), stream));
  float* wcur = w[0].wbuf;
  int s_in = 1;
  float* wnext = w[0].wparts;
  {
    const int p = np - 1, j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    float* Esub = bb.E + (int64_t)j0 * bb.ldE + j0;
    MAO_TRY(skinny_product(len, nb, len, Esub, bb.ldE, bb.sE, w[0].vstore + vo[p], round_up(len, 8),
                           wsf, wcur, w[0].wparts, wsf, nj, bb.pred, bb.spred, stream));
  }
  for (int p = np - 1; p >= 1; --p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    const int pp = p - 1, lenn = n - pp * NB, nbn = std::min(NB, lenn);
    // V T of panel p and the vectors of panel pp, split
    MAO_TRY(presplit(w[0].zo + zo[p], len, nb, w[0].vstore + vo[pp], round_up(lenn, 8), nbn,
                     lenn, kQrBf16x6, stream));
    QrFusedArgs fa;
    fa.C = bb.E + (int64_t)j0 * bb.ldE + j0;
    fa.ldC = bb.ldE;
    fa.sC = bb.sE;
    fa.sW = wsf;
    // panel pp's vectors start NB columns left of this block
    split_args(fa, 0, NB);
    fa.ldV = round_up(lenn, 8);
    fa.sV = wsf;
    fa.Wn = wnext + (int64_t)NB * NB;
    fa.sWn = wsf;
    fa.Wt = wnext;
    fa.Vt = w[0].vstore + vo[pp];
    fa.trows = NB;
    fa.M = len;
    fa.L = len;
    fa.nb = nb;
    fa.nbn = nbn;
    fa.pred = bb.pred;
    fa.spred = bb.spred;
    fa.W = wcur;
    fa.wslices_in = s_in;
    fa.wslice = wsl;
    fa.splits = fused_splits(len, len, nj);
    fa.prec = kQrBf16x6;
    MAO_TRY(qr_fused_update(fa, nj, stream));
    wcur = wnext;
    s_in = fa.splits;
    wnext = wnext == w[0].wparts ? w[0].wparts + kQrFusedMaxSplits * wsl : w[0].wparts;
  }
  if (s_in > 1) {
    const int64_t count = (int64_t)n * NB;
    const int blocks = (int)std::min<int64_t>(1024, (count + 255) / 256);
    hipLaunchKernelGGL(sum_parts_kernel, dim3(blocks, nj), dim3(256), 0, stream, w[0].wbuf, wcur,
                       wsl, s_in, count, wsf, bb.pred, bb.spred);
    MAO_LAUNCH_CHECK();
    wcur = w[0].wbuf;
  }
  {
    // first block: column signs, and each job's Q written as the transposed copy
    const int len = n, nb = std::min(NB, len);
    float* Esub = bb.E;
    GemmProblem p2 = gemm_problem(len, len, nb, -1.f, wcur, NB, w[0].zo + zo[0], NB, 1.f,
                                  Esub, bb.ldE, Esub, bb.ldE, GF_D_F32 | GF_C0_F32);
    p2.batch = nj;
    p2.sA = p2.sB = wsf;
    p2.sC0 = p2.sD = bb.sE;
    p2.pred = bb.pred;
    p2.spred = bb.spred;
    p2.row_scale = w[0].sign;
    p2.srs = wsf;
    bool anyq = false;
    for (int j = 0; j < nj; ++j) anyq = anyq || (bb.Q && bb.Q[j]);
    if (!anyq) {
      MAO_TRY(launch_gemm(MAO_F32, &p2, 1, stream, TAG_QR));
    } else {
      for (int c0 = 0; c0 < nj; c0 += kMaxProblems) {
        const int cn = std::min(kMaxProblems, nj - c0);
        GemmProblem pq[kMaxProblems];
        for (int q = 0; q < cn; ++q) {
          const int j = c0 + q;
          pq[q] = p2;
          pq[q].batch = 1;
          pq[q].A = wcur + j * wsf;
          pq[q].B = w[j].zo + zo[0];
          pq[q].C0 = pq[q].D = Esub + j * bb.sE;
          pq[q].row_scale = w[j].sign;
          pq[q].pred = job_pred(j);
          pq[q].spred = 0;
          if (bb.Q && bb.Q[j]) {
            pq[q].Dt = bb.Q[j];
            pq[q].lddt = bb.ldQ[j];
          }
        }
        MAO_TRY(launch_gemm(MAO_F32, pq, cn, stream, TAG_QR));
      }
    }
  }

  for (int c0 = 0; c0 < nj; c0 += kPoisonJobs) {
    const int cn = std::min(kPoisonJobs, nj - c0);
    PoisonArgs pa;
    pa.err = w[0].err;
    pa.err_stride = (int64_t)(wst / sizeof(int));
    pa.E = bb.E;
    pa.ldE = bb.ldE;
    pa.sE = bb.sE;
    for (int q = 0; q < kPoisonJobs; ++q) {
      const bool has = q < cn && bb.Q && bb.Q[c0 + q];
      pa.Q[q] = has ? bb.Q[c0 + q] : nullptr;
      pa.ldQ[q] = has ? bb.ldQ[c0 + q] : 0;
    }
    pa.pred = bb.pred;
    pa.spred = bb.spred;
    pa.n = n;
    pa.j0 = c0;
    const int blocks = (int)std::min<int64_t>(256, ceil_div((int64_t)n * n, 256));
    hipLaunchKernelGGL(qr_poison_kernel, dim3(blocks, cn), dim3(256), 0, stream, pa);
    MAO_LAUNCH_CHECK();
  }
  return MAO_OK;
}

}  // namespace

mao_status qr_core(float* S, int64_t ldS, int n, float* E, int64_t ldE, float* Qout, int64_t ldQ,
                   QrWork& w, const int* pred, hipStream_t stream, bool abort_barriers,
                   bool fact_bf16x3, bool no_fallback) {
  QrBatch b;
  b.abort_barriers = abort_barriers;
  b.no_fallback = no_fallback;
  b.fact_bf16x3 = fact_bf16x3;
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
