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

__global__ __launch_bounds__(TPB) void qr_panel_kernel(PanelArgs a) {
  if (a.pred != nullptr && *a.pred == 0) return;
  __shared__ float X[NB][LDX];
  __shared__ float red[NB][LDX];
  __shared__ float Tl[NB][NB + 1];
  __shared__ float qs[4][NB];
  __shared__ float tot[NB], dgv[NB], taus[NB], betas[NB];

  const int t = threadIdx.x, g = blockIdx.x, G = gridDim.x;
  const int n = a.n, j0 = a.j0, nb = a.nb;
  const int r = j0 + g * TPB + t;
  const bool valid = r < n;

  for (int k = 0; k < NB; ++k) X[k][t] = (valid && k < nb) ? a.S[(int64_t)(j0 + k) * a.ldS + r] : 0.f;
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
    for (int c = 0; c < NB; ++c) {
      float sf = 0.f, so = 0.f;
      for (int i = 0; i < nb; ++i) {
        sf += X[i][t] * Tl[c][i];
        so += X[i][t] * Tl[i][c];
      }
      zf[c] = sf;
      zo[c] = so;
    }
  }
}

__global__ void zero_u32_kernel(unsigned* p, int n, int* err) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
  if (threadIdx.x == 0) *err = 0;
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
  w.sign = c.take<float>(n);
  w.part = c.take<float>((size_t)2 * G * NB);
  w.dg = c.take<float>(2 * NB);
  w.gram = c.take<float>((size_t)G * NB * NB);
  w.T = c.take<float>(NB * NB);
  w.counters = c.take<unsigned>(panels(n));
  w.err = c.take<int>(1);
  return w;
}

size_t qr_work_bytes(int n) {
  Carver c(nullptr);
  carve_qr_work(c, n);
  return c.used + 256;
}

mao_status qr_core(float* S, int64_t ldS, int n, float* E, int64_t ldE, float* Qout, int64_t ldQ,
                   QrWork& w, const int* pred, hipStream_t stream) {
  const int np = panels(n);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(256), 0, stream, w.counters, np, w.err);
  MAO_LAUNCH_CHECK();

  // offsets of the packed panels
  int64_t voff = 0, zoff = 0;
  std::vector<int64_t> vo(np), zo(np);
  for (int p = 0; p < np; ++p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    vo[p] = voff;
    zo[p] = zoff;
    voff += round_up((int64_t)nb * round_up(len, 8), 64);
    zoff += round_up((int64_t)len * NB, 64);
  }

  for (int p = 0; p < np; ++p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    const int G = (len + TPB - 1) / TPB;
    PanelArgs a;
    a.S = S;
    a.ldS = ldS;
    a.n = n;
    a.j0 = j0;
    a.nb = nb;
    a.V = w.vstore + vo[p];
    a.ldV = round_up(len, 8);
    a.Zf = w.zf;
    a.Zo = w.zo + zo[p];
    a.sign = w.sign;
    a.part = w.part;
    a.dg = w.dg;
    a.gram = w.gram;
    a.T = w.T;
    a.counter = w.counters + p;
    a.err = w.err;
    a.pred = pred;
    void* kargs[] = {&a};
    MAO_HIP_CHECK(hipLaunchCooperativeKernel((const void*)qr_panel_kernel, dim3(G), dim3(TPB),
                                             kargs, 0, stream));
    const int mt = n - j0 - nb;
    if (mt > 0) {
      float* Strail = S + (int64_t)(j0 + nb) * ldS + j0;
      // W = S_trail V^T   (mt x nb)
      GemmProblem p1 = gemm_problem(mt, nb, len, 1.f, Strail, ldS, a.V, a.ldV, 0.f, nullptr, 0,
                                    w.wbuf, NB, GF_D_F32);
      p1.pred = pred;
      MAO_TRY(launch_gemm(MAO_F32, &p1, 1, stream, TAG_QR));
      // S_trail -= W Zf^T  (mt x len)
      GemmProblem p2 = gemm_problem(mt, len, nb, -1.f, w.wbuf, NB, w.zf, NB, 1.f, Strail, ldS,
                                    Strail, ldS, GF_D_F32 | GF_C0_F32);
      p2.pred = pred;
      MAO_TRY(launch_gemm(MAO_F32, &p2, 1, stream, TAG_QR));
    }
  }

  // explicit Q: E = Q^T, backward accumulation
  MAO_TRY(fill_identity(view(E, ldE), n, pred, stream));
  for (int p = np - 1; p >= 0; --p) {
    const int j0 = p * NB, len = n - j0, nb = std::min(NB, len);
    float* Esub = E + (int64_t)j0 * ldE + j0;
    GemmProblem p1 = gemm_problem(len, nb, len, 1.f, Esub, ldE, w.vstore + vo[p], round_up(len, 8),
                                  0.f, nullptr, 0, w.wbuf, NB, GF_D_F32);
    p1.pred = pred;
    MAO_TRY(launch_gemm(MAO_F32, &p1, 1, stream, TAG_QR));
    GemmProblem p2 = gemm_problem(len, len, nb, -1.f, w.wbuf, NB, w.zo + zo[p], NB, 1.f, Esub, ldE,
                                  Esub, ldE, GF_D_F32 | GF_C0_F32);
    p2.pred = pred;
    if (p == 0) {
      p2.row_scale = w.sign;
      if (Qout) {
        p2.Dt = Qout;
        p2.lddt = ldQ;
      }
    }
    MAO_TRY(launch_gemm(MAO_F32, &p2, 1, stream, TAG_QR));
  }
  return MAO_OK;
}

}  // namespace mao
