// Observability reductions (see observe.hpp). Memory-bound passes over
// buffers the steps already hold; each reduction runs in a fixed order, with
// fp64 accumulation, so repeated calls are bitwise identical.
#include <math.h>

#include "observe.hpp"

namespace mao {
namespace {

constexpr int kObs = 256;

// Rows start 16-byte aligned (data 16-byte aligned, ld and batch strides
// multiples of 8 elements, checked on the host), so every lane reads 16
// bytes: 4 fp32 or 8 bf16 values.
__device__ __forceinline__ int vec_load(const float* p, float* v) {
  const float4 q = *(const float4*)p;
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  return 4;
}
__device__ __forceinline__ int vec_load(const bf16_t* p, float* v) {
  const uint4 q = *(const uint4*)p;
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bf16_to_f32((bf16_t)(w[e] & 0xffff));
    v[2 * e + 1] = bf16_to_f32((bf16_t)(w[e] >> 16));
  }
  return 8;
}
template <typename T> constexpr int vec_width() { return 16 / (int)sizeof(T); }

template <typename T>
__global__ __launch_bounds__(kObs) void sumsq_partial_kernel(View X, int rows, int cols, int rpb,
                                                             int nrb, int sub_identity,
                                                             double* part) {
  __shared__ double sc[16];
  const int b = blockIdx.y, blk = blockIdx.x;
  const T* base = (const T*)X.p + (int64_t)b * X.stride;
  const int r0 = blk * rpb, r1 = min(rows, r0 + rpb);
  constexpr int VW = vec_width<T>();
  const int colsv = cols - cols % VW;
  double acc = 0.0;
  for (int i = r0; i < r1; ++i) {
    const T* row = base + (int64_t)i * X.ld;
    float rs = 0.f;  // this row's share, fp32 (at most cols / 256 / VW + 1 terms per lane)
    for (int j = threadIdx.x * VW; j < colsv; j += kObs * VW) {
      float v[VW];
      vec_load(row + j, v);
      if (sub_identity && i >= j && i < j + VW) v[i - j] -= 1.f;
#pragma unroll
      for (int e = 0; e < VW; ++e) rs = fmaf(v[e], v[e], rs);
    }
    for (int j = colsv + threadIdx.x; j < cols; j += kObs) {
      float v = load_f32<T>(row + j);
      if (sub_identity && i == j) v -= 1.f;
      rs = fmaf(v, v, rs);
    }
    acc += (double)rs;
  }
  acc = block_sum_d(acc, sc);
  if (threadIdx.x == 0) part[(int64_t)b * nrb + blk] = acc;
}

__global__ __launch_bounds__(kObs) void finalize_rms_kernel(const double* part, int nrb,
                                                            double divisor, float* out) {
  __shared__ double sc[16];
  const int b = blockIdx.x;
  double acc = 0.0;
  for (int i = threadIdx.x; i < nrb; i += kObs) acc += part[(int64_t)b * nrb + i];
  acc = block_sum_d(acc, sc);
  if (threadIdx.x == 0) out[b] = (float)sqrt(acc / divisor);
}

__global__ __launch_bounds__(kObs) void row_dots_kernel(View A, View B, int n, int cols,
                                                        float* d) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kObs / 64) + (threadIdx.x >> 6);
  if (i >= n) return;
  const float* a = (const float*)A.p + (int64_t)i * A.ld;
  const float* bb = (const float*)B.p + (int64_t)i * B.ld;
  double acc = 0.0;
  for (int k = lane; k < cols; k += 64) acc += (double)a[k] * (double)bb[k];
  acc = wave_sum_d(acc);
  if (lane == 0) d[i] = (float)acc;
}

__global__ __launch_bounds__(1024) void kappa_kernel(const float* d, int n, float* kappa) {
  __shared__ float smax[16], smin[16];
  float mx = -INFINITY, mn = INFINITY;
  for (int i = threadIdx.x; i < n; i += 1024) {
    mx = fmaxf(mx, d[i]);
    mn = fminf(mn, d[i]);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    mn = fminf(mn, __shfl_xor(mn, off, 64));
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    smax[wid] = mx;
    smin[wid] = mn;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 0; w < 16; ++w) {
      mx = fmaxf(mx, smax[w]);
      mn = fminf(mn, smin[w]);
    }
    kappa[0] = mn > 0.f ? mx / mn : INFINITY;
  }
}

__global__ __launch_bounds__(kObs) void gemv_rows_kernel(View V, int m, int n, const float* x,
                                                         float* y) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kObs / 64) + (threadIdx.x >> 6);
  if (i >= m) return;
  const float* row = (const float*)V.p + (int64_t)i * V.ld;
  const int nv = n & ~3;
  double acc = 0.0;
  // four 16-byte loads in flight per lane before they are consumed
  int j = lane * 4;
  for (; j + 768 < nv; j += 1024) {
    float a[4][4], b[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      vec_load(row + j + 256 * u, a[u]);
      vec_load(x + j + 256 * u, b[u]);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc += (double)(a[u][0] * b[u][0] + a[u][1] * b[u][1]) +
             (double)(a[u][2] * b[u][2] + a[u][3] * b[u][3]);
  }
  for (; j < nv; j += 256) {
    float a[4], b[4];
    vec_load(row + j, a);
    vec_load(x + j, b);
    acc += (double)(a[0] * b[0] + a[1] * b[1]) + (double)(a[2] * b[2] + a[3] * b[3]);
  }
  for (int jj = nv + lane; jj < n; jj += 64) acc += (double)row[jj] * (double)x[jj];
  acc = wave_sum_d(acc);
  if (lane == 0) y[i] = (float)acc;
}

// Each lane owns 4 adjacent columns (16-byte loads along a row).
__global__ __launch_bounds__(kObs) void gemv_cols_partial_kernel(View V, int m, int n, int rpb,
                                                                 const float* y, float* part) {
  const int blk = blockIdx.x;
  const int j = (blockIdx.y * kObs + threadIdx.x) * 4;
  if (j >= n) return;
  const int r0 = blk * rpb, r1 = min(m, r0 + rpb);
  const float* col = (const float*)V.p + j;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (j + 3 < n) {
#pragma unroll 4
    for (int i = r0; i < r1; ++i) {
      float a[4];
      vec_load(col + (int64_t)i * V.ld, a);
      const double yi = (double)y[i];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += (double)a[e] * yi;
    }
  } else {
    for (int i = r0; i < r1; ++i)
      for (int e = 0; j + e < n; ++e) acc[e] += (double)col[(int64_t)i * V.ld + e] * (double)y[i];
  }
  for (int e = 0; e < 4 && j + e < n; ++e) part[(int64_t)blk * n + j + e] = (float)acc[e];
}

// 64 columns per workgroup, four lanes per column: lane group g sums row
// blocks [g q, (g + 1) q) in order with eight loads in flight, then the four
// group sums are added in order g = 0..3 (fixed order: bitwise repeatable).
__global__ __launch_bounds__(kObs) void gemv_cols_final_kernel(const float* part, int nrb, int n,
                                                               float* z) {
  __shared__ double gs[4][64];
  const int c = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + c;
  const int q = (nrb + 3) / 4, b0 = g * q, b1 = min(nrb, b0 + q);
  double acc = 0.0;
  if (j < n) {
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(b + u) * n + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += (double)v[u];
    }
    for (; b < b1; ++b) acc += (double)part[(int64_t)b * n + j];
  }
  gs[g][c] = acc;
  __syncthreads();
  if (g == 0 && j < n) z[j] = (float)(((gs[0][c] + gs[1][c]) + gs[2][c]) + gs[3][c]);
}

__global__ __launch_bounds__(1024) void normalize_kernel(float* v, int n) {
  __shared__ double sc[16];
  double acc = 0.0;
  for (int j = threadIdx.x; j < n; j += 1024) acc += (double)v[j] * (double)v[j];
  acc = block_sum_d(acc, sc);
  if (!(acc > 0.0)) return;  // a zero vector stays as it is
  const float inv = (float)(1.0 / sqrt(acc));
  for (int j = threadIdx.x; j < n; j += 1024) v[j] *= inv;
}

__global__ __launch_bounds__(kObs) void fill_unit_kernel(float* v, int n) {
  const int j = blockIdx.x * kObs + threadIdx.x;
  if (j < n) v[j] = (float)(1.0 / sqrt((double)n));
}

__global__ __launch_bounds__(1024) void share_kernel(const float* y, int m, const double* vpart,
                                                     int nrb, float* out) {
  __shared__ double sc[16];
  double s = 0.0, f = 0.0;
  for (int i = threadIdx.x; i < m; i += 1024) s += (double)y[i] * (double)y[i];
  for (int i = threadIdx.x; i < nrb; i += 1024) f += vpart[i];
  s = block_sum_d(s, sc);
  f = block_sum_d(f, sc);
  if (threadIdx.x == 0) out[0] = f > 0.0 ? (float)(s / f) : 0.f;
}

__global__ void basis_age_kernel(const float* aux, float* age) {
  age[0] = aux[1] != 0.f ? 0.f : age[0] + 1.f;
}

int rows_per(int rows, int nrb) { return (rows + nrb - 1) / nrb; }

}  // namespace

int obs_rowblocks(int64_t rows) {
  // about 2048 rows blocks, at least 4 rows each
  int64_t nrb = (rows + 3) / 4;
  if (nrb > 2048) nrb = 2048;
  return (int)(nrb < 1 ? 1 : nrb);
}

mao_status sumsq_partials(View X, int x_dtype, int rows, int cols, int batch, int nrb,
                          bool sub_identity, double* part, hipStream_t s) {
  const int rpb = rows_per(rows, nrb);
  dim3 grid(nrb, batch);
  if (x_dtype == MAO_BF16)
    hipLaunchKernelGGL(sumsq_partial_kernel<bf16_t>, grid, dim3(kObs), 0, s, X, rows, cols, rpb,
                       nrb, sub_identity ? 1 : 0, part);
  else
    hipLaunchKernelGGL(sumsq_partial_kernel<float>, grid, dim3(kObs), 0, s, X, rows, cols, rpb,
                       nrb, sub_identity ? 1 : 0, part);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status finalize_rms(const double* part, int nrb, int batch, double divisor, float* out,
                        hipStream_t s) {
  hipLaunchKernelGGL(finalize_rms_kernel, dim3(batch), dim3(kObs), 0, s, part, nrb, divisor, out);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status row_dots(View A, View B, int n, int cols, float* d, hipStream_t s) {
  hipLaunchKernelGGL(row_dots_kernel, dim3((n + 3) / 4), dim3(kObs), 0, s, A, B, n, cols, d);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status kappa_of(const float* d, int n, float* kappa, hipStream_t s) {
  hipLaunchKernelGGL(kappa_kernel, dim3(1), dim3(1024), 0, s, d, n, kappa);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status gemv_rows(View V, int m, int n, const float* x, float* y, hipStream_t s) {
  hipLaunchKernelGGL(gemv_rows_kernel, dim3((m + 3) / 4), dim3(kObs), 0, s, V, m, n, x, y);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status gemv_cols(View V, int m, int n, const float* y, float* part, int nrb, float* z,
                     hipStream_t s) {
  const int rpb = rows_per(m, nrb);
  hipLaunchKernelGGL(gemv_cols_partial_kernel, dim3(nrb, (n + 4 * kObs - 1) / (4 * kObs)),
                     dim3(kObs), 0, s, V, m, n, rpb, y, part);
  MAO_LAUNCH_CHECK();
  hipLaunchKernelGGL(gemv_cols_final_kernel, dim3((n + 63) / 64), dim3(kObs), 0, s, part, nrb, n,
                     z);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status normalize_vec(float* v, int n, hipStream_t s) {
  hipLaunchKernelGGL(normalize_kernel, dim3(1), dim3(1024), 0, s, v, n);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status fill_unit(float* v, int n, hipStream_t s) {
  hipLaunchKernelGGL(fill_unit_kernel, dim3((n + kObs - 1) / kObs), dim3(kObs), 0, s, v, n);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status share_of(const float* y, int m, const double* vpart, int nrb, float* out,
                    hipStream_t s) {
  hipLaunchKernelGGL(share_kernel, dim3(1), dim3(1024), 0, s, y, m, vpart, nrb, out);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status basis_age(const float* aux, float* age, hipStream_t s) {
  hipLaunchKernelGGL(basis_age_kernel, dim3(1), dim3(1), 0, s, aux, age);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

}  // namespace mao
