// Memory-bound passes: EMAs, norms, Muon+ scaling, rotated-space Adam,
// FOAM's factored moment, weight updates and transposes.
//
// Access pattern: every pass streams row-major matrices in 4-element chunks
// (16-byte fp32 / 8-byte bf16 vector accesses; leading dimensions are
// multiples of 8 elements, so chunk addresses are aligned), with a block
// owning a contiguous range of rows of one matrix of a batch (blockIdx.y).
// Reductions write one partial per block and a second pass sums the
// partials in a fixed order: no atomics, bitwise-repeatable results.
#include "elementwise.hpp"
#include "tiled.hpp"

#include <algorithm>

namespace mao {

namespace {

constexpr int kBlock = 256;

template <typename T> struct Vec4;
template <> struct Vec4<float> {
  static __device__ __forceinline__ void load(const float* p, float v[4]) {
    float4 x = *(const float4*)p;
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
  static __device__ __forceinline__ void store(float* p, const float v[4]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct Vec4<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float v[4]) {
    uint2 u = *(const uint2*)p;
    v[0] = bf16_to_f32((bf16_t)(u.x & 0xffff));
    v[1] = bf16_to_f32((bf16_t)(u.x >> 16));
    v[2] = bf16_to_f32((bf16_t)(u.y & 0xffff));
    v[3] = bf16_to_f32((bf16_t)(u.y >> 16));
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float v[4]) {
    uint2 u;
    u.x = pack_bf16x2(v[0], v[1]);
    u.y = pack_bf16x2(v[2], v[3]);
    *(uint2*)p = u;
  }
};

// Load up to 4 elements starting at column j of a row with `cols` columns.
template <typename T>
__device__ __forceinline__ void load4(const T* row, int j, int cols, float v[4]) {
  if (j + 4 <= cols) {
    Vec4<T>::load(row + j, v);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (j + e < cols) ? load_f32<T>(row + j + e) : 0.f;
  }
}

template <typename T>
__device__ __forceinline__ void store4(T* row, int j, int cols, const float v[4]) {
  if (j + 4 <= cols) {
    Vec4<T>::store(row + j, v);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e < cols) store_f32<T>(row + j + e, v[e]);
  }
}

// 8 consecutive elements starting at column j (a multiple of 8) of a row with
// `cols` columns: 2 x 16-byte (fp32) or one 16-byte (bf16) access, element
// by element at the ragged end.
template <typename T>
__device__ __forceinline__ void load8(const T* row, int j, int cols, float v[8]) {
  if (j + 8 <= cols) {
    if constexpr (sizeof(T) == 4) {
      Vec4<float>::load((const float*)row + j, v);
      Vec4<float>::load((const float*)row + j + 4, v + 4);
    } else {
      const uint4 u = *(const uint4*)(row + j);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_to_f32((bf16_t)(w[e] & 0xffff));
        v[2 * e + 1] = bf16_to_f32((bf16_t)(w[e] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (j + e < cols) ? load_f32<T>(row + j + e) : 0.f;
  }
}

template <typename T>
__device__ __forceinline__ void store8(T* row, int j, int cols, const float v[8]) {
  if (j + 8 <= cols) {
    if constexpr (sizeof(T) == 4) {
      Vec4<float>::store((float*)row + j, v);
      Vec4<float>::store((float*)row + j + 4, v + 4);
    } else {
      uint4 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      u.z = pack_bf16x2(v[4], v[5]);
      u.w = pack_bf16x2(v[6], v[7]);
      *(uint4*)(row + j) = u;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (j + e < cols) store_f32<T>(row + j + e, v[e]);
  }
}

// 8 fp32 values from p[j..j+7] that may not be 16-byte aligned (per-matrix
// vectors at a stride of cols elements): vector loads when aligned, else
// element by element; zero past cols.
__device__ __forceinline__ void load8_f32_any(const float* p, int j, int cols, float v[8]) {
  if (j + 8 <= cols && ((uintptr_t)(p + j) & 15) == 0) {
    load8<float>(p, j, cols, v);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (j + e < cols) ? p[j + e] : 0.f;
  }
}

// Row range of this block for a matrix split into nrb row-blocks.
__device__ __forceinline__ void row_range(int rows, int nrb, int& r0, int& r1) {
  const int per = (rows + nrb - 1) / nrb;
  r0 = blockIdx.x * per;
  r1 = min(rows, r0 + per);
}

// ---------------------------------------------------------------------------

// The 8-column chunks of this block's rows, numbered row by row: chunk q is
// row r0 + q / c8, columns 8 (q % c8) .. + 7 (32-bit arithmetic).
struct Chunks {
  int r0;
  unsigned c8, n;
  __device__ __forceinline__ void at(unsigned q, int& i, int& j) const {
    const unsigned ii = q / c8;
    i = r0 + (int)ii;
    j = (int)(q - ii * c8) * 8;
  }
};

__device__ __forceinline__ Chunks block_chunks(int rows, int cols, int nrb) {
  int r0, r1;
  row_range(rows, nrb, r0, r1);
  Chunks c;
  c.r0 = r0;
  c.c8 = (unsigned)((cols + 7) >> 3);
  c.n = (unsigned)max(0, r1 - r0) * c.c8;
  return c;
}

template <typename TG>
__global__ __launch_bounds__(kBlock) void ema_sumsq_kernel(View M, View G, int rows, int cols,
                                                           float beta, float* partial, int nrb) {
  const int b = blockIdx.y;
  float* Mb = (float*)M.p + (int64_t)b * M.stride;
  const TG* Gb = (const TG*)G.p + (int64_t)b * G.stride;
  const Chunks ch = block_chunks(rows, cols, nrb);
  const float om = 1.f - beta;
  float acc = 0.f;
#pragma unroll 2
  for (unsigned q = threadIdx.x; q < ch.n; q += kBlock) {
    int i, j;
    ch.at(q, i, j);
    float m[8], g[8];
    float* mrow = Mb + (int64_t)i * M.ld;
    load8<float>(mrow, j, cols, m);
    load8<TG>(Gb + (int64_t)i * G.ld, j, cols, g);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      m[e] = beta * m[e] + om * g[e];
      acc += m[e] * m[e];
    }
    store8<float>(mrow, j, cols, m);
  }
  if (partial) {
    __shared__ float sc[16];
    const float tot = block_sum(acc, sc);
    if (threadIdx.x == 0) partial[(int64_t)b * nrb + blockIdx.x] = tot;
  }
}

// One block per matrix: fixed-order sum of the per-block partials.
__global__ __launch_bounds__(kBlock) void finalize_inv_norm_kernel(const float* partial, int nrb,
                                                                   float eps, float* scale) {
  const int b = blockIdx.x;
  double s = 0.0;
  for (int i = threadIdx.x; i < nrb; i += kBlock) s += (double)partial[(int64_t)b * nrb + i];
  __shared__ double sc[16];
  s = block_sum_d(s, sc);
  if (threadIdx.x == 0) scale[b] = (float)(1.0 / (sqrt(s) + (double)eps));
}

// 64 x 64 tiles through LDS: direct copy and transposed copy, optional scale.
template <typename TI, typename TO>
__global__ __launch_bounds__(kBlock) void transpose_kernel(View In, int rows, int cols,
                                                           const float* scale, View Dir, View Tr) {
  __shared__ float tile[64][65];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const float s = scale ? scale[b] : 1.f;
  const TI* in = (const TI*)In.p + (int64_t)b * In.stride;
  TO* dir = Dir.p ? (TO*)Dir.p + (int64_t)b * Dir.stride : nullptr;
  TO* tr = Tr.p ? (TO*)Tr.p + (int64_t)b * Tr.stride : nullptr;
  const int t = threadIdx.x;
  const int cc = (t & 15) * 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = (t >> 4) + 16 * p;
    const int i = i0 + r, j = j0 + cc;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < rows && j < cols) {
      load4<TI>(in + (int64_t)i * In.ld, j, cols, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= s;
      if (dir) store4<TO>(dir + (int64_t)i * Dir.ld, j, cols, v);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[r][cc + e] = v[e];
  }
  if (!tr) return;
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = (t >> 4) + 16 * p;  // original column
    const int jj = j0 + c, ii = i0 + cc;
    if (jj < cols && ii < rows) {
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[cc + e][c];
      store4<TO>(tr + (int64_t)jj * Tr.ld, ii, rows, v);
    }
  }
}

// Direct-only variant of transpose_kernel: out = scale * in, cast.
template <typename TI, typename TO>
__global__ __launch_bounds__(kBlock) void scale_cast_kernel(View In, int rows, int cols,
                                                            const float* scale, View Out, int nrb) {
  const int b = blockIdx.y;
  const TI* in = (const TI*)In.p + (int64_t)b * In.stride;
  TO* out = (TO*)Out.p + (int64_t)b * Out.stride;
  const float sc = scale ? scale[b] : 1.f;
  const Chunks ch = block_chunks(rows, cols, nrb);
#pragma unroll 2
  for (unsigned q = threadIdx.x; q < ch.n; q += kBlock) {
    int i, j;
    ch.at(q, i, j);
    float v[8];
    load8<TI>(in + (int64_t)i * In.ld, j, cols, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] *= sc;
    store8<TO>(out + (int64_t)i * Out.ld, j, cols, v);
  }
}

// X0 = scale * M (or its transpose) cast to bf16 in the tiled layout
// (tiled.hpp), pad zero: a 64 x 64 region of X per block through LDS, then
// written as whole 1 KB half-blocks (thread q of a 128-chunk block writes its
// q-th 16-byte chunk, so consecutive lanes write consecutive addresses).
__global__ __launch_bounds__(kBlock) void x0_tiled_kernel(View In, int rows, int cols,
                                                          const float* scale, bool trans,
                                                          bf16_t* X, int64_t xcp, int64_t xstride) {
  __shared__ float tile[64][65];
  const int b = blockIdx.z;
  const int i0 = blockIdx.y * 64, k0 = blockIdx.x * 64;  // region of X
  const int sr0 = trans ? k0 : i0, sc0 = trans ? i0 : k0;  // region of M
  const float s = scale ? scale[b] : 1.f;
  const float* in = (const float*)In.p + (int64_t)b * In.stride;
  const int t = threadIdx.x;
  const int cc = (t & 15) * 4;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = (t >> 4) + 16 * p;
    const int i = sr0 + r, j = sc0 + cc;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < rows && j < cols) {
      load4<float>(in + (int64_t)i * In.ld, j, cols, v);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] *= s;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[r][cc + e] = v[e];
  }
  __syncthreads();
  bf16_t* xb = X + (int64_t)b * xstride;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int q = t + p * kBlock;            // chunk of the region, 0..511
    const int blk = q >> 7, r = (q >> 2) & 31, pc = q & 3;
    const int lc = pc ^ t32_swz(r);          // logical chunk stored at pc
    const int ri = (blk >> 1) * 32 + r;      // row of X in the region
    const int ck = (blk & 1) * 32 + lc * 8;  // first column of X in the region
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = trans ? tile[ck + e][ri] : tile[ri][ck + e];
    uint4 pk;
    pk.x = pack_bf16x2(v[0], v[1]);
    pk.y = pack_bf16x2(v[2], v[3]);
    pk.z = pack_bf16x2(v[4], v[5]);
    pk.w = pack_bf16x2(v[6], v[7]);
    *(uint4*)(xb + t32_off(i0 + ri, k0 + ck, xcp)) = pk;
  }
}

template <typename TX>
__global__ __launch_bounds__(kBlock) void row_sumsq_kernel(View X, int rows, int cols,
                                                           const float* w, float* ss) {
  const int b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  if (i >= rows) return;
  const TX* row = (const TX*)X.p + (int64_t)b * X.stride + (int64_t)i * X.ld;
  const float* wb = w ? w + (int64_t)b * cols : nullptr;
  float acc = 0.f;
  // one wavefront per row, 8 consecutive elements per lane and step (16- or
  // 32-byte loads, weights as two 16-byte loads), four steps in flight
#pragma unroll 4
  for (int j = lane * 8; j < cols; j += 512) {
    float v[8];
    load8<TX>(row, j, cols, v);
    if (wb) {
      float wt[8];
      load8_f32_any(wb, j, cols, wt);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += wt[e] * v[e] * v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += v[e] * v[e];
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) ss[(int64_t)b * rows + i] = acc;
}

__global__ __launch_bounds__(kBlock) void equalise_kernel(const float* ss, int n, float eps,
                                                          float* scale, float* sq) {
  const int b = blockIdx.x;
  const float* s = ss + (int64_t)b * n;
  float acc = 0.f;
  for (int j = threadIdx.x; j < n; j += kBlock) acc += s[j];
  __shared__ float sc[16];
  const float tot = block_sum(acc, sc);
  const float target = sqrtf(tot / (float)n);
  for (int j = threadIdx.x; j < n; j += kBlock) {
    const float v = target / (sqrtf(s[j]) + eps);
    scale[(int64_t)b * n + j] = v;
    if (sq) sq[(int64_t)b * n + j] = v * v;
  }
}

template <typename TW, typename TO>
__global__ __launch_bounds__(kBlock) void update_kernel(View W, View O, int rows, int cols,
                                                        float lr, float wd, float s,
                                                        const float* rs, const float* cs,
                                                        View Out, int nrb) {
  const int b = blockIdx.y;
  TW* Wb = (TW*)W.p + (int64_t)b * W.stride;
  const TO* Ob = (const TO*)O.p + (int64_t)b * O.stride;
  float* outb = Out.p ? (float*)Out.p + (int64_t)b * Out.stride : nullptr;
  const float* rsb = rs ? rs + (int64_t)b * rows : nullptr;
  const float* csb = cs ? cs + (int64_t)b * cols : nullptr;
  const Chunks ch = block_chunks(rows, cols, nrb);
#pragma unroll 2
  for (unsigned q = threadIdx.x; q < ch.n; q += kBlock) {
    int i, j;
    ch.at(q, i, j);
    float w[8], o[8];
    TW* wrow = Wb + (int64_t)i * W.ld;
    load8<TW>(wrow, j, cols, w);
    load8<TO>(Ob + (int64_t)i * O.ld, j, cols, o);
    const float si = s * (rsb ? rsb[i] : 1.f);
    float cj[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
    if (csb) load8_f32_any(csb, j, cols, cj);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      o[e] = si * cj[e] * o[e];
      w[e] = w[e] - lr * (wd * w[e] + o[e]);
    }
    store8<TW>(wrow, j, cols, w);
    if (outb) store8<float>(outb + (int64_t)i * Out.ld, j, cols, o);
  }
}

// N goes over Gt (TN = float) or to a separate bf16 copy (TN = bf16_t).
template <typename TN>
__global__ __launch_bounds__(kBlock) void soap_adam_kernel(View Gt, View Mt, View V, View Nout,
                                                           int rows, int cols, float beta2,
                                                           float bc1, float bc2, float eps,
                                                           int nrb) {
  const Chunks ch = block_chunks(rows, cols, nrb);
  const float ob = 1.f - beta2, ib1 = 1.f / bc1, ib2 = 1.f / bc2;
#pragma unroll 2
  for (unsigned q = threadIdx.x; q < ch.n; q += kBlock) {
    int i, j;
    ch.at(q, i, j);
    float g[8], m[8], v[8];
    const float* grow = (const float*)Gt.p + (int64_t)i * Gt.ld;
    float* vrow = (float*)V.p + (int64_t)i * V.ld;
    load8<float>(grow, j, cols, g);
    load8<float>((const float*)Mt.p + (int64_t)i * Mt.ld, j, cols, m);
    load8<float>(vrow, j, cols, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = beta2 * v[e] + ob * g[e] * g[e];
      g[e] = (m[e] * ib1) / (sqrtf(v[e] * ib2) + eps);
    }
    store8<float>(vrow, j, cols, v);
    store8<TN>((TN*)Nout.p + (int64_t)i * Nout.ld, j, cols, g);
  }
}

// fp32-accurate products on bf16 MFMA: X = hi + lo with hi = bf16(X),
// lo = bf16(X - hi); a row of K elements becomes 3K (or 2K) bf16 in one of
// three orders: kSplitA [hi | lo | hi], kSplitB [hi | hi | lo] (so that
// A3 B3^T = hi_a hi_b^T + lo_a hi_b^T + hi_a lo_b^T), kSplitDup [x | x] for an
// operand already exact in bf16 (against the last 2K of a kSplitB operand).
template <typename TI>
__global__ __launch_bounds__(kBlock) void split3_kernel(View In, int rows, int K, int Kp, View Out,
                                                        int layout, int nrb) {
  const Chunks ch = block_chunks(rows, Kp, nrb);
#pragma unroll 2
  for (unsigned q = threadIdx.x; q < ch.n; q += kBlock) {
    int i, j;
    ch.at(q, i, j);
    float x[8], hi[8], lo[8];
    load8<TI>((const TI*)In.p + (int64_t)i * In.ld, j, K, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      hi[e] = bf16_to_f32(f32_to_bf16(x[e]));
      lo[e] = x[e] - hi[e];
    }
    // columns K..Kp read as zero and are stored as zero (segment padding)
    bf16_t* out = (bf16_t*)Out.p + (int64_t)i * Out.ld;
    if (layout == kSplitDup) {
      store8<bf16_t>(out, j, Kp, x);
      store8<bf16_t>(out + Kp, j, Kp, x);
    } else {
      store8<bf16_t>(out, j, Kp, hi);
      store8<bf16_t>(out + Kp, j, Kp, layout == kSplitA ? lo : hi);
      store8<bf16_t>(out + 2 * Kp, j, Kp, layout == kSplitA ? hi : lo);
    }
  }
}

__global__ __launch_bounds__(kBlock) void fill_identity_kernel(View E, int n, const int* pred) {
  if (pred && *pred == 0) return;
  const int64_t total = (int64_t)n * n;
  for (int64_t q = blockIdx.x * (int64_t)kBlock + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * kBlock) {
    const int i = (int)(q / n), j = (int)(q % n);
    ((float*)E.p)[(int64_t)i * E.ld + j] = (i == j) ? 1.f : 0.f;
  }
}

__global__ __launch_bounds__(kBlock) void fill_kernel(float* p, int64_t n, float v) {
  for (int64_t q = blockIdx.x * (int64_t)kBlock + threadIdx.x; q < n; q += (int64_t)gridDim.x * kBlock)
    p[q] = v;
}

// ---- FOAM factored moment -------------------------------------------------

__global__ __launch_bounds__(kBlock) void col_partial_kernel(View X, int rows, int cols, int nrb,
                                                             float* colpart) {
  const int j = blockIdx.x * kBlock + threadIdx.x;
  if (j >= cols) return;
  int r0, r1;
  const int per = (rows + nrb - 1) / nrb;
  r0 = blockIdx.y * per;
  r1 = min(rows, r0 + per);
  float acc = 0.f;
  for (int i = r0; i < r1; ++i) {
    const float v = ((const float*)X.p)[(int64_t)i * X.ld + j];
    acc += v * v;
  }
  colpart[(int64_t)blockIdx.y * cols + j] = acc;
}

// Factored moment, wide pass. Workgroup b < nbr: r_i <- beta2 r_i + (1 -
// beta2) rowss_i / n over rows [256 b, 256 b + 256) and the sum of the new
// r there; workgroup nbr + b: c_j <- beta2 c_j + (1 - beta2) colsum_j / m
// over columns [256 b, 256 b + 256), colsum_j summed from the row-block
// partials in block order, and the sums of the new c and of diag(R) there.
__global__ __launch_bounds__(256) void foam_rc_kernel(const float* rowss, const float* colpart,
                                                      int nrb, int m, int n, float beta2,
                                                      const float* R, int64_t ldR, float* r,
                                                      float* c, float* bp, int nbr, int nbc) {
  __shared__ float sc[4];
  const float ob = 1.f - beta2;
  const int b = blockIdx.x;
  if (b < nbr) {
    const int i = b * 256 + threadIdx.x;
    float v = 0.f;
    if (i < m) {
      v = beta2 * r[i] + ob * (rowss[i] / (float)n);
      r[i] = v;
    }
    v = block_sum(v, sc);
    if (threadIdx.x == 0) bp[b] = v;
    return;
  }
  const int cb = b - nbr;
  const int j = cb * 256 + threadIdx.x;
  float v = 0.f, d = 0.f;
  if (j < n) {
    float s = 0.f;
    for (int k = 0; k < nrb; ++k) s += colpart[(int64_t)k * n + j];
    v = beta2 * c[j] + ob * (s / (float)m);
    c[j] = v;
    d = R[(int64_t)j * ldR + j];
  }
  v = block_sum(v, sc);
  d = block_sum(d, sc);
  if (threadIdx.x == 0) {
    bp[nbr + cb] = v;
    bp[nbr + nbc + cb] = d;
  }
}

// tau = (tr(R) / bc2) / ((sum r / bc2) (sum c / bc2)) from the wide pass's
// block sums, added in block order (0 when the denominator is 0).
__global__ __launch_bounds__(64) void foam_tau_kernel(const float* bp, int nbr, int nbc,
                                                      float bc2, float* tau_out, float* aux) {
  if (threadIdx.x != 0) return;
  double sr = 0.0, scs = 0.0, tr = 0.0;
  for (int b = 0; b < nbr; ++b) sr += bp[b];
  for (int b = 0; b < nbc; ++b) {
    scs += bp[nbr + b];
    tr += bp[nbr + nbc + b];
  }
  const double denom = (sr / bc2) * (scs / bc2);
  const float tau = denom > 0.0 ? (float)((tr / bc2) / denom) : 0.f;
  tau_out[0] = tau;
  if (aux) aux[2] = tau;
}

template <typename TN>
__global__ __launch_bounds__(kBlock) void foam_precond_kernel(View Mr, View Nout, int m, int n,
                                                              const float* r, const float* c,
                                                              const float* tau, float bc1,
                                                              float bc2, float eps, int nrb) {
  const Chunks ch = block_chunks(m, n, nrb);
  const float t = tau[0], ib1 = 1.f / bc1, ib2 = 1.f / bc2;
#pragma unroll 2
  for (unsigned q = threadIdx.x; q < ch.n; q += kBlock) {
    int i, j;
    ch.at(q, i, j);
    float* row = (float*)Mr.p + (int64_t)i * Mr.ld;
    float x[8];
    load8<float>(row, j, n, x);
    const float ri = r[i] * ib2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float cj = (j + e < n) ? c[j + e] * ib2 : 0.f;
      x[e] = (x[e] * ib1) / (sqrtf(t * ri * cj) + eps);
    }
    store8<TN>((TN*)Nout.p + (int64_t)i * Nout.ld, j, n, x);
  }
}

__global__ __launch_bounds__(kBlock) void offdiag_rows_kernel(View D, int n, float* work) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);
  if (i >= n) return;
  const float* row = (const float*)D.p + (int64_t)i * D.ld;
  float off = 0.f;
  for (int j = lane * 4; j < n; j += 256) {
    float v[4];
    load4<float>(row, j, n, v);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j + e != i) off += v[e] * v[e];
  }
  off = wave_sum(off);
  if (lane == 0) {
    const float d = row[i];
    work[i] = off;
    work[n + i] = d * d;
  }
}

__global__ __launch_bounds__(1024) void offdiag_final_kernel(const float* work, int n, float tol,
                                                             float* aux, int* flag) {
  __shared__ double sc[16];
  double off = 0.0, dg = 0.0;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    off += work[i];
    dg += work[n + i];
  }
  off = block_sum_d(off, sc);
  dg = block_sum_d(dg, sc);
  if (threadIdx.x == 0) {
    const double total = off + dg;
    const float rho = total > 0.0 ? (float)sqrt(off / total) : 0.f;
    const int f = rho > tol ? 1 : 0;
    aux[0] = rho;
    aux[1] = (float)f;
    aux[3] = 1.f;
    *flag = f;
  }
}

__global__ void no_check_kernel(float* aux, int* flag) {
  aux[1] = 0.f;
  aux[3] = 0.f;
  *flag = 0;
}

template <typename TW, typename TG>
__global__ __launch_bounds__(kBlock) void adamw_kernel(TW* w, const TG* g, float* m, float* v,
                                                       int64_t n, float lr, float beta1,
                                                       float beta2, float bc1, float bc2,
                                                       float eps, float wd, float* out) {
  const int64_t n4 = (n + 3) >> 2;
  const float ob1 = 1.f - beta1, ob2 = 1.f - beta2, ib1 = 1.f / bc1, ib2 = 1.f / bc2;
  for (int64_t q = blockIdx.x * (int64_t)kBlock + threadIdx.x; q < n4;
       q += (int64_t)gridDim.x * kBlock) {
    const int64_t base = q * 4;
    const int cnt = (int)min((int64_t)4, n - base);
    float ww[4], gg[4], mm[4], vv[4];
    load4<TW>(w + base, 0, cnt, ww);
    load4<TG>(g + base, 0, cnt, gg);
    load4<float>(m + base, 0, cnt, mm);
    load4<float>(v + base, 0, cnt, vv);
    float uu[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mm[e] = beta1 * mm[e] + ob1 * gg[e];
      vv[e] = beta2 * vv[e] + ob2 * gg[e] * gg[e];
      uu[e] = (mm[e] * ib1) / (sqrtf(vv[e] * ib2) + eps);
      ww[e] = ww[e] - lr * (wd * ww[e] + uu[e]);
    }
    store4<TW>(w + base, 0, cnt, ww);
    store4<float>(m + base, 0, cnt, mm);
    store4<float>(v + base, 0, cnt, vv);
    if (out) store4<float>(out + base, 0, cnt, uu);
  }
}

int grid_for(int64_t work, int per_block = 4 * kBlock) {
  int64_t g = (work + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 8192) g = 8192;
  return (int)g;
}

}  // namespace

int rowblocks_for(int64_t rows, int64_t batch) {
  // about 8192 blocks over the whole batch, at least one row each (measured
  // 3-4% faster on the streaming passes than 2048)
  int64_t want = (8192 + batch - 1) / batch;
  if (want < 1) want = 1;
  if (want > rows) want = rows;
  if (want > 65535) want = 65535;
  return (int)want;
}

mao_status ema_sumsq(View M, View G, int g_dtype, int rows, int cols, int batch, float beta,
                     float* partial, int nrb, hipStream_t s) {
  dim3 grid(nrb, batch);
  if (g_dtype == MAO_BF16)
    hipLaunchKernelGGL(ema_sumsq_kernel<bf16_t>, grid, dim3(kBlock), 0, s, M, G, rows, cols, beta, partial, nrb);
  else
    hipLaunchKernelGGL(ema_sumsq_kernel<float>, grid, dim3(kBlock), 0, s, M, G, rows, cols, beta, partial, nrb);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status finalize_inv_norm(const float* partial, int nrb, int batch, float eps, float* scale,
                             hipStream_t s) {
  hipLaunchKernelGGL(finalize_inv_norm_kernel, dim3(batch), dim3(kBlock), 0, s, partial, nrb, eps, scale);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status scale_cast_transpose(View M, int rows, int cols, int batch, const float* scale,
                                View direct, View trans, int x_dtype, hipStream_t s) {
  if (trans.p == nullptr) {
    if (direct.p == nullptr) return MAO_OK;
    const int nrb = rowblocks_for(rows, batch);
    if (x_dtype == MAO_BF16)
      hipLaunchKernelGGL((scale_cast_kernel<float, bf16_t>), dim3(nrb, batch), dim3(kBlock), 0, s, M, rows, cols, scale, direct, nrb);
    else
      hipLaunchKernelGGL((scale_cast_kernel<float, float>), dim3(nrb, batch), dim3(kBlock), 0, s, M, rows, cols, scale, direct, nrb);
    MAO_LAUNCH_CHECK();
    return MAO_OK;
  }
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  if (x_dtype == MAO_BF16)
    hipLaunchKernelGGL((transpose_kernel<float, bf16_t>), grid, dim3(kBlock), 0, s, M, rows, cols, scale, direct, trans);
  else
    hipLaunchKernelGGL((transpose_kernel<float, float>), grid, dim3(kBlock), 0, s, M, rows, cols, scale, direct, trans);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status scale_cast_tiled(View M, int rows, int cols, int batch, const float* scale, bool trans,
                            void* X, int64_t xrp, int64_t xcp, int64_t xstride, hipStream_t s) {
  const int64_t a = trans ? cols : rows, bb = trans ? rows : cols;
  if (xrp % 64 || xcp % 256 || xrp < a || xcp < bb) {
    set_error("scale_cast_tiled: padded %lld x %lld does not hold %lld x %lld", (long long)xrp,
              (long long)xcp, (long long)a, (long long)bb);
    return MAO_E_LAYOUT;
  }
  dim3 grid((unsigned)(xcp / 64), (unsigned)(xrp / 64), batch);
  hipLaunchKernelGGL(x0_tiled_kernel, grid, dim3(kBlock), 0, s, M, rows, cols, scale, trans,
                     (bf16_t*)X, xcp, xstride);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status cast_transpose_f32(View in, int in_dtype, int rows, int cols, View direct, View trans,
                              hipStream_t s) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, 1);
  if (in_dtype == MAO_BF16)
    hipLaunchKernelGGL((transpose_kernel<bf16_t, float>), grid, dim3(kBlock), 0, s, in, rows, cols, (const float*)nullptr, direct, trans);
  else
    hipLaunchKernelGGL((transpose_kernel<float, float>), grid, dim3(kBlock), 0, s, in, rows, cols, (const float*)nullptr, direct, trans);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status transpose(View in, View out, int rows, int cols, int batch, int dtype, hipStream_t s) {
  dim3 grid((cols + 63) / 64, (rows + 63) / 64, batch);
  View none = view(nullptr, 0, 0);
  if (dtype == MAO_BF16)
    hipLaunchKernelGGL((transpose_kernel<bf16_t, bf16_t>), grid, dim3(kBlock), 0, s, in, rows, cols, (const float*)nullptr, none, out);
  else
    hipLaunchKernelGGL((transpose_kernel<float, float>), grid, dim3(kBlock), 0, s, in, rows, cols, (const float*)nullptr, none, out);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status row_sumsq(View X, int x_dtype, int rows, int cols, int batch, const float* w,
                     float* ss, hipStream_t s) {
  dim3 grid((rows + 3) / 4, batch);
  if (x_dtype == MAO_BF16)
    hipLaunchKernelGGL(row_sumsq_kernel<bf16_t>, grid, dim3(kBlock), 0, s, X, rows, cols, w, ss);
  else
    hipLaunchKernelGGL(row_sumsq_kernel<float>, grid, dim3(kBlock), 0, s, X, rows, cols, w, ss);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status equalise_scales(const float* ss, int n, int batch, float eps, float* scale, float* sq,
                           hipStream_t s) {
  hipLaunchKernelGGL(equalise_kernel, dim3(batch), dim3(kBlock), 0, s, ss, n, eps, scale, sq);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status apply_update(View W, int w_dtype, View O, int o_dtype, int rows, int cols, int batch,
                        float lr, float wd, float sc, const float* rs, const float* cs, View out,
                        hipStream_t s) {
  const int nrb = rowblocks_for(rows, batch);
  dim3 grid(nrb, batch);
#define MAO_UPD(TW, TO)                                                                    \
  hipLaunchKernelGGL((update_kernel<TW, TO>), grid, dim3(kBlock), 0, s, W, O, rows, cols, lr, \
                     wd, sc, rs, cs, out, nrb)
  if (w_dtype == MAO_BF16 && o_dtype == MAO_BF16) MAO_UPD(bf16_t, bf16_t);
  else if (w_dtype == MAO_BF16) MAO_UPD(bf16_t, float);
  else if (o_dtype == MAO_BF16) MAO_UPD(float, bf16_t);
  else MAO_UPD(float, float);
#undef MAO_UPD
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status soap_adam(View Gt, View Mt, View V, int rows, int cols, float beta2, float bc1,
                     float bc2, float eps, hipStream_t s, View Nb) {
  const int nrb = rowblocks_for(rows, 1);
  if (Nb.p != nullptr)
    hipLaunchKernelGGL(soap_adam_kernel<bf16_t>, dim3(nrb), dim3(kBlock), 0, s, Gt, Mt, V, Nb, rows, cols, beta2, bc1, bc2, eps, nrb);
  else
    hipLaunchKernelGGL(soap_adam_kernel<float>, dim3(nrb), dim3(kBlock), 0, s, Gt, Mt, V, Gt, rows, cols, beta2, bc1, bc2, eps, nrb);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status split3_bf16(View In, int in_dtype, int rows, int K, View Out, int layout, hipStream_t s) {
  const int Kp = (int)split_width(K);
  const int nrb = rowblocks_for(rows, 1);
  if (in_dtype == MAO_BF16)
    hipLaunchKernelGGL(split3_kernel<bf16_t>, dim3(nrb), dim3(kBlock), 0, s, In, rows, K, Kp, Out, layout, nrb);
  else
    hipLaunchKernelGGL(split3_kernel<float>, dim3(nrb), dim3(kBlock), 0, s, In, rows, K, Kp, Out, layout, nrb);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status fill_identity(View E, int n, const int* pred, hipStream_t s) {
  hipLaunchKernelGGL(fill_identity_kernel, dim3(grid_for((int64_t)n * n)), dim3(kBlock), 0, s, E, n, pred);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  hipLaunchKernelGGL(fill_kernel, dim3(grid_for(n)), dim3(kBlock), 0, s, p, n, v);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status foam_moments(View Gr, int m, int n, float beta2, float bc2, const float* R, int64_t ldR,
                        float* r, float* c, float* work, float* tau_out, float* aux,
                        hipStream_t s) {
  // work: rowss[m], colpart[nrb * n], then the wide pass's block sums
  float* rowss = work;
  float* colpart = work + round_up(m, 64);
  const int nrb = (int)std::min<int64_t>(64, std::max<int64_t>(1, m / 32));
  float* bp = colpart + round_up((int64_t)nrb * n, 64);
  const int nbr = (m + 255) / 256, nbc = (n + 255) / 256;
  hipLaunchKernelGGL(row_sumsq_kernel<float>, dim3((m + 3) / 4, 1), dim3(kBlock), 0, s, Gr, m, n, (const float*)nullptr, rowss);
  MAO_LAUNCH_CHECK();
  hipLaunchKernelGGL(col_partial_kernel, dim3((n + kBlock - 1) / kBlock, nrb), dim3(kBlock), 0, s, Gr, m, n, nrb, colpart);
  MAO_LAUNCH_CHECK();
  hipLaunchKernelGGL(foam_rc_kernel, dim3(nbr + nbc), dim3(256), 0, s, rowss, colpart, nrb, m, n, beta2, R, ldR, r, c, bp, nbr, nbc);
  MAO_LAUNCH_CHECK();
  hipLaunchKernelGGL(foam_tau_kernel, dim3(1), dim3(64), 0, s, bp, nbr, nbc, bc2, tau_out, aux);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

int64_t foam_moments_work_floats(int m, int n) {
  const int nrb = (int)std::min<int64_t>(64, std::max<int64_t>(1, m / 32));
  return round_up(m, 64) + round_up((int64_t)nrb * n, 64) + (m + 255) / 256 + 2 * ((n + 255) / 256);
}

mao_status foam_precondition(View Mr, int m, int n, const float* r, const float* c,
                             const float* tau, float bc1, float bc2, float eps, hipStream_t s,
                             View Nb) {
  const int nrb = rowblocks_for(m, 1);
  if (Nb.p != nullptr)
    hipLaunchKernelGGL(foam_precond_kernel<bf16_t>, dim3(nrb), dim3(kBlock), 0, s, Mr, Nb, m, n, r, c, tau, bc1, bc2, eps, nrb);
  else
    hipLaunchKernelGGL(foam_precond_kernel<float>, dim3(nrb), dim3(kBlock), 0, s, Mr, Mr, m, n, r, c, tau, bc1, bc2, eps, nrb);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status offdiag_check(View D, int n, float tol, float* work, float* aux, int* flag,
                         hipStream_t s) {
  hipLaunchKernelGGL(offdiag_rows_kernel, dim3((n + 3) / 4), dim3(kBlock), 0, s, D, n, work);
  MAO_LAUNCH_CHECK();
  hipLaunchKernelGGL(offdiag_final_kernel, dim3(1), dim3(1024), 0, s, work, n, tol, aux, flag);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status no_check(float* aux, int* flag, hipStream_t s) {
  hipLaunchKernelGGL(no_check_kernel, dim3(1), dim3(1), 0, s, aux, flag);
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

mao_status adamw(void* w, int w_dtype, const void* g, int g_dtype, float* m, float* v, int64_t n,
                 float lr, float beta1, float beta2, float bc1, float bc2, float eps, float wd,
                 float* out, hipStream_t s) {
  const int grid = grid_for((n + 3) / 4, kBlock);
#define MAO_ADAM(TW, TG)                                                                      \
  hipLaunchKernelGGL((adamw_kernel<TW, TG>), dim3(grid), dim3(kBlock), 0, s, (TW*)w,           \
                     (const TG*)g, m, v, n, lr, beta1, beta2, bc1, bc2, eps, wd, out)
  if (w_dtype == MAO_BF16 && g_dtype == MAO_BF16) MAO_ADAM(bf16_t, bf16_t);
  else if (w_dtype == MAO_BF16) MAO_ADAM(bf16_t, float);
  else if (g_dtype == MAO_BF16) MAO_ADAM(float, bf16_t);
  else MAO_ADAM(float, float);
#undef MAO_ADAM
  MAO_LAUNCH_CHECK();
  return MAO_OK;
}

}  // namespace mao
