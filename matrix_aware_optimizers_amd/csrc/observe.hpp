// Observability reductions over buffers the optimizer steps already hold:
// Frobenius RMS, ||X X^T - I||, Rayleigh quotients of a factor in its basis,
// the rank-1 share of a nonnegative second moment, basis age. All reductions
// are two-stage in a fixed order (bitwise repeatable).
#pragma once

#include "elementwise.hpp"

namespace mao {

// Row blocks per matrix of the sum-of-squares pass.
int obs_rowblocks(int64_t rows);

// part[b * nrb + blk] = sum over row block blk of matrix b of (X_ij - d_ij)^2,
// d_ij = [i == j] when sub_identity, else 0 (fp64 partials).
mao_status sumsq_partials(View X, int x_dtype, int rows, int cols, int batch, int nrb,
                          bool sub_identity, double* part, hipStream_t s);

// out[b] = sqrt(sum_blk part[b * nrb + blk] / divisor)
mao_status finalize_rms(const double* part, int nrb, int batch, double divisor, float* out,
                        hipStream_t s);

// d[i] = sum_k A[i][k] * B[i][k]  (fp32 rows, fp64 sums)
mao_status row_dots(View A, View B, int n, int cols, float* d, hipStream_t s);

// kappa[0] = max(d) / min(d), +inf when min(d) <= 0 (one workgroup)
mao_status kappa_of(const float* d, int n, float* kappa, hipStream_t s);

// Power-iteration building blocks on V (fp32 m x n):
// y = V x
mao_status gemv_rows(View V, int m, int n, const float* x, float* y, hipStream_t s);
// z = V^T y through nrb row-block partials in part (nrb * n floats)
mao_status gemv_cols(View V, int m, int n, const float* y, float* part, int nrb, float* z,
                     hipStream_t s);
// v <- v / ||v|| (left unchanged when ||v|| = 0)
mao_status normalize_vec(float* v, int n, hipStream_t s);
// v <- 1 / sqrt(n)
mao_status fill_unit(float* v, int n, hipStream_t s);
// out[0] = ||y||^2 / sum_blk vpart[blk] (0 when the denominator is 0)
mao_status share_of(const float* y, int m, const double* vpart, int nrb, float* out,
                    hipStream_t s);

// age[0] <- 0 if aux[1] != 0 (the step refreshed), else age[0] + 1
mao_status basis_age(const float* aux, float* age, hipStream_t s);

}  // namespace mao
