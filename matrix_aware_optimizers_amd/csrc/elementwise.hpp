// Memory-bound passes of the optimizer steps (EMA, norms, Muon+ scaling,
// Adam in the rotated basis, FOAM's factored moment, weight updates,
// transposes). All reductions are two-stage with a fixed order, so results
// are bitwise repeatable.
#pragma once

#include "common.hpp"

namespace mao {

// A strided batch of row-major matrices (element type given separately).
struct View {
  void* p;
  int64_t ld;      // elements
  int64_t stride;  // elements between consecutive matrices of the batch
};

inline View view(void* p, int64_t ld, int64_t stride = 0) { return View{p, ld, stride}; }

// Number of row-blocks per matrix used by the reduction passes.
int rowblocks_for(int64_t rows, int64_t batch);

// M <- beta M + (1 - beta) G (M fp32, G fp32/bf16); if partial != nullptr the
// per-block sums of the new M^2 go to partial[b * nrb + blk].
mao_status ema_sumsq(View M, View G, int g_dtype, int rows, int cols, int batch, float beta,
                     float* partial, int nrb, hipStream_t s);

// scale[b] = 1 / (sqrt(sum_blk partial[b*nrb + blk]) + eps)
mao_status finalize_inv_norm(const float* partial, int nrb, int batch, float eps, float* scale,
                             hipStream_t s);

// X0 = scale[b] * M cast to x_dtype: direct[i][j] = X0[i][j] and
// trans[j][i] = X0[i][j] (either may be nullptr).
mao_status scale_cast_transpose(View M, int rows, int cols, int batch, const float* scale,
                                View direct, View trans, int x_dtype, hipStream_t s);

// X0 = scale[b] * M (trans: its transpose), bf16, written tiled (tiled.hpp)
// into X of padded size xrp x xcp (xrp a multiple of 64, xcp of 256) with
// the pad zeroed; batch b at X + b * xstride.
mao_status scale_cast_tiled(View M, int rows, int cols, int batch, const float* scale, bool trans,
                            void* X, int64_t xrp, int64_t xcp, int64_t xstride, hipStream_t s);

// fp32 copies of a bf16 or fp32 matrix: direct[i][j] = in[i][j] and
// trans[j][i] = in[i][j] (either may be nullptr).
mao_status cast_transpose_f32(View in, int in_dtype, int rows, int cols, View direct, View trans,
                              hipStream_t s);

// Plain transpose out[j][i] = in[i][j] for fp32 or bf16 (same dtype in/out).
mao_status transpose(View in, View out, int rows, int cols, int batch, int dtype, hipStream_t s);

// ss[b*rows + i] = sum_j w[b*cols + j] * X[i][j]^2  (w may be nullptr = 1)
mao_status row_sumsq(View X, int x_dtype, int rows, int cols, int batch, const float* w,
                     float* ss, hipStream_t s);

// Muon+ scale vector: scale[b*n + j] = sqrt(sum(ss_b) / n) / (sqrt(ss[b*n+j]) + eps); the
// squares of the scales go to sq (for a following weighted pass) when non-null.
mao_status equalise_scales(const float* ss, int n, int batch, float eps, float* scale,
                           float* sq, hipStream_t s);

// W <- W - lr (wd W + s * rs[i] * cs[j] * O[i][j]); out[i][j] = s * rs * cs * O (fp32,
// dense per matrix: ld = cols, stride out_stride) when out != nullptr.
mao_status apply_update(View W, int w_dtype, View O, int o_dtype, int rows, int cols, int batch,
                        float lr, float wd, float s, const float* rs, const float* cs, View out,
                        hipStream_t st);

// SOAP Adam in the rotated space: V <- b2 V + (1-b2) Gt^2;
// N = (Mt / bc1) / (sqrt(V / bc2) + eps), written over Gt, or in bf16 to Nb
// when Nb.p is set (Gt then unchanged).
mao_status soap_adam(View Gt, View Mt, View V, int rows, int cols, float beta2, float bc1,
                     float bc2, float eps, hipStream_t s, View Nb = View{nullptr, 0, 0});

// bf16 split of a row-major rows x K matrix (fp32, or bf16 for kSplitDup)
// into Out (rows x 3 Kp, or 2 Kp for kSplitDup, Kp = split_width(K) = K
// rounded up to 8, the segments zero-padded; ld >= that): kSplitA = [hi | lo
// | hi], kSplitB = [hi | hi | lo], kSplitDup = [x | x]. A kSplitA operand
// times a kSplitB one over the 3 Kp is the fp32 product up to the lo.lo term
// and the residue of the split (relative 2^-16).
enum SplitLayout : int { kSplitA = 0, kSplitB = 1, kSplitDup = 2 };
inline int64_t split_width(int64_t K) { return (K + 7) / 8 * 8; }
mao_status split3_bf16(View In, int in_dtype, int rows, int K, View Out, int layout,
                       hipStream_t s);

// E <- I (n x n fp32); skipped when pred != nullptr and *pred == 0.
mao_status fill_identity(View E, int n, const int* pred, hipStream_t s);

// Fill n floats (or ints viewed as floats) with a value.
mao_status fill_f32(float* p, int64_t n, float v, hipStream_t s);

// FOAM moment statistics of Gr (fp32 m x n): row means and column means of
// Gr^2, then r, c EMAs, tau = tr(R)/bc2 / (|r|/bc2 * |c|/bc2); writes tau to
// tau_out[0] and aux[2].
int64_t foam_moments_work_floats(int m, int n);
mao_status foam_moments(View Gr, int m, int n, float beta2, float bc2, const float* Rdiag_src,
                        int64_t ldR, float* r, float* c, float* work, float* tau_out,
                        float* aux, hipStream_t s);

// N = (Mr / bc1) / (sqrt(tau * r_i/bc2 * c_j/bc2) + eps), written over Mr, or in
// bf16 to Nb when Nb.p is set.
mao_status foam_precondition(View Mr, int m, int n, const float* r, const float* c,
                             const float* tau, float bc1, float bc2, float eps, hipStream_t s,
                             View Nb = View{nullptr, 0, 0});

// FOAM refresh criterion on D (n x n): rho = ||offdiag||_F / ||D||_F, flag =
// rho > tol. Writes aux[0] = rho, aux[1] = flag, aux[3] = 1 and *flag_out.
mao_status offdiag_check(View D, int n, float tol, float* work, float* aux, int* flag_out,
                         hipStream_t s);

// Set aux[1] = 0, aux[3] = 0 and *flag_out = 0 (steps without a check).
mao_status no_check(float* aux, int* flag_out, hipStream_t s);

// Flat AdamW.
mao_status adamw(void* w, int w_dtype, const void* g, int g_dtype, float* m, float* v, int64_t n,
                 float lr, float beta1, float beta2, float bc1, float bc2, float eps, float wd,
                 float* out, hipStream_t s);

}  // namespace mao
