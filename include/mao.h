/*
 * mao.h -- C ABI of the matrix-aware optimizer step library (libmao.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * One call advances one weight matrix (or a group of same-shape matrices) by
 * one optimizer step, entirely on the GPU, asynchronously on the caller's HIP
 * stream. Sources for every operation are cited at the entry point, by page
 * title and section:
 *
 *   [SMB]  "SOAP, Muon, and Beyond" review (dimensionstp.github.io)
 *   [PX]   picx.dev summary of the same paper (numbered equations)
 *   [FOAM] "Factored One-sided Adam-Moment for Practical and Scalable SOAP"
 *          review
 *   [M+]   "Muon+: Towards Better Muon via One Additional Normalization Step"
 *          (gist.science)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Matrices are row-major device views: element (i, j) of a mao_mat lives at
 *   data + i*ld + j (in elements of its dtype); ld >= cols, ld a multiple of
 *   8, data 16-byte aligned. A strided view (ld > cols) lets a caller step a
 *   logical sub-matrix of a fused tensor, e.g. one of Q, K, V inside a fused
 *   QKV weight ([SMB] section 3-2 (2): fused QKV is split into logical
 *   matrices before orthogonalisation).
 * - Buffers that must be distinct (MAO_E_ALIAS otherwise) are compared byte
 *   by byte when both have the same row pitch (ld times the element size) and
 *   a batch stride that is a multiple of ld: column views of one wider buffer
 *   with disjoint column ranges (the logical Q, K and V of one fused weight,
 *   stepped as separate groups of one muon_step_batched call) are distinct.
 *   Other pairs are compared by the byte ranges they span.
 * - Ownership: the caller owns every buffer (weights, gradients, optimizer
 *   state, workspace, outputs). The library allocates no device memory and
 *   keeps no device state between calls. Sizes of the workspace come from the
 *   *_workspace_size queries; the workspace must be 256-byte aligned. The
 *   caller supplies the 1-based step counter t.
 * - Updates are in place: W and the state buffers are overwritten; G is
 *   read-only.
 * - Errors: every entry point validates all arguments on the host before it
 *   enqueues anything and returns a mao_status; an invalid call enqueues
 *   nothing. mao_last_error() gives a thread-local message for the last
 *   failure. A failed kernel launch returns MAO_E_HIP; faults inside kernels
 *   surface at the caller's next synchronisation, as for any HIP work.
 * - No call synchronises the device or the stream, and none allocates; all
 *   work runs on `stream` (a hipStream_t; NULL = the null stream). Results are
 *   deterministic: the same inputs on the same stream order give bitwise the
 *   same outputs (no floating-point atomics).
 * - Calls that share a workspace must be ordered on one stream.
 */
#ifndef MAO_H
#define MAO_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MAO_API __attribute__((visibility("default")))
#else
#define MAO_API
#endif

#define MAO_ABI_VERSION 4
#define MAO_MAX_GROUPS 8

typedef enum {
  MAO_OK = 0,
  MAO_E_NULL = 1,        /* a required pointer is NULL */
  MAO_E_SHAPE = 2,       /* sizes < 1, or shapes that do not agree */
  MAO_E_DTYPE = 3,       /* unsupported dtype for that argument */
  MAO_E_LAYOUT = 4,      /* ld < cols, ld not a multiple of 8, misaligned */
  MAO_E_ALIAS = 5,       /* two buffers that must be distinct overlap */
  MAO_E_HPARAM = 6,      /* hyperparameter out of range */
  MAO_E_WORKSPACE = 7,   /* workspace NULL, misaligned or too small */
  MAO_E_HIP = 8,         /* a HIP runtime call or launch failed */
  MAO_E_UNSUPPORTED = 9  /* a valid request this build does not serve */
} mao_status;

typedef enum { MAO_F32 = 0, MAO_BF16 = 1 } mao_dtype;

/* Row-major device matrix view. */
typedef struct {
  void* data;
  int64_t rows, cols, ld;
  int32_t dtype; /* mao_dtype */
} mao_mat;

/* A group of `count` same-shape row-major matrices, matrix b at
 * data + b*stride (elements). stride >= rows*ld. */
typedef struct {
  void* data;
  int64_t count, rows, cols, ld, stride;
  int32_t dtype; /* mao_dtype */
} mao_batch;

/* ------------------------------------------------------------------------ */
/* Muon / Muon+                                                              */
/* ------------------------------------------------------------------------ */

/* Muon+ normalisation direction ([M+] section 2, step 3). */
typedef enum {
  MAO_NORM_NONE = 0,
  MAO_NORM_ROW = 1,
  MAO_NORM_COL = 2,
  MAO_NORM_COL_ROW = 3, /* columns first, then rows */
  MAO_NORM_ROW_COL = 4
} mao_norm_mode;

typedef struct {
  float lr;            /* learning rate, >= 0 */
  float mu;            /* momentum, 0 <= mu < 1 */
  float weight_decay;  /* decoupled, >= 0 */
  float eps;           /* > 0: X0 = M / (||M||_F + eps) (1e-7 in [SMB] 3-2 (2)) */
  int32_t ns_steps;    /* Newton-Schulz iterations, 0..64 */
  const float* ns_coeffs; /* host array [ns_steps][3] of (a, b, c), or NULL for
                             the classical quintic (15/8, -10/8, 3/8) */
  int32_t ns_dtype;    /* MAO_BF16: bf16 MFMA with fp32 accumulation;
                          MAO_F32: fp32 MFMA */
  int32_t norm_mode;   /* mao_norm_mode */
  float norm_eps;      /* > 0, denominator guard of the Muon+ pass */
} mao_muon_hparams;

/* Workspace bytes for one muon_step on a rows x cols matrix. */
MAO_API size_t muon_workspace_size(int64_t rows, int64_t cols, const mao_muon_hparams* hp);

/*
 * muon_step -- one Muon (Muon+) step on one matrix.
 * [M+] section 2 (steps 1-4); [SMB] sections 2-1 (polar factor UV^T) and
 * 3-2 (2) (Newton-Schulz recipe, eps, weight decay).
 *
 *   M <- mu M + (1 - mu) G
 *   X_0 = M / (||M||_F + eps), on the wide orientation (rows <= cols; a tall
 *         matrix is transposed internally)
 *   for k < ns_steps: A = X X^T; B = b_k A + c_k A A; X <- a_k X + B X
 *   O = Norm^(norm_mode)(X)   (Muon+; scale-preserving: each column (row) is
 *         rescaled to ||O||_F / sqrt(cols) (||O||_F / sqrt(rows)))
 *   U = sqrt(rows / cols) * O
 *   W <- W - lr (weight_decay W + U)
 *
 * W: rows x cols, bf16 or fp32 (bf16 results are rounded to nearest even).
 * G: rows x cols, bf16 or fp32. M: rows x cols, fp32 momentum (state).
 * update_out: NULL, or a device fp32 buffer of rows*cols (dense, ld = cols)
 *   that receives U (the update before the learning rate).
 * W, G, M and update_out must not overlap.
 */
MAO_API mao_status muon_step(mao_mat W, mao_mat G, mao_mat M, const mao_muon_hparams* hp,
                     void* workspace, size_t workspace_bytes, float* update_out,
                     void* stream);

/* Workspace bytes for muon_step_batched over these groups. */
MAO_API size_t muon_batched_workspace_size(int32_t ngroups, const mao_batch* W,
                                   const mao_muon_hparams* hp);

/*
 * muon_step_batched -- the muon_step above on every matrix of up to
 * MAO_MAX_GROUPS groups of same-shape matrices (e.g. the gate, up and down
 * banks of all experts of an MoE layer), with one launch per Newton-Schulz
 * stage covering every matrix. Each matrix is stepped exactly as muon_step
 * would step it alone. Groups may have different shapes.
 * W[g], G[g], M[g] describe group g (same count/rows/cols); W and G bf16 or
 * fp32, M fp32. update_out: NULL, or ngroups batches of fp32 receiving U.
 */
MAO_API mao_status muon_step_batched(int32_t ngroups, const mao_batch* W, const mao_batch* G,
                             const mao_batch* M, const mao_muon_hparams* hp,
                             void* workspace, size_t workspace_bytes,
                             const mao_batch* update_out, void* stream);

/*
 * muon_step_noalloc -- muon_step for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, kernels and results as muon_step, minus
 * the workspace: the step's scratch memory is one static device array of
 * MAO_NOALLOC_SCRATCH_BYTES inside the library, which every GPU the library
 * runs on holds from the library's first kernel on that GPU until the process
 * ends. The call itself allocates nothing (its first call on a device looks
 * up that device's address of the array, once).
 *
 * Limits: the step must fit the array -- muon_workspace_size(rows, cols, hp)
 * <= MAO_NOALLOC_SCRATCH_BYTES (64 MiB: square matrices up to 2304 with
 * bf16 Newton-Schulz and 1616 with fp32; the 1536 x 2048 and 2048 x 1536
 * expert matrices of a fine-grained MoE bank in bf16), else MAO_E_WORKSPACE
 * before anything is enqueued.
 * The stream must belong to the current device (MAO_E_UNSUPPORTED
 * otherwise). All calls on one GPU share the one array and each call leaves
 * its contents behind: calls that may overlap in time on one GPU (different
 * streams, different host threads) race and must be serialised by the
 * caller. Nothing in the array needs to start at zero.
 */
#define MAO_NOALLOC_SCRATCH_BYTES (64u << 20)
MAO_API size_t muon_step_noalloc_max_bytes(void);
MAO_API mao_status muon_step_noalloc(mao_mat W, mao_mat G, mao_mat M, const mao_muon_hparams* hp,
                                     float* update_out, void* stream);

/* ------------------------------------------------------------------------ */
/* SOAP with the real-time eigenbasis refresh                                */
/* ------------------------------------------------------------------------ */

/* Precision of the products that must stay fp32-accurate ([SMB] section 3-2
 * (3)): the forward rotations (G~ = QL^T G QR, M~ = QL^T M QR, FOAM's G QR and
 * M QR) and the power-iteration products F Q that feed the refresh. */
typedef enum {
  MAO_ROT_F32 = 0,    /* fp32 MFMA */
  MAO_ROT_BF16X3 = 1  /* bf16 MFMA on split operands: x = hi + lo (both bf16),
                         A B^T = hi_a hi_b^T + lo_a hi_b^T + hi_a lo_b^T as one
                         product over three times K (fp32 accumulation;
                         relative error about 2^-16) */
} mao_rot_mode;

typedef struct {
  float lr, beta1, beta2; /* 0 <= beta < 1 */
  float eps;              /* > 0, Adam denominator sqrt(v_hat) + eps */
  float weight_decay;     /* decoupled, >= 0 */
  int32_t refresh_every;  /* 1: refresh every step; k > 1: at t = 1, k+1, ...;
                             0: basis frozen */
  int32_t back_rot_dtype; /* MAO_F32: the rotation back U = QL N QR^T on fp32
                             MFMA; MAO_BF16: on bf16 MFMA (operands rounded to
                             bf16, fp32 accumulation; [SMB] section 3-2 (3)
                             allows the reduced precision on this product) */
  int32_t fwd_rot;        /* mao_rot_mode of the forward rotations */
  int32_t refresh_prod;   /* mao_rot_mode of the power-iteration products L QL
                             and R QR (the QR inputs) */
} mao_soap_hparams;

/* SOAP optimizer state, all fp32, rows = m, cols = n of W.
 * Initial values: M = V = L = R = 0, QL = I_m, QR = I_n. */
typedef struct {
  mao_mat M;  /* m x n momentum (original space) */
  mao_mat V;  /* m x n second moment (rotated space) */
  mao_mat L;  /* m x m factor EMA of G G^T */
  mao_mat R;  /* n x n factor EMA of G^T G */
  mao_mat QL; /* m x m basis, columns = basis vectors */
  mao_mat QR; /* n x n basis, columns = basis vectors */
} mao_soap_state;

MAO_API size_t soap_workspace_size(int64_t rows, int64_t cols, const mao_soap_hparams* hp);

/*
 * soap_step -- one SOAP step with per-step basis refresh by one QR
 * power-iteration step. [SMB] section 1-1 (factor EMAs), section 3-2 (3)
 * (rotation, Adam in the eigenbasis, rotation back) and 3-2 (4) (real-time
 * update: current gradient first, then refresh with QR, then precondition the
 * same step); [PX] Eq. (1).
 *
 *   M <- b1 M + (1-b1) G
 *   L <- b2 L + (1-b2) G G^T;  R <- b2 R + (1-b2) G^T G
 *   if refresh(t): QL <- qr(L QL), QR <- qr(R QR)  (Householder, diag(R) >= 0)
 *   G~ = QL^T G QR;  M~ = QL^T M QR
 *   V <- b2 V + (1-b2) G~ . G~
 *   N = (M~ / (1-b1^t)) / (sqrt(V / (1-b2^t)) + eps)
 *   U = QL N QR^T;  W <- W - lr (weight_decay W + U)
 *
 * The factor EMAs of a bf16 G run on bf16 MFMA (exact products), the
 * refresh products in fp32 or as bf16x3 (refresh_prod), the QR in fp32; the
 * forward rotations in fp32 or as bf16x3 (fwd_rot), the rotation back in fp32
 * or bf16 (back_rot_dtype). W, G: bf16 or fp32.
 * update_out: NULL or fp32 rows*cols (dense) receiving U. t >= 1.
 */
MAO_API mao_status soap_step(mao_mat W, mao_mat G, const mao_soap_state* state, int64_t t,
                     const mao_soap_hparams* hp, void* workspace, size_t workspace_bytes,
                     float* update_out, void* stream);

/* ------------------------------------------------------------------------ */
/* FOAM                                                                      */
/* ------------------------------------------------------------------------ */

/* Which side of W carries FOAM's rotation. */
typedef enum {
  MAO_FOAM_INPUT = 0,  /* the method: basis of G^T G (n x n), G_rot = G QR */
  MAO_FOAM_OUTPUT = 1  /* the output-only ablation of [FOAM] section 3: basis of
                          G G^T (m x m), G_rot = QR^T G */
} mao_foam_side;

/* How a refresh recomputes the basis. */
typedef enum {
  MAO_REFRESH_QR = 0,  /* one power-iteration step: Q <- qr(F Q) */
  MAO_REFRESH_EIGH = 1 /* full eigendecomposition of F ([FOAM] section 1): the
                          eigenvectors, by descending eigenvalue */
} mao_refresh_mode;

typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t pf; /* >= 1: the refresh criterion is evaluated at t = 1, pf+1, ... */
  float tol;  /* >= 0: refresh when rho > tol */
  int32_t side; /* mao_foam_side */
  int32_t refresh; /* mao_refresh_mode; MAO_REFRESH_EIGH needs k <= 16384 */
  int32_t back_rot_dtype; /* MAO_F32 or MAO_BF16: precision of U = N QR^T
                             (QR N on the output side), as for SOAP */
  int32_t fwd_rot;        /* mao_rot_mode of G_rot and M_rot */
  int32_t refresh_prod;   /* mao_rot_mode of the criterion products S = QR^T R
                             (the QR refresh's input) and S QR; MAO_ROT_BF16X3
                             only with MAO_REFRESH_QR (MAO_E_UNSUPPORTED with
                             the eigendecomposition, whose eigenvectors are
                             only as accurate as its input relative to the
                             eigenvalue gaps) */
} mao_foam_hparams;

/* FOAM state, fp32, W is m x n; k = n for MAO_FOAM_INPUT, m for
 * MAO_FOAM_OUTPUT. Initial: M = R = 0, QR = I_k, r = c = 0.
 * aux: device float[4] written by every step: aux[0] = rho of the last
 * evaluated criterion, aux[1] = 1 if this step refreshed else 0, aux[2] = tau,
 * aux[3] = 1 if this step evaluated the criterion else 0. */
typedef struct {
  mao_mat M;  /* m x n momentum */
  mao_mat R;  /* k x k factor EMA of G^T G (input side) or G G^T (output side) */
  mao_mat QR; /* k x k basis, columns = basis vectors */
  float* r;   /* m, EMA of row means of G_rot^2 */
  float* c;   /* n, EMA of column means of G_rot^2 */
  float* aux; /* 4 floats */
} mao_foam_state;

MAO_API size_t foam_workspace_size(int64_t rows, int64_t cols, const mao_foam_hparams* hp);

/*
 * foam_step -- one FOAM step: input-side rotation only and a factored second
 * moment. [FOAM] section 1 (G_rot = G QR; r, c EMAs of row / column means of
 * G_rot^2; V_hat = tau r_hat c_hat^T, tau = tr(R_hat)/(|r_hat|_1 |c_hat|_1))
 * and section 3 (R EMA; adaptive-tolerance refresh with pf, tol; bias-corrected
 * Adam in the rotated space).
 *
 *   M <- b1 M + (1-b1) G;  R <- b2 R + (1-b2) G^T G
 *   if (t-1) % pf == 0: D = QR^T R QR, rho = ||D - diag D||_F / ||D||_F;
 *                       if rho > tol: QR <- qr(R QR)       (decided on device)
 *                       (hp->refresh = MAO_REFRESH_EIGH: QR <- the
 *                       eigenvectors of R by descending eigenvalue, from a
 *                       block-Jacobi diagonalisation of D warm-started in the
 *                       current basis)
 *   G_rot = G QR;  M_rot = M QR
 *   r <- b2 r + (1-b2) rowmean(G_rot^2);  c <- b2 c + (1-b2) colmean(G_rot^2)
 *   tau = tr(R / (1-b2^t)) / (|r_hat|_1 |c_hat|_1)  (0 if r = c = 0)
 *   N = (M_rot / (1-b1^t)) / (sqrt(tau r_hat c_hat^T) + eps)
 *   U = N QR^T;  W <- W - lr (weight_decay W + U)
 *
 * With hp->side = MAO_FOAM_OUTPUT (the output-only ablation of [FOAM] section
 * 3, read as the mirror of the steps above): R <- b2 R + (1-b2) G G^T (m x m),
 * the same criterion and refresh on that factor, G_rot = QR^T G,
 * M_rot = QR^T M, r and c the row and column means of G_rot^2 as above, tau
 * with tr(R_hat), U = QR N.
 */
MAO_API mao_status foam_step(mao_mat W, mao_mat G, const mao_foam_state* state, int64_t t,
                     const mao_foam_hparams* hp, void* workspace, size_t workspace_bytes,
                     float* update_out, void* stream);

/* ------------------------------------------------------------------------ */
/* Many matrices per call                                                    */
/* ------------------------------------------------------------------------ */

/* Workspace bytes for soap_step_many / foam_step_many on these shapes (only
 * W[i].rows and W[i].cols are read); 0 for count outside 1..4096 or an empty
 * shape. */
MAO_API size_t soap_step_many_workspace_size(int32_t count, const mao_mat* W,
                                             const mao_soap_hparams* hp);
MAO_API size_t foam_step_many_workspace_size(int32_t count, const mao_mat* W,
                                             const mao_foam_hparams* hp);

/*
 * soap_step_many / foam_step_many -- soap_step / foam_step on `count`
 * matrices of any shapes (the layers of a model), with the same t and
 * hyperparameters; results equal `count` separate calls up to fp32 rounding
 * order. The step runs in phases, and the products of one phase for all
 * matrices go out as grouped launches (equal shapes as one batch, its
 * per-matrix operand pointers in a table inside the workspace), which may
 * use other tile sizes than a lone product and so sum over K in another
 * order. The QR refreshes of equal size (SOAP: the L factor of an m x n
 * matrix is of size m, the R factor of size n; FOAM: R only) run as one
 * batched QR each: the panels of all of them share each cooperative launch
 * and the updates run as batched products, so that the per-panel latency is
 * paid once per size instead of once per factor ([SMB] section 3-2 (4) for
 * the refresh; [FOAM] section 3 for FOAM's criterion, decided per matrix on
 * the device).
 *
 * W, G, state: arrays of `count` (host memory, read during the call).
 * update_out: NULL, or a host array of `count` pointers, each NULL or as in
 * soap_step. Buffers of different matrices must not overlap (MAO_E_ALIAS).
 * count outside 1..4096: MAO_E_SHAPE; NULL W, G or state: MAO_E_NULL; other
 * errors as in the single-matrix calls, reported for the first failing
 * matrix before anything is launched.
 */
MAO_API mao_status soap_step_many(int32_t count, const mao_mat* W, const mao_mat* G,
                                  const mao_soap_state* state, int64_t t,
                                  const mao_soap_hparams* hp, void* workspace,
                                  size_t workspace_bytes, float* const* update_out, void* stream);
MAO_API mao_status foam_step_many(int32_t count, const mao_mat* W, const mao_mat* G,
                                  const mao_foam_state* state, int64_t t,
                                  const mao_foam_hparams* hp, void* workspace,
                                  size_t workspace_bytes, float* const* update_out, void* stream);

/* ------------------------------------------------------------------------ */
/* AdamW (flat)                                                              */
/* ------------------------------------------------------------------------ */

/*
 * adamw_step -- AdamW on n contiguous elements ([SMB] section 1-1; the FOAM
 * review, section 4, keeps embeddings on AdamW):
 *   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
 *   u = (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps);  w <- w - lr (wd w + u)
 * w: bf16 or fp32 (w_dtype); g: bf16 or fp32 (g_dtype); m, v fp32.
 * update_out: NULL or fp32[n].
 */
MAO_API mao_status adamw_step(void* w, int32_t w_dtype, const void* g, int32_t g_dtype, float* m,
                      float* v, int64_t n, int64_t t, float lr, float beta1, float beta2,
                      float eps, float weight_decay, float* update_out, void* stream);

/* ------------------------------------------------------------------------ */
/* Building blocks exposed for kernel-level checks                           */
/* ------------------------------------------------------------------------ */

/* mode bits of mao_gemm_nt */
#define MAO_GEMM_SYMMETRIC 1 /* lower triangle of a square result, mirrored (SYRK) */
#define MAO_GEMM_B_KMAJOR 2  /* B stored K x N: D = alpha A B + beta C0 */

/*
 * mao_gemm_nt -- D = alpha * A B^T + beta * C0, the contraction every step
 * above is built from. A: M x K, B: N x K (row-major, both K-contiguous),
 * C0/D: M x N. in_dtype: MAO_BF16 (bf16 MFMA) or MAO_F32 (fp32 MFMA) for A
 * and B; C0 and D fp32. C0 may be NULL (beta ignored) and may equal D.
 * mode: 0, or MAO_GEMM_SYMMETRIC -- only the lower triangle of a square
 * result is computed (A == B, M == N) and mirrored -- or MAO_GEMM_B_KMAJOR --
 * B is stored K x N (ldb >= N), bf16 only: the Newton-Schulz product B X
 * reads X this way. Other bits: MAO_E_HPARAM; unsupported combinations:
 * MAO_E_UNSUPPORTED.
 */
MAO_API mao_status mao_gemm_nt(int64_t M, int64_t N, int64_t K, float alpha, const void* A,
                       int64_t lda, const void* B, int64_t ldb, int32_t in_dtype, float beta,
                       const float* C0, int64_t ldc0, float* D, int64_t ldd, int32_t mode,
                       void* stream);

/* Workspace bytes for mao_eigh on an n x n matrix (0 outside 1..16384). */
MAO_API size_t mao_eigh_workspace_size(int64_t n);

/*
 * mao_eigh -- eigendecomposition of a symmetric fp32 matrix F (row-major
 * n x n, 1 <= n <= 16384; only its symmetric part (F + F^T)/2 is used), the
 * refresh primitive of foam_step with MAO_REFRESH_EIGH ([FOAM] section 1:
 * the basis is the eigenvectors of the factor). Q (n x n, row-major) receives
 * the orthonormal eigenvectors as columns, ordered by descending eigenvalue
 * (ties by index); evals (NULL or n device floats) the eigenvalues in that
 * order; info (NULL or 13 device floats) the off-diagonal ratio
 * ||D - diag D||_F / ||D||_F after each of up to 12 block-Jacobi sweeps (0
 * after convergence), then the number of sweeps run. F and Q must not
 * overlap. Accuracy: fp32 -- eigenvalues to about 1e-6 of the largest,
 * eigenvectors to that over the eigenvalue gap.
 */
MAO_API mao_status mao_eigh(const float* F, int64_t ldf, float* Q, int64_t ldq, float* evals,
                            float* info, int64_t n, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Workspace bytes for mao_qr on an n x n matrix. */
MAO_API size_t mao_qr_workspace_size(int64_t n);

/*
 * mao_qr -- Q of the Householder QR of a square fp32 matrix P (row-major,
 * n x n), with column signs chosen so that diag(R) >= 0 -- the refresh
 * primitive of soap_step and foam_step ([SMB] section 3-2 (4): per-step QR of
 * the power-iteration product). P is read only; Q (n x n, row-major) is
 * written. P and Q must not overlap.
 */
MAO_API mao_status mao_qr(const float* P, int64_t ldp, float* Q, int64_t ldq, int64_t n,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Failure of the refresh. The panels of the QR synchronise their workgroups
 * with bounded grid barriers inside cooperative launches. Should a barrier
 * wait time out (about a second; only a device that cannot keep the grid
 * resident would), every barrier of that QR stops waiting, the kernels exit,
 * and the QR writes NaN to its whole output basis: mao_qr's Q, the refreshed
 * Q_L / Q_R of soap_step and the Q_R of foam_step (and of the many-matrix
 * calls). The step's update and weights then come out NaN rather than
 * silently wrong; the error surfaces at the caller's next check of the
 * results, as for any asynchronous fault.
 *
 * mao_dbg_qr -- mao_qr with test flags (kernel-level checks only).
 * MAO_DBG_QR_ABORT_BARRIERS starts the QR with its time-out flag raised, so
 * that every barrier gives up at once -- what a real time-out does -- and the
 * NaN result above can be checked without waiting for one.
 * MAO_DBG_QR_NO_FALLBACK: a CholeskyQR panel that breaks down (and would fall
 * back to the per-column Householder panel, with the same result) raises the
 * time-out flag instead, so Q comes out NaN -- a test of a well-conditioned
 * P then shows that the fast panels ran. Other bits: MAO_E_HPARAM.
 */
#define MAO_DBG_QR_ABORT_BARRIERS 1
#define MAO_DBG_QR_NO_FALLBACK 2
MAO_API mao_status mao_dbg_qr(const float* P, int64_t ldp, float* Q, int64_t ldq, int64_t n,
                              void* workspace, size_t workspace_bytes, int32_t flags,
                              void* stream);

/* ------------------------------------------------------------------------ */
/* Observability: reductions over buffers the steps already hold             */
/* ------------------------------------------------------------------------ */
/*
 * [SMB] section 7-2, item 4 lists what an optimizer log should carry:
 * layer-wise update RMS, the Newton-Schulz residual, the SOAP factor
 * condition number and the basis update age; [FOAM] section 3 reports the
 * rank-1 share of the rotated second moment. The calls below compute these on
 * the device into caller-owned device floats, without synchronising, like the
 * steps (host-side validation, caller-owned workspace, fixed-order fp64
 * reductions, bitwise repeatable).
 */

/* Workspace bytes for mao_matrix_rms over the batch X. */
MAO_API size_t mao_matrix_rms_workspace_size(mao_batch X);

/*
 * mao_matrix_rms -- out[b] = ||X_b||_F / sqrt(rows * cols) for every matrix of
 * the batch (count <= 65535; X bf16 or fp32). This is [SMB] section 2-1's
 * update RMS, ||dW||_F / sqrt(|W|), when X holds the update: applied to a
 * step's update_out (U, before the learning rate) it gives RMS(dW) / lr of
 * the optimizer term, weight decay excluded. out: count device floats.
 */
MAO_API mao_status mao_matrix_rms(mao_batch X, float* out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Workspace bytes for mao_ns_residual over the batch O. */
MAO_API size_t mao_ns_residual_workspace_size(mao_batch O);

/*
 * mao_ns_residual -- the Newton-Schulz residual of each matrix of the batch:
 * with X = scale * O_b taken in its wide orientation (a = min(rows, cols)
 * rows), out[b] = ||X X^T - I_a||_F / sqrt(a), the RMS over the singular
 * values s_i of X of s_i^2 - 1, which is 0 exactly when X has orthonormal rows
 * (the polar factor U V^T that the iteration approaches, [SMB] section 2-1).
 * O: fp32 (a muon_step update_out with scale = sqrt(cols / rows) recovers the
 * Newton-Schulz output when norm_mode is none). The a x a product runs on the
 * fp32 MFMA path. scale: finite, nonzero. out: count device floats.
 */
MAO_API mao_status mao_ns_residual(mao_batch O, float scale, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace bytes for mao_rayleigh on n x n operands. */
MAO_API size_t mao_rayleigh_workspace_size(int64_t n);

/*
 * mao_rayleigh -- Rayleigh quotients of a Kronecker factor in its current
 * basis: diag_out[i] = q_i^T F q_i for every column q_i of Q (F, Q fp32
 * n x n, F a SOAP L / R or a FOAM R, Q its basis Q_L / Q_R), and, when
 * kappa_out is not NULL, kappa_out[0] = max_i d_i / min_i d_i (+inf when
 * min_i d_i <= 0) -- the factor condition-number estimate of [SMB] section
 * 7-2. For orthonormal Q every d_i lies in [lambda_min(F), lambda_max(F)], so
 * the estimate never exceeds the condition number of F, and equals it when Q
 * diagonalises F. diag_out: n device floats; kappa_out: NULL or 1 float.
 */
MAO_API mao_status mao_rayleigh(mao_mat F, mao_mat Q, float* diag_out, float* kappa_out,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes for mao_rank1_share on a rows x cols matrix. */
MAO_API size_t mao_rank1_share_workspace_size(int64_t rows, int64_t cols);

/*
 * mao_rank1_share -- out[0] = s_1(V)^2 / ||V||_F^2, the share of the squared
 * Frobenius mass of V (fp32 m x n, e.g. SOAP's second moment V in its
 * rotated basis) that its best rank-1 approximation captures ([FOAM]
 * section 3: the rank-1 share that motivates factoring the rotated moment).
 * s_1 comes from `iters` (1..1000) steps of power iteration on V^T V from the
 * unit all-ones vector, each normalised; the estimate is ||V v||^2 for the
 * last unit iterate v, which never exceeds the true share beyond rounding.
 * A zero V gives 0. Applied to the momentum M it is 1 / stable rank of M
 * (s_1^2 / sum s_i^2), the one-number summary of M's singular-value
 * distribution ([SMB] section 7-2); for a signed matrix the start vector is
 * not aligned with a Perron vector, so give it enough iterations for the gap
 * s_2 / s_1.
 */
MAO_API mao_status mao_rank1_share(mao_mat V, int32_t iters, float* out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * mao_basis_age -- steps since FOAM last refreshed its basis ([SMB] section
 * 7-2: basis update age), kept on the device: after a foam_step, age[0] <- 0
 * when the step refreshed (aux[1] != 0), else age[0] + 1. The caller owns the
 * float and sets it to 0 before the first step. (For SOAP the age is
 * (t - 1) mod refresh_every, known on the host.) aux: the foam_state aux
 * array; age: 1 device float.
 */
MAO_API mao_status mao_basis_age(const float* aux, float* age, void* stream);

/* ------------------------------------------------------------------------ */
/* Measurement instrumentation (not part of any optimizer step)              */
/* ------------------------------------------------------------------------ */

/*
 * mao_timing_enable -- when on != 0, every contraction launch made by the
 * library is bracketed by two HIP events recorded on its stream, tagged by
 * what it computes (0: Newton-Schulz Gram X X^T, 1: Newton-Schulz A A,
 * 2: Newton-Schulz B X, 3: other contractions on fp32 inputs, 4: QR rank
 * updates, 5: other contractions on bf16 inputs, 6: QR projections onto a
 * panel's vectors, 7: QR fused update-and-projection, 8: QR panel
 * factorisations, counted at zero flops, 9: launches gated by a device-side
 * flag, such as FOAM's refresh, whose flops assume every job ran) with its
 * algorithmic flop count (symmetric products at half cost); the memory-bound
 * passes of a Muon step (momentum EMA with its norm, X0 cast, Muon+ sums of
 * squares, update) are bracketed the same way under tag 10 with the bytes
 * they must move in place of flops. Tags at or past ntags are not
 * reported. Off by default;
 * this is the only host-side state the library keeps, and it exists for
 * benchmarking only.
 * mao_timing_collect -- waits for the recorded events, sums elapsed
 * milliseconds, launch counts and flops per tag into the caller's arrays of
 * ntags entries, releases the events and returns the number of launches.
 */
MAO_API void mao_timing_enable(int on);
MAO_API int mao_timing_collect(double* ms, int64_t* count, double* flops, int ntags);

/* ------------------------------------------------------------------------ */
/* Status                                                                    */
/* ------------------------------------------------------------------------ */

MAO_API const char* mao_status_string(mao_status s);
MAO_API const char* mao_last_error(void); /* thread-local detail of the last failure */
MAO_API int mao_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MAO_H */
