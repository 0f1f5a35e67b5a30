// Blocked Householder QR with explicit Q, the eigenbasis refresh primitive.
#pragma once

#include "common.hpp"

namespace mao {

constexpr int kQrNB = 64;       // panel width
constexpr int kQrThreads = 256; // positions per panel workgroup

struct QrWork {
  float* vstore;     // packed V panels
  float* zo;         // packed V T panels (orgqr)
  float* zf;         // V T^T of the even panels (n x 64)
  float* zf2;        // V T^T of the odd panels (the factorisation looks one panel ahead)
  float* wbuf;       // n x 64 intermediate
  float* wparts;     // 4 x n x 64 split-K partials of it
  float* sign;       // n
  float* part;       // 2 x Gmax x 64
  float* dg;         // 2 x 64
  float* gram;       // Gmax x 4096
  float* T;          // 4096
  unsigned* counters;// 2 x panels (per-column panel kernel, CholeskyQR panel kernel)
  int* err;          // barrier timeout flag
  int* fail;         // panels: 1 when the CholeskyQR panel fell back
  double* part64;    // Gmax x 2080 Gram partials
  double* gram64;    // 2080
  double* bcast;     // 64 x 64 + 64
  bf16_t* zsp;       // a panel's Z split into up to 3 bf16 parts (3 x n x 64)
  bf16_t* vsp;       // its vectors split likewise (3 x 64 x round_up(n, 8))
};

size_t qr_work_bytes(int n);
QrWork carve_qr_work(Carver& c, int n);

// Byte distance between consecutive jobs' workspaces in a batch (a multiple
// of 256: every job's QrWork carves to the same offsets from its base).
size_t qr_work_stride(int n);

// Several QRs of one size n in one set of launches: job j factors P_j given
// column-major in S + j sS (ld ldS; overwritten), writes E_j = Q_j^T to
// E + j sE (ld ldE) and, where Q[j] != nullptr, Q_j row-major (ld ldQ[j]).
// Its workspace is the j-th block of qr_work_stride(n) bytes at `work`
// (256-byte aligned). Job j is skipped where pred != nullptr and
// pred[j spred] == 0. The panels of all jobs share each cooperative launch
// (as many jobs as fit on the device at once), the trailing and explicit-Q
// updates are batched products.
struct QrBatch {
  int n = 0, njob = 0;
  float* S = nullptr;
  int64_t ldS = 0, sS = 0;
  float* E = nullptr;
  int64_t ldE = 0, sE = 0;
  float* const* Q = nullptr;     // host array of njob pointers (or nullptr)
  const int64_t* ldQ = nullptr;  // host array of njob leading dimensions
  const int* pred = nullptr;
  int64_t spred = 0;
  char* work = nullptr;
  // Start every job with its barrier time-out flag raised (test hook): every
  // grid barrier then stops waiting at once, every kernel still exits, and
  // the job's E and Q come out NaN -- what a real time-out produces.
  bool abort_barriers = false;
  // the factorisation's panel updates as bf16x3 products (for a QR input
  // that is itself a bf16x3 product); the explicit Q is accumulated in fp32
  bool fact_bf16x3 = false;
  // test hook: a CholeskyQR panel that breaks down raises the job's time-out
  // flag (NaN basis) instead of falling back to the per-column panel, so that
  // a test can tell the fast panel ran
  bool no_fallback = false;
};
mao_status qr_core_batched(const QrBatch& b, hipStream_t stream);
// Several batches of different sizes refreshed together: panel by panel, the
// panels of every batch share cooperative launches (the batches are
// independent; each keeps its own order of steps).
mao_status qr_core_multi(const QrBatch* batches, int ngroups, hipStream_t stream);

// Fused panel step (qr_update.hip), per job j (pointers advanced by j times
// their stride): C (M x L, ld ldC) <- C - W Z^T with W (M x nb) the sum of
// wslices_in slices wslice floats apart and Z (L x nb), both at leading
// dimension 64; then, when nbn > 0, Wn (M x nbn, ld 64) = C Vn^T, the nbn
// rows of Vn (ld ldV) spanning C's L columns, written as `splits` partial
// slices (one per column range; wslice floats apart) whose sum is Wn
// (splits <= kQrFusedMaxSplits; without the projection any count). With Wt != nullptr,
// also Wt[c][i] = Vt[i][c] for c < trows in slice 0 and zero in the others
// (ld 64; Vt at ld ldV and stride sV). Jobs whose predicate (pred[j spred])
// is zero are skipped. nb, nbn <= 64.
constexpr int kQrFusedMaxSplits = 4;
// Arithmetic of the fused products on bf16 MFMA: bf16x3 (about 2^-17
// relative) or bf16x6 (three-way splits, fp32-equivalent).
enum QrPrec : int { kQrBf16x3 = 1, kQrBf16x6 = 2 };
struct QrFusedArgs {
  float* C = nullptr;
  int64_t ldC = 0, sC = 0;
  const float* W = nullptr;
  int64_t sW = 0;
  // Z and Vn split into bf16 parts by qr_presplit (2 for bf16x3, 3 for
  // bf16x6): Z's parts at row pitch 64, zpart apart; Vn's at ldVp, vpart
  // apart; sZp / sVp between jobs
  const bf16_t* Zp = nullptr;
  int64_t sZp = 0, zpart = 0;
  const bf16_t* Vp = nullptr;
  int64_t ldVp = 0, sVp = 0, vpart = 0;
  int64_t ldV = 0, sV = 0;  // Vt (the identity rows' source) at ldV, sV
  float* Wn = nullptr;
  int64_t sWn = 0;
  float* Wt = nullptr;
  const float* Vt = nullptr;
  int trows = 0;
  int M = 0, L = 0, nb = 0, nbn = 0;
  int splits = 1, wslices_in = 1;
  int64_t wslice = 0;
  int prec = kQrBf16x6;  // QrPrec of both products
  const int* pred = nullptr;
  int64_t spred = 0;
  int strips = 0;  // set by qr_fused_update
};
mao_status qr_fused_update(const QrFusedArgs& a, int njob, hipStream_t stream);
// Workgroups of qr_fused_update's kernel resident on the current device at once.
int qr_fused_slots();

// A panel's Z (zrows x 64, ld 64, columns >= znb zero) and V (vrows x vcols,
// ld ldV) split into `parts` bf16 arrays for qr_fused_update, per job.
struct QrSplitArgs {
  const float* Z = nullptr;
  int64_t sZ = 0;
  int zrows = 0, znb = 0;
  bf16_t* Zp = nullptr;
  int64_t sZp = 0, zpart = 0;
  const float* V = nullptr;
  int64_t ldV = 0, sV = 0;
  int vrows = 0, vcols = 0;
  bf16_t* Vp = nullptr;
  int64_t sVp = 0, vpart = 0, ldVp = 0;
  int parts = 3;
  const int* pred = nullptr;
  int64_t spred = 0;
};
mao_status qr_presplit(const QrSplitArgs& a, int njob, hipStream_t stream);

// Householder QR of P given column-major in S (S[j][i] = P[i][j], n x n,
// leading dimension ldS); S is overwritten. Writes E = Q^T (row-major, ldE)
// and, if Qout != nullptr, Q (row-major, ldQ), with column signs such that
// diag(R) >= 0. Every kernel is skipped when pred != nullptr and *pred == 0.
// If a grid barrier times out, E and Q are set to NaN.
mao_status qr_core(float* S, int64_t ldS, int n, float* E, int64_t ldE, float* Qout,
                   int64_t ldQ, QrWork& w, const int* pred, hipStream_t stream,
                   bool abort_barriers = false, bool fact_bf16x3 = false,
                   bool no_fallback = false);

}  // namespace mao
