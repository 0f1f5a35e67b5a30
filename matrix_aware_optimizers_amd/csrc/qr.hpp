// Blocked Householder QR with explicit Q, the eigenbasis refresh primitive.
#pragma once

#include "common.hpp"

namespace mao {

constexpr int kQrNB = 64;       // panel width
constexpr int kQrThreads = 256; // positions per panel workgroup

struct QrWork {
  float* vstore;     // packed V panels
  float* zo;         // packed V T panels (orgqr)
  float* zf;         // one V T^T panel (n x 64)
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
};
mao_status qr_core_batched(const QrBatch& b, hipStream_t stream);

// Householder QR of P given column-major in S (S[j][i] = P[i][j], n x n,
// leading dimension ldS); S is overwritten. Writes E = Q^T (row-major, ldE)
// and, if Qout != nullptr, Q (row-major, ldQ), with column signs such that
// diag(R) >= 0. Every kernel is skipped when pred != nullptr and *pred == 0.
mao_status qr_core(float* S, int64_t ldS, int n, float* E, int64_t ldE, float* Qout,
                   int64_t ldQ, QrWork& w, const int* pred, hipStream_t stream);

}  // namespace mao
