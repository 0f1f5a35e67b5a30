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

// Householder QR of P given column-major in S (S[j][i] = P[i][j], n x n,
// leading dimension ldS); S is overwritten. Writes E = Q^T (row-major, ldE)
// and, if Qout != nullptr, Q (row-major, ldQ), with column signs such that
// diag(R) >= 0. Every kernel is skipped when pred != nullptr and *pred == 0.
mao_status qr_core(float* S, int64_t ldS, int n, float* E, int64_t ldE, float* Qout,
                   int64_t ldQ, QrWork& w, const int* pred, hipStream_t stream);

}  // namespace mao
