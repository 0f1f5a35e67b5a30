// Symmetric eigendecomposition (block Jacobi) for FOAM's eigenbasis refresh.
#pragma once

#include "common.hpp"

namespace mao {

constexpr int kEighMaxN = 16384;   // largest factor the eigensolver takes
constexpr int kEighMaxSweeps = 12; // outer Jacobi sweeps at most

// One job: D (n x n, row-major, ld ldD) is the factor expressed in the basis
// whose columns are Q (n x n, ld ldQ): D = Q^T F Q. The solver finds V with
// V^T D V diagonal and overwrites Q by Q V with its columns ordered by
// descending eigenvalue; where E != nullptr it also writes E = (Q V)^T. D is
// read only (its symmetric part is used). evals (nullable) receives the n
// eigenvalues in the same order.
struct EighJob {
  const float* D = nullptr;
  int64_t ldD = 0;
  float* Q = nullptr;
  int64_t ldQ = 0;
  float* E = nullptr;
  int64_t ldE = 0;
  float* evals = nullptr;
};

// Several eigendecompositions of one size n in one set of launches. Job j
// uses the j-th block of eigh_work_stride(n) bytes at `work` (256-byte
// aligned) and is skipped where pred != nullptr and pred[j spred] == 0.
// info (nullable): per job kEighMaxSweeps + 1 floats -- the off-diagonal
// ratio ||D - diag D||_F / ||D||_F after each sweep (0 once converged), then
// the number of sweeps run.
struct EighBatch {
  int n = 0, njob = 0;
  const EighJob* jobs = nullptr;  // host array of njob
  const int* pred = nullptr;
  int64_t spred = 0;
  char* work = nullptr;
  float* info = nullptr;
};

size_t eigh_work_stride(int n);
mao_status eigh_batched(const EighBatch& b, hipStream_t stream);

}  // namespace mao
