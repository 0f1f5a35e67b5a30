// muon_step without a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). The step's scratch memory (the Newton-Schulz
// iterates, the Gram and polynomial matrices, the norm partials) lives in one
// file-scope device array of fixed size, which the code object brings onto
// every GPU the library runs on and which stays there until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: on the host
// that name stands for a host-side shadow, not for device memory. Each
// device's own address comes from hipGetSymbolAddress, taken once per device
// (on the first call made with that device current) and kept in a table.
#include <mutex>

#include "common.hpp"

namespace mao {

constexpr size_t kScratchBytes = (size_t)MAO_NOALLOC_SCRATCH_BYTES;

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

mao_status scratch_on_current_device(void** out) {
  int dev = -1;
  MAO_HIP_CHECK(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device %d outside the %d-entry scratch table", dev, kMaxDevices);
    return MAO_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    MAO_HIP_CHECK(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (p == nullptr || (uintptr_t)p % 256 != 0) {
      set_error("scratch array address %p on device %d is not 256-byte aligned", p, dev);
      return MAO_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MAO_OK;
}

}  // namespace
}  // namespace mao

using namespace mao;

extern "C" {

MAO_API size_t muon_step_noalloc_max_bytes(void) { return kScratchBytes; }

MAO_API mao_status muon_step_noalloc(mao_mat W, mao_mat G, mao_mat M, const mao_muon_hparams* hp,
                                     float* update_out, void* stream) {
  if (hp == nullptr) {
    set_error("hp is NULL");
    return MAO_E_NULL;
  }
  // sizes first: a request beyond the scratch array fails before any HIP call
  const size_t need = muon_workspace_size(W.rows, W.cols, hp);
  if (need > kScratchBytes) {
    set_error("muon_step_noalloc: a %lldx%lld step needs %zu bytes of scratch, above the "
              "%zu-byte static array (use muon_step with a workspace)",
              (long long)W.rows, (long long)W.cols, need, kScratchBytes);
    return MAO_E_WORKSPACE;
  }
  if (stream != nullptr) {
    int sdev = -1, cdev = -1;
    MAO_HIP_CHECK(hipStreamGetDevice((hipStream_t)stream, &sdev));
    MAO_HIP_CHECK(hipGetDevice(&cdev));
    if (sdev != cdev) {
      set_error("muon_step_noalloc: stream of device %d, current device %d", sdev, cdev);
      return MAO_E_UNSUPPORTED;
    }
  }
  void* ws = nullptr;
  MAO_TRY(scratch_on_current_device(&ws));
  return muon_step(W, G, M, hp, ws, kScratchBytes, update_out, stream);
}

}  // extern "C"
