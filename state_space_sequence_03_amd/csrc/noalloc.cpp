// mamba3_ssm_chunked_fwd_noalloc: the chunked forward with its workspace taken
// from a fixed device array of the library instead of the caller, for callers
// that cannot allocate (code under HIP graph capture, tight serving loops).
//
// The array is a file-scope __device__ variable, so every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Its
// device address is looked up once per device (hipGetSymbolAddress, with that
// device current) and kept; host code never uses the variable's name as an
// address.  The forward's workspace needs no initial contents (every byte the
// walk reads is written first in the same call), so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mamba3_ssm.h"

namespace {

__device__ __align__(256) unsigned char scratch[M3_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
void* g_ptr[MAX_DEVICES];
hipError_t g_err[MAX_DEVICES];
std::once_flag g_once[MAX_DEVICES];

// The device address of this device's copy of the array (nullptr on error).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" m3_status mamba3_ssm_chunked_fwd_noalloc(const m3_dims* d, const void* x, const void* B, const void* C,
                                                    const float* dt, const float* A, const float* lam,
                                                    const float* theta, const float* h0, const void* prev_B,
                                                    const void* prev_x, void* y, float* h_final, void* stream) {
  if (!d) return M3_ERR_NULL;
  // host-side size check first: no HIP call for a request the array cannot hold
  const size_t need = mamba3_ssm_chunked_fwd_workspace_size(d);
  if (need > (size_t)M3_NOALLOC_SCRATCH_BYTES) return M3_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (!ws) return M3_ERR_HIP;
  }
  return mamba3_ssm_chunked_fwd(d, x, B, C, dt, A, lam, theta, h0, prev_B, prev_x, y, h_final, ws,
                                ws ? (size_t)M3_NOALLOC_SCRATCH_BYTES : 0, stream);
}
