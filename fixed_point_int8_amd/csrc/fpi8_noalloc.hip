// fpi8_noalloc.hip - the standalone matrix row over packed tiles for callers
// that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// fpi8_matrix_rows_packed takes a workspace from its caller: the overflow
// word and the digit planes of the inputs.  This variant keeps that
// workspace in a file-scope device array instead, one per GPU, so a call
// allocates nothing.  The array's device address comes from
// hipGetSymbolAddress, taken once per device on the first call made with
// that device current, and is what every launch receives; the array's name
// is never passed to a kernel (in host code it is only a stand-in).
//
// Nothing in the array needs clearing between calls: each call marks an
// input word beyond three digits with a number of its own (a stale match
// only selects the exact path, with the same result), and digit words past
// the inputs only fill product columns that are never stored.  All calls
// on one GPU share its array: calls that overlap on one GPU race.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fpi8.h"
#include "fpi8_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[FPI8_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
void *g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of this GPU's array (nullptr on failure).
void *scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int32_t fpi8_matrix_rows_packed_noalloc(const uint8_t *d_P, const uint32_t *d_scale,
                                                   uint32_t rows, uint32_t cols, const int64_t *d_x,
                                                   uint32_t batch, int64_t *d_y, void *stream) {
  if (!d_P || rows == 0 || cols == 0 || batch == 0 || cols > FPI8_NOALLOC_MAX_COLS ||
      batch > FPI8_NOALLOC_MAX_BATCH)
    return FPI8_ERR_ARGUMENT;
  const uint64_t need = fpi8_matrix_rows_workspace_size(rows, cols, batch);
  if (need > FPI8_NOALLOC_WORKSPACE_BYTES) return FPI8_ERR_ARGUMENT;
  void *ws = scratch_on_current_device();
  if (!ws) return FPI8_ERR_HIP;
  return fpi8::matrix_rows(nullptr, d_P, d_scale, rows, cols, d_x, batch, d_y, ws,
                           FPI8_NOALLOC_WORKSPACE_BYTES, stream, false);
}
