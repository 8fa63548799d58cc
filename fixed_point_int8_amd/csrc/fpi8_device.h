// fpi8_device.h - device helpers shared by the HIP kernel files of the
// fixed-point forward pass: wrapping 64-bit arithmetic ("Fixed-point
// arithmetic"), the signed base-256 digits of an input word and their
// fragment-major planes, and wave-level wait and barrier primitives.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fpi8_internal.h"

namespace fpi8 {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t wmul(int64_t a, int64_t b) {
  return (int64_t)((uint64_t)a * (uint64_t)b);
}
__device__ __forceinline__ int64_t wadd(int64_t a, int64_t b) {
  return (int64_t)((uint64_t)a + (uint64_t)b);
}
__device__ __forceinline__ int64_t wsub(int64_t a, int64_t b) {
  return (int64_t)((uint64_t)a - (uint64_t)b);
}

// Signed base-256 digits of x (three of them); false when x needs more.
__device__ __forceinline__ bool digits3(int64_t x, int8_t &d0, int8_t &d1, int8_t &d2) {
  const bool fits = x >= -8421504LL && x <= 8355711LL;  // -128*65793 .. 127*65793
  d0 = (int8_t)(uint8_t)(x & 0xFF);
  const int64_t t1 = wsub(x, d0) >> 8;
  d1 = (int8_t)(uint8_t)(t1 & 0xFF);
  const int64_t t2 = wsub(t1, d1) >> 8;
  d2 = (int8_t)(uint8_t)(t2 & 0xFF);
  return fits;
}

// Digit planes are stored fragment-major: the 16 bytes a lane of a
// 16x16x64 MFMA needs are contiguous, and so are the 1 KB fragments of a
// 64-column block, so the row kernel stages them with whole-line loads.
// Byte (run b, column k) of a limb plane:
//   (((b / 16) * (kp / 64) + k / 64) * 64 + ((k % 64) / 16) * 16 + b % 16) * 16 + k % 16
__device__ __forceinline__ uint64_t digit_at(uint32_t b, uint32_t k, uint32_t kp) {
  return ((((uint64_t)(b >> 4) * (kp >> 6) + (k >> 6)) * 64 + ((k & 63) >> 4) * 16 + (b & 15)) << 4) +
         (k & 15);
}

// Whether some input word of the launch needs more than three digits, read
// through the scalar cache so the check does not queue behind vector loads.
__device__ __forceinline__ bool input_needs_exact(const RowsArgs &a) {
  if (a.oflag == nullptr) return false;
  const uint32_t f = *(const __attribute__((address_space(4))) uint32_t *)(uintptr_t)a.oflag;
  return a.oflag_seq ? f == a.oflag_seq : f != 0;
}

typedef __attribute__((address_space(3))) void lds_void;

// Waits until at most N vector memory operations of this wave are still
// outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt holds six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// A workgroup barrier that orders LDS accesses only.  __syncthreads() would
// also wait for every outstanding global load of the wave (its release
// fence), which would empty the prefetch ring at each stage; the staging
// loads a stage needs are awaited explicitly before this barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace fpi8
