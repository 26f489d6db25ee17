// Test infrastructure: the two correctly rounded binary32 operations the AdamW
// update relies on (square root and division), compiled with the same
// compiler and numerics flags as the library's kernels, so that tests can
// compare them against the host's IEEE-754 results over every input pattern
// (square root) and over random and edge-case operand pairs (division).
// Not part of the library; nothing in the product loads it.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;

__global__ void k_sqrt_range(uint32_t base, uint32_t count, float* out) {
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i < count) out[i] = sqrtf(__uint_as_float(base + i));
}

__global__ void k_div(const float* a, const float* b, float* out, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (i < n) out[i] = a[i] / b[i];
}

}  // namespace

// out[i] = sqrtf(bit pattern base + i) for i < count. Requires
// base + count <= 2^32 and count <= 2^30 (returns 1 otherwise, 2 on a launch
// error). `out` is a device buffer of count floats.
extern "C" int probe_sqrt_range(uint32_t base, uint32_t count, float* out, hipStream_t stream) {
  if (uint64_t(base) + count > (uint64_t(1) << 32) || count > (1u << 30) || (count && !out))
    return 1;
  if (count == 0) return 0;
  k_sqrt_range<<<(count + kThreads - 1) / kThreads, kThreads, 0, stream>>>(base, count, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// out[i] = a[i] / b[i] for i < n; device buffers of n floats each.
extern "C" int probe_div(const float* a, const float* b, float* out, int64_t n,
                         hipStream_t stream) {
  if (n < 0 || n > (int64_t(1) << 30) || (n && (!a || !b || !out))) return 1;
  if (n == 0) return 0;
  const unsigned grid = static_cast<unsigned>((n + kThreads - 1) / kThreads);
  k_div<<<grid, kThreads, 0, stream>>>(a, b, out, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
