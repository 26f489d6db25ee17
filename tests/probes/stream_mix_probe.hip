// Measurement reference (test and bench infrastructure, not part of the
// library): the memory traffic of the fused reduce + AdamW + bf16 step with
// the AdamW arithmetic taken out. It reads 8 bf16 rows and three fp32 arrays
// and writes three fp32 arrays and one bf16 array, 42 bytes per element, with
// the fused kernel's lane layout (4 consecutive elements per lane: one 8-byte
// load per row, one 16-byte load or store per fp32 array, one 8-byte bf16
// store), its loads (buffer loads through per-tile descriptors; streaming on
// the rows, ordinary on the fp32 arrays) in its stages (the 8 rows issued
// together and added, then the fp32 state), its stores (device-scope
// streaming buffer stores bounded to the workgroup's tile), one tile per
// workgroup and a caller-chosen workgroup size and per-CU cap. What it
// computes is only a pass-through that keeps every load live: p + (sum of the
// rows), m and v unchanged, and the high half of the new p as the bf16 value.
// Its time is the stream-mix ceiling the fused kernel is compared with.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 8;
constexpr int kCpol = 18;   // sc1 nt: device-scope streaming store

struct Args {
  const uint16_t* g[kRows];
  float* p;
  float* m;
  float* v;
  uint16_t* w;
  int64_t n;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ u32x2 ld8(const uint16_t* base, int64_t len, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(rsrc(const_cast<uint16_t*>(base), 2 * len), off, 0,
                                              2);   // nt
}
__device__ __forceinline__ u32x4 ld16(const float* base, int64_t len, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc(const_cast<float*>(base), 4 * len), off, 0, 0);
}

__global__ __launch_bounds__(256) void k_stream_mix(Args a) {
  const int64_t tile = int64_t(blockDim.x) * 4;
  const int64_t t0 = int64_t(blockIdx.x) * tile;
  const int64_t i = t0 + int64_t(threadIdx.x) * 4;
  // n and the row pointers fetched together, as the fused kernel does
#pragma unroll
  for (int k = 0; k < kRows; ++k) asm volatile("" : : "s"(a.g[k]), "s"(a.n));
  if (i + 4 > a.n) return;   // the caller passes n a multiple of 4
  const int64_t tl = a.n - t0 < tile ? a.n - t0 : tile;
  const int off = int(4 * (i - t0));
  u32x2 q[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) q[k] = ld8(a.g[k] + t0, tl, off / 2);
  asm volatile("" : : "s"(a.p), "s"(a.m), "s"(a.v), "s"(a.w));   // fetched while the rows load
  __builtin_amdgcn_sched_barrier(0);
  float s[4] = {-0.0f, -0.0f, -0.0f, -0.0f};
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    s[0] = s[0] + __uint_as_float(q[k].x << 16);
    s[1] = s[1] + __uint_as_float(q[k].x & 0xFFFF0000u);
    s[2] = s[2] + __uint_as_float(q[k].y << 16);
    s[3] = s[3] + __uint_as_float(q[k].y & 0xFFFF0000u);
  }
  __builtin_amdgcn_sched_barrier(0);
  const u32x4 p = ld16(a.p + t0, tl, off);
  const u32x4 m = ld16(a.m + t0, tl, off);
  const u32x4 v = ld16(a.v + t0, tl, off);
  const u32x4 po = {__float_as_uint(__uint_as_float(p.x) + s[0]),
                    __float_as_uint(__uint_as_float(p.y) + s[1]),
                    __float_as_uint(__uint_as_float(p.z) + s[2]),
                    __float_as_uint(__uint_as_float(p.w) + s[3])};
  const u32x2 wo = {(po.x >> 16) | (po.y & 0xFFFF0000u), (po.z >> 16) | (po.w & 0xFFFF0000u)};
  __builtin_amdgcn_raw_buffer_store_b128(po, rsrc(a.p + t0, 4 * tl), off, 0, kCpol);
  __builtin_amdgcn_raw_buffer_store_b128(m, rsrc(a.m + t0, 4 * tl), off, 0, kCpol);
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc(a.v + t0, 4 * tl), off, 0, kCpol);
  __builtin_amdgcn_raw_buffer_store_b64(wo, rsrc(a.w + t0, 2 * tl), off / 2, 0, kCpol);
}

}  // namespace

// One launch over n elements (n a positive multiple of 4). rows: 8 device
// pointers to bf16 arrays of n elements (8-byte aligned); p, m, v: fp32
// arrays of n elements (16-byte aligned), updated in place; w: bf16 output of
// n elements (8-byte aligned). threads: 64, 128 or 256 per workgroup;
// wg_per_cu: resident workgroups per CU (0 = no cap; else held down with
// unused dynamic LDS). Returns 0, 1 on a bad argument (nothing launched) or
// 2 on a launch error.
extern "C" int probe_stream_mix(const void* const* rows, float* p, float* m, float* v, void* w,
                                int64_t n, int threads, int wg_per_cu, hipStream_t stream) {
  if (n <= 0 || n % 4 || n / 4 > (int64_t(1) << 31) || !rows || !p || !m || !v || !w) return 1;
  if (threads != 64 && threads != 128 && threads != 256) return 1;
  Args a{};
  for (int k = 0; k < kRows; ++k) {
    if (!rows[k] || (reinterpret_cast<uintptr_t>(rows[k]) & 7u)) return 1;
    a.g[k] = static_cast<const uint16_t*>(rows[k]);
  }
  if ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(m) |
       reinterpret_cast<uintptr_t>(v)) & 15u)
    return 1;
  if (reinterpret_cast<uintptr_t>(w) & 7u) return 1;
  a.p = p;
  a.m = m;
  a.v = v;
  a.w = static_cast<uint16_t*>(w);
  a.n = n;
  size_t lds = 0;
  if (wg_per_cu > 0) {
    int dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
            hipSuccess)
      return 2;
    for (int64_t granule : {int64_t(4096), int64_t(512)}) {
      const int64_t r = int64_t(per_cu) / wg_per_cu / granule * granule;
      if (r > 0 && (wg_per_cu + 1) * r > per_cu) { lds = size_t(r); break; }
    }
    if (!lds) return 1;
  }
  const int64_t tile = int64_t(threads) * 4;
  const unsigned grid = static_cast<unsigned>((n + tile - 1) / tile);
  k_stream_mix<<<grid, threads, lds, stream>>>(a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
