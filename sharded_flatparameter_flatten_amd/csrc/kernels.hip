// HIP kernels of libfsdpshard.so for CDNA4 (gfx950) and the device entry
// points of the C ABI (include/fsdp_shard.h).
//
// Everything on this path streams through HBM once; nothing is a dense
// contraction, so there is no MFMA here. The design is about bytes:
//  * step kernels (reduce, AdamW, fused): each lane owns 4 consecutive shard
//    elements, so a gradient row is one 8-byte load and each fp32 state array
//    one 16-byte access; every load and store instruction of a 64-lane
//    wavefront covers one contiguous range (no line is written in pieces by
//    different instructions, which costs dearly on the write path);
//  * the fused step reads the n_grads gradient rows, master, m and v once and
//    writes master, m, v (and the bf16 parameter) once: the fp32 reduced
//    gradient never touches memory;
//  * cache policy, chosen by measurement on MI355X with rotating buffer sets
//    (no reuse between steps): the gradient rows are read once, so their
//    loads carry the streaming (nontemporal) hint; the fp32 state loads stay
//    ordinary; every vector store of the step and copy kernels is a
//    device-scope streaming store (buffer store with sc1 nt) through a
//    descriptor bounded to the workgroup's tile. With ordinary or plain
//    nontemporal stores, part of a kernel's writes was still being written
//    back while the next kernel ran and slowed it; the streaming stores
//    finish inside the kernel that issues them, and the 7B-block step
//    (fused + gather) went from ~318 us to ~307 us;
//  * occupancy, also chosen by measurement (step_shape below): long launches
//    of the reduce, AdamW and fused kernels run one-wave workgroups
//    (256-element tiles), as many per CU as keep about 80 KiB of loads and
//    stores in flight per CU, except the fused step with 8 or more rows,
//    which stages its tile loads (8 rows at a time, then the fp32 state) and
//    runs 10 per CU in a one-tile kernel; the per-CU counts are held down by
//    unused dynamic LDS sized from the device's LDS per CU;
//  * buffers that are not aligned (e.g. a rank window r*S with S odd) take a
//    lane-strided scalar path, still coalesced per instruction;
//  * the gather/unflatten and flatten/pad copies are planned on the host as
//    (source, destination, length) segments (tensor x shard intersections),
//    passed in kernel arguments and walked per workgroup with a scalar
//    cursor; each lane moves one 16-byte source vector.
//
// Numerics: every floating-point step is one binary32 operation with round to
// nearest even. The file is compiled with -ffp-contract=off (and the pragma
// below) so no multiply-add is fused; division and sqrt use the correctly
// rounded expansions (the HIP default, never -ffast-math); fp32 denormals are
// kept.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <string>
#include <vector>

#include "fsdp_internal.h"

#pragma clang fp contract(off)

#ifndef FSDP_COPY_BLOCK
#define FSDP_COPY_BLOCK 64    // threads per workgroup, copy kernels (one wave)
#endif
#ifndef FSDP_STEP_BLOCK
#define FSDP_STEP_BLOCK 256   // threads per workgroup of the step launches not in one-wave shape
#endif
#ifndef FSDP_GRAD_NT_LOAD
#define FSDP_GRAD_NT_LOAD 1   // streaming hint on the gradient-row loads (read once)
#endif
#ifndef FSDP_STATE_NT_LOAD
#define FSDP_STATE_NT_LOAD 0  // streaming hint on the fp32 state loads
#endif
#ifndef FSDP_COPY_NT_LOAD
#define FSDP_COPY_NT_LOAD 0    // streaming hint on the copy kernels' source loads
#endif
// Cache policy of the step and copy kernels' vector stores: the CPol operand
// of the gfx950 buffer store (1 = sc0, 2 = nt, 16 = sc1). The default, 18, is a
// device-scope streaming store (sc1 nt). -1 selects plain global stores
// instead (with the nontemporal hint on the step kernels).
#ifndef FSDP_STEP_STORE_CPOL
#define FSDP_STEP_STORE_CPOL 18
#endif
#ifndef FSDP_COPY_STORE_CPOL
#define FSDP_COPY_STORE_CPOL 18
#endif

// Resident 256-thread workgroups per CU of the batched many-unit fused kernel
// (0: no cap), imposed with unused dynamic LDS on batches of at least
// 2^FSDP_CAP_MIN_LOG2 elements; the single-unit step launches of that size
// take their shape from step_shape.
#ifndef FSDP_MULTI_WG_PER_CU
#define FSDP_MULTI_WG_PER_CU 3
#endif
#ifndef FSDP_CAP_MIN_LOG2
#define FSDP_CAP_MIN_LOG2 23
#endif
// Bytes each lane of a one-wave workgroup should have moving per CU slot (see
// step_shape): one-wave workgroups per CU = FSDP_LANE_BUDGET / lane bytes.
#ifndef FSDP_LANE_BUDGET
#define FSDP_LANE_BUDGET 1280
#endif
// One-wave workgroups per CU for the fused step with a run-time row count
// (folded flat in chunks of 8 rows) on 2^FSDP_CAP_MIN_LOG2+ elements.
#ifndef FSDP_CHUNKED_WG_PER_CU
#define FSDP_CHUNKED_WG_PER_CU 12
#endif

// One-wave workgroups per CU for the fused step with a compile-time fold of 8
// or more rows (its tile loads staged: see step_tile).
#ifndef FSDP_STAGED_WG_PER_CU
#define FSDP_STAGED_WG_PER_CU 10
#endif

using fsdp::fail;

namespace {

constexpr int kThreads = FSDP_COPY_BLOCK;
constexpr int kStepThreads = FSDP_STEP_BLOCK;
constexpr int kSmallThreads = 64;   // one wave
constexpr int kSV = 4;   // consecutive elements per lane in the step kernels
constexpr int64_t kStepTile = int64_t(kStepThreads) * kSV;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// element numerics
// ---------------------------------------------------------------------------

// bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float widen(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN -> canonical quiet NaN.
// Adding 0x7FFF plus the lowest kept bit rounds the dropped half correctly and
// carries into the exponent (up to infinity) when the kept part overflows.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t x = __float_as_uint(f);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (x + 0x7FFFu + ((x >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return to_bf16(a) | (to_bf16(b) << 16);
}

struct Adam {
  float gs, b1, omb1, b2, omb2, bc1, bc2, lr, eps, wd;
};

// One AdamW element (Adam with bias correction, decoupled decay scaled by lr).
__device__ __forceinline__ void adamw(float g, float& p, float& m, float& v, const Adam& s) {
  const float m_new = s.b1 * m + s.omb1 * g;
  const float v_new = s.b2 * v + s.omb2 * (g * g);
  const float m_hat = m_new / s.bc1;
  const float v_hat = v_new / s.bc2;
  const float denom = sqrtf(v_hat) + s.eps;
  const float u = m_hat / denom;
  p = p - s.lr * (u + s.wd * p);
  m = m_new;
  v = v_new;
}

// ---------------------------------------------------------------------------
// memory helpers (128-bit)
// ---------------------------------------------------------------------------

template <typename V, bool NT>
__device__ __forceinline__ V ldh(const void* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}
template <typename V, bool NT>
__device__ __forceinline__ void st(void* p, V x) {
  if constexpr (NT) __builtin_nontemporal_store(x, reinterpret_cast<V*>(p));
  else *reinterpret_cast<V*>(p) = x;
}
constexpr int kStepCpol = FSDP_STEP_STORE_CPOL;
constexpr int kCopyCpol = FSDP_COPY_STORE_CPOL;
constexpr bool kGradNt = FSDP_GRAD_NT_LOAD != 0;
constexpr bool kCopyNtLoad = FSDP_COPY_NT_LOAD != 0;
constexpr bool kStateNt = FSDP_STATE_NT_LOAD != 0;

// A lane's 4 consecutive elements: one 8-byte bf16 access per row and one
// 16-byte access per fp32 array.
__device__ __forceinline__ void unpack(u32x2 q, float (&x)[4]) {
  x[0] = lo_bf16(q.x); x[1] = hi_bf16(q.x);
  x[2] = lo_bf16(q.y); x[3] = hi_bf16(q.y);
}
__device__ __forceinline__ void accumulate(u32x2 q, float (&x)[4]) {
  x[0] = x[0] + lo_bf16(q.x); x[1] = x[1] + hi_bf16(q.x);
  x[2] = x[2] + lo_bf16(q.y); x[3] = x[3] + hi_bf16(q.y);
}

// Buffer descriptor over [base, base + bytes) with the gfx9 raw-buffer format
// word; a store beyond it is dropped by the hardware.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, static_cast<int>(bytes), kRsrcWord3);
}
template <int CP>
__device__ __forceinline__ void bst(__amdgpu_buffer_rsrc_t r, int off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP);
}
template <int CP>
__device__ __forceinline__ void bst(__amdgpu_buffer_rsrc_t r, int off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CP);
}

// Where a lane's accesses of one tile start: the tile's first element t0 and
// its length (both workgroup-uniform) and the lane's element offset within
// the tile. A load is a buffer load through a descriptor over the tile, so
// its base stays in scalar registers and the lane adds a 32-bit byte offset
// (no 64-bit address arithmetic per row in vector registers, which otherwise
// limits how many loads the compiler keeps in flight).
struct At {
  int64_t t0;
  int64_t len;
  uint32_t off;
};
// present == false: a zero-length descriptor, so the load reads no memory and
// returns zeros.
template <typename V, bool NT, typename T>
__device__ __forceinline__ V ld_tile(const T* base, At at, bool present = true) {
  const __amdgpu_buffer_rsrc_t r =
      rsrc(const_cast<T*>(base) + at.t0, present ? int64_t(sizeof(T)) * at.len : 0);
  const int off = int(at.off * uint32_t(sizeof(T)));
  constexpr int cp = NT ? 2 : 0;   // 2: nt (streaming)
  if constexpr (sizeof(V) == 8) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, cp);
  else return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, cp);
}

// A lane's 4 consecutive fp32 values of a tile.
__device__ __forceinline__ void loadf(const float* base, At at, float (&x)[4]) {
  const u32x4 a = ld_tile<u32x4, kStateNt>(base, at);
  x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
  x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
}

// One lane's 4 results at element i of a workgroup tile that starts at
// element t0 of `base` and holds `len` elements (all workgroup-uniform but i).
// Each store is a single 16-byte (fp32) or 8-byte (bf16) access.
__device__ __forceinline__ void out_f32(float* base, int64_t t0, int64_t len, int64_t i,
                                        const float (&x)[4]) {
  const u32x4 b = {__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                   __float_as_uint(x[3])};
  if constexpr (kStepCpol >= 0) bst<kStepCpol>(rsrc(base + t0, 4 * len), int(4 * (i - t0)), b);
  else st<u32x4, true>(base + i, b);
}
__device__ __forceinline__ void out_bf16(uint16_t* base, int64_t t0, int64_t len, int64_t i,
                                         const float (&x)[4]) {
  const u32x2 b = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
  if constexpr (kStepCpol >= 0) bst<kStepCpol>(rsrc(base + t0, 2 * len), int(2 * (i - t0)), b);
  else st<u32x2, true>(base + i, b);
}

// ---------------------------------------------------------------------------
// reduce / AdamW / fused step kernels
// ---------------------------------------------------------------------------

struct StepArgs {
  // rank-window start of each contribution; 8 more null entries, so that a
  // chunk of 8 row pointers starting below n_grads stays inside the array
  const uint16_t* g[FSDP_MAX_RANKS + 8];
  const float* grad;                  // AdamW input (unfused)
  float* out;                         // reduce output (unfused)
  float* p;
  float* m;
  float* v;
  uint16_t* w;                        // bf16 parameter out, or null
  int64_t n;                          // shard_valid
  int32_t n_grads;
  int32_t group;                      // rows per replica group (== n_grads: one flat fold)
  int32_t bf16acc;                    // 1: every partial sum rounded to bf16
  int32_t runs;                       // 1: tiles visited in XCD runs (shift_tile)
  Adam s;
};

enum class Op { Reduce, AdamW, Fused };

// Left fold of the gradient rows for SV consecutive elements of a tile,
// times gs. NG > 0 is the compile-time count: every row load is issued (and
// held issued by a scheduling barrier) before the first add; with STAGE the
// rows go in stages of up to 8 instead, each stage's loads issued together and
// added before the next stage is issued (same adds, same order). NG == 0 reads the
// count at run time and folds chunks of 8 rows, each chunk's loads issued
// before its first add. That fold starts from -0.0, the exact identity of IEEE
// addition (-0 + x is x for every x, -0, infinities and NaN included), so its
// sums are those of the fold that starts from the first row; in the last,
// partial chunk the rows past the count load nothing (a zero-length
// descriptor) and add -0.0. Reading g[k + j] there stays inside the array: the
// chunk starts at a multiple of 8 below n_grads <= FSDP_MAX_RANKS, so its last
// pointer is below FSDP_MAX_RANKS.
template <int NG, int SV, bool STAGE = false>
__device__ __forceinline__ void reduce_rows(const uint16_t* const* g, int ng, float gs,
                                            At at, float (&acc)[SV]) {
  using G = u32x2;
  if constexpr (NG > 0 && STAGE) {
    constexpr int C = NG < 8 ? NG : 8;
    static_assert(NG % C == 0, "whole stages");
#pragma unroll
    for (int c = 0; c < NG; c += C) {
      G q[C];
#pragma unroll
      for (int k = 0; k < C; ++k) q[k] = ld_tile<G, kGradNt>(g[c + k], at);
      __builtin_amdgcn_sched_barrier(0);
      if (c == 0) unpack(q[0], acc);
      else accumulate(q[0], acc);
#pragma unroll
      for (int k = 1; k < C; ++k) accumulate(q[k], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else if constexpr (NG > 0) {
    G q[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) q[k] = ld_tile<G, kGradNt>(g[k], at);
    __builtin_amdgcn_sched_barrier(0);
    unpack(q[0], acc);
#pragma unroll
    for (int k = 1; k < NG; ++k) accumulate(q[k], acc);
  } else {
    static_assert(FSDP_MAX_RANKS % 8 == 0, "whole chunks of row pointers");
#pragma unroll
    for (int e = 0; e < SV; ++e) acc[e] = -0.0f;
    int k = 0;
    for (; k + 8 <= ng; k += 8) {
      G q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = ld_tile<G, kGradNt>(g[k + j], at);
#pragma unroll
      for (int j = 0; j < 8; ++j) accumulate(q[j], acc);
    }
    if (k < ng) {
      G q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = ld_tile<G, kGradNt>(g[k + j], at, k + j < ng);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t dead = k + j < ng ? 0u : 0x80008000u;   // both halves -0.0
        accumulate(G{q[j].x | dead, q[j].y | dead}, acc);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < SV; ++e) acc[e] = acc[e] * gs;
}

// fp32 value -> nearest bf16 (ties to even), kept as an fp32 value.
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(to_bf16(f) << 16); }

// x += row, with every partial rounded to bf16 when BACC.
template <bool BACC>
__device__ __forceinline__ void add_row(u32x2 q, float (&x)[4]) {
  float t[4];
  unpack(q, t);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = BACC ? round_bf16(x[e] + t[e]) : x[e] + t[e];
}

// x += row (add_row) for a row of the group; a row past it (it loaded nothing)
// is skipped (live is uniform across the workgroup).
template <bool BACC>
__device__ __forceinline__ void add_chunk_row(u32x2 q, bool live, float (&x)[4]) {
  if (live) add_row<BACC>(q, x);
}

// The general left fold, for hybrid sharding and for bf16 partial sums. Rows
// [rho*group, (rho+1)*group) are one replica group: each group is folded on
// its own (the reduce-scatter inside the group), then the group sums are
// folded in group order (the all-reduce across groups), then scaled. With
// BACC every addition is an fp32 add followed by rounding to bf16. A group's
// rows are loaded in chunks of 8, each chunk's loads issued before its first
// add; the group's first row starts its partial sum. In the last, partial
// chunk the rows past the group load nothing and are not added.
template <int SV, bool BACC>
__device__ __forceinline__ void reduce_rows_general(const uint16_t* const* g, int ng, int group,
                                                    float gs, At at, float (&acc)[SV]) {
  using G = u32x2;
  for (int base = 0; base < ng; base += group) {
    float part[SV];
    for (int k = 0; k < group; k += 8) {   // g[base + k + 7]: inside the padded array
      G q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) q[j] = ld_tile<G, kGradNt>(g[base + k + j], at, k + j < group);
      if (k == 0) unpack(q[0], part);
      else add_chunk_row<BACC>(q[0], 0 < group - k, part);
#pragma unroll
      for (int j = 1; j < 8; ++j) add_chunk_row<BACC>(q[j], j < group - k, part);
    }
    if (base == 0) {
#pragma unroll
      for (int e = 0; e < SV; ++e) acc[e] = part[e];
    } else {
#pragma unroll
      for (int e = 0; e < SV; ++e) acc[e] = BACC ? round_bf16(acc[e] + part[e]) : acc[e] + part[e];
    }
  }
#pragma unroll
  for (int e = 0; e < SV; ++e) acc[e] = acc[e] * gs;
}

// The grouped fold of reduce_rows_general with compile-time counts: NG rows in
// groups of GRP (GRP == NG: one group, i.e. the flat fold with bf16 partials),
// all NG row loads issued before the first add, or with STAGE in stages of 8
// rows as in reduce_rows. Same operations in the same order as
// reduce_rows_general.
template <int NG, int GRP, bool BACC, bool STAGE = false>
__device__ __forceinline__ void reduce_rows_grouped(const uint16_t* const* g, float gs, At at,
                                                    float (&acc)[4]) {
  static_assert(NG % GRP == 0, "whole groups");
  if constexpr (STAGE) {
    constexpr int C = NG < 8 ? NG : 8;
    static_assert(NG % C == 0, "whole stages");
    float part[4];
#pragma unroll
    for (int c = 0; c < NG; c += C) {
      u32x2 q[C];
#pragma unroll
      for (int k = 0; k < C; ++k) q[k] = ld_tile<u32x2, kGradNt>(g[c + k], at);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < C; ++k) {
        const int r = c + k;                     // row index, a compile-time constant
        if (r % GRP == 0) unpack(q[k], part);
        else add_row<BACC>(q[k], part);
        if (r % GRP == GRP - 1) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[e] = r < GRP ? part[e] : (BACC ? round_bf16(acc[e] + part[e]) : acc[e] + part[e]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] * gs;
    return;
  }
  u32x2 q[NG];
#pragma unroll
  for (int k = 0; k < NG; ++k) q[k] = ld_tile<u32x2, kGradNt>(g[k], at);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < NG; b += GRP) {
    float part[4];
    unpack(q[b], part);
#pragma unroll
    for (int k = 1; k < GRP; ++k) add_row<BACC>(q[b + k], part);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc[e] = b == 0 ? part[e] : (BACC ? round_bf16(acc[e] + part[e]) : acc[e] + part[e]);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = acc[e] * gs;
}

// Scalar form of the general fold of the rows at element i.
__device__ __forceinline__ float reduce_element(const uint16_t* const* g, int ng, int group,
                                                bool bacc, float gs, int64_t i) {
  float acc = 0.f;
  for (int base = 0; base < ng; base += group) {
    float part = widen(g[base][i]);
    for (int k = 1; k < group; ++k) {
      part = part + widen(g[base + k][i]);
      if (bacc) part = round_bf16(part);
    }
    if (base == 0) {
      acc = part;
    } else {
      acc = acc + part;
      if (bacc) acc = round_bf16(acc);
    }
  }
  return acc * gs;
}

// One element of the fused step from raw pointers (tails of the vector paths).
__device__ __forceinline__ void fused_scalar(const uint16_t* const* g, int ng, float* p_,
                                             float* m_, float* v_, uint16_t* w_, int64_t i,
                                             const Adam& s) {
  const float gr = reduce_element(g, ng, ng, false, s.gs, i);
  float p = p_[i], m = m_[i], v = v_[i];
  adamw(gr, p, m, v, s);
  p_[i] = p;
  m_[i] = m;
  v_[i] = v;
  if (w_) w_[i] = static_cast<uint16_t>(to_bf16(p));
}

// A gradient row whose rank window does not start on an 8-byte boundary: the
// lane reads the two aligned 8-byte words that cover its 4 elements and
// funnel-shifts them together. Callers keep both words inside the window
// (group index >= 4 and at least 8 elements left), so nothing outside the
// bytes the step may read is touched.
__device__ __forceinline__ u32x2 ld_row_shifted(const uint16_t* p) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const uint64_t* q = reinterpret_cast<const uint64_t*>(a & ~uintptr_t(7));
  const unsigned sh = unsigned(a & 7u) * 8u;
  const uint64_t lo = ldh<uint64_t, kGradNt>(q);
  const uint64_t hi = ldh<uint64_t, kGradNt>(q + 1);
  const uint64_t v = sh ? (lo >> sh) | (hi << (64u - sh)) : lo;
  return u32x2{uint32_t(v), uint32_t(v >> 32)};
}

// Left fold of the shifted rows for the 4 elements at i, times gs. NG > 0:
// the compile-time count, every load issued before the first add. NG == 0:
// chunks of 8 rows from -0.0, as in reduce_rows (rows past the count are not
// read and add -0.0).
template <int NG>
__device__ __forceinline__ void reduce_rows_shifted(const StepArgs& a, int64_t i,
                                                    float (&acc)[4]) {
  if constexpr (NG > 0) {
    u32x2 q[NG];
#pragma unroll
    for (int k = 0; k < NG; ++k) q[k] = ld_row_shifted(a.g[k] + i);
    __builtin_amdgcn_sched_barrier(0);
    unpack(q[0], acc);
#pragma unroll
    for (int k = 1; k < NG; ++k) accumulate(q[k], acc);
  } else {
    static_assert(FSDP_MAX_RANKS % 8 == 0, "whole chunks of row pointers");
    const int ng = a.n_grads;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = -0.0f;
    for (int k = 0; k < ng; k += 8) {   // k + 7 < FSDP_MAX_RANKS: k is a multiple of 8 below ng
      u32x2 q[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        q[j] = k + j < ng ? ld_row_shifted(a.g[k + j] + i) : u32x2{0x80008000u, 0x80008000u};
#pragma unroll
      for (int j = 0; j < 8; ++j) accumulate(q[j], acc);
    }
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = acc[e] * a.s.gs;
}

template <Op OP>
__device__ __forceinline__ void step_scalar(const StepArgs& a, int64_t i) {
  float g;
  if constexpr (OP == Op::AdamW) {
    g = a.grad[i];
  } else {
    g = reduce_element(a.g, a.n_grads, a.group, a.bf16acc != 0, a.s.gs, i);
  }
  if constexpr (OP == Op::Reduce) {
    a.out[i] = g;
  } else {
    float p = a.p[i], m = a.m[i], v = a.v[i];
    adamw(g, p, m, v, a.s);
    a.p[i] = p;
    a.m[i] = m;
    a.v[i] = v;
    if (a.w) a.w[i] = static_cast<uint16_t>(to_bf16(p));
  }
}

// Tile of workgroup b when the tiles are visited in XCD runs: runs of kShiftRun
// consecutive tiles on one XCD (workgroup b runs on XCD b % 8). When an array's
// window does not start on a 128-byte line (every misaligned gradient row, and
// any array placed off a line boundary), each tile's first and last line of it
// also belong to the neighbouring tiles; tiles that share a line then share an
// L2, and the line moves between HBM and L2 once instead of once per XCD (with
// consecutive tiles on different XCDs, misaligned rows cost up to a quarter
// more HBM reads). The workgroups past the last whole group of 8 runs keep
// their own index. With every window on a line boundary the plain order is
// kept: the runs measured no faster there.
constexpr unsigned kShiftRun = 8;
__device__ __forceinline__ int64_t shift_tile(unsigned b, unsigned nb) {
  const unsigned whole = nb / (8 * kShiftRun) * (8 * kShiftRun);
  if (b >= whole) return b;
  const unsigned j = b / 8;
  return int64_t(j / kShiftRun) * (8 * kShiftRun) + (b % 8) * kShiftRun + j % kShiftRun;
}

// Whether the fused step stages its tile loads: the gradient rows in stages of
// 8 (each added before the next is issued), then the fp32 state. Measured on
// MI355X with rotating buffer sets, a wave that issues its 8 or 16 rows and
// its state at once (64-80% of a tile's loads in one burst) kept the stream
// mix 1-2% below a wave that keeps at most 8 rows' or the state's loads in
// flight, with 10 rather than 8 one-wave workgroups per CU. The run-time fold
// (chunks of 8 already) takes its state last too: 0-1.3% faster for 11 and 13
// rows, 1-5% for 64. With 1-7 rows a stage is too small to stand alone.
template <Op OP, int NG>
constexpr bool staged_tile() { return OP == Op::Fused && (NG >= 8 || NG == 0); }

// One workgroup tile of the vector path: elements [t0, t0 + tl), lane element i.
template <Op OP, int NG, bool EMIT, int GRP, bool BACC>
__device__ __forceinline__ void step_tile(const StepArgs& a, int64_t t0, int64_t tl, int64_t i) {
  const At at{t0, tl, uint32_t(threadIdx.x) * kSV};
  float g[kSV], p[kSV], m[kSV], v[kSV];
  // Unstaged, the state loads go first: with a compile-time row count every
  // load of the tile is then in flight before the first add, and the run-time
  // fold overlaps them with its first chunks.
  constexpr bool state_last = staged_tile<OP, NG>();
  if constexpr (OP != Op::Reduce && !state_last) {
    loadf(a.p, at, p);
    loadf(a.m, at, m);
    loadf(a.v, at, v);
  }
  if constexpr (OP == Op::AdamW) {
    loadf(a.grad, at, g);
  } else {
    if constexpr (NG == 0) {
      if (a.bf16acc)
        reduce_rows_general<kSV, true>(a.g, a.n_grads, a.group, a.s.gs, at, g);
      else if (a.group < a.n_grads)
        reduce_rows_general<kSV, false>(a.g, a.n_grads, a.group, a.s.gs, at, g);
      else
        reduce_rows<0, kSV>(a.g, a.n_grads, a.s.gs, at, g);
    } else if constexpr (GRP > 0) {
      reduce_rows_grouped<NG, GRP, BACC, state_last>(a.g, a.s.gs, at, g);
    } else {
      reduce_rows<NG, kSV, state_last>(a.g, a.n_grads, a.s.gs, at, g);
    }
  }
  if constexpr (state_last) {
    __builtin_amdgcn_sched_barrier(0);
    loadf(a.p, at, p);
    loadf(a.m, at, m);
    loadf(a.v, at, v);
  }
  if constexpr (OP == Op::Reduce) {
    out_f32(a.out, t0, tl, i, g);
  } else {
#pragma unroll
    for (int e = 0; e < kSV; ++e) adamw(g[e], p[e], m[e], v[e], a.s);
    out_f32(a.p, t0, tl, i, p);
    out_f32(a.m, t0, tl, i, m);
    out_f32(a.v, t0, tl, i, v);
    if constexpr (EMIT) out_bf16(a.w, t0, tl, i, p);
  }
}

// Vector path: bf16 rows aligned to 2*kSV bytes, fp32 buffers to 16 bytes.
// Lane t of a tile owns elements [tile + kSV*t, tile + kSV*t + kSV), so every
// load and store instruction of a wavefront covers one contiguous range; the
// last partial group falls back to scalars.
template <Op OP, int NG, bool EMIT, int GRP = 0, bool BACC = false>
__global__ __launch_bounds__(kStepThreads) void k_step_vec(StepArgs a) {
  const int64_t n = a.n;
  const int64_t tile = int64_t(blockDim.x) * kSV;          // 64 or 256 threads per workgroup
  const int64_t stride = int64_t(gridDim.x) * tile;
  const int64_t first = a.runs ? shift_tile(blockIdx.x, gridDim.x) : int64_t(blockIdx.x);
  for (int64_t t0 = first * tile; t0 < n; t0 += stride) {
    // t0, this tile's first element, is workgroup-uniform (the store descriptors
    // are built from it in scalar registers)
    const int64_t i = t0 + int64_t(threadIdx.x) * kSV;
    if (i >= n) continue;
    if (i + kSV <= n) {
      const int64_t tl = n - t0 < tile ? n - t0 : tile;
      step_tile<OP, NG, EMIT, GRP, BACC>(a, t0, tl, i);
    } else {
      for (int64_t j = i; j < n; ++j) step_scalar<OP>(a, j);
    }
  }
}

// The vector path with one-wave workgroups and one tile each (grid = the tile
// count, tiles in plain order), for the staged fused step (8 or 16 rows, the
// compile-time grouped folds, and the flat run-time fold). The kernel
// arguments the first stage needs are fetched in one scalar round trip (the
// general kernel's loop and XCD-run test cost a second one before the first
// row load); that start-up latency is paid once per tile and, with staged
// loads, showed up in the stream rate.
template <int NG, bool EMIT, int GRP = 0, bool BACC = false>
__global__ __launch_bounds__(kSmallThreads) void k_step_one(StepArgs a) {
  constexpr int64_t tile = int64_t(kSmallThreads) * kSV;
  const int64_t t0 = int64_t(blockIdx.x) * tile;
  const int64_t i = t0 + int64_t(threadIdx.x) * kSV;
  const int64_t n = a.n;
  // empty uses that make the compiler fetch n and the row pointers together
#pragma unroll
  for (int k = 0; k < NG; ++k) asm volatile("" : : "s"(a.g[k]), "s"(n));
  if (t0 + tile <= n) {
    step_tile<Op::Fused, NG, EMIT, GRP, BACC>(a, t0, tile, i);
  } else if (i + kSV <= n) {
    step_tile<Op::Fused, NG, EMIT, GRP, BACC>(a, t0, n - t0, i);
  } else {
    for (int64_t j = i; j < n; ++j) step_scalar<Op::Fused>(a, j);
  }
}

// Shifted-row path: fp32 state (and the bf16 output) aligned, gradient rows
// only 2-byte aligned (a rank window r*S with r*S not a multiple of 4). The
// lane layout and tiles of the vector path, the tiles always visited in XCD
// runs; the first group and the last 8 elements go through the scalar step.
template <Op OP, int NG, bool EMIT>
__global__ __launch_bounds__(kStepThreads) void k_step_shift(StepArgs a) {
  static_assert(OP != Op::AdamW, "only the gradient rows are shifted");
  constexpr int V = 4;
  const int64_t TILE = int64_t(blockDim.x) * V;          // 64 or 256 threads
  const int64_t n = a.n;
  const int64_t stride = int64_t(gridDim.x) * TILE;
  for (int64_t t0 = shift_tile(blockIdx.x, gridDim.x) * TILE; t0 < n; t0 += stride) {
    const int64_t i = t0 + int64_t(threadIdx.x) * V;     // t0 is workgroup-uniform
    if (i >= n) continue;
    if (i >= V && i + 2 * V <= n) {
      float g[V], p[V], m[V], v[V];
      const int64_t tl = n - t0 < TILE ? n - t0 : TILE;
      const At at{t0, tl, uint32_t(threadIdx.x) * V};
      // the state loads first: loading them after the rows measured 6% slower here
      if constexpr (OP != Op::Reduce) {
        loadf(a.p, at, p);
        loadf(a.m, at, m);
        loadf(a.v, at, v);
      }
      reduce_rows_shifted<NG>(a, i, g);
      if constexpr (OP == Op::Reduce) {
        out_f32(a.out, t0, tl, i, g);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) adamw(g[e], p[e], m[e], v[e], a.s);
        out_f32(a.p, t0, tl, i, p);
        out_f32(a.m, t0, tl, i, m);
        out_f32(a.v, t0, tl, i, v);
        if constexpr (EMIT) out_bf16(a.w, t0, tl, i, p);
      }
    } else {
      const int64_t end = i + V < n ? i + V : n;
      for (int64_t j = i; j < end; ++j) step_scalar<OP>(a, j);
    }
  }
}

// Scalar path for unaligned buffers: element tile + j*kStepThreads + t, so
// each instruction of a wavefront still touches 64 consecutive elements.
template <Op OP>
__global__ __launch_bounds__(kStepThreads) void k_step_scalar(StepArgs a) {
  const int64_t n = a.n;
  const int64_t stride = int64_t(gridDim.x) * kStepTile;
  for (int64_t base = int64_t(blockIdx.x) * kStepTile; base < n; base += stride) {
#pragma unroll
    for (int j = 0; j < kSV; ++j) {
      const int64_t i = base + int64_t(j) * kStepThreads + threadIdx.x;
      if (i < n) step_scalar<OP>(a, i);
    }
  }
}

// ---------------------------------------------------------------------------
// batched fused step over many units (one launch per up to kMaxMultiUnits)
// ---------------------------------------------------------------------------

constexpr int kMultiRows = 8;        // row pointers per unit descriptor
constexpr int kMaxMultiUnits = 30;   // descriptors per launch (kernel arguments < 4 KB)
// Units at least this long get a launch of their own: there the per-launch
// cost is negligible and the single-unit kernel, whose pointers sit at fixed
// kernel-argument offsets, starts its workgroups sooner.
// Units with fewer shard elements than this go through the batched kernel.
constexpr int64_t kBatchMaxElems = int64_t(1) << 22;

struct UnitDesc {
  const uint16_t* g[kMultiRows];     // rank-window start of each contribution
  float* p;
  float* m;
  float* v;
  uint16_t* w;                       // bf16 parameter out, or null
  int64_t n;                         // shard_valid
  int64_t tile_end;                  // exclusive prefix of tiles over the batch
};

struct MultiArgs {
  UnitDesc u[kMaxMultiUnits];
  int64_t tiles;
  int32_t nu;
  int32_t n_grads;
  Adam s;
};

// Index of the first entry whose exclusive tile prefix exceeds t: a
// workgroup-uniform binary search over kernel arguments (a handful of
// dependent scalar loads instead of a linear walk).
template <typename E>
__device__ __forceinline__ int find_entry(const E* e, int count, int64_t t) {
  int lo = 0, hi = count - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (t < e[mid].tile_end) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

// Tiles of all units of the batch laid end to end; a workgroup finds its unit
// by binary search over the descriptors (scalar registers) and runs the same
// vector body as k_step_vec<Fused> on it.
template <int NG>
__global__ __launch_bounds__(kStepThreads) void k_step_multi(MultiArgs a) {
  for (int64_t t = blockIdx.x; t < a.tiles; t += gridDim.x) {
    const int s = find_entry(a.u, a.nu, t);
    const int64_t tile0 = s == 0 ? 0 : a.u[s - 1].tile_end;
    const UnitDesc& d = a.u[s];
    const int64_t t0 = (t - tile0) * kStepTile;              // this tile's first element
    const int64_t i = t0 + int64_t(threadIdx.x) * kSV;
    if (i + kSV <= d.n) {
      const int64_t tl = d.n - t0 < kStepTile ? d.n - t0 : int64_t(kStepTile);
      const At at{t0, tl, uint32_t(threadIdx.x) * kSV};
      float g[kSV], p[kSV], m[kSV], v[kSV];
      loadf(d.p, at, p);            // state first: every load in flight before the first add
      loadf(d.m, at, m);
      loadf(d.v, at, v);
      reduce_rows<NG, kSV>(d.g, a.n_grads, a.s.gs, at, g);
#pragma unroll
      for (int e = 0; e < kSV; ++e) adamw(g[e], p[e], m[e], v[e], a.s);
      out_f32(d.p, t0, tl, i, p);
      out_f32(d.m, t0, tl, i, m);
      out_f32(d.v, t0, tl, i, v);
      if (d.w) out_bf16(d.w, t0, tl, i, p);
    } else {
      for (int64_t j = i; j < d.n; ++j) fused_scalar(d.g, a.n_grads, d.p, d.m, d.v, d.w, j, a.s);
    }
  }
}

// ---------------------------------------------------------------------------
// segment copy: flatten/pad and gather/unflatten
// ---------------------------------------------------------------------------

enum : int32_t { kSegVec = 0, kSegScalar = 1, kSegZeroVec = 2, kSegZeroScalar = 3 };

struct Seg {
  const void* src;     // null for zero fill
  void* dst;
  int64_t len;         // elements
  int64_t tile_end;    // exclusive prefix of tiles over the batch
  int32_t mode;
  int32_t pad_;
};

constexpr int kMaxSeg = 64;

struct SegArgs {
  Seg seg[kMaxSeg];
  int64_t tiles;
  int32_t nseg;
  int32_t pad_;
};

// KIND 0: 4-byte bit copy; 1: 2-byte bit copy; 2: fp32 -> bf16 (nearest even);
// 3: bf16 -> fp32 (exact). A lane moves EPL consecutive elements: one 16-byte
// source vector (8 bytes for KIND 3, whose 16-byte store is the wider side),
// so every load and store instruction of a wavefront is one contiguous range
// and no cache line is written in pieces by different instructions.
template <int KIND>
struct CopyKind;
template <>
struct CopyKind<0> {
  using S = uint32_t;
  using D = uint32_t;
  static constexpr int EPL = 4;
  static __device__ __forceinline__ D cvt(S x) { return x; }
  using V = u32x4;
  static __device__ __forceinline__ V bits(const S* s) { return ldh<u32x4, kCopyNtLoad>(s); }
};
template <>
struct CopyKind<1> {
  using S = uint16_t;
  using D = uint16_t;
  static constexpr int EPL = 8;
  static __device__ __forceinline__ D cvt(S x) { return x; }
  using V = u32x4;
  static __device__ __forceinline__ V bits(const S* s) { return ldh<u32x4, kCopyNtLoad>(s); }
};
template <>
struct CopyKind<2> {
  using S = float;
  using D = uint16_t;
  static constexpr int EPL = 4;
  static __device__ __forceinline__ D cvt(S x) { return static_cast<uint16_t>(to_bf16(x)); }
  using V = u32x2;
  static __device__ __forceinline__ V bits(const S* s) {
    const f32x4 x = ldh<f32x4, kCopyNtLoad>(s);
    return V{pack_bf16(x.x, x.y), pack_bf16(x.z, x.w)};
  }
};

template <>
struct CopyKind<3> {
  using S = uint16_t;
  using D = float;
  static constexpr int EPL = 4;
  static __device__ __forceinline__ D cvt(S x) { return widen(x); }
  using V = u32x4;
  static __device__ __forceinline__ V bits(const S* s) {
    const u32x2 q = ldh<u32x2, kCopyNtLoad>(s);
    return V{__float_as_uint(lo_bf16(q.x)), __float_as_uint(hi_bf16(q.x)),
             __float_as_uint(lo_bf16(q.y)), __float_as_uint(hi_bf16(q.y))};
  }
};

// Elements per lane, and per workgroup tile, of each copy kind (host and device).
constexpr int copy_epl(int kind) { return kind == 1 ? 8 : 4; }
constexpr int64_t copy_tile(int kind) { return int64_t(kThreads) * copy_epl(kind); }

template <int KIND>
__global__ __launch_bounds__(kThreads) void k_segcopy(SegArgs a) {
  using K = CopyKind<KIND>;
  using S = typename K::S;
  using D = typename K::D;
  constexpr int EPL = K::EPL;
  constexpr int64_t TILE = int64_t(kThreads) * EPL;
  for (int64_t t = blockIdx.x; t < a.tiles; t += gridDim.x) {
    const int s = find_entry(a.seg, a.nseg, t);
    const int64_t tile0 = s == 0 ? 0 : a.seg[s - 1].tile_end;
    const int64_t base = (t - tile0) * TILE;
    const int64_t len = a.seg[s].len;
    const int32_t mode = a.seg[s].mode;
    const S* src = static_cast<const S*>(a.seg[s].src);
    D* dst = static_cast<D*>(a.seg[s].dst);
    if (mode == kSegVec || mode == kSegZeroVec) {
      const int64_t i = base + int64_t(threadIdx.x) * EPL;
      if (i + EPL <= len) {
        const typename K::V x = mode == kSegVec ? K::bits(src + i) : typename K::V{};
        if constexpr (kCopyCpol >= 0) {
          const int64_t tl = len - base < TILE ? len - base : TILE;
          bst<kCopyCpol>(rsrc(dst + base, tl * int64_t(sizeof(D))),
                         int(threadIdx.x) * EPL * int(sizeof(D)), x);
        } else {
          st<typename K::V, false>(dst + i, x);
        }
      } else {
        for (int64_t j = i; j < len; ++j) dst[j] = mode == kSegVec ? K::cvt(src[j]) : D(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const int64_t e = base + int64_t(j) * kThreads + threadIdx.x;
        if (e < len) dst[e] = mode == kSegScalar ? K::cvt(src[e]) : D(0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host-side launch helpers
// ---------------------------------------------------------------------------

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// a lane's 4 bf16 elements form one 8-byte access
bool aligned_bf16_vec(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

unsigned grid_for(int64_t tiles) { return static_cast<unsigned>(std::max<int64_t>(tiles, 1)); }

fsdp_status after_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(FSDP_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return FSDP_OK;
}

// LDS per CU of the current device (queried once; 0 if the query fails, which
// leaves every launch uncapped).
int lds_per_cu() {
  static std::atomic<int> cached{-1};
  int v = cached.load(std::memory_order_relaxed);
  if (v >= 0) return v;
  int dev = 0, bytes = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&bytes, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess) {
    bytes = 0;
    (void)hipGetLastError();   // the caller checked that no earlier error was pending
  }
  cached.store(bytes, std::memory_order_relaxed);
  return bytes;
}

// Unused dynamic LDS that caps resident workgroups at wg_per_cu per CU: the
// largest 4 KiB multiple (else 512 B multiple) of which wg_per_cu fit in a CU
// and wg_per_cu + 1 do not, so allocation granules cannot round it past that
// count. 0 (no cap) when no such size exists.
size_t lds_reservation(int wg_per_cu) {
  const int64_t per_cu = lds_per_cu();
  if (wg_per_cu <= 0 || per_cu <= 0) return 0;
  for (int64_t granule : {int64_t(4096), int64_t(512)}) {
    const int64_t r = per_cu / wg_per_cu / granule * granule;
    if (r > 0 && (wg_per_cu + 1) * r > per_cu) return size_t(r);
  }
  return 0;
}

// Occupancy plan of a vector-path (and shifted-path) step launch: workgroup
// size and resident workgroups per CU (0: as many as fit). Chosen by
// measurement on MI355X (rotating buffer sets, each variant on the same
// buffers, several boxes and allocations):
//  * launches under 2^FSDP_CAP_MIN_LOG2 elements run 256-thread workgroups, all
//    resident at once: they have fewer tiles than a few rounds of the machine;
//  * the stand-alone AdamW and the reduce and fused kernels with a
//    compile-time fold (flat, or grouped for hybrid sharding and bf16 partial
//    sums) run one-wave workgroups (64 threads, 256-element tiles), with the
//    per-CU count set so that a CU keeps about
//    FSDP_LANE_BUDGET * 64 bytes of loads and stores in flight: count =
//    round(FSDP_LANE_BUDGET / bytes a lane moves per tile), within [8, 32]. A
//    lane moves 8 bytes per gradient row and 16 bytes per fp32 array, read or
//    written (and 8 for the bf16 output): the fused step with 8 rows and the
//    emission moves 168 bytes (8 per CU), the stand-alone AdamW 120 (11), the
//    reduce of 8 rows 80 (16), of 2 rows 32 (32). Little's law gives the same
//    size: a CU's 1/256 share of 8 TB/s over a loaded latency of a few
//    microseconds. The one-wave tiles keep each CU's write streams short and
//    the end of a launch short;
//  * the fused step with a compile-time fold of 8 or more rows stages its
//    tile loads (step_tile) and runs FSDP_STAGED_WG_PER_CU (10) one-wave
//    workgroups per CU, without XCD runs in k_step_one (9-11 measured alike
//    for 8 and 16 rows; 8 and 12 were slower); with fewer rows a stage holds
//    too few bytes and the unstaged tile keeps the lane-budget count;
//  * the fused step with a run-time row count, folded flat, runs one-wave
//    workgroups, FSDP_CHUNKED_WG_PER_CU per CU: a lane has one chunk of 8 rows
//    in flight at a time, so it needs more waves than its bytes suggest (11
//    and 13 rows: best at 12 out of 6 to 24; 2-7% faster than 256-thread
//    workgroups at rank 0, -1 to +3% at the last rank; with the state loads
//    last, 12 stayed best out of 10, 12 and 16), in k_step_one without XCD
//    runs;
//  * the reduce with a run-time row count, and the grouped folds of a
//    run-time count, are not capped (256 threads): one-wave workgroups made
//    that reduce 3-20% slower.
struct Shape {
  int threads;
  int wg_per_cu;
};

// Hybrid sharding with 3 or 4 replica groups of 8 ranks: compile-time grouped
// folds of the fused step only (its staged loads, 3 or 4 stages of one group
// each: 4-6% faster than the run-time grouped fold on the 7B block); the reduce
// folds them at run time.
bool fused_wide_hybrid(const StepArgs& a) {
  return !a.bf16acc && a.group == 8 && (a.n_grads == 24 || a.n_grads == 32);
}

bool compile_time_fold(const StepArgs& a, Op op) {
  if (a.group < a.n_grads || a.bf16acc)
    return (!a.bf16acc && a.n_grads == 16 && a.group == 8) ||
           (!a.bf16acc && a.n_grads == 8 && a.group == 4) ||
           (a.bf16acc && a.n_grads == 16 && a.group == 16) ||
           (a.bf16acc && a.n_grads == 8 && a.group == 8) ||
           (op == Op::Fused && fused_wide_hybrid(a));
  return (a.n_grads >= 1 && a.n_grads <= 8) || a.n_grads == 16;
}

// Bytes one lane (4 consecutive elements) reads and writes per tile.
template <Op OP>
int lane_bytes(const StepArgs& a) {
  const int w = a.w ? 8 : 0;
  if (OP == Op::Reduce) return 8 * a.n_grads + 16;
  if (OP == Op::AdamW) return 16 + 48 + 48 + w;
  return 8 * a.n_grads + 96 + w;
}

template <Op OP>
Shape step_shape(const StepArgs& a) {
  if (a.n < (int64_t(1) << FSDP_CAP_MIN_LOG2)) return Shape{kStepThreads, 0};
  if (OP == Op::Fused && compile_time_fold(a, OP) && a.n_grads >= 8)
    return Shape{kSmallThreads, FSDP_STAGED_WG_PER_CU};   // staged tile loads (step_tile)
  if (OP == Op::AdamW || compile_time_fold(a, OP)) {
    const int b = lane_bytes<OP>(a);
    const int wg = std::min(32, std::max(8, (FSDP_LANE_BUDGET + b / 2) / b));
    return Shape{kSmallThreads, wg};
  }
  if (OP == Op::Fused && a.group == a.n_grads && !a.bf16acc)
    return Shape{kSmallThreads, FSDP_CHUNKED_WG_PER_CU};   // a run-time count, folded flat
  return Shape{kStepThreads, 0};   // a run-time row count: the reduce, the grouped folds
}

template <Op OP, bool EMIT>
void launch_vec_ng(const StepArgs& a, unsigned grid, int threads, size_t lds, hipStream_t stream) {
  if constexpr (OP == Op::AdamW) {
    k_step_vec<OP, 0, EMIT><<<grid, threads, lds, stream>>>(a);
  } else if (a.group < a.n_grads || a.bf16acc) {
    // grouped folds: the common shapes with compile-time counts, the rest general
    if (!a.bf16acc && a.n_grads == 16 && a.group == 8)
      k_step_vec<OP, 16, EMIT, 8, false><<<grid, threads, lds, stream>>>(a);
    else if (!a.bf16acc && a.n_grads == 8 && a.group == 4)
      k_step_vec<OP, 8, EMIT, 4, false><<<grid, threads, lds, stream>>>(a);
    else if (a.bf16acc && a.n_grads == 16 && a.group == 16)
      k_step_vec<OP, 16, EMIT, 16, true><<<grid, threads, lds, stream>>>(a);
    else if (a.bf16acc && a.n_grads == 8 && a.group == 8)
      k_step_vec<OP, 8, EMIT, 8, true><<<grid, threads, lds, stream>>>(a);
    else if (OP == Op::Fused && fused_wide_hybrid(a) && a.n_grads == 24)
      k_step_vec<Op::Fused, 24, EMIT, 8, false><<<grid, threads, lds, stream>>>(a);
    else if (OP == Op::Fused && fused_wide_hybrid(a))
      k_step_vec<Op::Fused, 32, EMIT, 8, false><<<grid, threads, lds, stream>>>(a);
    else
      k_step_vec<OP, 0, EMIT><<<grid, threads, lds, stream>>>(a);
  } else {
  switch (a.n_grads) {
#define FSDP_NG_CASE(K) \
  case K: k_step_vec<OP, K, EMIT><<<grid, threads, lds, stream>>>(a); break;
    FSDP_NG_CASE(1)
    FSDP_NG_CASE(2)
    FSDP_NG_CASE(3)
    FSDP_NG_CASE(4)
    FSDP_NG_CASE(5)
    FSDP_NG_CASE(6)
    FSDP_NG_CASE(7)
    FSDP_NG_CASE(8)
    FSDP_NG_CASE(16)
#undef FSDP_NG_CASE
    default: k_step_vec<OP, 0, EMIT><<<grid, threads, lds, stream>>>(a); break;
  }
  }
}
// The staged fused step in its one-tile kernel (one-wave workgroups, tiles in
// plain order, grid = the tile count); false when the fold has no one-tile
// instantiation (1-7 rows, the grouped folds of run-time counts).
template <bool EMIT>
bool launch_one(const StepArgs& a, unsigned grid, size_t lds, hipStream_t stream) {
  if (a.group < a.n_grads || a.bf16acc) {
    if (!a.bf16acc && a.n_grads == 16 && a.group == 8)
      k_step_one<16, EMIT, 8, false><<<grid, kSmallThreads, lds, stream>>>(a);
    else if (!a.bf16acc && a.n_grads == 8 && a.group == 4)
      k_step_one<8, EMIT, 4, false><<<grid, kSmallThreads, lds, stream>>>(a);
    else if (a.bf16acc && a.n_grads == 16 && a.group == 16)
      k_step_one<16, EMIT, 16, true><<<grid, kSmallThreads, lds, stream>>>(a);
    else if (a.bf16acc && a.n_grads == 8 && a.group == 8)
      k_step_one<8, EMIT, 8, true><<<grid, kSmallThreads, lds, stream>>>(a);
    else if (fused_wide_hybrid(a) && a.n_grads == 24)
      k_step_one<24, EMIT, 8, false><<<grid, kSmallThreads, lds, stream>>>(a);
    else if (fused_wide_hybrid(a))
      k_step_one<32, EMIT, 8, false><<<grid, kSmallThreads, lds, stream>>>(a);
    else
      return false;
  } else if (a.n_grads == 8) {
    k_step_one<8, EMIT><<<grid, kSmallThreads, lds, stream>>>(a);
  } else if (a.n_grads == 16) {
    k_step_one<16, EMIT><<<grid, kSmallThreads, lds, stream>>>(a);
  } else if (!compile_time_fold(a, Op::Fused)) {
    k_step_one<0, EMIT><<<grid, kSmallThreads, lds, stream>>>(a);   // run-time count, flat
  } else {
    return false;
  }
  return true;
}

template <Op OP, bool EMIT>
void launch_shift_ng(const StepArgs& a, unsigned grid, int threads, size_t lds,
                     hipStream_t stream) {
  switch (a.n_grads) {
#define FSDP_NG_CASE(K) \
  case K: k_step_shift<OP, K, EMIT><<<grid, threads, lds, stream>>>(a); break;
    FSDP_NG_CASE(1)
    FSDP_NG_CASE(2)
    FSDP_NG_CASE(3)
    FSDP_NG_CASE(4)
    FSDP_NG_CASE(5)
    FSDP_NG_CASE(6)
    FSDP_NG_CASE(7)
    FSDP_NG_CASE(8)
    FSDP_NG_CASE(16)
#undef FSDP_NG_CASE
    default: k_step_shift<OP, 0, EMIT><<<grid, threads, lds, stream>>>(a); break;
  }
}

enum class Path { Vector, Shifted, Scalar };

// Whether a vector-path launch visits its tiles in XCD runs: some window it
// reads or writes does not start on a 128-byte line.
bool off_line(const void* p) { return p && (reinterpret_cast<uintptr_t>(p) & 127u); }
bool needs_runs(const StepArgs& a, Op op) {
  bool r = false;
  if (op != Op::AdamW)
    for (int k = 0; k < a.n_grads; ++k) r = r || off_line(a.g[k]);
  if (op == Op::AdamW) r = r || off_line(a.grad);
  if (op == Op::Reduce) return r || off_line(a.out);
  return r || off_line(a.p) || off_line(a.m) || off_line(a.v) || off_line(a.w);
}

template <Op OP>
fsdp_status launch_step(const StepArgs& args, Path path, hipStream_t stream, const char* what) {
  if (args.n <= 0) return FSDP_OK;
  StepArgs a = args;
  a.runs = needs_runs(a, OP) ? 1 : 0;
  if (path == Path::Vector) {
    const Shape sh = step_shape<OP>(a);
    const int64_t tile = int64_t(sh.threads) * kSV;
    const unsigned grid = grid_for((a.n + tile - 1) / tile);
    const size_t lds = lds_reservation(sh.wg_per_cu);
    bool done = false;
    if constexpr (OP == Op::Fused) {
      // grid * tile covers n (the grid's x size holds the tile count): one tile each
      if (sh.threads == kSmallThreads && !a.runs && (a.n + tile - 1) / tile <= INT32_MAX)
        done = a.w ? launch_one<true>(a, grid, lds, stream) : launch_one<false>(a, grid, lds, stream);
    }
    if (!done) {
      if (a.w) launch_vec_ng<OP, true>(a, grid, sh.threads, lds, stream);
      else launch_vec_ng<OP, false>(a, grid, sh.threads, lds, stream);
    }
  } else if (path == Path::Shifted) {
    if constexpr (OP != Op::AdamW) {
      // the same occupancy plan as the vector path (the shifted path only folds flat)
      const Shape sh = step_shape<OP>(a);
      const int64_t tile = int64_t(sh.threads) * 4;
      const unsigned grid = grid_for((a.n + tile - 1) / tile);
      const size_t lds = lds_reservation(sh.wg_per_cu);
      if (a.w) launch_shift_ng<OP, true>(a, grid, sh.threads, lds, stream);
      else launch_shift_ng<OP, false>(a, grid, sh.threads, lds, stream);
    }
  } else {
    const unsigned grid = grid_for((a.n + kStepTile - 1) / kStepTile);
    k_step_scalar<OP><<<grid, kStepThreads, 0, stream>>>(a);
  }
  return after_launch(what);
}

struct Piece {
  const void* src;   // null: zero fill
  void* dst;
  int64_t len;
};

// Per-thread scratch vectors of the host side, reused from call to call so
// that a call's validation and planning allocate nothing once a thread has
// made a few calls.
template <typename T, int TAG>
std::vector<T>& scratch() {
  thread_local std::vector<T> v;
  v.clear();
  return v;
}

// A HIP error left pending by earlier work on this thread would come back as
// this call's launch failure: refuse to enqueue anything instead, and leave
// the error where it is for its owner (nothing is cleared).
fsdp_status check_no_pending_error(const char* what) {
  const hipError_t e = hipPeekAtLastError();
  if (e != hipSuccess)
    return fail(FSDP_ERR_HIP, "%s: a HIP error from earlier work is pending (%s); nothing was "
                "enqueued", what, hipGetErrorString(e));
  return FSDP_OK;
}

// Plans the segment-copy launches of `pieces`: each piece splits into an
// unaligned scalar head and an aligned vector body (each side on one lane's
// access width) when some head length h < EPL aligns both sides, otherwise
// the whole piece is scalar; the segments then go in batches of kMaxSeg.
void plan_pieces(const std::vector<Piece>& pieces, int kind, std::vector<SegArgs>* batches) {
  const int64_t ss = (kind == 1 || kind == 3) ? 2 : 4;   // source element bytes
  const int64_t ds = (kind == 0 || kind == 3) ? 4 : 2;   // destination element bytes
  const int64_t epl = copy_epl(kind);
  const uintptr_t smask = uintptr_t(epl * ss - 1);
  const uintptr_t dmask = uintptr_t(epl * ds - 1);
  std::vector<Seg>& segs = scratch<Seg, 0>();
  for (const Piece& pc : pieces) {
    if (pc.len <= 0) continue;
    const uintptr_t s0 = reinterpret_cast<uintptr_t>(pc.src);
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(pc.dst);
    int64_t head = -1;
    for (int64_t h = 0; h < epl && h < pc.len; ++h) {
      const bool s_ok = pc.src == nullptr || ((s0 + h * ss) & smask) == 0;
      const bool d_ok = ((d0 + h * ds) & dmask) == 0;
      if (s_ok && d_ok) { head = h; break; }
    }
    const int32_t vmode = pc.src ? kSegVec : kSegZeroVec;
    const int32_t smode = pc.src ? kSegScalar : kSegZeroScalar;
    if (head < 0) {
      segs.push_back(Seg{pc.src, pc.dst, pc.len, 0, smode, 0});
      continue;
    }
    if (head > 0) segs.push_back(Seg{pc.src, pc.dst, head, 0, smode, 0});
    const void* vs = pc.src ? reinterpret_cast<const void*>(s0 + head * ss) : nullptr;
    void* vd = reinterpret_cast<void*>(d0 + head * ds);
    segs.push_back(Seg{vs, vd, pc.len - head, 0, vmode, 0});
  }
  for (size_t b = 0; b < segs.size(); b += kMaxSeg) {
    batches->emplace_back();
    SegArgs& a = batches->back();
    a = SegArgs{};
    const size_t nb = std::min<size_t>(kMaxSeg, segs.size() - b);
    int64_t tiles = 0;
    for (size_t j = 0; j < nb; ++j) {
      a.seg[j] = segs[b + j];
      tiles += (a.seg[j].len + copy_tile(kind) - 1) / copy_tile(kind);
      a.seg[j].tile_end = tiles;
    }
    a.nseg = static_cast<int32_t>(nb);
    a.tiles = tiles;
  }
}

// Launches planned segment-copy batches in order. If the runtime refuses
// launch k, launches 0..k-1 stay enqueued (documented in the header).
fsdp_status launch_batches(const std::vector<SegArgs>& batches, int kind, hipStream_t stream,
                           const char* what) {
  for (const SegArgs& a : batches) {
    const unsigned grid = grid_for(a.tiles);
    switch (kind) {
      case 0: k_segcopy<0><<<grid, kThreads, 0, stream>>>(a); break;
      case 1: k_segcopy<1><<<grid, kThreads, 0, stream>>>(a); break;
      case 2: k_segcopy<2><<<grid, kThreads, 0, stream>>>(a); break;
      default: k_segcopy<3><<<grid, kThreads, 0, stream>>>(a); break;
    }
    if (fsdp_status st = after_launch(what)) return st;
  }
  return FSDP_OK;
}

void launch_multi(const MultiArgs& a, hipStream_t stream) {
  const unsigned grid = grid_for(a.tiles);
  const size_t lds =
      a.tiles * kStepTile >= (int64_t(1) << FSDP_CAP_MIN_LOG2) ? lds_reservation(FSDP_MULTI_WG_PER_CU) : 0;
  switch (a.n_grads) {
#define FSDP_NG_CASE(K) \
  case K: k_step_multi<K><<<grid, kStepThreads, lds, stream>>>(a); break;
    FSDP_NG_CASE(1)
    FSDP_NG_CASE(2)
    FSDP_NG_CASE(3)
    FSDP_NG_CASE(4)
    FSDP_NG_CASE(5)
    FSDP_NG_CASE(6)
    FSDP_NG_CASE(7)
    FSDP_NG_CASE(8)
#undef FSDP_NG_CASE
    default: break;   // callers batch only n_grads <= kMultiRows
  }
}

Adam to_device(const fsdp::AdamScalars& h) {
  return Adam{h.gs, h.b1, h.omb1, h.b2, h.omb2, h.bc1, h.bc2, h.lr, h.eps, h.wd};
}

fsdp_status check_n_grads(int32_t n_grads) {
  if (n_grads < 1 || n_grads > FSDP_MAX_RANKS)
    return fail(FSDP_ERR_INVALID_ARG, "n_grads must be in [1, %d] (got %d)", FSDP_MAX_RANKS,
                n_grads);
  return FSDP_OK;
}

// The gradient rows of a step call (only when the rank's window holds data).
fsdp_status check_grads(const fsdp_unit* u, int32_t n_grads, const void* const* grads,
                        std::vector<fsdp::ByteRange>* ranges, StepArgs* a, int32_t unit = -1) {
  if (!grads) return fail(FSDP_ERR_INVALID_ARG, "grads array is NULL");
  for (int32_t k = 0; k < n_grads; ++k) {
    if (!grads[k]) return fail(FSDP_ERR_INVALID_ARG, "grads[%d] is NULL", k);
    if (reinterpret_cast<uintptr_t>(grads[k]) & 1u)
      return fail(FSDP_ERR_INVALID_ARG, "grads[%d] is not 2-byte aligned", k);
    const uint16_t* w = static_cast<const uint16_t*>(grads[k]) + u->begin;
    a->g[k] = w;
    ranges->push_back(fsdp::range_of(w, u->valid, 2, false, "grads", k, unit));
  }
  a->n_grads = n_grads;
  a->group = n_grads;
  return FSDP_OK;
}

fsdp_status check_f32(const void* p, const char* name) {
  if (!p) return fail(FSDP_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & 3u)
    return fail(FSDP_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
  return FSDP_OK;
}

// Vector when every buffer is aligned for its vector access; Shifted when only
// gradient rows fall short (the 4-element shifted loads need 2-byte rows);
// Scalar otherwise.
Path step_path(const StepArgs& a, Op op) {
  bool state_ok = true;
  if (op == Op::AdamW) state_ok = state_ok && aligned16(a.grad);
  if (op == Op::Reduce) state_ok = state_ok && aligned16(a.out);
  if (op != Op::Reduce) {
    state_ok = state_ok && aligned16(a.p) && aligned16(a.m) && aligned16(a.v);
    if (a.w) state_ok = state_ok && aligned_bf16_vec(a.w);
  }
  if (!state_ok) return Path::Scalar;
  if (op == Op::AdamW) return Path::Vector;
  bool rows_ok = true;
  for (int k = 0; k < a.n_grads; ++k) rows_ok = rows_ok && aligned_bf16_vec(a.g[k]);
  if (rows_ok) return Path::Vector;
  // the shifted path folds the rows flat in fp32; other folds take the scalar path
  if (a.group < a.n_grads || a.bf16acc) return Path::Scalar;
  return Path::Shifted;
}

fsdp_status check_state(const fsdp_unit* u, float* master, float* exp_avg, float* exp_avg_sq,
                        void* w, std::vector<fsdp::ByteRange>* ranges, StepArgs* a,
                        int32_t unit = -1) {
  if (fsdp_status st = check_f32(master, "master")) return st;
  if (fsdp_status st = check_f32(exp_avg, "exp_avg")) return st;
  if (fsdp_status st = check_f32(exp_avg_sq, "exp_avg_sq")) return st;
  if (w && (reinterpret_cast<uintptr_t>(w) & 1u))
    return fail(FSDP_ERR_INVALID_ARG, "param_bf16_out is not 2-byte aligned");
  a->p = master;
  a->m = exp_avg;
  a->v = exp_avg_sq;
  a->w = static_cast<uint16_t*>(w);
  ranges->push_back(fsdp::range_of(master, u->valid, 4, true, "master", -1, unit));
  ranges->push_back(fsdp::range_of(exp_avg, u->valid, 4, true, "exp_avg", -1, unit));
  ranges->push_back(fsdp::range_of(exp_avg_sq, u->valid, 4, true, "exp_avg_sq", -1, unit));
  if (w) ranges->push_back(fsdp::range_of(w, u->valid, 2, true, "param_bf16_out", -1, unit));
  return FSDP_OK;
}

// The shared body of the reduce-only entry points (flat, hybrid, bf16 partials).
fsdp_status reduce_entry(const fsdp_unit* u, int32_t n_grads, const void* const* grads,
                         double grad_scale, float* out, int32_t group, int32_t bf16acc,
                         hipStream_t stream, const char* what) {
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if (fsdp_status st = check_n_grads(n_grads)) return st;
  if (!std::isfinite(grad_scale)) return fail(FSDP_ERR_INVALID_ARG, "grad_scale must be finite");
  if (u->valid == 0) return FSDP_OK;            // a window of pad only: nothing to do
  StepArgs a{};
  std::vector<fsdp::ByteRange>& ranges = scratch<fsdp::ByteRange, 0>();
  if (fsdp_status st = check_grads(u, n_grads, grads, &ranges, &a)) return st;
  if (fsdp_status st = check_f32(out, "out")) return st;
  ranges.push_back(fsdp::range_of(out, u->valid, 4, true, "out"));
  if (fsdp_status st = fsdp::check_alias(ranges)) return st;
  a.group = group > 0 ? group : n_grads;
  a.bf16acc = bf16acc;
  a.out = out;
  a.n = u->valid;
  a.s.gs = static_cast<float>(grad_scale);
  if (fsdp_status st = check_no_pending_error(what)) return st;
  return launch_step<Op::Reduce>(a, step_path(a, Op::Reduce), stream, what);
}

// The shared body of the fused single-unit entry points.
fsdp_status fused_entry(const fsdp_unit* u, int32_t n_grads, const void* const* grads,
                        float* master, float* exp_avg, float* exp_avg_sq, void* param_bf16_out,
                        const fsdp_adamw_hparams* hp, int32_t group, int32_t bf16acc,
                        hipStream_t stream, const char* what) {
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if (fsdp_status st = check_n_grads(n_grads)) return st;
  fsdp::AdamScalars hs;
  if (fsdp_status st = fsdp::derive_adam_scalars(hp, true, &hs)) return st;
  if (u->valid == 0) return FSDP_OK;            // a window of pad only: nothing to do
  StepArgs a{};
  std::vector<fsdp::ByteRange>& ranges = scratch<fsdp::ByteRange, 0>();
  if (fsdp_status st = check_grads(u, n_grads, grads, &ranges, &a)) return st;
  if (fsdp_status st = check_state(u, master, exp_avg, exp_avg_sq, param_bf16_out, &ranges, &a))
    return st;
  if (fsdp_status st = fsdp::check_alias(ranges)) return st;
  a.group = group > 0 ? group : n_grads;
  a.bf16acc = bf16acc;
  a.n = u->valid;
  a.s = to_device(hs);
  if (fsdp_status st = check_no_pending_error(what)) return st;
  return launch_step<Op::Fused>(a, step_path(a, Op::Fused), stream, what);
}

fsdp_status check_replicas(const fsdp_unit* u, int32_t replicas) {
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if (replicas < 1 || int64_t(replicas) * u->F > FSDP_MAX_RANKS)
    return fail(FSDP_ERR_INVALID_ARG, "replicas * F must be in [1, %d] (replicas=%d, F=%d)",
                FSDP_MAX_RANKS, replicas, u->F);
  return FSDP_OK;
}

}  // namespace

extern "C" {

fsdp_status fsdp_reduce_shard(const fsdp_unit* u, int32_t n_grads, const void* const* grads,
                              double grad_scale, float* out, hipStream_t stream) {
  fsdp::clear_error();
  return reduce_entry(u, n_grads, grads, grad_scale, out, 0, 0, stream, "fsdp_reduce_shard");
}

fsdp_status fsdp_adamw_shard(const fsdp_unit* u, const float* grad, float* master,
                             float* exp_avg, float* exp_avg_sq, void* param_bf16_out,
                             const fsdp_adamw_hparams* hp, hipStream_t stream) {
  fsdp::clear_error();
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  fsdp::AdamScalars hs;
  if (fsdp_status st = fsdp::derive_adam_scalars(hp, false, &hs)) return st;
  if (u->valid == 0) return FSDP_OK;            // a window of pad only: nothing to do
  StepArgs a{};
  std::vector<fsdp::ByteRange>& ranges = scratch<fsdp::ByteRange, 0>();
  if (fsdp_status st = check_f32(grad, "grad")) return st;
  ranges.push_back(fsdp::range_of(grad, u->valid, 4, false, "grad"));
  if (fsdp_status st = check_state(u, master, exp_avg, exp_avg_sq, param_bf16_out, &ranges, &a))
    return st;
  if (fsdp_status st = fsdp::check_alias(ranges)) return st;
  a.grad = grad;
  a.n = u->valid;
  a.s = to_device(hs);
  if (fsdp_status st = check_no_pending_error("fsdp_adamw_shard")) return st;
  return launch_step<Op::AdamW>(a, step_path(a, Op::AdamW), stream, "fsdp_adamw_shard");
}

fsdp_status fsdp_reduce_adamw_shard(const fsdp_unit* u, int32_t n_grads,
                                    const void* const* grads, float* master, float* exp_avg,
                                    float* exp_avg_sq, void* param_bf16_out,
                                    const fsdp_adamw_hparams* hp, hipStream_t stream) {
  fsdp::clear_error();
  return fused_entry(u, n_grads, grads, master, exp_avg, exp_avg_sq, param_bf16_out, hp, 0, 0,
                     stream, "fsdp_reduce_adamw_shard");
}

fsdp_status fsdp_reduce_shard_bf16acc(const fsdp_unit* u, int32_t n_grads,
                                      const void* const* grads, double grad_scale, float* out,
                                      hipStream_t stream) {
  fsdp::clear_error();
  return reduce_entry(u, n_grads, grads, grad_scale, out, 0, 1, stream,
                      "fsdp_reduce_shard_bf16acc");
}

fsdp_status fsdp_reduce_adamw_shard_bf16acc(const fsdp_unit* u, int32_t n_grads,
                                            const void* const* grads, float* master,
                                            float* exp_avg, float* exp_avg_sq,
                                            void* param_bf16_out, const fsdp_adamw_hparams* hp,
                                            hipStream_t stream) {
  fsdp::clear_error();
  return fused_entry(u, n_grads, grads, master, exp_avg, exp_avg_sq, param_bf16_out, hp, 0, 1,
                     stream, "fsdp_reduce_adamw_shard_bf16acc");
}

fsdp_status fsdp_reduce_shard_hybrid(const fsdp_unit* u, int32_t replicas,
                                     const void* const* grads, double grad_scale, float* out,
                                     hipStream_t stream) {
  fsdp::clear_error();
  if (fsdp_status st = check_replicas(u, replicas)) return st;
  return reduce_entry(u, replicas * u->F, grads, grad_scale, out, u->F, 0, stream,
                      "fsdp_reduce_shard_hybrid");
}

fsdp_status fsdp_reduce_adamw_shard_hybrid(const fsdp_unit* u, int32_t replicas,
                                           const void* const* grads, float* master,
                                           float* exp_avg, float* exp_avg_sq,
                                           void* param_bf16_out, const fsdp_adamw_hparams* hp,
                                           hipStream_t stream) {
  fsdp::clear_error();
  if (fsdp_status st = check_replicas(u, replicas)) return st;
  return fused_entry(u, replicas * u->F, grads, master, exp_avg, exp_avg_sq, param_bf16_out, hp,
                     u->F, 0, stream, "fsdp_reduce_adamw_shard_hybrid");
}

fsdp_status fsdp_reduce_adamw_units(int32_t n_units, const fsdp_unit_step* steps, int32_t n_grads,
                                    const fsdp_adamw_hparams* hp, hipStream_t stream) {
  fsdp::clear_error();
  const char* what = "fsdp_reduce_adamw_units";
  if (n_units < 0) return fail(FSDP_ERR_INVALID_ARG, "n_units must be >= 0 (got %d)", n_units);
  if (n_units == 0) return FSDP_OK;
  if (!steps) return fail(FSDP_ERR_INVALID_ARG, "steps array is NULL");
  if (fsdp_status st = check_n_grads(n_grads)) return st;
  fsdp::AdamScalars hs;
  if (fsdp_status st = fsdp::derive_adam_scalars(hp, true, &hs)) return st;
  std::vector<StepArgs>& args = scratch<StepArgs, 0>();
  std::vector<fsdp::ByteRange>& ranges = scratch<fsdp::ByteRange, 0>();
  for (int32_t i = 0; i < n_units; ++i) {
    const fsdp_unit_step& st_i = steps[i];
    if (!st_i.unit) return fail(FSDP_ERR_INVALID_ARG, "steps[%d].unit is NULL", i);
    if (st_i.unit->valid == 0) continue;        // a window of pad only: nothing to do
    args.emplace_back();
    StepArgs& a = args.back();
    a = StepArgs{};
    if (fsdp_status st = check_grads(st_i.unit, n_grads, st_i.grads, &ranges, &a, i)) {
      const std::string msg = fsdp_last_error();
      return fail(st, "steps[%d]: %s", i, msg.c_str());
    }
    if (fsdp_status st = check_state(st_i.unit, st_i.master, st_i.exp_avg, st_i.exp_avg_sq,
                                     st_i.param_bf16_out, &ranges, &a, i)) {
      const std::string msg = fsdp_last_error();
      return fail(st, "steps[%d]: %s", i, msg.c_str());
    }
    a.n = st_i.unit->valid;
    a.s = to_device(hs);
  }
  if (fsdp_status st = fsdp::check_alias(ranges)) return st;
  // Plan every launch before the first: aligned units of fewer than
  // kBatchMaxElems shard elements go in batches through k_step_multi, the rest
  // one by one through the single-unit kernels, in the order given.
  struct Launch {
    int32_t batch;    // index into `batches`, or -1 for a single-unit launch
    int32_t unit;     // index into `args` for a single-unit launch
  };
  std::vector<MultiArgs>& batches = scratch<MultiArgs, 0>();
  std::vector<Launch>& plan = scratch<Launch, 0>();
  for (int32_t i = 0; i < int32_t(args.size()); ++i) {
    const StepArgs& a = args[size_t(i)];
    if (n_grads > kMultiRows || a.n >= kBatchMaxElems ||
        step_path(a, Op::Fused) != Path::Vector) {
      plan.push_back(Launch{-1, i});
      continue;
    }
    if (plan.empty() || plan.back().batch < 0 || batches.back().nu == kMaxMultiUnits) {
      batches.emplace_back();
      MultiArgs& b = batches.back();
      b = MultiArgs{};
      b.n_grads = n_grads;
      b.s = to_device(hs);
      plan.push_back(Launch{int32_t(batches.size()) - 1, -1});
    }
    MultiArgs& b = batches.back();
    UnitDesc& d = b.u[b.nu];
    for (int k = 0; k < n_grads; ++k) d.g[k] = a.g[k];
    d.p = a.p;
    d.m = a.m;
    d.v = a.v;
    d.w = a.w;
    d.n = a.n;
    b.tiles += (a.n + kStepTile - 1) / kStepTile;
    d.tile_end = b.tiles;
    ++b.nu;
  }
  if (plan.empty()) return FSDP_OK;               // every window holds only pad
  if (fsdp_status st = check_no_pending_error(what)) return st;
  // If the runtime refuses launch k, launches 0..k-1 stay enqueued (documented).
  for (const Launch& l : plan) {
    if (l.batch >= 0) {
      launch_multi(batches[size_t(l.batch)], stream);
      if (fsdp_status st = after_launch(what)) return st;
    } else {
      const StepArgs& a = args[size_t(l.unit)];
      if (fsdp_status st = launch_step<Op::Fused>(a, step_path(a, Op::Fused), stream, what))
        return st;
    }
  }
  return FSDP_OK;
}

fsdp_status fsdp_flatten_pad(const fsdp_unit* u, fsdp_dtype dtype, const void* const* tensors,
                             int64_t begin, int64_t len, void* dst, hipStream_t stream) {
  fsdp::clear_error();
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if (dtype != FSDP_F32 && dtype != FSDP_BF16)
    return fail(FSDP_ERR_UNSUPPORTED, "dtype %d not supported", static_cast<int>(dtype));
  const int64_t es = dtype == FSDP_F32 ? 4 : 2;
  if (begin < 0 || len < 0 || begin > u->padded || len > u->padded - begin)
    return fail(FSDP_ERR_RANGE, "window [%lld, %lld) outside [0, %lld)",
                static_cast<long long>(begin), static_cast<long long>(begin + len),
                static_cast<long long>(u->padded));
  if (len == 0) return FSDP_OK;
  if (!tensors) return fail(FSDP_ERR_INVALID_ARG, "tensors array is NULL");
  if (!dst) return fail(FSDP_ERR_INVALID_ARG, "dst is NULL");
  if (reinterpret_cast<uintptr_t>(dst) % es)
    return fail(FSDP_ERR_INVALID_ARG, "dst is not element aligned");
  std::vector<Piece>& pieces = scratch<Piece, 0>();
  std::vector<fsdp::ByteRange>& ranges = scratch<fsdp::ByteRange, 0>();
  ranges.push_back(fsdp::range_of(dst, len, es, true, "dst"));
  const int64_t end = begin + len;
  for (int32_t i = 0; i < u->T; ++i) {
    const int64_t a = std::max(begin, u->offset[i]);
    const int64_t b = std::min(end, u->offset[i + 1]);
    if (a >= b) continue;
    if (!tensors[i]) return fail(FSDP_ERR_INVALID_ARG, "tensors[%d] is NULL", i);
    if (reinterpret_cast<uintptr_t>(tensors[i]) % es)
      return fail(FSDP_ERR_INVALID_ARG, "tensors[%d] is not element aligned", i);
    const char* src = static_cast<const char*>(tensors[i]) + (a - u->offset[i]) * es;
    char* d = static_cast<char*>(dst) + (a - begin) * es;
    pieces.push_back(Piece{src, d, b - a});
    ranges.push_back(fsdp::range_of(src, b - a, es, false, "tensors", i));
  }
  const int64_t pa = std::max(begin, u->U);
  if (pa < end) pieces.push_back(Piece{nullptr, static_cast<char*>(dst) + (pa - begin) * es,
                                       end - pa});
  if (fsdp_status st = fsdp::check_alias(ranges)) return st;
  const int kind = dtype == FSDP_F32 ? 0 : 1;
  std::vector<SegArgs>& batches = scratch<SegArgs, 0>();
  plan_pieces(pieces, kind, &batches);
  if (fsdp_status st = check_no_pending_error("fsdp_flatten_pad")) return st;
  return launch_batches(batches, kind, stream, "fsdp_flatten_pad");
}

fsdp_status fsdp_unflatten(const fsdp_unit* u, fsdp_dtype src_dtype, fsdp_dtype dst_dtype,
                           const void* const* shards, void* const* tensors, hipStream_t stream) {
  fsdp::clear_error();
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if ((src_dtype != FSDP_F32 && src_dtype != FSDP_BF16) ||
      (dst_dtype != FSDP_F32 && dst_dtype != FSDP_BF16))
    return fail(FSDP_ERR_UNSUPPORTED, "dtype pair (%d, %d) not supported",
                static_cast<int>(src_dtype), static_cast<int>(dst_dtype));
  if (!shards) return fail(FSDP_ERR_INVALID_ARG, "shards array is NULL");
  if (!tensors) return fail(FSDP_ERR_INVALID_ARG, "tensors array is NULL");
  const int64_t ss = src_dtype == FSDP_F32 ? 4 : 2;
  const int64_t ds = dst_dtype == FSDP_F32 ? 4 : 2;
  const int kind = src_dtype == dst_dtype ? (ss == 4 ? 0 : 1) : (src_dtype == FSDP_F32 ? 2 : 3);
  std::vector<Piece>& pieces = scratch<Piece, 0>();
  std::vector<fsdp::ByteRange>& ranges = scratch<fsdp::ByteRange, 0>();
  for (int32_t k = 0; k < u->F; ++k) {
    const int64_t kv = std::max<int64_t>(0, std::min<int64_t>(u->S, u->U - k * u->S));
    if (kv == 0) continue;                 // a shard holding only pad is never read
    if (!shards[k]) return fail(FSDP_ERR_INVALID_ARG, "shards[%d] is NULL", k);
    if (reinterpret_cast<uintptr_t>(shards[k]) % ss)
      return fail(FSDP_ERR_INVALID_ARG, "shards[%d] is not element aligned", k);
    ranges.push_back(fsdp::range_of(shards[k], kv, ss, false, "shards", k));
  }
  for (int32_t i = 0; i < u->T; ++i) {
    if (u->numel[i] == 0) continue;
    if (!tensors[i]) return fail(FSDP_ERR_INVALID_ARG, "tensors[%d] is NULL", i);
    if (reinterpret_cast<uintptr_t>(tensors[i]) % ds)
      return fail(FSDP_ERR_INVALID_ARG, "tensors[%d] is not element aligned", i);
    ranges.push_back(fsdp::range_of(tensors[i], u->numel[i], ds, true, "tensors", i));
    const int64_t lo = u->offset[i], hi = u->offset[i + 1];
    for (int64_t k = lo / u->S; k * u->S < hi; ++k) {
      const int64_t a = std::max(lo, k * u->S);
      const int64_t b = std::min(hi, (k + 1) * u->S);
      pieces.push_back(Piece{static_cast<const char*>(shards[k]) + (a - k * u->S) * ss,
                             static_cast<char*>(tensors[i]) + (a - lo) * ds, b - a});
    }
  }
  if (fsdp_status st = fsdp::check_alias(ranges)) return st;
  std::vector<SegArgs>& batches = scratch<SegArgs, 0>();
  plan_pieces(pieces, kind, &batches);
  if (fsdp_status st = check_no_pending_error("fsdp_unflatten")) return st;
  return launch_batches(batches, kind, stream, "fsdp_unflatten");
}

fsdp_status fsdp_cast_unflatten(const fsdp_unit* u, fsdp_dtype src_dtype,
                                const void* const* shards, void* const* tensors_bf16,
                                hipStream_t stream) {
  return fsdp_unflatten(u, src_dtype, FSDP_BF16, shards, tensors_bf16, stream);
}

}  // extern "C"
