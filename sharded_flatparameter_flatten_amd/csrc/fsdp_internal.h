// Internal declarations shared by the host indexer (unit.cpp) and the HIP
// kernels/launchers (kernels.hip) of libfsdpshard.so.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "fsdp_shard.h"

// One FSDP unit as seen by one rank: tensor sizes, flat offsets, shard window.
struct fsdp_unit {
  int32_t F = 0;
  int32_t rank = 0;
  int32_t T = 0;
  std::vector<int32_t> ndim;
  std::vector<int64_t> dims;
  std::vector<int64_t> numel;    // T entries
  std::vector<int64_t> offset;   // T + 1 entries; offset[T] == U
  int64_t U = 0;
  int64_t S = 0;
  int64_t padded = 0;
  int64_t pad = 0;
  int64_t begin = 0;
  int64_t valid = 0;
  int64_t persistent = 0;
  uint64_t fingerprint = 0;
};

namespace fsdp {

// Records a thread-local message and returns `st`.
fsdp_status fail(fsdp_status st, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();

// A byte range [lo, hi) a call reads or writes. Its name for error messages
// is built only when a conflict is reported: `label` (a string literal),
// `index` within a pointer array (or -1), and the unit of a multi-unit call
// (or -1).
struct ByteRange {
  uintptr_t lo;
  uintptr_t hi;
  bool write;
  const char* label;
  int32_t index;
  int32_t unit;
};

ByteRange range_of(const void* p, int64_t elems, int64_t elem_bytes, bool write,
                   const char* label, int32_t index = -1, int32_t unit = -1);

// FSDP_OK when no written range overlaps any other range; reads may overlap
// each other. Sorts `ranges` in place.
fsdp_status check_alias(std::vector<ByteRange>& ranges);

// Host fp32 scalars of one AdamW step, each rounded once from double.
struct AdamScalars {
  float gs, b1, omb1, b2, omb2, bc1, bc2, lr, eps, wd;
};
fsdp_status derive_adam_scalars(const fsdp_adamw_hparams* hp, bool need_grad_scale,
                                AdamScalars* out);

fsdp_status check_unit(const fsdp_unit* u);

}  // namespace fsdp
