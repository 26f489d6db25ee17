// Host side of libfsdpshard.so: the unit indexer, status strings, the
// thread-local error message, alias checks and the AdamW scalar derivation.
//
// Indexer: [FSDP-math, "The sharding unit: FlatParameter and the wrapping
// policy"] (one flat buffer per wrapped unit, split evenly, one contiguous
// slice per rank); [NOTE-003, "Key results"] (the sharding factor F);
// [FSDP-math, "Per-unit memory and communication, in numbers"] (16 bytes of
// persistent state per parameter of the slice).

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <limits>
#include <new>
#include <string>

#include "fsdp_internal.h"

namespace fsdp {

namespace {
thread_local std::string g_last_error;

constexpr int kMaxNdim = 16;
constexpr int64_t kMaxElems = (int64_t(1) << 62) / 4;   // 4*F*S < 2^62

uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= 0x100000001B3ull;
  }
  return h;
}
}  // namespace

fsdp_status fail(fsdp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

ByteRange range_of(const void* p, int64_t elems, int64_t elem_bytes, bool write,
                   const char* label, int32_t index, int32_t unit) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return ByteRange{lo, lo + static_cast<uintptr_t>(elems * elem_bytes), write, label, index, unit};
}

namespace {
std::string range_name(const ByteRange& r) {
  std::string s;
  if (r.unit >= 0) s += "unit " + std::to_string(r.unit) + " ";
  s += r.label;
  if (r.index >= 0) s += "[" + std::to_string(r.index) + "]";
  return s;
}
}  // namespace

fsdp_status check_alias(std::vector<ByteRange>& ranges) {
  ranges.erase(std::remove_if(ranges.begin(), ranges.end(),
                              [](const ByteRange& r) { return r.hi <= r.lo; }),
               ranges.end());
  std::sort(ranges.begin(), ranges.end(),
            [](const ByteRange& a, const ByteRange& b) { return a.lo < b.lo; });
  // Sweep in start order: an interval overlaps an earlier one iff it starts
  // before that one's end, so the running maximum end of earlier writes (and
  // of earlier reads, for a write) decides every conflict.
  uintptr_t max_hi_w = 0, max_hi_r = 0;
  const ByteRange* last_w = nullptr;
  const ByteRange* last_r = nullptr;
  for (const ByteRange& x : ranges) {
    if (last_w && x.lo < max_hi_w)
      return fail(FSDP_ERR_ALIAS, "%s overlaps %s", range_name(x).c_str(),
                  range_name(*last_w).c_str());
    if (x.write && last_r && x.lo < max_hi_r)
      return fail(FSDP_ERR_ALIAS, "%s overlaps %s", range_name(x).c_str(),
                  range_name(*last_r).c_str());
    if (x.write) {
      if (!last_w || x.hi > max_hi_w) { max_hi_w = x.hi; last_w = &x; }
    } else {
      if (!last_r || x.hi > max_hi_r) { max_hi_r = x.hi; last_r = &x; }
    }
  }
  return FSDP_OK;
}

fsdp_status derive_adam_scalars(const fsdp_adamw_hparams* hp, bool need_grad_scale,
                                AdamScalars* out) {
  if (!hp) return fail(FSDP_ERR_INVALID_ARG, "hyper-parameters pointer is NULL");
  if (hp->step < 1) return fail(FSDP_ERR_INVALID_ARG, "step must be >= 1 (got %lld)",
                                static_cast<long long>(hp->step));
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(FSDP_ERR_INVALID_ARG, "betas must lie in [0, 1)");
  if (!std::isfinite(hp->lr) || hp->lr < 0.0)
    return fail(FSDP_ERR_INVALID_ARG, "lr must be finite and >= 0");
  if (!std::isfinite(hp->eps) || !(hp->eps > 0.0))
    return fail(FSDP_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (!std::isfinite(hp->weight_decay))
    return fail(FSDP_ERR_INVALID_ARG, "weight_decay must be finite");
  if (need_grad_scale && !std::isfinite(hp->grad_scale))
    return fail(FSDP_ERR_INVALID_ARG, "grad_scale must be finite");
  const double t = static_cast<double>(hp->step);
  out->gs = static_cast<float>(hp->grad_scale);
  out->b1 = static_cast<float>(hp->beta1);
  out->omb1 = static_cast<float>(1.0 - hp->beta1);
  out->b2 = static_cast<float>(hp->beta2);
  out->omb2 = static_cast<float>(1.0 - hp->beta2);
  out->bc1 = static_cast<float>(1.0 - std::pow(hp->beta1, t));
  out->bc2 = static_cast<float>(1.0 - std::pow(hp->beta2, t));
  out->lr = static_cast<float>(hp->lr);
  out->eps = static_cast<float>(hp->eps);
  out->wd = static_cast<float>(hp->weight_decay);
  if (!(out->bc1 > 0.0f) || !(out->bc2 > 0.0f))
    return fail(FSDP_ERR_INVALID_ARG, "bias correction 1-beta^t rounds to zero in fp32");
  return FSDP_OK;
}

fsdp_status check_unit(const fsdp_unit* u) {
  if (!u) return fail(FSDP_ERR_INVALID_ARG, "unit handle is NULL");
  return FSDP_OK;
}

}  // namespace fsdp

using fsdp::fail;

extern "C" {

int32_t fsdp_abi_version(void) { return FSDP_ABI_VERSION; }

const char* fsdp_status_string(fsdp_status st) {
  switch (st) {
    case FSDP_OK: return "ok";
    case FSDP_ERR_INVALID_ARG: return "invalid argument";
    case FSDP_ERR_RANGE: return "out of range";
    case FSDP_ERR_ALIAS: return "overlapping buffers";
    case FSDP_ERR_UNSUPPORTED: return "unsupported";
    case FSDP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* fsdp_last_error(void) { return fsdp::g_last_error.c_str(); }

fsdp_status fsdp_unit_create(int32_t F, int32_t rank, int32_t n_tensors,
                             const int32_t* ndim, const int64_t* dims, fsdp_unit** out) {
  fsdp::clear_error();
  if (!out) return fail(FSDP_ERR_INVALID_ARG, "out pointer is NULL");
  *out = nullptr;
  if (F < 1 || F > FSDP_MAX_RANKS)
    return fail(FSDP_ERR_INVALID_ARG, "F must be in [1, %d] (got %d)", FSDP_MAX_RANKS, F);
  if (rank < 0 || rank >= F)
    return fail(FSDP_ERR_INVALID_ARG, "rank must be in [0, F) (got %d, F=%d)", rank, F);
  if (n_tensors < 1 || n_tensors > FSDP_MAX_TENSORS)
    return fail(FSDP_ERR_INVALID_ARG, "n_tensors must be in [1, %d] (got %d)",
                FSDP_MAX_TENSORS, n_tensors);
  if (!ndim) return fail(FSDP_ERR_INVALID_ARG, "ndim is NULL");

  fsdp_unit* u = new (std::nothrow) fsdp_unit();
  if (!u) return fail(FSDP_ERR_INVALID_ARG, "out of host memory");
  u->F = F;
  u->rank = rank;
  u->T = n_tensors;
  u->ndim.assign(ndim, ndim + n_tensors);
  u->offset.push_back(0);
  uint64_t h = 0xCBF29CE484222325ull;
  h = fsdp::fnv1a(h, &F, sizeof F);
  h = fsdp::fnv1a(h, &n_tensors, sizeof n_tensors);
  int64_t pos = 0;
  for (int32_t i = 0; i < n_tensors; ++i) {
    const int32_t nd = ndim[i];
    if (nd < 0 || nd > fsdp::kMaxNdim) {
      delete u;
      return fail(FSDP_ERR_INVALID_ARG, "tensor %d: ndim %d outside [0, %d]", i, nd, fsdp::kMaxNdim);
    }
    if (nd > 0 && !dims) {
      delete u;
      return fail(FSDP_ERR_INVALID_ARG, "dims is NULL");
    }
    h = fsdp::fnv1a(h, &nd, sizeof nd);
    int64_t n = 1;
    for (int32_t d = 0; d < nd; ++d) {
      const int64_t dim = dims[pos++];
      u->dims.push_back(dim);
      h = fsdp::fnv1a(h, &dim, sizeof dim);
      if (dim < 0) {
        delete u;
        return fail(FSDP_ERR_INVALID_ARG, "tensor %d: negative dim", i);
      }
      if (dim != 0 && n > fsdp::kMaxElems / dim) {
        delete u;
        return fail(FSDP_ERR_RANGE, "tensor %d: element count overflows", i);
      }
      n *= dim;
    }
    if (u->offset.back() > fsdp::kMaxElems - n) {
      delete u;
      return fail(FSDP_ERR_RANGE, "unit element count overflows");
    }
    u->numel.push_back(n);
    u->offset.push_back(u->offset.back() + n);
  }
  u->U = u->offset.back();
  if (u->U < 1) {
    delete u;
    return fail(FSDP_ERR_RANGE, "unit has no elements");
  }
  u->S = (u->U + F - 1) / F;
  u->padded = u->S * F;
  if (u->padded > fsdp::kMaxElems) {
    delete u;
    return fail(FSDP_ERR_RANGE, "padded unit too large");
  }
  u->pad = u->padded - u->U;
  u->begin = static_cast<int64_t>(rank) * u->S;
  u->valid = std::max<int64_t>(0, std::min<int64_t>(u->S, u->U - u->begin));
  u->persistent = 16 * u->S;
  u->fingerprint = h;
  *out = u;
  return FSDP_OK;
}

fsdp_status fsdp_unit_destroy(fsdp_unit* unit) {
  fsdp::clear_error();
  delete unit;
  return FSDP_OK;
}

fsdp_status fsdp_unit_query(const fsdp_unit* u, fsdp_unit_info* info) {
  fsdp::clear_error();
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if (!info) return fail(FSDP_ERR_INVALID_ARG, "info pointer is NULL");
  info->U = u->U;
  info->S = u->S;
  info->padded = u->padded;
  info->pad = u->pad;
  info->shard_begin = u->begin;
  info->shard_valid = u->valid;
  info->persistent_bytes = u->persistent;
  info->F = u->F;
  info->rank = u->rank;
  info->n_tensors = u->T;
  info->reserved = 0;
  info->fingerprint = u->fingerprint;
  return FSDP_OK;
}

fsdp_status fsdp_unit_tensor(const fsdp_unit* u, int32_t i, int64_t* offset, int64_t* numel) {
  fsdp::clear_error();
  if (fsdp_status st = fsdp::check_unit(u)) return st;
  if (i < 0 || i >= u->T) return fail(FSDP_ERR_RANGE, "tensor index %d outside [0, %d)", i, u->T);
  if (!offset || !numel) return fail(FSDP_ERR_INVALID_ARG, "output pointer is NULL");
  *offset = u->offset[i];
  *numel = u->numel[i];
  return FSDP_OK;
}

}  // extern "C"
