// Host-side argument checks of attnres_fwd.  Pure C++: no HIP call and no
// pointer dereference, so it can be exercised without a GPU.
//
// The accepted domain follows the dispatch gate in the prhub digest of vLLM
// PR #54261 ("Implementation breakdown" item 3 and the attn_res.py snippet):
// hidden size 7168, dense prefix/delta rows, 0 <= num_blocks <= 8,
// num_blocks <= capacity, -1 <= block_write_idx < capacity.  Inputs outside
// it are rejected with an error code (there is no fallback path).  Alignment,
// stride and overlap checks protect the 16-byte vector accesses and the
// in-place writes.
#include "attnres_internal.h"

#include <cmath>
#include <cstdint>

namespace attnres {
namespace {

using i128 = __int128;

struct Span {
  uintptr_t lo = 0, hi = 0;  // [lo, hi) in bytes; empty when lo == hi
  bool used = false;
  bool written = false;
};

Span span(const void *p, i128 bytes, bool written) {
  Span s;
  if (p == nullptr || bytes <= 0) return s;
  s.lo = reinterpret_cast<uintptr_t>(p);
  s.hi = s.lo + static_cast<uintptr_t>(bytes);
  s.used = true;
  s.written = written;
  return s;
}

bool overlap(const Span &a, const Span &b) {
  return a.used && b.used && a.lo < b.hi && b.lo < a.hi;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bank rows (t, i) for t < T, i < cap start at t*ts + i*ss and are H long.
// They do not overlap iff, ordering the axes that have more than one row by
// stride, the inner stride is >= H and the outer stride clears the whole
// inner run.
bool bank_rows_disjoint(int64_t T, int64_t ts, int64_t cap, int64_t ss, int64_t H) {
  struct Axis { int64_t n, s; };
  Axis a{T, ts}, b{cap, ss};
  if (a.n <= 1 && b.n <= 1) return true;
  if (a.n <= 1) return b.s >= H;
  if (b.n <= 1) return a.s >= H;
  if (a.s > b.s) { Axis t = a; a = b; b = t; }
  if (a.s < H) return false;
  return static_cast<i128>(b.s) >= static_cast<i128>(a.n - 1) * a.s + H;
}

}  // namespace

int validate(const FwdArgs &a) {
  if (a.T < 0 || a.H <= 0 || a.max_blocks < 0) return ATTNRES_E_SHAPE;
  if (a.T > kMaxTokens) return ATTNRES_E_SHAPE;
  if (a.H != kHidden) return ATTNRES_E_UNSUPPORTED;
  if (a.num_blocks < 0 || a.num_blocks > kMaxBlocks || a.num_blocks > a.max_blocks)
    return ATTNRES_E_NUM_BLOCKS;
  if (a.block_write_idx < -1 || a.block_write_idx >= a.max_blocks) return ATTNRES_E_WRITE_IDX;
  if (!(a.rms_eps >= 0.0f) || !std::isfinite(a.rms_eps)) return ATTNRES_E_EPS;
  if (a.output_norm_weight && (!(a.output_norm_eps >= 0.0f) || !std::isfinite(a.output_norm_eps)))
    return ATTNRES_E_EPS;
  if (a.T == 0) return ATTNRES_OK;

  const bool bank_used = a.num_blocks > 0 || a.block_write_idx >= 0;
  if (!a.prefix || !a.res_w || !a.rms_w || !a.out) return ATTNRES_E_NULL;
  if (bank_used && !a.blocks) return ATTNRES_E_NULL;

  if (!aligned16(a.prefix) || !aligned16(a.res_w) || !aligned16(a.rms_w) || !aligned16(a.out) ||
      (a.delta && !aligned16(a.delta)) ||
      (a.output_norm_weight && !aligned16(a.output_norm_weight)) ||
      (bank_used && !aligned16(a.blocks)))
    return ATTNRES_E_ALIGN;

  i128 bank_bytes = 0;
  if (bank_used) {
    if (a.block_token_stride < 0 || a.block_slot_stride < 0) return ATTNRES_E_STRIDE;
    if (a.block_token_stride > kMaxStride || a.block_slot_stride > kMaxStride) return ATTNRES_E_SHAPE;
    if ((a.block_token_stride % 8) != 0 || (a.block_slot_stride % 8) != 0) return ATTNRES_E_ALIGN;
    if (!bank_rows_disjoint(a.T, a.block_token_stride, a.max_blocks, a.block_slot_stride, a.H))
      return ATTNRES_E_STRIDE;
    bank_bytes = 2 * (static_cast<i128>(a.T - 1) * a.block_token_stride +
                      static_cast<i128>(a.max_blocks - 1) * a.block_slot_stride + a.H);
  }

  const i128 rows_bytes = 2 * static_cast<i128>(a.T) * a.H;
  const i128 w_bytes = 2 * static_cast<i128>(a.H);
  const bool has_delta = a.delta != nullptr;
  Span s[7] = {
      span(a.prefix, rows_bytes, has_delta),
      span(a.delta, rows_bytes, false),
      span(bank_used ? a.blocks : nullptr, bank_bytes, a.block_write_idx >= 0),
      span(a.res_w, w_bytes, false),
      span(a.rms_w, w_bytes, false),
      span(a.output_norm_weight, w_bytes, false),
      span(a.out, rows_bytes, true),
  };
  // A buffer the call writes must not overlap any other argument.
  for (int i = 0; i < 7; ++i)
    for (int j = 0; j < 7; ++j)
      if (i != j && s[i].written && overlap(s[i], s[j])) return ATTNRES_E_ALIAS;
  return ATTNRES_OK;
}

const char *strerror_text(int status) {
  switch (status) {
    case ATTNRES_OK: return "ok";
    case ATTNRES_E_NULL: return "a required pointer is NULL";
    case ATTNRES_E_SHAPE: return "invalid or too large T, H, max_blocks or stride";
    case ATTNRES_E_UNSUPPORTED: return "unsupported size (H must be 7168; forced split path needs T <= 256)";
    case ATTNRES_E_NUM_BLOCKS: return "num_blocks must be in 0..min(8, max_blocks)";
    case ATTNRES_E_WRITE_IDX: return "block_write_idx must be -1 or in 0..max_blocks-1";
    case ATTNRES_E_ALIGN: return "pointers must be 16-byte aligned and bank strides multiples of 8 elements";
    case ATTNRES_E_STRIDE: return "bank strides are negative or make rows overlap";
    case ATTNRES_E_ALIAS: return "a written buffer overlaps another argument";
    case ATTNRES_E_EPS: return "epsilon must be finite and >= 0";
    case ATTNRES_E_NOT_INIT: return "split-path workspace missing while the stream is capturing; call attnres_init first";
    case ATTNRES_E_HIP: return "a HIP runtime call failed";
    case ATTNRES_E_PATH: return "unknown path selector";
    case ATTNRES_E_DEVICE_WAIT: return "a cross-workgroup wait on the device gave up";
    default: return "unknown status";
  }
}

}  // namespace attnres

extern "C" int attnres_validate(const void *prefix, const void *delta, const void *blocks,
                                int64_t block_token_stride, int64_t block_slot_stride,
                                int max_blocks, int num_blocks, const void *res_w,
                                const void *rms_w, float rms_eps, const void *output_norm_weight,
                                float output_norm_eps, int block_write_idx, const void *out,
                                int64_t T, int64_t H) {
  attnres::FwdArgs a;
  a.prefix = prefix;
  a.delta = delta;
  a.blocks = blocks;
  a.block_token_stride = block_token_stride;
  a.block_slot_stride = block_slot_stride;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.res_w = res_w;
  a.rms_w = rms_w;
  a.rms_eps = rms_eps;
  a.output_norm_weight = output_norm_weight;
  a.output_norm_eps = output_norm_eps;
  a.block_write_idx = block_write_idx;
  a.out = out;
  a.T = T;
  a.H = H;
  return attnres::validate(a);
}

extern "C" const char *attnres_strerror(int status) { return attnres::strerror_text(status); }
