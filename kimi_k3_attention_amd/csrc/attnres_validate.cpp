// Host-side argument checks of attnres_fwd / attnres_fwd_strided.  Pure C++:
// no HIP call and no pointer dereference, so it can be exercised without a GPU.
//
// The block-count and write-index domain follows the dispatch gate in the
// prhub digest of vLLM PR #54261 ("Implementation breakdown" item 3 and the
// attn_res.py snippet): 0 <= num_blocks <= 8, num_blocks <= capacity,
// -1 <= block_write_idx < capacity.  That gate also requires hidden size 7168
// and dense rows, which its fallback path covers otherwise; here any H that is
// a multiple of 8 up to ATTNRES_MAX_HIDDEN and any row strides are served
// instead (there is no fallback path: inputs outside the domain are rejected
// with an error code).  Alignment, stride and overlap checks protect the
// 16-byte vector accesses and the in-place writes.
#include "attnres_internal.h"

#include <climits>
#include <cmath>
#include <cstdint>

namespace attnres {
namespace {

using i128 = __int128;

// A set of n equally spaced byte ranges [base + k*stride, base + k*stride + len),
// k < n.  A single range has n == 1 (stride unused).
struct Rows {
  i128 base = 0, n = 0, stride = 0, len = 0;
  bool used = false;
  bool written = false;
};

Rows rows(const void *p, i128 n, i128 stride_bytes, i128 len_bytes, bool written) {
  Rows r;
  if (p == nullptr || n <= 0 || len_bytes <= 0) return r;
  r.base = static_cast<i128>(reinterpret_cast<uintptr_t>(p));
  r.n = n;
  r.stride = n > 1 ? stride_bytes : 0;
  r.len = len_bytes;
  r.used = true;
  r.written = written;
  return r;
}

i128 floor_div(i128 a, i128 b) {  // b > 0
  i128 q = a / b;
  if (a % b != 0 && a < 0) --q;
  return q;
}

// Whether some range of `a` shares a byte with some range of `b`.  Exact when
// the two sets have the same spacing (or one is a single range); otherwise it
// compares the spans they cover, which may reject interleavings that do not
// actually overlap.
bool overlap(const Rows &a, const Rows &b) {
  if (!a.used || !b.used) return false;
  const i128 a_hi = a.base + (a.n - 1) * a.stride + a.len;
  const i128 b_hi = b.base + (b.n - 1) * b.stride + b.len;
  if (!(a.base < b_hi && b.base < a_hi)) return false;
  if (a.stride != 0 && b.stride != 0 && a.stride != b.stride) return true;
  if (a.stride == 0 && b.stride == 0) return true;
  // Range i of a meets range j of b iff d - a.len < k*s < d + b.len with
  // k = i - j in [-(b.n - 1), a.n - 1] and d = b.base - a.base.
  const i128 s = a.stride != 0 ? a.stride : b.stride;
  const i128 d = b.base - a.base;
  i128 k_lo = floor_div(d - a.len, s) + 1;
  i128 k_hi = -floor_div(-(d + b.len), s) - 1;
  if (k_lo < -(b.n - 1)) k_lo = -(b.n - 1);
  if (k_hi > a.n - 1) k_hi = a.n - 1;
  return k_lo <= k_hi;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A [T, H] matrix's row stride: T <= 1 ignores it; otherwise >= H (rows must
// not overlap), a multiple of 8 (16-byte rows), and bounded.
int check_row_stride(int64_t s, int64_t T, int64_t H) {
  if (T <= 1) return ATTNRES_OK;
  if (s < 0) return ATTNRES_E_STRIDE;
  if (s > kMaxStride) return ATTNRES_E_SHAPE;
  if (s % 8 != 0) return ATTNRES_E_ALIGN;
  if (s < H) return ATTNRES_E_STRIDE;
  return ATTNRES_OK;
}

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
  if (a.H % 8 != 0 || a.H > kMaxHidden) return ATTNRES_E_UNSUPPORTED;
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

  int rc = check_row_stride(a.prefix_stride, a.T, a.H);
  if (rc == ATTNRES_OK && a.delta) rc = check_row_stride(a.delta_stride, a.T, a.H);
  if (rc == ATTNRES_OK) rc = check_row_stride(a.out_stride, a.T, a.H);
  if (rc != ATTNRES_OK) return rc;

  i128 bank_bytes = 0;
  if (bank_used) {
    if (a.block_token_stride < 0 || a.block_slot_stride < 0) return ATTNRES_E_STRIDE;
    if (a.block_token_stride > kMaxStride || a.block_slot_stride > kMaxStride) return ATTNRES_E_SHAPE;
    if ((a.block_token_stride % 8) != 0 || (a.block_slot_stride % 8) != 0) return ATTNRES_E_ALIGN;
    if (!bank_rows_disjoint(a.T, a.block_token_stride, a.max_blocks, a.block_slot_stride, a.H))
      return ATTNRES_E_STRIDE;
    bank_bytes = 2 * ((static_cast<i128>(a.T) - 1) * a.block_token_stride +
                      (static_cast<i128>(a.max_blocks) - 1) * a.block_slot_stride + a.H);
  }

  const i128 row_bytes = 2 * static_cast<i128>(a.H);
  const bool has_delta = a.delta != nullptr;
  auto mat = [&](const void *p, int64_t stride, bool written) {
    return rows(p, a.T, 2 * static_cast<i128>(row_stride(stride, a.T, a.H)), row_bytes, written);
  };
  // The bank is compared by the span it covers.
  const Rows r[7] = {
      mat(a.prefix, a.prefix_stride, has_delta),
      mat(a.delta, a.delta_stride, false),
      rows(bank_used ? a.blocks : nullptr, 1, 0, bank_bytes, a.block_write_idx >= 0),
      rows(a.res_w, 1, 0, row_bytes, false),
      rows(a.rms_w, 1, 0, row_bytes, false),
      rows(a.output_norm_weight, 1, 0, row_bytes, false),
      mat(a.out, a.out_stride, true),
  };
  // A buffer the call writes must not overlap any other argument.
  for (int i = 0; i < 7; ++i)
    for (int j = 0; j < 7; ++j)
      if (i != j && r[i].written && overlap(r[i], r[j])) return ATTNRES_E_ALIAS;
  return ATTNRES_OK;
}

int64_t partial_bytes(int64_t T, int64_t H) {
  if (T < 0 || T > kMaxTokens || H <= 0) return ATTNRES_E_SHAPE;
  if (H % 8 != 0 || H > kMaxHidden) return ATTNRES_E_UNSUPPORTED;
  return 4 * T * H + 8 * T;  // fp32 [T, H], then (m, s) per token
}

int validate_partial(const FwdArgs &a, const void *partial, int64_t bytes) {
  if (a.T == 0 || a.num_blocks == 0) return ATTNRES_OK;
  if (!partial) return ATTNRES_E_NULL;
  if (!aligned16(partial)) return ATTNRES_E_ALIGN;
  const int64_t need = partial_bytes(a.T, a.H);
  if (need < 0) return int(need);
  if (bytes < need) return ATTNRES_E_SHAPE;
  // Written by the bank part and read by the cur part: it must not share a
  // byte with any argument.
  const Rows w = rows(partial, 1, 0, need, true);
  const bool bank_used = a.num_blocks > 0 || a.block_write_idx >= 0;
  const i128 row_bytes = 2 * static_cast<i128>(a.H);
  auto mat = [&](const void *p, int64_t stride) {
    return rows(p, a.T, 2 * static_cast<i128>(row_stride(stride, a.T, a.H)), row_bytes, false);
  };
  i128 bank_bytes = 0;
  if (bank_used)
    bank_bytes = 2 * ((static_cast<i128>(a.T) - 1) * a.block_token_stride +
                      (static_cast<i128>(a.max_blocks) - 1) * a.block_slot_stride + a.H);
  const Rows r[7] = {
      mat(a.prefix, a.prefix_stride), mat(a.delta, a.delta_stride),
      rows(bank_used ? a.blocks : nullptr, 1, 0, bank_bytes, false),
      rows(a.res_w, 1, 0, row_bytes, false), rows(a.rms_w, 1, 0, row_bytes, false),
      rows(a.output_norm_weight, 1, 0, row_bytes, false), mat(a.out, a.out_stride)};
  for (const Rows &x : r)
    if (overlap(w, x)) return ATTNRES_E_ALIAS;
  return ATTNRES_OK;
}

const char *strerror_text(int status) {
  switch (status) {
    case ATTNRES_OK: return "ok";
    case ATTNRES_E_NULL: return "a required pointer is NULL";
    case ATTNRES_E_SHAPE: return "invalid or too large T, H, max_blocks or stride";
    case ATTNRES_E_UNSUPPORTED: return "unsupported size (H must be a multiple of 8 up to 16384; the split path takes T <= 256)";
    case ATTNRES_E_NUM_BLOCKS: return "num_blocks must be in 0..min(8, max_blocks)";
    case ATTNRES_E_WRITE_IDX: return "block_write_idx must be -1 or in 0..max_blocks-1";
    case ATTNRES_E_ALIGN: return "pointers must be 16-byte aligned and strides multiples of 8 elements";
    case ATTNRES_E_STRIDE: return "strides are negative or make rows overlap";
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

extern "C" int attnres_validate_strided(const void *prefix, int64_t prefix_stride,
                                        const void *delta, int64_t delta_stride,
                                        const void *blocks, int64_t block_token_stride,
                                        int64_t block_slot_stride, int max_blocks, int num_blocks,
                                        const void *res_w, const void *rms_w, float rms_eps,
                                        const void *output_norm_weight, float output_norm_eps,
                                        int block_write_idx, const void *out, int64_t out_stride,
                                        int64_t T, int64_t H) {
  attnres::FwdArgs a;
  a.prefix = prefix;
  a.prefix_stride = prefix_stride;
  a.delta = delta;
  a.delta_stride = delta_stride;
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
  a.out_stride = out_stride;
  a.T = T;
  a.H = H;
  return attnres::validate(a);
}

extern "C" int attnres_validate(const void *prefix, const void *delta, const void *blocks,
                                int64_t block_token_stride, int64_t block_slot_stride,
                                int max_blocks, int num_blocks, const void *res_w,
                                const void *rms_w, float rms_eps, const void *output_norm_weight,
                                float output_norm_eps, int block_write_idx, const void *out,
                                int64_t T, int64_t H) {
  return attnres_validate_strided(prefix, H, delta, H, blocks, block_token_stride,
                                  block_slot_stride, max_blocks, num_blocks, res_w, rms_w, rms_eps,
                                  output_norm_weight, output_norm_eps, block_write_idx, out, H, T,
                                  H);
}

extern "C" const char *attnres_strerror(int status) { return attnres::strerror_text(status); }

namespace attnres {

void choose_frames(const int (&ticks)[kFrameXcds][kFrameCandidates], int *fa, int *fb,
                   unsigned *near) {
  *fa = 0;
  *fb = 1;
  int64_t best = -1;
  for (int i = 0; i < kFrameCandidates; ++i)
    for (int j = i + 1; j < kFrameCandidates; ++j) {
      int64_t cost = 0;
      for (int x = 0; x < kFrameXcds; ++x) {
        if (ticks[x][i] == INT_MAX && ticks[x][j] == INT_MAX) continue;  // not timed
        cost += ticks[x][i] < ticks[x][j] ? ticks[x][i] : ticks[x][j];
      }
      if (best < 0 || cost < best) {
        best = cost;
        *fa = i;
        *fb = j;
      }
    }
  *near = 0;
  for (int x = 0; x < kFrameXcds; ++x)
    if (ticks[x][*fb] < ticks[x][*fa]) *near |= 1u << x;
}

}  // namespace attnres
