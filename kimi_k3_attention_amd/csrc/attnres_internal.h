// Internal declarations shared by the host-side translation units of
// libattnres (validation and launch).  Not part of the public ABI.
#pragma once

#include <cstdint>

#include "../../include/attnres.h"

namespace attnres {

constexpr int kHidden = 7168;          // the hidden size of the tuned row and split kernels
constexpr int kMaxHidden = ATTNRES_MAX_HIDDEN;  // largest H of the any-H row kernel
constexpr int kMaxBlocks = 8;          // bank rows a token may mix
// A dispatch counts its lanes (workgroups x lanes per workgroup) in 32 bits;
// every kernel uses at most 512 lanes per token.
constexpr int64_t kMaxTokens = 4294967295LL / 512;  // 8,388,607
constexpr int64_t kMaxStride = int64_t(1) << 46;

// Row strides (prefix_stride, delta_stride, out_stride) are in elements and
// ignored when T <= 1.
struct FwdArgs {
  const void *prefix = nullptr;
  int64_t prefix_stride = 0;
  const void *delta = nullptr;
  int64_t delta_stride = 0;
  const void *blocks = nullptr;
  int64_t block_token_stride = 0;
  int64_t block_slot_stride = 0;
  int max_blocks = 0;
  int num_blocks = 0;
  const void *res_w = nullptr;
  const void *rms_w = nullptr;
  float rms_eps = 0.f;
  const void *output_norm_weight = nullptr;
  float output_norm_eps = 0.f;
  int block_write_idx = -1;
  const void *out = nullptr;
  int64_t out_stride = 0;
  int64_t T = 0;
  int64_t H = 0;
};

int validate(const FwdArgs &a);
// The two-kernel form's partial-state buffer: bytes it needs for T tokens of
// hidden size H (an error code for sizes attnres_fwd rejects), and the checks
// of a given buffer against a validated call (NULL allowed when no bank row
// is read: num_blocks == 0 or T == 0).
int64_t partial_bytes(int64_t T, int64_t H);
int validate_partial(const FwdArgs &a, const void *partial, int64_t bytes);
// The row stride actually used for a [T, H] matrix argument.
inline int64_t row_stride(int64_t given, int64_t T, int64_t H) { return T <= 1 ? H : given; }
const char *strerror_text(int status);

// The split path's workspace frames.  ticks[x][c]: the set-up timing of
// candidate frame c from XCD x (smaller is nearer; INT_MAX where XCD x ran no
// timing workgroup).  Picks the pair {fa, fb} (fa < fb) whose nearer member
// gives the least total over the XCDs that were timed, the lowest indices on
// a tie, and sets bit x of *near when frame fb is strictly nearer XCD x than
// fa.  Host only.
constexpr int kFrameXcds = 8;
constexpr int kFrameCandidates = 4;
void choose_frames(const int (&ticks)[kFrameXcds][kFrameCandidates], int *fa, int *fb,
                   unsigned *near);

}  // namespace attnres
