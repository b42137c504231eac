// Host-side argument checks of libattnres under the address and undefined-
// behaviour sanitizers: a seeded stream of argument sets, from plausible
// layouts to extreme sizes, strides, indices, epsilons and pointers, goes
// through validate, validate_partial and partial_bytes.  Every call must
// return a documented status (no crash, no overflow, no out-of-range shift);
// a few fixed cases pin the answer.  Built and run by tests/test_boundary.py
// with g++ (host code only); prints "ok <calls>" on success.  Also pins the
// choice of the split path's two workspace frames from set-up timings.
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>

#include "attnres_internal.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}
int64_t pick(const int64_t *v, int n) { return v[next() % uint64_t(n)]; }

const int64_t kSizes[] = {-1, 0, 1, 2, 3, 7, 8, 9, 16, 64, 1024, 7168, 16384, 16392,
                          8388607, 8388608, int64_t(1) << 31, int64_t(1) << 40,
                          std::numeric_limits<int64_t>::max(),
                          std::numeric_limits<int64_t>::min()};
const int64_t kStrides[] = {-8, 0, 8, 16, 24, 64, 7168, 8 * 7168, 8 * 7168 + 64,
                            int64_t(1) << 40, int64_t(1) << 46, (int64_t(1) << 46) + 8,
                            int64_t(1) << 62, std::numeric_limits<int64_t>::max(),
                            std::numeric_limits<int64_t>::min()};
const int64_t kSmall[] = {-1000, -2, -1, 0, 1, 2, 3, 4, 7, 8, 9, 1000, 2147483647,
                          -2147483647 - 1};
const float kEps[] = {0.f, 1e-6f, 1.f, -1e-6f, std::numeric_limits<float>::infinity(),
                      -std::numeric_limits<float>::infinity(),
                      std::numeric_limits<float>::quiet_NaN(),
                      std::numeric_limits<float>::denorm_min()};

const void *ptr() {
  static const uintptr_t bases[] = {0,
                                    0x1000,
                                    0x10000000,
                                    0x10000008,
                                    0x7fff00000000,
                                    uintptr_t(-16),
                                    uintptr_t(-1) - 64};
  uintptr_t p = bases[next() % 7];
  if (next() % 3 == 0) p += 16 * (next() % 4096);
  return reinterpret_cast<const void *>(p);
}

bool documented(int rc) { return rc <= 0 && rc >= ATTNRES_E_DEVICE_WAIT; }

}  // namespace

int main() {
  using namespace attnres;
  long calls = 0;
  for (int it = 0; it < 200000; ++it) {
    FwdArgs a;
    const bool plausible = next() % 2 == 0;
    a.T = plausible ? int64_t(next() % 6) : pick(kSizes, 20);
    a.H = plausible ? int64_t(8 * (1 + next() % 4)) : pick(kSizes, 20);
    a.max_blocks = int(plausible ? next() % 10 : pick(kSmall, 14));
    a.num_blocks = int(plausible ? next() % 10 : pick(kSmall, 14));
    a.block_write_idx = int(plausible ? int64_t(next() % 11) - 1 : pick(kSmall, 14));
    a.block_token_stride = plausible ? int64_t(8 * (next() % 40)) : pick(kStrides, 15);
    a.block_slot_stride = plausible ? int64_t(8 * (next() % 10)) : pick(kStrides, 15);
    a.prefix_stride = plausible ? a.H + int64_t(8 * (next() % 3)) : pick(kStrides, 15);
    a.delta_stride = plausible ? a.H : pick(kStrides, 15);
    a.out_stride = plausible ? a.H + int64_t(8 * (next() % 3)) : pick(kStrides, 15);
    a.prefix = ptr();
    a.delta = next() % 3 ? ptr() : nullptr;
    a.blocks = next() % 4 ? ptr() : nullptr;
    a.res_w = ptr();
    a.rms_w = ptr();
    a.output_norm_weight = next() % 3 ? ptr() : nullptr;
    a.out = ptr();
    a.rms_eps = kEps[next() % 8];
    a.output_norm_eps = kEps[next() % 8];

    const int rc = validate(a);
    const int64_t need = partial_bytes(a.T, a.H);
    const int rp = validate_partial(a, ptr(), plausible ? need : pick(kSizes, 20));
    calls += 3;
    if (!documented(rc) || !documented(rp) || (need < 0 && !documented(int(need)))) {
      std::printf("undocumented status: validate %d, partial %d, bytes %lld\n", rc, rp,
                  static_cast<long long>(need));
      return 1;
    }
    (void)strerror_text(rc);
  }

  // Fixed answers: a valid call, and one just over each of the size limits.
  FwdArgs v;
  v.T = 4;
  v.H = 7168;
  v.prefix = reinterpret_cast<const void *>(0x10000000);
  v.prefix_stride = 7168;
  v.blocks = reinterpret_cast<const void *>(0x40000000);
  v.block_token_stride = 8 * 7168;
  v.block_slot_stride = 7168;
  v.max_blocks = 8;
  v.num_blocks = 4;
  v.res_w = reinterpret_cast<const void *>(0x30000000);
  v.rms_w = reinterpret_cast<const void *>(0x30100000);
  v.out = reinterpret_cast<const void *>(0x50000000);
  v.out_stride = 7168;
  v.rms_eps = 1e-6f;
  FwdArgs big_t = v, big_h = v, big_stride = v;
  big_t.T = kMaxTokens + 1;
  big_h.H = kMaxHidden + 8;
  big_stride.block_token_stride = kMaxStride + 8;
  if (validate(v) != ATTNRES_OK || validate(big_t) != ATTNRES_E_SHAPE ||
      validate(big_h) != ATTNRES_E_UNSUPPORTED || validate(big_stride) != ATTNRES_E_SHAPE ||
      partial_bytes(4, 7168) != 4 * 4 * 7168 + 8 * 4) {
    std::printf("fixed cases: %d %d %d %d %lld\n", validate(v), validate(big_t), validate(big_h),
                validate(big_stride), static_cast<long long>(partial_bytes(4, 7168)));
    return 1;
  }
  // The workspace frames' choice: two XCD halves that each find a different
  // pair member near, ties, and XCDs that ran no timing workgroup.
  {
    int ticks[kFrameXcds][kFrameCandidates];
    for (int x = 0; x < kFrameXcds; ++x)
      for (int c = 0; c < kFrameCandidates; ++c)
        ticks[x][c] = ((x < 4) == (c % 2 == 0)) ? 30 : 55;  // even frames near XCDs 0-3
    int fa = -1, fb = -1;
    unsigned near = 0;
    choose_frames(ticks, &fa, &fb, &near);
    if (fa != 0 || fb != 1 || near != 0xF0u) {
      std::printf("frames: alternating halves gave %d %d %x\n", fa, fb, near);
      return 1;
    }
    for (auto &row : ticks)
      for (int &v : row) v = 40;
    choose_frames(ticks, &fa, &fb, &near);
    if (fa != 0 || fb != 1 || near != 0u) {
      std::printf("frames: equal timings gave %d %d %x\n", fa, fb, near);
      return 1;
    }
    // frames 2 and 3 are the good pair; XCDs 5-7 were not timed
    for (int x = 0; x < kFrameXcds; ++x)
      for (int c = 0; c < kFrameCandidates; ++c)
        ticks[x][c] = x >= 5 ? INT_MAX : c == 3 ? (x < 2 ? 20 : 60) : c == 2 ? (x < 2 ? 60 : 20) : 70;
    choose_frames(ticks, &fa, &fb, &near);
    if (fa != 2 || fb != 3 || near != 0x3u) {
      std::printf("frames: partial timing gave %d %d %x\n", fa, fb, near);
      return 1;
    }
    calls += 3;
  }
  std::printf("ok %ld\n", calls);
  return 0;
}
