// libattnres kernels and launch layer: the Kimi-K3 attention-residual forward
// on MI355X (gfx950, CDNA4, wave64).
//
// The operation is defined in include/attnres.h (vllm-ascend PR #14840,
// "Implementation walkthrough"; prhub digest of vLLM PR #54261, kernel
// snippet under "Key source snippets").  The work is a streaming reduction:
// per token it reads num_blocks + 1 (+1 with a delta) rows of H bf16 once,
// reduces each row to two scalars, and writes 1-3 rows.  Arithmetic intensity
// is about 2 flop/byte, far below the fp32 ridge, so HBM bandwidth bounds it
// and the streaming reduction uses no matrix core.  The one dense contraction
// is the split path's Gram matrix of a part's rows (for the output norm),
// formed on the matrix cores when it is large.
//
// Layout of the work: a "segment" is 8 consecutive bf16 (16 bytes); a row of
// 7168 is 896 segments.  A lane owns one or more segments of every source row
// of its token, so each row is read with 128-bit loads and the whole token
// stays in VGPRs between the reduction and the mixture (no second read).
//
//  * Row path (H = 7168, many tokens): one 448-lane workgroup (7 waves, two
//    segments per lane) per token.  Per-lane fp32 sum-of-squares and query
//    dot of every source (packed bf16 dot products), a 16-lane DPP reduction,
//    a cross-row reduction through LDS, logits, an online softmax (running
//    maximum and rescaled sum, merged as a tree over at most 9 lanes), the
//    fp32 mixture, the
//    optional output RMSNorm (a second LDS reduction), bf16
//    round-to-nearest-even stores.  With no bank rows the only source has
//    weight 1: no logit, and at most the output norm's reduction.
//  * Split path (H = 7168, few tokens): 14 single-wave workgroups per token,
//    each owning 512 elements of every row, so one token is spread over 14
//    CUs.  Per-part sums (and, with an output norm, the sources' Gram matrix),
//    summed over the wave by DPP (few words), an LDS transposition (more) or
//    one matrix-core product X X^T of the part's rows (the most, nb >= 7 with
//    a norm), are exchanged once through a device workspace of self-validating tagged
//    words read and written with agent-scope atomics (the 8 XCDs do not share
//    L2); no reset is needed between calls or graph replays.  Waits are
//    bounded: a wait that gives up raises a device flag instead of hanging.
//  * Any-H row path (other hidden sizes, multiples of 8 up to 16384): the row
//    path's steps with a runtime row length, 64-512 lanes per token and two
//    or four segments per lane; segments past the row end are masked.
//
// Compile-time specialisation on num_blocks (0..8), delta and output norm,
// and on whether the rows a call rewrites are read through the cache;
// block_write_idx stays a uniform runtime branch.  Row strides of prefix,
// delta and out are runtime values.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <mutex>

#include "attnres_internal.h"

// Tuning knobs, fixed at compile time.  Every setting computes the full
// result; they only change occupancy, grid shape and cache policy.
#ifndef ATTNRES_ROW_MAX_VGPRS
#define ATTNRES_ROW_MAX_VGPRS 128       // <= 128: 4 waves/SIMD, so two 7-wave workgroups
#endif                                  // fit a CU however its waves spread over SIMDs
#ifndef ATTNRES_ROW_WGS_PER_CU
#define ATTNRES_ROW_WGS_PER_CU 0        // 0: by block count (below); k: k per CU, looping, always
#endif
#ifndef ATTNRES_SPIN_SLEEP
#define ATTNRES_SPIN_SLEEP 1              // s_sleep argument between polls (x64 cycles)
#endif
#ifndef ATTNRES_NT_LOADS
#define ATTNRES_NT_LOADS 1              // streaming rows read non-temporally
#endif
#ifndef ATTNRES_NT_STORES
#define ATTNRES_NT_STORES 1             // streaming rows written non-temporally
#endif
#ifndef ATTNRES_NT_STORE_CUR
#define ATTNRES_NT_STORE_CUR ATTNRES_NT_STORES  // policy for the in-place prefix / bank rows
#endif
#ifndef ATTNRES_SPLIT_DPP_WORDS
#define ATTNRES_SPLIT_DPP_WORDS 8       // split path: words summed by DPP instead of via LDS
#endif
#ifndef ATTNRES_SPLIT_MFMA_WORDS
#define ATTNRES_SPLIT_MFMA_WORDS 35     // split path: from this many words, one matrix-core product
#endif
#ifndef ATTNRES_ANYH_STAGED
#define ATTNRES_ANYH_STAGED 1           // any-H: three bank rows staged in LDS where it pays
#endif
#ifndef ATTNRES_CUR_FIRST
#define ATTNRES_CUR_FIRST 1             // issue prefix and delta before the bank rows
#endif
#ifndef ATTNRES_EARLY_CUR_STORE
#define ATTNRES_EARLY_CUR_STORE 1       // row kernel, cached in-place rows: write prefix /
#endif                                  // bank rows once every load has landed, not with out

namespace attnres {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kSeg = 8;                       // bf16 per 16-byte segment
constexpr int kSegs = kHidden / kSeg;         // 896 segments per row
constexpr int kWave = 64;
constexpr int kRowSegsPerLane = 2;           // row path: two segments per lane
constexpr int kRowThreads = kSegs / kRowSegsPerLane;  // 448 = 7 waves
constexpr int kRowWaves = kRowThreads / kWave;        // 7
constexpr int kParts = 14;                    // split path: workgroups per token
constexpr int kPartThreads = kSegs / kParts;  // 64 = one wave
constexpr int kSlot = 64;                     // 64-bit words per (token, part) workspace slot
constexpr int kSlotYsq = kSlot - 1;           // where a part's sum of y^2 goes
constexpr int kSpinLimit = 1 << 20;           // bounded cross-workgroup wait
// Fourth word of a raw buffer resource: 32-bit data format, no swizzle.
constexpr int kBufferFormat = 0x00020000;
constexpr int kAuxNt = 2;  // cache-policy operand of a load: non-temporal
constexpr float kInvHidden = 1.0f / kHidden;

// Row path: calls of at most kRowRangedMaxT[nb] tokens with two or more
// bank rows read them with range-checked loads (the row kernel's RANGED
// form).  Measured against plain loads, bit-identical: T = 32-176 at nb =
// 2-8 0.3-3.7 % faster, T = 192 0.2-0.8 %; T = 208-256 0.2-1 % slower at
// nb = 4-8 but 0.8-2.3 % faster at nb = 2; T = 384-768 slower at every nb;
// nb = 1 no faster at any T.  nb = 3 at T = 208-256 and nb = 2 at 288-320:
// within the 1.3 % spread between library copies.
constexpr int kRowRangedMinBlocks = 2;
constexpr int kRowRangedMaxT[kMaxBlocks + 1] = {0, 0, 256, 192, 192, 192, 192, 192, 192};

// Row path grid.  With few source rows a token moves little data, and with
// one workgroup per token the whole grid is resident at once, so every token
// loads, computes and stores in lockstep; a persistent grid of three
// workgroups per CU looping over tokens desynchronises those phases (measured
// 5-12% faster at T = 1024 for nb <= 1).  With more rows the loop's hoisted
// weights cost registers and one workgroup per token is faster.
constexpr int kRowPersistMaxNb = 1;
constexpr int kRowPersistWgsPerCu = 3;
__host__ __device__ constexpr int row_wgs_per_cu(int nb) {
  return ATTNRES_ROW_WGS_PER_CU > 0 ? ATTNRES_ROW_WGS_PER_CU
                                    : (nb <= kRowPersistMaxNb ? kRowPersistWgsPerCu : 0);
}

static_assert(kSegs * kSeg == kHidden, "hidden size must be a multiple of 8");
static_assert(kRowThreads % kWave == 0 && kRowThreads * kRowSegsPerLane == kSegs,
              "row workgroup must be whole waves covering the row");
static_assert(kPartThreads == kWave, "a split part is one wave");
static_assert((kMaxBlocks + 1) * (kMaxBlocks + 2) / 2 + kMaxBlocks + 1 <= kSlotYsq,
              "workspace slot too small");

struct KParams {
  uint16_t *prefix;
  const uint16_t *delta;
  uint16_t *blocks;
  const uint16_t *res_w;
  const uint16_t *rms_w;
  const uint16_t *onw;
  uint16_t *out;
  int64_t tok_stride;     // bank, elements
  int64_t slot_stride;
  int64_t prefix_stride;  // row strides, elements
  int64_t delta_stride;
  int64_t out_stride;
  float rms_eps;
  float out_eps;
  int widx;
  int T;
  int nseg;               // segments per row (H / 8); the any-H kernel's row length
  int threads;            // lanes per workgroup of the any-H launch shape (a kernel
                          // argument: blockDim.x would be read with a vector load)
  float inv_h;            // 1 / H
  uint64_t *ws_part;       // split path: tagged words, 14 parts per token (frame A)
  uint64_t *ws_part_b;     // the same words in frame B (== ws_part: one frame)
  unsigned ws_near;        // bit x: frame B is the one a part on XCD x writes
  int ws_by_part;          // tests only: bit `part` of ws_near chooses instead
  unsigned *ws_flag;
  int spin_limit;          // split path: polls before a wait gives up
  uint32_t wait_skew;      // split path: added to the awaited generation (0; tests only)
  float *partial;          // two-kernel form: the bank part's state (see attnres_bank_kernel)
};

// ---------------------------------------------------------------------------
// device helpers
// ---------------------------------------------------------------------------

// Streaming rows are touched exactly once: non-temporal 128-bit accesses keep
// them from evicting the weights, which every workgroup re-reads from L2.
__device__ __forceinline__ u32x4 load_stream(const uint16_t *p) {
#if ATTNRES_NT_LOADS
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
#else
  return *reinterpret_cast<const u32x4 *>(p);
#endif
}
__device__ __forceinline__ u32x4 load_cached(const uint16_t *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}
template <bool NT = ATTNRES_NT_STORES>
__device__ __forceinline__ void store_stream(uint16_t *p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
  else
    *reinterpret_cast<u32x4 *>(p) = v;
}

// bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32.
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (gfx950 converts in one
// instruction under the default rounding mode).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// acc + a.lo * b.lo + a.hi * b.hi on packed bf16 pairs, fp32 accumulate
// (v_dot2c_f32_bf16): the products of bf16 values are exact in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_src(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, false));
}

// Butterfly sum inside each 16-lane row of a wave (xor 1, xor 2, half-row
// mirror, row mirror): afterwards every lane of a row holds its row's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_src<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_src<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_src<0x141>(v);  // row_half_mirror
  v += dpp_src<0x140>(v);  // row_mirror
  return v;
}

// Sum over the 64 lanes of a wave, valid in lane 63: the row sums, then row 0
// folded into row 1 and row 2 into row 3 (broadcast of lanes 15 / 47), then
// rows 0+1 into row 3 (broadcast of lane 31).  Fixed order: repeatable.
__device__ __forceinline__ float wave_sum_lane63(float v) {
  v = row16_sum(v);
  v += dpp_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// v of lane `src` (any lane of the wave), through the LDS crossbar.
__device__ __forceinline__ float lane_shuffle(float v, int src) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// One token's data for SPL segments per lane: segment i of this lane is
// seg0 + i * seg_step.  Everything is issued in one burst: the L2-resident
// weights first (the wait counter is in order, so the query can be formed
// while the rows are still in flight), then the rows: prefix and delta
// before the bank rows (kCurFirst, from three bank rows up) or after them.
// Row bases are workgroup-uniform (scalar registers); lanes add their
// 16-byte segment offsets.
//
// MASKED (rows whose length is not a multiple of the workgroup's reach):
// a segment at or past p.nseg reads zero (a range-checked load), which adds
// nothing to any sum, and is never stored.
// CUR = false: the bank rows only (the first kernel of the two-kernel form),
// no prefix, delta or cur.  Q: load the scoring weights for the fused query
// (needed whenever a logit is formed: with bank rows, or in the second
// kernel of the two-kernel form, which scores cur alone).
//
// LR > 0 (STG): the first LR sources (bank rows) are staged into LDS, which
// frees 4 SPL registers per row, so that more workgroups fit a CU (see the
// any-H kernel).  They are loaded into registers right after cur's rows,
// their partials are taken as they land, and then each lane copies them to
// its own LDS slots, from which the mixture reads them.  The other bank rows
// are issued as registers free up (issue_rest).  Every load is a plain one,
// so the waits stay progressive: with LDS-direct loads (global_load_lds) in
// flight, the compiler waits for every load at the first use of any.
template <int NB, bool DELTA, bool ONORM, int SPL, bool MASKED = false, bool CACHE_RW = false,
          bool CUR = true, bool Q = (NB > 0), int LR = 0>
struct Token {
  static constexpr int NS = NB + (CUR ? 1 : 0);
  static constexpr bool STG = LR > 0;
  static_assert(LR == 0 || (CUR && LR < NB), "LDS rows are bank rows of a full token");
  // STG: bank rows (in issue order) of the first burst, the staged ones;
  // the rest follow the staging.  With cur's two rows and the weights that
  // is what the register budgets leave room for (96 VGPRs at two segments
  // per lane, 168 at four).
  static constexpr int kFirst = STG ? LR : NB;
  u32x4 rms[SPL], res[SPL], onw[SPL];  // weights
  u32x4 x[NB + 1][SPL];                // bank slots 0..NB-1, then prefix (cur after finish_cur)
  u32x4 d[SPL];                        // delta
  u32x4 *lds_rows = nullptr;           // LR > 0: [LR][SPL][lanes] in LDS
  int nthr = 0;                        // lanes per workgroup (LR > 0)
  bool seg_ok[SPL];

  // Source j, segment i: from LDS for the first LR sources (zero past a
  // masked row's end: staged rows carry the zeros their loads gave), else
  // from registers.
  __device__ __forceinline__ u32x4 row(int j, int i) const {
    if (j < LR) return lds_rows[(j * SPL + i) * nthr + int(threadIdx.x)];
    return x[j][i];
  }
  // STG: staged row k from this lane's registers to its own LDS slots.
  __device__ __forceinline__ void stage(int k) {
    if constexpr (STG)
#pragma unroll
      for (int i = 0; i < SPL; ++i) lds_rows[(k * SPL + i) * nthr + int(threadIdx.x)] = x[k][i];
  }

  __device__ __forceinline__ static bool in_row(const KParams &p, int seg) {
    return !MASKED || seg < p.nseg;
  }
  // Byte offset of a lane's segment i within a row.  Past segment 0 it
  // exceeds the 4 KB immediate offset of a load or store, and the compiler
  // would then form a 64-bit address for every row (and keep the stores'
  // live through the kernel); held opaque in one 32-bit register, it is
  // shared by all rows, each addressed as scalar row base + this offset.
  // STG: recomputed at every use, from a fresh opaque copy of seg0 (kept
  // live anyway), so that the offsets are not merged into values live
  // through the kernel: there they spilled, and a spill's reload waits for
  // every load and store in flight.
  __device__ __forceinline__ static uint32_t seg_bytes(int seg0, int seg_step, int i) {
    if constexpr (STG) {
      uint32_t s0 = uint32_t(seg0);
      if (i > 0) asm volatile("" : "+v"(s0));
      return (s0 + uint32_t(i * seg_step)) * uint32_t(kSeg * sizeof(uint16_t));
    } else {
      uint32_t b = uint32_t(seg0 + i * seg_step) * uint32_t(kSeg * sizeof(uint16_t));
      if (i > 0) asm("" : "+v"(b));
      return b;
    }
  }
  __device__ __forceinline__ static const uint16_t *at(const uint16_t *row, uint32_t b) {
    return reinterpret_cast<const uint16_t *>(reinterpret_cast<const char *>(row) + b);
  }
  __device__ __forceinline__ static uint16_t *at(uint16_t *row, uint32_t b) {
    return reinterpret_cast<uint16_t *>(reinterpret_cast<char *>(row) + b);
  }
  // A row's segment at byte offset b.  MASKED: a buffer load whose record is
  // the row, so a segment at or past the row's end reads zero by the
  // hardware's range check, with no branch: a branch around each load left
  // the compiler unable to count the loads in flight, and every source's
  // arithmetic then waited for all of them.
  template <int AUX>
  __device__ __forceinline__ static u32x4 load_in_row(const KParams &p, const uint16_t *row,
                                                      uint32_t b) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(row), 0, p.nseg * kSeg * int(sizeof(uint16_t)), kBufferFormat);
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(b), 0, AUX);
  }
  // (Staged tokens take the buffer form whether masked or not: it holds fewer
  // registers, which decides how many of their workgroups fit a CU.)
  static constexpr bool kBufferRows = MASKED || STG;
  __device__ __forceinline__ static u32x4 load_row(const KParams &p, const uint16_t *row,
                                                   uint32_t b, bool ok) {
    (void)ok;
    if constexpr (kBufferRows) return load_in_row<ATTNRES_NT_LOADS ? kAuxNt : 0>(p, row, b);
    return load_stream(at(row, b));
  }
  // With CACHE_RW, the rows a call also writes (the bank slot widx, a source
  // here, and prefix when a delta is given) are read through the cache at
  // normal priority, so that their writes find the lines resident, while rows
  // only read stream past the cache (load_row).  The slot is chosen at run
  // time, so its load sits in a uniform branch beside the streaming one; it
  // is a buffer load, a different instruction, which the compiler cannot
  // merge with the streaming load (merging two plain loads would drop the
  // non-temporal hint).  The record size is the row, so a segment past a
  // masked row's end reads zero, as load_row's masking gives.
  __device__ __forceinline__ static u32x4 load_rewritten(const KParams &p, const uint16_t *row,
                                                         uint32_t bytes) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(row), 0, p.nseg * kSeg * int(sizeof(uint16_t)), kBufferFormat);
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(bytes), 0, 0);
  }
  __device__ __forceinline__ static u32x4 load_weight(const KParams &p, const uint16_t *w,
                                                      uint32_t b, bool ok) {
    (void)ok;
    if constexpr (MASKED) return load_in_row<0>(p, w, b);
    return load_cached(at(w, b));
  }

  // prefix and delta (cur's rows) before the bank rows, from three bank rows
  // up: cur's arithmetic, the longest of any source's (the add and rounding,
  // then its partials), then overlaps the bank rows' arrival instead of
  // following the last load.  With one or two bank rows the other order
  // measured faster.  (The LDS-row variant keeps its own order.)
  static constexpr bool kCurFirst = STG || (ATTNRES_CUR_FIRST && CUR && LR == 0 && NB >= 3);

  // Bank rows K0..K1-1 in issue order, each followed by a scheduling barrier.
  // Issue order k is slot k, or in the cached variant the slots other than
  // widx ascending and then widx (k = NB - 1) through the cache (see issue).
  template <int K0, int K1>
  __device__ __forceinline__ void issue_bank(const KParams &p, const uint16_t *bank,
                                             const uint32_t (&sb)[SPL], const bool (&ok)[SPL]) {
    constexpr int kPlain = CACHE_RW ? (K1 < NB - 1 ? K1 : NB - 1) : K1;
#pragma unroll
    for (int k = K0; k < kPlain; ++k) {
      const int slot = CACHE_RW ? k + (k >= p.widx ? 1 : 0) : k;
      const uint16_t *row = bank + slot * p.slot_stride;
#pragma unroll
      for (int i = 0; i < SPL; ++i) x[k][i] = load_row(p, row, sb[i], ok[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (CACHE_RW && K1 == NB) {
      const uint16_t *row = bank + p.widx * p.slot_stride;
#pragma unroll
      for (int i = 0; i < SPL; ++i) x[NB - 1][i] = load_rewritten(p, row, sb[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // STG: bank rows K0..K1-1 of those after the first burst (clamped to NB),
  // each as soon as registers are free for it: one once cur is formed
  // (delta's registers), one after each staged row but the last, the rest
  // after the last.
  template <int K0, int K1>
  __device__ __forceinline__ void issue_rest(const KParams &p, int64_t t, int seg0, int seg_step) {
    constexpr int k0 = K0 < NB ? K0 : NB, k1 = K1 < NB ? K1 : NB;
    if constexpr (STG && k0 < k1) {
      bool ok[SPL];
      uint32_t sb[SPL];
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        ok[i] = seg_ok[i];
        sb[i] = seg_bytes(seg0, seg_step, i);
      }
      __builtin_amdgcn_sched_barrier(0);
      issue_bank<k0, k1>(p, p.blocks + t * p.tok_stride, sb, ok);
    }
  }

  // cur's rows: prefix (through the cache when the call rewrites it) and delta.
  __device__ __forceinline__ void issue_cur(const KParams &p, int64_t t, const uint16_t *prow,
                                            const uint32_t (&sb)[SPL], const bool (&ok)[SPL]) {
    if constexpr (CUR) {
      if constexpr (CACHE_RW && DELTA) {
#pragma unroll
        for (int i = 0; i < SPL; ++i) x[NB][i] = load_rewritten(p, prow, sb[i]);
      } else {
#pragma unroll
        for (int i = 0; i < SPL; ++i) x[NB][i] = load_row(p, prow, sb[i], ok[i]);
      }
      if constexpr (DELTA)
#pragma unroll
        for (int i = 0; i < SPL; ++i)
          d[i] = load_row(p, p.delta + t * p.delta_stride, sb[i], ok[i]);
    }
  }

  __device__ __forceinline__ void issue(const KParams &p, int64_t t, int seg0, int seg_step) {
    bool ok[SPL];
    uint32_t sb[SPL];
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      ok[i] = in_row(p, seg0 + i * seg_step);
      seg_ok[i] = ok[i];
      sb[i] = seg_bytes(seg0, seg_step, i);
    }
    if constexpr (Q)  // a single source needs no logit, hence no query
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        rms[i] = load_weight(p, p.rms_w, sb[i], ok[i]);
        res[i] = load_weight(p, p.res_w, sb[i], ok[i]);
      }
    const uint16_t *bank = p.blocks + t * p.tok_stride;
    const uint16_t *prow = p.prefix + t * p.prefix_stride;
    if constexpr (kCurFirst) {
      issue_cur(p, t, prow, sb, ok);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (STG) {
      // cur, then the staged rows and two more; the rest after the staging.
      issue_bank<0, kFirst>(p, bank, sb, ok);
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    if constexpr (!CUR) {
      // The bank rows alone, in source order.
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < SPL; ++i)
          x[j][i] = load_row(p, bank + j * p.slot_stride, sb[i], ok[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      return;
    } else if constexpr (CACHE_RW) {
      // The in-place rows (the written slot, a source here, and prefix when
      // a delta rewrites it) are read through the cache.  The slot is chosen
      // at run time, so the sources are taken in a different order with no
      // branch: the other slots ascending (streamed, a scalar index skipping
      // widx), then slot widx; the mixture is the same sum in another order.
      // A branch per slot would leave the compiler unable to count the loads
      // in flight, and every source's arithmetic would wait for all of them.
      static_assert(NB > 0, "a rewritten source row needs a source slot");
#pragma unroll
      for (int k = 0; k + 1 < NB; ++k) {
        const int slot = k + (k >= p.widx ? 1 : 0);
        const uint16_t *row = bank + slot * p.slot_stride;
#pragma unroll
        for (int i = 0; i < SPL; ++i) x[k][i] = load_row(p, row, sb[i], ok[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
      {
        const uint16_t *row = bank + p.widx * p.slot_stride;
#pragma unroll
        for (int i = 0; i < SPL; ++i) x[NB - 1][i] = load_rewritten(p, row, sb[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // Rows are issued in source order (the scheduler would otherwise order
      // them by when their addresses are ready), so that the partials of each
      // source can start as soon as its own rows land.
#pragma unroll
      for (int j = 0; j < NB; ++j) {
#pragma unroll
        for (int i = 0; i < SPL; ++i)
          x[j][i] = load_row(p, bank + j * p.slot_stride, sb[i], ok[i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (!kCurFirst) issue_cur(p, t, prow, sb, ok);
    // Keep the scheduler from sinking any of these loads below the arithmetic.
    __builtin_amdgcn_sched_barrier(0);
  }

  // The output-norm weight is needed only by the final store: loading it once
  // the logits are known (an L2 hit) keeps it out of the registers that hold
  // the rows during the reductions.
  __device__ __forceinline__ void issue_onw(const KParams &p, int seg0, int seg_step) {
    if constexpr (ONORM)
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        onw[i] = load_weight(p, p.onw, seg_bytes(seg0, seg_step, i), in_row(p, seg0 + i * seg_step));
      }
  }

  // Between the last source's partials and the logits (row and any-H
  // kernels): the workgroup barrier, then the output-norm weight's load; or,
  // EARLY, that load, then cur's in-place writes (every load of the lane has
  // landed), then the barrier.  The weight goes first because loads and
  // stores share one in-order counter: a load issued after the writes would
  // wait for them.
  // ONW = false: the weight is loaded later by the caller (after the
  // mixture, where the rows no longer hold registers).
  template <bool EARLY, bool ONW = true>
  __device__ __forceinline__ void after_partials(const KParams &p, int64_t t, int seg0,
                                                 int seg_step) {
    if constexpr (EARLY) {
      if constexpr (ONW) issue_onw(p, seg0, seg_step);
      store_cur(p, t, seg0, seg_step);
      __syncthreads();
    } else {
      __syncthreads();
      if constexpr (ONW) issue_onw(p, seg0, seg_step);
    }
  }

  // Fused query q = rms_w * res_w, split exactly into two packed bf16 words:
  // q has at most 16 significant bits (a product of two 8-bit significands),
  // so q_hi = bf16_RNE(q) and the residual q_lo = q - q_hi (computed exactly
  // in fp32) is itself a bf16 value, and q = q_hi + q_lo.
  __device__ __forceinline__ void query(u32x4 (&qh)[SPL], u32x4 (&ql)[SPL]) const {
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float a = bf_lo(rms[i][k]) * bf_lo(res[i][k]);
        const float b = bf_hi(rms[i][k]) * bf_hi(res[i][k]);
        qh[i][k] = pack_bf16x2(a, b);
        ql[i][k] = pack_bf16x2(a - bf_lo(qh[i][k]), b - bf_hi(qh[i][k]));
      }
    __builtin_amdgcn_sched_barrier(0);
  }

  // cur = bf16_RNE(prefix + delta) into x[NB].  The fp32 sum of two bf16
  // values is within 2^-24 (relative) of the exact sum, which is never close
  // enough to a bf16 rounding boundary to change the rounded result.
  __device__ __forceinline__ void finish_cur() {
    if constexpr (CUR && DELTA) {
#pragma unroll
      for (int i = 0; i < SPL; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          x[NB][i][k] = pack_bf16x2(bf_lo(x[NB][i][k]) + bf_lo(d[i][k]),
                                    bf_hi(x[NB][i][k]) + bf_hi(d[i][k]));
    }
  }

  // Per-lane partial sum of squares and query dot of source j.
  // REGS: from registers even for an LDS row (a staged row before staging).
  template <bool REGS = false>
  __device__ __forceinline__ void partial(int j, const u32x4 (&qh)[SPL], const u32x4 (&ql)[SPL],
                                          float &ss, float &dq) const {
    float s = 0.f, dd = 0.f;
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const u32x4 v = REGS ? x[j][i] : row(j, i);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        s = dot2(v[k], v[k], s);
        dd = dot2(qh[i][k], v[k], dd);
        dd = dot2(ql[i][k], v[k], dd);
      }
    }
    ss = s;
    dq = dd;
  }

  // The same for every source.
  __device__ __forceinline__ void partials(const u32x4 (&qh)[SPL], const u32x4 (&ql)[SPL],
                                           float (&ss)[NS], float (&dq)[NS]) const {
#pragma unroll
    for (int j = 0; j < NS; ++j) partial(j, qh, ql, ss[j], dq[j]);
  }

  // Hides the packed rows from the optimiser between the reduction and the
  // mixture, so it keeps the packed words live rather than unpacked fp32
  // copies.  Emits no instruction.
  __device__ __forceinline__ void keep_packed() {
#pragma unroll
    for (int j = LR; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < SPL; ++i) asm volatile("" : "+v"(x[j][i]));
  }

  // y = sum_j p_j x_j over the raw rows, fp32 accumulation; lane j holds p_j.
  // Sources go in pairs (a, b): one byte permute gathers (x_a[h], x_b[h]) of
  // an element pair's two elements each, and two packed bf16 dot products add
  // p_a x_a[h] + p_b x_b[h] with each weight split into two bf16 values,
  // p = p_hi + p_lo, p_lo = bf16(p - p_hi).  That keeps 16 significant bits
  // of p (relative error at most 2^-17, 2^8 below the output's bf16 rounding),
  // and every product is exact in fp32: 1.5 instructions per element and
  // source instead of an unpack and an FMA.  An odd last source is unpacked
  // and multiplied by the full fp32 weight.
  __device__ __forceinline__ void mix(float p_lane, float (&y)[SPL][8]) const {
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
      for (int k = 0; k < 8; ++k) y[i][k] = 0.f;
    // lane j: (bf16(p_j), bf16(p_j - bf16(p_j))) in one word
    const uint32_t hi = pack_bf16x2(p_lane, 0.f);
    const uint32_t halves = pack_bf16x2(p_lane, p_lane - bf_lo(hi));
#pragma unroll
    for (int a = 0; a + 1 < NS; a += 2) {
      const uint32_t wa = uint32_t(__builtin_amdgcn_readlane(int(halves), a));
      const uint32_t wb = uint32_t(__builtin_amdgcn_readlane(int(halves), a + 1));
      const uint32_t ph = (wa & 0xffffu) | (wb << 16);          // (pa_hi, pb_hi)
      const uint32_t pl = (wa >> 16) | (wb & 0xffff0000u);      // (pa_lo, pb_lo)
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const u32x4 va = row(a, i), vb = row(a + 1, i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // {S0 = x_b, S1 = x_a}: bytes 0-3 are x_a's, 4-7 x_b's
          const uint32_t lo2 = __builtin_amdgcn_perm(vb[k], va[k], 0x05040100u);
          const uint32_t hi2 = __builtin_amdgcn_perm(vb[k], va[k], 0x07060302u);
          y[i][2 * k] = dot2(pl, lo2, dot2(ph, lo2, y[i][2 * k]));
          y[i][2 * k + 1] = dot2(pl, hi2, dot2(ph, hi2, y[i][2 * k + 1]));
        }
      }
    }
    if constexpr (NS % 2 == 1) {
      constexpr int j = NS - 1;
      const float pj = lane_value(p_lane, j);
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const u32x4 v = row(j, i);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          y[i][2 * k] = fmaf(pj, bf_lo(v[k]), y[i][2 * k]);
          y[i][2 * k + 1] = fmaf(pj, bf_hi(v[k]), y[i][2 * k + 1]);
        }
      }
    }
  }

  // y = cur in fp32 (exact): the mixture when cur is the only source, whose
  // softmax weight is exactly 1.
  __device__ __forceinline__ void cur_as_mix(float (&y)[SPL][8]) const {
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[i][2 * k] = bf_lo(x[NB][i][k]);
        y[i][2 * k + 1] = bf_hi(x[NB][i][k]);
      }
  }

  // The in-place writes of cur (prefix with a delta, bank slot widx).  A lane
  // only rewrites elements it has read itself; the writes go out once all of
  // its loads have completed: with out, or right after the last source's
  // partials, whose wait retires every earlier load (after_partials).
  // A row's segment at byte offset b, written.  MASKED: a buffer store whose
  // record is the row, so a segment past the row's end is dropped by the
  // hardware's range check, with no branch (as for the loads).
  template <bool NT>
  __device__ __forceinline__ static void store_row(const KParams &p, uint16_t *row, uint32_t b,
                                                   u32x4 v) {
    if constexpr (kBufferRows) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          row, 0, p.nseg * kSeg * int(sizeof(uint16_t)), kBufferFormat);
      __builtin_amdgcn_raw_buffer_store_b128(v, r, int(b), 0, NT ? kAuxNt : 0);
    } else {
      store_stream<NT>(at(row, b), v);
    }
  }

  __device__ __forceinline__ void store_cur(const KParams &p, int64_t t, int seg0,
                                            int seg_step) const {
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const uint32_t b = seg_bytes(seg0, seg_step, i);
      if constexpr (DELTA)
        store_row<ATTNRES_NT_STORE_CUR>(p, p.prefix + t * p.prefix_stride, b, x[NB][i]);
      if (p.widx >= 0)
        store_row<ATTNRES_NT_STORE_CUR>(p, p.blocks + t * p.tok_stride + p.widx * p.slot_stride,
                                        b, x[NB][i]);
    }
  }

  // The in-place writes of cur (unless CUR_DONE: already issued), then out =
  // bf16_RNE(y * rsig * w) (or y).  Writing cur first was faster everywhere
  // measured (T = 1, nb = 0: 2.70 -> 2.65 us; T = 1024, nb = 8: 32.76 ->
  // 32.63 us; T = 512-768: about 2 %): the rewritten lines are still
  // resident when those rows were read through the cache.
  template <bool CUR_DONE = false>
  __device__ __forceinline__ void store(const KParams &p, int64_t t, int seg0, int seg_step,
                                        const float (&y)[SPL][8], float rsig) const {
    if constexpr (!CUR_DONE) store_cur(p, t, seg0, seg_step);
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      u32x4 o;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if constexpr (ONORM)
          o[k] = pack_bf16x2(y[i][2 * k] * rsig * bf_lo(onw[i][k]),
                             y[i][2 * k + 1] * rsig * bf_hi(onw[i][k]));
        else
          o[k] = pack_bf16x2(y[i][2 * k], y[i][2 * k + 1]);
      }
      store_row<ATTNRES_NT_STORES>(p, p.out + t * p.out_stride, seg_bytes(seg0, seg_step, i), o);
    }
  }
};

template <int SPL>
__device__ __forceinline__ float sum_sq(const float (&y)[SPL][8]) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < SPL; ++i)
#pragma unroll
    for (int k = 0; k < 8; ++k) s = fmaf(y[i][k], y[i][k], s);
  return s;
}

// Softmax over the NS sources, lane j (< NS) holding logit j; lane j of the
// result holds p_j (lanes >= NS hold 0).  The normaliser is computed online:
// each source enters as the pair (m, s) = (l_j, 1), a running maximum and the
// sum of exp(l - m) over the sources it covers, and two pairs merge into
// (max(m1, m2), s1 exp(m1 - max) + s2 exp(m2 - max)); one of the two factors
// is exp(0) = 1, so a merge takes one exponential, exp(-|m1 - m2|), applied
// to the side with the smaller maximum.  Every logit already sits in a lane,
// so the merges run as a tree in a fixed pairwise order (depth
// ceil(log2 NS)) rather than as a chain, and every wave obtains the same
// (m, s).  Then p_j = exp(l_j - m) / s, with s >= 1 (the maximum's own term
// is 1), so the hardware reciprocal serves.  A NaN logit makes s, hence
// every p_j, NaN.
// The online normaliser's state (m, s) of NS logits (lane j holds logit j),
// merged as a fixed-order tree; wave-uniform.
template <int NS>
__device__ __forceinline__ void softmax_state(float logit_lane, float &m_out, float &s_out) {
  float m[NS], s[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    m[j] = lane_value(logit_lane, j);
    s[j] = 1.f;
  }
#pragma unroll
  for (int w = 1; w < NS; w *= 2)
#pragma unroll
    for (int j = 0; j + w < NS; j += 2 * w) {
      const float d = m[j + w] - m[j];
      const float e = __expf(-fabsf(d));
      s[j] = d <= 0.f ? fmaf(s[j + w], e, s[j]) : fmaf(s[j], e, s[j + w]);
      m[j] = fmaxf(m[j], m[j + w]);
    }
  m_out = m[0];
  s_out = s[0];
}

template <int NS>
__device__ __forceinline__ float softmax_lanes(float logit_lane) {
  if constexpr (NS == 1) {
    // A single source: exp(l - l) / exp(l - l), i.e. 1, or NaN for a
    // non-finite logit (l - l is not folded without fast-math).
    return (logit_lane - logit_lane) + 1.f;
  } else {
    const int lane = threadIdx.x & (kWave - 1);
    float m, s;
    softmax_state<NS>(logit_lane, m, s);
    return lane < NS ? __expf(logit_lane - m) * __builtin_amdgcn_rcpf(s) : 0.f;
  }
}

// ---------------------------------------------------------------------------
// row path: one workgroup (7 waves, two segments per lane) per token
// ---------------------------------------------------------------------------

constexpr int kRowRows = kRowWaves * 4;  // 16-lane row partials per workgroup

// Sums N groups of four partials (LDS) in a fixed order: every read is issued
// before the first add (one LDS round trip, not one per few reads), then four
// running sums, one per float4 component, and (x + y) + (z + w).
template <int N>
__device__ __forceinline__ float sum_float4s(const float4 *v4) {
  float4 a[N];
#pragma unroll
  for (int i = 0; i < N; ++i) a[i] = v4[i];
  __builtin_amdgcn_sched_barrier(0);
  float sx = 0.f, sy = 0.f, sz = 0.f, sw = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    sx += a[i].x;
    sy += a[i].y;
    sz += a[i].z;
    sw += a[i].w;
  }
  return (sx + sy) + (sz + sw);
}


// Sums the kRowRows row partials of one value in a fixed order.
__device__ __forceinline__ float sum_row_partials(const float *v) {
  return sum_float4s<kRowRows / 4>(reinterpret_cast<const float4 *>(v));
}

// Sum of n (<= 64) row partials, one per lane, over the wave in a fixed order
// (DPP), returned in every lane: one LDS read per lane instead of a lane
// summing all n.
__device__ __forceinline__ float wave_sum_of_partials(const float *v, int n) {
  const int lane = threadIdx.x & (kWave - 1);
  const float x = lane < n ? v[lane] : 0.f;
  return lane_value(wave_sum_lane63(x), kWave - 1);
}

// The grid either has one workgroup per token or is persistent (a few
// workgroups per CU looping over tokens); LDS partials are double-buffered by
// iteration parity so one barrier per phase suffices.
// RANGED: rows and weights are read with range-checked (buffer) loads, the
// form the masked kernels use, here over whole rows (nothing is cut off).
// Small calls take it (kRowRangedMaxT): the compiler then issues the
// weights' loads (L2 hits) ahead of the rows, where with plain loads it
// interleaves them with prefix and delta and the fused query waits on an HBM
// load.  With about one token per CU that wait is not hidden.
template <int NB, bool DELTA, bool ONORM, bool CACHE_RW = false, bool RANGED = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(kRowThreads, kRowThreads),
                               // the unified arch+acc register file counts double
                               amdgpu_num_vgpr(ATTNRES_ROW_MAX_VGPRS / 2)))
attnres_row_kernel(KParams p) {
  constexpr int NS = NB + 1;
  constexpr int SPL = kRowSegsPerLane;
  static_assert(!(RANGED && CACHE_RW), "the ranged form reads every row streaming");
  // cur's in-place writes as soon as every load has landed, in the variant
  // that read those rows through the cache (calls of T * H >= 1024 * 7168):
  // there T = 1024 with 4 or 8 bank rows measured 1.2-1.8 % faster, T =
  // 2048-4096 within 0.4 %.  Smaller calls, whose rows stream past the cache,
  // measured slower (T = 256 +6 %), and so did the any-H kernel's forms.
  constexpr bool kEarlyCur = ATTNRES_EARLY_CUR_STORE && CACHE_RW;
  __shared__ __align__(16) float s_part[2][2 * NS][kRowRows];
  __shared__ __align__(16) float s_ysq[2][kRowRows];

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rowslot = wave * 4 + (lane >> 4);  // this lane's 16-lane row in the workgroup
  const bool row_leader = (lane & 15) == 0;

  // One token per workgroup unless the grid is persistent (row_wgs_per_cu);
  // only then is the loop compiled, since the weights it hoists cost
  // registers.
  constexpr bool kLoop = row_wgs_per_cu(NB) > 0;
  const int64_t t_step = kLoop ? int64_t(gridDim.x) : p.T;
  int par = 0;
  // Segment i of a lane is lane + i * 448, so that each load instruction of a
  // wave covers 1 KB of one row, whole cache lines.  (Adjacent segments per
  // lane would save address registers but cover half lines per instruction,
  // which measured 30% slower.)
  const int seg0 = int(threadIdx.x);
  const int seg_step = kRowThreads;
  if constexpr (NB == 0 && kLoop && ONORM) {
    // One source with an output norm, looping over tokens: the next token's
    // rows are issued before this token's arithmetic and stores, so that its
    // loads wait neither behind this token's stores (one in-order counter)
    // nor idle across the norm's barrier.  The rows are range-checked
    // (buffer) loads, so that past the last token the next-token loads get
    // an empty range and read nothing.  Measured against the loop below,
    // bit-identical (us per call, without / with delta): T = 1 2.45 -> 2.23,
    // 2.65 -> 2.56; T = 16 2.70 -> 2.49, 2.94 -> 2.84; T = 256 3.24 -> 3.06,
    // 4.09 -> 3.98; T = 1024 7.21 -> 6.93, 11.27 -> 11.44; T = 2048 12.31 ->
    // 11.67, 21.27 -> 20.96; T = 8192 43.1 -> 42.3, 81.8 -> 81.9.  Without a
    // norm it measured no better.
    using Tk = Token<NB, DELTA, ONORM, SPL, true, CACHE_RW>;
    int64_t t = blockIdx.x;
    if (t >= p.T) return;
    Tk a;
    a.issue(p, t, seg0, seg_step);
    for (;; par ^= 1) {
      const int64_t tn = t + t_step;
      KParams pn = p;
      pn.nseg = tn < p.T ? p.nseg : 0;
      Tk b;
      b.issue(pn, tn < p.T ? tn : t, seg0, seg_step);
      a.finish_cur();
      a.issue_onw(p, seg0, seg_step);
      float y[SPL][8];
      a.cur_as_mix(y);
      const float sy = row16_sum(sum_sq<SPL>(y));
      if (row_leader) s_ysq[par][rowslot] = sy;
      __syncthreads();
      const float rsig =
          rsqrtf(wave_sum_of_partials(s_ysq[par], kRowRows) * kInvHidden + p.out_eps);
      a.store(p, t, seg0, seg_step, y, rsig);
      if (tn >= p.T) break;
      t = tn;
      a = b;
    }
    return;
  }
  for (int64_t t = blockIdx.x; t < p.T; t += t_step, par ^= 1) {
    Token<NB, DELTA, ONORM, SPL, RANGED, CACHE_RW> tk;
    tk.issue(p, t, seg0, seg_step);
    if constexpr (NB == 0) {
      // One source, weight exactly 1: y = cur, no logit, and the output
      // norm's sum of squares is cur's (one reduction, none without a norm).
      tk.finish_cur();
      tk.issue_onw(p, seg0, seg_step);
      float y[SPL][8];
      tk.cur_as_mix(y);
      float rsig = 1.f;
      if constexpr (ONORM) {
        const float sy = row16_sum(sum_sq<SPL>(y));
        if (row_leader) s_ysq[par][rowslot] = sy;
        __syncthreads();
        rsig = rsqrtf(wave_sum_of_partials(s_ysq[par], kRowRows) * kInvHidden + p.out_eps);
      }
      tk.store(p, t, seg0, seg_step, y, rsig);
      continue;
    }
    u32x4 qh[SPL], ql[SPL];
    tk.query(qh, ql);

    // Each source's partials as soon as its rows land (loads retire in issue
    // order), reduced within 16-lane rows and parked in LDS, so that this
    // work overlaps the later rows' arrival.  cur (prefix + delta) comes in
    // the order its rows were issued: first by default.
#pragma unroll
    for (int jj = 0; jj < NS; ++jj) {
      const int j = decltype(tk)::kCurFirst ? (jj == 0 ? NB : jj - 1) : jj;
      if (j == NB) tk.finish_cur();
      float sj, dj;
      tk.partial(j, qh, ql, sj, dj);
      sj = row16_sum(sj);
      dj = row16_sum(dj);
      if (row_leader) {
        s_part[par][j][rowslot] = sj;
        s_part[par][NS + j][rowslot] = dj;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    tk.keep_packed();
    tk.template after_partials<kEarlyCur>(p, t, seg0, seg_step);

    // Lane j < NS sums source j's squares and lane 32 + j its query dots;
    // lane j then takes the dot from lane 32 + j.
    float tot = 0.f;
    if ((lane & 31) < NS) tot = sum_row_partials(s_part[par][(lane & 31) + (lane >> 5) * NS]);
    const float dq_j = lane_shuffle(tot, (lane + 32) & (kWave - 1));
    const float logit = lane < NS ? dq_j * rsqrtf(tot * kInvHidden + p.rms_eps) : 0.f;
    const float p_lane = softmax_lanes<NS>(logit);
    float y[SPL][8];
    tk.keep_packed();
    tk.mix(p_lane, y);

    float rsig = 1.f;
    if constexpr (ONORM) {
      const float sy = row16_sum(sum_sq<SPL>(y));
      if (row_leader) s_ysq[par][rowslot] = sy;
      __syncthreads();
      rsig = rsqrtf(wave_sum_of_partials(s_ysq[par], kRowRows) * kInvHidden + p.out_eps);
    }
    tk.template store<kEarlyCur>(p, t, seg0, seg_step, y, rsig);
  }
}

// ---------------------------------------------------------------------------
// any-H row path: one workgroup (1-8 waves) per token, runtime row length
// ---------------------------------------------------------------------------

constexpr int kAnyMaxThreads = 512;               // 8 waves
constexpr int kAnyMaxRows = kAnyMaxThreads / 16;  // 16-lane row partials per workgroup

// Sums the first n4 (<= kAnyMaxRows / 4) groups of four row partials in a
// fixed order.  All kAnyMaxRows / 4 groups of the row are read at once (the
// row always holds that many, so the reads stay in bounds) and the groups
// past n4 count as zero.
// CHUNK: float4 reads issued together (fewer hold fewer registers while the
// rows are live; the sum is the same).
template <int CHUNK = kAnyMaxRows / 4>
__device__ __forceinline__ float sum_row_partials_n(const float *v, int n4) {
  constexpr int kMax4 = kAnyMaxRows / 4;
  static_assert(kMax4 % CHUNK == 0, "whole chunks");
  const float4 *v4 = reinterpret_cast<const float4 *>(v);
  float sx = 0.f, sy = 0.f, sz = 0.f, sw = 0.f;
#pragma unroll
  for (int c = 0; c < kMax4; c += CHUNK) {
    float4 a[CHUNK];
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) a[i] = v4[c + i];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < CHUNK; ++i) {
      if (c + i < n4) {
        sx += a[i].x;
        sy += a[i].y;
        sz += a[i].z;
        sw += a[i].w;
      }
    }
  }
  return (sx + sy) + (sz + sw);
}

// The row path's steps for a runtime row of p.nseg segments: blockDim.x lanes
// (whole waves, at most kAnyMaxThreads) with SPL segments each, blockDim.x *
// SPL >= p.nseg.  With two segments per lane a token fits 128 VGPRs (four
// waves per SIMD); four segments may take 256.
//
// LR > 0 (kAnyLdsRows bank rows staged in LDS, launched with LR * SPL *
// blockDim.x * 16 bytes of dynamic LDS): the same steps with those rows held
// in LDS instead of registers, for one more resident workgroup per CU where
// the registers are what limits it (see anyh_lds_rows).  Register budgets
// for that: four segments per lane, 168 VGPRs (two workgroups of 5-6 waves);
// two segments, 96 for four 5-wave workgroups, or with W6 80 for four 6-wave
// ones (six waves per SIMD).
template <int SPL, bool MASKED, int NB, bool DELTA, bool ONORM, bool CACHE_RW = false, int LR = 0,
          bool W6 = false>
__global__ void __attribute__((amdgpu_flat_work_group_size(kWave, kAnyMaxThreads),
                               amdgpu_waves_per_eu(LR == 0 ? (SPL <= 2 ? 4 : 2)
                                                           : (SPL <= 2 ? (W6 ? 6 : 5) : 3))))
attnres_anyh_kernel(KParams p) {
  constexpr int NS = NB + 1;
  constexpr bool STG = LR > 0;
  __shared__ __align__(16) float s_part[2 * NS][kAnyMaxRows];
  __shared__ __align__(16) float s_ysq[kAnyMaxRows];
  extern __shared__ __align__(16) u32x4 s_rows[];

  const int nthreads = p.threads;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rowslot = wave * 4 + (lane >> 4);
  const bool row_leader = (lane & 15) == 0;
  const int n4 = nthreads / kWave;  // four row partials per wave
  const int64_t t = blockIdx.x;
  const int seg0 = int(threadIdx.x);  // whole-line loads, as in the row kernel
  const int seg_step = nthreads;

  Token<NB, DELTA, ONORM, SPL, MASKED, CACHE_RW, true, (NB > 0), LR> tk;
  tk.lds_rows = s_rows;
  tk.nthr = p.threads;
  tk.issue(p, t, seg0, seg_step);
  if constexpr (NB == 0) {
    // One source, weight exactly 1 (as in the row kernel).
    tk.finish_cur();
    tk.issue_onw(p, seg0, seg_step);
    float y[SPL][8];
    tk.cur_as_mix(y);
    float rsig = 1.f;
    if constexpr (ONORM) {
      const float sy = row16_sum(sum_sq<SPL>(y));
      if (row_leader) s_ysq[rowslot] = sy;
      __syncthreads();
      rsig = rsqrtf(wave_sum_of_partials(s_ysq, 4 * n4) * p.inv_h + p.out_eps);
    }
    tk.store(p, t, seg0, seg_step, y, rsig);
    return;
  }
  u32x4 qh[SPL], ql[SPL];
  tk.query(qh, ql);

  // Each source's partials as its rows land, in issue order as in the row
  // kernel.  STG: cur, then bank rows in order; a staged row goes to LDS
  // right after its partials, and each step releases the next loads
  // (issue_rest).
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int src = decltype(tk)::kCurFirst ? (j == 0 ? NB : j - 1) : j;
    if (src == NB) tk.finish_cur();
    float sj, dj;
    if (STG && src < LR)
      tk.template partial<true>(src, qh, ql, sj, dj);
    else
      tk.partial(src, qh, ql, sj, dj);
    sj = row16_sum(sj);
    dj = row16_sum(dj);
    if (row_leader) {
      s_part[src][rowslot] = sj;
      s_part[NS + src][rowslot] = dj;
    }
    if constexpr (STG) {
      static_assert(!STG || LR == 3, "the release points below are for three staged rows");
      constexpr int F = decltype(tk)::kFirst;
      if (src == NB) tk.template issue_rest<F, F + 1>(p, t, seg0, seg_step);
      if (src < LR) tk.stage(src);
      if (src == 0) tk.template issue_rest<F + 1, F + 2>(p, t, seg0, seg_step);
      if (src == 1) tk.template issue_rest<F + 2, F + 3>(p, t, seg0, seg_step);
      if (src == 2) tk.template issue_rest<F + 3, NB>(p, t, seg0, seg_step);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  tk.keep_packed();
  // STG: the output-norm weight after the mixture (registers are tightest
  // while the mixture runs), overlapping the norm's reduction.
  tk.template after_partials<false, !STG>(p, t, seg0, seg_step);

  // Lane j < NS sums source j's squares, lane 32 + j its query dots.
  float tot = 0.f;
  if ((lane & 31) < NS)
    tot = sum_row_partials_n<LR == 0 ? kAnyMaxRows / 4 : kAnyMaxRows / 16>(
        s_part[(lane & 31) + (lane >> 5) * NS], n4);
  const float dq_j = lane_shuffle(tot, (lane + 32) & (kWave - 1));
  const float logit = lane < NS ? dq_j * rsqrtf(tot * p.inv_h + p.rms_eps) : 0.f;
  const float p_lane = softmax_lanes<NS>(logit);
  float y[SPL][8];
  tk.keep_packed();
  tk.mix(p_lane, y);
  if constexpr (STG) tk.issue_onw(p, seg0, seg_step);

  float rsig = 1.f;
  if constexpr (ONORM) {
    const float sy = row16_sum(sum_sq<SPL>(y));
    if (row_leader) s_ysq[rowslot] = sy;
    __syncthreads();
    rsig = rsqrtf(wave_sum_of_partials(s_ysq, 4 * n4) * p.inv_h + p.out_eps);
  }
  tk.store(p, t, seg0, seg_step, y, rsig);
}

// ---------------------------------------------------------------------------
// two-kernel form: the bank part (independent of delta), then the cur part
// ---------------------------------------------------------------------------
//
// The bank part of token t leaves in p.partial: u_t = sum_{j < nb} exp(l_j -
// m_t) x_j, fp32, H elements at p.partial + t H; then, after all T rows, the
// online normaliser's state (m_t, s_t) of the bank logits l_j (two floats at
// p.partial + T H + 2 t).  The cur part merges cur's logit l_c into that
// state, as one more step of the online softmax: M = max(m_t, l_c),
// S = s_t exp(m_t - M) + exp(l_c - M), y = (u_t exp(m_t - M) + cur
// exp(l_c - M)) / S; then the output norm and every store.  Both run in the
// any-H kernel's launch shape, one workgroup per token.

template <int SPL, bool MASKED, int NB>
__global__ void __attribute__((amdgpu_flat_work_group_size(kWave, kAnyMaxThreads),
                               amdgpu_waves_per_eu(SPL <= 2 ? 4 : 2)))
attnres_bank_kernel(KParams p) {
  static_assert(NB > 0, "the bank part needs bank rows");
  __shared__ __align__(16) float s_part[2 * NB][kAnyMaxRows];

  const int nthreads = p.threads;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rowslot = wave * 4 + (lane >> 4);
  const bool row_leader = (lane & 15) == 0;
  const int n4 = nthreads / kWave;
  const int64_t t = blockIdx.x;
  const int seg0 = int(threadIdx.x);
  const int seg_step = nthreads;

  Token<NB, false, false, SPL, MASKED, false, /*CUR=*/false> tk;
  tk.issue(p, t, seg0, seg_step);
  u32x4 qh[SPL], ql[SPL];
  tk.query(qh, ql);
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    float sj, dj;
    tk.partial(j, qh, ql, sj, dj);
    sj = row16_sum(sj);
    dj = row16_sum(dj);
    if (row_leader) {
      s_part[j][rowslot] = sj;
      s_part[NB + j][rowslot] = dj;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  tk.keep_packed();
  __syncthreads();

  float tot = 0.f;
  if ((lane & 31) < NB) tot = sum_row_partials_n(s_part[(lane & 31) + (lane >> 5) * NB], n4);
  const float dq_j = lane_shuffle(tot, (lane + 32) & (kWave - 1));
  const float logit = lane < NB ? dq_j * rsqrtf(tot * p.inv_h + p.rms_eps) : 0.f;
  float m, sum;
  softmax_state<NB>(logit, m, sum);
  const float w_lane = lane < NB ? __expf(logit - m) : 0.f;
  float u[SPL][8];
  tk.keep_packed();
  tk.mix(w_lane, u);

  const int64_t H = int64_t(p.nseg) * kSeg;
  float *urow = p.partial + t * H;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int seg = seg0 + i * seg_step;
    if (MASKED && seg >= p.nseg) continue;
    f32x4 *dst = reinterpret_cast<f32x4 *>(urow + int64_t(seg) * kSeg);
    dst[0] = f32x4{u[i][0], u[i][1], u[i][2], u[i][3]};
    dst[1] = f32x4{u[i][4], u[i][5], u[i][6], u[i][7]};
  }
  if (threadIdx.x == 0) {
    float *st = p.partial + int64_t(p.T) * H + 2 * t;
    st[0] = m;
    st[1] = sum;
  }
}

template <int SPL, bool MASKED, bool DELTA, bool ONORM, bool BANK>
__global__ void __attribute__((amdgpu_flat_work_group_size(kWave, kAnyMaxThreads),
                               amdgpu_waves_per_eu(SPL <= 2 ? 4 : 2)))
attnres_cur_kernel(KParams p) {
  __shared__ __align__(16) float s_part[2][kAnyMaxRows];
  __shared__ __align__(16) float s_ysq[kAnyMaxRows];

  const int nthreads = p.threads;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int rowslot = wave * 4 + (lane >> 4);
  const bool row_leader = (lane & 15) == 0;
  const int n4 = nthreads / kWave;
  const int64_t t = blockIdx.x;
  const int seg0 = int(threadIdx.x);
  const int seg_step = nthreads;
  const int64_t H = int64_t(p.nseg) * kSeg;

  // cur is the only row this part reads from the bank side; the bank's
  // contribution arrives as the partial state.
  Token<0, DELTA, ONORM, SPL, MASKED, false, true, /*Q=*/BANK> tk;
  tk.issue(p, t, seg0, seg_step);
  f32x4 u[SPL][2];
  float m_b = 0.f, s_b = 0.f;
  if constexpr (BANK) {
    const float *urow = p.partial + t * H;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int seg = seg0 + i * seg_step;
      const bool ok = !MASKED || seg < p.nseg;
      const f32x4 *src = reinterpret_cast<const f32x4 *>(urow + int64_t(seg) * kSeg);
      u[i][0] = ok ? src[0] : zero;
      u[i][1] = ok ? src[1] : zero;
    }
    const float *st = p.partial + int64_t(p.T) * H + 2 * t;
    m_b = st[0];
    s_b = st[1];
  }
  float y[SPL][8];
  if constexpr (BANK) {
    u32x4 qh[SPL], ql[SPL];
    tk.query(qh, ql);
    tk.finish_cur();
    float sc, dc;
    tk.partial(0, qh, ql, sc, dc);
    sc = row16_sum(sc);
    dc = row16_sum(dc);
    if (row_leader) {
      s_part[0][rowslot] = sc;
      s_part[1][rowslot] = dc;
    }
    __syncthreads();
    tk.issue_onw(p, seg0, seg_step);
    float tot = 0.f;
    if ((lane & 31) == 0) tot = sum_row_partials_n(s_part[lane >> 5], n4);
    const float lc = lane_value(tot, 32) * rsqrtf(lane_value(tot, 0) * p.inv_h + p.rms_eps);
    // One more step of the online softmax: (m_b, s_b) merged with (lc, 1).
    // One of the two factors is exp(0) = 1, so the normaliser is >= 1.
    const float mx = fmaxf(m_b, lc);
    const float fa = __expf(m_b - mx), fc = __expf(lc - mx);
    const float inv = __builtin_amdgcn_rcpf(fmaf(s_b, fa, fc));
    const float ca = fa * inv, cc = fc * inv;
#pragma unroll
    for (int i = 0; i < SPL; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float u0 = u[i][k >> 1][(k & 1) * 2], u1 = u[i][k >> 1][(k & 1) * 2 + 1];
        y[i][2 * k] = fmaf(ca, u0, cc * bf_lo(tk.x[0][i][k]));
        y[i][2 * k + 1] = fmaf(ca, u1, cc * bf_hi(tk.x[0][i][k]));
      }
  } else {
    // No bank rows: cur alone, weight exactly 1.
    tk.finish_cur();
    tk.issue_onw(p, seg0, seg_step);
    tk.cur_as_mix(y);
  }
  float rsig = 1.f;
  if constexpr (ONORM) {
    const float sy = row16_sum(sum_sq<SPL>(y));
    if (row_leader) s_ysq[rowslot] = sy;
    __syncthreads();
    rsig = rsqrtf(wave_sum_of_partials(s_ysq, 4 * n4) * p.inv_h + p.out_eps);
  }
  tk.store(p, t, seg0, seg_step, y, rsig);
}

// Launch shape of the any-H kernel for a row of nseg segments.
struct AnyShape {
  int spl;
  int threads;
  bool masked;
};
AnyShape anyh_shape(int64_t H) {
  const int nseg = int(H / kSeg);
  const int spl = nseg <= 2 * kAnyMaxThreads ? 2 : 4;
  const int reach = kWave * spl;  // segments one wave covers
  const int waves = (nseg + reach - 1) / reach;
  return {spl, waves * kWave, nseg % reach != 0};
}
static_assert(4 * kAnyMaxThreads * kSeg >= kMaxHidden, "any-H kernel must reach the largest H");
static_assert(3 * kParts * kPartThreads * kSeg >= kMaxHidden,
              "three segments per lane of the split path must reach the largest H");

// ---------------------------------------------------------------------------
// split path: kParts single-wave workgroups per token
// ---------------------------------------------------------------------------

// The kParts workgroups of a token are placed on one XCD (see the kernel),
// but nothing in the launch guarantees that placement, and the L2 caches of
// different XCDs are not coherent with each other.  So every exchanged value
// is a self-validating 64-bit word, (generation << 32) | float bits, written
// and read with single device-coherent (agent-scope atomic) accesses, which
// bypass the non-coherent L2: no L2 writeback or invalidate, no counter, and
// a reader needs one round trip once the words are there.  (A load with only
// the workgroup-scope bit would be served from the reading CU's own L1 and
// never see a partner's store.)  A part's generation for this
// call is one past the later of its own word 0's generations in the two
// frames below: every call rewrites word 0 of all kParts parts of a token
// with the same generation, in one frame or the other, so the parts agree
// without communicating (the workspace starts at zero).  Waits are bounded; a
// wait that gives up raises the device flag.
__device__ __forceinline__ uint64_t tagged_load(const uint64_t *w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void tagged_store(uint64_t *w, float v, uint32_t gen) {
  __hip_atomic_store(w, (uint64_t(gen) << 32) | __float_as_uint(v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t tag_of(uint64_t w) { return uint32_t(w >> 32); }
__device__ __forceinline__ float value_of(uint64_t w) { return __uint_as_float(uint32_t(w)); }

// The later of two generations (they count calls, modulo 2^32).
__device__ __forceinline__ uint32_t later_gen(uint32_t a, uint32_t b) {
  return int32_t(a - b) > 0 ? a : b;
}

// Two memory frames hold a copy each of the split path's words.  A device-
// scope store is acknowledged about twice as fast when its 2 MB frame is homed
// on the writing XCD's half of the chip (about 220 against 460 ns on MI355X),
// and a part's first poll waits for its own store's acknowledgement (loads and
// stores retire in order); a poll of the far frame costs a far round trip too.
// So a part writes its words to the frame that the host found nearer its XCD
// and polls that frame, where a token's parts (all on one XCD) put theirs;
// after kNearPolls polls it reads both frames.  Where the parts of a token run
// decides only speed, never what is read.
constexpr int kNearPolls = 16;
__device__ __forceinline__ unsigned hw_xcc_id() {
  return __builtin_amdgcn_s_getreg(20 | (3 << 11)) & 7u;  // HW_REG_XCC_ID, 4 bits
}

// Sums word `idx` over the kParts parts (fixed order), once every part has
// written it with generation `gen` into either frame (the near one is polled
// first); after `spin_limit` polls it gives up and raises the device flag
// (the sum is then not valid).
__device__ __forceinline__ float gather(const uint64_t *tok_near, const uint64_t *tok_far,
                                        int idx, uint32_t gen, unsigned *flag, int spin_limit) {
  uint64_t w[kParts];
  for (int spins = 0;; ++spins) {
    bool ready = true;
#pragma unroll
    for (int r = 0; r < kParts; ++r) w[r] = tagged_load(tok_near + r * kSlot + idx);
    if (spins >= kNearPolls) {
      uint64_t wf[kParts];
#pragma unroll
      for (int r = 0; r < kParts; ++r) wf[r] = tagged_load(tok_far + r * kSlot + idx);
#pragma unroll
      for (int r = 0; r < kParts; ++r) w[r] = tag_of(w[r]) == gen ? w[r] : wf[r];
    }
#pragma unroll
    for (int r = 0; r < kParts; ++r) ready = ready && tag_of(w[r]) == gen;
    if (ready) break;
    if (spins >= spin_limit) {
      __hip_atomic_store(flag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(ATTNRES_SPIN_SLEEP);
  }
  // Two interleaved running sums (even and odd parts), then their sum.
  static_assert(kParts % 2 == 0, "parts are summed in pairs");
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int r = 0; r < kParts; r += 2) {
    s0 += value_of(w[r]);
    s1 += value_of(w[r + 1]);
  }
  return s0 + s1;
}

// Row j of the upper-triangular pair list (j <= k, row-major) starts here.
__host__ __device__ constexpr int pair_row_start(int ns, int j) { return j * ns - j * (j - 1) / 2; }

// The values one part publishes.  With an output norm: the Gram matrix of the
// sources over this part's elements, G_jk = sum x_j x_k for j <= k (its
// diagonal is the sum of squares), followed by the query dots; the output
// norm's sum of squares then follows from ||y||^2 = sum_jk p_j p_k G_jk with
// no second exchange.  Without one: the sums of squares, then the query dots.
template <int NS, bool ONORM>
struct SplitWords {
  static constexpr int kPairs = NS * (NS + 1) / 2;
  static constexpr int kCount = ONORM ? kPairs + NS : 2 * NS;
  static constexpr int kDot = ONORM ? kPairs : NS;  // first query-dot word
  __device__ static constexpr int ss_word(int j) { return ONORM ? pair_row_start(NS, j) : j; }
};

// ||y||^2 is taken from the Gram matrix only when it is not much smaller than
// its triangle-inequality bound (sum_j p_j ||x_j||)^2; below this fraction the
// sources cancel, the Gram form loses relative accuracy, and the sum of
// squares of y is exchanged directly instead.
constexpr float kGramGuard = 1.f / 16.f;

// The mixture weights from a token's exchanged totals (lane v < NV holds word
// v): lane j < NS returns p_j; ss_j receives lane j's sum of squares.
template <int NS, bool ONORM>
__device__ __forceinline__ float weights_from_totals(float total, float rms_eps, float inv_h,
                                                    float &ss_j) {
  using Words = SplitWords<NS, ONORM>;
  const int lane = threadIdx.x & (kWave - 1);
  const int jl = lane < NS ? lane : 0;
  ss_j = lane_shuffle(total, Words::ss_word(jl));
  const float dq_j = lane_shuffle(total, Words::kDot + jl);
  const float logit = lane < NS ? dq_j * rsqrtf(ss_j * inv_h + rms_eps) : 0.f;
  return softmax_lanes<NS>(logit);
}

// ||y||^2 = sum_jk c_jk p_j p_k G_jk from the Gram words of the totals (c = 1
// on the diagonal, 2 off it), and its guard bound b = sum_j p_j ||x_j||; both
// wave-uniform.  The Gram form is used only when ysq >= kGramGuard * b^2.
template <int NS>
__device__ __forceinline__ void gram_ysq(float total, float p_lane, float ss_j, float &ysq,
                                         float &b) {
  using Words = SplitWords<NS, true>;
  const int lane = threadIdx.x & (kWave - 1);
  // Lane w < kPairs holds G_jk for the w-th pair (j <= k).
  int j = 0, rem = lane;
#pragma unroll
  for (int r = 0; r < NS; ++r)
    if (rem >= NS - j && j < NS - 1) {
      rem -= NS - j;
      ++j;
    }
  const int k = j + rem;
  const float pj = lane_shuffle(p_lane, j);
  const float pk = lane_shuffle(p_lane, k < NS ? k : 0);
  const float term = lane < Words::kPairs ? (j == k ? 1.f : 2.f) * pj * pk * total : 0.f;
  const float bound = lane < NS ? p_lane * sqrtf(fmaxf(ss_j, 0.f)) : 0.f;
  ysq = lane_value(wave_sum_lane63(term), kWave - 1);
  b = lane_value(wave_sum_lane63(bound), kWave - 1);
}

template <int NB, bool DELTA, bool ONORM, int SPL = 1, bool MASKED = false>
__global__ void __launch_bounds__(kPartThreads) attnres_split_kernel(KParams p) {
  constexpr int NS = NB + 1;
  using Words = SplitWords<NS, ONORM>;
  constexpr int NV = Words::kCount;
  constexpr int kTrStride = kWave + 4;  // padded: conflict-free 128-bit reads
  static_assert(NV <= kSlotYsq, "workspace slot too small");
  __shared__ __align__(16) float s_tr[NV][kTrStride];

  // The dispatcher hands workgroup b to XCD b mod 8.  Token t's parts are
  // workgroups 8 (kParts floor(t / 8) + part) + t mod 8, all on XCD t mod 8,
  // so the exchanged words stay within one XCD's memory path (10 % off a
  // single-token call).  Correctness does not rest on this placement: the
  // exchange is agent-scope.  Workgroups past the last token exit at once.
  const unsigned xcd = blockIdx.x & 7u, local = blockIdx.x >> 3;
  const unsigned group = local / kParts;
  const int part = int(local - group * kParts);
  const int64_t t = int64_t(group) * 8 + xcd;
  if (t >= p.T) return;
  const int lane = threadIdx.x;
  // Part `part` owns SPL segments per lane, part * 64 * SPL + lane + 64 i; at
  // H = 7168, one (512 elements per part).
  const int seg0 = part * kPartThreads * SPL + lane;
  constexpr int seg_step = kPartThreads;
  const float inv_h = SPL == 1 && !MASKED ? kInvHidden : p.inv_h;
  // The token's words in frames A and B; this part writes `slot`, in the
  // frame nearer its XCD, and reads both.  Its own word 0 holds the last
  // call's generation in one of the two frames.
  uint64_t *const tok_a = p.ws_part + size_t(t) * kParts * kSlot;
  uint64_t *const tok_b = p.ws_part_b + size_t(t) * kParts * kSlot;
  const unsigned near_b = (p.ws_near >> (p.ws_by_part ? unsigned(part) : hw_xcc_id())) & 1u;
  uint64_t *const tok_near = near_b ? tok_b : tok_a;
  uint64_t *const tok_far = near_b ? tok_a : tok_b;
  uint64_t *const slot = tok_near + part * kSlot;

  if constexpr (NB == 0) {
    // One source, weight exactly 1: y = cur.  Only an output norm needs the
    // token's sum of squares; the parts exchange it through word 0 alone
    // (so every such call still rewrites word 0 of all parts).  Without a
    // norm nothing is exchanged.
    uint32_t gen0 = 0;
    if constexpr (ONORM)
      gen0 = later_gen(tag_of(tagged_load(tok_a + part * kSlot)),
                       tag_of(tagged_load(tok_b + part * kSlot))) + 1u;
    Token<NB, DELTA, ONORM, SPL, MASKED> tk;
    tk.issue(p, t, seg0, seg_step);
    tk.finish_cur();
    tk.issue_onw(p, seg0, seg_step);
    float y[SPL][8];
    tk.cur_as_mix(y);
    float rsig = 1.f;
    if constexpr (ONORM) {
      const float s = wave_sum_lane63(sum_sq<SPL>(y));
      if (lane == kWave - 1) tagged_store(slot, s, gen0);
      float total = 0.f;
      if (lane == 0)
        total = gather(tok_near, tok_far, 0, gen0 + p.wait_skew, p.ws_flag, p.spin_limit);
      rsig = rsqrtf(lane_value(total, 0) * inv_h + p.out_eps);
    }
    tk.store(p, t, seg0, seg_step, y, rsig);
    return;
  }

  // This call's generation (issued first; used only when publishing).
  const uint32_t gen = later_gen(tag_of(tagged_load(tok_a + part * kSlot)),
                                 tag_of(tagged_load(tok_b + part * kSlot))) + 1u;

  Token<NB, DELTA, ONORM, SPL, MASKED> tk;
  tk.issue(p, t, seg0, seg_step);
  u32x4 qh[SPL], ql[SPL];
  tk.query(qh, ql);
  tk.finish_cur();

  // Per-lane values summed over the wave, then published with one store of
  // tagged words (lane v holds word v).  A few words are summed with DPP
  // wave reductions (independent chains); more are transposed through LDS so
  // that lane v sums value v over the wave; the most (an output norm's Gram
  // matrix at nb >= 6) come from one matrix-core product.  Measured at T = 1
  // with an output norm, transposition / product: nb = 4 3.78 / 3.91 us,
  // nb = 5 3.97 / 4.03, nb = 6 4.12 / 4.09; earlier, nb = 7 4.84 / 4.79 and
  // nb = 8 5.07 / 4.89.
  if constexpr (NV <= ATTNRES_SPLIT_DPP_WORDS) {
    float ss[NS], dq[NS], val[NV];
    tk.partials(qh, ql, ss, dq);
    if constexpr (ONORM) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        val[pair_row_start(NS, j)] = ss[j];
#pragma unroll
        for (int k = j + 1; k < NS; ++k) {
          float g = 0.f;
#pragma unroll
          for (int i = 0; i < SPL; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) g = dot2(tk.x[j][i][w], tk.x[k][i][w], g);
          val[pair_row_start(NS, j) + (k - j)] = g;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) val[j] = ss[j];
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) val[Words::kDot + j] = dq[j];
    float word = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      const float sum = lane_value(wave_sum_lane63(val[v]), kWave - 1);
      word = lane == v ? sum : word;
    }
    tk.keep_packed();
    if (lane < NV) tagged_store(slot + lane, word, gen);
  } else if constexpr (NV >= ATTNRES_SPLIT_MFMA_WORDS) {
    // X: the part's rows over its 512 elements -- the NS sources, then q_hi
    // and q_lo -- so that G = X X^T holds every sum this part publishes: the
    // Gram matrix of the sources (sums of squares on its diagonal) and, in
    // rows NS and NS + 1, the two halves of the query dots.  Each lane parks
    // its 16-byte segment of every row in LDS.  16 matrix-core steps of 32
    // elements (v_mfma_f32_16x16x32_bf16, one register as both A and B) then
    // read X in the operand layout, lane l supplying row l % 16 and elements
    // 32 c + 8 (l / 16) .. + 8 of step c (rows from NR on are zero), and lane
    // l ends with G[4 (l / 16) + i][l % 16] in accumulator element i.  The
    // products of bf16 values are exact in fp32, as in the dot products.
    constexpr int NR = NS + 2;
    static_assert(NR <= 16, "the rows of one 16 x 16 product");
    constexpr int kSteps = kPartThreads * SPL * kSeg / 32;
    constexpr int kXStride = kPartThreads * SPL * kSeg + kSeg;  // +16 B: conflict-free 128-bit accesses
    __shared__ __align__(16) uint16_t s_x[NR][kXStride];
    __shared__ __align__(16) float s_g[16][17];
    // (segments past a masked row's end hold zeros and add nothing)
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int e = (i * kPartThreads + lane) * kSeg;
#pragma unroll
      for (int j = 0; j < NS; ++j) *reinterpret_cast<u32x4 *>(&s_x[j][e]) = tk.x[j][i];
      *reinterpret_cast<u32x4 *>(&s_x[NS][e]) = qh[i];
      *reinterpret_cast<u32x4 *>(&s_x[NS + 1][e]) = ql[i];
    }
    tk.keep_packed();
    __syncthreads();
    const int r = lane & 15, kb = lane >> 4;
    const int rr = r < NR ? r : 0;  // rows from NR on read row 0, then count as zero
    const u32x4 zero = {0u, 0u, 0u, 0u};
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kSteps; c += 2) {
      u32x4 w0 = *reinterpret_cast<const u32x4 *>(&s_x[rr][32 * c + 8 * kb]);
      u32x4 w1 = *reinterpret_cast<const u32x4 *>(&s_x[rr][32 * (c + 1) + 8 * kb]);
      w0 = r < NR ? w0 : zero;
      w1 = r < NR ? w1 : zero;
      const bf16x8 a0 = __builtin_bit_cast(bf16x8, w0), a1 = __builtin_bit_cast(bf16x8, w1);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, a0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, a1, acc1, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s_g[4 * kb + i][r] = acc0[i] + acc1[i];
    __syncthreads();
    // Lane v takes word v: a Gram entry (pairs j <= k in row-major order) or
    // a sum of squares, then the query dots.
    float word = 0.f;
    if (lane < NV) {
      if (lane >= Words::kDot) {
        const int j = lane - Words::kDot;
        word = s_g[NS][j] + s_g[NS + 1][j];
      } else if (ONORM) {
        int j = 0, rem = lane;
#pragma unroll
        for (int q = 0; q < NS; ++q)
          if (rem >= NS - j && j < NS - 1) {
            rem -= NS - j;
            ++j;
          }
        word = s_g[j][j + rem];
      } else {
        word = s_g[lane][lane];
      }
      tagged_store(slot + lane, word, gen);
    }
  } else {
  {
    float ss[NS], dq[NS];
    tk.partials(qh, ql, ss, dq);
    if constexpr (ONORM) {
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        s_tr[pair_row_start(NS, j)][lane] = ss[j];
#pragma unroll
        for (int k = j + 1; k < NS; ++k) {
          float g = 0.f;
#pragma unroll
          for (int i = 0; i < SPL; ++i)
#pragma unroll
            for (int w = 0; w < 4; ++w) g = dot2(tk.x[j][i][w], tk.x[k][i][w], g);
          s_tr[pair_row_start(NS, j) + (k - j)][lane] = g;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NS; ++j) s_tr[j][lane] = ss[j];
    }
#pragma unroll
    for (int j = 0; j < NS; ++j) s_tr[Words::kDot + j][lane] = dq[j];
  }
  tk.keep_packed();
  __syncthreads();
  if (lane < NV) {
    const float v = sum_float4s<kWave / 4>(reinterpret_cast<const float4 *>(s_tr[lane]));
    tagged_store(slot + lane, v, gen);
  }
  }

  tk.issue_onw(p, seg0, seg_step);
  // The token's totals: lane v holds word v summed over the parts.
  const float total =
      lane < NV ? gather(tok_near, tok_far, lane, gen + p.wait_skew, p.ws_flag, p.spin_limit)
                : 0.f;
  float ss_j;
  const float p_lane = weights_from_totals<NS, ONORM>(total, p.rms_eps, inv_h, ss_j);
  float y[SPL][8];
  tk.keep_packed();
  tk.mix(p_lane, y);

  float rsig = 1.f;
  if constexpr (ONORM) {
    float ysq, b;
    gram_ysq<NS>(total, p_lane, ss_j, ysq, b);
    float tot = ysq;
    if (!(ysq >= kGramGuard * b * b)) {
      // Every part sees the same totals and takes the same branch.
      const float sy = wave_sum_lane63(sum_sq<SPL>(y));
      if (lane == kWave - 1) tagged_store(slot + kSlotYsq, sy, gen);
      tot = gather(tok_near, tok_far, kSlotYsq, gen + p.wait_skew, p.ws_flag, p.spin_limit);
    }
    rsig = rsqrtf(tot * inv_h + p.out_eps);
  }
  tk.store(p, t, seg0, seg_step, y, rsig);
}

// ---------------------------------------------------------------------------
// workspace frames: which one is nearer each XCD
// ---------------------------------------------------------------------------

constexpr int kCalibWgs = 64;        // eight per XCD (kFrameCandidates 2 MB frames timed)
constexpr int kCalibRounds = 8;

struct CalibArgs {
  uint64_t *lines[kFrameCandidates];  // a spare area of each candidate frame
  int *out;                           // per workgroup: its XCD, then ticks per candidate
  int candidates;
};

// Lane 0 of each workgroup times kCalibRounds device-scope store-then-load
// round trips to its own 128-byte line of every candidate frame: the load
// retires after the store's acknowledgement, which is what a publishing part
// of the split path waits for.  Every wait is bounded.
__global__ void __launch_bounds__(kWave) attnres_frame_calibration_kernel(CalibArgs a) {
  if (threadIdx.x != 0) return;
  int *const o = a.out + blockIdx.x * (1 + kFrameCandidates);
  o[0] = int(hw_xcc_id());
  for (int c = 0; c < a.candidates; ++c) {
    uint64_t *const w = a.lines[c] + blockIdx.x * 16;
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    for (int k = 1; k <= kCalibRounds; ++k) {
      __hip_atomic_store(w, uint64_t(k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int s = 0; s < 1000; ++s)
        if (__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == uint64_t(k)) break;
    }
    o[1 + c] = int(__builtin_amdgcn_s_memrealtime() - t0);
  }
}

// ---------------------------------------------------------------------------
// specialisation tables
// ---------------------------------------------------------------------------

using KernelFn = void (*)(KParams);

template <int NB>
KernelFn row_fn(bool d, bool o, bool cache_rw, bool ranged) {
  if constexpr (NB > 0)
    if (cache_rw) {
      if (d) return o ? attnres_row_kernel<NB, true, true, true> : attnres_row_kernel<NB, true, false, true>;
      return o ? attnres_row_kernel<NB, false, true, true> : attnres_row_kernel<NB, false, false, true>;
    }
  if constexpr (NB >= kRowRangedMinBlocks)
    if (ranged) {
      if (d)
        return o ? attnres_row_kernel<NB, true, true, false, true>
                 : attnres_row_kernel<NB, true, false, false, true>;
      return o ? attnres_row_kernel<NB, false, true, false, true>
               : attnres_row_kernel<NB, false, false, false, true>;
    }
  if (d) return o ? attnres_row_kernel<NB, true, true> : attnres_row_kernel<NB, true, false>;
  return o ? attnres_row_kernel<NB, false, true> : attnres_row_kernel<NB, false, false>;
}
template <int NB>
KernelFn split_fn(bool d, bool o) {
  if (d) return o ? attnres_split_kernel<NB, true, true> : attnres_split_kernel<NB, true, false>;
  return o ? attnres_split_kernel<NB, false, true> : attnres_split_kernel<NB, false, false>;
}
// The split path above 7168: SPL segments per lane per part, masked at the
// row end.
template <int NB, int SPL>
KernelFn split_masked_fn(bool d, bool o) {
  if (d)
    return o ? attnres_split_kernel<NB, true, true, SPL, true>
             : attnres_split_kernel<NB, true, false, SPL, true>;
  return o ? attnres_split_kernel<NB, false, true, SPL, true>
           : attnres_split_kernel<NB, false, false, SPL, true>;
}
// The split kernel at H != 7168: SPL segments per lane and part, masked at
// the row end (SPL = 1 below 7168, 2 or 3 above).
KernelFn pick_split_masked(int nb, bool d, bool o, int spl) {
  switch (nb) {
#define ATTNRES_CASE(N)                                                     \
  case N:                                                                   \
    return spl == 1   ? split_masked_fn<N, 1>(d, o)                         \
           : spl == 2 ? split_masked_fn<N, 2>(d, o)                         \
                      : split_masked_fn<N, 3>(d, o);
    ATTNRES_CASE(0) ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4)
    ATTNRES_CASE(5) ATTNRES_CASE(6) ATTNRES_CASE(7) ATTNRES_CASE(8)
#undef ATTNRES_CASE
    default: return nullptr;
  }
}

template <int SPL, bool MASKED, int NB>
KernelFn anyh_fn(bool d, bool o, bool cache_rw) {
  if constexpr (NB > 0)
    if (cache_rw) {
      if (d)
        return o ? attnres_anyh_kernel<SPL, MASKED, NB, true, true, true>
                 : attnres_anyh_kernel<SPL, MASKED, NB, true, false, true>;
      return o ? attnres_anyh_kernel<SPL, MASKED, NB, false, true, true>
               : attnres_anyh_kernel<SPL, MASKED, NB, false, false, true>;
    }
  if (d)
    return o ? attnres_anyh_kernel<SPL, MASKED, NB, true, true>
             : attnres_anyh_kernel<SPL, MASKED, NB, true, false>;
  return o ? attnres_anyh_kernel<SPL, MASKED, NB, false, true>
           : attnres_anyh_kernel<SPL, MASKED, NB, false, false>;
}

// The any-H kernel with kAnyLdsRows bank rows staged into LDS (4..8 bank
// rows, two or four segments per lane).
constexpr int kAnyLdsRows = 3;
template <int SPL, bool MASKED, int NB, bool W6>
KernelFn anyh_lds_fn(bool d, bool o, bool c) {
  if constexpr (NB >= 4) {
    constexpr int L = kAnyLdsRows;
    if (c) {
      if (d)
        return o ? attnres_anyh_kernel<SPL, MASKED, NB, true, true, true, L, W6>
                 : attnres_anyh_kernel<SPL, MASKED, NB, true, false, true, L, W6>;
      return o ? attnres_anyh_kernel<SPL, MASKED, NB, false, true, true, L, W6>
               : attnres_anyh_kernel<SPL, MASKED, NB, false, false, true, L, W6>;
    }
    if (d)
      return o ? attnres_anyh_kernel<SPL, MASKED, NB, true, true, false, L, W6>
               : attnres_anyh_kernel<SPL, MASKED, NB, true, false, false, L, W6>;
    return o ? attnres_anyh_kernel<SPL, MASKED, NB, false, true, false, L, W6>
             : attnres_anyh_kernel<SPL, MASKED, NB, false, false, false, L, W6>;
  }
  return nullptr;
}
template <int NB>
KernelFn anyh_lds_pick(const AnyShape &sh, bool d, bool o, bool c) {
  if (sh.spl == 2) {
    if (sh.threads / kWave >= 6)
      return sh.masked ? anyh_lds_fn<2, true, NB, true>(d, o, c)
                       : anyh_lds_fn<2, false, NB, true>(d, o, c);
    return sh.masked ? anyh_lds_fn<2, true, NB, false>(d, o, c)
                     : anyh_lds_fn<2, false, NB, false>(d, o, c);
  }
  return sh.masked ? anyh_lds_fn<4, true, NB, false>(d, o, c)
                   : anyh_lds_fn<4, false, NB, false>(d, o, c);
}
KernelFn pick_anyh_lds(const AnyShape &sh, int nb, bool d, bool o, bool cache_rw) {
  switch (nb) {
#define ATTNRES_CASE(N) \
  case N: return anyh_lds_pick<N>(sh, d, o, cache_rw);
    ATTNRES_CASE(4) ATTNRES_CASE(5) ATTNRES_CASE(6) ATTNRES_CASE(7) ATTNRES_CASE(8)
#undef ATTNRES_CASE
    default: return nullptr;
  }
}

// Whether an any-H call stages kAnyLdsRows bank rows into LDS, and the
// dynamic LDS bytes it then takes.  Registers bound the resident workgroups
// per CU of the plain kernel; staging three rows frees 12 (two segments per
// lane) or 48 (four) VGPRs per lane for one more workgroup, at the cost of a
// second round of loads per token (the rows after the staged ones wait for
// registers).
// - Two segments per lane: the plain kernel may take 128 VGPRs (four waves
//   per SIMD), so three 5-wave workgroups fit (H = 4104..5120) or two 6-wave
//   ones (H = 5128..6144), and a call of more tokens than that runs a partial
//   second round (T = 1024 at H = 5120: 768 + 256).  Staged, four fit: the
//   5-wave kernels are built for 96 VGPRs (30 KB of LDS each), the 6-wave
//   ones for 80 (six waves per SIMD; 37 KB of LDS each, 157 KB per CU).
//   Measured (T = 1024, delta and norm, µs per call, plain / LDS-direct rows
//   / staged): H = 5120 nb = 8 28.6 / 24.8 / 23.6, nb = 4 19.9 / 18.6 /
//   18.8; H = 4104 - / 22.8 / 20.9; H = 4608 T = 2048 - / 45.1 / 42.5; 6
//   waves, plain / staged: H = 5632 30.8 / 26.3, H = 6144 32.2 / 28.7 (nb = 4
//   24.1 / 21.2), T = 2048 56.0 / 54.3, T = 600 19.1 / 19.8.  So 5- and
//   6-wave workgroups, for more tokens than three per CU.  (The 6-wave
//   kernels at 96 VGPRs fitted three per CU, not four, and then lost.)
// - Four segments per lane: a token of 5-6 waves (H = 8200..12288) fills a
//   CU's registers (200+ VGPRs), one workgroup per CU; staged it takes at
//   most 168 (three waves per SIMD), so two fit, with 61-74 KB of LDS each.
//   Measured (delta, norm, 8 bank rows, µs per call, plain / staged): 5
//   waves, H = 8704 T = 300 22.3 / 21.2, T = 1024 53.7 / 51.7, T = 2048
//   97.5 / 94.2; H = 9216 T = 4096 without delta or norm 150.7 / 141.9;
//   H = 10240 T = 300 23.5 / 22.5, T = 2048 103.7 / 105.9.  6 waves,
//   H = 12288: T = 300 26.0 / 25.3, T = 1024 64.8 / 65.6, T = 2048 119.2 /
//   121.8 (H = 11264 and 12032 alike).  So 5-wave workgroups from one token
//   per CU up, 6-wave ones only up to two.
bool anyh_lds_rows(const AnyShape &sh, int64_t T, int nb, int cus, size_t *dyn) {
  const int waves = sh.threads / kWave;
  if (!ATTNRES_ANYH_STAGED || nb < 4) return false;
  bool use;
  if (sh.spl == 2)
    use = (waves == 5 || waves == 6) && T > int64_t(3) * cus;
  else
    use = T > int64_t(cus) && (waves == 5 || (waves == 6 && T <= int64_t(2) * cus));
  if (!use) return false;
  *dyn = size_t(kAnyLdsRows) * sh.spl * sh.threads * 16;
  return true;
}

template <int NB>
KernelFn anyh_pick(const AnyShape &sh, bool d, bool o, bool c) {
  if (sh.spl == 2)
    return sh.masked ? anyh_fn<2, true, NB>(d, o, c) : anyh_fn<2, false, NB>(d, o, c);
  return sh.masked ? anyh_fn<4, true, NB>(d, o, c) : anyh_fn<4, false, NB>(d, o, c);
}

KernelFn pick_anyh(const AnyShape &sh, int nb, bool d, bool o, bool cache_rw) {
  switch (nb) {
#define ATTNRES_CASE(N) \
  case N: return anyh_pick<N>(sh, d, o, cache_rw);
    ATTNRES_CASE(0) ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4)
    ATTNRES_CASE(5) ATTNRES_CASE(6) ATTNRES_CASE(7) ATTNRES_CASE(8)
#undef ATTNRES_CASE
    default: return nullptr;
  }
}

template <int SPL, bool MASKED>
KernelFn bank_fn(int nb) {
  switch (nb) {
#define ATTNRES_CASE(N) \
  case N: return attnres_bank_kernel<SPL, MASKED, N>;
    ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4)
    ATTNRES_CASE(5) ATTNRES_CASE(6) ATTNRES_CASE(7) ATTNRES_CASE(8)
#undef ATTNRES_CASE
    default: return nullptr;
  }
}
KernelFn pick_bank(const AnyShape &sh, int nb) {
  if (sh.spl == 2) return sh.masked ? bank_fn<2, true>(nb) : bank_fn<2, false>(nb);
  return sh.masked ? bank_fn<4, true>(nb) : bank_fn<4, false>(nb);
}
template <int SPL, bool MASKED, bool BANK>
KernelFn cur_fn(bool d, bool o) {
  if (d) return o ? attnres_cur_kernel<SPL, MASKED, true, true, BANK>
                  : attnres_cur_kernel<SPL, MASKED, true, false, BANK>;
  return o ? attnres_cur_kernel<SPL, MASKED, false, true, BANK>
           : attnres_cur_kernel<SPL, MASKED, false, false, BANK>;
}
template <int SPL, bool MASKED>
KernelFn cur_fn_b(bool d, bool o, bool bank) {
  return bank ? cur_fn<SPL, MASKED, true>(d, o) : cur_fn<SPL, MASKED, false>(d, o);
}
KernelFn pick_cur(const AnyShape &sh, bool d, bool o, bool bank) {
  if (sh.spl == 2) return sh.masked ? cur_fn_b<2, true>(d, o, bank) : cur_fn_b<2, false>(d, o, bank);
  return sh.masked ? cur_fn_b<4, true>(d, o, bank) : cur_fn_b<4, false>(d, o, bank);
}

enum class Kind { kRow, kSplit, kAnyH };

// Smallest call, in elements per row array (T * H), for which the row
// kernels read the two rewritten rows through the cache.  Measured crossover:
// between 512 and 1024 tokens at H = 7168 (nb = 1, 4, 8), and for the any-H
// kernel between about 4 and 8 million elements from H = 2048 to 16384.
constexpr int64_t kCacheRewrittenMinElems = int64_t(1024) * 7168;

// Whether a row-kernel call reads its rewritten rows through the cache: it
// writes a bank slot that is also a source, and is large enough.  With a
// delta, prefix is rewritten too; with the written slot as the only such
// row the gain starts at about twice the size (T = 1024 at H = 7168 was
// +2 % at nb = 4 and -2 % at nb = 8; T = 2048 +3-6 %, T = 4096 +5-12 %).
bool cache_rewritten(const FwdArgs &a) {
  if (a.block_write_idx < 0 || a.block_write_idx >= a.num_blocks) return false;
  const int64_t min_elems = a.delta != nullptr ? kCacheRewrittenMinElems : 2 * kCacheRewrittenMinElems;
  return a.T * a.H >= min_elems;
}

// attnres_fwd's choice of kernel at H = 7168, from measured latency per call
// (graph replay, cold inputs, delta and output norm): spreading a token over
// 14 CUs (split) beats one CU per token (row) up to this many tokens, by
// block count.  A single source (nb = 0) needs no exchange on the row path,
// which is then faster at every T.  The row side near these limits is the
// row kernel's ranged form (kRowRangedMaxT), which moved them down from
// 48/64/64/72/64/64/60 at nb = 2..8.
constexpr int kSplitMaxT[kMaxBlocks + 1] = {0, 40, 40, 48, 56, 56, 52, 60, 56};
static_assert(72 <= ATTNRES_SPLIT_MAX_TOKENS, "split crossover beyond the workspace");
Kind auto_kind(int64_t T, int nb) {
  return nb > 0 && T <= kSplitMaxT[nb] ? Kind::kSplit : Kind::kRow;
}
// Away from H = 7168, from latency grids against the any-H row kernel (graph
// replay, cold inputs, delta and output norm; us per call, any-H / split).
// Above 8192 (2-3 segments per lane and part) the split path leads at every
// block count up to 72 tokens (H = 10240, nb = 8, T = 72: 10.64 / 8.93;
// H = 16384, nb = 8, T = 80: 13.04 / 16.06).  From 7176 to 8192 the any-H
// kernel is relatively fast and the split path's reach depends on the block
// count (H = 8192: nb = 1 leads to T = 16, T = 24 4.32 / 4.35; nb = 8 to
// T = 40, T = 48 7.47 / 7.60; H = 7680 alike).  Between 4096 and 7168 (one
// masked segment per lane and part) likewise, measured at 4608, 5120 and
// 6144 (H = 5120: nb = 1 ties at T = 8, 3.75 / 3.74; nb = 4 leads to T = 40,
// T = 48 4.92 / 5.00; nb = 8 still leads at T = 48, 6.40 / 6.12).  At 4096
// and below the any-H kernel leads almost everywhere: only nb = 8 (at 4096
// also nb = 7) gains, by at most 3 %, at a few tokens (H = 4096, nb = 8,
// T = 16: 4.81 / 4.79; T = 24: 4.84 / 5.02; H = 3584, nb = 8, T = 1: 4.34 /
// 4.20; H = 2880 and 3072: never).
constexpr int64_t kWiderHidden = 8192;
constexpr int kSplitMaxTWider = 72;
constexpr int kSplitMaxTWide[kMaxBlocks + 1] = {0, 16, 24, 32, 40, 32, 32, 32, 40};
constexpr int64_t kNarrowSplitHidden = 4096;
constexpr int kSplitMaxTNarrow[kMaxBlocks + 1] = {0, 8, 16, 24, 40, 40, 48, 48, 48};
constexpr int kSplitMaxT4096[kMaxBlocks + 1] = {0, 0, 0, 0, 0, 0, 0, 8, 16};
constexpr int64_t kSmallSplitHidden = 3072;  // above it (below 4096): nb = 8 only
constexpr int kSplitMaxTSmall8 = 8;

// The kernel attnres_fwd runs for T tokens, hidden size H and nb block rows.
Kind auto_choice(int64_t T, int64_t H, int nb) {
  if (H == kHidden) return auto_kind(T, nb);
  if (nb <= 0) return Kind::kAnyH;
  int64_t limit = 0;
  if (H > kWiderHidden)
    limit = kSplitMaxTWider;
  else if (H > kHidden)
    limit = kSplitMaxTWide[nb];
  else if (H > kNarrowSplitHidden)
    limit = kSplitMaxTNarrow[nb];
  else if (H == kNarrowSplitHidden)
    limit = kSplitMaxT4096[nb];
  else if (H > kSmallSplitHidden && nb == kMaxBlocks)
    limit = kSplitMaxTSmall8;
  return T <= limit ? Kind::kSplit : Kind::kAnyH;
}

KernelFn pick(Kind kind, int nb, bool d, bool o, bool cache_rw, bool ranged) {
  switch (nb) {
#define ATTNRES_CASE(N) \
  case N: return kind == Kind::kSplit ? split_fn<N>(d, o) : row_fn<N>(d, o, cache_rw, ranged);
    ATTNRES_CASE(0) ATTNRES_CASE(1) ATTNRES_CASE(2) ATTNRES_CASE(3) ATTNRES_CASE(4)
    ATTNRES_CASE(5) ATTNRES_CASE(6) ATTNRES_CASE(7) ATTNRES_CASE(8)
#undef ATTNRES_CASE
    default: return nullptr;
  }
}

// ---------------------------------------------------------------------------
// per-device split-path workspace
// ---------------------------------------------------------------------------

constexpr int kMaxDevices = 64;
constexpr size_t kPartBytes = size_t(ATTNRES_SPLIT_MAX_TOKENS) * kParts * kSlot * sizeof(uint64_t);
constexpr size_t kFlagBytes = 256;
constexpr size_t kWorkspaceBytes = kPartBytes + kFlagBytes;
// The allocated workspace is two 2 MB frames (A holds the fault flag too);
// the calibration uses their last 16 KB.
constexpr size_t kFrameBytes = size_t(2) << 20;
constexpr size_t kCalibLines = kFrameBytes - 16384;
constexpr size_t kCalibOut = kFrameBytes - 4096;
static_assert(kWorkspaceBytes <= kCalibLines, "split workspace overlaps the calibration area");
static_assert(size_t(kCalibWgs) * 128 <= kCalibOut - kCalibLines, "calibration lines");
static_assert(sizeof(int) * kCalibWgs * (1 + kFrameCandidates) <= kFrameBytes - kCalibOut,
              "calibration output");
static_assert(size_t(kCalibWgs) * (1 + kFrameCandidates) * sizeof(int) <= 4096, "calibration out");

// Split calls on one device must run one after another: they share the
// workspace, and two split kernels running at once could each hold the
// compute-unit slots the other's remaining parts need.  A split call on a
// different stream than the previous one therefore makes its stream wait for
// everything enqueued on the previous stream so far (outside graph capture).
struct DeviceWorkspace {
  void *base = nullptr;           // frame A: the parts' words, then the fault flag
  void *base_b = nullptr;         // frame B: the parts' words
  uint64_t *part = nullptr;
  uint64_t *part_b = nullptr;
  unsigned near = 0;              // bit x: a part on XCD x writes frame B
  unsigned *flag = nullptr;
  hipEvent_t handoff = nullptr;   // recorded on the previous stream at a switch
  hipStream_t last_stream = nullptr;
  bool has_last = false;
};

DeviceWorkspace g_ws[kMaxDevices];
std::mutex g_ws_mu;
std::atomic<int> g_last_hip{0};
std::atomic<bool> g_force_wait_failure{false};  // attnres_debug_force_wait_failure
std::atomic<int> g_frames_mode{-1};               // attnres_debug_workspace_frames
constexpr int kForcedSpinLimit = 64;

}  // namespace

// The split path's workspace for attnres_fwd_noalloc, in static device
// memory so that this entry point never allocates: the tagged words of
// ATTNRES_SPLIT_MAX_TOKENS tokens, then the fault flag, laid out as in the
// allocated workspace.  Each device that runs the library holds its own copy
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address is taken once per device with
// hipGetSymbolAddress (static_scratch_locked below), and only that address
// is ever passed to a kernel or to a HIP memory call.
constexpr size_t kScratchWords = kWorkspaceBytes / sizeof(uint64_t);
static_assert(kScratchWords * sizeof(uint64_t) == kWorkspaceBytes, "scratch layout");
static __device__ __align__(256) uint64_t scratch[kScratchWords];

namespace {

void *g_scratch[kMaxDevices];  // scratch's address on each device (under g_ws_mu)

// Records a failed HIP call's error for attnres_last_hip_error and clears the
// runtime's last-error state, so that the caller's next unrelated error check
// does not report it again (the call has already returned ATTNRES_E_HIP).
int hip_fail(hipError_t e) {
  g_last_hip.store(int(e));
  (void)hipGetLastError();
  return ATTNRES_E_HIP;
}

// Times a device-scope store and load from every XCD to each candidate frame
// (the calibration kernel); ticks[x][c] is the fastest workgroup on XCD x,
// INT_MAX for an XCD that ran none (a partition with fewer).
hipError_t calibrate_frames(void *const (&cand)[kFrameCandidates],
                            int (&ticks)[kFrameXcds][kFrameCandidates]) {
  CalibArgs a{};
  for (int c = 0; c < kFrameCandidates; ++c)
    a.lines[c] = reinterpret_cast<uint64_t *>(static_cast<char *>(cand[c]) + kCalibLines);
  a.out = reinterpret_cast<int *>(static_cast<char *>(cand[0]) + kCalibOut);
  a.candidates = kFrameCandidates;
  void *args[] = {&a};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(attnres_frame_calibration_kernel),
                                 dim3(kCalibWgs), dim3(kWave), args, 0, nullptr);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  int out[kCalibWgs * (1 + kFrameCandidates)];
  if (e == hipSuccess) e = hipMemcpy(out, a.out, sizeof out, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  for (auto &row : ticks)
    for (int &v : row) v = INT_MAX;
  for (int b = 0; b < kCalibWgs; ++b) {
    const int *o = out + b * (1 + kFrameCandidates);
    const int x = o[0] & (kFrameXcds - 1);
    for (int c = 0; c < kFrameCandidates; ++c) ticks[x][c] = std::min(ticks[x][c], o[1 + c]);
  }
  return hipSuccess;
}

int init_device_locked(int device) {
  if (g_ws[device].base) return ATTNRES_OK;
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = hipSetDevice(device)) != hipSuccess) return hip_fail(e);
  // Candidate frames, each its own 2 MB allocation; consecutive ones have
  // alternated between the two halves of the chip.
  void *cand[kFrameCandidates] = {};
  hipEvent_t ev = nullptr;
  for (int c = 0; c < kFrameCandidates && e == hipSuccess; ++c) {
    e = hipMalloc(&cand[c], kFrameBytes);
    if (e == hipSuccess) e = hipMemset(cand[c], 0, kFrameBytes);
  }
  int ticks[kFrameXcds][kFrameCandidates];
  if (e == hipSuccess) e = calibrate_frames(cand, ticks);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
  if (e != hipSuccess) {
    for (void *c : cand)
      if (c) (void)hipFree(c);
    (void)hipSetDevice(prev);
    return hip_fail(e);
  }
  // The pair of frames whose nearer member serves every XCD fastest.
  int fa = 0, fb = 1;
  unsigned near = 0;
  choose_frames(ticks, &fa, &fb, &near);
  for (int c = 0; c < kFrameCandidates; ++c)
    if (c != fa && c != fb) (void)hipFree(cand[c]);
  DeviceWorkspace &w = g_ws[device];
  w.base = cand[fa];
  w.base_b = cand[fb];
  w.near = near;
  w.handoff = ev;
  w.part = static_cast<uint64_t *>(w.base);
  w.part_b = static_cast<uint64_t *>(w.base_b);
  w.flag = reinterpret_cast<unsigned *>(static_cast<char *>(w.base) + kPartBytes);
  (void)hipSetDevice(prev);
  return ATTNRES_OK;
}

// Takes scratch's address on `device` (with that device current) the first
// time, and clears it then: the generation tags of a token's parts must agree
// and the fault flag must start at zero.  Synchronous; outside graph capture.
int static_scratch_locked(int device) {
  if (g_scratch[device]) return ATTNRES_OK;
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = hipSetDevice(device)) != hipSuccess) return hip_fail(e);
  void *ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e == hipSuccess && ptr == nullptr) e = hipErrorInvalidSymbol;
  if (e == hipSuccess) e = hipMemset(ptr, 0, kWorkspaceBytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return hip_fail(e);
  g_scratch[device] = ptr;
  return ATTNRES_OK;
}

// The device a call's kernels run on: the stream's (the current device for
// the null stream), whatever device is current.
int launch_device(hipStream_t s, int *dev) {
  hipError_t e = s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e);
  if (*dev < 0 || *dev >= kMaxDevices) return ATTNRES_E_UNSUPPORTED;
  return ATTNRES_OK;
}

// A device's compute-unit count, cached per device.
std::atomic<int> g_cus[kMaxDevices];
int compute_units(int dev, int *cus) {
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    if (n <= 0) n = 1;
    g_cus[dev].store(n, std::memory_order_relaxed);
  }
  *cus = n;
  return ATTNRES_OK;
}

// Lets `fn` take `bytes` of dynamic LDS, beyond the runtime's default per
// workgroup limit; set once per kernel (the attribute stays with it).
std::mutex g_lds_attr_mu;
const void *g_lds_attr_done[128];  // more than the staged kernels
int allow_dynamic_lds(KernelFn fn, size_t bytes) {
  const void *f = reinterpret_cast<const void *>(fn);
  std::lock_guard<std::mutex> lock(g_lds_attr_mu);
  for (const void *d : g_lds_attr_done)
    if (d == f) return ATTNRES_OK;
  const hipError_t e =
      hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes));
  if (e != hipSuccess) return hip_fail(e);
  for (const void *&d : g_lds_attr_done)
    if (d == nullptr) {
      d = f;
      break;
    }
  return ATTNRES_OK;
}

// The dynamic-LDS attribute of every any-H kernel with staged rows, so that
// a first call under graph capture makes no attribute call.  The largest
// such workgroup (384 lanes, four segments) takes 72 KB.
constexpr size_t kAnyLdsMaxBytes = size_t(kAnyLdsRows) * 4 * 384 * 16;
int allow_staged_lds() {
  const AnyShape shapes[6] = {{2, 5 * kWave, false}, {2, 5 * kWave, true},
                              {2, 6 * kWave, false}, {2, 6 * kWave, true},
                              {4, 6 * kWave, false}, {4, 6 * kWave, true}};
  for (const AnyShape &sh : shapes)
    for (int nb = 4; nb <= kMaxBlocks; ++nb)
      for (int f = 0; f < 8; ++f) {
        const KernelFn fn = pick_anyh_lds(sh, nb, f & 1, f & 2, f & 4);
        if (!fn) continue;
        const int rc = allow_dynamic_lds(fn, kAnyLdsMaxBytes);
        if (rc != ATTNRES_OK) return rc;
      }
  return ATTNRES_OK;
}

// noalloc: the split path takes the static scratch instead of the allocated
// workspace, and no stream hand-off is made (calls that overlap race).
int fwd_impl(const FwdArgs &a, void *stream, int path, bool noalloc = false) {
  if (path != ATTNRES_PATH_AUTO && path != ATTNRES_PATH_ROW && path != ATTNRES_PATH_SPLIT &&
      path != ATTNRES_PATH_ANY_H)
    return ATTNRES_E_PATH;
  int rc = validate(a);
  if (rc != ATTNRES_OK) return rc;
  if (a.T == 0) return ATTNRES_OK;

  // The tuned kernels are built for H = 7168; every other H runs the any-H
  // row kernel, which can also be forced at 7168.  The split path runs at
  // every H: away from 7168 its 14 parts take 1 (below), 2 or 3 (above)
  // segments per lane, masked at the row end, and above 7168 the automatic
  // choice uses it for small batches.
  const bool tuned = a.H == kHidden;
  const bool wide = a.H > kHidden;
  const int split_spl = wide ? int((a.H / kSeg + kParts * kPartThreads - 1) / (kParts * kPartThreads)) : 1;
  Kind kind;
  if (path == ATTNRES_PATH_ANY_H)
    kind = Kind::kAnyH;
  else if (path == ATTNRES_PATH_SPLIT)
    kind = Kind::kSplit;
  else if (path == ATTNRES_PATH_ROW)
    kind = tuned ? Kind::kRow : Kind::kAnyH;
  else
    kind = auto_choice(a.T, a.H, a.num_blocks);
  const bool any_h = kind == Kind::kAnyH;
  const bool split = kind == Kind::kSplit;
  if (split && a.T > ATTNRES_SPLIT_MAX_TOKENS) return ATTNRES_E_UNSUPPORTED;

  KParams kp{};
  kp.prefix = static_cast<uint16_t *>(const_cast<void *>(a.prefix));
  kp.delta = static_cast<const uint16_t *>(a.delta);
  kp.blocks = static_cast<uint16_t *>(const_cast<void *>(a.blocks));
  kp.res_w = static_cast<const uint16_t *>(a.res_w);
  kp.rms_w = static_cast<const uint16_t *>(a.rms_w);
  kp.onw = static_cast<const uint16_t *>(a.output_norm_weight);
  kp.out = static_cast<uint16_t *>(const_cast<void *>(a.out));
  kp.tok_stride = a.block_token_stride;
  kp.slot_stride = a.block_slot_stride;
  kp.prefix_stride = row_stride(a.prefix_stride, a.T, a.H);
  kp.delta_stride = a.delta ? row_stride(a.delta_stride, a.T, a.H) : 0;
  kp.out_stride = row_stride(a.out_stride, a.T, a.H);
  kp.nseg = int(a.H / kSeg);
  kp.inv_h = 1.0f / float(a.H);
  kp.rms_eps = a.rms_eps;
  kp.out_eps = a.output_norm_weight ? a.output_norm_eps : 0.f;
  kp.widx = a.block_write_idx;
  kp.T = int(a.T);
  // A test of the failure path may have the split path's waits look for a
  // generation that never comes, and give up after a few polls.
  const bool force_fail = g_force_wait_failure.load();
  kp.spin_limit = force_fail ? kForcedSpinLimit : kSpinLimit;
  kp.wait_skew = force_fail ? 0x40000000u : 0u;

  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  rc = launch_device(s, &dev);
  if (rc != ATTNRES_OK) return rc;
  // A split call holds the workspace lock from the stream hand-off through
  // its launch: another thread's split call on another stream may then only
  // record its hand-off after this kernel is enqueued.
  std::unique_lock<std::mutex> ws_lock;
  if (split) {
    ws_lock = std::unique_lock<std::mutex>(g_ws_mu);
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(s, &st);
    if (e != hipSuccess) return hip_fail(e);
    const bool capturing = st != hipStreamCaptureStatusNone;
    if (noalloc) {
      if (!g_scratch[dev]) {
        if (capturing) return ATTNRES_E_NOT_INIT;
        rc = static_scratch_locked(dev);
        if (rc != ATTNRES_OK) return rc;
      }
      // One frame: both copies are the static array.
      kp.ws_part = kp.ws_part_b = static_cast<uint64_t *>(g_scratch[dev]);
      kp.ws_flag = reinterpret_cast<unsigned *>(static_cast<char *>(g_scratch[dev]) + kPartBytes);
      kp.ws_by_part = g_frames_mode.load() >= 256;
    }
    DeviceWorkspace &w = g_ws[dev];
    if (noalloc) {
      // nothing to allocate or order
    } else if (!w.base) {
      if (capturing) return ATTNRES_E_NOT_INIT;
      rc = init_device_locked(dev);
      if (rc != ATTNRES_OK) return rc;
    }
    if (!capturing && !noalloc) {
      if (w.has_last && w.last_stream != s) {
        e = hipEventRecord(w.handoff, w.last_stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(s, w.handoff, 0);
        if (e != hipSuccess) return hip_fail(e);
      }
      w.last_stream = s;
      w.has_last = true;
    }
    if (!noalloc) {
      kp.ws_part = w.part;
      kp.ws_part_b = w.part_b;
      kp.ws_flag = w.flag;
      const int fm = g_frames_mode.load();
      kp.ws_near = fm < 0 ? w.near : fm >= 256 ? 0xAAAAu : unsigned(fm);
      kp.ws_by_part = fm >= 256;
    }
  }

  const bool has_d = a.delta != nullptr, has_o = a.output_norm_weight != nullptr;
  hipError_t e;
  if (any_h) {
    const AnyShape sh = anyh_shape(a.H);
    kp.threads = sh.threads;
    int cus = 0;
    rc = compute_units(dev, &cus);
    if (rc != ATTNRES_OK) return rc;
    size_t dyn = 0;
    KernelFn fn = nullptr;
    if (anyh_lds_rows(sh, a.T, a.num_blocks, cus, &dyn)) {
      fn = pick_anyh_lds(sh, a.num_blocks, has_d, has_o, cache_rewritten(a));
      if (fn) {
        rc = allow_dynamic_lds(fn, kAnyLdsMaxBytes);
        if (rc != ATTNRES_OK) return rc;
      }
    }
    if (!fn) {
      dyn = 0;
      fn = pick_anyh(sh, a.num_blocks, has_d, has_o, cache_rewritten(a));
    }
    if (!fn) return ATTNRES_E_NUM_BLOCKS;
    void *args[] = {&kp};
    e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(unsigned(a.T)),
                        dim3(unsigned(sh.threads)), args, dyn, s);
    return e == hipSuccess ? ATTNRES_OK : hip_fail(e);
  }

  // Reading the rows a call also writes (a written slot that is a source,
  // and prefix with a delta) through the cache pays once a call streams many
  // tokens: T = 1024, nb = 8, with a delta: 33.7 -> 32.6 us, T = 4096:
  // 131 -> 117 us.  Smaller calls (latency-bound) read them streaming.
  const bool cache_rw = kind == Kind::kRow && cache_rewritten(a);
  const bool ranged = kind == Kind::kRow && !cache_rw && a.num_blocks >= kRowRangedMinBlocks &&
                      a.T <= kRowRangedMaxT[a.num_blocks];
  KernelFn fn = split && !tuned ? pick_split_masked(a.num_blocks, has_d, has_o, split_spl)
                              : pick(kind, a.num_blocks, has_d, has_o, cache_rw, ranged);
  if (!fn) return ATTNRES_E_NUM_BLOCKS;
  unsigned row_grid = unsigned(a.T);
  const int wpc = row_wgs_per_cu(a.num_blocks);
  if (kind == Kind::kRow && wpc > 0) {
    int cus = 0;
    rc = compute_units(dev, &cus);
    if (rc != ATTNRES_OK) return rc;
    const int64_t cap = int64_t(cus) * wpc;
    if (a.T > cap) row_grid = unsigned(cap);
  }
  // Split: 8 tokens per group of 8 kParts workgroups, placed per XCD (the
  // kernel's token mapping).
  const dim3 grid = split ? dim3(unsigned((a.T + 7) / 8) * 8 * kParts) : dim3(row_grid);
  const dim3 block = split ? dim3(kPartThreads) : dim3(kRowThreads);
  void *args[] = {&kp};
  e = hipLaunchKernel(reinterpret_cast<const void *>(fn), grid, block, args, 0, s);
  if (e != hipSuccess) return hip_fail(e);
  return ATTNRES_OK;
}

// The two kernels of the two-kernel form.  Both take the whole call's
// arguments (each validated as attnres_fwd would) and the partial-state
// buffer; the bank part launches nothing without bank rows.
int two_part_impl(const FwdArgs &a, const void *partial, int64_t partial_bytes, void *stream,
                  bool bank_part) {
  int rc = validate(a);
  if (rc == ATTNRES_OK) rc = validate_partial(a, partial, partial_bytes);
  if (rc != ATTNRES_OK) return rc;
  if (a.T == 0 || (bank_part && a.num_blocks == 0)) return ATTNRES_OK;

  KParams kp{};
  kp.prefix = static_cast<uint16_t *>(const_cast<void *>(a.prefix));
  kp.delta = static_cast<const uint16_t *>(a.delta);
  kp.blocks = static_cast<uint16_t *>(const_cast<void *>(a.blocks));
  kp.res_w = static_cast<const uint16_t *>(a.res_w);
  kp.rms_w = static_cast<const uint16_t *>(a.rms_w);
  kp.onw = static_cast<const uint16_t *>(a.output_norm_weight);
  kp.out = static_cast<uint16_t *>(const_cast<void *>(a.out));
  kp.tok_stride = a.block_token_stride;
  kp.slot_stride = a.block_slot_stride;
  kp.prefix_stride = row_stride(a.prefix_stride, a.T, a.H);
  kp.delta_stride = a.delta ? row_stride(a.delta_stride, a.T, a.H) : 0;
  kp.out_stride = row_stride(a.out_stride, a.T, a.H);
  kp.nseg = int(a.H / kSeg);
  kp.inv_h = 1.0f / float(a.H);
  kp.rms_eps = a.rms_eps;
  kp.out_eps = a.output_norm_weight ? a.output_norm_eps : 0.f;
  kp.widx = a.block_write_idx;
  kp.T = int(a.T);
  kp.partial = static_cast<float *>(const_cast<void *>(partial));

  const AnyShape sh = anyh_shape(a.H);
  kp.threads = sh.threads;
  KernelFn fn = bank_part ? pick_bank(sh, a.num_blocks)
                          : pick_cur(sh, a.delta != nullptr, a.output_norm_weight != nullptr,
                                     a.num_blocks > 0);
  if (!fn) return ATTNRES_E_NUM_BLOCKS;
  void *args[] = {&kp};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(unsigned(a.T)),
                                 dim3(unsigned(sh.threads)), args, 0,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTNRES_OK : hip_fail(e);
}

FwdArgs make_args(const void *prefix, int64_t prefix_stride, const void *delta,
                  int64_t delta_stride, const void *blocks, int64_t ts, int64_t ss,
                  int max_blocks, int num_blocks, const void *res_w, const void *rms_w,
                  float rms_eps, const void *onw, float oeps, int widx, const void *out,
                  int64_t out_stride, int64_t T, int64_t H) {
  FwdArgs a;
  a.prefix = prefix;
  a.prefix_stride = prefix_stride;
  a.delta = delta;
  a.delta_stride = delta_stride;
  a.blocks = blocks;
  a.block_token_stride = ts;
  a.block_slot_stride = ss;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.res_w = res_w;
  a.rms_w = rms_w;
  a.rms_eps = rms_eps;
  a.output_norm_weight = onw;
  a.output_norm_eps = oeps;
  a.block_write_idx = widx;
  a.out = out;
  a.out_stride = out_stride;
  a.T = T;
  a.H = H;
  return a;
}

}  // namespace
}  // namespace attnres

using namespace attnres;

extern "C" int attnres_fwd(void *prefix, const void *delta, void *blocks,
                           int64_t block_token_stride, int64_t block_slot_stride, int max_blocks,
                           int num_blocks, const void *res_w, const void *rms_w, float rms_eps,
                           const void *output_norm_weight, float output_norm_eps,
                           int block_write_idx, void *out, int64_t T, int64_t H, void *stream) {
  return fwd_impl(make_args(prefix, H, delta, H, blocks, block_token_stride, block_slot_stride,
                            max_blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                            output_norm_eps, block_write_idx, out, H, T, H),
                  stream, ATTNRES_PATH_AUTO);
}

extern "C" int attnres_fwd_path(void *prefix, const void *delta, void *blocks,
                                int64_t block_token_stride, int64_t block_slot_stride,
                                int max_blocks, int num_blocks, const void *res_w,
                                const void *rms_w, float rms_eps, const void *output_norm_weight,
                                float output_norm_eps, int block_write_idx, void *out, int64_t T,
                                int64_t H, void *stream, int path) {
  return fwd_impl(make_args(prefix, H, delta, H, blocks, block_token_stride, block_slot_stride,
                            max_blocks, num_blocks, res_w, rms_w, rms_eps, output_norm_weight,
                            output_norm_eps, block_write_idx, out, H, T, H),
                  stream, path);
}

extern "C" int attnres_fwd_strided(void *prefix, int64_t prefix_stride, const void *delta,
                                   int64_t delta_stride, void *blocks,
                                   int64_t block_token_stride, int64_t block_slot_stride,
                                   int max_blocks, int num_blocks, const void *res_w,
                                   const void *rms_w, float rms_eps,
                                   const void *output_norm_weight, float output_norm_eps,
                                   int block_write_idx, void *out, int64_t out_stride, int64_t T,
                                   int64_t H, void *stream, int path) {
  return fwd_impl(make_args(prefix, prefix_stride, delta, delta_stride, blocks,
                            block_token_stride, block_slot_stride, max_blocks, num_blocks, res_w,
                            rms_w, rms_eps, output_norm_weight, output_norm_eps, block_write_idx,
                            out, out_stride, T, H),
                  stream, path);
}

extern "C" int attnres_fwd_noalloc(void *prefix, int64_t prefix_stride, const void *delta,
                                   int64_t delta_stride, void *blocks,
                                   int64_t block_token_stride, int64_t block_slot_stride,
                                   int max_blocks, int num_blocks, const void *res_w,
                                   const void *rms_w, float rms_eps,
                                   const void *output_norm_weight, float output_norm_eps,
                                   int block_write_idx, void *out, int64_t out_stride, int64_t T,
                                   int64_t H, void *stream, int path) {
  return fwd_impl(make_args(prefix, prefix_stride, delta, delta_stride, blocks,
                            block_token_stride, block_slot_stride, max_blocks, num_blocks, res_w,
                            rms_w, rms_eps, output_norm_weight, output_norm_eps, block_write_idx,
                            out, out_stride, T, H),
                  stream, path, /*noalloc=*/true);
}

extern "C" int64_t attnres_partial_bytes(int64_t T, int64_t H) {
  return attnres::partial_bytes(T, H);
}

extern "C" int attnres_fwd_bank(const void *prefix, int64_t prefix_stride, const void *delta,
                                int64_t delta_stride, const void *blocks,
                                int64_t block_token_stride, int64_t block_slot_stride,
                                int max_blocks, int num_blocks, const void *res_w,
                                const void *rms_w, float rms_eps, const void *output_norm_weight,
                                float output_norm_eps, int block_write_idx, const void *out,
                                int64_t out_stride, int64_t T, int64_t H, void *partial,
                                int64_t partial_bytes, void *stream) {
  return two_part_impl(make_args(prefix, prefix_stride, delta, delta_stride, blocks,
                                 block_token_stride, block_slot_stride, max_blocks, num_blocks,
                                 res_w, rms_w, rms_eps, output_norm_weight, output_norm_eps,
                                 block_write_idx, out, out_stride, T, H),
                       partial, partial_bytes, stream, /*bank_part=*/true);
}

extern "C" int attnres_fwd_cur(void *prefix, int64_t prefix_stride, const void *delta,
                               int64_t delta_stride, void *blocks, int64_t block_token_stride,
                               int64_t block_slot_stride, int max_blocks, int num_blocks,
                               const void *res_w, const void *rms_w, float rms_eps,
                               const void *output_norm_weight, float output_norm_eps,
                               int block_write_idx, void *out, int64_t out_stride, int64_t T,
                               int64_t H, const void *partial, int64_t partial_bytes,
                               void *stream) {
  return two_part_impl(make_args(prefix, prefix_stride, delta, delta_stride, blocks,
                                 block_token_stride, block_slot_stride, max_blocks, num_blocks,
                                 res_w, rms_w, rms_eps, output_norm_weight, output_norm_eps,
                                 block_write_idx, out, out_stride, T, H),
                       partial, partial_bytes, stream, /*bank_part=*/false);
}

extern "C" int attnres_init(int device) {
  if (device < 0 || device >= kMaxDevices) return ATTNRES_E_UNSUPPORTED;
  int n = 0;
  hipError_t e = hipGetDeviceCount(&n);
  if (e != hipSuccess) return hip_fail(e);
  if (device >= n) return ATTNRES_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  int rc = init_device_locked(device);
  if (rc == ATTNRES_OK) rc = static_scratch_locked(device);
  if (rc == ATTNRES_OK && ATTNRES_ANYH_STAGED) rc = allow_staged_lds();
  return rc;
}

extern "C" void attnres_shutdown(void) {
  std::lock_guard<std::mutex> lock(g_ws_mu);
  for (int d = 0; d < kMaxDevices; ++d) {
    if (g_ws[d].base) {
      int prev = 0;
      (void)hipGetDevice(&prev);
      (void)hipSetDevice(d);
      (void)hipDeviceSynchronize();
      (void)hipFree(g_ws[d].base);
      if (g_ws[d].base_b) (void)hipFree(g_ws[d].base_b);
      if (g_ws[d].handoff) (void)hipEventDestroy(g_ws[d].handoff);
      (void)hipSetDevice(prev);
      g_ws[d] = DeviceWorkspace{};
    }
  }
}

extern "C" int attnres_device_status(int device) {
  if (device < 0 || device >= kMaxDevices) return ATTNRES_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_ws_mu);
  // The allocated workspace (frames A and B) and, once attnres_fwd_noalloc
  // has used it on this device, the static scratch; the flag is in the first.
  void *const bases[2][2] = {{g_ws[device].base, g_ws[device].base_b},
                             {g_scratch[device], nullptr}};
  if (!bases[0][0] && !bases[1][0]) return ATTNRES_OK;
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = hipSetDevice(device)) != hipSuccess) return hip_fail(e);
  e = hipDeviceSynchronize();
  int rc = ATTNRES_OK;
  for (const auto &frames : bases) {
    void *const base = frames[0];
    if (!base || e != hipSuccess) continue;
    unsigned flag = 0;
    e = hipMemcpy(&flag, static_cast<char *>(base) + kPartBytes, sizeof flag,
                  hipMemcpyDeviceToHost);
    if (e == hipSuccess && flag != 0) {
      // A wait gave up: parts of a token may disagree on the generation, so
      // restart every word, in both frames, at generation zero.
      e = hipMemset(base, 0, kWorkspaceBytes);
      if (e == hipSuccess && frames[1]) e = hipMemset(frames[1], 0, kPartBytes);
      if (e == hipSuccess) e = hipDeviceSynchronize();
      rc = ATTNRES_E_DEVICE_WAIT;
    }
  }
  (void)hipSetDevice(prev);
  if (e != hipSuccess) return hip_fail(e);
  return rc;
}

extern "C" int attnres_last_hip_error(void) { return g_last_hip.load(); }

extern "C" int attnres_debug_force_wait_failure(int enable) {
  g_force_wait_failure.store(enable != 0);
  return ATTNRES_OK;
}

extern "C" int attnres_debug_workspace_frames(int mode) {
  if (mode < -1 || mode > 256) return ATTNRES_E_SHAPE;
  g_frames_mode.store(mode);
  return ATTNRES_OK;
}

extern "C" int attnres_auto_path(int64_t T, int64_t H, int num_blocks) {
  using namespace attnres;
  if (T < 0 || T > kMaxTokens || H <= 0) return ATTNRES_E_SHAPE;
  if (H % kSeg != 0 || H > kMaxHidden) return ATTNRES_E_UNSUPPORTED;
  if (num_blocks < 0 || num_blocks > kMaxBlocks) return ATTNRES_E_NUM_BLOCKS;
  switch (auto_choice(T, H, num_blocks)) {
    case Kind::kSplit: return ATTNRES_PATH_SPLIT;
    case Kind::kRow: return ATTNRES_PATH_ROW;
    default: return ATTNRES_PATH_ANY_H;
  }
}
