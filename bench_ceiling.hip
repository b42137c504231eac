// Memory-traffic ceiling probes for bench.py (measurement only, not part of
// libattnres).  Each launch moves exactly the row traffic of an
// attention-residual call with hidden size 7168, in the row kernel's launch
// shape: one 448-lane workgroup per token, two 16-byte segments per lane at
// lane and lane + 448 (whole cache lines per instruction), 128-bit loads and
// stores.  The only arithmetic is an XOR fold that keeps every load live.
// The rate is what the access pattern reaches on the device, the reference
// point for the library's kernels.
//
// ceiling_mid: the mid-prefill call's own buffers and row roles.  bank is
// [T][8 rows], prefix, delta and out are [T][1 row]; per token the 8 bank rows,
// prefix and delta are read, out receives the XOR of all ten, prefix and bank
// slot 3 receive cur = prefix ^ delta.  Rows only read stream past the cache
// (non-temporal); with `cached`, prefix and slot 3, the two rows written back,
// are read through the cache, as the library's row kernel does for long
// calls.  All stores are non-temporal.
//
// ceiling_stream: generic mixes with every row of a token in one buffer, all
// accesses non-temporal:
//   src: element (t, r, h) at src[t * src_token_stride + r * 7168 + h], r < R
//   dst: element (t, w, h) at dst[t * dst_token_stride + w * 7168 + h], w < WD
//   in-place row k < WI of token t (source row k) receives
//       XOR of source rows k and R-1;
//   dst row w of token t receives XOR of all R source rows, rotated by w bits.
// With no writes at all, a lane whose XOR equals `never` (a value the caller
// picks so that it does not occur) would store it to dst[0]: the loads stay
// live without adding traffic.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowSegs = 896;  // 16-byte segments in a row of 7168 bf16
constexpr int kThreads = 448;
constexpr int kSpl = 2;
constexpr int kMidSlot = 3;    // the bank slot the mid-prefill call writes

__device__ __forceinline__ u32x4 ld(const u32x4 *p) { return __builtin_nontemporal_load(p); }
// Through the cache, as a raw buffer load: a distinct instruction, so the
// compiler cannot fold it with a non-temporal load of the same address in the
// other branch of a select (which would drop the non-temporal hint of both).
__device__ __forceinline__ u32x4 ld_cached(const u32x4 *row, int seg) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(row), 0, kRowSegs * 16, 0x00020000);
  return __builtin_amdgcn_raw_buffer_load_b128(r, seg * 16, 0, 0);
}
__device__ __forceinline__ void st(u32x4 *p, u32x4 v) { __builtin_nontemporal_store(v, p); }

__device__ __forceinline__ u32x4 rotl(u32x4 v, int s) {
  if (s == 0) return v;
  return (v << s) | (v >> (32 - s));
}

template <bool CACHED>
__global__ void __launch_bounds__(kThreads) mid_kernel(u32x4 *bank, u32x4 *prefix,
                                                       const u32x4 *delta, u32x4 *out) {
  const int64_t t = blockIdx.x;
  u32x4 *bk = bank + t * 8 * kRowSegs;
  u32x4 *pf = prefix + t * kRowSegs;
  const u32x4 *dl = delta + t * kRowSegs;
  u32x4 *o = out + t * kRowSegs;
  u32x4 x[10][kSpl];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int i = 0; i < kSpl; ++i) {
      const int seg = threadIdx.x + i * kThreads;
      if (CACHED && r == kMidSlot)
        x[r][i] = ld_cached(bk + r * kRowSegs, seg);
      else
        x[r][i] = ld(bk + r * kRowSegs + seg);
    }
#pragma unroll
  for (int i = 0; i < kSpl; ++i) {
    const int seg = threadIdx.x + i * kThreads;
    x[8][i] = CACHED ? ld_cached(pf, seg) : ld(pf + seg);
  }
#pragma unroll
  for (int i = 0; i < kSpl; ++i) x[9][i] = ld(dl + threadIdx.x + i * kThreads);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kSpl; ++i) {
    const int seg = threadIdx.x + i * kThreads;
    u32x4 acc = x[0][i];
#pragma unroll
    for (int r = 1; r < 10; ++r) acc ^= x[r][i];
    const u32x4 cur = x[8][i] ^ x[9][i];
    st(o + seg, acc);
    st(pf + seg, cur);
    st(bk + kMidSlot * kRowSegs + seg, cur);
  }
}

// The mid-prefill pattern of mid_kernel for any hidden size: nseg 16-byte
// segments per row, the library's any-H launch shape (blockDim.x lanes of
// SPL segments each, lane + i * blockDim.x, segments past the row end masked).
template <int SPL, bool CACHED>
__global__ void __launch_bounds__(512) mid_any_kernel(u32x4 *bank, u32x4 *prefix,
                                                      const u32x4 *delta, u32x4 *out, int nseg) {
  const int64_t t = blockIdx.x;
  u32x4 *bk = bank + t * 8 * nseg;
  u32x4 *pf = prefix + t * nseg;
  const u32x4 *dl = delta + t * nseg;
  u32x4 *o = out + t * nseg;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto ldc = [&](const u32x4 *row, int seg) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(row), 0, nseg * 16, 0x00020000);
    return __builtin_amdgcn_raw_buffer_load_b128(r, seg * 16, 0, 0);
  };
  u32x4 x[10][SPL];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int seg = threadIdx.x + i * blockDim.x;
      if (CACHED && r == kMidSlot)  // the buffer load masks the row end itself
        x[r][i] = ldc(bk + r * nseg, seg);
      else
        x[r][i] = seg < nseg ? ld(bk + r * nseg + seg) : zero;
    }
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int seg = threadIdx.x + i * blockDim.x;
    if (CACHED)
      x[8][i] = ldc(pf, seg);
    else
      x[8][i] = seg < nseg ? ld(pf + seg) : zero;
    x[9][i] = seg < nseg ? ld(dl + seg) : zero;
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int seg = threadIdx.x + i * blockDim.x;
    if (seg >= nseg) continue;
    u32x4 acc = x[0][i];
#pragma unroll
    for (int r = 1; r < 10; ++r) acc ^= x[r][i];
    const u32x4 cur = x[8][i] ^ x[9][i];
    st(o + seg, acc);
    st(pf + seg, cur);
    st(bk + kMidSlot * nseg + seg, cur);
  }
}

template <int R, int WD, int WI>
__global__ void __launch_bounds__(kThreads) ceiling_kernel(u32x4 *src, int64_t src_stride,
                                                           u32x4 *dst, int64_t dst_stride,
                                                           uint32_t never) {
  static_assert(WI <= R, "in-place rows must be source rows");
  const int64_t t = blockIdx.x;
  u32x4 *s = src + t * src_stride;
  u32x4 *d = dst + t * dst_stride;
  u32x4 x[R][kSpl];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < kSpl; ++i) x[r][i] = ld(s + r * kRowSegs + threadIdx.x + i * kThreads);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kSpl; ++i) {
    const int seg = threadIdx.x + i * kThreads;
    u32x4 acc = x[0][i];
#pragma unroll
    for (int r = 1; r < R; ++r) acc ^= x[r][i];
#pragma unroll
    for (int w = 0; w < WD; ++w) st(d + w * kRowSegs + seg, rotl(acc, w));
#pragma unroll
    for (int k = 0; k < WI; ++k) st(s + k * kRowSegs + seg, x[k][i] ^ x[R - 1][i]);
    if constexpr (WD == 0 && WI == 0) {
      if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == never) dst[0] = acc;
    }
  }
}

typedef void (*Fn)(u32x4 *, int64_t, u32x4 *, int64_t, uint32_t);

Fn pick(int reads, int wd, int wi) {
#define CEIL_CASE(R, D, I) \
  if (reads == R && wd == D && wi == I) return ceiling_kernel<R, D, I>;
  CEIL_CASE(10, 1, 2)  // mid prefill's row counts in one buffer
  CEIL_CASE(10, 3, 0)  // the same bytes, every write to a separate buffer
  CEIL_CASE(9, 1, 0)   // long prefill: 8 bank rows + prefix; out
  CEIL_CASE(10, 0, 0)  // reads only
  CEIL_CASE(1, 1, 0)   // copy
#undef CEIL_CASE
  return nullptr;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// The mid-prefill layout above.  Returns 0 on success, -1 for bad arguments,
// -2 if the launch failed.  Asynchronous on `stream`.
extern "C" int ceiling_mid(void *bank, void *prefix, const void *delta, void *out, int64_t T,
                           int cached, void *stream) {
  if (T < 0 || T > 0x7fffffff) return -1;
  if (T == 0) return 0;
  if (!bank || !prefix || !delta || !out) return -1;
  if (!aligned16(bank) || !aligned16(prefix) || !aligned16(delta) || !aligned16(out)) return -1;
  void *a_bank = bank, *a_prefix = prefix, *a_delta = const_cast<void *>(delta), *a_out = out;
  void *args[] = {&a_bank, &a_prefix, &a_delta, &a_out};
  const void *fn = cached ? reinterpret_cast<const void *>(mid_kernel<true>)
                          : reinterpret_cast<const void *>(mid_kernel<false>);
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(T)), dim3(kThreads), args, 0,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -2;
}

// Returns 0 on success, -1 for an unsupported (reads, writes) combination or
// bad sizes / alignment, -2 if the launch failed.  Asynchronous on `stream`.
// dst must hold at least 16 bytes even when dst_writes == 0.
extern "C" int ceiling_stream(void *src, int64_t src_token_stride, void *dst,
                              int64_t dst_token_stride, int reads, int dst_writes,
                              int inplace_writes, int64_t T, uint32_t never, void *stream) {
  Fn fn = pick(reads, dst_writes, inplace_writes);
  if (!fn || T < 0 || T > 0x7fffffff) return -1;
  if (T == 0) return 0;
  if (!src || !dst) return -1;
  if (!aligned16(src) || !aligned16(dst)) return -1;
  if (src_token_stride % 8 != 0 || dst_token_stride % 8 != 0) return -1;
  if (src_token_stride < int64_t(reads) * 7168 ||
      (dst_writes > 0 && dst_token_stride < int64_t(dst_writes) * 7168))
    return -1;
  void *args_src = src;
  void *args_dst = dst;
  int64_t ss = src_token_stride / 8, ds = dst_token_stride / 8;  // in 16-byte segments
  void *args[] = {&args_src, &ss, &args_dst, &ds, &never};
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(unsigned(T)),
                                 dim3(kThreads), args, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -2;
}

// The mid-prefill layout at hidden size H (a multiple of 8, at most 16384),
// `threads` lanes per workgroup (a multiple of 64, at most 512) with two (H
// up to 8192) or four segments per lane covering the row.  Returns 0 on
// success, -1 for bad arguments, -2 if the launch failed.
extern "C" int ceiling_mid_h(void *bank, void *prefix, const void *delta, void *out, int64_t T,
                             int64_t H, int threads, int cached, void *stream) {
  if (T < 0 || T > 0x7fffffff || H <= 0 || H % 8 != 0 || H > 16384) return -1;
  if (threads <= 0 || threads > 512 || threads % 64 != 0) return -1;
  if (T == 0) return 0;
  if (!bank || !prefix || !delta || !out) return -1;
  if (!aligned16(bank) || !aligned16(prefix) || !aligned16(delta) || !aligned16(out)) return -1;
  int nseg = int(H / 8);
  const int spl = nseg <= 1024 ? 2 : 4;
  if (int64_t(threads) * spl < nseg) return -1;
  void *a_bank = bank, *a_prefix = prefix, *a_delta = const_cast<void *>(delta), *a_out = out;
  void *args[] = {&a_bank, &a_prefix, &a_delta, &a_out, &nseg};
  const void *fn =
      spl == 2 ? (cached ? reinterpret_cast<const void *>(mid_any_kernel<2, true>)
                         : reinterpret_cast<const void *>(mid_any_kernel<2, false>))
               : (cached ? reinterpret_cast<const void *>(mid_any_kernel<4, true>)
                         : reinterpret_cast<const void *>(mid_any_kernel<4, false>));
  hipError_t e = hipLaunchKernel(fn, dim3(unsigned(T)), dim3(unsigned(threads)), args, 0,
                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? 0 : -2;
}
