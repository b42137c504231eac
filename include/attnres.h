/*
 * attnres.h -- C ABI of libattnres: the Kimi-K3 attention-residual (AttnRes)
 * forward on AMD MI355X (gfx950).
 *
 * The operation (defined by the vllm-ascend PR #14840 page, author's
 * "Implementation walkthrough", and the prhub digest of vLLM PR #54261,
 * "Implementation breakdown" items 1-3 and the kernel snippet under "Key
 * source snippets"):
 *
 *   for every token t:
 *     cur      = delta ? bf16_RNE(prefix[t] + delta[t]) : prefix[t]
 *     sources  = blocks[t, 0], ..., blocks[t, num_blocks-1], cur
 *     q        = rms_w * res_w                      (fused query, PR #50185)
 *     logit_j  = sum_h q[h] * x_j[h] / sqrt(mean_h(x_j^2) + rms_eps)
 *     p        = softmax(logit)                     (over the num_blocks+1 sources)
 *     y        = sum_j p_j * x_j                    (raw rows)
 *     out[t]   = bf16_RNE(output_norm_weight
 *                  ? y / sqrt(mean_h(y^2) + output_norm_eps) * output_norm_weight
 *                  : y)
 *     if delta:               prefix[t] = cur                     (in place)
 *     if block_write_idx>=0:  blocks[t, block_write_idx] = cur    (in place)
 *
 * With num_blocks == 0 the only source, cur, has weight exactly 1 (y = cur),
 * also when its logit is not a number (rms_eps = 0 and an all-zero row).
 *
 * All reads see the state before the call (a written slot that is also a
 * source contributes its old value).  Bank slots num_blocks..max_blocks-1 are
 * never read, and nothing but out, prefix (with a delta) and the one bank row
 * per token is ever written; with strided rows, the elements between rows are
 * neither read nor written.
 *
 * Hidden size: any H that is a multiple of 8, up to ATTNRES_MAX_HIDDEN.  H =
 * 7168 (Kimi-K3) runs on tuned kernels; other sizes on one any-H row kernel,
 * and above 7168 small batches also on the split kernel.
 *
 * Tensors are bf16 (passed as raw 16-bit patterns) in device memory.  The
 * library keeps no pointer after a call returns; the caller owns every buffer
 * and keeps it alive until the stream work completes.  Arithmetic is fp32:
 * inputs must be finite, and a row's sum of squares must stay within fp32's
 * range (at H = 7168, an RMS below about 2e17), or it overflows.
 *
 * Errors: every entry point returns ATTNRES_OK (0) or a negative code.  All
 * argument checks run on the host before any GPU work, so a rejected call
 * launches nothing and touches no buffer.
 */
#ifndef ATTNRES_H
#define ATTNRES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define ATTNRES_OK 0
#define ATTNRES_E_NULL -1        /* a required pointer is NULL */
#define ATTNRES_E_SHAPE -2       /* T < 0 or > 8388607, H <= 0, max_blocks < 0, or sizes too large */
#define ATTNRES_E_UNSUPPORTED -3 /* H not a multiple of 8 or > ATTNRES_MAX_HIDDEN, or a forced
                                    path that cannot run these sizes */
#define ATTNRES_E_NUM_BLOCKS -4  /* num_blocks < 0, > 8 or > max_blocks */
#define ATTNRES_E_WRITE_IDX -5   /* block_write_idx < -1 or >= max_blocks */
#define ATTNRES_E_ALIGN -6       /* a pointer not 16-byte aligned, or a stride not a multiple of 8 */
#define ATTNRES_E_STRIDE -7      /* a negative stride, or rows of one argument that overlap */
#define ATTNRES_E_ALIAS -8       /* a written buffer overlaps another argument */
#define ATTNRES_E_EPS -9         /* an epsilon that is negative or not finite */
#define ATTNRES_E_NOT_INIT -10   /* the split path needs attnres_init() first (stream is capturing) */
#define ATTNRES_E_HIP -11        /* a HIP call failed; see attnres_last_hip_error() */
#define ATTNRES_E_PATH -12       /* unknown path selector */
#define ATTNRES_E_DEVICE_WAIT -13 /* a split-path cross-workgroup wait gave up (device flag) */

/* ---- path selectors for attnres_fwd_path -------------------------------- */
#define ATTNRES_PATH_AUTO 0  /* what attnres_fwd does: at H = 7168 split for T up to
                                -/40/40/48/56/56/52/60/56 with 0..8 blocks (never with
                                0 blocks), else row; elsewhere the any-H kernel,
                                except split with 1..8 blocks for T up to 72 above
                                H = 8192, 16/24/32/40/32/32/32/40 from 7176 to 8192,
                                8/16/24/40/40/48/48/48 from 4104 to 7160, 8 with 7
                                blocks and 16 with 8 at 4096, and 8 with 8 blocks
                                from 3080 to 4088 */
#define ATTNRES_PATH_ROW 1   /* one workgroup per token (the any-H kernel when H != 7168) */
#define ATTNRES_PATH_SPLIT 2 /* hidden dim split over 14 workgroups per token (any H,
                                T <= 256) */
#define ATTNRES_PATH_ANY_H 3 /* the any-H row kernel, also at H = 7168 */

/* Largest T the split path accepts (its per-device workspace). */
#define ATTNRES_SPLIT_MAX_TOKENS 256
/* Largest hidden size (a multiple of 8). */
#define ATTNRES_MAX_HIDDEN 16384

/*
 * attnres_fwd -- the forward above, enqueued on `stream`.
 *
 *   prefix   [T, H] bf16, row stride H, device.  Read; overwritten with cur
 *            when delta != NULL.
 *   delta    [T, H] bf16, row stride H, device, or NULL (no delta).
 *   blocks   the block bank: element (t, i, h) at
 *            blocks[t*block_token_stride + i*block_slot_stride + h], for
 *            i < max_blocks.  Strides in elements, >= 0, multiples of 8, rows
 *            must not overlap.  May be NULL only when num_blocks == 0 and
 *            block_write_idx == -1.  Slots 0..num_blocks-1 are the sources;
 *            slot block_write_idx (if >= 0) receives cur.
 *   max_blocks   bank capacity (slots per token); num_blocks <= max_blocks.
 *   num_blocks   valid slots, 0..8.
 *   res_w, rms_w [H] bf16, device: scoring projection and RMSNorm weight.
 *   rms_eps      >= 0, finite.
 *   output_norm_weight [H] bf16, device, or NULL = no output norm.
 *   output_norm_eps    >= 0, finite (ignored without an output norm).
 *   block_write_idx    -1 = no bank write, else 0..max_blocks-1.
 *   out      [T, H] bf16, row stride H, device; must not overlap any input.
 *   T, H     tokens (0..8388607; T == 0 is a no-op: a dispatch counts its
 *            lanes in 32 bits and a token takes at most 512) and hidden size
 *            (a multiple of 8, at most ATTNRES_MAX_HIDDEN).
 *   stream   a hipStream_t (NULL = the default stream of the current
 *            device).  Kernels run on the stream's device, and the split
 *            path uses that device's workspace, whichever device is current.
 *
 * All device pointers must be 16-byte aligned.  Asynchronous: returns after
 * enqueueing.  No allocation or host synchronisation happens once the split
 * path's workspace exists (attnres_init, or the first uncaptured call that
 * needs it), so calls can be captured into a hipGraph.  Calls that use the
 * split path share one workspace per device and run one after another: when
 * one comes on a different stream than the previous split call on that
 * device, its stream first waits for the work enqueued on the previous stream
 * (so that stream must still exist).  Inside graph capture no such wait is
 * added: replays of graphs holding split calls must not overlap each other or
 * other split calls on the device.  The ordering is per process: split calls
 * of two processes running on one GPU at the same time can fill the compute
 * units with waiting workgroups; the bounded wait then gives up and
 * attnres_device_status reports ATTNRES_E_DEVICE_WAIT (the results of those
 * calls are not valid).
 */
int attnres_fwd(void *prefix, const void *delta, void *blocks,
                int64_t block_token_stride, int64_t block_slot_stride,
                int max_blocks, int num_blocks,
                const void *res_w, const void *rms_w, float rms_eps,
                const void *output_norm_weight, float output_norm_eps,
                int block_write_idx, void *out, int64_t T, int64_t H,
                void *stream);

/* attnres_fwd with an explicit path (ATTNRES_PATH_*); all paths compute the
 * same result within the fp32 rounding of their reduction orders. */
int attnres_fwd_path(void *prefix, const void *delta, void *blocks,
                     int64_t block_token_stride, int64_t block_slot_stride,
                     int max_blocks, int num_blocks,
                     const void *res_w, const void *rms_w, float rms_eps,
                     const void *output_norm_weight, float output_norm_eps,
                     int block_write_idx, void *out, int64_t T, int64_t H,
                     void *stream, int path);

/*
 * attnres_fwd_path with row strides for prefix, delta and out (in elements),
 * e.g. views into wider activation buffers.  The reference dispatch gate (prhub
 * digest of vLLM PR #54261, the attn_res.py snippet under "Key source
 * snippets") sends hidden sizes other than 7168 and non-dense rows to a Triton
 * fallback, and the code review on the vllm-ascend PR #14840 page asks for
 * masked accesses when H is not a power of two; here both run natively.  Each stride must be >= H and a
 * multiple of 8 when T > 1 (it is ignored when T <= 1); the elements between
 * rows are never touched.  A written buffer must not share any element with
 * another argument: row sets with equal strides are checked exactly (so
 * interleaved rows of one wider buffer are accepted), other combinations by
 * the address spans they cover.
 */
int attnres_fwd_strided(void *prefix, int64_t prefix_stride,
                        const void *delta, int64_t delta_stride, void *blocks,
                        int64_t block_token_stride, int64_t block_slot_stride,
                        int max_blocks, int num_blocks,
                        const void *res_w, const void *rms_w, float rms_eps,
                        const void *output_norm_weight, float output_norm_eps,
                        int block_write_idx, void *out, int64_t out_stride,
                        int64_t T, int64_t H, void *stream, int path);

/*
 * attnres_fwd_noalloc -- attnres_fwd_strided for callers that cannot allocate
 * device memory: code under hipGraph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and checks as
 * attnres_fwd_strided; it never calls hipMalloc, hipFree or any allocating
 * routine.  The only kernel that needs memory beyond the arguments is the
 * split path's (its cross-workgroup exchange words and fault flag).  This
 * entry point gives it a static device array of 1,835,264 bytes per device
 * (ATTNRES_SPLIT_MAX_TOKENS tokens), held until the process ends, instead of
 * the allocated workspace (one frame: without the allocated workspace's
 * choice of the frame nearer each XCD).  A split-path call of more than
 * ATTNRES_SPLIT_MAX_TOKENS tokens is rejected with ATTNRES_E_UNSUPPORTED
 * before any GPU work.  The array's device address is taken, and the array
 * cleared, once per device: in attnres_init(device), or else at the first
 * split-path call on that device outside graph capture (a call that needs it
 * inside capture before that returns ATTNRES_E_NOT_INIT).  Nothing needs
 * clearing between calls: the exchange words carry their own generation tags,
 * and attnres_device_status reads and clears this array's fault flag too.
 * Every call on a device shares that device's array, and calls are not
 * ordered against each other: split-path calls that overlap on one GPU race
 * (their results are not valid, and the bounded wait may give up).
 */
int attnres_fwd_noalloc(void *prefix, int64_t prefix_stride,
                        const void *delta, int64_t delta_stride, void *blocks,
                        int64_t block_token_stride, int64_t block_slot_stride,
                        int max_blocks, int num_blocks,
                        const void *res_w, const void *rms_w, float rms_eps,
                        const void *output_norm_weight, float output_norm_eps,
                        int block_write_idx, void *out, int64_t out_stride,
                        int64_t T, int64_t H, void *stream, int path);

/*
 * Two-kernel form of attnres_fwd_strided, so that the part of the work that
 * does not depend on delta can run before delta exists.  The prhub digest of
 * vLLM PR #54261 ("Implementation breakdown" and the kernel under "Key source
 * snippets") describes the reference kernel's programmatic dependent launch:
 * it issues its bank-row copies before waiting on delta's producer, and waits
 * only before the first copy that needs the producer's output (the prefix/delta
 * row).  HIP has no dependent launch, so the work is split in two kernels that
 * a hipGraph (or two streams) can place beside the producer:
 *
 *   attnres_fwd_bank  reads only the bank rows 0..num_blocks-1 and the scoring
 *                     weights: their logits, the online softmax state (m, s) of
 *                     those logits, and the unnormalised mixture
 *                     u = sum_j exp(l_j - m) x_j (fp32), into `partial`;
 *   attnres_fwd_cur   forms cur = prefix (+ delta), its logit, merges it into
 *                     (m, s) as one more online-softmax step, applies the
 *                     output norm and does every store of attnres_fwd.
 *
 * Results equal attnres_fwd's within the fp32 rounding of a different order.
 * Both take attnres_fwd_strided's arguments (pass the same values to both; each
 * call validates them as attnres_fwd_strided would), plus `partial`: device
 * memory of at least attnres_partial_bytes(T, H) bytes, 16-byte aligned, owned
 * by the caller and not overlapping any argument (ATTNRES_E_NULL,
 * ATTNRES_E_ALIGN, ATTNRES_E_SHAPE for too small, ATTNRES_E_ALIAS).  It may be
 * NULL when num_blocks == 0 (attnres_fwd_bank then launches nothing).  The
 * caller orders attnres_fwd_cur after attnres_fwd_bank of the same call, and
 * the next call's attnres_fwd_bank after this call's attnres_fwd_cur when the
 * two share `partial` or bank rows.  attnres_fwd_bank writes only `partial`.
 * Layout of `partial`: u as fp32 [T, H], then (m, s) as two fp32 per token.
 * Neither kernel allocates memory or uses the split path's workspace, so both
 * can be captured into a hipGraph.
 */
int64_t attnres_partial_bytes(int64_t T, int64_t H);  /* < 0: an error code */
int attnres_fwd_bank(const void *prefix, int64_t prefix_stride,
                     const void *delta, int64_t delta_stride, const void *blocks,
                     int64_t block_token_stride, int64_t block_slot_stride,
                     int max_blocks, int num_blocks,
                     const void *res_w, const void *rms_w, float rms_eps,
                     const void *output_norm_weight, float output_norm_eps,
                     int block_write_idx, const void *out, int64_t out_stride,
                     int64_t T, int64_t H, void *partial, int64_t partial_bytes,
                     void *stream);
int attnres_fwd_cur(void *prefix, int64_t prefix_stride,
                    const void *delta, int64_t delta_stride, void *blocks,
                    int64_t block_token_stride, int64_t block_slot_stride,
                    int max_blocks, int num_blocks,
                    const void *res_w, const void *rms_w, float rms_eps,
                    const void *output_norm_weight, float output_norm_eps,
                    int block_write_idx, void *out, int64_t out_stride,
                    int64_t T, int64_t H, const void *partial, int64_t partial_bytes,
                    void *stream);

/* The host-side argument checks of attnres_fwd, alone.  Makes no HIP call and
 * dereferences no pointer, so it runs without a GPU. */
int attnres_validate(const void *prefix, const void *delta, const void *blocks,
                     int64_t block_token_stride, int64_t block_slot_stride,
                     int max_blocks, int num_blocks,
                     const void *res_w, const void *rms_w, float rms_eps,
                     const void *output_norm_weight, float output_norm_eps,
                     int block_write_idx, const void *out, int64_t T, int64_t H);

/* The host-side argument checks of attnres_fwd_strided, alone (no HIP call). */
int attnres_validate_strided(const void *prefix, int64_t prefix_stride,
                             const void *delta, int64_t delta_stride, const void *blocks,
                             int64_t block_token_stride, int64_t block_slot_stride,
                             int max_blocks, int num_blocks,
                             const void *res_w, const void *rms_w, float rms_eps,
                             const void *output_norm_weight, float output_norm_eps,
                             int block_write_idx, const void *out, int64_t out_stride,
                             int64_t T, int64_t H);

/* Allocates and clears the split path's workspace on `device`: tagged
 * partial-sum words and a fault flag, in two 2 MB frames (4 MB).  It tries
 * four 2 MB allocations, times a device-scope store and load to each from
 * every XCD with one short kernel (64 single-wave workgroups, synchronous),
 * keeps the pair that best serves all XCDs and frees the other two: a store
 * to a frame homed on the writer's half of the chip is acknowledged about
 * twice as fast, and the split path's workgroups write and poll the nearer
 * frame (reading both if their partners' words are not there).  It also takes the address of (and clears)
 * attnres_fwd_noalloc's static array there.  It also lets the any-H
 * kernels that stage bank rows in LDS (H = 8200..12288) take their 61-72 KB of
 * dynamic LDS, which a call would otherwise set up at its first use.
 * Idempotent.  Call it outside stream capture. */
int attnres_init(int device);

/* Frees every device's workspace.  No call may be in flight. */
void attnres_shutdown(void);

/* Reads (synchronously) and clears the split path's device fault flags on
 * `device` (the allocated workspace's and attnres_fwd_noalloc's):
 * ATTNRES_E_DEVICE_WAIT if a cross-workgroup wait ever gave up since the last
 * check (the exchange words are then reset), else ATTNRES_OK. */
int attnres_device_status(int device);

/* Static description of a status code. */
const char *attnres_strerror(int status);

/* The hipError_t of the last failed HIP call in this library (0 if none). */
int attnres_last_hip_error(void);

/* For tests of the failure path only.  While enabled (enable != 0), every
 * split-path call of this process waits for a generation of the exchanged
 * words that never comes, gives up after 64 polls and raises the device flag
 * that attnres_device_status reports; the results of those calls are not
 * valid.  Every kernel still exits.  Disabled by default; returns ATTNRES_OK. */
int attnres_debug_force_wait_failure(int enable);

/* For tests only.  Which of the split path's two workspace frames each
 * workgroup writes.  A workgroup polls the frame it writes and, after 16
 * polls, both, so the choice may change speed but not results: mode -1 (the
 * default) follows the set-up timing by the workgroup's XCD; 0..255 is a
 * mask with one bit per XCD (set: frame B); 256 writes frame B from the odd
 * parts of a token and frame A from the even ones.
 * Affects calls made after it, in this process.  Returns ATTNRES_OK, or
 * ATTNRES_E_SHAPE for another mode. */
int attnres_debug_workspace_frames(int mode);

/* The kernel attnres_fwd (ATTNRES_PATH_AUTO) runs for a call of T tokens,
 * hidden size H and num_blocks block rows: ATTNRES_PATH_ROW (the tuned row
 * kernel, H = 7168), ATTNRES_PATH_SPLIT or ATTNRES_PATH_ANY_H; or
 * ATTNRES_E_SHAPE, ATTNRES_E_UNSUPPORTED or ATTNRES_E_NUM_BLOCKS for sizes
 * attnres_fwd rejects.  Host only: makes no HIP call. */
int attnres_auto_path(int64_t T, int64_t H, int num_blocks);

#ifdef __cplusplus
}
#endif

#endif /* ATTNRES_H */
