/*
 * dcconv.h -- C ABI of the MI355X (gfx950) depthwise causal conv1d library.
 *
 * The operation is the decode update described on the cuDNN FE-OSS page
 * "Causal Conv1d Decode Update" (docs.nvidia.com/cudnn/latest/fe-oss-apis/
 * causal_conv1d_update): for every decode row n, channel d and the cache slot s
 * the row selects,
 *
 *     history            = concat(conv_state[s, d, :], x[n, d])      (length L+1)
 *     conv_state[s, d, :] = newest L values of history
 *     out[n, d]          = act(sum_j history[L+1-W+j] * weight[d, j] + bias[d])
 *
 * (page section "Causal Conv1d Decode Update").  Sums are formed in FP32 and
 * rounded once to BF16 (round to nearest even).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP device memory or memory the
 *    device can address), except where a comment says otherwise.
 *  - The caller owns every buffer.  The library allocates nothing, never
 *    synchronises, never reads device memory from the host and converts nothing,
 *    so a call may be captured into a HIP graph (stable pointers).
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and is
 *    asynchronous; results are visible after the stream is synchronised.
 *  - Metadata is validated on the host, in full, before anything is enqueued.
 *    A non-zero return means nothing was enqueued; dcconv_last_error() then
 *    describes the problem (thread-local, valid until the next call on the same
 *    thread).
 *  - Elements are BF16 carried as 16-bit patterns; indices are int32.
 */
#ifndef DCCONV_H
#define DCCONV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DCCONV_ABI_VERSION 1

/* Return codes.  The page distinguishes a contract violation (Python ValueError)
 * from a valid request the implementation does not serve (NotImplementedError);
 * section "Current native implementation". */
enum {
    DCCONV_OK = 0,
    DCCONV_EINVAL = 1,       /* contract violation: shape, stride, alignment, overlap, null */
    DCCONV_EUNSUPPORTED = 2, /* semantically valid but not served (e.g. W != 4) */
    DCCONV_EHIP = 3          /* the HIP runtime refused the launch (hipGetLastError) */
};

/* Activations (page section "Causal Conv1d Decode Update": None/"identity" and
 * "silu"/"swish").  Each is a separate compiled kernel; the identity kernel
 * contains no activation code. */
enum { DCCONV_ACT_IDENTITY = 0, DCCONV_ACT_SILU = 1 };

/* Bits OR-ed into *dev_status by the device when a routing entry is rejected. */
enum {
    DCCONV_DEV_BAD_INDEX = 1, /* an index below -1, or not below S           */
    DCCONV_DEV_DUP_INDEX = 2, /* two rows of the batch select one real slot  */
    DCCONV_DEV_BAD_SEQ = 4,   /* dcconv_prefill: seq_starts is not 0 = starts[0]
                                 <= starts[1] <= ... <= starts[n] = t          */
    DCCONV_DEV_BAD_SEQLEN = 8 /* dcconv_update, dcconv_update_tokens: a
                                 cache_seqlens entry below 0                  */
};

/* The DCCONV_ABI_VERSION the library was built with. */
int dcconv_abi_version(void);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char *dcconv_last_error(void);

/* Name of the kernel specialisation the last successful call on the calling
 * thread enqueued ("" if that call enqueued nothing).  Lets a benchmark prove
 * which route ran. */
const char *dcconv_last_kernel(void);

/*
 * dcconv_update -- one decode step, in place.
 * Defined by the page section "Causal Conv1d Decode Update" (update rule, bias
 * default, activations, slot routing, padding rows) and section "Semantic tensor
 * contract" (shapes, strides, alignment); the limits of the served subset follow
 * section "Current native implementation".
 *
 * x           BF16 [n, d], element (r, c) at x[r*ld_x + c].  ld_x == d, or
 *             ld_x > d with ld_x % 8 == 0 (16-byte aligned rows).  Columns
 *             d..ld_x-1 are never read.
 * n           decode rows, n >= 0.  n == 0 returns DCCONV_OK and enqueues nothing.
 * d           channels, d >= 1.
 * conv_state  BF16 [s, d, l], READ AND WRITTEN.  Element (slot, c, k) at
 *             conv_state[slot*st_s + c*st_d + k*st_l]; k = 0 is the oldest value.
 *             Accepted layouts: compact (st_d == l, st_l == 1, st_s >= d*l) and
 *             channel-last (st_d == 1, st_l == d, st_s >= l*d; the layout a
 *             full-sequence prefill hands over).
 * s           slots, s >= 0; without an index table s >= n (row r uses slot r).
 *             With s == 0 every row must be padding and conv_state may be NULL.
 * l           history length, l >= w - 1.
 * weight      BF16 [d, w] contiguous.  Only w == 4 is served.
 * bias        BF16 [d] or NULL (zero bias).
 * conv_state_indices  int32 [n] or NULL.  Row r uses slot conv_state_indices[r];
 *             -1 marks a padding row: its output is zero and no slot changes
 *             (repeated -1 is allowed).  Other values must lie in [0, s) and be
 *             unique within the call.  An entry below -1 or >= s makes that row
 *             behave as a padding row and sets DCCONV_DEV_BAD_INDEX.  When
 *             dev_status is non-NULL every row whose slot is shared with another
 *             row is also treated as padding (so that slot is left untouched)
 *             and DCCONV_DEV_DUP_INDEX is set; when dev_status is NULL duplicates
 *             are not detected and the result for the shared slot is unspecified
 *             (the page calls such an update "not transactional").
 * cache_seqlens  NULL, or int32 [n]: circular-buffer state, the use the page
 *             reserves this keyword for (section "Causal Conv1d Decode Update").
 *             c = cache_seqlens[r] is the number of tokens row r's slot has seen;
 *             the slot keeps token i at position i mod l (k is then a ring
 *             position, not an age).  The taps are tokens c-3, c-2, c-1, read at
 *             positions (c-3+k) mod l before any write, and x; x then replaces
 *             the oldest token at position c mod l, and no other value moves
 *             (one element per channel is written).  cache_seqlens is only read
 *             (the caller advances it).  An entry below 0 makes the row behave
 *             as padding and sets DCCONV_DEV_BAD_SEQLEN.  Read-only; 4-byte
 *             aligned; must not overlap anything the call writes.
 * activation  DCCONV_ACT_IDENTITY or DCCONV_ACT_SILU (SiLU(v) = v / (1 + e^-v)).
 * out         BF16 [n, d] contiguous, written.  Must not overlap any operand.
 * dev_status  NULL, or a device int32 the kernel ORs DCCONV_DEV_* bits into.
 *             It is never cleared by the library.
 * stream      hipStream_t to enqueue on; NULL = null stream.
 *
 * Alignment: every BF16 pointer 16-byte aligned, indices and dev_status 4-byte
 * aligned (page section "Current native implementation").  conv_state must not
 * overlap x, weight, bias, the index table, out or dev_status.
 *
 * Returns DCCONV_OK, DCCONV_EINVAL (contract violation), DCCONV_EUNSUPPORTED
 * (valid but not served), or DCCONV_EHIP (launch refused by the runtime).
 */
int dcconv_update(const void *x, int64_t n, int64_t d, int64_t ld_x,
                  void *conv_state, int64_t s, int64_t l,
                  int64_t st_s, int64_t st_d, int64_t st_l,
                  const void *weight, int64_t w,
                  const void *bias,
                  const int32_t *conv_state_indices,
                  const int32_t *cache_seqlens,
                  int activation,
                  void *out,
                  int32_t *dev_status,
                  void *stream);

/*
 * dcconv_update_tokens -- T successive decode steps on the same slots, in place.
 * The multi-token form the page reserves for x[N, D, Tstep] (section "Semantic
 * tensor contract": the state and weight meanings do not change): token t of
 * every row is applied, in order t = 0..T-1, by exactly the rule of
 * dcconv_update, and out[:, :, t] is that step's output.  One call reads and
 * writes each selected state once instead of T times.
 *
 * x           BF16, element (r, c, t) at x[r*xs_n + c*xs_d + t*xs_t]; strides >= 0.
 * n, d, t     rows, channels, tokens (t == 0 or n == 0: DCCONV_OK, nothing enqueued).
 * out         BF16, element (r, c, t) at out[r*os_n + c*os_d + t*os_t]; the strides
 *             must give every element its own address (no two (r, c, t) alias).
 * cache_seqlens  NULL, or int32 [n]: circular-buffer state as for
 * dcconv_update; token t of row r is the (cache_seqlens[r] + t)-th token its
 * slot sees: its taps are tokens c+t-3 .. c+t-1 (from the ring for the first
 * three, from x after that) and it lands at position (c + t) mod l.  Only the
 * last min(t, l) tokens remain in the ring; the count is only read.
 * conv_state, s, l, st_*, weight, w, bias, conv_state_indices,
 * activation, dev_status, stream: exactly as for dcconv_update (the routing of a
 * row is the same for all of its tokens; a padding or rejected row writes zeros
 * for every token and leaves the state untouched).
 *
 * Alignment: x, out and the other BF16 pointers 16-byte aligned.  The fast path
 * additionally needs unit channel strides and row/token strides that are
 * multiples of 8 elements; other strides are served by a per-element path.
 * Nothing the call writes may overlap any other operand.
 *
 * Returns DCCONV_OK, DCCONV_EINVAL, DCCONV_EUNSUPPORTED or DCCONV_EHIP, with the
 * same meanings as for dcconv_update.
 */
int dcconv_update_tokens(const void *x, int64_t n, int64_t d, int64_t t,
                         int64_t xs_n, int64_t xs_d, int64_t xs_t,
                         void *conv_state, int64_t s, int64_t l,
                         int64_t st_s, int64_t st_d, int64_t st_l,
                         const void *weight, int64_t w,
                         const void *bias,
                         const int32_t *conv_state_indices,
                         const int32_t *cache_seqlens,
                         int activation,
                         void *out, int64_t os_n, int64_t os_d, int64_t os_t,
                         int32_t *dev_status,
                         void *stream);

/*
 * dcconv_prefill -- full-sequence causal convolution (prefill), returning the
 * final state that dcconv_update continues.
 *
 * The decode page names this operation at its top (cudnn.ops.causal_conv1d, for
 * full sequences; its width-four final state is handed to the update, section
 * "Semantic tensor contract": an L=3 state from prefill is accepted in place).
 * Its own page is not among the sources; this follows the plainest reading the
 * decode page supports.  For sequence i (slot s) and channel c:
 *
 *     ext          = concat(init[0:L], x[i, c, 0:T_i])     init = slot s's state or zeros
 *     out[i, c, j] = act(sum_k ext[L + j - 3 + k] * weight[c, k] + bias[c])
 *     slot s       = ext[T_i : T_i + L]                     (the newest L values)
 *
 * Sequences -- two forms:
 *   seq_starts == NULL  n sequences of t tokens each; token j of sequence i,
 *                       channel c at x[i*xs_n + c*xs_d + j*xs_t] (out likewise).
 *   seq_starts != NULL  device int32 [n+1], 0 = starts[0] <= ... <= starts[n] = t:
 *                       sequence i is packed tokens starts[i] .. starts[i+1]-1,
 *                       token p at x[c*xs_d + p*xs_t]; xs_n and os_n are unused.
 *                       A table that breaks the ordering sets DCCONV_DEV_BAD_SEQ
 *                       in *dev_status; outputs and states are then unspecified
 *                       (every access still stays inside the operands).
 * State:
 *   conv_state == NULL  no initial and no final state (history starts at zero);
 *                       s must be 0, conv_state_indices and has_initial_state
 *                       NULL; l and st_* are ignored.
 *   conv_state != NULL  [s, d, l] at strides (st_s, st_d, st_l), compact or
 *                       channel-last as for dcconv_update (channel-last l = 3 is
 *                       the hand-off layout).  Sequence i uses slot
 *                       conv_state_indices[i] (or i); -1 is a padding sequence:
 *                       zero outputs, no slot touched; bad and duplicate indices
 *                       as for dcconv_update.  The final state replaces the slot.
 *   has_initial_state   device uint8 [n] or NULL.  Nonzero: sequence i continues
 *                       from its slot's state; zero or NULL: from zeros.
 * x, out           BF16 at element strides >= 0; out must give every element its
 *                  own address.  16-byte aligned; seq_starts 4-byte aligned.
 *                  Nothing the call writes may overlap any other operand.
 * weight, w, bias, activation, dev_status, stream: as for dcconv_update.
 *
 * t == 0 (or every sequence empty) still writes the final states (the initial
 * state unchanged, or zeros).  n == 0: DCCONV_OK, nothing enqueued.
 * The fast path needs d % 8 == 0, unit channel strides, token and row strides
 * that are multiples of 8 and 3 <= l <= 8; other shapes take a per-element path.
 *
 * Returns DCCONV_OK, DCCONV_EINVAL, DCCONV_EUNSUPPORTED or DCCONV_EHIP, with the
 * same meanings as for dcconv_update.
 */
int dcconv_prefill(const void *x, int64_t n, int64_t d, int64_t t,
                   int64_t xs_n, int64_t xs_d, int64_t xs_t,
                   const int32_t *seq_starts,
                   void *conv_state, int64_t s, int64_t l,
                   int64_t st_s, int64_t st_d, int64_t st_l,
                   const int32_t *conv_state_indices,
                   const uint8_t *has_initial_state,
                   const void *weight, int64_t w,
                   const void *bias,
                   int activation,
                   void *out, int64_t os_n, int64_t os_d, int64_t os_t,
                   int32_t *dev_status,
                   void *stream);

/*
 * dcconv_stream_copy -- measurement control, not part of the operation.
 * The page "Composing multi-kernel blocks in Python" (section "Measuring a block
 * honestly") asks for a plain baseline timed in the same run as the block it
 * judges.  This copies `bytes` bytes from src to dst with the access pattern of
 * the update kernels (coalesced 16-byte non-temporal loads and stores, about
 * 2048 wavefronts for 16 MiB), so a benchmark can time what moving the update's
 * bytes costs with no arithmetic at all.
 *
 * dst, src  device pointers, 16-byte aligned, not overlapping.  The caller owns
 *           both; dst is written, src only read.
 * bytes     a multiple of 16, 0 <= bytes <= 2^47.  0 returns DCCONV_OK and
 *           enqueues nothing.
 * stream    hipStream_t (NULL = the null stream); asynchronous like every call.
 *
 * Returns DCCONV_OK, DCCONV_EINVAL (negative, unaligned or overlapping
 * arguments, or a size not a multiple of 16) or DCCONV_EHIP.
 */
int dcconv_stream_copy(void *dst, const void *src, int64_t bytes, void *stream);

/*
 * dcconv_busy_spin -- measurement control, not part of the operation.
 * Enqueues a kernel that keeps every SIMD of the current device busy with FP32
 * arithmetic for about `microseconds` (timed by the device's constant-rate wall
 * clock).  A benchmark puts it ahead of a timed region: the host enqueues the
 * region's launches meanwhile, and the region starts on a chip at its working
 * clocks.  (Behind a one-thread spin the chip idles, and the prefill, whose
 * arithmetic is a large part of its time, measured 3 % slower in the region.)
 *
 * microseconds  0 <= microseconds <= 1e6; 0 returns DCCONV_OK and enqueues
 *               nothing.
 * stream        hipStream_t (NULL = the null stream); asynchronous.
 *
 * Returns DCCONV_OK, DCCONV_EINVAL (out of range or NaN) or DCCONV_EHIP.
 */
int dcconv_busy_spin(double microseconds, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* DCCONV_H */
