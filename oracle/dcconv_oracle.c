/*
 * Oracle for the depthwise causal conv1d decode update -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU definition of what the GPU library
 * computes, used to check it.  Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load or call this file; the product path
 * never does.  It shares no source, header, helper or table with the HIP library.
 *
 * Source of the semantics: the cuDNN FE-OSS page "Causal Conv1d Decode Update"
 * (docs.nvidia.com/cudnn/latest/fe-oss-apis/causal_conv1d_update), sections
 * "Causal Conv1d Decode Update" (the update rule, bias default, activations,
 * slot routing and padding rows) and "Semantic tensor contract" (shapes, strides,
 * the reserved multi-token form).  The full-sequence prefill (oracle_prefill) is
 * the operation that page names at its top for whole sequences; its own page is
 * not among the sources, and the reading taken is stated above the function.
 * The circular-buffer step (oracle_update_ring) serves the cache_seqlens keyword
 * the same section reserves; the ring reading is stated above that function.
 *
 * Arithmetic: FP32, one rounding to BF16 at the end, as the accuracy contract of
 * this library fixes ("FP32-accumulated oracle rounded once").  The page itself
 * does not state an accumulation precision.
 *
 * Pins: every function here is checked against things other than itself in the
 * CPU test suite (float64 library convolution, one-hot taps, closed forms,
 * library BF16 conversion, hand-worked examples); no function is parity-unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EARGS 1   /* malformed arguments (shape, null pointer, L < W-1) */
#define ORACLE_EINDEX 2  /* a slot index below -1 or not below S              */
#define ORACLE_EDUP 3    /* two non-padding rows select the same slot         */

#define ORACLE_ACT_IDENTITY 0
#define ORACLE_ACT_SILU 1

/* ---- BF16 <-> FP32 bit conversion (own code, IEEE binary32 / bfloat16) ---- */

/* A BF16 value is the upper 16 bits of the FP32 with the same value: exact. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* FP32 -> BF16, round to nearest, ties to even, on the bit pattern: add half an
 * output ulp minus one, plus the would-be result's lowest bit, then truncate.
 * Overflow past the largest finite BF16 carries into the exponent and yields
 * infinity, as IEEE rounding does.  NaN stays NaN (quiet bit forced).        */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

/* The two conversions on bit patterns, for callers that cannot pass an FP32
 * value unchanged (a float handed through a double, as a scripting-language
 * binding does, turns a signalling NaN quiet). */
uint32_t oracle_bf16_to_f32_bits(uint16_t b)
{
    float f = oracle_bf16_to_f32(b);
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

uint16_t oracle_f32_bits_to_bf16(uint32_t bits)
{
    float f;
    memcpy(&f, &bits, sizeof f);
    return oracle_f32_to_bf16(f);
}

int oracle_update_tokens(const uint16_t *x, int64_t n_rows, int64_t d, int64_t t_steps,
                         int64_t xs_n, int64_t xs_d, int64_t xs_t,
                         uint16_t *state, int64_t s_slots, int64_t l,
                         int64_t st_s, int64_t st_d, int64_t st_l,
                         const uint16_t *weight, int64_t w, const uint16_t *bias,
                         const int32_t *indices, int activation,
                         uint16_t *out, float *out_f32, int64_t os_n, int64_t os_d, int64_t os_t);

/* ---- helpers of the oracle itself ---- */

static float act_apply(float acc, int activation)
{
    if (activation == ORACLE_ACT_SILU)
        return acc / (1.0f + expf(-acc)); /* SiLU(v) = v / (1 + exp(-v)) */
    return acc;
}

/* Resolve and validate the slot of every row before anything is mutated.
 * Row n uses slot n when no table is given, else table[n]; -1 is padding.
 * Other slots must satisfy 0 <= s < S and be unique in the batch.            */
static int resolve_slots(const int32_t *indices, int64_t n_rows, int64_t s_slots,
                         int64_t *slot_of_row)
{
    for (int64_t n = 0; n < n_rows; ++n) {
        int64_t s = indices ? (int64_t)indices[n] : n;
        if (s < -1 || s >= s_slots)
            return ORACLE_EINDEX;
        slot_of_row[n] = s;
    }
    if (s_slots > 0) {
        unsigned char *seen = (unsigned char *)calloc((size_t)s_slots, 1);
        if (!seen)
            return ORACLE_EARGS;
        for (int64_t n = 0; n < n_rows; ++n) {
            int64_t s = slot_of_row[n];
            if (s < 0)
                continue;
            if (seen[s]) {
                free(seen);
                return ORACLE_EDUP;
            }
            seen[s] = 1;
        }
        free(seen);
    }
    return ORACLE_OK;
}

/*
 * The update of every row for one token (the body of the decode step below).
 * x element (n, c) at x[n*xs_n + c*xs_d]; out element (n, c) at out[n*os_n + c*os_d];
 * slot_of_row[n] already resolved (-1 = padding row).
 */
static void update_rows(const uint16_t *x, int64_t xs_n, int64_t xs_d, int64_t n_rows, int64_t d,
                        uint16_t *state, int64_t l, int64_t st_s, int64_t st_d, int64_t st_l,
                        const uint16_t *weight, int64_t w, const uint16_t *bias,
                        const int64_t *slot_of_row, int activation,
                        uint16_t *out, float *out_f32, int64_t os_n, int64_t os_d,
                        float *hist, uint16_t *hist_bits)
{
    for (int64_t n = 0; n < n_rows; ++n) {
        int64_t s = slot_of_row[n];
        if (s == -1) {                       /* padding row: zero output, no mutation */
            for (int64_t c = 0; c < d; ++c) {
                out[n * os_n + c * os_d] = 0;
                if (out_f32)
                    out_f32[n * os_n + c * os_d] = 0.0f;
            }
            continue;
        }
        for (int64_t c = 0; c < d; ++c) {
            uint16_t *slot = state + s * st_s + c * st_d;
            /* history = concat(conv_state[s, c, :], x[n, c]) */
            for (int64_t k = 0; k < l; ++k)
                hist_bits[k] = slot[k * st_l];
            hist_bits[l] = x[n * xs_n + c * xs_d];
            /* conv_state[s, c, :] = history[-l:]  (a copy of bit patterns) */
            for (int64_t k = 0; k < l; ++k)
                slot[k * st_l] = hist_bits[k + 1];
            for (int64_t k = 0; k <= l; ++k)
                hist[k] = oracle_bf16_to_f32(hist_bits[k]);
            /* acc = sum_j history[-w + j] * weight[c, j] + bias[c] */
            float acc = 0.0f;
            for (int64_t j = 0; j < w; ++j)
                acc = acc + hist[l + 1 - w + j] * oracle_bf16_to_f32(weight[c * w + j]);
            if (bias)
                acc = acc + oracle_bf16_to_f32(bias[c]);
            float y = act_apply(acc, activation);
            if (out_f32)
                out_f32[n * os_n + c * os_d] = y;
            out[n * os_n + c * os_d] = oracle_f32_to_bf16(y);
        }
    }
}

/*
 * One decode step ("Causal Conv1d Decode Update" page, section of the same name).
 *
 *   x        BF16 bits [n_rows, d], element (n, c) at x[n*ld + c]
 *   state    BF16 bits [s_slots, d, l], element (s, c, k) at
 *            state[s*st_s + c*st_d + k*st_l]; k = 0 is the oldest value,
 *            k = l-1 the newest.  Updated in place.
 *   weight   BF16 bits [d, w] contiguous
 *   bias     BF16 bits [d] or NULL (zero bias)
 *   indices  int32 [n_rows] or NULL (row n -> slot n); -1 = padding row
 *   out      BF16 bits [n_rows, d] contiguous
 *   out_f32  optional FP32 [n_rows, d]: the value before the one BF16 rounding
 *
 * For a row with slot s and channel c the history is the slot's l values
 * followed by x[n, c] (length l+1).  The state keeps the newest l of them, and
 * the output is act(sum_j history[l+1-w+j] * weight[c, j] + bias[c]), the sum
 * taken in FP32 with j ascending from zero and the bias added last.
 * A padding row writes a zero output and leaves every slot untouched.
 * Returns ORACLE_OK, or an error code before mutating anything.
 */
int oracle_update(const uint16_t *x, int64_t n_rows, int64_t d, int64_t ld,
                  uint16_t *state, int64_t s_slots, int64_t l,
                  int64_t st_s, int64_t st_d, int64_t st_l,
                  const uint16_t *weight, int64_t w, const uint16_t *bias,
                  const int32_t *indices, int activation,
                  uint16_t *out, float *out_f32)
{
    if (ld < d)
        return ORACLE_EARGS;
    return oracle_update_tokens(x, n_rows, d, 1, ld, 1, 0, state, s_slots, l, st_s, st_d, st_l,
                                weight, w, bias, indices, activation, out, out_f32, d, 1, 0);
}

/*
 * T successive decode steps on the same slots: the reading of the page's future
 * multi-token form x[N, D, Tstep] ("Semantic tensor contract": the state and
 * weight keep their meaning).  Token t of every row is applied, in order, by
 * exactly the single-step rule above, and out[:, :, t] is that step's output.
 *
 *   x    element (n, c, t) at x[n*xs_n + c*xs_d + t*xs_t]
 *   out  element (n, c, t) at out[n*os_n + c*os_d + t*os_t] (out_f32 the same)
 */
int oracle_update_tokens(const uint16_t *x, int64_t n_rows, int64_t d, int64_t t_steps,
                         int64_t xs_n, int64_t xs_d, int64_t xs_t,
                         uint16_t *state, int64_t s_slots, int64_t l,
                         int64_t st_s, int64_t st_d, int64_t st_l,
                         const uint16_t *weight, int64_t w, const uint16_t *bias,
                         const int32_t *indices, int activation,
                         uint16_t *out, float *out_f32, int64_t os_n, int64_t os_d, int64_t os_t)
{
    if (n_rows < 0 || d < 1 || t_steps < 0 || s_slots < 0 || w < 1 || l < w - 1 || l < 1)
        return ORACLE_EARGS;
    if (activation != ORACLE_ACT_IDENTITY && activation != ORACLE_ACT_SILU)
        return ORACLE_EARGS;
    if (n_rows == 0 || t_steps == 0)
        return ORACLE_OK;
    if (!x || !state || !weight || !out)
        return ORACLE_EARGS;
    if (!indices && s_slots < n_rows)
        return ORACLE_EARGS;

    int64_t *slot_of_row = (int64_t *)malloc((size_t)n_rows * sizeof(int64_t));
    float *hist = (float *)malloc((size_t)(l + 1) * sizeof(float));
    uint16_t *hist_bits = (uint16_t *)malloc((size_t)(l + 1) * sizeof(uint16_t));
    if (!slot_of_row || !hist || !hist_bits) {
        free(slot_of_row); free(hist); free(hist_bits);
        return ORACLE_EARGS;
    }
    int rc = resolve_slots(indices, n_rows, s_slots, slot_of_row);
    if (rc == ORACLE_OK) {
        for (int64_t t = 0; t < t_steps; ++t)
            update_rows(x + t * xs_t, xs_n, xs_d, n_rows, d, state, l, st_s, st_d, st_l, weight, w, bias,
                        slot_of_row, activation, out + t * os_t, out_f32 ? out_f32 + t * os_t : NULL,
                        os_n, os_d, hist, hist_bits);
    }
    free(slot_of_row); free(hist); free(hist_bits);
    return rc;
}

/*
 * Full-sequence causal convolution (prefill), the operation the page names
 * cudnn.ops.causal_conv1d at its top: it produces the final state that the
 * decode update then continues.  The prefill page itself is not among the
 * sources, so this follows the plainest reading that the decode page supports:
 * a sequence of tokens x_0..x_{T-1} convolved causally over its history, which
 * is the initial state (or zeros), with the final state the newest L values of
 * that history.  For one channel c of sequence i:
 *
 *   ext          = concat(init[0:L], x[i, c, 0:T])           (L + T values)
 *   out[i, c, j] = act(sum_k ext[L + j - (w-1) + k] * weight[c, k] + bias[c])
 *   final[0:L]   = ext[T : T + L]                             (the newest L)
 *
 * with the sum in FP32, k ascending from zero, the bias last, one BF16 rounding;
 * init is the slot's state when has_init[i] is nonzero, else zeros.
 *
 *   starts   NULL: n sequences of t tokens each, token j of sequence i at
 *            x[i*xs_n + c*xs_d + j*xs_t] (out likewise with os_*).
 *            Else int32 [n+1] with 0 = starts[0] <= ... <= starts[n] = t:
 *            sequence i is packed tokens starts[i] .. starts[i+1]-1, token j at
 *            x[c*xs_d + (starts[i] + j)*xs_t]; xs_n and os_n are not used.
 *   state    NULL: no initial and no final state (history starts at zero, L is
 *            taken as w-1).  Else [s_slots, d, l] at strides (st_s, st_d, st_l);
 *            sequence i uses slot indices[i] (or i), -1 = padding: its outputs
 *            are zero and it touches no slot.  The final state replaces the slot.
 *   has_init NULL (every sequence starts from zeros) or uint8 [n].
 * Returns ORACLE_OK, or an error code before mutating anything.
 */
int oracle_prefill(const uint16_t *x, int64_t n_seqs, int64_t d, int64_t t,
                   int64_t xs_n, int64_t xs_d, int64_t xs_t, const int32_t *starts,
                   uint16_t *state, int64_t s_slots, int64_t l,
                   int64_t st_s, int64_t st_d, int64_t st_l,
                   const int32_t *indices, const uint8_t *has_init,
                   const uint16_t *weight, int64_t w, const uint16_t *bias, int activation,
                   uint16_t *out, float *out_f32, int64_t os_n, int64_t os_d, int64_t os_t)
{
    if (n_seqs < 0 || d < 1 || t < 0 || w < 1)
        return ORACLE_EARGS;
    if (activation != ORACLE_ACT_IDENTITY && activation != ORACLE_ACT_SILU)
        return ORACLE_EARGS;
    if (state == NULL) {
        if (indices || has_init)
            return ORACLE_EARGS;
        l = w - 1;
        s_slots = 0;
    } else if (l < w - 1 || l < 1 || s_slots < 0 || (!indices && s_slots < n_seqs)) {
        return ORACLE_EARGS;
    }
    if (starts) {
        if (starts[0] != 0 || starts[n_seqs] != t)
            return ORACLE_EARGS;
        for (int64_t i = 0; i < n_seqs; ++i)
            if (starts[i + 1] < starts[i])
                return ORACLE_EARGS;
    }
    if (n_seqs == 0)
        return ORACLE_OK;
    if (!weight || (t > 0 && (!x || !out)))
        return ORACLE_EARGS;

    int64_t *slot_of_seq = (int64_t *)malloc((size_t)n_seqs * sizeof(int64_t));
    if (!slot_of_seq)
        return ORACLE_EARGS;
    int rc = ORACLE_OK;
    if (state)
        rc = resolve_slots(indices, n_seqs, s_slots, slot_of_seq);
    else
        for (int64_t i = 0; i < n_seqs; ++i)
            slot_of_seq[i] = i;   /* every sequence live, no slot behind it */
    int64_t max_len = 0;
    for (int64_t i = 0; i < n_seqs; ++i) {
        int64_t len = starts ? (int64_t)starts[i + 1] - starts[i] : t;
        if (len > max_len)
            max_len = len;
    }
    uint16_t *ext = (uint16_t *)malloc((size_t)(l + max_len) * sizeof(uint16_t));
    if (!ext)
        rc = ORACLE_EARGS;
    for (int64_t i = 0; rc == ORACLE_OK && i < n_seqs; ++i) {
        int64_t len = starts ? (int64_t)starts[i + 1] - starts[i] : t;
        const uint16_t *xi = starts ? x + (int64_t)starts[i] * xs_t : x + i * xs_n;
        uint16_t *oi = starts ? out + (int64_t)starts[i] * os_t : out + i * os_n;
        float *fi = out_f32 ? (starts ? out_f32 + (int64_t)starts[i] * os_t : out_f32 + i * os_n) : NULL;
        int64_t slot = slot_of_seq[i];
        if (slot == -1) {                     /* padding sequence: zero outputs only */
            for (int64_t c = 0; c < d; ++c)
                for (int64_t j = 0; j < len; ++j) {
                    oi[c * os_d + j * os_t] = 0;
                    if (fi)
                        fi[c * os_d + j * os_t] = 0.0f;
                }
            continue;
        }
        int from_state = state != NULL && has_init != NULL && has_init[i] != 0;
        for (int64_t c = 0; c < d; ++c) {
            uint16_t *sc = state ? state + slot * st_s + c * st_d : NULL;
            for (int64_t k = 0; k < l; ++k)
                ext[k] = from_state ? sc[k * st_l] : (uint16_t)0;
            for (int64_t j = 0; j < len; ++j)
                ext[l + j] = xi[c * xs_d + j * xs_t];
            for (int64_t j = 0; j < len; ++j) {
                float acc = 0.0f;
                for (int64_t k = 0; k < w; ++k)
                    acc = acc + oracle_bf16_to_f32(ext[l + j - (w - 1) + k]) *
                                    oracle_bf16_to_f32(weight[c * w + k]);
                if (bias)
                    acc = acc + oracle_bf16_to_f32(bias[c]);
                float y = act_apply(acc, activation);
                if (fi)
                    fi[c * os_d + j * os_t] = y;
                oi[c * os_d + j * os_t] = oracle_f32_to_bf16(y);
            }
            if (sc)
                for (int64_t k = 0; k < l; ++k)
                    sc[k * st_l] = ext[len + k];
        }
    }
    free(slot_of_seq);
    free(ext);
    return rc;
}

/*
 * One decode step on circular-buffer state, selected by cache_seqlens.  The page
 * reserves the keyword "for circular-buffer state" and fixes nothing else, so
 * this takes the plainest ring reading: a slot whose row has seen c tokens keeps
 * token i (i = c-L .. c-1) at state[s, d, i mod L]; the step's history is those
 * L tokens followed by x (the same history as the shifting update), so
 *
 *   out[n, d]               = act(sum_j token[c+1-w+j] * weight[d, j] + bias[d])
 *                             with token[c] = x[n, d] and the others read at
 *                             positions (c+1-w+j) mod L, taken before any write;
 *   state[s, d, c mod L]    = x[n, d]     (the oldest token is replaced; the
 *                                          other L-1 values do not move)
 *
 * c = cache_seqlens[n] >= 0 (ORACLE_EARGS otherwise); routing and padding rows as
 * for oracle_update.  Arguments as for oracle_update.
 */
int oracle_update_ring(const uint16_t *x, int64_t n_rows, int64_t d, int64_t ld,
                       uint16_t *state, int64_t s_slots, int64_t l,
                       int64_t st_s, int64_t st_d, int64_t st_l,
                       const uint16_t *weight, int64_t w, const uint16_t *bias,
                       const int32_t *indices, const int32_t *cache_seqlens, int activation,
                       uint16_t *out, float *out_f32)
{
    if (n_rows < 0 || d < 1 || ld < d || s_slots < 0 || w < 1 || l < w - 1 || l < 1)
        return ORACLE_EARGS;
    if (activation != ORACLE_ACT_IDENTITY && activation != ORACLE_ACT_SILU)
        return ORACLE_EARGS;
    if (n_rows == 0)
        return ORACLE_OK;
    if (!x || !state || !weight || !out || !cache_seqlens)
        return ORACLE_EARGS;
    if (!indices && s_slots < n_rows)
        return ORACLE_EARGS;
    for (int64_t n = 0; n < n_rows; ++n)
        if (cache_seqlens[n] < 0)
            return ORACLE_EARGS;
    int64_t *slot_of_row = (int64_t *)malloc((size_t)n_rows * sizeof(int64_t));
    if (!slot_of_row)
        return ORACLE_EARGS;
    int rc = resolve_slots(indices, n_rows, s_slots, slot_of_row);
    for (int64_t n = 0; rc == ORACLE_OK && n < n_rows; ++n) {
        int64_t s = slot_of_row[n];
        if (s == -1) {                       /* padding row: zero output, no mutation */
            for (int64_t c = 0; c < d; ++c) {
                out[n * d + c] = 0;
                if (out_f32)
                    out_f32[n * d + c] = 0.0f;
            }
            continue;
        }
        int64_t seen = cache_seqlens[n];
        for (int64_t c = 0; c < d; ++c) {
            uint16_t *ring = state + s * st_s + c * st_d;
            uint16_t xb = x[n * ld + c];
            float acc = 0.0f;
            for (int64_t j = 0; j < w; ++j) {
                int64_t tok = seen + 1 - w + j;              /* token index of tap j */
                uint16_t v = xb;
                if (tok < seen) {
                    int64_t pos = ((tok % l) + l) % l;       /* non-negative remainder */
                    v = ring[pos * st_l];
                }
                acc = acc + oracle_bf16_to_f32(v) * oracle_bf16_to_f32(weight[c * w + j]);
            }
            if (bias)
                acc = acc + oracle_bf16_to_f32(bias[c]);
            float y = act_apply(acc, activation);
            if (out_f32)
                out_f32[n * d + c] = y;
            out[n * d + c] = oracle_f32_to_bf16(y);
            ring[(seen % l) * st_l] = xb;
        }
    }
    free(slot_of_row);
    return rc;
}

/* Library self-description, so a loader can check it has the file it expects. */
int oracle_version(void) { return 1; }
