// C-ABI front end: host-side validation of the decode-update contract and
// dispatch to the gfx950 kernels.  Reads metadata only -- never device memory --
// allocates nothing and never synchronises.
//
// Contract: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections "Semantic
// tensor contract" (shapes, the x row-stride rule, L >= W-1) and "Current native
// implementation" (W = 4, alignment); cache_seqlens selects the circular-buffer
// state the page reserves that keyword for.  Contract
// violations return DCCONV_EINVAL (the page's ValueError); valid requests that
// are not served return DCCONV_EUNSUPPORTED (the page's NotImplementedError).
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "dcconv.h"
#include "update_params.h"

namespace {

thread_local char g_error[512];
thread_local const char *g_kernel = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    g_kernel = "";
    return code;
}

int succeed(const char *kernel) {
    g_error[0] = '\0';
    g_kernel = kernel;
    return DCCONV_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A byte range [lo, hi) of one operand, for the overlap checks.
struct Span {
    const char *name;
    uintptr_t lo, hi;
};

Span span(const char *name, const void *p, int64_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{name, lo, p ? lo + (uintptr_t)(bytes > 0 ? bytes : 0) : lo};
}

bool overlaps(const Span &a, const Span &b) {
    return a.hi > a.lo && b.hi > b.lo && a.lo < b.hi && b.lo < a.hi;
}

constexpr int64_t kI32Max = 2147483647;

// Bytes spanned by an [e0, e1, e2] BF16 array at element strides st (strides
// >= 0): 2 * (sum (e_i - 1) * st_i + 1), or 0 for an empty array.  False when
// the span overflows or exceeds 2^47 bytes, more than any device address space.
bool span_bytes(const int64_t e[3], const int64_t st[3], int64_t *bytes) {
    const int64_t kMaxElems = (int64_t)1 << 46;
    int64_t last = 0;
    for (int i = 0; i < 3; ++i)
        if (e[i] <= 0) {
            *bytes = 0;
            return true;
        }
    for (int i = 0; i < 3; ++i) {
        int64_t term;
        if (__builtin_mul_overflow(e[i] - 1, st[i], &term) || term > kMaxElems) return false;
        last += term;
        if (last > kMaxElems) return false;
    }
    *bytes = 2 * (last + 1);
    return true;
}


// Metadata shared by both entry points: shapes, state strides, the served subset.
int check_state_and_shapes(int64_t n, int64_t d, int64_t s, int64_t l, int64_t st_s, int64_t st_d, int64_t st_l,
                           int64_t w, int activation, dcconv::StateLayout *layout) {
    if (n < 0) return fail(DCCONV_EINVAL, "n (decode rows) must be >= 0, got %lld", (long long)n);
    if (d < 1) return fail(DCCONV_EINVAL, "d (channels) must be >= 1, got %lld", (long long)d);
    if (s < 0) return fail(DCCONV_EINVAL, "s (state slots) must be >= 0, got %lld", (long long)s);
    if (w < 1) return fail(DCCONV_EINVAL, "w (filter width) must be >= 1, got %lld", (long long)w);
    if (l < w - 1)
        return fail(DCCONV_EINVAL, "conv_state length l=%lld must be >= w-1=%lld", (long long)l,
                    (long long)(w - 1));
    if (activation != DCCONV_ACT_IDENTITY && activation != DCCONV_ACT_SILU)
        return fail(DCCONV_EINVAL, "activation must be DCCONV_ACT_IDENTITY (0) or DCCONV_ACT_SILU (1), got %d",
                    activation);
    if (st_s < 0 || st_d < 0 || st_l < 0) return fail(DCCONV_EINVAL, "conv_state strides must be non-negative");
    if (w != 4) return fail(DCCONV_EUNSUPPORTED, "only filter width w=4 is served, got w=%lld", (long long)w);
    if (n > kI32Max || d > kI32Max || s > kI32Max || l > 65536)
        return fail(DCCONV_EUNSUPPORTED, "sizes beyond n, d, s < 2^31 and l <= 65536 are not served");
    {
        const int64_t e[3] = {s, d, l}, st[3] = {st_s, st_d, st_l};
        int64_t bytes;
        if (!span_bytes(e, st, &bytes))
            return fail(DCCONV_EINVAL, "conv_state strides (%lld, %lld, %lld) span more than 2^47 bytes",
                        (long long)st_s, (long long)st_d, (long long)st_l);
    }
    if (st_l == 1 && st_d == l && (st_s >= d * l || s <= 1)) {
        *layout = dcconv::StateLayout::Compact;
    } else if (st_d == 1 && st_l == d && (st_s >= l * d || s <= 1)) {
        *layout = dcconv::StateLayout::ChannelLast;
    } else {
        return fail(DCCONV_EUNSUPPORTED,
                    "conv_state strides (%lld, %lld, %lld) are neither compact (>=d*l, l, 1) nor "
                    "channel-last (>=l*d, 1, d)",
                    (long long)st_s, (long long)st_d, (long long)st_l);
    }
    return DCCONV_OK;
}

// Pointers, alignment and overlap, once the byte extent of x and out is known.
// `extra` lists further read-only operands (prefill's sequence table and
// initial-state flags); x and out may be NULL only when x_bytes == 0.
int check_pointers(const void *x, int64_t x_bytes, void *conv_state, int64_t s, int64_t d, int64_t l, int64_t st_s,
                   int64_t st_d, int64_t st_l, const void *weight, int64_t w, const void *bias,
                   const int32_t *conv_state_indices, int64_t n, void *out, int64_t out_bytes, int32_t *dev_status,
                   const Span *extra = nullptr, int n_extra = 0, bool stateless = false) {
    if ((x_bytes > 0 && (!x || !out)) || !weight || (!conv_state && s > 0))
        return fail(DCCONV_EINVAL, "x, weight, out (and conv_state when s > 0) must be non-NULL when n > 0");
    if (!stateless && conv_state_indices == nullptr && s < n)
        return fail(DCCONV_EINVAL, "without conv_state_indices row r uses slot r, so s=%lld must be >= n=%lld",
                    (long long)s, (long long)n);
    if (!aligned(x, 16) || !aligned(conv_state, 16) || !aligned(weight, 16) || !aligned(out, 16) ||
        (bias && !aligned(bias, 16)))
        return fail(DCCONV_EINVAL, "BF16 tensors must be 16-byte aligned");
    if ((conv_state_indices && !aligned(conv_state_indices, 4)) || (dev_status && !aligned(dev_status, 4)))
        return fail(DCCONV_EINVAL, "conv_state_indices and dev_status must be 4-byte aligned");
    // nothing the call writes may alias anything else it touches
    const int64_t se[3] = {s, d, l}, sst_[3] = {st_s, st_d, st_l};
    int64_t state_bytes = 0;
    span_bytes(se, sst_, &state_bytes);  // bounded by check_state_and_shapes
    const Span sx = span("x", x, x_bytes);
    const Span sst = span("conv_state", conv_state, state_bytes);
    const Span sw = span("weight", weight, 2 * d * w);
    const Span sb = span("bias", bias, 2 * d);
    const Span si = span("conv_state_indices", conv_state_indices, 4 * n);
    const Span so = span("out", out, out_bytes);
    const Span ss = span("dev_status", dev_status, 4);
    const Span written[] = {sst, so, ss};
    const Span all[] = {sx, sst, sw, sb, si, so, ss};
    for (const Span &a : written) {
        for (const Span &b : all)
            if (a.name != b.name && overlaps(a, b))
                return fail(DCCONV_EINVAL, "%s overlaps %s", a.name, b.name);
        for (int k = 0; k < n_extra; ++k)
            if (overlaps(a, extra[k])) return fail(DCCONV_EINVAL, "%s overlaps %s", a.name, extra[k].name);
    }
    return DCCONV_OK;
}

// True when no two elements of an [e0, e1, e2] array at strides s0, s1, s2 share
// an address: sorted by stride, each dimension must step over the whole extent of
// the ones below it.
bool strides_distinct(const int64_t e[3], const int64_t st[3]) {
    int64_t ext[3], str[3];
    int k = 0;
    for (int i = 0; i < 3; ++i)
        if (e[i] > 1) {
            ext[k] = e[i];
            str[k] = st[i];
            ++k;
        }
    for (int i = 1; i < k; ++i)
        for (int j = i; j > 0 && str[j] < str[j - 1]; --j) {
            const int64_t te = ext[j], ts = str[j];
            ext[j] = ext[j - 1];
            str[j] = str[j - 1];
            ext[j - 1] = te;
            str[j - 1] = ts;
        }
    int64_t span_below = 1;
    for (int i = 0; i < k; ++i) {
        if (str[i] < span_below) return false;
        span_below = str[i] * (ext[i] - 1) + span_below;
    }
    return true;
}

}  // namespace

extern "C" int dcconv_abi_version(void) { return DCCONV_ABI_VERSION; }

extern "C" const char *dcconv_last_error(void) { return g_error; }

extern "C" const char *dcconv_last_kernel(void) { return g_kernel; }

extern "C" int dcconv_update(const void *x, int64_t n, int64_t d, int64_t ld_x,
                             void *conv_state, int64_t s, int64_t l,
                             int64_t st_s, int64_t st_d, int64_t st_l,
                             const void *weight, int64_t w,
                             const void *bias,
                             const int32_t *conv_state_indices,
                             const int32_t *cache_seqlens,
                             int activation,
                             void *out,
                             int32_t *dev_status,
                             void *stream) {
    // ---- shape metadata and the served subset
    dcconv::StateLayout layout;
    if (n >= 0 && d >= 1 && ld_x < d)
        return fail(DCCONV_EINVAL, "x row stride ld_x=%lld is smaller than d=%lld", (long long)ld_x,
                    (long long)d);
    if (n >= 0 && d >= 1 && ld_x > d && ld_x % 8 != 0)
        return fail(DCCONV_EINVAL,
                    "padded x rows need ld_x %% 8 == 0 (16-byte aligned rows), got ld_x=%lld for d=%lld",
                    (long long)ld_x, (long long)d);
    int rc = check_state_and_shapes(n, d, s, l, st_s, st_d, st_l, w, activation, &layout);
    if (rc != DCCONV_OK) return rc;
    if (n == 0) return succeed("");
    if (cache_seqlens != nullptr && !aligned(cache_seqlens, 4))
        return fail(DCCONV_EINVAL, "cache_seqlens must be 4-byte aligned");
    const Span extra[] = {span("cache_seqlens", cache_seqlens, 4 * n)};
    const int64_t xe[3] = {n, d, 1}, xst[3] = {ld_x, 1, 0};
    int64_t x_bytes;
    if (!span_bytes(xe, xst, &x_bytes))
        return fail(DCCONV_EINVAL, "x with row stride %lld spans more than 2^47 bytes", (long long)ld_x);
    rc = check_pointers(x, x_bytes, conv_state, s, d, l, st_s, st_d, st_l, weight, w, bias,
                        conv_state_indices, n, out, 2 * n * d, dev_status, extra, 1);
    if (rc != DCCONV_OK) return rc;

    dcconv::UpdateParams p;
    p.x = static_cast<const uint16_t *>(x);
    p.state = static_cast<uint16_t *>(conv_state);
    p.weight = static_cast<const uint16_t *>(weight);
    p.bias = static_cast<const uint16_t *>(bias);
    p.idx = conv_state_indices;
    p.seqlens = cache_seqlens;
    p.status = dev_status;
    p.out = static_cast<uint16_t *>(out);
    p.ld = n > 1 ? ld_x : d;
    p.st_s = st_s;
    p.st_d = st_d;
    p.st_l = st_l;
    p.n = (int32_t)n;
    p.d = (int32_t)d;
    p.s = (int32_t)s;
    p.l = (int32_t)l;
    const char *name = "";
    const hipError_t err =
        dcconv::launch_update(p, layout, activation, static_cast<hipStream_t>(stream), &name);
    if (err != hipSuccess) return fail(DCCONV_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return succeed(name);
}

extern "C" int dcconv_update_tokens(const void *x, int64_t n, int64_t d, int64_t t,
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
                                    void *stream) {
    dcconv::StateLayout layout;
    if (t < 0) return fail(DCCONV_EINVAL, "t (tokens) must be >= 0, got %lld", (long long)t);
    if (xs_n < 0 || xs_d < 0 || xs_t < 0 || os_n < 0 || os_d < 0 || os_t < 0)
        return fail(DCCONV_EINVAL, "x and out strides must be non-negative");
    int rc = check_state_and_shapes(n, d, s, l, st_s, st_d, st_l, w, activation, &layout);
    if (rc != DCCONV_OK) return rc;
    if (t > kI32Max) return fail(DCCONV_EUNSUPPORTED, "t >= 2^31 tokens is not served");
    if (n == 0 || t == 0) return succeed("");
    const int64_t ext[3] = {n, d, t}, ost[3] = {os_n, os_d, os_t};
    if (!strides_distinct(ext, ost))
        return fail(DCCONV_EINVAL, "out strides (%lld, %lld, %lld) give two elements the same address",
                    (long long)os_n, (long long)os_d, (long long)os_t);
    const int64_t xst[3] = {xs_n, xs_d, xs_t};
    int64_t x_bytes, out_bytes;
    if (!span_bytes(ext, xst, &x_bytes) || !span_bytes(ext, ost, &out_bytes))
        return fail(DCCONV_EINVAL, "x or out strides span more than 2^47 bytes");
    if (cache_seqlens != nullptr && !aligned(cache_seqlens, 4))
        return fail(DCCONV_EINVAL, "cache_seqlens must be 4-byte aligned");
    const Span extra[] = {span("cache_seqlens", cache_seqlens, 4 * n)};
    rc = check_pointers(x, x_bytes, conv_state, s, d, l, st_s, st_d, st_l, weight, w, bias, conv_state_indices, n,
                        out, out_bytes, dev_status, extra, 1);
    if (rc != DCCONV_OK) return rc;

    dcconv::TokensParams p;
    p.x = static_cast<const uint16_t *>(x);
    p.state = static_cast<uint16_t *>(conv_state);
    p.weight = static_cast<const uint16_t *>(weight);
    p.bias = static_cast<const uint16_t *>(bias);
    p.idx = conv_state_indices;
    p.seqlens = cache_seqlens;
    p.status = dev_status;
    p.out = static_cast<uint16_t *>(out);
    p.xs_n = xs_n;
    p.xs_d = xs_d;
    p.xs_t = xs_t;
    p.os_n = os_n;
    p.os_d = os_d;
    p.os_t = os_t;
    p.st_s = st_s;
    p.st_d = st_d;
    p.st_l = st_l;
    p.n = (int32_t)n;
    p.d = (int32_t)d;
    p.t = (int32_t)t;
    p.s = (int32_t)s;
    p.l = (int32_t)l;
    const char *name = "";
    const hipError_t err =
        dcconv::launch_update_tokens(p, layout, activation, static_cast<hipStream_t>(stream), &name);
    if (err != hipSuccess) return fail(DCCONV_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return succeed(name);
}

extern "C" int dcconv_prefill(const void *x, int64_t n, int64_t d, int64_t t,
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
                              void *stream) {
    const bool stateful = conv_state != nullptr;
    const bool packed = seq_starts != nullptr;
    if (t < 0) return fail(DCCONV_EINVAL, "t (tokens) must be >= 0, got %lld", (long long)t);
    if (xs_n < 0 || xs_d < 0 || xs_t < 0 || os_n < 0 || os_d < 0 || os_t < 0)
        return fail(DCCONV_EINVAL, "x and out strides must be non-negative");
    if (!stateful) {
        if (s != 0 || conv_state_indices != nullptr || has_initial_state != nullptr)
            return fail(DCCONV_EINVAL,
                        "without conv_state, s must be 0 and conv_state_indices and has_initial_state NULL");
        // no state: validate the rest against a virtual compact [0, d, w-1] state
        l = w - 1 > 0 ? w - 1 : 1;
        st_l = 1;
        st_d = l;
        st_s = d * l;
    }
    dcconv::StateLayout layout;
    int rc = check_state_and_shapes(n, d, s, l, st_s, st_d, st_l, w, activation, &layout);
    if (rc != DCCONV_OK) return rc;
    if (t > kI32Max) return fail(DCCONV_EUNSUPPORTED, "t >= 2^31 tokens is not served");
    if (n == 0) return succeed("");
    if (packed && !aligned(seq_starts, 4)) return fail(DCCONV_EINVAL, "seq_starts must be 4-byte aligned");
    if (t == 0 && !stateful) return succeed("");  // nothing to read or write
    const int64_t rows = packed ? 1 : n;
    int64_t x_bytes = 0, out_bytes = 0;
    if (t > 0) {
        const int64_t ext[3] = {rows, d, t}, ost[3] = {os_n, os_d, os_t};
        if (!strides_distinct(ext, ost))
            return fail(DCCONV_EINVAL, "out strides (%lld, %lld, %lld) give two elements the same address",
                        (long long)os_n, (long long)os_d, (long long)os_t);
        const int64_t xst[3] = {xs_n, xs_d, xs_t};
        if (!span_bytes(ext, xst, &x_bytes) || !span_bytes(ext, ost, &out_bytes))
            return fail(DCCONV_EINVAL, "x or out strides span more than 2^47 bytes");
    }
    const Span extra[] = {span("seq_starts", seq_starts, 4 * (n + 1)), span("has_initial_state", has_initial_state, n)};
    rc = check_pointers(x, x_bytes, conv_state, s, d, l, st_s, st_d, st_l, weight, w, bias, conv_state_indices, n,
                        out, out_bytes, dev_status, extra, 2, !stateful);
    if (rc != DCCONV_OK) return rc;

    dcconv::PrefillParams p;
    p.x = static_cast<const uint16_t *>(x);
    p.state = static_cast<uint16_t *>(conv_state);
    p.weight = static_cast<const uint16_t *>(weight);
    p.bias = static_cast<const uint16_t *>(bias);
    p.starts = seq_starts;
    p.idx = conv_state_indices;
    p.has_init = has_initial_state;
    p.status = dev_status;
    p.out = static_cast<uint16_t *>(out);
    p.xs_n = packed ? 0 : xs_n;
    p.xs_d = xs_d;
    p.xs_t = xs_t;
    p.os_n = packed ? 0 : os_n;
    p.os_d = os_d;
    p.os_t = os_t;
    p.st_s = st_s;
    p.st_d = st_d;
    p.st_l = st_l;
    p.n = (int32_t)n;
    p.d = (int32_t)d;
    p.t = (int32_t)t;
    p.s = (int32_t)s;
    p.l = (int32_t)l;
    const char *name = "";
    const hipError_t err = dcconv::launch_prefill(p, layout, activation, static_cast<hipStream_t>(stream), &name);
    if (err != hipSuccess) return fail(DCCONV_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return succeed(name);
}

extern "C" int dcconv_stream_copy(void *dst, const void *src, int64_t bytes, void *stream) {
    if (bytes < 0) return fail(DCCONV_EINVAL, "bytes=%lld is negative", (long long)bytes);
    if (bytes == 0) return succeed("");
    if (dst == nullptr || src == nullptr) return fail(DCCONV_EINVAL, "dst and src must not be NULL");
    if (bytes % 16 != 0) return fail(DCCONV_EINVAL, "bytes=%lld is not a multiple of 16", (long long)bytes);
    if (bytes > ((int64_t)1 << 47)) return fail(DCCONV_EINVAL, "bytes=%lld exceeds 2^47", (long long)bytes);
    if (!aligned(dst, 16) || !aligned(src, 16)) return fail(DCCONV_EINVAL, "dst and src must be 16-byte aligned");
    if (overlaps(span("dst", dst, bytes), span("src", src, bytes)))
        return fail(DCCONV_EINVAL, "dst and src overlap");
    const hipError_t err = dcconv::launch_stream_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(DCCONV_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return succeed("stream_copy_v8");
}

extern "C" int dcconv_busy_spin(double microseconds, void *stream) {
    if (!(microseconds >= 0.0 && microseconds <= 1e6))
        return fail(DCCONV_EINVAL, "microseconds=%g is not in [0, 1e6]", microseconds);
    if (microseconds == 0.0) return succeed("");
    int dev = 0, khz = 0, cus = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return fail(DCCONV_EHIP, "device query failed: %s", hipGetErrorString(err));
    if (khz <= 0 || cus <= 0) return fail(DCCONV_EHIP, "device reports wall clock %d kHz, %d CUs", khz, cus);
    // one wave per SIMD (four per CU)
    const uint64_t ticks = (uint64_t)(microseconds * (double)khz / 1000.0) + 1;
    err = dcconv::launch_busy_spin(ticks, 4 * cus, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return fail(DCCONV_EHIP, "kernel launch failed: %s", hipGetErrorString(err));
    return succeed("busy_spin");
}
