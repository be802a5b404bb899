// C-ABI front end: host-side validation of the decode-update contract and
// dispatch to the gfx950 kernels.  Reads metadata only -- never device memory --
// allocates nothing and never synchronises.
//
// Contract: cuDNN FE-OSS page "Causal Conv1d Decode Update", sections "Semantic
// tensor contract" (shapes, the x row-stride rule, L >= W-1) and "Current native
// implementation" (W = 4, alignment, cache_seqlens must be absent).  Contract
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
    // ---- shape metadata
    if (n < 0) return fail(DCCONV_EINVAL, "n (decode rows) must be >= 0, got %lld", (long long)n);
    if (d < 1) return fail(DCCONV_EINVAL, "d (channels) must be >= 1, got %lld", (long long)d);
    if (s < 0) return fail(DCCONV_EINVAL, "s (state slots) must be >= 0, got %lld", (long long)s);
    if (w < 1) return fail(DCCONV_EINVAL, "w (filter width) must be >= 1, got %lld", (long long)w);
    if (l < w - 1)
        return fail(DCCONV_EINVAL, "conv_state length l=%lld must be >= w-1=%lld", (long long)l,
                    (long long)(w - 1));
    if (ld_x < d)
        return fail(DCCONV_EINVAL, "x row stride ld_x=%lld is smaller than d=%lld", (long long)ld_x,
                    (long long)d);
    if (ld_x > d && ld_x % 8 != 0)
        return fail(DCCONV_EINVAL,
                    "padded x rows need ld_x %% 8 == 0 (16-byte aligned rows), got ld_x=%lld for d=%lld",
                    (long long)ld_x, (long long)d);
    if (activation != DCCONV_ACT_IDENTITY && activation != DCCONV_ACT_SILU)
        return fail(DCCONV_EINVAL, "activation must be DCCONV_ACT_IDENTITY (0) or DCCONV_ACT_SILU (1), got %d",
                    activation);
    if (st_s < 0 || st_d < 0 || st_l < 0)
        return fail(DCCONV_EINVAL, "conv_state strides must be non-negative");

    // ---- served subset
    if (cache_seqlens != nullptr)
        return fail(DCCONV_EUNSUPPORTED,
                    "cache_seqlens is reserved and must be NULL (circular-buffer state is not served)");
    if (w != 4) return fail(DCCONV_EUNSUPPORTED, "only filter width w=4 is served, got w=%lld", (long long)w);
    if (n > kI32Max || d > kI32Max || s > kI32Max || l > 65536)
        return fail(DCCONV_EUNSUPPORTED, "sizes beyond n, d, s < 2^31 and l <= 65536 are not served");
    dcconv::StateLayout layout;
    if (st_l == 1 && st_d == l && (st_s >= d * l || s <= 1)) {
        layout = dcconv::StateLayout::Compact;
    } else if (st_d == 1 && st_l == d && (st_s >= l * d || s <= 1)) {
        layout = dcconv::StateLayout::ChannelLast;
    } else {
        return fail(DCCONV_EUNSUPPORTED,
                    "conv_state strides (%lld, %lld, %lld) are neither compact (>=d*l, l, 1) nor "
                    "channel-last (>=l*d, 1, d)",
                    (long long)st_s, (long long)st_d, (long long)st_l);
    }

    if (n == 0) return succeed("");

    // ---- pointers
    if (!x || !weight || !out || (!conv_state && s > 0))
        return fail(DCCONV_EINVAL, "x, weight, out (and conv_state when s > 0) must be non-NULL when n > 0");
    if (conv_state_indices == nullptr && s < n)
        return fail(DCCONV_EINVAL, "without conv_state_indices row r uses slot r, so s=%lld must be >= n=%lld",
                    (long long)s, (long long)n);
    if (!aligned(x, 16) || !aligned(conv_state, 16) || !aligned(weight, 16) || !aligned(out, 16) ||
        (bias && !aligned(bias, 16)))
        return fail(DCCONV_EINVAL, "BF16 tensors must be 16-byte aligned");
    if ((conv_state_indices && !aligned(conv_state_indices, 4)) || (dev_status && !aligned(dev_status, 4)))
        return fail(DCCONV_EINVAL, "conv_state_indices and dev_status must be 4-byte aligned");

    // ---- overlap: nothing the call writes may alias anything else it touches
    const int64_t state_elems = s > 0 ? (s - 1) * st_s + (d - 1) * st_d + (l - 1) * st_l + 1 : 0;
    const Span sx = span("x", x, 2 * ((n - 1) * ld_x + d));
    const Span sst = span("conv_state", conv_state, 2 * state_elems);
    const Span sw = span("weight", weight, 2 * d * w);
    const Span sb = span("bias", bias, 2 * d);
    const Span si = span("conv_state_indices", conv_state_indices, 4 * n);
    const Span so = span("out", out, 2 * n * d);
    const Span ss = span("dev_status", dev_status, 4);
    const Span written[] = {sst, so, ss};
    const Span all[] = {sx, sst, sw, sb, si, so, ss};
    for (const Span &a : written)
        for (const Span &b : all)
            if (a.name != b.name && overlaps(a, b))
                return fail(DCCONV_EINVAL, "%s overlaps %s", a.name, b.name);

    dcconv::UpdateParams p;
    p.x = static_cast<const uint16_t *>(x);
    p.state = static_cast<uint16_t *>(conv_state);
    p.weight = static_cast<const uint16_t *>(weight);
    p.bias = static_cast<const uint16_t *>(bias);
    p.idx = conv_state_indices;
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
