// Internal interface between the C-ABI front end (abi.hip) and the kernels
// (update.hip, update_tokens.hip, prefill.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dcconv {

// Everything one decode-update launch needs, already validated on the host.
struct UpdateParams {
    const uint16_t *x;      // BF16 [n, d], row stride ld (elements)
    uint16_t *state;        // BF16 logical [s, d, l] at strides (st_s, st_d, st_l)
    const uint16_t *weight; // BF16 [d, 4]
    const uint16_t *bias;   // BF16 [d] or nullptr
    const int32_t *idx;     // int32 [n] or nullptr
    const int32_t *seqlens; // int32 [n] (circular-buffer state) or nullptr
    int32_t *status;        // device int32 or nullptr
    uint16_t *out;          // BF16 [n, d]
    int64_t ld;
    int64_t st_s, st_d, st_l;
    int32_t n, d, s, l;
};

enum class StateLayout { Compact, ChannelLast };

// A multi-token update: T successive decode steps, x and out [n, d, t] at element
// strides (n, channel, token).  Validated on the host.
struct TokensParams {
    const uint16_t *x;
    uint16_t *state;
    const uint16_t *weight;
    const uint16_t *bias;
    const int32_t *idx;
    const int32_t *seqlens;  // int32 [n] (circular-buffer state) or nullptr
    int32_t *status;
    uint16_t *out;
    int64_t xs_n, xs_d, xs_t;
    int64_t os_n, os_d, os_t;
    int64_t st_s, st_d, st_l;
    int32_t n, d, t, s, l;
};

// A prefill: n sequences (batch form, or packed with `starts`), validated on the
// host.  state == nullptr means stateless (no initial and no final state).
struct PrefillParams {
    const uint16_t *x;
    uint16_t *state;
    const uint16_t *weight;
    const uint16_t *bias;
    const int32_t *starts;   // int32 [n+1] or nullptr (batch form)
    const int32_t *idx;
    const uint8_t *has_init;
    int32_t *status;
    uint16_t *out;
    int64_t xs_n, xs_d, xs_t;
    int64_t os_n, os_d, os_t;
    int64_t st_s, st_d, st_l;
    int32_t n, d, t, s, l;
};

// Picks the specialisation, launches it on `stream` and stores its name in
// *kernel_name.  Returns hipSuccess or the launch error.
hipError_t launch_update(const UpdateParams &p, StateLayout layout, int activation,
                         hipStream_t stream, const char **kernel_name);

// The circular-buffer form of launch_update (p.seqlens != nullptr).
hipError_t launch_update_ring(const UpdateParams &p, StateLayout layout, int activation, hipStream_t stream,
                              const char **kernel_name);

hipError_t launch_update_tokens(const TokensParams &p, StateLayout layout, int activation, hipStream_t stream,
                                const char **kernel_name);

// The circular-buffer form of launch_update_tokens (p.seqlens != nullptr).
hipError_t launch_update_tokens_ring(const TokensParams &p, StateLayout layout, int activation, hipStream_t stream,
                                     const char **kernel_name);

hipError_t launch_prefill(const PrefillParams &p, StateLayout layout, int activation, hipStream_t stream,
                          const char **kernel_name);

// The measurement control behind dcconv_stream_copy (validated on the host).
hipError_t launch_stream_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream);
hipError_t launch_busy_spin(uint64_t ticks, int waves, hipStream_t stream);

}  // namespace dcconv
