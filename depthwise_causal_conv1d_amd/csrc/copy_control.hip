// Measurement control: a plain device copy with the access pattern of the
// update kernels, so a benchmark can time the bandwidth ceiling of the same
// bytes in the same run (page "Composing multi-kernel blocks in Python",
// section "Measuring a block honestly": an op-by-op baseline beside the
// measured block).
//
// A block of one wavefront copies 8 KiB: each lane loads eight 16-byte
// vectors (every load instruction covers one contiguous KiB), then stores the
// eight.  Loads and stores carry the non-temporal hint the update kernels use
// for their single-use streams, and a raw buffer descriptor bounds the block's
// piece, so a ragged end needs no branch.  A 16.8 MB copy is then about 2048
// waves, as the large decode update is; of the shapes tried for a 16.8 MB copy
// (1, 2 or 4 waves per block, 1 to 16 vectors per lane) this one was the
// fastest.
//
// A second control, busy_spin, keeps every SIMD busy with arithmetic for a
// given time: enqueued ahead of a timed region it lets the host enqueue the
// region's launches while the chip stays at its working clocks.
#include <stdint.h>

#include "dcconv.h"
#include "device_common.h"

namespace dcconv {
namespace {

constexpr int kCopyVecsPerLane = 8;
constexpr int64_t kCopyBlockBytes = (int64_t)kWave * kCopyVecsPerLane * 16;  // 8 KiB

__global__ __launch_bounds__(kWave) void stream_copy_v8(uint8_t *dst, const uint8_t *src, int64_t bytes,
                                                        int64_t blocks) {
    const int lane = threadIdx.x;
    int64_t b = blockIdx.x;
    do {
        const int64_t base = b * kCopyBlockBytes;
        const int64_t left = bytes - base;
        const uint32_t piece = (uint32_t)(left < kCopyBlockBytes ? left : kCopyBlockBytes);
        const Buffer in = make_buffer(src + base, piece);
        const Buffer out = make_buffer(dst + base, piece);
        u32x4 v[kCopyVecsPerLane];
#pragma unroll
        for (int k = 0; k < kCopyVecsPerLane; ++k)
            v[k] = buffer_load<kStream>(in, (uint32_t)((k * kWave + lane) * 16));
#pragma unroll
        for (int k = 0; k < kCopyVecsPerLane; ++k)
            buffer_store<kStream>(v[k], out, (uint32_t)((k * kWave + lane) * 16));
        b += kMaxBlocks;
    } while (b < blocks);
}

// Measurement control: every wave runs FP32 FMAs until `ticks` of the
// constant-rate wall clock have passed since it started, so the whole chip is
// busy for the span (a benchmark's head ahead of a timed region).  The chain's
// result feeds an empty asm statement, which keeps the loop without a store.
__global__ __launch_bounds__(kWave) void busy_spin(uint64_t ticks) {
    const uint64_t t0 = wall_clock64();
    float a = (float)threadIdx.x * 1e-3f;
    do {
#pragma unroll
        for (int i = 0; i < 32; ++i) a = __builtin_fmaf(a, 1.0000001f, 1e-7f);
    } while (wall_clock64() - t0 < ticks);
    asm volatile("" : : "v"(a));
}

}  // namespace

hipError_t launch_busy_spin(uint64_t ticks, int waves, hipStream_t stream) {
    void *args[] = {&ticks};
    return hipLaunchKernel(reinterpret_cast<const void *>(busy_spin), dim3((unsigned)waves), dim3(kWave), args, 0,
                           stream);
}

hipError_t launch_stream_copy(void *dst, const void *src, int64_t bytes, hipStream_t stream) {
    int64_t blocks = (bytes + kCopyBlockBytes - 1) / kCopyBlockBytes;
    const int64_t grid = blocks < kMaxBlocks ? blocks : kMaxBlocks;
    uint8_t *d = static_cast<uint8_t *>(dst);
    const uint8_t *s = static_cast<const uint8_t *>(src);
    void *args[] = {&d, &s, &bytes, &blocks};
    return hipLaunchKernel(reinterpret_cast<const void *>(stream_copy_v8), dim3((unsigned)grid), dim3(kWave), args,
                           0, stream);
}

}  // namespace dcconv
