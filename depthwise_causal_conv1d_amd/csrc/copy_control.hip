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

}  // namespace

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
