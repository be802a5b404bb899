// Decode-update kernels for gfx950 (CDNA4, wave64).
//
// The operation (cuDNN FE-OSS page "Causal Conv1d Decode Update", section of the
// same name): for row n, channel c and the slot s the row selects, append x[n, c]
// to the slot's length-L history, keep the newest L values, and output
// act(sum_j history[L+1-W+j] * weight[c, j] + bias[c]) with W = 4.
//
// The update is a pure stream: every byte of x, of the selected state and of the
// output is touched exactly once, weight and bias are re-read from L2 by every
// row.  It is bound by HBM bandwidth, so the kernels are organised around
// coalesced 16-byte accesses, not around arithmetic (there is no contraction, so
// no MFMA).
//
//  * update_compact_v8<L, ACT>: the fast path for the compact [S, D, L] layout.
//    One wavefront owns one (row, 512-channel tile); each lane owns 8 adjacent
//    channels, so x, weight, bias and out move as one 16-byte vector per lane.
//    The tile's state is a contiguous 1 KiB * L run.  It is loaded with L fully
//    coalesced 16-byte loads per lane into a per-wave LDS buffer, read back in
//    per-lane channel order, shifted in registers, written back to LDS and
//    stored with L coalesced 16-byte stores.  Waves never share LDS, so the only
//    synchronisation is wave-local.
//  * update_channel_last_v8<ACT>: the [S, L, D] layout a prefill hands over.
//    Every history position is a contiguous plane over channels, so the lane
//    that owns 8 channels loads and stores each plane with one coalesced 16-byte
//    access and the shift is a plane renaming; no LDS is needed.
//  * update_scalar<ACT>: one thread per (row, channel), any stride, any L >= 3,
//    any D.  Serves what the vector paths do not (D or row stride not a multiple
//    of 8, L > 8).
//
// Routing is resolved per wavefront: the slot index is wave-uniform, so a padding
// or rejected row is one uniform branch that writes zeros and touches no state.
#include <stdint.h>

#include "dcconv.h"
#include "update_params.h"

namespace dcconv {
namespace {

constexpr int kWave = 64;
constexpr int kChPerLane = 8;                   // one 16-byte BF16 vector
constexpr int kChPerWave = kWave * kChPerLane;  // 512 channels
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kScalarTile = kBlock;             // channels per block in the scalar path
constexpr int64_t kMaxBlocks = 1 << 20;         // grid cap; the kernels stride over units

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Two FP32 values -> one word holding two BF16 (round to nearest even; gfx950
// converts a pair in one instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float v) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));
}

template <int ACT>
__device__ __forceinline__ float activate(float a);
template <>
__device__ __forceinline__ float activate<DCCONV_ACT_IDENTITY>(float a) {
    return a;
}
template <>
__device__ __forceinline__ float activate<DCCONV_ACT_SILU>(float a) {
    return a / (1.0f + __expf(-a));  // SiLU(a) = a / (1 + e^-a)
}

// Orders this wave's LDS accesses across lanes.  LDS instructions of one
// wavefront execute in order, so wavefront-scope fences (which keep the compiler
// from moving LDS accesses across this point) are all that is needed.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Slot of `row`, or -1 when the row must not touch the state (a padding row, an
// out-of-range index, or -- when a status word is given -- a slot another row of
// the batch also selects).  Must be called by all 64 lanes of the wave; the
// result is wave-uniform.
__device__ __forceinline__ int route_row(const UpdateParams &p, int row, int lane) {
    if (p.idx == nullptr) return row;
    const int slot = p.idx[row];
    if (slot == -1) return -1;
    if (slot < -1 || slot >= p.s) {
        if (p.status != nullptr && lane == 0) atomicOr(p.status, DCCONV_DEV_BAD_INDEX);
        return -1;
    }
    if (p.status != nullptr) {
        bool hit = false;
        for (int base = 0; base < p.n; base += kWave) {
            const int r = base + lane;
            if (r < p.n && r != row && p.idx[r] == slot) hit = true;
        }
        if (__any(hit)) {
            if (lane == 0) atomicOr(p.status, DCCONV_DEV_DUP_INDEX);
            return -1;
        }
    }
    return slot;
}

// 16-bit element e of a register array of packed BF16 pairs (e is a constant
// after unrolling, so this folds to a shift or a mask).
template <int NW>
__device__ __forceinline__ uint32_t elem(const uint32_t (&w)[NW], int e) {
    return (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
}

// The arithmetic for the 8 channels a lane owns.
//   hist[8*L]: the old state of the 8 channels, channel-major (oldest first)
//   xw[4], ww[16], bw[4]: x, weight [8][4] and bias of the 8 channels
// Produces the 8 outputs (packed) and the new state (same order as hist).
template <int L, int ACT>
__device__ __forceinline__ void update8(const uint32_t (&hist)[4 * L], const uint32_t (&xw)[4],
                                        const uint32_t (&ww)[16], const uint32_t (&bw)[4],
                                        bool has_bias, uint32_t (&outw)[4],
                                        uint32_t (&nhist)[4 * L]) {
    float y[kChPerLane];
#pragma unroll
    for (int c = 0; c < kChPerLane; ++c) {
        // history[L+1-W+j] for W = 4: the newest three state values, then x.
        const float h0 = bf16_bits_to_f32(elem(hist, c * L + L - 3));
        const float h1 = bf16_bits_to_f32(elem(hist, c * L + L - 2));
        const float h2 = bf16_bits_to_f32(elem(hist, c * L + L - 1));
        const float h3 = bf16_bits_to_f32(elem(xw, c));
        // BF16 x BF16 products are exact in FP32, so the fused multiply-adds give
        // the same bits as separate products summed from j = 0 upward.
        float acc = h0 * bf16_bits_to_f32(elem(ww, 4 * c + 0));
        acc = __builtin_fmaf(h1, bf16_bits_to_f32(elem(ww, 4 * c + 1)), acc);
        acc = __builtin_fmaf(h2, bf16_bits_to_f32(elem(ww, 4 * c + 2)), acc);
        acc = __builtin_fmaf(h3, bf16_bits_to_f32(elem(ww, 4 * c + 3)), acc);
        if (has_bias) acc += bf16_bits_to_f32(elem(bw, c));
        y[c] = activate<ACT>(acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) outw[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    // New state: each channel's history moves one place towards the oldest end
    // and x becomes the newest value.  Bit copies only.
#pragma unroll
    for (int i = 0; i < 4 * L; ++i) {
        uint32_t half[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = 2 * i + k;
            half[k] = (e % L == L - 1) ? elem(xw, e / L) : elem(hist, e + 1);
        }
        nhist[i] = half[0] | (half[1] << 16);
    }
}

__device__ __forceinline__ void unpack4(const uint4 &v, uint32_t *w) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
}

template <int L, int ACT>
__global__ __launch_bounds__(kBlock) void update_compact_v8(UpdateParams p, int tiles_per_row,
                                                            int64_t units) {
    __shared__ uint4 stage_all[kWavesPerBlock][kWave * L];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    uint4 *stage = stage_all[wave];

    for (int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + wave; unit < units;
         unit += (int64_t)gridDim.x * kWavesPerBlock) {
        const int row = (int)(unit / tiles_per_row);
        const int c0 = (int)(unit - (int64_t)row * tiles_per_row) * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const bool owns = lane < lanes_used;
        uint4 *out_v = reinterpret_cast<uint4 *>(p.out + (int64_t)row * p.d + c0) + lane;

        const int slot = route_row(p, row, lane);
        if (slot < 0) {
            if (owns) *out_v = make_uint4(0u, 0u, 0u, 0u);
            continue;
        }

        // Issue every load of the unit before any use.
        uint4 *chunks = reinterpret_cast<uint4 *>(p.state + (int64_t)slot * p.st_s + (int64_t)c0 * L);
        const int n_chunks = lanes_used * L;
        uint4 sv[L];
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int g = j * kWave + lane;
            sv[j] = g < n_chunks ? chunks[g] : make_uint4(0u, 0u, 0u, 0u);
        }
        uint4 xv = make_uint4(0u, 0u, 0u, 0u), bv = make_uint4(0u, 0u, 0u, 0u);
        uint4 wv[4] = {};
        const bool has_bias = p.bias != nullptr;
        if (owns) {
            const int c = c0 + lane * kChPerLane;
            xv = *reinterpret_cast<const uint4 *>(p.x + (int64_t)row * p.ld + c);
            const uint4 *wp = reinterpret_cast<const uint4 *>(p.weight + (int64_t)c * 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) wv[k] = wp[k];
            if (has_bias) bv = *reinterpret_cast<const uint4 *>(p.bias + c);
        }

        // Coalesced chunk order -> per-lane channel order, through LDS.
#pragma unroll
        for (int j = 0; j < L; ++j) stage[j * kWave + lane] = sv[j];
        wave_lds_sync();
        uint32_t hist[4 * L];
#pragma unroll
        for (int k = 0; k < L; ++k) unpack4(stage[lane * L + k], &hist[4 * k]);

        uint32_t xw[4], ww[16], bw[4], outw[4], nhist[4 * L];
        unpack4(xv, xw);
        unpack4(bv, bw);
#pragma unroll
        for (int k = 0; k < 4; ++k) unpack4(wv[k], &ww[4 * k]);
        update8<L, ACT>(hist, xw, ww, bw, has_bias, outw, nhist);

        // Per-lane channel order -> coalesced chunk order, through LDS.
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < L; ++k)
            stage[lane * L + k] = make_uint4(nhist[4 * k], nhist[4 * k + 1], nhist[4 * k + 2], nhist[4 * k + 3]);
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < L; ++j) {
            const int g = j * kWave + lane;
            const uint4 v = stage[g];
            if (g < n_chunks) chunks[g] = v;
        }
        if (owns) *out_v = make_uint4(outw[0], outw[1], outw[2], outw[3]);
        wave_lds_sync();  // the stage is reused by the next unit
    }
}

template <int ACT>
__global__ __launch_bounds__(kBlock) void update_channel_last_v8(UpdateParams p, int tiles_per_row,
                                                                 int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    for (int64_t unit = (int64_t)blockIdx.x * kWavesPerBlock + wave; unit < units;
         unit += (int64_t)gridDim.x * kWavesPerBlock) {
        const int row = (int)(unit / tiles_per_row);
        const int c0 = (int)(unit - (int64_t)row * tiles_per_row) * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const bool owns = lane < lanes_used;
        uint4 *out_v = reinterpret_cast<uint4 *>(p.out + (int64_t)row * p.d + c0) + lane;

        const int slot = route_row(p, row, lane);
        if (!owns) continue;
        if (slot < 0) {
            *out_v = make_uint4(0u, 0u, 0u, 0u);
            continue;
        }
        const int c = c0 + lane * kChPerLane;
        const int L = p.l;
        uint16_t *base = p.state + (int64_t)slot * p.st_s + c;  // plane k at base + k * st_l
        // The dot product needs planes L-3..L-1; the shift needs planes 1..L-1.
        const uint4 xv = *reinterpret_cast<const uint4 *>(p.x + (int64_t)row * p.ld + c);
        const uint4 *wp = reinterpret_cast<const uint4 *>(p.weight + (int64_t)c * 4);
        uint4 wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) wv[k] = wp[k];
        const bool has_bias = p.bias != nullptr;
        const uint4 bv = has_bias ? *reinterpret_cast<const uint4 *>(p.bias + c) : make_uint4(0u, 0u, 0u, 0u);
        uint4 p3 = *reinterpret_cast<const uint4 *>(base + (int64_t)(L - 3) * p.st_l);
        uint4 p2 = *reinterpret_cast<const uint4 *>(base + (int64_t)(L - 2) * p.st_l);
        uint4 p1 = *reinterpret_cast<const uint4 *>(base + (int64_t)(L - 1) * p.st_l);

        // Channel-major history of the 8 channels with L' = 3 (the three planes
        // the taps read), so update8<3> does the arithmetic.
        uint32_t hist[12], xw[4], ww[16], bw[4], outw[4], nhist[12];
        uint32_t a[4], b[4], cc[4];
        unpack4(p3, a); unpack4(p2, b); unpack4(p1, cc);
#pragma unroll
        for (int ch = 0; ch < kChPerLane; ++ch) {
            const uint32_t va = elem(a, ch), vb = elem(b, ch), vc = elem(cc, ch);
            const int e = 3 * ch;
            // place (va, vb, vc) at elements e, e+1, e+2
            const uint32_t vals[3] = {va, vb, vc};
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int ei = e + k;
                if (ei & 1) hist[ei >> 1] = (hist[ei >> 1] & 0xFFFFu) | (vals[k] << 16);
                else hist[ei >> 1] = vals[k];
            }
        }
        unpack4(xv, xw); unpack4(bv, bw);
#pragma unroll
        for (int k = 0; k < 4; ++k) unpack4(wv[k], &ww[4 * k]);
        update8<3, ACT>(hist, xw, ww, bw, has_bias, outw, nhist);

        // Shift: plane k <- plane k+1 for k < L-1, plane L-1 <- x.  Planes below
        // L-3 are moved without being part of the arithmetic.
        for (int k = 0; k < L - 3; ++k) {
            const uint4 v = *reinterpret_cast<const uint4 *>(base + (int64_t)(k + 1) * p.st_l);
            *reinterpret_cast<uint4 *>(base + (int64_t)k * p.st_l) = v;
        }
        *reinterpret_cast<uint4 *>(base + (int64_t)(L - 3) * p.st_l) = p2;
        *reinterpret_cast<uint4 *>(base + (int64_t)(L - 2) * p.st_l) = p1;
        *reinterpret_cast<uint4 *>(base + (int64_t)(L - 1) * p.st_l) = xv;
        *out_v = make_uint4(outw[0], outw[1], outw[2], outw[3]);
    }
}

template <int ACT>
__global__ __launch_bounds__(kBlock) void update_scalar(UpdateParams p, int tiles_per_row, int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    for (int64_t unit = blockIdx.x; unit < units; unit += gridDim.x) {
        const int row = (int)(unit / tiles_per_row);
        const int c = (int)(unit - (int64_t)row * tiles_per_row) * kScalarTile + (int)threadIdx.x;
        const int slot = route_row(p, row, lane);
        if (c >= p.d) continue;
        uint16_t *o = p.out + (int64_t)row * p.d + c;
        if (slot < 0) {
            *o = 0;
            continue;
        }
        const int L = p.l;
        uint16_t *h = p.state + (int64_t)slot * p.st_s + (int64_t)c * p.st_d;
        const int64_t sl = p.st_l;
        const uint32_t x = p.x[(int64_t)row * p.ld + c];
        const float h0 = bf16_bits_to_f32(h[(L - 3) * sl]);
        const float h1 = bf16_bits_to_f32(h[(L - 2) * sl]);
        const float h2 = bf16_bits_to_f32(h[(L - 1) * sl]);
        for (int k = 0; k < L - 1; ++k) h[k * sl] = h[(k + 1) * sl];
        h[(L - 1) * sl] = (uint16_t)x;
        const uint16_t *wt = p.weight + (int64_t)c * 4;
        float acc = h0 * bf16_bits_to_f32(wt[0]);
        acc = __builtin_fmaf(h1, bf16_bits_to_f32(wt[1]), acc);
        acc = __builtin_fmaf(h2, bf16_bits_to_f32(wt[2]), acc);
        acc = __builtin_fmaf(bf16_bits_to_f32(x), bf16_bits_to_f32(wt[3]), acc);
        if (p.bias != nullptr) acc += bf16_bits_to_f32(p.bias[c]);
        *o = f32_to_bf16_bits(activate<ACT>(acc));
    }
}

template <typename Kernel>
hipError_t launch(Kernel kernel, const UpdateParams &p, int tiles_per_row, int64_t units,
                  int64_t units_per_block, hipStream_t stream) {
    int64_t blocks = (units + units_per_block - 1) / units_per_block;
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    UpdateParams args_p = p;
    void *args[] = {&args_p, &tiles_per_row, &units};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks), dim3(kBlock),
                           args, 0, stream);
}

template <int ACT>
hipError_t launch_compact_v8(const UpdateParams &p, int tiles, int64_t units, hipStream_t stream,
                             const char **name) {
#define DCCONV_CASE(LL)                                                                  \
    case LL:                                                                             \
        *name = ACT ? "update_compact_v8<L=" #LL ",silu>" : "update_compact_v8<L=" #LL ",identity>"; \
        return launch(update_compact_v8<LL, ACT>, p, tiles, units, kWavesPerBlock, stream);
    switch (p.l) {
        DCCONV_CASE(3)
        DCCONV_CASE(4)
        DCCONV_CASE(5)
        DCCONV_CASE(6)
        DCCONV_CASE(7)
        DCCONV_CASE(8)
        default:
            return hipErrorInvalidValue;
    }
#undef DCCONV_CASE
}

}  // namespace

hipError_t launch_update(const UpdateParams &p, StateLayout layout, int activation, hipStream_t stream,
                         const char **kernel_name) {
    const bool rows_v8 = (p.d % kChPerLane == 0) && (p.ld % kChPerLane == 0);
    const bool silu = activation == DCCONV_ACT_SILU;
    if (layout == StateLayout::Compact && rows_v8 && p.st_s % kChPerLane == 0 && p.l >= 3 && p.l <= 8) {
        const int tiles = (p.d + kChPerWave - 1) / kChPerWave;
        const int64_t units = (int64_t)p.n * tiles;
        return silu ? launch_compact_v8<DCCONV_ACT_SILU>(p, tiles, units, stream, kernel_name)
                    : launch_compact_v8<DCCONV_ACT_IDENTITY>(p, tiles, units, stream, kernel_name);
    }
    if (layout == StateLayout::ChannelLast && rows_v8 && p.st_s % kChPerLane == 0) {
        const int tiles = (p.d + kChPerWave - 1) / kChPerWave;
        const int64_t units = (int64_t)p.n * tiles;
        *kernel_name = silu ? "update_channel_last_v8<silu>" : "update_channel_last_v8<identity>";
        return silu ? launch(update_channel_last_v8<DCCONV_ACT_SILU>, p, tiles, units, kWavesPerBlock, stream)
                    : launch(update_channel_last_v8<DCCONV_ACT_IDENTITY>, p, tiles, units, kWavesPerBlock, stream);
    }
    const int tiles = (p.d + kScalarTile - 1) / kScalarTile;
    const int64_t units = (int64_t)p.n * tiles;
    *kernel_name = silu ? "update_scalar<silu>" : "update_scalar<identity>";
    return silu ? launch(update_scalar<DCCONV_ACT_SILU>, p, tiles, units, 1, stream)
                : launch(update_scalar<DCCONV_ACT_IDENTITY>, p, tiles, units, 1, stream);
}

}  // namespace dcconv
