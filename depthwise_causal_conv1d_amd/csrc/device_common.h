// Device helpers shared by the gfx950 kernels of this library (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcconv.h"

namespace dcconv {
namespace {

constexpr int kWave = 64;
constexpr int kChPerLane = 8;                   // one 16-byte BF16 vector
constexpr int kChPerWave = kWave * kChPerLane;  // 512 channels
constexpr int kWavesPerBlock = 2;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kScalarBlock = 256;               // channels per block in the scalar path
constexpr int64_t kMaxBlocks = 1 << 20;         // grid cap: min(units, kMaxBlocks) blocks, stride kMaxBlocks
// Two rows per wave once the grid still has this many waves: fewer, fuller waves
// keep more bytes in flight per wave and share one weight load between rows.
constexpr int64_t kMinWavesForTwoRows = 1024;
// The one-token update spreads a batch over 128-channel waves (the narrow form)
// when its 512-channel grid, rows x tiles, holds at most this many waves.
constexpr int64_t kNarrowMaxWaves = 512;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Raw buffer accesses: a descriptor holds a base address and a byte count, and
// the hardware turns any access at or beyond the count into a zero read or a
// dropped write.  Word 3 is the gfx9 raw-buffer format (32-bit data format).
typedef __amdgpu_buffer_rsrc_t Buffer;
constexpr int kBufferWord3 = 0x00020000;
// Cache policies: single-use streams (x, state, out) carry the non-temporal
// hint, which keeps them out of the Infinity Cache and from displacing reused
// data; weights and bias use the default policy.
constexpr int kCached = 0;  // cache policy: default
constexpr int kStream = 2;  // cache policy: non-temporal
__device__ __forceinline__ Buffer make_buffer(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, kBufferWord3);
}
template <int POLICY>
__device__ __forceinline__ u32x4 buffer_load(Buffer b, uint32_t offset) {
    return __builtin_amdgcn_raw_buffer_load_b128(b, offset, 0, POLICY);
}
template <int POLICY>
__device__ __forceinline__ void buffer_store(u32x4 v, Buffer b, uint32_t offset) {
    __builtin_amdgcn_raw_buffer_store_b128(v, b, offset, 0, POLICY);
}

// NW consecutive 32-bit words at byte `offset` of a buffer, moved with the widest
// accesses that fit (16, 12, 8 or 4 bytes), so a lane's run of 4*NW bytes is
// one access when NW <= 4.
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int NW, int POLICY>
__device__ __forceinline__ void buffer_load_words(Buffer b, uint32_t offset, uint32_t (&w)[NW]) {
#pragma unroll
    for (int i = 0; i < NW; i += 4) {
        const uint32_t at = offset + 4u * (uint32_t)i;
        if (NW - i >= 4) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(b, at, 0, POLICY);
            w[i] = v[0], w[i + 1] = v[1], w[i + 2] = v[2], w[i + 3] = v[3];
        } else if (NW - i == 3) {
            const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(b, at, 0, POLICY);
            w[i] = v[0], w[i + 1] = v[1], w[i + 2] = v[2];
        } else if (NW - i == 2) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(b, at, 0, POLICY);
            w[i] = v[0], w[i + 1] = v[1];
        } else {
            w[i] = __builtin_amdgcn_raw_buffer_load_b32(b, at, 0, POLICY);
        }
    }
}
template <int NW, int POLICY>
__device__ __forceinline__ void buffer_store_words(const uint32_t (&w)[NW], Buffer b, uint32_t offset) {
#pragma unroll
    for (int i = 0; i < NW; i += 4) {
        const uint32_t at = offset + 4u * (uint32_t)i;
        if (NW - i >= 4) {
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[i], w[i + 1], w[i + 2], w[i + 3]}, b, at, 0, POLICY);
        } else if (NW - i == 3) {
            __builtin_amdgcn_raw_buffer_store_b96(u32x3{w[i], w[i + 1], w[i + 2]}, b, at, 0, POLICY);
        } else if (NW - i == 2) {
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{w[i], w[i + 1]}, b, at, 0, POLICY);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(w[i], b, at, 0, POLICY);
        }
    }
}

// BF16 held in the low / high half of a 32-bit word, as FP32 (exact).
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

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
// SiLU(a) = a / (1 + e^-a), with the hardware base-2 exponential and reciprocal
// (each within about one FP32 ulp; the result is far inside one BF16 ulp).
// a -> -inf gives a * rcp(inf) = -0, a -> +inf gives a.
template <>
__device__ __forceinline__ float activate<DCCONV_ACT_SILU>(float a) {
    constexpr float kMinusLog2e = -1.4426950408889634f;
    return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * kMinusLog2e));
}

// Calls body(u) for the units u = blockIdx.x, blockIdx.x + kMaxBlocks, ... below
// `units`.  Every kernel here is launched with min(units, kMaxBlocks) blocks, so
// the first unit needs no test and the stride is the constant kMaxBlocks (one
// pass when units <= kMaxBlocks).  Neither the unit count nor the grid size is
// then needed before the first load: every kernel argument is requested at
// once, one round trip instead of two.
template <typename Body>
__device__ __forceinline__ void for_each_unit(int64_t units, Body &&body) {
    int64_t u = blockIdx.x;
    do {
        body(u);
        u += kMaxBlocks;
    } while (u < units);
}

// Orders this wave's LDS accesses across lanes.  LDS instructions of one
// wavefront execute in order, so wavefront-scope fences (which keep the compiler
// from moving LDS accesses across this point) are all that is needed.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Element i of an int32 table the kernel never writes, for a wave-uniform i:
// read through the constant address space, so it is a scalar load whose wait
// does not drain the vector loads in flight (a plain load issued after a store
// of the kernel cannot be proven unclobbered and becomes a vector load).
__device__ __forceinline__ int32_t load_uniform(const int32_t *table, int i) {
    return ((const __attribute__((address_space(4))) int32_t *)table)[i];
}

// Slot of `row`, or -1 when the row must not touch the state (a padding row, an
// out-of-range index, or -- when a status word is given -- a slot another row of
// the batch also selects).  idx/status may be null.  Must be called by all 64
// lanes of the wave; the result is wave-uniform.
__device__ __forceinline__ int route_row(const int32_t *idx, int32_t *status, int n_rows, int n_slots, int row,
                                         int lane) {
    if (idx == nullptr) return row;
    const int slot = load_uniform(idx, row);
    if (slot == -1) return -1;
    if (slot < -1 || slot >= n_slots) {
        if (status != nullptr && lane == 0) atomicOr(status, DCCONV_DEV_BAD_INDEX);
        return -1;
    }
    if (status != nullptr) {
        bool hit = false;
        for (int base = 0; base < n_rows; base += kWave) {
            const int r = base + lane;
            if (r < n_rows && r != row && idx[r] == slot) hit = true;
        }
        if (__any(hit)) {
            if (lane == 0) atomicOr(status, DCCONV_DEV_DUP_INDEX);
            return -1;
        }
    }
    return slot;
}

// 16-bit element e of an array of packed BF16 pairs, as FP32 (e is a constant
// after unrolling, so this folds to one shift or mask).
template <int NW>
__device__ __forceinline__ float elem_f32(const uint32_t (&w)[NW], int e) {
    return (e & 1) ? hi_f32(w[e >> 1]) : lo_f32(w[e >> 1]);
}


// ---- the block-shared weight tile -------------------------------------------
// A block's waves share one 512-channel tile, whose weights (4 KiB) are fetched
// once per block with coalesced loads and passed to every lane through LDS.
// 16-byte unit u of the tile holds lane u/4's taps for channels 2(u%4), 2(u%4)+1
// of its 8; it is stored at u ^ ((u >> 4) & 3), which keeps both the coalesced
// writes and the per-lane reads (stride 64 bytes) free of LDS bank conflicts.
constexpr int kWeightChunks = 4 / kWavesPerBlock;  // 1-KiB pieces of the tile per wave

__device__ __forceinline__ void weight_tile_issue(u32x4 (&raw)[kWeightChunks], const uint16_t *weight, int c0,
                                                  uint32_t vec_bytes, int wave, uint32_t lane_bytes) {
    const Buffer wbuf = make_buffer(weight + (int64_t)c0 * 4, vec_bytes * 4u);
#pragma unroll
    for (int q = 0; q < kWeightChunks; ++q)
        raw[q] = buffer_load<kCached>(wbuf, (uint32_t)((wave * kWeightChunks + q) * 1024) + lane_bytes);
}

// Publishes this wave's pieces, waits for the whole block, and returns this
// lane's 32 taps (channel-major) as FP32.
__device__ __forceinline__ void weight_tile_share(u32x4 *tile, const u32x4 (&raw)[kWeightChunks], int wave, int lane,
                                                  float (&wf)[32]) {
#pragma unroll
    for (int q = 0; q < kWeightChunks; ++q) {
        const int u = (wave * kWeightChunks + q) * kWave + lane;
        tile[u ^ ((u >> 4) & 3)] = raw[q];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int u = 4 * lane + k;
        const u32x4 wk = tile[u ^ ((u >> 4) & 3)];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wf[8 * k + 2 * q] = lo_f32(wk[q]);
            wf[8 * k + 2 * q + 1] = hi_f32(wk[q]);
        }
    }
}

// ---- the compact-state stage ----------------------------------------------------
// A wave moves a tile's compact state (L 16-byte chunks per lane) through LDS
// between coalesced order (chunk j*64 + lane, as it is loaded and stored) and
// per-lane order (chunk lane*L + k: the lane's 8 channels).  A per-lane access
// steps L chunks from lane to lane; at L = 8 (128 bytes) that puts every lane
// of a 16-byte access on the same LDS banks, so the stage keeps a pitch of 9
// chunks per lane there: chunk c of the coalesced order sits at c + c / 8.
// (Smaller even L conflict less and gain nothing from a pitch of L + 1, which
// costs LDS: at L = 4 a two-row block would grow from 20 to 24 KiB.)
template <int L>
constexpr int stage_pitch() {
    return L == 8 ? L + 1 : L;
}
template <int L>
constexpr int stage_chunks() {
    return kWave * stage_pitch<L>();
}
template <int L>
__device__ __forceinline__ int stage_coalesced(int j, int lane) {
    const int c = j * kWave + lane;
    return stage_pitch<L>() == L ? c : c + c / L;
}
template <int L>
__device__ __forceinline__ int stage_lane(int lane, int k) {
    return lane * stage_pitch<L>() + k;
}

// ---- history planes -----------------------------------------------------------
// A lane's 8 channels of one history position form a "plane" vector (word q
// holds channels 2q, 2q+1).  The compact state holds the same values
// channel-major (channel c, position k at element c*L + k of the lane's run).

// Two 16-bit halves -> one word: the half `half_lo` of `lo_src` becomes the low
// half, the half `half_hi` of `hi_src` the high half (one v_perm_b32).
__device__ __forceinline__ uint32_t pick_halves(uint32_t lo_src, int half_lo, uint32_t hi_src, int half_hi) {
    const uint32_t sel_lo = half_lo ? 0x0302u : 0x0100u;  // bytes of the second operand
    const uint32_t sel_hi = half_hi ? 0x0706u : 0x0504u;  // bytes of the first operand
    return __builtin_amdgcn_perm(hi_src, lo_src, (sel_hi << 16) | sel_lo);
}

__device__ __forceinline__ float half_f32(uint32_t w, int half) { return half ? hi_f32(w) : lo_f32(w); }

// Channel-major words (channel c, position k at element c*L + k) -> planes
// (plane k, word q holds channels 2q, 2q+1 at position k), and back.
template <int L>
__device__ __forceinline__ void to_planes(const uint32_t (&h)[4 * L], u32x4 (&pl)[L]) {
#pragma unroll
    for (int k = 0; k < L; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e_lo = (2 * q) * L + k, e_hi = (2 * q + 1) * L + k;
            pl[k][q] = pick_halves(h[e_lo >> 1], e_lo & 1, h[e_hi >> 1], e_hi & 1);
        }
}
template <int L>
__device__ __forceinline__ void from_planes(const u32x4 (&pl)[L], uint32_t (&h)[4 * L]) {
#pragma unroll
    for (int i = 0; i < 4 * L; ++i) {
        const int e0 = 2 * i, e1 = 2 * i + 1;
        const int c0 = e0 / L, k0 = e0 % L, c1 = e1 / L, k1 = e1 % L;
        h[i] = pick_halves(pl[k0][c0 >> 1], c0 & 1, pl[k1][c1 >> 1], c1 & 1);
    }
}

__device__ __forceinline__ void unpack_bias(const u32x4 &bv, float (&bf)[8]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        bf[2 * q] = lo_f32(bv[q]);
        bf[2 * q + 1] = hi_f32(bv[q]);
    }
}

// out = act(w0*h0 + w1*h1 + w2*h2 + w3*xt + b) for the lane's 8 channels, in
// the oracle's order (taps ascending, bias last); BF16 products are exact.
template <int ACT>
__device__ __forceinline__ u32x4 conv8(const u32x4 &h0, const u32x4 &h1, const u32x4 &h2, const u32x4 &xt,
                                       const float (&wf)[32], const float (&bf)[8]) {
    float y[kChPerLane];
#pragma unroll
    for (int ch = 0; ch < kChPerLane; ++ch) {
        const int q = ch >> 1, hh = ch & 1;
        float acc = half_f32(h0[q], hh) * wf[4 * ch + 0];
        acc = __builtin_fmaf(half_f32(h1[q], hh), wf[4 * ch + 1], acc);
        acc = __builtin_fmaf(half_f32(h2[q], hh), wf[4 * ch + 2], acc);
        acc = __builtin_fmaf(half_f32(xt[q], hh), wf[4 * ch + 3], acc);
        acc += bf[ch];
        y[ch] = activate<ACT>(acc);
    }
    return u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}


// ---- host side: the launch shape of the one-token kernels --------------------

// Compute units of the current device (cached per device; 0 if unknown).
constexpr int kMaxCachedDevices = 64;
inline int64_t device_cu_count() {
    static int cache[kMaxCachedDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxCachedDevices) {
        const int c = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 0;
    if (dev < kMaxCachedDevices) __atomic_store_n(&cache[dev], cus, __ATOMIC_RELAXED);
    return cus;
}

// Whether the one-token kernels take two rows per wave for n rows of `tiles`
// 512-channel tiles.  Only when the grid keeps kMinWavesForTwoRows waves, and
// only when the blocks, spread over the CUs in whole rounds, do not cost more
// rounds x rows than one row per wave would: with C CUs, ceil(blocks_2 / C) * 2
// against ceil(blocks_1 / C).  (N = 160, D = 8192: 640 two-row blocks in 3
// rounds of 2 rows against 1280 one-row blocks in 5 rounds; 5.44 against
// 5.06 us measured.  N = 256: 4 x 2 against 8, a tie, and two rows win:
// 6.24 against 6.34-6.41 us.)
inline bool two_rows_per_wave(int64_t n, int64_t tiles) {
    const int64_t groups_two = (n + 1) / 2;
    if (n < 2 || groups_two * tiles < kMinWavesForTwoRows) return false;
    const int64_t cus = device_cu_count();
    if (cus <= 0) return true;
    const int64_t blocks_one = tiles * ((n + kWavesPerBlock - 1) / kWavesPerBlock);
    const int64_t blocks_two = tiles * ((groups_two + kWavesPerBlock - 1) / kWavesPerBlock);
    return (blocks_two + cus - 1) / cus * 2 <= (blocks_one + cus - 1) / cus;
}

}  // namespace
}  // namespace dcconv
