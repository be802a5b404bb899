// Decode step on circular-buffer state (cache_seqlens) for gfx950.
//
// The cuDNN FE-OSS page "Causal Conv1d Decode Update" reserves cache_seqlens for
// circular-buffer state (section "Causal Conv1d Decode Update").  Ring reading:
// a slot whose row has seen c = cache_seqlens[n] tokens keeps token i at
// position i mod L.  The step's taps are tokens c-3, c-2, c-1 (positions
// (c-3+k) mod L) and x; x then replaces the oldest token, at position c mod L.
// Only one value per channel is written, instead of the L a shifting update
// rewrites.
//
//  * update_ring_v8<ACT, R, HAS_BIAS, L3, INDEXED>: channel-last state, where each position is
//    a contiguous plane, so a row reads 3 planes and writes 1.  One wavefront
//    per (R rows, 512-channel tile), 8 channels per lane, the block's waves
//    sharing the tile's weights; every load is issued before the first row is
//    computed and every store after the last (the structure of the shifting
//    update's kernels).
//  * update_ring_scalar<ACT>: one thread per (row, channel), any layout.
//  * tokens_ring_v8<ACT, HAS_BIAS> / tokens_ring_scalar<ACT>: T tokens per call
//    on the same ring (the multi-token entry with cache_seqlens).
#include <stdint.h>

#include "dcconv.h"
#include "device_common.h"
#include "update_params.h"

namespace dcconv {
namespace {

constexpr uint32_t kBadLane = 1u << 31;  // beyond every descriptor here (all < 2^30 bytes)

// ((t mod L) + L) mod L for any t: the ring position of token t.
__device__ __forceinline__ int ring_pos(int t, int L) {
    const int r = t % L;
    return r < 0 ? r + L : r;
}

// A routed row's slot after the count check: a negative cache_seqlens entry
// rejects the row (-1) and sets DCCONV_DEV_BAD_SEQLEN.  All 64 lanes of the
// wave call it; the result is wave-uniform.
__device__ __forceinline__ int ring_reject(int32_t *status, int slot, int seen, int lane) {
    if (seen >= 0) return slot;
    if (status != nullptr && lane == 0) atomicOr(status, DCCONV_DEV_BAD_SEQLEN);
    return -1;
}

// The row's slot (or -1 when it must not touch the state) and its count.
__device__ __forceinline__ int route_ring_row(const UpdateParams &p, int row, int lane, int *seen) {
    const int slot = route_row(p.idx, p.status, p.n, p.s, row, lane);
    *seen = p.seqlens[row];
    return ring_reject(p.status, slot, *seen, lane);
}

// L3: the ring holds exactly the W-1 = 3 taps, so the three planes are read in
// plane order whatever the count and rotated afterwards (tap k is plane
// (c + k) mod 3): no load offset depends on the count.
// INDEXED: an index table selects the slots; without one row n is slot n.
// The weights and x need neither the count nor the slot, so they go out before
// the counts are examined; the planes once the slots are known.  (Issuing the
// L3 planes of an unindexed call before the counts too, reading the planes of
// a row its count rejects and writing nothing, measured slower: 5.90 against
// 5.80 us on the large decode batch.)
template <int ACT, int R, bool HAS_BIAS, bool L3, bool INDEXED>
__global__ __launch_bounds__(kBlock) void update_ring_v8(UpdateParams p, int tiles, int64_t block_units) {
    __shared__ u32x4 weight_tile[4 * kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    const uint32_t plane_bytes = (uint32_t)p.st_l * 2u;
    const int L = p.l;

    // A block owns one 512-channel tile and kWavesPerBlock groups of R rows.
    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t bu = blockIdx.x;
    do {
        const int tile = (int)(bu % tiles);
        const int group = (int)(bu / tiles) * kWavesPerBlock + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
        const uint32_t lane_off = lane < lanes_used ? lane_bytes : kBadLane;

        // The rows' counts, all requested before any is examined (scalar loads:
        // one round trip for the wave).
        int seen[R], slot[R], head[R];  // head: ring position of the newest slot value + 1 (= c mod L)
#pragma unroll
        for (int r = 0; r < R; ++r) seen[r] = load_uniform(p.seqlens, min(group * R + r, p.n - 1));

        __builtin_amdgcn_s_setprio(3);
        u32x4 wraw[kWeightChunks];
        weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        Buffer sbuf[R];
        u32x4 h[R][3], xv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool row_ok = group * R + r < p.n;
            const int row = min(group * R + r, p.n - 1);
            xv[r] = buffer_load<kStream>(make_buffer(p.x + (int64_t)row * p.ld + c0, row_ok ? vec_bytes : 0u), lane_off);
        }
        // the slots, once the counts (and index table) are in
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = group * R + r;
            slot[r] = __builtin_amdgcn_readfirstlane(
                row < p.n ? ring_reject(p.status, route_row(INDEXED ? p.idx : nullptr, p.status, p.n, p.s, row, lane),
                                        seen[r], lane)
                          : -2);
            head[r] = (seen[r] < 0 ? 0 : seen[r]) % (L3 ? 3 : L);  // seen >= 0 for a live row
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool live = slot[r] >= 0;
            sbuf[r] = make_buffer(p.state + (int64_t)(live ? slot[r] : 0) * p.st_s + c0,
                                  live ? plane_bytes * (uint32_t)(L - 1) + vec_bytes : 0u);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                // L3: plane k, placed below; else tap k's plane (c - 3 + k) mod L
                const int pos = L3 ? k : (head[r] - 3 + k < 0 ? head[r] - 3 + k + L : head[r] - 3 + k);
                h[r][k] = buffer_load<kStream>(sbuf[r], plane_bytes * (uint32_t)pos + lane_off);
            }
        }
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        __builtin_amdgcn_s_setprio(0);
        if (L3) {
            // tap k of row r is plane (c + k) mod 3: rotate the three planes by head
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const u32x4 p0 = h[r][0], p1 = h[r][1], p2 = h[r][2];
                h[r][0] = head[r] == 0 ? p0 : head[r] == 1 ? p1 : p2;
                h[r][1] = head[r] == 0 ? p1 : head[r] == 1 ? p2 : p0;
                h[r][2] = head[r] == 0 ? p2 : head[r] == 1 ? p0 : p1;
            }
        }

        float wf[32], bf[8];
        weight_tile_share(weight_tile, wraw, wave, lane, wf);
        unpack_bias(bv, bf);
        u32x4 o[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 y = conv8<ACT>(h[r][0], h[r][1], h[r][2], xv[r], wf, bf);
            o[r] = slot[r] >= 0 ? y : u32x4{0u, 0u, 0u, 0u};  // a padding row writes zeros
        }

        // every store last, after the taps are in registers: x overwrites the
        // oldest token, which is tap 0 when L == 3
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = min(group * R + r, p.n - 1);
            buffer_store<kStream>(o[r], make_buffer(p.out + (int64_t)row * p.d + c0, slot[r] != -2 ? vec_bytes : 0u),
                                  lane_off);
            buffer_store<kStream>(xv[r], sbuf[r], plane_bytes * (uint32_t)head[r] + lane_off);
        }
        __syncthreads();  // the weight tile is reused by the next unit
        bu += kMaxBlocks;
    } while (bu < block_units);
}

template <int ACT>
__global__ __launch_bounds__(kScalarBlock) void update_ring_scalar(UpdateParams p, int tiles_per_row, int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    for_each_unit(units, [&](int64_t unit) {
        const int row = (int)(unit / tiles_per_row);
        const int c = (int)(unit - (int64_t)row * tiles_per_row) * kScalarBlock + (int)threadIdx.x;
        int seen = 0;
        const int slot = route_ring_row(p, row, lane, &seen);
        if (c >= p.d) return;
        uint16_t *o = p.out + (int64_t)row * p.d + c;
        if (slot < 0) {
            *o = 0;
            return;
        }
        const int L = p.l;
        uint16_t *ring = p.state + (int64_t)slot * p.st_s + (int64_t)c * p.st_d;
        const int64_t sl = p.st_l;
        const uint16_t xb = p.x[(int64_t)row * p.ld + c];
        const uint16_t *wt = p.weight + (int64_t)c * 4;
        float acc = bf16_bits_to_f32(ring[ring_pos(seen - 3, L) * sl]) * bf16_bits_to_f32(wt[0]);
        acc = __builtin_fmaf(bf16_bits_to_f32(ring[ring_pos(seen - 2, L) * sl]), bf16_bits_to_f32(wt[1]), acc);
        acc = __builtin_fmaf(bf16_bits_to_f32(ring[ring_pos(seen - 1, L) * sl]), bf16_bits_to_f32(wt[2]), acc);
        acc = __builtin_fmaf(bf16_bits_to_f32(xb), bf16_bits_to_f32(wt[3]), acc);
        if (p.bias != nullptr) acc += bf16_bits_to_f32(p.bias[c]);
        *o = f32_to_bf16_bits(activate<ACT>(acc));
        ring[(int64_t)ring_pos(seen, L) * sl] = xb;
    });
}

template <typename Kernel>
hipError_t launch_ring(Kernel kernel, const UpdateParams &p, int tiles, int64_t units, int block,
                       hipStream_t stream) {
    const int64_t blocks = units < kMaxBlocks ? units : kMaxBlocks;
    UpdateParams args_p = p;
    int tiles_arg = tiles;
    int64_t units_arg = units;
    void *args[] = {&args_p, &tiles_arg, &units_arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks), dim3(block), args, 0,
                           stream);
}

// ---- T tokens per call on a ring ----------------------------------------------
// Token i of row n is the (c + i)-th token its slot sees: its taps are tokens
// c+i-3 .. c+i-1 (the first three come from the ring, later ones from this
// call's x) and it lands at position (c + i) mod L.  Only the last min(T, L)
// tokens survive in the ring, so only they are written; a window of the three
// previous tokens rides in registers, so no tap is read back after a write.

constexpr uint32_t kBadToken = 1u << 30;  // beyond every descriptor here (all < 2^30 bytes)

// The row's slot (or -1) and its count, as route_ring_row for a TokensParams.
__device__ __forceinline__ int route_ring_tokens_row(const TokensParams &p, int row, int lane, int *seen) {
    const int slot = route_row(p.idx, p.status, p.n, p.s, row, lane);
    *seen = p.seqlens[row];
    return ring_reject(p.status, slot, *seen, lane);
}

// R rows per wave, KP tokens per pass; L3: the ring holds exactly the three
// taps, so its planes are loaded in plane order and rotated by c mod 3
// afterwards (as in update_ring_v8).
template <int ACT, bool HAS_BIAS, int R, int KP, bool L3>
__global__ __launch_bounds__(kBlock) void tokens_ring_v8(TokensParams p, int tiles, int64_t block_units) {
    __shared__ u32x4 weight_tile[4 * kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    const uint32_t x_tok = (uint32_t)p.xs_t * 2u, o_tok = (uint32_t)p.os_t * 2u, plane_bytes = (uint32_t)p.st_l * 2u;
    const int L = L3 ? 3 : p.l;

    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t bu = blockIdx.x;
    do {
        const int tile = (int)(bu % tiles);
        const int group = (int)(bu / tiles) * kWavesPerBlock + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
        const uint32_t lane_off = lane < lanes_used ? lane_bytes : kBadLane;
        int slot[R], head[R];  // head: ring position of token c (c mod L; c >= 0 for a live row)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int row = group * R + r;
            int c = 0;
            slot[r] = __builtin_amdgcn_readfirstlane(row < p.n ? route_ring_tokens_row(p, row, lane, &c) : -2);
            head[r] = __builtin_amdgcn_readfirstlane(c) % L;
        }

        __builtin_amdgcn_s_setprio(3);
        u32x4 wraw[kWeightChunks];
        weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        Buffer sbuf[R], xbuf[R], obuf[R];
        u32x4 h[R][3], xv[R][KP];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool live = slot[r] >= 0;
            const int row = min(group * R + r, p.n - 1);
            sbuf[r] = make_buffer(p.state + (int64_t)(live ? slot[r] : 0) * p.st_s + c0,
                                  live ? plane_bytes * (uint32_t)(L - 1) + vec_bytes : 0u);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                // L3: plane k, rotated below; else token c-3+k's position
                const int pos = L3 ? k : (head[r] - 3 + k < 0 ? head[r] - 3 + k + L : head[r] - 3 + k);
                h[r][k] = buffer_load<kStream>(sbuf[r], plane_bytes * (uint32_t)pos + lane_off);
            }
            xbuf[r] = make_buffer(p.x + (int64_t)row * p.xs_n + c0, live ? x_tok * (uint32_t)(p.t - 1) + vec_bytes : 0u);
            obuf[r] = make_buffer(p.out + (int64_t)row * p.os_n + c0,
                                  slot[r] != -2 ? o_tok * (uint32_t)(p.t - 1) + vec_bytes : 0u);
#pragma unroll
            for (int i = 0; i < KP; ++i)
                xv[r][i] = buffer_load<kStream>(xbuf[r], (i < p.t ? x_tok * (uint32_t)i : kBadToken) + lane_off);
        }
        __builtin_amdgcn_s_setprio(0);
        if (L3) {
            // tap k (token c-3+k) is plane (c + k) mod 3
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const u32x4 p0 = h[r][0], p1 = h[r][1], p2 = h[r][2];
                h[r][0] = head[r] == 0 ? p0 : head[r] == 1 ? p1 : p2;
                h[r][1] = head[r] == 0 ? p1 : head[r] == 1 ? p2 : p0;
                h[r][2] = head[r] == 0 ? p2 : head[r] == 1 ? p0 : p1;
            }
        }

        float wf[32], bf[8];
        weight_tile_share(weight_tile, wraw, wave, lane, wf);
        unpack_bias(bv, bf);
        const int keep_from = p.t - min(p.t, L);  // tokens from here on stay in the ring

        for (int t0 = 0; t0 < p.t; t0 += KP) {
            if (t0 > 0) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        xv[r][i] = buffer_load<kStream>(
                            xbuf[r], (t0 + i < p.t ? x_tok * (uint32_t)(t0 + i) : kBadToken) + lane_off);
            }
            const int tokens = min(KP, p.t - t0);
            u32x4 ov[R][KP];
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int i = 0; i < KP; ++i) {
                    ov[r][i] = u32x4{0u, 0u, 0u, 0u};
                    if (i < tokens) {
                        const u32x4 y = conv8<ACT>(h[r][0], h[r][1], h[r][2], xv[r][i], wf, bf);
                        if (slot[r] >= 0) ov[r][i] = y;  // a padding row writes zeros
                        h[r][0] = h[r][1];
                        h[r][1] = h[r][2];
                        h[r][2] = xv[r][i];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < KP; ++i) {
                    const int tok = t0 + i;
                    buffer_store<kStream>(ov[r][i], obuf[r], (tok < p.t ? o_tok * (uint32_t)tok : kBadToken) + lane_off);
                    // a surviving token goes to ring position (c + tok) mod L
                    int pos = head[r] + tok % L;
                    pos = pos >= L ? pos - L : pos;
                    buffer_store<kStream>(xv[r][i], sbuf[r],
                                          (tok >= keep_from && tok < p.t ? plane_bytes * (uint32_t)pos : kBadToken) +
                                              lane_off);
                }
        }
        __syncthreads();  // the weight tile is reused by the next unit
        bu += kMaxBlocks;
    } while (bu < block_units);
}

template <int ACT>
__global__ __launch_bounds__(kScalarBlock) void tokens_ring_scalar(TokensParams p, int tiles_per_row, int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    for_each_unit(units, [&](int64_t unit) {
        const int row = (int)(unit / tiles_per_row);
        const int c = (int)(unit - (int64_t)row * tiles_per_row) * kScalarBlock + (int)threadIdx.x;
        int seen = 0;
        const int slot = route_ring_tokens_row(p, row, lane, &seen);
        if (c >= p.d) return;
        uint16_t *o = p.out + (int64_t)row * p.os_n + (int64_t)c * p.os_d;
        if (slot < 0) {
            for (int t = 0; t < p.t; ++t) o[(int64_t)t * p.os_t] = 0;
            return;
        }
        const int L = p.l;
        uint16_t *ring = p.state + (int64_t)slot * p.st_s + (int64_t)c * p.st_d;
        const int64_t sl = p.st_l;
        const uint16_t *xc = p.x + (int64_t)row * p.xs_n + (int64_t)c * p.xs_d;
        const uint16_t *wt = p.weight + (int64_t)c * 4;
        const float w0 = bf16_bits_to_f32(wt[0]), w1 = bf16_bits_to_f32(wt[1]);
        const float w2 = bf16_bits_to_f32(wt[2]), w3 = bf16_bits_to_f32(wt[3]);
        const float b = p.bias != nullptr ? bf16_bits_to_f32(p.bias[c]) : 0.0f;
        float h0 = bf16_bits_to_f32(ring[(int64_t)ring_pos(seen - 3, L) * sl]);
        float h1 = bf16_bits_to_f32(ring[(int64_t)ring_pos(seen - 2, L) * sl]);
        float h2 = bf16_bits_to_f32(ring[(int64_t)ring_pos(seen - 1, L) * sl]);
        for (int t = 0; t < p.t; ++t) {
            const uint16_t xb = xc[(int64_t)t * p.xs_t];
            const float xv = bf16_bits_to_f32(xb);
            float acc = h0 * w0;
            acc = __builtin_fmaf(h1, w1, acc);
            acc = __builtin_fmaf(h2, w2, acc);
            acc = __builtin_fmaf(xv, w3, acc);
            acc += b;
            o[(int64_t)t * p.os_t] = f32_to_bf16_bits(activate<ACT>(acc));
            ring[(int64_t)ring_pos(seen + t, L) * sl] = xb;  // in order: a later token overwrites an earlier one
            h0 = h1;
            h1 = h2;
            h2 = xv;
        }
    });
}

template <typename Kernel>
hipError_t launch_tokens_ring(Kernel kernel, const TokensParams &p, int tiles, int64_t units, int block,
                              hipStream_t stream) {
    const int64_t blocks = units < kMaxBlocks ? units : kMaxBlocks;
    TokensParams args_p = p;
    int tiles_arg = tiles;
    int64_t units_arg = units;
    void *args[] = {&args_p, &tiles_arg, &units_arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks), dim3(block), args, 0,
                           stream);
}

}  // namespace

hipError_t launch_update_tokens_ring(const TokensParams &p, StateLayout layout, int activation, hipStream_t stream,
                                     const char **kernel_name) {
    const bool silu = activation == DCCONV_ACT_SILU;
    const int64_t lim = (int64_t)1 << 30;
    const bool v8 = layout == StateLayout::ChannelLast && p.d % kChPerLane == 0 && p.xs_d == 1 && p.os_d == 1 &&
                    (p.n == 1 || (p.xs_n % 8 == 0 && p.os_n % 8 == 0)) &&
                    (p.t == 1 || (p.xs_t % 8 == 0 && p.os_t % 8 == 0)) && p.st_s % kChPerLane == 0 &&
                    p.xs_t * 2 * (int64_t)(p.t - 1) + 2 * kChPerWave < lim &&
                    p.os_t * 2 * (int64_t)(p.t - 1) + 2 * kChPerWave < lim &&
                    (int64_t)p.l * p.st_l * 2 + 2 * kChPerWave < lim;
    if (v8) {
        const int tiles = (p.d + kChPerWave - 1) / kChPerWave;
        const bool two = ((int64_t)p.n + 1) / 2 * tiles >= kMinWavesForTwoRows;
        const int64_t rows_per_block = kWavesPerBlock * (two ? 2 : 1);
        const int64_t units = ((int64_t)p.n + rows_per_block - 1) / rows_per_block * tiles;
        const bool l3 = p.l == 3;
#define DCCONV_TR_GO(R_, KP_, B_, L3_)                                                                          \
    return silu ? launch_tokens_ring(tokens_ring_v8<DCCONV_ACT_SILU, B_, R_, KP_, L3_>, p, tiles, units, kBlock,  \
                                     stream)                                                                    \
                : launch_tokens_ring(tokens_ring_v8<DCCONV_ACT_IDENTITY, B_, R_, KP_, L3_>, p, tiles, units,      \
                                     kBlock, stream)
#define DCCONV_TR_B(R_, KP_, L3_)              \
    if (p.bias != nullptr) {                   \
        DCCONV_TR_GO(R_, KP_, true, L3_);      \
    } else {                                   \
        DCCONV_TR_GO(R_, KP_, false, L3_);     \
    }
        if (two && p.t > 4 && p.t <= 8) {  // one pass of 8: every load before the first store
            *kernel_name = silu ? "tokens_ring_v8<silu,R=2,one pass>" : "tokens_ring_v8<identity,R=2,one pass>";
            if (l3) { DCCONV_TR_B(2, 8, true) }
            DCCONV_TR_B(2, 8, false)
        }
        if (two) {
            *kernel_name = silu ? "tokens_ring_v8<silu,R=2>" : "tokens_ring_v8<identity,R=2>";
            if (l3) { DCCONV_TR_B(2, 4, true) }
            DCCONV_TR_B(2, 4, false)
        }
        *kernel_name = silu ? "tokens_ring_v8<silu,R=1>" : "tokens_ring_v8<identity,R=1>";
        if (l3) { DCCONV_TR_B(1, 8, true) }
        DCCONV_TR_B(1, 8, false)
#undef DCCONV_TR_B
#undef DCCONV_TR_GO
    }
    const int tiles = (p.d + kScalarBlock - 1) / kScalarBlock;
    const int64_t units = (int64_t)p.n * tiles;
    *kernel_name = silu ? "tokens_ring_scalar<silu>" : "tokens_ring_scalar<identity>";
    return silu ? launch_tokens_ring(tokens_ring_scalar<DCCONV_ACT_SILU>, p, tiles, units, kScalarBlock, stream)
                : launch_tokens_ring(tokens_ring_scalar<DCCONV_ACT_IDENTITY>, p, tiles, units, kScalarBlock, stream);
}

hipError_t launch_update_ring(const UpdateParams &p, StateLayout layout, int activation, hipStream_t stream,
                              const char **kernel_name) {
    const bool silu = activation == DCCONV_ACT_SILU;
    // Channel-last planes as 16-byte vectors, every descriptor below 2^30 bytes.
    const bool v8 = layout == StateLayout::ChannelLast && p.d % kChPerLane == 0 && p.ld % kChPerLane == 0 &&
                    p.st_s % kChPerLane == 0 && (int64_t)p.l * p.st_l * 2 + 2 * kChPerWave < ((int64_t)1 << 30);
    if (v8) {
        const int tiles = (p.d + kChPerWave - 1) / kChPerWave;
        const bool two = two_rows_per_wave(p.n, tiles);
        const int rows_per_block = kWavesPerBlock * (two ? 2 : 1);
        const int64_t units = ((int64_t)p.n + rows_per_block - 1) / rows_per_block * tiles;
        const bool l3 = p.l == 3;
#define DCCONV_RING_GO(R_, B_, L3_)                                                                              \
    if (p.idx != nullptr)                                                                                         \
        return silu ? launch_ring(update_ring_v8<DCCONV_ACT_SILU, R_, B_, L3_, true>, p, tiles, units, kBlock, stream) \
                    : launch_ring(update_ring_v8<DCCONV_ACT_IDENTITY, R_, B_, L3_, true>, p, tiles, units, kBlock,     \
                                  stream);                                                                        \
    return silu ? launch_ring(update_ring_v8<DCCONV_ACT_SILU, R_, B_, L3_, false>, p, tiles, units, kBlock, stream)    \
                : launch_ring(update_ring_v8<DCCONV_ACT_IDENTITY, R_, B_, L3_, false>, p, tiles, units, kBlock, stream)
#define DCCONV_RING_B(R_, L3_)              \
    if (p.bias != nullptr) {                \
        DCCONV_RING_GO(R_, true, L3_);      \
    } else {                                \
        DCCONV_RING_GO(R_, false, L3_);     \
    }
        if (two) {
            *kernel_name = silu ? "update_ring_v8<silu,R=2>" : "update_ring_v8<identity,R=2>";
            if (l3) { DCCONV_RING_B(2, true) }
            DCCONV_RING_B(2, false)
        }
        *kernel_name = silu ? "update_ring_v8<silu,R=1>" : "update_ring_v8<identity,R=1>";
        if (l3) { DCCONV_RING_B(1, true) }
        DCCONV_RING_B(1, false)
#undef DCCONV_RING_B
#undef DCCONV_RING_GO
    }
    const int tiles = (p.d + kScalarBlock - 1) / kScalarBlock;
    const int64_t units = (int64_t)p.n * tiles;
    *kernel_name = silu ? "update_ring_scalar<silu>" : "update_ring_scalar<identity>";
    return silu ? launch_ring(update_ring_scalar<DCCONV_ACT_SILU>, p, tiles, units, kScalarBlock, stream)
                : launch_ring(update_ring_scalar<DCCONV_ACT_IDENTITY>, p, tiles, units, kScalarBlock, stream);
}

}  // namespace dcconv
