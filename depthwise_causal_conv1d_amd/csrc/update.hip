// Decode-update kernels for gfx950 (CDNA4, wave64).
//
// The operation (cuDNN FE-OSS page "Causal Conv1d Decode Update", section of the
// same name): for row n, channel c and the slot s the row selects, append x[n, c]
// to the slot's length-L history, keep the newest L values, and output
// act(sum_j history[L+1-W+j] * weight[c, j] + bias[c]) with W = 4.
//
// The update is a pure stream: every byte of x, of the selected state and of the
// output is touched exactly once; weight and bias are re-read from L2 by every
// row group.  It is bound by HBM bandwidth, so the kernels are organised around
// coalesced 16-byte accesses and around keeping many of them in flight, not
// around arithmetic (there is no contraction, so no MFMA).
//
//  * update_compact_v8<L, ACT, R, HAS_BIAS, INDEXED>: the fast path for the
//    compact [S, D, L] layout.  One wavefront owns R rows of one 512-channel
//    tile; each lane owns 8 adjacent channels, so x, weight, bias and out move as
//    one 16-byte vector per lane.  A row's tile of state is a contiguous
//    1 KiB * L run.  The wave issues every load of its R rows up front (weights
//    and bias once for all R rows; with an index table, every x before the table
//    is read and the state runs after), then finishes the rows in order, each as
//    soon as its own loads have landed: the state run goes through a per-wave
//    LDS stage (written in coalesced order, read back in per-lane channel order),
//    is shifted in registers with byte permutes, goes back through the stage and
//    leaves with L coalesced 16-byte stores.  Waves never share LDS, so all
//    synchronisation is wave-local.  The single-use streams (x, state, out)
//    carry the non-temporal hint, which keeps them from displacing the reused
//    weights and routing table in the caches.
//  * update_channel_last_v8<L, ACT, R, HAS_BIAS, INDEXED>: the [S, L, D] layout
//    a prefill hands over.  Every history position is a contiguous plane over
//    channels, so the lane that owns 8 channels loads and stores each plane with
//    one coalesced 16-byte access and the shift is a renaming of planes; no state
//    goes through LDS, and position 0 is not read unless it is a tap (L = 3).
//    The same block structure, weight sharing and store ordering as the compact
//    kernel.
//  * update_narrow<L, ACT, HAS_BIAS, CHANNEL_LAST>: small batches (at most
//    kNarrowMaxWaves 512-channel waves).  One wavefront per (row, 128-channel
//    tile), 2 channels per lane: four times the waves, each with a short chain
//    and no LDS or block barrier (see below).
//  * update_scalar<ACT>: one thread per (row, channel), any stride, any L >= 3,
//    any D.  Serves what the vector paths do not (D or row stride not a multiple
//    of 8, L > 8).
//
// Routing is resolved per row and is wave-uniform, so a padding or rejected row
// is one uniform branch that writes zeros and touches no state.
#include <stdint.h>

#include "dcconv.h"
#include "device_common.h"
#include "update_params.h"

namespace dcconv {
namespace {

// The arithmetic for the C channels a lane owns (C even).
//   hist[C*L/2]: the old state of the C channels, channel-major (oldest first)
//   xw[C/2]:     x of the C channels;  wf[4C]: weights [C][4] as FP32;  bf[C]: bias
// Produces the C outputs (packed BF16) and the new state (same order as hist).
template <int L, int ACT, int C>
__device__ __forceinline__ void update_lane(const uint32_t (&hist)[C * L / 2], const uint32_t (&xw)[C / 2],
                                            const float (&wf)[4 * C], const float (&bf)[C], bool has_bias,
                                            uint32_t (&outw)[C / 2], uint32_t (&nhist)[C * L / 2]) {
    float y[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        // history[L+1-W+j] for W = 4: the newest three state values, then x.
        // BF16 x BF16 products are exact in FP32, so the fused multiply-adds give
        // the same bits as separate products summed from j = 0 upward.
        float acc = elem_f32(hist, c * L + L - 3) * wf[4 * c + 0];
        acc = __builtin_fmaf(elem_f32(hist, c * L + L - 2), wf[4 * c + 1], acc);
        acc = __builtin_fmaf(elem_f32(hist, c * L + L - 1), wf[4 * c + 2], acc);
        acc = __builtin_fmaf(elem_f32(xw, c), wf[4 * c + 3], acc);
        if (has_bias) acc += bf[c];
        y[c] = activate<ACT>(acc);
    }
#pragma unroll
    for (int i = 0; i < C / 2; ++i) outw[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    // New state: each channel's history moves one place towards the oldest end
    // and x becomes the newest value.  New element e is x[e / L] when e is the
    // last position of its channel, else old element e + 1.  Each new word (two
    // elements) is one byte permute of the two words its halves come from.
#pragma unroll
    for (int i = 0; i < C * L / 2; ++i) {
        uint32_t src[2];
        int half[2];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = 2 * i + k;
            if (e % L == L - 1) {
                src[k] = xw[(e / L) >> 1];
                half[k] = (e / L) & 1;
            } else {
                src[k] = hist[(e + 1) >> 1];
                half[k] = (e + 1) & 1;
            }
        }
        nhist[i] = pick_halves(src[0], half[0], src[1], half[1]);
    }
}

template <int L, int ACT>
__device__ __forceinline__ void update8(const uint32_t (&hist)[4 * L], const uint32_t (&xw)[4],
                                        const float (&wf)[32], const float (&bf)[8], bool has_bias,
                                        uint32_t (&outw)[4], uint32_t (&nhist)[4 * L]) {
    update_lane<L, ACT, kChPerLane>(hist, xw, wf, bf, has_bias, outw, nhist);
}

template <int L, int ACT, int R, bool HAS_BIAS, bool INDEXED>
__global__ __launch_bounds__(kBlock) void update_compact_v8(UpdateParams p, int tiles_per_row,
                                                            int64_t block_units) {
    __shared__ u32x4 stage_all[kWavesPerBlock][R][stage_chunks<L>()];
    __shared__ u32x4 weight_tile[4 * kWave];  // the tile's 4 KiB of weights, swizzled
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;  // this lane's 16-byte vector in a 512-channel run

    // A block owns one 512-channel tile and kWavesPerBlock groups of R rows, one
    // group per wave, so the tile's weights are fetched once per block with
    // coalesced loads and shared through LDS.
    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t bu = blockIdx.x;
    do {
        const int tile = (int)(bu % tiles_per_row);
        const int group = (int)(bu / tiles_per_row) * kWavesPerBlock + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;  // x / out / bias bytes of the tile

        // Issue every load up front: this wave's share of the weight tile, the
        // bias, then each row's x and state run.  Buffer descriptors bound each
        // access: a row that must not touch the state gets an empty state
        // descriptor (its loads return zeros, its stores are dropped), a row
        // past the batch gets empty x and out descriptors, and the lanes past a
        // ragged tile's end fall outside every descriptor.  Nothing below
        // branches on the row, so the compiler can wait for each row's own
        // loads only.
        __builtin_amdgcn_s_setprio(3);  // get the loads of every wave queued early
        u32x4 wraw[kWeightChunks];
        weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        u32x4 xv[R], sv[R][L];
        Buffer sbuf[R], obuf[R];
        int slot[R];
        auto load_x = [&](int r) {
            const int row = min(group * R + r, p.n - 1);
            xv[r] = buffer_load<kStream>(make_buffer(p.x + (int64_t)row * p.ld + c0, group * R + r < p.n ? vec_bytes : 0u),
                                         lane_bytes);
        };
        // Route a row (wave-uniform): slot, -1 = write zeros, -2 = no such row.
        // route_row's result is the same in every lane; saying so keeps the
        // buffer descriptors built from it in scalar registers.
        auto route = [&](int r) {
            const int row = group * R + r;
            slot[r] = __builtin_amdgcn_readfirstlane(
                row < p.n ? route_row(INDEXED ? p.idx : nullptr, p.status, p.n, p.s, row, lane) : -2);
        };
        auto load_state = [&](int r) {
            const bool live = slot[r] >= 0;
            const int row = min(group * R + r, p.n - 1);
            sbuf[r] = make_buffer(live ? p.state + (int64_t)slot[r] * p.st_s + (int64_t)c0 * L : p.x,
                                  live ? vec_bytes * L : 0u);
            obuf[r] = make_buffer(p.out + (int64_t)row * p.d + c0, slot[r] != -2 ? vec_bytes : 0u);
#pragma unroll
            for (int j = 0; j < L; ++j) sv[r][j] = buffer_load<kStream>(sbuf[r], (uint32_t)(j * kWave) * 16u + lane_bytes);
        };
        if constexpr (!INDEXED) {
            // row r uses slot r: each row's x and state in row order, so the
            // first row's data is complete first
#pragma unroll
            for (int r = 0; r < R; ++r) load_x(r), route(r), load_state(r);
        } else {
            // every x ahead of the index table, whose latency it then shares;
            // the state runs once their slots are known (x of a padding row is
            // read but not used)
#pragma unroll
            for (int r = 0; r < R; ++r) load_x(r);
#pragma unroll
            for (int r = 0; r < R; ++r) route(r);
#pragma unroll
            for (int r = 0; r < R; ++r) load_state(r);
        }
        __builtin_amdgcn_s_setprio(0);

        float wf[32], bf[8];
        weight_tile_share(weight_tile, wraw, wave, lane, wf);
        unpack_bias(bv, bf);

        // Finish the rows in order, each once its own loads have landed, and
        // issue every store at the end.  On gfx9 loads and stores share one
        // completion counter that drains in order, and a store's data registers
        // may not be reused before it completes; so any wait placed after a store
        // (for the next row's loads, or for a register the store still holds)
        // would also wait for that store to be acknowledged by memory.  Keeping
        // all stores last means no wait ever follows one.
#pragma unroll
        for (int j = 0; j < L; ++j) stage_all[wave][0][stage_coalesced<L>(j, lane)] = sv[0][j];
        u32x4 nv[R][L], ov[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            u32x4 *stage = stage_all[wave][r];
            // coalesced chunk order -> per-lane channel order
            wave_lds_sync();
            uint32_t hist[4 * L];
#pragma unroll
            for (int k = 0; k < L; ++k) {
                const u32x4 t = stage[stage_lane<L>(lane, k)];
#pragma unroll
                for (int q = 0; q < 4; ++q) hist[4 * k + q] = t[q];
            }
            uint32_t xw[4] = {xv[r][0], xv[r][1], xv[r][2], xv[r][3]};
            uint32_t outw[4], nhist[4 * L];
            update8<L, ACT>(hist, xw, wf, bf, HAS_BIAS, outw, nhist);
            const bool live = slot[r] >= 0;  // a padding row writes zeros
            ov[r] = u32x4{live ? outw[0] : 0u, live ? outw[1] : 0u, live ? outw[2] : 0u, live ? outw[3] : 0u};
            // per-lane channel order -> coalesced chunk order
            wave_lds_sync();
#pragma unroll
            for (int k = 0; k < L; ++k)
                stage[stage_lane<L>(lane, k)] = u32x4{nhist[4 * k], nhist[4 * k + 1], nhist[4 * k + 2], nhist[4 * k + 3]};
            wave_lds_sync();
#pragma unroll
            for (int j = 0; j < L; ++j) nv[r][j] = stage[stage_coalesced<L>(j, lane)];
            if (r + 1 < R) {
#pragma unroll
                for (int j = 0; j < L; ++j) stage_all[wave][r + 1][stage_coalesced<L>(j, lane)] = sv[r + 1][j];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // all stores below, after all of the above
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < L; ++j) buffer_store<kStream>(nv[r][j], sbuf[r], (uint32_t)(j * kWave) * 16u + lane_bytes);
            buffer_store<kStream>(ov[r], obuf[r], lane_bytes);
        }
        __syncthreads();  // the stages and the weight tile are reused by the next unit
        bu += kMaxBlocks;
    } while (bu < block_units);
}

template <int L, int ACT, int R, bool HAS_BIAS, bool INDEXED>
__global__ __launch_bounds__(kBlock) void update_channel_last_v8(UpdateParams p, int tiles_per_row,
                                                                 int64_t block_units) {
    __shared__ u32x4 weight_tile[4 * kWave];
    // Planes the update reads: the taps need positions L-3..L-1, the shift needs
    // 1..L-1; position 0 is only read when it is also a tap (L = 3).
    constexpr int kFirst = L == 3 ? 0 : 1;
    constexpr int kRead = L - kFirst;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    const uint32_t plane_bytes = (uint32_t)p.st_l * 2u;  // distance between history positions

    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t bu = blockIdx.x;
    do {
        const int tile = (int)(bu % tiles_per_row);
        const int group = (int)(bu / tiles_per_row) * kWavesPerBlock + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
        // One descriptor spans a row's L planes of this tile; a lane past a ragged
        // tile's end gets an offset beyond every descriptor (2^31 > its size), so
        // it can neither read nor write a neighbouring plane.
        const uint32_t plane_lane = lane < lanes_used ? lane_bytes : 0x80000000u;

        // Loads in the compact kernel's order: per row without an index table,
        // every x ahead of the index table with one.
        __builtin_amdgcn_s_setprio(3);
        u32x4 wraw[kWeightChunks];
        weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        u32x4 xv[R], pv[R][kRead];
        Buffer sbuf[R], obuf[R];
        int slot[R];
        auto load_x = [&](int r) {
            const int row = min(group * R + r, p.n - 1);
            xv[r] = buffer_load<kStream>(make_buffer(p.x + (int64_t)row * p.ld + c0, group * R + r < p.n ? vec_bytes : 0u),
                                         lane_bytes);
        };
        auto route = [&](int r) {
            const int row = group * R + r;
            slot[r] = __builtin_amdgcn_readfirstlane(
                row < p.n ? route_row(INDEXED ? p.idx : nullptr, p.status, p.n, p.s, row, lane) : -2);
        };
        auto load_state = [&](int r) {
            const bool live = slot[r] >= 0;
            const int row = min(group * R + r, p.n - 1);
            sbuf[r] = make_buffer(live ? p.state + (int64_t)slot[r] * p.st_s + c0 : p.x,
                                  live ? plane_bytes * (uint32_t)(L - 1) + vec_bytes : 0u);
            obuf[r] = make_buffer(p.out + (int64_t)row * p.d + c0, slot[r] != -2 ? vec_bytes : 0u);
#pragma unroll
            for (int k = 0; k < kRead; ++k)
                pv[r][k] = buffer_load<kStream>(sbuf[r], plane_bytes * (uint32_t)(kFirst + k) + plane_lane);
        };
        if constexpr (!INDEXED) {
#pragma unroll
            for (int r = 0; r < R; ++r) load_x(r), route(r), load_state(r);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) load_x(r);
#pragma unroll
            for (int r = 0; r < R; ++r) route(r);
#pragma unroll
            for (int r = 0; r < R; ++r) load_state(r);
        }
        __builtin_amdgcn_s_setprio(0);

        float wf[32], bf[8];
        weight_tile_share(weight_tile, wraw, wave, lane, wf);
        unpack_bias(bv, bf);

        // Each plane vector already holds this lane's 8 channels at one history
        // position, so the taps read planes L-3..L-1 directly and the shift is a
        // renaming of planes.  All stores come last (see the compact kernel).
        u32x4 ov[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const u32x4 &pa = pv[r][L - 3 - kFirst], &pb = pv[r][L - 2 - kFirst], &pc = pv[r][L - 1 - kFirst];
            float y[kChPerLane];
#pragma unroll
            for (int ch = 0; ch < kChPerLane; ++ch) {
                const int q = ch >> 1;
                const bool h = ch & 1;
                float acc = (h ? hi_f32(pa[q]) : lo_f32(pa[q])) * wf[4 * ch + 0];
                acc = __builtin_fmaf(h ? hi_f32(pb[q]) : lo_f32(pb[q]), wf[4 * ch + 1], acc);
                acc = __builtin_fmaf(h ? hi_f32(pc[q]) : lo_f32(pc[q]), wf[4 * ch + 2], acc);
                acc = __builtin_fmaf(h ? hi_f32(xv[r][q]) : lo_f32(xv[r][q]), wf[4 * ch + 3], acc);
                if (HAS_BIAS) acc += bf[ch];
                y[ch] = activate<ACT>(acc);
            }
            const bool live = slot[r] >= 0;  // a padding row writes zeros
            ov[r] = u32x4{live ? pack_bf16x2(y[0], y[1]) : 0u, live ? pack_bf16x2(y[2], y[3]) : 0u,
                          live ? pack_bf16x2(y[4], y[5]) : 0u, live ? pack_bf16x2(y[6], y[7]) : 0u};
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            // plane k <- old plane k+1 (k < L-1), plane L-1 <- x
#pragma unroll
            for (int k = 0; k < L - 1; ++k)
                buffer_store<kStream>(pv[r][k + 1 - kFirst], sbuf[r], plane_bytes * (uint32_t)k + plane_lane);
            buffer_store<kStream>(xv[r], sbuf[r], plane_bytes * (uint32_t)(L - 1) + plane_lane);
            buffer_store<kStream>(ov[r], obuf[r], lane_bytes);
        }
        __syncthreads();  // the weight tile is reused by the next unit
        bu += kMaxBlocks;
    } while (bu < block_units);
}

// The narrow form, for batches too small to fill the GPU with 512-channel
// waves (few rows): one wavefront per (row, 128-channel tile), 2 channels per
// lane, so a row spreads over four times as many waves.  A lane's two channels
// of compact state are 4L contiguous bytes, so the wave's L*256-byte run moves
// as one coalesced access per lane (12 bytes at L = 3) and needs no LDS
// transpose; channel-last planes are one 4-byte access per lane.  Weights (16
// bytes per lane) are loaded directly, so there is no block barrier either:
// every wave runs its own short chain (x, weights and bias ahead of the index
// table, then the state, the arithmetic and all stores).
constexpr int kNarrowCh = 2;                    // channels per lane
constexpr int kNarrowTile = kWave * kNarrowCh;  // 128 channels per wave

template <int L, int ACT, bool HAS_BIAS, bool CHANNEL_LAST>
__global__ __launch_bounds__(kWave) void update_narrow(UpdateParams p, int tiles_per_row, int64_t units) {
    constexpr int kFirst = (CHANNEL_LAST && L > 3) ? 1 : 0;  // see update_channel_last_v8
    const int lane = threadIdx.x;
    const uint32_t lane_word = (uint32_t)lane * 4u;
    const uint32_t plane_bytes = (uint32_t)p.st_l * 2u;
    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t u = blockIdx.x;
    do {
        const int row = (int)(u / tiles_per_row);
        const int c0 = (int)(u - (int64_t)row * tiles_per_row) * kNarrowTile;
        const int lanes_used = min(kWave, (p.d - c0) / kNarrowCh);
        const uint32_t word_bytes = (uint32_t)lanes_used * 4u;  // x / out / bias bytes of the tile

        __builtin_amdgcn_s_setprio(3);
        const u32x4 wv = buffer_load<kCached>(make_buffer(p.weight + (int64_t)c0 * 4, word_bytes * 4u), lane * 16u);
        uint32_t bw = 0u;
        if (HAS_BIAS) bw = __builtin_amdgcn_raw_buffer_load_b32(make_buffer(p.bias + c0, word_bytes), lane_word, 0, kCached);
        const uint32_t xw[1] = {__builtin_amdgcn_raw_buffer_load_b32(
            make_buffer(p.x + (int64_t)row * p.ld + c0, word_bytes), lane_word, 0, kStream)};
        const int slot = __builtin_amdgcn_readfirstlane(route_row(p.idx, p.status, p.n, p.s, row, lane));
        const bool live = slot >= 0;
        // compact: channel-major words (channel 0's L values, then channel 1's);
        // channel-last: word k = position k of both channels
        uint32_t hist[L];
        Buffer sbuf;
        uint32_t plane_lane = 0u;
        if (CHANNEL_LAST) {
            sbuf = make_buffer(live ? p.state + (int64_t)slot * p.st_s + c0 : p.x,
                               live ? plane_bytes * (uint32_t)(L - 1) + word_bytes : 0u);
            plane_lane = lane < lanes_used ? lane_word : 0x80000000u;
#pragma unroll
            for (int k = 0; k < L; ++k)
                hist[k] = k < kFirst ? 0u
                                     : __builtin_amdgcn_raw_buffer_load_b32(sbuf, plane_bytes * (uint32_t)k + plane_lane,
                                                                            0, kStream);
        } else {
            sbuf = make_buffer(live ? p.state + (int64_t)slot * p.st_s + (int64_t)c0 * L : p.x,
                               live ? word_bytes * L : 0u);
            buffer_load_words<L, kStream>(sbuf, lane_word * L, hist);
        }
        __builtin_amdgcn_s_setprio(0);

        float wf[4 * kNarrowCh], bf[kNarrowCh];
#pragma unroll
        for (int q = 0; q < 4; ++q) wf[2 * q] = lo_f32(wv[q]), wf[2 * q + 1] = hi_f32(wv[q]);
        bf[0] = lo_f32(bw), bf[1] = hi_f32(bw);
        uint32_t outw[1], nhist[L];
        if (CHANNEL_LAST) {
            float y[kNarrowCh];
#pragma unroll
            for (int c = 0; c < kNarrowCh; ++c) {
                float acc = half_f32(hist[L - 3], c) * wf[4 * c + 0];
                acc = __builtin_fmaf(half_f32(hist[L - 2], c), wf[4 * c + 1], acc);
                acc = __builtin_fmaf(half_f32(hist[L - 1], c), wf[4 * c + 2], acc);
                acc = __builtin_fmaf(half_f32(xw[0], c), wf[4 * c + 3], acc);
                if (HAS_BIAS) acc += bf[c];
                y[c] = activate<ACT>(acc);
            }
            outw[0] = pack_bf16x2(y[0], y[1]);
#pragma unroll
            for (int k = 0; k < L - 1; ++k) nhist[k] = hist[k + 1];
            nhist[L - 1] = xw[0];
        } else {
            update_lane<L, ACT, kNarrowCh>(hist, xw, wf, bf, HAS_BIAS, outw, nhist);
        }
        // all stores last; a padding row writes zeros and no state
        __builtin_amdgcn_sched_barrier(0);
        if (CHANNEL_LAST) {
#pragma unroll
            for (int k = 0; k < L; ++k)
                __builtin_amdgcn_raw_buffer_store_b32(nhist[k], sbuf, plane_bytes * (uint32_t)k + plane_lane, 0, kStream);
        } else {
            buffer_store_words<L, kStream>(nhist, sbuf, lane_word * L);
        }
        __builtin_amdgcn_raw_buffer_store_b32(live ? outw[0] : 0u, make_buffer(p.out + (int64_t)row * p.d + c0, word_bytes),
                                              lane_word, 0, kStream);
        u += kMaxBlocks;
    } while (u < units);
}

template <int ACT>
__global__ __launch_bounds__(kScalarBlock) void update_scalar(UpdateParams p, int tiles_per_row, int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    for_each_unit(units, [&](int64_t unit) {
        const int row = (int)(unit / tiles_per_row);
        const int c = (int)(unit - (int64_t)row * tiles_per_row) * kScalarBlock + (int)threadIdx.x;
        const int slot = route_row(p.idx, p.status, p.n, p.s, row, lane);
        if (c >= p.d) return;
        uint16_t *o = p.out + (int64_t)row * p.d + c;
        if (slot < 0) {
            *o = 0;
            return;
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
    });
}

// Launches `units` block units (the kernels stride over them when the grid is capped).
template <typename Kernel>
hipError_t launch(Kernel kernel, const UpdateParams &p, int tiles_per_row, int64_t units, int block,
                  hipStream_t stream) {
    const int64_t blocks = units < kMaxBlocks ? units : kMaxBlocks;
    UpdateParams args_p = p;
    void *args[] = {&args_p, &tiles_per_row, &units};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks), dim3(block), args, 0,
                           stream);
}

template <int L, int ACT>
hipError_t launch_compact_l(const UpdateParams &p, int tiles, hipStream_t stream, const char **name,
                            const char *name_one_row, const char *name_two_rows) {
    const bool bias = p.bias != nullptr;
    const int64_t groups_two = (p.n + 1) / 2;
    const bool indexed = p.idx != nullptr;
    if (two_rows_per_wave(p.n, tiles)) {
        *name = name_two_rows;
        const int64_t block_units = tiles * ((groups_two + kWavesPerBlock - 1) / kWavesPerBlock);
        return bias ? (indexed ? launch(update_compact_v8<L, ACT, 2, true, true>, p, tiles, block_units, kBlock, stream)
                               : launch(update_compact_v8<L, ACT, 2, true, false>, p, tiles, block_units, kBlock, stream))
                    : (indexed ? launch(update_compact_v8<L, ACT, 2, false, true>, p, tiles, block_units, kBlock, stream)
                               : launch(update_compact_v8<L, ACT, 2, false, false>, p, tiles, block_units, kBlock, stream));
    }
    *name = name_one_row;
    const int64_t block_units = tiles * (((int64_t)p.n + kWavesPerBlock - 1) / kWavesPerBlock);
    return bias ? (indexed ? launch(update_compact_v8<L, ACT, 1, true, true>, p, tiles, block_units, kBlock, stream)
                           : launch(update_compact_v8<L, ACT, 1, true, false>, p, tiles, block_units, kBlock, stream))
                : (indexed ? launch(update_compact_v8<L, ACT, 1, false, true>, p, tiles, block_units, kBlock, stream)
                           : launch(update_compact_v8<L, ACT, 1, false, false>, p, tiles, block_units, kBlock, stream));
}

template <int ACT>
hipError_t launch_compact(const UpdateParams &p, int tiles, hipStream_t stream, const char **name) {
#define DCCONV_COMPACT_CASE(LL, ACTNAME)                                                                   \
    case LL:                                                                                               \
        return launch_compact_l<LL, ACT>(p, tiles, stream, name, "update_compact_v8<L=" #LL "," ACTNAME ",R=1>", \
                                         "update_compact_v8<L=" #LL "," ACTNAME ",R=2>");
    if (ACT == DCCONV_ACT_SILU) {
        switch (p.l) {
            DCCONV_COMPACT_CASE(3, "silu")
            DCCONV_COMPACT_CASE(4, "silu")
            DCCONV_COMPACT_CASE(5, "silu")
            DCCONV_COMPACT_CASE(6, "silu")
            DCCONV_COMPACT_CASE(7, "silu")
            DCCONV_COMPACT_CASE(8, "silu")
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.l) {
        DCCONV_COMPACT_CASE(3, "identity")
        DCCONV_COMPACT_CASE(4, "identity")
        DCCONV_COMPACT_CASE(5, "identity")
        DCCONV_COMPACT_CASE(6, "identity")
        DCCONV_COMPACT_CASE(7, "identity")
        DCCONV_COMPACT_CASE(8, "identity")
        default: return hipErrorInvalidValue;
    }
#undef DCCONV_COMPACT_CASE
}

template <int L, int ACT>
hipError_t launch_channel_last_l(const UpdateParams &p, int tiles, hipStream_t stream, const char **name,
                                 const char *name_one_row, const char *name_two_rows) {
    const bool bias = p.bias != nullptr;
    const int64_t groups_two = (p.n + 1) / 2;
    const bool indexed = p.idx != nullptr;
    if (two_rows_per_wave(p.n, tiles)) {
        *name = name_two_rows;
        const int64_t block_units = tiles * ((groups_two + kWavesPerBlock - 1) / kWavesPerBlock);
        return bias ? (indexed ? launch(update_channel_last_v8<L, ACT, 2, true, true>, p, tiles, block_units, kBlock, stream)
                               : launch(update_channel_last_v8<L, ACT, 2, true, false>, p, tiles, block_units, kBlock, stream))
                    : (indexed ? launch(update_channel_last_v8<L, ACT, 2, false, true>, p, tiles, block_units, kBlock, stream)
                               : launch(update_channel_last_v8<L, ACT, 2, false, false>, p, tiles, block_units, kBlock,
                                        stream));
    }
    *name = name_one_row;
    const int64_t block_units = tiles * (((int64_t)p.n + kWavesPerBlock - 1) / kWavesPerBlock);
    return bias ? (indexed ? launch(update_channel_last_v8<L, ACT, 1, true, true>, p, tiles, block_units, kBlock, stream)
                           : launch(update_channel_last_v8<L, ACT, 1, true, false>, p, tiles, block_units, kBlock, stream))
                : (indexed ? launch(update_channel_last_v8<L, ACT, 1, false, true>, p, tiles, block_units, kBlock, stream)
                           : launch(update_channel_last_v8<L, ACT, 1, false, false>, p, tiles, block_units, kBlock, stream));
}

template <int ACT>
hipError_t launch_channel_last(const UpdateParams &p, int tiles, hipStream_t stream, const char **name) {
#define DCCONV_CL_CASE(LL, ACTNAME)                                                                          \
    case LL:                                                                                                  \
        return launch_channel_last_l<LL, ACT>(p, tiles, stream, name,                                         \
                                              "update_channel_last_v8<L=" #LL "," ACTNAME ",R=1>",            \
                                              "update_channel_last_v8<L=" #LL "," ACTNAME ",R=2>");
    if (ACT == DCCONV_ACT_SILU) {
        switch (p.l) {
            DCCONV_CL_CASE(3, "silu")
            DCCONV_CL_CASE(4, "silu")
            DCCONV_CL_CASE(5, "silu")
            DCCONV_CL_CASE(6, "silu")
            DCCONV_CL_CASE(7, "silu")
            DCCONV_CL_CASE(8, "silu")
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.l) {
        DCCONV_CL_CASE(3, "identity")
        DCCONV_CL_CASE(4, "identity")
        DCCONV_CL_CASE(5, "identity")
        DCCONV_CL_CASE(6, "identity")
        DCCONV_CL_CASE(7, "identity")
        DCCONV_CL_CASE(8, "identity")
        default: return hipErrorInvalidValue;
    }
#undef DCCONV_CL_CASE
}

template <int ACT, bool CHANNEL_LAST>
hipError_t launch_narrow(const UpdateParams &p, hipStream_t stream, const char **name) {
    const int tiles = (p.d + kNarrowTile - 1) / kNarrowTile;
    const int64_t units = (int64_t)p.n * tiles;
    const bool bias = p.bias != nullptr;
#define DCCONV_NARROW_CASE(LL)                                                                                 \
    case LL:                                                                                                    \
        *name = CHANNEL_LAST ? (ACT == DCCONV_ACT_SILU ? "update_narrow<L=" #LL ",silu,channel_last>"           \
                                                       : "update_narrow<L=" #LL ",identity,channel_last>")      \
                             : (ACT == DCCONV_ACT_SILU ? "update_narrow<L=" #LL ",silu,compact>"                \
                                                       : "update_narrow<L=" #LL ",identity,compact>");          \
        return bias ? launch(update_narrow<LL, ACT, true, CHANNEL_LAST>, p, tiles, units, kWave, stream)        \
                    : launch(update_narrow<LL, ACT, false, CHANNEL_LAST>, p, tiles, units, kWave, stream);
    switch (p.l) {
        DCCONV_NARROW_CASE(3)
        DCCONV_NARROW_CASE(4)
        DCCONV_NARROW_CASE(5)
        DCCONV_NARROW_CASE(6)
        DCCONV_NARROW_CASE(7)
        DCCONV_NARROW_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef DCCONV_NARROW_CASE
}

}  // namespace

hipError_t launch_update(const UpdateParams &p, StateLayout layout, int activation, hipStream_t stream,
                         const char **kernel_name) {
    if (p.seqlens != nullptr) return launch_update_ring(p, layout, activation, stream, kernel_name);
    const bool rows_v8 = (p.d % kChPerLane == 0) && (p.ld % kChPerLane == 0);
    const bool silu = activation == DCCONV_ACT_SILU;
    const int tiles_v8 = (p.d + kChPerWave - 1) / kChPerWave;
    // A batch whose 512-channel waves would not cover the CUs spreads over
    // 128-channel waves instead.
    const bool narrow = (int64_t)p.n * tiles_v8 <= kNarrowMaxWaves;
    if (narrow && rows_v8 && p.st_s % kChPerLane == 0 && p.l >= 3 && p.l <= 8 &&
        (layout == StateLayout::Compact || (int64_t)p.l * p.st_l * 2 < (int64_t)1 << 30)) {
        const bool cl = layout == StateLayout::ChannelLast;
        return silu ? (cl ? launch_narrow<DCCONV_ACT_SILU, true>(p, stream, kernel_name)
                          : launch_narrow<DCCONV_ACT_SILU, false>(p, stream, kernel_name))
                    : (cl ? launch_narrow<DCCONV_ACT_IDENTITY, true>(p, stream, kernel_name)
                          : launch_narrow<DCCONV_ACT_IDENTITY, false>(p, stream, kernel_name));
    }
    if (layout == StateLayout::Compact && rows_v8 && p.st_s % kChPerLane == 0 && p.l >= 3 && p.l <= 8) {
        return silu ? launch_compact<DCCONV_ACT_SILU>(p, tiles_v8, stream, kernel_name)
                    : launch_compact<DCCONV_ACT_IDENTITY>(p, tiles_v8, stream, kernel_name);
    }
    if (layout == StateLayout::ChannelLast && rows_v8 && p.st_s % kChPerLane == 0 && p.l >= 3 && p.l <= 8 &&
        (int64_t)p.l * p.st_l * 2 < (int64_t)1 << 30) {
        return silu ? launch_channel_last<DCCONV_ACT_SILU>(p, tiles_v8, stream, kernel_name)
                    : launch_channel_last<DCCONV_ACT_IDENTITY>(p, tiles_v8, stream, kernel_name);
    }
    const int tiles = (p.d + kScalarBlock - 1) / kScalarBlock;
    const int64_t units = (int64_t)p.n * tiles;
    *kernel_name = silu ? "update_scalar<silu>" : "update_scalar<identity>";
    return silu ? launch(update_scalar<DCCONV_ACT_SILU>, p, tiles, units, kScalarBlock, stream)
                : launch(update_scalar<DCCONV_ACT_IDENTITY>, p, tiles, units, kScalarBlock, stream);
}

}  // namespace dcconv
