// Multi-token decode update for gfx950: T successive decode steps on the same
// slots in one call, x[N, D, T] -> out[N, D, T].
//
// This is the multi-token form the cuDNN FE-OSS page "Causal Conv1d Decode
// Update" reserves (section "Semantic tensor contract": a future x[N, D, Tstep]
// keeps the meaning of the state and the weights).  Token t of every row is
// applied, in order, by the single-step rule, and out[:, :, t] is that step's
// output.  Doing all T steps in one pass reads and writes each selected state
// once instead of T times: per active channel-row the bytes drop from
// T * (4 + 4L) + 2T to 4L + 4T (compact layout).
//
//  * tokens_v8<L, ACT, HAS_BIAS, CHANNEL_LAST, R, KP, SPLIT, PREFETCH, INDEXED>: one wavefront owns
//    R rows of one 512-channel tile (8 channels per lane), the block shares the
//    tile's weights.  With SPLIT (one row per block, T >= 2L) the block's two
//    waves share one row and split its tokens at h = T/2: outputs from token 3
//    on depend on x alone, so wave 1 starts from the three tokens before h,
//    produces outputs [h, T) and writes the final state (with T >= 2L it holds
//    tokens of that half only), while wave 0 reads the state and produces
//    outputs [0, h).  That doubles the waves of a thin grid (few rows, long
//    calls) and halves each wave's dependent chain.
//    The history lives in registers in plane-major form (one 16-byte vector per
//    history position, 8 channels each), so a token's shift is a renaming of
//    registers.  Tokens go in passes of KP: the pass's x vectors are all loaded
//    before the first is used (with PREFETCH, for one-row waves of several
//    passes, the next pass's loads are issued before this pass is computed)
//    and its outputs are all stored after the last is computed.  A wave of 5
//    to 8 tokens takes them in a single pass of 8.  Compact state
//    goes through the same LDS stage as the single-token kernel; channel-last
//    state is already plane-major.
//  * tokens_scalar<ACT>: one thread per (row, channel), any strides, any L >= 3;
//    each token is one single-step update of the thread's channel in memory.
#include <stdint.h>

#include "dcconv.h"
#include "device_common.h"
#include "update_params.h"

namespace dcconv {
namespace {

// Buffer offsets that lie beyond every descriptor (all descriptors used here are
// smaller than 2^30 bytes): one for a token past the end, one for a lane past a
// ragged tile.  Their sum stays below 2^32.
constexpr uint32_t kBadToken = 1u << 30;
constexpr uint32_t kBadLane = 1u << 31;

template <int L, int ACT, bool HAS_BIAS, bool CHANNEL_LAST, int R, int KP, bool SPLIT, bool PREFETCH, bool INDEXED>
__global__ __launch_bounds__(kBlock) void tokens_v8(TokensParams p, int tiles_per_row, int64_t block_units) {
    static_assert(!SPLIT || R == 1, "a split block holds one row");
    static_assert(!PREFETCH || R == 1, "only one-row waves prefetch");
    __shared__ u32x4 stage_all[kWavesPerBlock][CHANNEL_LAST ? 1 : stage_chunks<L>()];
    __shared__ u32x4 weight_tile[4 * kWave];
    // Positions read in the channel-last layout: the first token's taps need
    // L-3..L-1 and the shift needs 1..L-1; position 0 only when it is a tap.
    constexpr int kFirst = (CHANNEL_LAST && L > 3) ? 1 : 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    const uint32_t x_tok = (uint32_t)p.xs_t * 2u, o_tok = (uint32_t)p.os_t * 2u, plane_bytes = (uint32_t)p.st_l * 2u;

    // A block owns one 512-channel tile and kWavesPerBlock groups of R rows, or
    // with SPLIT one row whose tokens [tb, te) are this wave's share.
    const int tb = (SPLIT && wave == 1) ? p.t / 2 : 0;
    const int te = (SPLIT && wave == 0) ? p.t / 2 : p.t;
    const bool reads_state = !SPLIT || wave == 0;
    const bool writes_state = !SPLIT || wave == 1;
    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t bu = blockIdx.x;
    do {
        const int tile = (int)(bu % tiles_per_row);
        const int group = SPLIT ? (int)(bu / tiles_per_row) : (int)(bu / tiles_per_row) * kWavesPerBlock + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
        const uint32_t lane_off = lane < lanes_used ? lane_bytes : kBadLane;
        // every load of the first pass up front: weights, bias, each row's
        // state (or, for the second half of a split row, the three tokens
        // before it) and its first KP tokens
        __builtin_amdgcn_s_setprio(3);
        u32x4 wraw[kWeightChunks];
        weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        Buffer sbuf[R], xbuf[R], obuf[R];
        u32x4 sv[R][L], xv[R][KP], hx[3];
        int slot[R];
        // x and out of a row: one descriptor each, spanning every token
        auto x_descriptors = [&](int r) {
            const bool row_ok = group * R + r < p.n;
            const int row = min(group * R + r, p.n - 1);
            xbuf[r] = make_buffer(p.x + (int64_t)row * p.xs_n + c0, row_ok ? x_tok * (uint32_t)(p.t - 1) + vec_bytes : 0u);
            obuf[r] = make_buffer(p.out + (int64_t)row * p.os_n + c0,
                                  row_ok ? o_tok * (uint32_t)(p.t - 1) + vec_bytes : 0u);
        };
        auto load_x = [&](int r) {
            if (!CHANNEL_LAST && !reads_state) {
#pragma unroll
                for (int k = 0; k < 3; ++k) hx[k] = buffer_load<kStream>(xbuf[r], x_tok * (uint32_t)(tb - 3 + k) + lane_off);
            }
#pragma unroll
            for (int i = 0; i < KP; ++i)
                xv[r][i] = buffer_load<kStream>(xbuf[r], (tb + i < te ? x_tok * (uint32_t)(tb + i) : kBadToken) + lane_off);
        };
        auto route = [&](int r) {
            const int row = group * R + r;
            slot[r] = __builtin_amdgcn_readfirstlane(
                row < p.n ? route_row(INDEXED ? p.idx : nullptr, p.status, p.n, p.s, row, lane) : -2);
        };
        auto load_state = [&](int r) {
            const bool live = slot[r] >= 0;
            // State: compact = the tile's contiguous run of L KiB, read coalesced;
            // channel-last = planes kFirst..L-1 of this tile.
            if (CHANNEL_LAST) {
                sbuf[r] = make_buffer(live ? p.state + (int64_t)slot[r] * p.st_s + c0 : p.x,
                                      live ? plane_bytes * (uint32_t)(L - 1) + vec_bytes : 0u);
                // The second half of a split row takes the three tokens before
                // its first as the three newest positions and zeros below them
                // (an empty descriptor): one load sequence for both halves.
                const Buffer older = reads_state ? sbuf[r] : make_buffer(p.x, 0u);
                const Buffer newest = reads_state ? sbuf[r] : xbuf[r];
#pragma unroll
                for (int k = 0; k < L; ++k) {
                    if (k < kFirst)
                        sv[r][k] = u32x4{0u, 0u, 0u, 0u};
                    else if (k < L - 3)
                        sv[r][k] = buffer_load<kStream>(older, plane_bytes * (uint32_t)k + lane_off);
                    else
                        sv[r][k] = buffer_load<kStream>(
                            newest,
                            (reads_state ? plane_bytes * (uint32_t)k : x_tok * (uint32_t)(tb - L + k)) + lane_off);
                }
            } else {
                sbuf[r] = make_buffer(live ? p.state + (int64_t)slot[r] * p.st_s + (int64_t)c0 * L : p.x,
                                      live ? vec_bytes * L : 0u);
                if (reads_state) {
#pragma unroll
                    for (int j = 0; j < L; ++j)
                        sv[r][j] = buffer_load<kStream>(sbuf[r], (uint32_t)(j * kWave) * 16u + lane_bytes);
                }
            }
        };
        if constexpr (!INDEXED) {
            // row r uses slot r: each row's state, then its tokens, in row order
#pragma unroll
            for (int r = 0; r < R; ++r) x_descriptors(r), route(r), load_state(r), load_x(r);
        } else {
            // the tokens ahead of the index table, whose latency they then
            // share; the state once the slots are known (x of a padding row is
            // read but not used)
#pragma unroll
            for (int r = 0; r < R; ++r) x_descriptors(r), load_x(r);
#pragma unroll
            for (int r = 0; r < R; ++r) route(r);
#pragma unroll
            for (int r = 0; r < R; ++r) load_state(r);
        }
        __builtin_amdgcn_s_setprio(0);

        float wf[32], bf[8];
        weight_tile_share(weight_tile, wraw, wave, lane, wf);
        unpack_bias(bv, bf);

        u32x4 pl[R][L];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (CHANNEL_LAST) {
#pragma unroll
                for (int k = 0; k < L; ++k) pl[r][k] = sv[r][k];
            } else if (!reads_state) {
                // the second half of a split row: only the three newest
                // positions matter (the T - h >= L tokens ahead shift out the rest)
#pragma unroll
                for (int k = 0; k < L - 3; ++k) pl[r][k] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int k = 0; k < 3; ++k) pl[r][L - 3 + k] = hx[k];
            } else {
                u32x4 *stage = stage_all[wave];
                wave_lds_sync();
#pragma unroll
                for (int j = 0; j < L; ++j) stage[stage_coalesced<L>(j, lane)] = sv[r][j];
                wave_lds_sync();
                uint32_t h[4 * L];
#pragma unroll
                for (int k = 0; k < L; ++k) {
                    const u32x4 t = stage[stage_lane<L>(lane, k)];
#pragma unroll
                    for (int q = 0; q < 4; ++q) h[4 * k + q] = t[q];
                }
                to_planes<L>(h, pl[r]);
            }
        }

        // A split row's state is read by wave 0 and rewritten by wave 1.  The
        // empty asm consumes the loaded state, so wave 0's loads have returned
        // before the barrier and wave 1's write, after it, cannot overtake them.
        if (SPLIT) {
            if (reads_state) {
#pragma unroll
                for (int k = 0; k < L; ++k) asm volatile("" ::"v"(sv[0][k]));
            }
            __syncthreads();
        }

        // PREFETCH (one row per wave, more than one pass): the next pass's x
        // is loaded before this pass is computed, so its latency runs under
        // this pass's arithmetic and stores (a thin grid has no other wave on
        // the SIMD to cover it).  Otherwise each pass is loaded at its start;
        // a wave whose tokens fit one pass then has every load issued before
        // its first store, so its waits never cover a store.
        constexpr bool kPrefetch = PREFETCH;
        for (int t0 = tb; t0 < te; t0 += KP) {
            // The prefetch is issued on the last pass too (its offsets then lie
            // past the descriptor: nothing is read): with one path into the
            // pass, each wait covers only the loads it needs.
            u32x4 xn[R][KP];
            if (kPrefetch) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        xn[r][i] = buffer_load<kStream>(
                            xbuf[r], (t0 + KP + i < te ? x_tok * (uint32_t)(t0 + KP + i) : kBadToken) + lane_off);
            } else if (!kPrefetch && t0 > tb) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < KP; ++i)
                        xv[r][i] = buffer_load<kStream>(
                            xbuf[r], (t0 + i < te ? x_tok * (uint32_t)(t0 + i) : kBadToken) + lane_off);
            }
            const int tokens = min(KP, te - t0);
            u32x4 ov[R][KP];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const bool live = slot[r] >= 0;
#pragma unroll
                for (int i = 0; i < KP; ++i) {
                    ov[r][i] = u32x4{0u, 0u, 0u, 0u};
                    if (i < tokens) {
                        // history[L+1-W+j] for W = 4: positions L-3..L-1, then x
                        const u32x4 y = conv8<ACT>(pl[r][L - 3], pl[r][L - 2], pl[r][L - 1], xv[r][i], wf, bf);
                        if (live) ov[r][i] = y;  // a padding row writes zeros
                        // the shift: every position moves one place older, x is the newest
#pragma unroll
                        for (int k = 0; k < L - 1; ++k) pl[r][k] = pl[r][k + 1];
                        pl[r][L - 1] = xv[r][i];
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < KP; ++i)
                    buffer_store<kStream>(ov[r][i], obuf[r],
                                          (t0 + i < te ? o_tok * (uint32_t)(t0 + i) : kBadToken) + lane_off);
            if (kPrefetch) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < KP; ++i) xv[r][i] = xn[r][i];
            }
        }

        // Write the final history back (a split row's second half holds it).
#pragma unroll
        for (int r = 0; r < R && writes_state; ++r) {
            if (CHANNEL_LAST) {
#pragma unroll
                for (int k = 0; k < L; ++k) buffer_store<kStream>(pl[r][k], sbuf[r], plane_bytes * (uint32_t)k + lane_off);
            } else {
                u32x4 *stage = stage_all[wave];
                uint32_t h[4 * L];
                from_planes<L>(pl[r], h);
                wave_lds_sync();
#pragma unroll
                for (int k = 0; k < L; ++k)
                    stage[stage_lane<L>(lane, k)] = u32x4{h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]};
                wave_lds_sync();
                u32x4 nv[L];
#pragma unroll
                for (int j = 0; j < L; ++j) nv[j] = stage[stage_coalesced<L>(j, lane)];
#pragma unroll
                for (int j = 0; j < L; ++j)
                    buffer_store<kStream>(nv[j], sbuf[r], (uint32_t)(j * kWave) * 16u + lane_bytes);
            }
        }
        __syncthreads();  // the stage and the weight tile are reused by the next unit
        bu += kMaxBlocks;
    } while (bu < block_units);
}

template <int ACT>
__global__ __launch_bounds__(kScalarBlock) void tokens_scalar(TokensParams p, int tiles_per_row, int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    for_each_unit(units, [&](int64_t unit) {
        const int row = (int)(unit / tiles_per_row);
        const int c = (int)(unit - (int64_t)row * tiles_per_row) * kScalarBlock + (int)threadIdx.x;
        const int slot = route_row(p.idx, p.status, p.n, p.s, row, lane);
        if (c >= p.d) return;
        uint16_t *o = p.out + (int64_t)row * p.os_n + (int64_t)c * p.os_d;
        if (slot < 0) {
            for (int t = 0; t < p.t; ++t) o[(int64_t)t * p.os_t] = 0;
            return;
        }
        const int L = p.l;
        uint16_t *h = p.state + (int64_t)slot * p.st_s + (int64_t)c * p.st_d;
        const int64_t sl = p.st_l;
        const uint16_t *xc = p.x + (int64_t)row * p.xs_n + (int64_t)c * p.xs_d;
        const uint16_t *wt = p.weight + (int64_t)c * 4;
        const float w0 = bf16_bits_to_f32(wt[0]), w1 = bf16_bits_to_f32(wt[1]);
        const float w2 = bf16_bits_to_f32(wt[2]), w3 = bf16_bits_to_f32(wt[3]);
        const float b = p.bias != nullptr ? bf16_bits_to_f32(p.bias[c]) : 0.0f;
        for (int t = 0; t < p.t; ++t) {
            const uint32_t x = xc[(int64_t)t * p.xs_t];
            const float h0 = bf16_bits_to_f32(h[(L - 3) * sl]);
            const float h1 = bf16_bits_to_f32(h[(L - 2) * sl]);
            const float h2 = bf16_bits_to_f32(h[(L - 1) * sl]);
            for (int k = 0; k < L - 1; ++k) h[k * sl] = h[(k + 1) * sl];
            h[(L - 1) * sl] = (uint16_t)x;
            float acc = h0 * w0;
            acc = __builtin_fmaf(h1, w1, acc);
            acc = __builtin_fmaf(h2, w2, acc);
            acc = __builtin_fmaf(bf16_bits_to_f32(x), w3, acc);
            if (p.bias != nullptr) acc += b;
            o[(int64_t)t * p.os_t] = f32_to_bf16_bits(activate<ACT>(acc));
        }
    });
}

template <typename Kernel>
hipError_t launch_tokens(Kernel kernel, const TokensParams &p, int tiles_per_row, int64_t units, int block,
                         hipStream_t stream) {
    int64_t blocks = units < kMaxBlocks ? units : kMaxBlocks;
    TokensParams args_p = p;
    void *args[] = {&args_p, &tiles_per_row, &units};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks), dim3(block), args, 0,
                           stream);
}

template <int L, int ACT, bool CL, int R, int KP, bool SPLIT, bool PREFETCH>
hipError_t launch_tokens_l(const TokensParams &p, int tiles, hipStream_t stream) {
    const int64_t rows_per_block = SPLIT ? 1 : kWavesPerBlock * R;
    const int64_t block_units = tiles * (((int64_t)p.n + rows_per_block - 1) / rows_per_block);
    if (p.idx != nullptr)
        return p.bias != nullptr
                   ? launch_tokens(tokens_v8<L, ACT, true, CL, R, KP, SPLIT, PREFETCH, true>, p, tiles, block_units,
                                   kBlock, stream)
                   : launch_tokens(tokens_v8<L, ACT, false, CL, R, KP, SPLIT, PREFETCH, true>, p, tiles, block_units,
                                   kBlock, stream);
    return p.bias != nullptr
               ? launch_tokens(tokens_v8<L, ACT, true, CL, R, KP, SPLIT, PREFETCH, false>, p, tiles, block_units,
                               kBlock, stream)
               : launch_tokens(tokens_v8<L, ACT, false, CL, R, KP, SPLIT, PREFETCH, false>, p, tiles, block_units,
                               kBlock, stream);
}

// A grid of one row per wave below this many waves (under two per SIMD) splits
// each row's tokens over two waves when the call is long enough (T >= 2L).
constexpr int64_t kMaxWavesForSplit = 2048;

template <int ACT, bool CL>
hipError_t launch_tokens_v8(const TokensParams &p, int tiles, hipStream_t stream, const char **name) {
    // Two rows per wave when the history is short and the blocks' whole rounds
    // over the CUs cost no more than with one row (two_rows_per_wave; 4 tokens
    // at D = 8192: 144 and 160 rows 8.8-8.9 -> 7.2-7.3 us, 208 and 224 rows
    // 9.7-9.8 -> 9.2-9.3 us with one row); else one row per wave, its tokens split over two waves
    // when the grid is thin and the call long.  A wave with 5 to 8 tokens takes
    // them in one pass of 8; a longer one-row wave goes in passes of 4 with the
    // next pass in flight, a longer two-row wave in passes of 4 loaded at their
    // start.  Every form stays within 256 registers.
    const bool two = p.l <= 4 && two_rows_per_wave(p.n, tiles);
    const bool split = !two && (int64_t)p.n * tiles < kMaxWavesForSplit && p.t >= 2 * p.l;
    const int per_wave = split ? p.t - p.t / 2 : p.t;
    const bool one_pass = per_wave > 4 && per_wave <= 8;
#define DCCONV_TOK_NAME(LL, SUF)                                                              \
    (CL ? (ACT ? "tokens_v8<L=" #LL ",silu,channel_last," SUF ">"                            \
               : "tokens_v8<L=" #LL ",identity,channel_last," SUF ">")                       \
        : (ACT ? "tokens_v8<L=" #LL ",silu,compact," SUF ">" : "tokens_v8<L=" #LL ",identity,compact," SUF ">"))
#define DCCONV_TOK_CASE(LL)                                                                   \
    case LL:                                                                                  \
        if (split && one_pass) {                                                              \
            *name = DCCONV_TOK_NAME(LL, "R=1,split,one pass");                                \
            return launch_tokens_l<LL, ACT, CL, 1, 8, true, false>(p, tiles, stream);         \
        }                                                                                     \
        if (split) {                                                                          \
            *name = DCCONV_TOK_NAME(LL, "R=1,split");                                         \
            return launch_tokens_l<LL, ACT, CL, 1, 4, true, true>(p, tiles, stream);          \
        }                                                                                     \
        if (one_pass) {                                                                       \
            *name = DCCONV_TOK_NAME(LL, "R=1,one pass");                                      \
            return launch_tokens_l<LL, ACT, CL, 1, 8, false, false>(p, tiles, stream);        \
        }                                                                                     \
        *name = DCCONV_TOK_NAME(LL, "R=1");                                                   \
        return launch_tokens_l<LL, ACT, CL, 1, 4, false, true>(p, tiles, stream);
    if (two) {
        const bool one_pass_two = p.t > 4 && p.t <= 8;
        if (p.l == 3) {
            if (one_pass_two) {
                *name = DCCONV_TOK_NAME(3, "R=2,one pass");
                return launch_tokens_l<3, ACT, CL, 2, 8, false, false>(p, tiles, stream);
            }
            *name = DCCONV_TOK_NAME(3, "R=2");
            return launch_tokens_l<3, ACT, CL, 2, 4, false, false>(p, tiles, stream);
        }
        if (one_pass_two) {
            *name = DCCONV_TOK_NAME(4, "R=2,one pass");
            return launch_tokens_l<4, ACT, CL, 2, 8, false, false>(p, tiles, stream);
        }
        *name = DCCONV_TOK_NAME(4, "R=2");
        return launch_tokens_l<4, ACT, CL, 2, 4, false, false>(p, tiles, stream);
    }
    switch (p.l) {
        DCCONV_TOK_CASE(3)
        DCCONV_TOK_CASE(4)
        DCCONV_TOK_CASE(5)
        DCCONV_TOK_CASE(6)
        DCCONV_TOK_CASE(7)
        DCCONV_TOK_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef DCCONV_TOK_CASE
#undef DCCONV_TOK_NAME
}

}  // namespace

hipError_t launch_update_tokens(const TokensParams &p, StateLayout layout, int activation, hipStream_t stream,
                                const char **kernel_name) {
    if (p.seqlens != nullptr) return launch_update_tokens_ring(p, layout, activation, stream, kernel_name);
    const bool silu = activation == DCCONV_ACT_SILU;
    const int64_t lim = (int64_t)1 << 30;
    // The vector path needs 16-byte channel vectors everywhere and every buffer
    // descriptor below 2^30 bytes (see kBadToken / kBadLane).
    const bool v8 = p.d % kChPerLane == 0 && p.xs_d == 1 && p.os_d == 1 && (p.n == 1 || p.xs_n % 8 == 0) &&
                    (p.n == 1 || p.os_n % 8 == 0) && (p.t == 1 || (p.xs_t % 8 == 0 && p.os_t % 8 == 0)) &&
                    p.st_s % kChPerLane == 0 && p.l >= 3 && p.l <= 8 && p.xs_t * 2 * (int64_t)(p.t - 1) + 2 * kChPerWave < lim &&
                    p.os_t * 2 * (int64_t)(p.t - 1) + 2 * kChPerWave < lim && p.st_l * 2 * (int64_t)p.l + 2 * kChPerWave < lim;
    if (v8) {
        const int tiles = (p.d + kChPerWave - 1) / kChPerWave;
        if (layout == StateLayout::ChannelLast)
            return silu ? launch_tokens_v8<DCCONV_ACT_SILU, true>(p, tiles, stream, kernel_name)
                        : launch_tokens_v8<DCCONV_ACT_IDENTITY, true>(p, tiles, stream, kernel_name);
        return silu ? launch_tokens_v8<DCCONV_ACT_SILU, false>(p, tiles, stream, kernel_name)
                    : launch_tokens_v8<DCCONV_ACT_IDENTITY, false>(p, tiles, stream, kernel_name);
    }
    const int tiles = (p.d + kScalarBlock - 1) / kScalarBlock;
    *kernel_name = silu ? "tokens_scalar<silu>" : "tokens_scalar<identity>";
    return silu ? launch_tokens(tokens_scalar<DCCONV_ACT_SILU>, p, tiles, (int64_t)p.n * tiles, kScalarBlock, stream)
                : launch_tokens(tokens_scalar<DCCONV_ACT_IDENTITY>, p, tiles, (int64_t)p.n * tiles, kScalarBlock,
                                stream);
}

}  // namespace dcconv
