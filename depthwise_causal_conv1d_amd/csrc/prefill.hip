// Full-sequence causal convolution (prefill) for gfx950.
//
// The cuDNN FE-OSS page "Causal Conv1d Decode Update" names at its top a
// full-sequence prefill whose final state the decode update continues.  For
// sequence i (slot s) and channel c, with init = the slot's L values or zeros:
//
//   ext          = concat(init, x[i, c, 0:T])
//   out[i, c, j] = act(sum_k ext[L + j - 3 + k] * w[c, k] + bias[c])
//   final state  = ext[T : T + L]
//
// Outputs j >= 3 depend on x alone, so they need no ordering at all.  A call
// is one launch of one of two kernels, each with two roles: the edge role and
// a streaming role for the rest.  prefill_v8<L, ACT, layout, HAS_BIAS> (the
// column form, for wide rows with long columns):
//  * chunk blocks: one wavefront per (512-channel tile,
//    chunk of tokens), 8 channels per lane; the block's two waves take
//    neighbouring chunks of one tile and share its weights.  The chunk length
//    is set per call so that about 8 waves per CU each stream one long run (a
//    single resident round; 128 tokens for 8 x 2048 tokens at D = 8192).  A
//    chunk re-reads the 3 tokens before it (its halo).  Blocks go in plain
//    order, the tile varying fastest.  Tokens go in passes of 4, double
//    buffered: the next pass's loads are issued before the current pass is
//    computed and stored.
//  * edge blocks: everything that touches a slot -- the first min(3, T)
//    outputs, which read the initial state, and the final state, which
//    replaces it -- one wavefront per (sequence, tile), so each slot is read
//    and written by exactly one wave.  They come first in the grid, so their
//    short dependent chains run under the chunk blocks' streaming.
// prefill_sweep_v8<L, ACT, layout, HAS_BIAS> (the sweep form, for rows of at
// most 4096 channels or columns of at most 64 tokens): blocks of four waves,
// as many as the GPU holds at once, walk (16-token group, tile) items in
// memory order, so every block does nearly the same work and the grid reads
// one compact stretch of x at a time; a group's halo comes from the previous
// wave through LDS (see sweep_block).  Its edge blocks come after the sweep
// blocks and start as the first of those finish.  prefill_scalar<ACT> serves
// everything else (any strides, any L >= 3): one thread per (sequence,
// channel) walking its tokens in order.
// The roles write disjoint outputs and read x only, so they need no ordering
// between them.
#include <stdint.h>

#include "dcconv.h"
#include "device_common.h"
#include "update_params.h"

namespace dcconv {
namespace {

// Tokens per wave unit of the chunk kernel: chosen per call so that the grid
// holds about kTargetWaves waves (8 per CU: one resident round at this kernel's
// register use), within [kMinChunk, kMaxChunk] and a multiple of kPass.
constexpr int kMinChunk = 16;
constexpr int kMaxChunk = 256;
constexpr int64_t kTargetWaves = 2048;
constexpr int kPass = 4;    // tokens per load pass
// Buffer offsets beyond every descriptor used here (all are below 2^30 bytes):
// a token outside the piece, and a lane past a ragged tile.  Their sum and any
// valid offset plus either stay below 2^32.
constexpr uint32_t kBadToken = 1u << 30;
constexpr uint32_t kBadLane = 1u << 31;

enum { kStateless = 0, kCompactState = 1, kChannelLastState = 2 };

// Largest i in [0, n] with starts[i] <= q, or -1.  Each round the 64 lanes
// probe 64 evenly spaced entries of the remaining range at once, so the search
// costs ceil(log64(n + 1)) dependent loads instead of log2(n + 1).  All 64
// lanes call it; the result is wave-uniform.  Any table (ordered or not)
// narrows the range every round, so the loop ends.
__device__ __forceinline__ int find_seq(const int32_t *starts, int n, int q, int lane) {
    int lo = 0, hi = n;  // candidates lo..hi
    for (;;) {
        const int step = (hi - lo + kWave) / kWave;  // ceil((hi - lo + 1) / 64)
        const int idx = lo + lane * step;
        const bool le = idx <= hi && starts[idx] <= q;
        const int below = __popcll(__ballot(le));  // probes <= q: a prefix of the lanes for an ordered table
        if (below == 0) return lo - 1;
        const int base = lo + (below - 1) * step;
        if (step == 1) return base;
        lo = base;
        hi = min(hi, base + step - 1);
    }
}

// Outputs j in [max(j0, 3), j1) of sequence i, whose token j (channel c0 + ...)
// is at xseq[j*xs_t] and output at oseq[j*os_t].
template <int ACT>
__device__ __forceinline__ void chunk_piece(const PrefillParams &p, int i, int j0, int j1, const uint16_t *xseq,
                                            uint16_t *oseq, int c0, uint32_t vec_bytes, uint32_t lane_off, int lane,
                                            const float (&wf)[32], const float (&bf)[8]) {
    // The x loads do not wait for the routing: a padding sequence's tokens are
    // read too (they are valid memory) and its outputs are then zeroed, which
    // keeps the index load off the loads' dependence chain.
    const bool live = route_row(p.idx, p.status, p.n, p.s, i, lane) >= 0;
    const uint32_t x_tok = (uint32_t)p.xs_t * 2u, o_tok = (uint32_t)p.os_t * 2u;
    const int jb = max(j0 - 3, 0);  // first token read: the halo, clipped at the sequence start
    const Buffer xbuf = make_buffer(xseq + (int64_t)jb * p.xs_t + c0, x_tok * (uint32_t)(j1 - 1 - jb) + vec_bytes);
    const Buffer obuf = make_buffer(oseq + (int64_t)j0 * p.os_t + c0, o_tok * (uint32_t)(j1 - 1 - j0) + vec_bytes);
    auto xoff = [&](int j) -> uint32_t {
        return ((j >= jb && j < j1) ? x_tok * (uint32_t)(j - jb) : kBadToken) + lane_off;
    };
    // the three tokens before j0 (zero before the sequence start; never used there)
    u32x4 h0 = buffer_load<kStream>(xbuf, xoff(j0 - 3));
    u32x4 h1 = buffer_load<kStream>(xbuf, xoff(j0 - 2));
    u32x4 h2 = buffer_load<kStream>(xbuf, xoff(j0 - 1));
    u32x4 cur[kPass];
#pragma unroll
    for (int k = 0; k < kPass; ++k) cur[k] = buffer_load<kStream>(xbuf, xoff(j0 + k));
    for (int jj = j0; jj < j1; jj += kPass) {
        u32x4 nxt[kPass];
#pragma unroll
        for (int k = 0; k < kPass; ++k) nxt[k] = buffer_load<kStream>(xbuf, xoff(jj + kPass + k));
        u32x4 ov[kPass];
#pragma unroll
        for (int k = 0; k < kPass; ++k) {
            const u32x4 y = conv8<ACT>(h0, h1, h2, cur[k], wf, bf);
            ov[k] = live ? y : u32x4{0u, 0u, 0u, 0u};  // a padding sequence writes zeros
            h0 = h1;
            h1 = h2;
            h2 = cur[k];
        }
#pragma unroll
        for (int k = 0; k < kPass; ++k) {
            const int j = jj + k;
            buffer_store<kStream>(ov[k], obuf,
                                  ((j >= 3 && j < j1) ? o_tok * (uint32_t)(j - j0) : kBadToken) + lane_off);
        }
#pragma unroll
        for (int k = 0; k < kPass; ++k) cur[k] = nxt[k];
    }
}

// A wave-uniform cursor over the packed sequence table: sequence i covers
// packed tokens [a, e); ok is false past the table and for an entry that is not
// ordered (which sets DCCONV_DEV_BAD_SEQ); live is ok and routed to a slot.
struct SeqCursor {
    int i = 0, a = 0, e = 0;
    bool ok = false, live = false;

    __device__ __forceinline__ void enter(const PrefillParams &p, int next, int lane) {
        i = next;
        ok = i >= 0 && i < p.n;
        if (ok) {
            a = load_uniform(p.starts, i);
            e = load_uniform(p.starts, i + 1);
            ok = a >= 0 && a <= e && e <= p.t;
            if (!ok && p.status != nullptr && lane == 0) atomicOr(p.status, DCCONV_DEV_BAD_SEQ);
        }
        live = ok && route_row(p.idx, p.status, p.n, p.s, i, lane) >= 0;
    }
    // on to the sequence holding packed token q, past empty ones (ends at the
    // table's end: every step moves i forward)
    __device__ __forceinline__ void advance(const PrefillParams &p, int q, int lane) {
        while (ok && q >= e) enter(p, i + 1, lane);
    }
};

// The packed form: outputs of packed tokens [q0, q1).  A token's history is
// the three packed tokens before it whenever it is at least three tokens into
// its sequence, so the window rolls over the packed stream across sequence
// boundaries and the x loads are issued before the sequence table is read; the
// table only decides which outputs are stored (those at least three tokens
// into their sequence; the edge blocks write the first three) and which are
// zero (padding or rejected sequences).  A table that is not ordered stops the
// stores and sets DCCONV_DEV_BAD_SEQ; every access stays in bounds.
template <int ACT>
__device__ __forceinline__ void chunk_packed(const PrefillParams &p, int q0, int q1, int c0, uint32_t vec_bytes,
                                             uint32_t lane_off, int lane, const float (&wf)[32],
                                             const float (&bf)[8]) {
    const uint32_t x_tok = (uint32_t)p.xs_t * 2u, o_tok = (uint32_t)p.os_t * 2u;
    const int qb = max(q0 - 3, 0);
    const Buffer xbuf = make_buffer(p.x + (int64_t)qb * p.xs_t + c0, x_tok * (uint32_t)(q1 - 1 - qb) + vec_bytes);
    const Buffer obuf = make_buffer(p.out + (int64_t)q0 * p.os_t + c0, o_tok * (uint32_t)(q1 - 1 - q0) + vec_bytes);
    auto xoff = [&](int q) -> uint32_t {
        return ((q >= qb && q < q1) ? x_tok * (uint32_t)(q - qb) : kBadToken) + lane_off;
    };
    u32x4 h0 = buffer_load<kStream>(xbuf, xoff(q0 - 3));
    u32x4 h1 = buffer_load<kStream>(xbuf, xoff(q0 - 2));
    u32x4 h2 = buffer_load<kStream>(xbuf, xoff(q0 - 1));
    u32x4 cur[kPass];
#pragma unroll
    for (int k = 0; k < kPass; ++k) cur[k] = buffer_load<kStream>(xbuf, xoff(q0 + k));

    // the sequence holding q0: its first token a, its end e, and its routing
    SeqCursor sc;
    sc.enter(p, find_seq(p.starts, p.n, q0, lane), lane);
    for (int qq = q0; qq < q1; qq += kPass) {
        u32x4 nxt[kPass];
#pragma unroll
        for (int k = 0; k < kPass; ++k) nxt[k] = buffer_load<kStream>(xbuf, xoff(qq + kPass + k));
        u32x4 ov[kPass];
        uint32_t off[kPass];
        if (sc.ok && qq - sc.a >= 3 && qq + kPass <= sc.e && qq + kPass <= q1) {
            // the common pass: inside one sequence, past its first three tokens
#pragma unroll
            for (int k = 0; k < kPass; ++k) {
                const u32x4 y = conv8<ACT>(h0, h1, h2, cur[k], wf, bf);
                h0 = h1;
                h1 = h2;
                h2 = cur[k];
                ov[k] = sc.live ? y : u32x4{0u, 0u, 0u, 0u};
                off[k] = o_tok * (uint32_t)(qq + k - q0) + lane_off;
            }
        } else {
#pragma unroll
            for (int k = 0; k < kPass; ++k) {
                const int q = qq + k;
                const u32x4 y = conv8<ACT>(h0, h1, h2, cur[k], wf, bf);
                h0 = h1;
                h1 = h2;
                h2 = cur[k];
                if (q < q1) sc.advance(p, q, lane);
                ov[k] = sc.live ? y : u32x4{0u, 0u, 0u, 0u};
                off[k] = ((sc.ok && q < q1 && q - sc.a >= 3) ? o_tok * (uint32_t)(q - q0) : kBadToken) + lane_off;
            }
        }
#pragma unroll
        for (int k = 0; k < kPass; ++k) buffer_store<kStream>(ov[k], obuf, off[k]);
#pragma unroll
        for (int k = 0; k < kPass; ++k) cur[k] = nxt[k];
    }
}

// One block of the chunk role: block v of the chunk blocks, the (tile, pair of
// chunks) with the tile varying fastest.
template <int ACT, bool HAS_BIAS>
__device__ __forceinline__ void chunk_block(const PrefillParams &p, u32x4 *weight_tile, int tiles, int chunk,
                                            int64_t units, int64_t units_per_seq, int64_t v) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    {
        const int tile = (int)(v % tiles);
        const int64_t unit = (v / tiles) * kWavesPerBlock + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
        const uint32_t lane_off = lane < lanes_used ? lane_bytes : kBadLane;

        u32x4 wraw[kWeightChunks];
        weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        float wf[32], bf[8];
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        weight_tile_share(weight_tile, wraw, wave, lane, wf);
        unpack_bias(bv, bf);

        if (unit < units) {
            if (p.starts == nullptr) {
                // batch form: the unit is chunk c of sequence i
                const int i = (int)(unit / units_per_seq);
                const int j0 = (int)(unit % units_per_seq) * chunk;
                const int j1 = min(p.t, j0 + chunk);
                chunk_piece<ACT>(p, i, j0, j1, p.x + (int64_t)i * p.xs_n, p.out + (int64_t)i * p.os_n, c0, vec_bytes,
                                 lane_off, lane, wf, bf);
            } else {
                // packed form: the unit is packed tokens [q0, q1)
                const int q0 = (int)unit * chunk;
                chunk_packed<ACT>(p, q0, min(p.t, q0 + chunk), c0, vec_bytes, lane_off, lane, wf, bf);
            }
        }
        __syncthreads();  // the weight tile is reused by the next block unit
    }
}

// ---- the sweep role ---------------------------------------------------------
// Tokens per wave and waves per block of the sweep role; an item is kSweepSpan
// consecutive tokens of one 512-channel tile.  Four tokens per wave keep the
// kernel at 123 VGPRs, four waves per SIMD (eight tokens: 143, three).  A wave
// hands its last three tokens to the next as that wave's halo, so it must own
// at least three.
constexpr int kSweepG = 4;
constexpr int kSweepWaves = 4;
constexpr int kSweepSpan = kSweepG * kSweepWaves;
constexpr int kSweepBlock = kWave * kSweepWaves;
static_assert(kSweepG >= 3, "a wave's last three tokens are the next wave's halo");

// This lane's 8 channels x 4 taps (64 contiguous bytes of the [D, 4] weight) as
// FP32, channel-major; zeros for a lane past a ragged tile.
__device__ __forceinline__ void lane_weights(const uint16_t *weight, int c0, uint32_t vec_bytes, uint32_t lane_bytes,
                                             float (&wf)[32]) {
    const Buffer wbuf = make_buffer(weight + (int64_t)c0 * 4, vec_bytes * 4u);
    u32x4 wd[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) wd[k] = buffer_load<kCached>(wbuf, lane_bytes * 4u + 16u * (uint32_t)k);
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wf[8 * k + 2 * q] = lo_f32(wd[k][q]);
            wf[8 * k + 2 * q + 1] = hi_f32(wd[k][q]);
        }
}

// One block of the sweep role, block b of `grid` (a multiple of tiles, so the
// block keeps one tile and its weights): items b, b + grid, ... in memory order,
// item = (group of kSweepSpan tokens, tile) with the tile fastest.  Wave w
// takes tokens [g0 + w*kSweepG, +kSweepG) of the item's [g0, g1); wave 0 loads
// the 3 tokens before g0, every other wave takes its 3 from the previous wave's
// last three through LDS (`tails`, kSweepWaves x 3 vectors per lane).  The
// batch form's groups do not cross sequences; the packed form's run over the
// packed stream, and the sequence table decides the stores as in chunk_packed.
template <int ACT, bool HAS_BIAS>
__device__ __forceinline__ void sweep_block(const PrefillParams &p, u32x4 *tails, int tiles, int64_t items,
                                            int64_t groups_per_seq, int64_t b, int64_t grid) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    const int tile = (int)(b % tiles);
    const int c0 = tile * kChPerWave;
    const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
    const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
    const uint32_t lane_off = lane < lanes_used ? lane_bytes : kBadLane;
    const uint32_t x_tok = (uint32_t)p.xs_t * 2u, o_tok = (uint32_t)p.os_t * 2u;
    const bool packed = p.starts != nullptr;
    float wf[32], bf[8];
    {
        u32x4 bv = u32x4{0u, 0u, 0u, 0u};
        if (HAS_BIAS) bv = buffer_load<kCached>(make_buffer(p.bias + c0, vec_bytes), lane_bytes);
        lane_weights(p.weight, c0, vec_bytes, lane_bytes, wf);
        unpack_bias(bv, bf);
    }
    for (int64_t item = b; item < items; item += grid) {  // block-uniform
        const int64_t group = item / tiles;
        const int i = packed ? 0 : (int)(group / groups_per_seq);
        const int g0 = (int)(packed ? group : group % groups_per_seq) * kSweepSpan;
        const int g1 = min(p.t, g0 + kSweepSpan);
        const int lo = max(g0 - 3, 0);
        const int j0 = g0 + wave * kSweepG;
        const uint16_t *xs = p.x + (packed ? 0 : (int64_t)i * p.xs_n) + c0;
        uint16_t *os = p.out + (packed ? 0 : (int64_t)i * p.os_n) + c0;
        const Buffer xbuf = make_buffer(xs + (int64_t)lo * p.xs_t, x_tok * (uint32_t)(g1 - 1 - lo) + vec_bytes);
        const Buffer obuf = make_buffer(os + (int64_t)g0 * p.os_t, o_tok * (uint32_t)(g1 - 1 - g0) + vec_bytes);
        auto xoff = [&](int j) -> uint32_t {
            return ((j >= lo && j < g1) ? x_tok * (uint32_t)(j - lo) : kBadToken) + lane_off;
        };
        // v[k] holds token j0 - 3 + k
        u32x4 v[kSweepG + 3];
#pragma unroll
        for (int k = 0; k < kSweepG; ++k) v[k + 3] = buffer_load<kStream>(xbuf, xoff(j0 + k));
        if (wave == 0) {
#pragma unroll
            for (int k = 0; k < 3; ++k) v[k] = buffer_load<kStream>(xbuf, xoff(g0 - 3 + k));
        }

        // which of this wave's outputs are stored (the edge role writes each
        // sequence's first three), and which are zeros (padding, rejected)
        uint32_t off[kSweepG];
        bool live[kSweepG];
        if (!packed) {
            const bool row_live = route_row(p.idx, p.status, p.n, p.s, i, lane) >= 0;
#pragma unroll
            for (int k = 0; k < kSweepG; ++k) {
                const int j = j0 + k;
                off[k] = ((j >= 3 && j < g1) ? o_tok * (uint32_t)(j - g0) : kBadToken) + lane_off;
                live[k] = row_live;
            }
        } else if (j0 < g1) {
            SeqCursor sc;
            sc.enter(p, find_seq(p.starts, p.n, j0, lane), lane);
            if (sc.ok && j0 - sc.a >= 3 && j0 + kSweepG <= sc.e && j0 + kSweepG <= g1) {
#pragma unroll
                for (int k = 0; k < kSweepG; ++k) {
                    off[k] = o_tok * (uint32_t)(j0 + k - g0) + lane_off;
                    live[k] = sc.live;
                }
            } else {
#pragma unroll
                for (int k = 0; k < kSweepG; ++k) {
                    const int q = j0 + k;
                    if (q < g1) sc.advance(p, q, lane);
                    off[k] = ((sc.ok && q < g1 && q - sc.a >= 3) ? o_tok * (uint32_t)(q - g0) : kBadToken) + lane_off;
                    live[k] = sc.live;
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < kSweepG; ++k) {
                off[k] = kBadToken + lane_off;
                live[k] = false;
            }
        }

        // the halos: publish this wave's last three tokens, take the previous wave's
        u32x4 *mine = tails + wave * 3 * kWave;
#pragma unroll
        for (int k = 0; k < 3; ++k) mine[k * kWave + lane] = v[kSweepG + k];
        __syncthreads();
        if (wave > 0) {
            const u32x4 *prev = tails + (wave - 1) * 3 * kWave;
#pragma unroll
            for (int k = 0; k < 3; ++k) v[k] = prev[k * kWave + lane];
        }
        // outputs from the last, each in place of its own token
#pragma unroll
        for (int k = kSweepG - 1; k >= 0; --k) {
            const u32x4 y = conv8<ACT>(v[k], v[k + 1], v[k + 2], v[k + 3], wf, bf);
            v[k + 3] = live[k] ? y : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int k = 0; k < kSweepG; ++k) buffer_store<kStream>(v[k + 3], obuf, off[k]);
        __syncthreads();  // the tails are rewritten by the next item
    }
}

// One block of the edge role: block unit bu = (WPB sequences, tile).
// stage_all holds kWave * L vectors per wave: the compact state's
// transposition, then the planes, which the final state picks at a run-time
// position.  Two-wave blocks share the tile's weights through weight_tile;
// other blocks load each lane's weights directly.
template <int L, int ACT, int LAYOUT, int WPB>
__device__ __forceinline__ void edge_block(const PrefillParams &p, u32x4 *stage_all, u32x4 *weight_tile, int tiles,
                                           int64_t bu) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const uint32_t lane_bytes = (uint32_t)lane * 16u;
    const uint32_t x_tok = (uint32_t)p.xs_t * 2u, o_tok = (uint32_t)p.os_t * 2u, plane_bytes = (uint32_t)p.st_l * 2u;
    {
        const int tile = (int)(bu % tiles);
        const int i_raw = (int)(bu / tiles) * WPB + wave;
        const int c0 = tile * kChPerWave;
        const int lanes_used = min(kWave, (p.d - c0) / kChPerLane);
        const uint32_t vec_bytes = (uint32_t)lanes_used * 16u;
        const uint32_t lane_off = lane < lanes_used ? lane_bytes : kBadLane;
        const bool in_range = i_raw < p.n;
        const int i = min(i_raw, p.n - 1);

        // the sequence's tokens; a packed table that is not ordered is flagged and
        // the sequence skipped
        int a = 0, e = p.t;
        bool ok = in_range;
        if (p.starts != nullptr) {
            a = p.starts[i];
            e = p.starts[i + 1];
            const bool ordered = a >= 0 && a <= e && e <= p.t && (i > 0 || a == 0) && (i < p.n - 1 || e == p.t);
            if (in_range && !ordered && p.status != nullptr && lane == 0) atomicOr(p.status, DCCONV_DEV_BAD_SEQ);
            ok = ok && ordered;
        }
        const int len = ok ? e - a : 0;
        const int slot = __builtin_amdgcn_readfirstlane(ok ? route_row(p.idx, p.status, p.n, p.s, i, lane) : -2);
        const bool live = slot >= 0;
        const bool stateful = LAYOUT != kStateless;
        const bool from_state = stateful && live && p.has_init != nullptr && p.has_init[i] != 0;
        const bool writes_state = stateful && live;
        const uint16_t *xseq = p.starts != nullptr ? p.x + (int64_t)a * p.xs_t : p.x + (int64_t)i * p.xs_n;
        uint16_t *oseq = p.starts != nullptr ? p.out + (int64_t)a * p.os_t : p.out + (int64_t)i * p.os_n;
        const int nf = min(len, 3);  // outputs written here

        __builtin_amdgcn_s_setprio(3);
        u32x4 wraw[kWeightChunks];
        if constexpr (WPB == kWavesPerBlock) weight_tile_issue(wraw, p.weight, c0, vec_bytes, wave, lane_bytes);
        const u32x4 bv = buffer_load<kCached>(make_buffer(p.bias != nullptr ? p.bias + c0 : p.weight,
                                                          p.bias != nullptr ? vec_bytes : 0u),
                                              lane_bytes);
        // initial state (zeros unless this sequence continues from its slot)
        const int64_t slot_base = (int64_t)(live ? slot : 0) * p.st_s;
        u32x4 sv[L];
        if (LAYOUT == kChannelLastState) {
            const Buffer sbuf = make_buffer(p.state + slot_base + c0, from_state ? plane_bytes * (uint32_t)(L - 1) + vec_bytes : 0u);
#pragma unroll
            for (int k = 0; k < L; ++k) sv[k] = buffer_load<kStream>(sbuf, plane_bytes * (uint32_t)k + lane_off);
        } else if (LAYOUT == kCompactState) {
            const Buffer sbuf = make_buffer(p.state + slot_base + (int64_t)c0 * L, from_state ? vec_bytes * L : 0u);
#pragma unroll
            for (int j = 0; j < L; ++j) sv[j] = buffer_load<kStream>(sbuf, (uint32_t)(j * kWave) * 16u + lane_bytes);
        } else {
#pragma unroll
            for (int k = 0; k < L; ++k) sv[k] = u32x4{0u, 0u, 0u, 0u};
        }
        // tokens 0..2 (the outputs here) and the last min(len, L) tokens (the final state)
        const Buffer xhead = make_buffer(xseq + c0, live && nf > 0 ? x_tok * (uint32_t)(nf - 1) + vec_bytes : 0u);
        u32x4 xf[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) xf[j] = buffer_load<kStream>(xhead, (j < nf ? x_tok * (uint32_t)j : kBadToken) + lane_off);
        const int tail0 = max(len - L, 0);
        const int ntail = len - tail0;
        const Buffer xtail = make_buffer(xseq + (int64_t)tail0 * p.xs_t + c0,
                                         writes_state && ntail > 0 ? x_tok * (uint32_t)(ntail - 1) + vec_bytes : 0u);
        u32x4 xl[L];
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int tok = len - L + k;  // token that lands at final position k, if >= 0
            xl[k] = buffer_load<kStream>(xtail, (tok >= 0 ? x_tok * (uint32_t)(tok - tail0) : kBadToken) + lane_off);
        }
        __builtin_amdgcn_s_setprio(0);

        float wf[32], bf[8];
        if constexpr (WPB == kWavesPerBlock)
            weight_tile_share(weight_tile, wraw, wave, lane, wf);
        else
            lane_weights(p.weight, c0, vec_bytes, lane_bytes, wf);
        unpack_bias(bv, bf);

        u32x4 pl[L];
        if (LAYOUT == kCompactState) {
            u32x4 *stage = stage_all + wave * (kWave * L);
#pragma unroll
            for (int j = 0; j < L; ++j) stage[j * kWave + lane] = sv[j];
            wave_lds_sync();
            uint32_t h[4 * L];
#pragma unroll
            for (int k = 0; k < L; ++k) {
                const u32x4 t = stage[lane * L + k];
#pragma unroll
                for (int q = 0; q < 4; ++q) h[4 * k + q] = t[q];
            }
            to_planes<L>(h, pl);
        } else {
#pragma unroll
            for (int k = 0; k < L; ++k) pl[k] = sv[k];
        }

        // outputs 0..2: ext position L + j - 3 + m is init plane (< L) or token (>= L)
        u32x4 ov[3];
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            u32x4 hv[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int pos = L + j - 3 + m;
                hv[m] = pos < L ? pl[pos < L ? pos : 0] : xf[pos >= L ? pos - L : 0];
            }
            const u32x4 y = conv8<ACT>(hv[0], hv[1], hv[2], hv[3], wf, bf);
            ov[j] = live ? y : u32x4{0u, 0u, 0u, 0u};
        }
        // final state: position k is ext[len + k], a token or (len + k < L) the
        // initial plane len + k, picked through LDS (a run-time position)
        u32x4 *stage = stage_all + wave * (kWave * L);
        wave_lds_sync();
#pragma unroll
        for (int k = 0; k < L; ++k) stage[k * kWave + lane] = pl[k];
        wave_lds_sync();
        u32x4 fs[L];
#pragma unroll
        for (int k = 0; k < L; ++k) {
            const int m = len + k < L ? len + k : 0;
            const u32x4 old = stage[m * kWave + lane];
            fs[k] = (len + k >= L) ? xl[k] : old;
        }

        __builtin_amdgcn_sched_barrier(0);
        const Buffer obuf = make_buffer(oseq + c0, ok && nf > 0 ? o_tok * (uint32_t)(nf - 1) + vec_bytes : 0u);
#pragma unroll
        for (int j = 0; j < 3; ++j) buffer_store<kStream>(ov[j], obuf, (j < nf ? o_tok * (uint32_t)j : kBadToken) + lane_off);
        if (LAYOUT == kChannelLastState) {
            const Buffer wbuf = make_buffer(p.state + slot_base + c0, writes_state ? plane_bytes * (uint32_t)(L - 1) + vec_bytes : 0u);
#pragma unroll
            for (int k = 0; k < L; ++k) buffer_store<kStream>(fs[k], wbuf, plane_bytes * (uint32_t)k + lane_off);
        } else if (LAYOUT == kCompactState) {
            uint32_t h[4 * L];
            from_planes<L>(fs, h);
            wave_lds_sync();
#pragma unroll
            for (int k = 0; k < L; ++k) stage[lane * L + k] = u32x4{h[4 * k], h[4 * k + 1], h[4 * k + 2], h[4 * k + 3]};
            wave_lds_sync();
            u32x4 nv[L];
#pragma unroll
            for (int j = 0; j < L; ++j) nv[j] = stage[j * kWave + lane];
            const Buffer wbuf = make_buffer(p.state + slot_base + (int64_t)c0 * L, writes_state ? vec_bytes * L : 0u);
#pragma unroll
            for (int j = 0; j < L; ++j) buffer_store<kStream>(nv[j], wbuf, (uint32_t)(j * kWave) * 16u + lane_bytes);
        }
        __syncthreads();  // the stage and the weight tile are reused by the next unit
    }
}

// Both roles in one launch: the edge blocks first (they start before the long
// chunk blocks and finish under them), then the chunk blocks.
template <int L, int ACT, int LAYOUT, bool HAS_BIAS>
__global__ __launch_bounds__(kBlock) void prefill_v8(PrefillParams p, int tiles, int chunk, int64_t units,
                                                     int64_t units_per_seq, int64_t chunk_blocks,
                                                     int64_t edge_blocks) {
    __shared__ u32x4 stage_all[kWavesPerBlock * kWave * L];
    __shared__ u32x4 weight_tile[4 * kWave];
    const int64_t total = edge_blocks + chunk_blocks;
    // min(units, kMaxBlocks) blocks: the first unit needs no test (see for_each_unit)
    int64_t b = blockIdx.x;
    do {
        if (b < edge_blocks)
            edge_block<L, ACT, LAYOUT, kWavesPerBlock>(p, stage_all, weight_tile, tiles, b);
        else
            chunk_block<ACT, HAS_BIAS>(p, weight_tile, tiles, chunk, units, units_per_seq, b - edge_blocks);
        b += kMaxBlocks;
    } while (b < total);
}

// The sweep form of the same call: `grid` sweep blocks and `edge_blocks` edge
// blocks of kSweepWaves sequences.  With few edge blocks they come last and
// start as the first sweep blocks finish; with many (many short sequences) they
// come first and the sweep grid leaves room for them.
template <int L, int ACT, int LAYOUT, bool HAS_BIAS>
__global__ __launch_bounds__(kSweepBlock) void prefill_sweep_v8(PrefillParams p, int tiles, int64_t items,
                                                                int64_t groups_per_seq, int64_t grid,
                                                                int64_t edge_blocks, int edges_first) {
    __shared__ u32x4 lds[kSweepWaves * kWave * L];  // the sweep role's halos, or the edge role's stages
    const int64_t b = blockIdx.x;
    const int64_t sweep_b = edges_first ? b - edge_blocks : b;
    if (sweep_b >= 0 && sweep_b < grid)
        sweep_block<ACT, HAS_BIAS>(p, lds, tiles, items, groups_per_seq, sweep_b, grid);
    else
        edge_block<L, ACT, LAYOUT, kSweepWaves>(p, lds, nullptr, tiles, edges_first ? b : b - grid);
}

template <int ACT>
__global__ __launch_bounds__(kScalarBlock) void prefill_scalar(PrefillParams p, int tiles_per_seq, int64_t units) {
    const int lane = threadIdx.x & (kWave - 1);
    for_each_unit(units, [&](int64_t unit) {
        const int i = (int)(unit / tiles_per_seq);
        const int c = (int)(unit - (int64_t)i * tiles_per_seq) * kScalarBlock + (int)threadIdx.x;
        int a = 0, e = p.t;
        bool ok = true;
        if (p.starts != nullptr) {
            a = p.starts[i];
            e = p.starts[i + 1];
            ok = a >= 0 && a <= e && e <= p.t && (i > 0 || a == 0) && (i < p.n - 1 || e == p.t);
            if (!ok && p.status != nullptr && threadIdx.x == 0) atomicOr(p.status, DCCONV_DEV_BAD_SEQ);
        }
        const int slot = ok ? route_row(p.idx, p.status, p.n, p.s, i, lane) : -2;
        if (c >= p.d || !ok) return;
        const int len = e - a;
        const uint16_t *xc = (p.starts != nullptr ? p.x + (int64_t)a * p.xs_t : p.x + (int64_t)i * p.xs_n) +
                             (int64_t)c * p.xs_d;
        uint16_t *oc = (p.starts != nullptr ? p.out + (int64_t)a * p.os_t : p.out + (int64_t)i * p.os_n) +
                       (int64_t)c * p.os_d;
        if (slot < 0) {  // padding (or rejected) sequence
            for (int j = 0; j < len; ++j) oc[(int64_t)j * p.os_t] = 0;
            return;
        }
        const bool stateful = p.state != nullptr;
        const bool from_state = stateful && p.has_init != nullptr && p.has_init[i] != 0;
        const int L = stateful ? p.l : 3;
        uint16_t *h = stateful ? p.state + (int64_t)slot * p.st_s + (int64_t)c * p.st_d : nullptr;
        const int64_t sl = p.st_l;
        const uint16_t *wt = p.weight + (int64_t)c * 4;
        const float w0 = bf16_bits_to_f32(wt[0]), w1 = bf16_bits_to_f32(wt[1]);
        const float w2 = bf16_bits_to_f32(wt[2]), w3 = bf16_bits_to_f32(wt[3]);
        const float b = p.bias != nullptr ? bf16_bits_to_f32(p.bias[c]) : 0.0f;
        float h0 = from_state ? bf16_bits_to_f32(h[(L - 3) * sl]) : 0.0f;
        float h1 = from_state ? bf16_bits_to_f32(h[(L - 2) * sl]) : 0.0f;
        float h2 = from_state ? bf16_bits_to_f32(h[(L - 1) * sl]) : 0.0f;
        for (int j = 0; j < len; ++j) {
            const float xv = bf16_bits_to_f32(xc[(int64_t)j * p.xs_t]);
            float acc = h0 * w0;
            acc = __builtin_fmaf(h1, w1, acc);
            acc = __builtin_fmaf(h2, w2, acc);
            acc = __builtin_fmaf(xv, w3, acc);
            acc += b;
            oc[(int64_t)j * p.os_t] = f32_to_bf16_bits(activate<ACT>(acc));
            h0 = h1;
            h1 = h2;
            h2 = xv;
        }
        if (stateful) {
            // final position k is ext[len + k]: a token, or (len + k < L) the initial
            // value at position len + k, read before it is overwritten (len + k >= k)
            for (int k = 0; k < L; ++k) {
                const int m = len + k;
                uint16_t v = 0;
                if (m >= L)
                    v = xc[(int64_t)(m - L) * p.xs_t];
                else if (from_state)
                    v = h[(int64_t)m * sl];
                h[(int64_t)k * sl] = v;
            }
        }
    });
}

template <typename Kernel, typename... Args>
hipError_t launch(Kernel kernel, int64_t blocks, int block, hipStream_t stream, Args... args) {
    void *argv[] = {&args...};
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks), dim3(block), argv, 0,
                           stream);
}

// Blocks of `kernel` (at `block` threads) that the current device holds at
// once, or 0.  `cache` holds the answer per device (a partitioned GPU shows
// devices of different sizes); concurrent first calls store the same value.
constexpr int kMaxDevices = 64;
int resident_blocks(const void *kernel, int block, int (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices && __atomic_load_n(&cache[dev], __ATOMIC_RELAXED) > 0)
        return __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess)
        return 0;
    const int n = cus * per_cu;
    if (dev < kMaxDevices) __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
    return n;
}

// The sweep grid: every block the GPU holds at once (cap), rounded down to a
// multiple of `tiles` so a block keeps one tile, or one block per item when
// there are fewer.  Every block then does ceil(items / grid) or one fewer
// items.  (Trading residency for whole rounds -- the multiple of `tiles` in
// [cap / 2, cap] that pads the item count least -- measured slower: with two
// blocks per CU instead of four, 8 x 2048 tokens at D = 4096 took 58.8 us
// against 51.3.)
int64_t sweep_grid(int64_t items, int tiles, int64_t cap) {
    const int64_t gmax = cap / tiles * tiles;
    if (gmax < tiles) return 0;
    return items <= gmax ? items : gmax;
}

// Column (chunk) or sweep form.  A/B on MI355X: the sweep wins where rows are
// narrow (D <= 4096: 7-25 %) or the columns short (64-token chunks at D = 8192:
// 6 %); long columns of wide rows run 1-3 % faster as chunks.
template <int L, int ACT, int LAYOUT>
hipError_t launch_prefill_l(const PrefillParams &p, int tiles, hipStream_t stream, bool *swept) {
    const bool packed = p.starts != nullptr;
    const int64_t tokens = packed ? (int64_t)p.t : (int64_t)p.t * p.n;
    int64_t chunk = (tokens * tiles + kTargetWaves - 1) / kTargetWaves;
    chunk = (chunk + kPass - 1) / kPass * kPass;
    chunk = chunk < kMinChunk ? kMinChunk : chunk > kMaxChunk ? kMaxChunk : chunk;
    PrefillParams pp = p;
    *swept = false;
    if (p.d <= 4096 || chunk <= 64) {
        const int64_t groups_per_seq = ((int64_t)p.t + kSweepSpan - 1) / kSweepSpan;
        const int64_t items = (packed ? groups_per_seq : groups_per_seq * p.n) * tiles;
        const int64_t edge_blocks = ((int64_t)p.n + kSweepWaves - 1) / kSweepWaves * tiles;
        auto kernel = p.bias != nullptr ? prefill_sweep_v8<L, ACT, LAYOUT, true> : prefill_sweep_v8<L, ACT, LAYOUT, false>;
        static int cache[kMaxDevices];
        const int64_t resident = resident_blocks(reinterpret_cast<const void *>(kernel), kSweepBlock, cache);
        const int edges_first = edge_blocks > resident / 8;
        const int64_t cap = edges_first ? (resident - edge_blocks > resident / 2 ? resident - edge_blocks : resident / 2)
                                        : resident;
        const int64_t grid = sweep_grid(items, tiles, cap);
        if (grid > 0 && grid + edge_blocks < kMaxBlocks) {
            *swept = true;
            return launch(kernel, grid + edge_blocks, kSweepBlock, stream, pp, tiles, items, groups_per_seq, grid,
                          edge_blocks, edges_first);
        }
    }
    const int64_t units_per_seq = ((int64_t)p.t + chunk - 1) / chunk;
    const int64_t units = packed ? units_per_seq : units_per_seq * p.n;
    const int64_t chunk_blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock * tiles;
    const int64_t edge_blocks = ((int64_t)p.n + kWavesPerBlock - 1) / kWavesPerBlock * tiles;
    const int64_t total = edge_blocks + chunk_blocks;
    const int64_t grid = total < kMaxBlocks ? total : kMaxBlocks;
    const int ch = (int)chunk;
    return p.bias != nullptr
               ? launch(prefill_v8<L, ACT, LAYOUT, true>, grid, kBlock, stream, pp, tiles, ch, units, units_per_seq,
                        chunk_blocks, edge_blocks)
               : launch(prefill_v8<L, ACT, LAYOUT, false>, grid, kBlock, stream, pp, tiles, ch, units, units_per_seq,
                        chunk_blocks, edge_blocks);
}

template <int ACT, int LAYOUT>
hipError_t launch_prefill_layout(const PrefillParams &p, int tiles, hipStream_t stream, const char **name) {
#define DCCONV_PF_NAME(KN, LL)                                                            \
    (LAYOUT == kStateless                                                                 \
         ? (ACT ? KN "<stateless,silu>" : KN "<stateless,identity>")                      \
         : LAYOUT == kCompactState                                                        \
               ? (ACT ? KN "<L=" #LL ",silu,compact>" : KN "<L=" #LL ",identity,compact>") \
               : (ACT ? KN "<L=" #LL ",silu,channel_last>" : KN "<L=" #LL ",identity,channel_last>"))
#define DCCONV_PF_CASE(LL)                                                                             \
    case LL: {                                                                                         \
        bool swept = false;                                                                            \
        const hipError_t err = launch_prefill_l<LL, ACT, LAYOUT>(p, tiles, stream, &swept);            \
        *name = swept ? DCCONV_PF_NAME("prefill_sweep_v8", LL) : DCCONV_PF_NAME("prefill_v8", LL);     \
        return err;                                                                                    \
    }
    if constexpr (LAYOUT == kStateless) {
        switch (3) { DCCONV_PF_CASE(3) }
    } else {
        switch (p.l) {
            DCCONV_PF_CASE(3)
            DCCONV_PF_CASE(4)
            DCCONV_PF_CASE(5)
            DCCONV_PF_CASE(6)
            DCCONV_PF_CASE(7)
            DCCONV_PF_CASE(8)
            default: return hipErrorInvalidValue;
        }
    }
#undef DCCONV_PF_CASE
#undef DCCONV_PF_NAME
    return hipErrorInvalidValue;
}

template <int ACT>
hipError_t launch_prefill_v8(const PrefillParams &p, StateLayout layout, hipStream_t stream, const char **name) {
    const int tiles = (p.d + kChPerWave - 1) / kChPerWave;
    if (p.state == nullptr) return launch_prefill_layout<ACT, kStateless>(p, tiles, stream, name);
    if (layout == StateLayout::ChannelLast) return launch_prefill_layout<ACT, kChannelLastState>(p, tiles, stream, name);
    return launch_prefill_layout<ACT, kCompactState>(p, tiles, stream, name);
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, StateLayout layout, int activation, hipStream_t stream,
                          const char **kernel_name) {
    const bool silu = activation == DCCONV_ACT_SILU;
    const int64_t lim = (int64_t)1 << 30;
    const bool stateful = p.state != nullptr;
    // The vector path needs 16-byte channel vectors everywhere and every buffer
    // descriptor below 2^30 bytes (see kBadToken / kBadLane): a chunk with its
    // halo, the 3 head or L tail tokens of the edges, the L state planes.
    const bool v8 = p.d % kChPerLane == 0 && p.xs_d == 1 && p.os_d == 1 && p.xs_t % 8 == 0 && p.os_t % 8 == 0 &&
                    (p.starts != nullptr || p.n == 1 || (p.xs_n % 8 == 0 && p.os_n % 8 == 0)) &&
                    p.xs_t * 2 * (int64_t)(kMaxChunk + 3) + 2 * kChPerWave < lim &&
                    p.os_t * 2 * (int64_t)(kMaxChunk + 3) + 2 * kChPerWave < lim &&
                    (!stateful || (p.st_s % kChPerLane == 0 && p.l >= 3 && p.l <= 8 &&
                                   p.st_l * 2 * (int64_t)p.l + 2 * kChPerWave < lim));
    if (v8) return silu ? launch_prefill_v8<DCCONV_ACT_SILU>(p, layout, stream, kernel_name)
                        : launch_prefill_v8<DCCONV_ACT_IDENTITY>(p, layout, stream, kernel_name);
    const int tiles = (p.d + kScalarBlock - 1) / kScalarBlock;
    const int64_t units = (int64_t)p.n * tiles;
    const int64_t grid = units < kMaxBlocks ? units : kMaxBlocks;
    *kernel_name = silu ? "prefill_scalar<silu>" : "prefill_scalar<identity>";
    PrefillParams pp = p;
    return silu ? launch(prefill_scalar<DCCONV_ACT_SILU>, grid, kScalarBlock, stream, pp, tiles, units)
                : launch(prefill_scalar<DCCONV_ACT_IDENTITY>, grid, kScalarBlock, stream, pp, tiles, units);
}

}  // namespace dcconv
