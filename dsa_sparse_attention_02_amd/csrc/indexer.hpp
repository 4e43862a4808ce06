// Indexer scoring kernels (gfx950, bf16 MFMA with fp32 accumulation).
//
// score[r][s] = sum_j w[r][j] * ReLU( sum_c iq[r][j][c] * ik[s][c] )
// for every key s visible to query row r.  The pages call for a lightweight
// scoring network whose matmul keeps more precision than the attention
// ("Day-0 Adaptation for LLMs: Implementing Sparse Attention and Low-Precision
// Weights", section III.1, and its Validation System section: index scoring
// stays in BF16/FP32); here the products are bf16 x bf16 accumulated in fp32
// by the matrix cores and the head reduction runs in fp32.
//
// MFMA mapping: D[j][s] = sum_c Q[j][c] K[s][c], M = 32 indexer heads per tile,
// N = 32 keys, K = 16 dims per instruction.  The contraction order over c is
// free, so lane half h supplies dims h*D/2 + 8*ks .. +7 at step ks for both
// operands: a key row is then read as D/2 contiguous bytes per lane.  After the
// MFMAs a lane holds 16 heads of one key; ReLU, the head weights and the head
// sum are applied in registers and the two lane halves are added with one swap.
#pragma once

#include <type_traits>

#include "device_common.hpp"

namespace sa {

// ------------------------------------------------------------------ decode --
// Persistent key scan.  The visible keys of all rows form one list of 32-key
// tiles (row-major, each row's tiles in key order); wave g of G takes the
// contiguous tiles [g*T/G, (g+1)*T/G), so every wave moves the same number of
// bytes whatever the context lengths.  Key tiles stream HBM -> LDS through the
// LDS-DMA path in a kStages-deep per-wave ring: one DMA instruction fetches four
// whole 256-byte key rows (1 KB contiguous per row group), and the 16-byte
// pieces are XOR-swizzled so that the MFMA operand reads (32 rows x one piece
// per half-wave) hit 16 distinct bank groups.  Waves never share LDS, so the
// only synchronisation is each wave's own vmcnt wait.
//
// Scores are not stored tile by tile: a wave keeps the scores of up to
// 2 * kScanScoreRegs tiles in registers (two tiles per register, one per lane
// half) and writes them when its row segment ends or the buffer is full.  For
// the usual share of a wave (under 80 tiles) that is one burst after its last
// key read.  Score writes mixed into the key stream slow it far more than their
// bytes (about 1.3 us per MB on MI355X, in 128-byte lines or 8 KiB bursts alike),
// while the same bytes written once reading is over cost a fraction of that.
#ifndef SA_SCAN_STAGES
#define SA_SCAN_STAGES 2
#endif
#ifndef SA_SCAN_WAVES
#define SA_SCAN_WAVES 8
#endif
constexpr int kScanStages = SA_SCAN_STAGES;       // tiles per wave ring (stages-1 in flight while one is scored)
constexpr int kScanWavesPerBlock = SA_SCAN_WAVES;
constexpr int kScanScoreRegs = 40;                // score buffer registers per lane (80 tiles)

// s_waitcnt vmcnt(n) that also fences the compiler: LDS written by the DMA path
// is not tracked by the compiler's own wait insertion.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their maxima)
constexpr int kWaitVmcnt0 = 0x0F70;

// Wait until the copies of the j-th tile of a segment have landed (see the ring
// comment in the kernel): the copies of the kScanStages - 1 tiles ahead are
// younger.  Stores (score bursts, tile ranges) issued since only lengthen it.
template <int DMA>
__device__ __forceinline__ void scan_wait()
{
    constexpr int S1 = kScanStages - 1;
    static_assert(S1 * DMA < 64, "vmcnt range");
    wait_vmcnt<S1 * DMA>();
}

// BLOCK_TILE: every cache block holds a whole number of 32-key tiles (block_size
// >= 32), so a tile's 32 rows are contiguous and its block id is one scalar load.
template <int IDX_DIM, int IDX_TILES, bool BLOCK_TILE>
__global__ __launch_bounds__(64 * kScanWavesPerBlock) void idx_score_decode_kernel(
    const uint16_t *__restrict__ idx_k, const int32_t *__restrict__ block_table, int max_blocks,
    int bs_log2, const int32_t *__restrict__ ctx_lens, int batch, const uint16_t *__restrict__ idx_q,
    const float *__restrict__ idx_w, int idx_heads, int relu, float *__restrict__ scores,
    int64_t score_stride, f32x2 *__restrict__ tile_mm, int64_t mm_stride)
{
    constexpr int KS = IDX_DIM / 16;            // MFMA steps per key row
    constexpr int PIECES = IDX_DIM / 8;         // 16-byte pieces per key row
    constexpr int TILE = 32 * IDX_DIM * 2;      // bytes per 32-key tile
    constexpr int DMA = TILE / 1024;            // DMA instructions per tile
    static_assert(PIECES == 16 || PIECES == 4, "key row of 256 or 64 bytes");
    constexpr int SW = PIECES - 1;              // swizzle mask
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kScanWavesPerBlock][kScanStages][TILE];
    __shared__ __attribute__((aligned(16))) float wlds[kScanWavesPerBlock][32 * IDX_TILES];

    // wave index made visibly wave-uniform so cursors live in scalar registers and
    // context lengths / block-table entries are scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int bmask = (1 << bs_log2) - 1;
    uint8_t *my = &ring[wave][0][0];

    // this wave's share [t_begin, t_end) of all tiles of all rows
    int64_t total = 0;
    for (int b = 0; b < batch; ++b) total += (ctx_lens[b] + 31) >> 5;
    const int64_t G = (int64_t)gridDim.x * kScanWavesPerBlock;
    const int64_t g = (int64_t)blockIdx.x * kScanWavesPerBlock + wave;
    int64_t t_cur = total * g / G;
    const int64_t t_end = total * (g + 1) / G;
    if (t_cur >= t_end) return;
    int b = 0;
    int64_t row_first = 0;  // global index of row b's first tile
    for (;; ++b) {
        const int nt = (ctx_lens[b] + 31) >> 5;
        if (t_cur < row_first + nt) break;
        row_first += nt;
    }

    // the DMA lane map: instruction i, lane l writes slot 64i + l = PIECES*r + q, which
    // holds piece q ^ (r & SW) of the tile's key row r
    // (recomputed from an opaque lane id at every tile: a few ALU operations
    // instead of 2 * DMA registers held across the loop)
    auto dma_map = [&](int i, int &r, int &piece) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int slot = 64 * i + ln;
        r = slot / PIECES;
        piece = (slot % PIECES) ^ (r & SW);
    };
    // lane (key col, half) reads piece half*KS + ks of its row at step ks
    const int koff = col * PIECES * 16;
    const int kx = col & SW;

    bf16x8 qa[IDX_TILES][KS];

    // per-segment state, read by the helpers below
    int ctx = 0, nt = 0;
    const int32_t *tbl = block_table;
    // Physical row of a tile's first key (BLOCK_TILE).  The block-table entry is a
    // scalar load (constant address space, wave-uniform index): scalar loads are
    // counted by lgkmcnt, so waiting for one never drains the copies in flight,
    // and it is issued a tile before its copies need it.
    typedef const __attribute__((address_space(4))) int32_t *ctbl_t;
    auto tile_base = [&](int t) -> int64_t {
        if constexpr (BLOCK_TILE) {
            const int s0 = (t < nt - 1 ? t : nt - 1) * 32;
            const int bi = __builtin_amdgcn_readfirstlane(s0 >> bs_log2);
            const int blk = ((ctbl_t)(uintptr_t)tbl)[bi];
            return ((int64_t)blk << bs_log2) | (s0 & bmask);
        } else {
            return 0;
        }
    };
    // The copies of a tile.  With BLOCK_TILE its 32 rows are contiguous: one
    // buffer resource over them, buffer-form LDS-DMA (after the global form the
    // compiler would drain every LDS read in flight at each later wait on one).
    auto issue = [&](int t, int stage, int64_t base) {
        const int s0 = t * 32;
        [[maybe_unused]] __amdgpu_buffer_rsrc_t rs;
        if constexpr (BLOCK_TILE) rs = buffer_rsrc(idx_k + base * IDX_DIM, TILE);
#pragma unroll
        for (int i = 0; i < DMA; ++i) {
            int dr, dp;
            dma_map(i, dr, dp);
            int s = s0 + dr;
            s = s < ctx ? s : ctx - 1;  // rows past the context re-read the last key; never scored
            SA_LDS void *dst = (SA_LDS void *)(my + stage * TILE + i * 1024);
            if constexpr (BLOCK_TILE) {
                buf_dma16_to_lds_stream(rs, (s - s0) * (IDX_DIM * 2) + dp * 16, dst);
            } else {
                const int64_t row = ((int64_t)tbl[s >> bs_log2] << bs_log2) | (s & bmask);
                dma16_to_lds_stream(idx_k + row * IDX_DIM + dp * 8, dst);
            }
        }
    };

    // one row segment at a time: [t0, t1) tiles of row b
    while (t_cur < t_end) {
        ctx = ctx_lens[b];
        nt = (ctx + 31) >> 5;
        const int t0 = (int)(t_cur - row_first);
        const int64_t rem = t_end - row_first;
        const int t1 = rem < nt ? (int)rem : nt;
        tbl = block_table + (int64_t)b * max_blocks;
        float *out = scores + (int64_t)b * score_stride;

        // queries and head weights of row b (waits for everything in flight: once per segment)
#pragma unroll
        for (int t = 0; t < IDX_TILES; ++t) {
            const int head = 32 * t + col;
            const uint16_t *qp = idx_q + ((int64_t)b * idx_heads + head) * IDX_DIM + half * (IDX_DIM / 2);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[t][ks] = head < idx_heads ? as_bf16x8(load16(qp + 8 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
        }
        // head weights of row b into this wave's LDS slot (read back per tile:
        // held in registers they would cost 16 per head tile)
        for (int h = lane; h < 32 * IDX_TILES; h += 64) wlds[wave][h] = h < idx_heads ? idx_w[(int64_t)b * idx_heads + h] : 0.0f;
        // A wait the compiler sees: the tile loop below then finds the queries
        // and weights complete and adds no memory wait of its own (which, next
        // to the LDS-DMA copies, it could only make a full drain on every tile).
        __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

        // Ring waits.  Every tile issues DMA copies, counted by vmcnt, which
        // completes in issue order; at the wait for tile j the younger copies are
        // those of the kScanStages - 1 tiles ahead.
        const int n = t1 - t0;
        float mm_lo = 0.0f, mm_hi = 0.0f;  // lane i: range of the segment's pending tile with index = i mod 16
        // Score buffer: the m tiles scored since the last burst, segment tiles
        // jb .. jb + m - 1.  `cur` collects a pair (tile jb + 2p in lane half 0,
        // jb + 2p + 1 in half 1); a complete pair is pushed onto sbuf, newest at
        // the end (a shift by register moves: the indices stay compile-time).
        constexpr int NB = kScanScoreRegs;
        float sbuf[NB];
#pragma unroll
        for (int i = 0; i < NB; ++i) sbuf[i] = 0.0f;
        float cur = 0.0f;
        int m = 0, jb = 0;
        auto push = [&]() {
#pragma unroll
            for (int i = 0; i + 1 < NB; ++i) sbuf[i] = sbuf[i + 1];
            sbuf[NB - 1] = cur;
        };
        // One burst: pair p goes to tiles jb + 2p (+1), i.e. 256 contiguous
        // bytes per store; the upper half of an incomplete last pair is masked.
        auto flush = [&]() {
            if (m & 1) push();
            const int npairs = (m + 1) >> 1;
            float *o = out + (int64_t)(t0 + jb + half) * 32 + col;
#pragma unroll
            for (int k = 0; k < NB; ++k) {  // k-th newest pair
                const int pr = npairs - 1 - k;
                if (k < npairs && (half == 0 || 2 * pr + 1 < m)) o[64 * pr] = sbuf[NB - 1 - k];
            }
            jb += m;
            m = 0;
        };
#pragma unroll
        for (int j = 0; j < kScanStages - 1; ++j)
            if (j < n) issue(t0 + j, j, tile_base(t0 + j));
        int64_t base_next = tile_base(t0 + kScanStages - 1);
        for (int j = 0; j < n; ++j) {
            const int stage = j % kScanStages;
            if (j + kScanStages - 1 < n) {
                issue(t0 + j + kScanStages - 1, (j + kScanStages - 1) % kScanStages, base_next);
                base_next = tile_base(t0 + j + kScanStages);
                scan_wait<DMA>();
            } else {
                wait_vmcnt<0>();
            }
            const uint8_t *tb = my + stage * TILE;
            // all B operands of the tile first, so the LDS reads overlap each other
            bf16x8 kb[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kb[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + koff + (((half * KS + ks) ^ kx) * 16)));
            // two accumulators per head tile (even / odd steps) halve the dependent MFMA chain
            f32x16 acc[IDX_TILES][2];
#pragma unroll
            for (int t = 0; t < IDX_TILES; ++t) acc[t][0] = acc[t][1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < IDX_TILES; ++t) acc[t][ks & 1] = mfma_32x32x16(qa[t][ks], kb[ks], acc[t][ks & 1]);
            float part[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            // head weights from LDS (an opaque lane id keeps these reads inside
            // the loop instead of 16 registers per head tile)
            int wl = lane;
            asm volatile("" : "+v"(wl));
            const float *wrow = &wlds[wave][4 * (wl >> 5)];
            auto head_sum = [&](auto relu_on) {
#pragma unroll
                for (int t = 0; t < IDX_TILES; ++t)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 w4 = *reinterpret_cast<const f32x4 *>(wrow + 32 * t + 8 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float d = acc[t][0][4 * g + e] + acc[t][1][4 * g + e];
                            if constexpr (decltype(relu_on)::value) d = fmaxf(d, 0.0f);
                            part[e] = fmaf(w4[e], d, part[e]);
                        }
                    }
            };
            if (relu) head_sum(std::true_type{});  // (uniform branch, outside the element loop)
            else head_sum(std::false_type{});
            const float p = (part[0] + part[1]) + (part[2] + part[3]);
            const float tot = add_wave_halves(p);
            const int tt = t0 + j;
            const int s = tt * 32 + col;
            // This tile's scores into the buffer (slots at or past ctx get values
            // nothing reads; every slot lies inside the row's score stride, which
            // is rounded up from the largest context).
            cur = half == (m & 1) ? tot + 0.0f : cur;
            ++m;
            if (!(m & 1)) push();
            if (m == 2 * NB) flush();
            // The tile's score range, for the range-binned top-k histogram.  Lane
            // tt % 16 keeps it, and a group of 16 tiles is written as one whole
            // 128-byte line (partial lines only at segment ends) instead of one
            // 8-byte store per tile.
            const f32x2 mm = minmax32_uniform(tot + 0.0f, s < ctx);
            if (lane == (tt & 15)) {
                mm_lo = mm[0];
                mm_hi = mm[1];
            }
            if ((tt & 15) == 15 || j == n - 1) {
                const int g0 = tt & ~15, first = (g0 > t0 ? g0 : t0) - g0;
                if (lane >= first && lane <= (tt & 15))
                    tile_mm[(int64_t)b * mm_stride + g0 + lane] = f32x2{mm_lo, mm_hi};
            }
        }
        if (m) flush();
        t_cur = row_first + t1;
        row_first += nt;
        ++b;
        while (t_cur < t_end && ((ctx_lens[b] + 31) >> 5) == 0) ++b;  // skip empty rows
    }
}

// ----------------------------------------------------------------- prefill --
// One workgroup of 8 waves owns 16 consecutive query rows (2 per wave) and
// streams every key those rows can see, [0, last row's position], in tiles of
// 32 keys read by all 8 waves.  Key tiles come HBM/L2 -> LDS through the
// LDS-DMA path into a kPrefillRing-deep ring, in the decode scan's swizzled
// layout (one 1 KiB copy per wave per tile for 128-dim keys).  Each wave keeps
// both of its rows' indexer queries in registers, so every key tile feeds
// 2 rows x IDX_TILES x (IDX_DIM/16) MFMAs per wave.  Blocks run heaviest (last
// rows) first.
constexpr int kPrefillRowsPerBlock = 16;
constexpr int kPrefillRing = 4;

template <int IDX_DIM, int IDX_TILES, bool BLOCK_TILE>
__global__ __launch_bounds__(512) void idx_score_prefill_kernel(
    const uint16_t *__restrict__ idx_k, const int32_t *__restrict__ block_table, int bs_log2,
    const uint16_t *__restrict__ idx_q, const float *__restrict__ idx_w, int idx_heads, int relu,
    int pos0, int nrows, float *__restrict__ scores, int64_t score_stride, f32x2 *__restrict__ tile_mm,
    int64_t mm_stride)
{
    constexpr int KS = IDX_DIM / 16;
    constexpr int PIECES = IDX_DIM / 8;         // 16-byte pieces per key row
    constexpr int TILE = 32 * IDX_DIM * 2;      // bytes per 32-key tile
    constexpr int DMA = TILE / 1024;            // copies per tile, one per wave for DMA <= 8
    static_assert(DMA <= 8, "one copy per wave and tile");
    constexpr int SW = PIECES - 1;
    constexpr int HP = 32 * IDX_TILES;
    constexpr int R = kPrefillRing;
    __shared__ __attribute__((aligned(1024))) uint8_t ring[R][TILE];
    __shared__ __attribute__((aligned(16))) float wts[kPrefillRowsPerBlock][HP];

    const int g = gridDim.x - 1 - blockIdx.x;
    const int r0 = g * kPrefillRowsPerBlock;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int rows_here = min(kPrefillRowsPerBlock, nrows - r0);
    const int nkeys = pos0 + r0 + rows_here;  // keys visible to the block's last row
    const int bmask = (1 << bs_log2) - 1;
    const int ntiles = (nkeys + 31) / 32;

    // this wave's copy of every tile: slot 64*wave + lane = PIECES*r + q holds
    // piece q ^ (r & SW) of the tile's key row r
    const int dslot = 64 * wave + lane;
    const int dr = dslot / PIECES, dpiece = (dslot % PIECES) ^ (dr & SW);
    typedef const __attribute__((address_space(4))) int32_t *ctbl_t;
    auto issue = [&](int kt) {
        if (wave >= DMA) return;  // (wave-uniform)
        const int ktc = kt < ntiles ? kt : ntiles - 1;  // past the end: copy the last tile again
        const int s0 = ktc * 32;
        int s = s0 + dr;
        s = s < nkeys ? s : nkeys - 1;  // rows past the last visible key re-read it; never scored
        SA_LDS void *dst = opaque_lds((SA_LDS void *)&ring[kt % R][64 * wave * 16]);
        if constexpr (BLOCK_TILE) {  // the tile's rows are contiguous: one buffer resource (see the decode scan)
            const int bi = __builtin_amdgcn_readfirstlane(s0 >> bs_log2);
            const int64_t row0 = (((int64_t)((ctbl_t)(uintptr_t)block_table)[bi]) << bs_log2) + (s0 & bmask);
            buf_dma16_to_lds(buffer_rsrc(idx_k + row0 * IDX_DIM, TILE), (s - s0) * (IDX_DIM * 2) + dpiece * 16, dst);
        } else {
            const int64_t row = ((int64_t)block_table[s >> bs_log2] << bs_log2) | (s & bmask);
            dma16_to_lds(idx_k + row * IDX_DIM + dpiece * 8, dst);
        }
    };
    // the ring is issued first: its copies overlap the query loads below
#pragma unroll
    for (int j = 0; j < R - 1; ++j) issue(j);

    for (int e = threadIdx.x; e < kPrefillRowsPerBlock * HP; e += blockDim.x) {
        const int rr = e / HP, hj = e % HP;
        wts[rr][hj] = (rr < rows_here && hj < idx_heads) ? idx_w[(int64_t)(r0 + rr) * idx_heads + hj] : 0.0f;
    }
    bf16x8 qa[2][IDX_TILES][KS];
    int pos[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int r = 2 * wave + rr;
        pos[rr] = r < rows_here ? pos0 + r0 + r : -1;
#pragma unroll
        for (int t = 0; t < IDX_TILES; ++t) {
            const int head = 32 * t + col;
            const uint16_t *qp = idx_q + ((int64_t)(r0 + r) * idx_heads + head) * IDX_DIM + half * (IDX_DIM / 2);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[rr][t][ks] = (r < rows_here && head < idx_heads) ? as_bf16x8(load16(qp + 8 * ks))
                                                                    : as_bf16x8(u32x4{0, 0, 0, 0});
        }
    }
    const int koff = col * PIECES * 16, kx = col & SW;
    float rlo[2] = {INFINITY, INFINITY}, rhi[2] = {-INFINITY, -INFINITY};

    // Ring: tile kt's copies were issued R-1 iterations earlier, and every later
    // iteration issued exactly one more copy per copying wave (tiles past the end
    // repeat the last one), so at the wait for tile kt at least R-2 younger copies
    // are in flight; copies complete in order, and the younger score stores only
    // lengthen the wait.  The barrier then makes every wave's copy of tile kt
    // visible and frees tile kt-1's buffer for tile kt+R-1.
    for (int kt = 0; kt < ntiles; ++kt) {
        wait_vmcnt<R - 2>();
        barrier_no_fence();
        issue(kt + R - 1);
        const int s0 = kt * 32;
        if (s0 > pos[0] && s0 > pos[1]) continue;  // (wave-uniform) both rows end before this tile
        const uint8_t *tb = &ring[kt % R][0];
        // all K operands of the tile first (their LDS reads overlap), then per row:
        // its MFMAs, then its head reduction, so that one wave's reduction runs
        // beside the other wave's MFMAs on the same SIMD
        bf16x8 kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kb[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + koff + (((half * KS + ks) ^ kx) * 16)));
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            if (s0 > pos[rr]) continue;  // wave-uniform
            f32x16 acc[IDX_TILES];
#pragma unroll
            for (int t = 0; t < IDX_TILES; ++t) acc[t] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < IDX_TILES; ++t) acc[t] = mfma_32x32x16(qa[rr][t][ks], kb[ks], acc[t]);
            const int lr = 2 * wave + rr;
            float part = 0.0f;
            auto head_sum = [&](auto relu_on) {
#pragma unroll
                for (int t = 0; t < IDX_TILES; ++t)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&wts[lr][32 * t + 8 * q4 + 4 * half]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float d = acc[t][4 * q4 + e];
                            if constexpr (decltype(relu_on)::value) d = fmaxf(d, 0.0f);
                            part = fmaf(w4[e], d, part);
                        }
                    }
            };
            if (relu) head_sum(std::true_type{});  // (uniform branch, outside the element loop)
            else head_sum(std::false_type{});
            const float tot = add_wave_halves(part);
            const int s = s0 + col;
            if (half == 0 && s <= pos[rr]) scores[(int64_t)(r0 + lr) * score_stride + s] = tot + 0.0f;
            if (s <= pos[rr]) {  // lane-local running range of the row's scores
                rlo[rr] = fminf(rlo[rr], tot + 0.0f);
                rhi[rr] = fmaxf(rhi[rr], tot + 0.0f);
            }
        }
    }
    wait_vmcnt<0>();  // the last (repeated) copies have landed before the block ends
    // each row's score range, stored as the row's first tile entry (the prefill
    // top-k reads one range entry per row)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const f32x2 lohi = minmax32(rlo[rr], true), hilo = minmax32(rhi[rr], true);
        if (lane == 0 && pos[rr] >= 0) tile_mm[(int64_t)(r0 + 2 * wave + rr) * mm_stride] = f32x2{lohi[0], hilo[1]};
    }
}

}  // namespace sa
