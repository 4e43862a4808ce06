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
// tiles (row-major, each row's tiles in key order), grouped in pairs; block b
// of B takes the contiguous pairs [b*P/B, (b+1)*P/B), so every block moves the
// same number of bytes whatever the context lengths, and its waves claim those
// pairs one at a time (below).  Key tiles stream HBM -> LDS through the
// LDS-DMA path in a kStages-deep per-wave ring: one DMA instruction fetches four
// whole 256-byte key rows (1 KB contiguous per row group), and the 16-byte
// pieces are XOR-swizzled so that the MFMA operand reads (32 rows x one piece
// per half-wave) hit 16 distinct bank groups.  Waves never share LDS, so the
// only synchronisation is each wave's own vmcnt wait.
//
// Scores are not stored tile by tile: a wave keeps the scores of up to
// 2 * kScanScoreRegs tiles in registers (two tiles per register, one per lane
// half) and writes them when the buffer is full or its work is done.  For the
// usual share of a wave (under 80 tiles) that is one burst after its last key
// read.  Score writes mixed into the key stream slow it far more than their
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

// vmcnt(n) as an immediate for the compiler-visible s_waitcnt builtin
// (expcnt and lgkmcnt at their maxima)
__device__ __forceinline__ constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Work of the scan.  Each row's tiles are grouped in pairs (the last pair of a
// row with an odd tile count holds one tile); the pairs of all rows form one
// list, split evenly into one contiguous range per block, and the block's 8
// waves claim its pairs one at a time from a counter in LDS.  Waves do not
// move bytes at one rate: on MI355X waves of one XCD finished equal static
// shares about 10% apart (and whole XCDs up to 20% apart), so a static split
// per wave leaves the kernel waiting on its slowest waves.  Global atomics
// would balance across blocks too, but their returns join the memory counter
// that the ring waits on, and each claim then stalled the tile it followed
// (the scan ran 30% slower that way); LDS atomics stay off that counter.

// BLOCK_TILE: every cache block holds a whole number of 32-key tiles (block_size
// >= 32), so a tile's 32 rows are contiguous and its block id is one scalar load.
template <int IDX_DIM, int IDX_TILES, bool BLOCK_TILE>
__global__ __launch_bounds__(64 * kScanWavesPerBlock) void idx_score_decode_kernel(
    const uint16_t *__restrict__ idx_k, const int32_t *__restrict__ block_table, int max_blocks,
    int bs_log2, const int32_t *__restrict__ ctx_lens, int batch, const uint16_t *__restrict__ idx_q,
    const float *__restrict__ idx_w, int idx_heads, int relu, float *__restrict__ scores,
    int64_t score_stride, f32x2 *__restrict__ tile_mm, int64_t mm_stride, const AppendArgs ap)
{
    constexpr int KS = IDX_DIM / 16;            // MFMA steps per key row
    constexpr int PIECES = IDX_DIM / 8;         // 16-byte pieces per key row
    constexpr int TILE = 32 * IDX_DIM * 2;      // bytes per 32-key tile
    constexpr int DMA = TILE / 1024;            // DMA instructions per tile
    constexpr int NB = kScanScoreRegs;          // score buffer: pairs of tiles
    static_assert(PIECES == 16 || PIECES == 4, "key row of 256 or 64 bytes");
    static_assert(kScanStages == 2, "the tile stream below keeps one tile in flight while one is scored");
    constexpr int SW = PIECES - 1;              // swizzle mask
    __shared__ __attribute__((aligned(1024))) uint8_t ring[kScanWavesPerBlock][kScanStages][TILE];
    __shared__ __attribute__((aligned(16))) float wlds[kScanWavesPerBlock][32 * IDX_TILES];
    // per buffered pair: its row, first tile (+ 1 << 30 when it holds one tile)
    // and the two tiles' score ranges
    __shared__ int2 pair_dst[kScanWavesPerBlock][NB];
    __shared__ f32x4 pair_mm[kScanWavesPerBlock][NB];

    // wave index made visibly wave-uniform so cursors live in scalar registers and
    // context lengths / block-table entries are scalar loads
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int bmask = (1 << bs_log2) - 1;
    uint8_t *my = &ring[wave][0][0];

    // ---- the pair list and this block's claims ----
    auto row_pairs = [&](int b) { return (((ctx_lens[b] + 31) >> 5) + 1) >> 1; };
    int64_t total_pairs = 0;
    for (int b = 0; b < batch; ++b) total_pairs += row_pairs(b);
    const int nblk = gridDim.x;
    auto range_lo = [&](int blk) { return total_pairs * blk / nblk; };
    int rb = 0;              // row cursor: row rb's first pair is list index rfirst
    int64_t rfirst = 0;
    auto locate = [&](int64_t p) {
        if (p < rfirst) {
            rb = 0;
            rfirst = 0;
        }
        for (;;) {  // (rows without keys are stepped over)
            const int np = row_pairs(rb);
            if (p < rfirst + np) break;
            rfirst += np;
            ++rb;
        }
    };
    __shared__ int blk_claims;
    if (threadIdx.x == 0) blk_claims = 0;
    __syncthreads();
    const int64_t my_lo = range_lo(blockIdx.x), my_hi = range_lo(blockIdx.x + 1);
    int claim = 0;  // lane 0: this wave's pending claim
    if (lane == 0) claim = atomicAdd(&blk_claims, 1);
    // The next pair of this wave: (row, first tile, tiles 1 or 2); false when
    // the block's range is used up.  Using a claim sets need_claim: the main
    // loop requests the next one after its ring wait, well before its use.
    bool need_claim = false;
    auto next_pair = [&](int &pb, int &pt, int &pn) -> bool {
        if (need_claim) {  // (a one-tile pair right after the last claim: request it now)
            if (lane == 0) claim = atomicAdd(&blk_claims, 1);
            need_claim = false;
        }
        const int64_t p = my_lo + __builtin_amdgcn_readfirstlane(claim);
        if (p >= my_hi) return false;
        need_claim = true;
        locate(p);
        const int nt = (ctx_lens[rb] + 31) >> 5;
        pb = rb;
        pt = 2 * (int)(p - rfirst);
        pn = pt + 1 < nt ? 2 : 1;
        return true;
    };
    int pr_b = 0, pr_t = 0, pr_n = 0, pr_i = 0;  // current pair and the next tile index within it
    auto next_tile = [&](int &b_out, int &t_out) -> bool {
        if (pr_i >= pr_n) {
            if (!next_pair(pr_b, pr_t, pr_n)) return false;
            pr_i = 0;
        }
        b_out = pr_b;
        t_out = pr_t + pr_i;
        ++pr_i;
        return true;
    };

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

    // Physical row of a tile's first key (BLOCK_TILE).  The block-table entry is a
    // scalar load (constant address space, wave-uniform index): scalar loads are
    // counted by lgkmcnt, so waiting for one never drains the copies in flight,
    // and it is issued a tile before its copies need it.
    typedef const __attribute__((address_space(4))) int32_t *ctbl_t;
    auto tile_base = [&](int b, int t) -> int64_t {
        if constexpr (BLOCK_TILE) {
            const int s0 = t * 32;
            const int bi = __builtin_amdgcn_readfirstlane(s0 >> bs_log2);
            const int blk = ((ctbl_t)(uintptr_t)(block_table + (int64_t)b * max_blocks))[bi];
            return ((int64_t)blk << bs_log2) | (s0 & bmask);
        } else {
            return 0;
        }
    };
    // The copies of tile t of row b.  With BLOCK_TILE its 32 rows are contiguous:
    // one buffer resource over them, buffer-form LDS-DMA (after the global form
    // the compiler would drain every LDS read in flight at each later wait on one).
    auto issue = [&](int b, int t, int stage, int64_t base) {
        const int ctx = ctx_lens[b];
        const int32_t *tbl = block_table + (int64_t)b * max_blocks;
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

    bf16x8 qa[IDX_TILES][KS];
    int loaded_b = -1;  // row whose queries and weights are in qa / wlds

    // Score buffer: one register per pair of tiles (first tile in lane half 0,
    // second in half 1), the newest at the end (a shift by register moves: the
    // indices stay compile-time); the m-th pair pushed since the last burst has
    // its destination and score ranges in pair_dst / pair_mm[wave][m].
    float sbuf[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) sbuf[i] = 0.0f;
    float cur = 0.0f;
    f32x4 cur_mm = f32x4{};
    int m = 0;
    auto push = [&](int b, int t0, int n) {
#pragma unroll
        for (int i = 0; i + 1 < NB; ++i) sbuf[i] = sbuf[i + 1];
        sbuf[NB - 1] = cur;
        if (lane == 0) {
            pair_dst[wave][m] = int2{b, t0 | (n == 1 ? (1 << 30) : 0)};
            pair_mm[wave][m] = cur_mm;
        }
        ++m;
    };
    // One burst: each pair's scores as one 256-byte store (half 1 masked for a
    // one-tile pair) and its score ranges as one 16-byte store.
    auto flush = [&]() {
#pragma unroll
        for (int k = 0; k < NB; ++k) {  // k-th newest pair
            if (k < m) {
                const int2 dst = pair_dst[wave][m - 1 - k];
                const bool one = (dst.y >> 30) & 1;
                const int t0 = dst.y & ((1 << 30) - 1);
                if (half == 0 || !one) scores[(int64_t)dst.x * score_stride + (int64_t)(t0 + half) * 32 + col] = sbuf[NB - 1 - k];
                if (lane == 0) {
                    const f32x4 mmv = pair_mm[wave][m - 1 - k];
                    f32x2 *mo = tile_mm + (int64_t)dst.x * mm_stride + t0;
                    mo[0] = f32x2{mmv[0], mmv[1]};
                    if (!one) mo[1] = f32x2{mmv[2], mmv[3]};
                }
            }
        }
        m = 0;
    };

    // Ring.  Per iteration: the next tile's copies are issued into the other
    // stage, the tile after it is found (its block-table entry loads
    // meanwhile), the wave waits for the current tile (younger: the next
    // tile's copies; stores issued since only lengthen the wait) and scores it.
    int a_b, a_t;
    if (!next_tile(a_b, a_t)) return;
    int a_n = pr_n, a_first = pr_t;  // the pair of tile a
    issue(a_b, a_t, 0, tile_base(a_b, a_t));
    int c_b = 0, c_t = 0;
    bool have_c = next_tile(c_b, c_t);
    int c_n = pr_n, c_first = pr_t;
    int64_t c_base = have_c ? tile_base(c_b, c_t) : 0;
    int stage = 0;
    for (;;) {
        const bool have_n = have_c;
        const int n_b = c_b, n_t = c_t, n_n = c_n, n_first = c_first;
        if (have_n) {
            issue(n_b, n_t, stage ^ 1, c_base);
            have_c = next_tile(c_b, c_t);
            c_n = pr_n;
            c_first = pr_t;
            if (have_c) c_base = tile_base(c_b, c_t);
        }
        // Row change: this row's queries and weights (a wait the compiler
        // sees: the loop then finds them complete and adds no memory wait of
        // its own, which next to the LDS-DMA copies it could only make a full
        // drain on every tile).
        if (a_b != loaded_b) {
#pragma unroll
            for (int t = 0; t < IDX_TILES; ++t) {
                const int head = 32 * t + col;
                const uint16_t *qp = idx_q + ((int64_t)a_b * idx_heads + head) * IDX_DIM + half * (IDX_DIM / 2);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    qa[t][ks] = head < idx_heads ? as_bf16x8(load16(qp + 8 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
            }
            // head weights into this wave's LDS slot (read back per tile: held in
            // registers they would cost 16 per head tile)
            for (int h = lane; h < 32 * IDX_TILES; h += 64)
                wlds[wave][h] = h < idx_heads ? idx_w[(int64_t)a_b * idx_heads + h] : 0.0f;
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
            loaded_b = a_b;
        }
        // (visible to the compiler, so that it knows the claims requested
        // before these copies have arrived; the fence keeps the tile reads below)
        if (have_n) __builtin_amdgcn_s_waitcnt(waitcnt_vm(DMA));
        else __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        asm volatile("" ::: "memory");
        if (need_claim) {
            if (lane == 0) claim = atomicAdd(&blk_claims, 1);
            need_claim = false;
        }

        const int ctx = ctx_lens[a_b];
        // Appending: the row's current token is scored with its new key (the
        // top-k kernel that follows writes it into the cache), so the landed
        // tile holding position ctx - 1 gets that key in its LDS image.
        if (ap.new_kv && ((ctx - 1) >> 5) == a_t) {  // (wave-uniform)
            const int rr = (ctx - 1) & 31;
            if (lane < PIECES)
                *reinterpret_cast<u32x4 *>(my + stage * TILE + 16 * (PIECES * rr + (lane ^ (rr & SW)))) =
                    load16(ap.new_idx_k + (int64_t)a_b * IDX_DIM + 8 * lane);
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
                for (int gq = 0; gq < 4; ++gq) {
                    const f32x4 w4 = *reinterpret_cast<const f32x4 *>(wrow + 32 * t + 8 * gq);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float d = acc[t][0][4 * gq + e] + acc[t][1][4 * gq + e];
                        if constexpr (decltype(relu_on)::value) d = fmaxf(d, 0.0f);
                        part[e] = fmaf(w4[e], d, part[e]);
                    }
                }
        };
        if (relu) head_sum(std::true_type{});  // (uniform branch, outside the element loop)
        else head_sum(std::false_type{});
        const float p = (part[0] + part[1]) + (part[2] + part[3]);
        const float tot = add_wave_halves(p);
        // The tile's scores and its score range (for the range-binned top-k
        // histogram) into the buffer.  Slots at or past ctx get values nothing
        // reads; every slot lies inside the row's score stride, which is
        // rounded up from the largest context.
        const int second = a_t - a_first;  // 0 or 1 within its pair
        const f32x2 mmt = minmax32_uniform(tot + 0.0f, a_t * 32 + col < ctx);
        cur = half == second ? tot + 0.0f : cur;
        if (second == 0) {
            cur_mm[0] = mmt[0];
            cur_mm[1] = mmt[1];
        } else {
            cur_mm[2] = mmt[0];
            cur_mm[3] = mmt[1];
        }
        if (second + 1 == a_n) {  // the pair is complete
            push(a_b, a_first, a_n);
            if (m == NB) flush();
        }
        if (!have_n) break;
        a_b = n_b;
        a_t = n_t;
        a_n = n_n;
        a_first = n_first;
        stage ^= 1;
    }
    if (m) flush();
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
    const uint16_t *__restrict__ idx_k, const int32_t *__restrict__ block_table, int bt_stride, int bs_log2,
    const uint16_t *__restrict__ idx_q, const float *__restrict__ idx_w, int idx_heads, int relu,
    const SeqMap blocks_map, float *__restrict__ scores, int64_t score_stride, f32x2 *__restrict__ tile_mm,
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

    // 16-row block g of piece pc (the pieces are listed shortest context first
    // and the blocks run from the last one, so the longest rows start first)
    const int g = gridDim.x - 1 - blockIdx.x;
    const int pc = map_piece(blocks_map, g);
    const int r0 = (g - blocks_map.first[pc]) * kPrefillRowsPerBlock;  // first row within the piece
    const int prow = blocks_map.row0[pc] + r0;                           // ... within the launch's rows
    const int p0 = blocks_map.pos0[pc] + r0;                             // ... its position
    block_table += (int64_t)blocks_map.bt_row[pc] * bt_stride;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int rows_here = min(kPrefillRowsPerBlock, blocks_map.nrows[pc] - r0);
    const int nkeys = p0 + rows_here;  // keys visible to the block's last row
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
        wts[rr][hj] = (rr < rows_here && hj < idx_heads) ? idx_w[(int64_t)(prow + rr) * idx_heads + hj] : 0.0f;
    }
    bf16x8 qa[2][IDX_TILES][KS];
    int pos[2];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int r = 2 * wave + rr;
        pos[rr] = r < rows_here ? p0 + r : -1;
#pragma unroll
        for (int t = 0; t < IDX_TILES; ++t) {
            const int head = 32 * t + col;
            const uint16_t *qp = idx_q + ((int64_t)(prow + r) * idx_heads + head) * IDX_DIM + half * (IDX_DIM / 2);
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
            if (half == 0 && s <= pos[rr]) scores[(int64_t)(prow + lr) * score_stride + s] = tot + 0.0f;
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
        if (lane == 0 && pos[rr] >= 0) tile_mm[(int64_t)(prow + 2 * wave + rr) * mm_stride] = f32x2{lohi[0], hilo[1]};
    }
}

}  // namespace sa
