// Sparse softmax attention over the kept keys of a paged latent cache (gfx950).
//
// For a query row r and head h:  l_s = scale * q[h] . latent[s][0:QK],
// o[h] = sum_s softmax(l)_s * latent[s][0:V] over the kept positions s.  The
// pages' operator takes queries, the cache and the index list and returns the
// aggregated context ("Day-0 Model Adaptation Depends on the Compute Software
// Stack", Operator Library Abstraction; "Day-0 Adaptation: Running
// Trillion-Parameter Models on Domestic AI Accelerators", section 3.1); the
// tile skeleton on "Day-0 Adaptation for LLMs: Implementing Sparse Attention
// and Low-Precision Weights" (section II) gathers the indexed KV tiles and
// reduces them with a softmax, which is done here tile by tile with an online
// softmax.  Decode splits the kept set across workgroups and merges the
// partial results with their log-sum-exp weights ("Engineering Practices for
// Day-0 Adaptation of Million-Token Context Models on Domestic AI Chips", Four
// Key Layers item 3: partial scores per KV block, then a cross-block reduction);
// the next tile's gather is in flight while the current one is computed (same
// item: prefetch of the next KV block during attention).
//
// gfx950 mapping.  One workgroup = one (row, split, head group of 32 * HB
// heads): 2 * HB waves, two per 32-head block.  The two waves of a head block
// ("partners" x = 0, 1) split both contractions: for q.k, partner x holds the
// query of its 32 heads over half of the QK dims (QK = 576: 72 registers) and
// computes a partial S^T over that half; for P.V it owns half of the V value
// columns (V = 512: 32 x 256 fp32 accumulators, 128 registers).  The partners
// add their partial S^T through LDS (the main rows of a spent tile buffer), so
// no logit is computed twice.  With 128 heads, HB = 2: two workgroups of 4 waves
// per (row, split), one wave per SIMD (the tile ring takes 158 KB of LDS).  Per
// tile of 32 kept tokens:
//   * the 32 latent rows are copied HBM -> LDS by buffer-form LDS-DMA, one
//     resource per token row and a 64-lane copy of its first 1 KiB; the 128-byte
//     rope tails go with each token's copy (an 8-lane copy) for tiles copied
//     whole, and in the tile loop as one 64-lane vector load per eight tokens,
//     stored into LDS a tile later; the main rows' and the tails' 16-byte pieces
//     are XOR-swizzled by token (through the per-lane source offsets) so that
//     MFMA operand reads do not collide on LDS banks; a ring of 4 tile buffers
//     keeps two tiles' copies in flight while one tile's values and the next
//     tile's keys are read, and the copies of tile t + 3 are issued between the
//     q.k MFMAs of tile t + 1, beside the softmax of tile t;
//   * partial S^T[token][head] = K . Q^T on 32x32x16 bf16 MFMAs (K from LDS,
//     Q^T from registers, contraction over the partner's QK half in 16-wide
//     steps), exchanged through LDS and summed;
//   * softmax in base 2 in fp32 against a per-head reference max taken from
//     the first tile with a valid token; it never moves, so the output
//     accumulators are touched only by MFMAs (a split whose weights reach 2^64,
//     its logits outgrowing the reference, is recomputed exactly with its true
//     max);
//   * the S^T accumulator already has the register layout of the B operand of
//     O^T[v][head] += V^T[v][token] . P^T[token][head]: P is only rounded to bf16.
//     Rows that keep fewer than kPreciseBelow keys carry P as a pair of bf16
//     values (hi + lo, two MFMAs), so the weights are exact to about 2^-16; the
//     softmax denominator sums exactly the weights the MFMAs multiply.
//     The V^T operand comes straight from the token-major tile through
//     transposed LDS reads (ds_read_b64_tr_b16), four tokens per read.
#pragma once

#include "device_common.hpp"

namespace sa {

constexpr int kAttnMaxSplitTokens = 2048;
constexpr uint32_t kNoRow = 0xFFFFFFFFu;
// Rows keeping fewer keys than this multiply V by P as a hi/lo pair of bf16
// values.  A row's output error from rounding P to bf16 alone is about
// 2^-9 / sqrt(effective keys) of its values, which for rows of a few keys is
// several percent of the output RMS of a batch of longer rows.
constexpr int kPreciseBelow = 2048;

struct AttnArgs {
    const uint16_t *q;           // [rows][H][QK]
    const uint16_t *kv;          // [num_blocks][bs][QK]
    const int32_t *block_table;  // [seqs][max_blocks]
    const int32_t *topk_idx;     // [rows][k]
    const int32_t *ctx_lens;     // decode: [rows]
    float *part_o;               // splits > 1: [rows][splits][H][V]
    float *part_ml;              // splits > 1: [rows][splits][H][4]  (max in log2 units, rounded sum, exact sum, 0)
    void *out;                   // splits == 1: [rows][H][V]
    float *lse;                  // splits == 1, nullable: [rows][H]
    int64_t num_blocks;
    int num_heads, max_blocks, bs_log2, k;
    int decode;                  // 1: row r = sequence r, limit ctx_lens[r]; 0: prefill rows of the pieces in rows_map
    SeqMap rows_map;             // prefill: row r's sequence and position (limit = position + 1)
    int tokens_per_split, splits, out_bf16;
    float scale_log2;            // softmax_scale * log2(e)
    int partners;                // (host side) partner waves per head block: 2 or 4
};

#ifndef SA_ATTN_KPF
#define SA_ATTN_KPF 4  // K operand steps read ahead of their MFMA
#endif
#ifndef SA_ATTN_VPF
#define SA_ATTN_VPF 3  // V operand steps read ahead of their MFMAs
#endif

constexpr int kAttnBuffers = 4;  // tile ring: two tiles in flight while two are read

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int QK, int V, int NP>
struct AttnShape {
    static constexpr int KS = QK / 16;                   // MFMA steps of q.k
    static constexpr int KP = KS / NP;                   // steps per partner
    static constexpr int VW = V / NP;                    // value columns per partner
    static constexpr int NVT = VW / 32;                  // 32-column output tiles per wave
    static constexpr int PIECES = QK / 8;                // 16-byte pieces per latent row
    // LDS image of a 32-token tile.  Main rows: pieces 0..63 of each token
    // (one 1 KiB copy per token), MAIN_STRIDE bytes apart, piece p of token t
    // stored at position p ^ main_swizzle(t).  Tail: the remaining 8 pieces
    // (128 bytes) of each token.  Behind main rows the tail rows are packed
    // (32 x 128 bytes, so eight tokens' tails are one contiguous kilobyte) with
    // piece p of token t at position p ^ (t & 7); rows shorter than 64 pieces
    // live in the tail only, TAIL_STRIDE = 144 bytes apart, unswizzled (the
    // extra 16 bytes move consecutive tokens to different 16-byte bank groups).
    // Either way the 16 tokens of a K operand read touch 16 distinct bank
    // groups.
    static constexpr int MAIN = PIECES >= 64 ? 64 : 0;
    static constexpr int TAIL = PIECES - MAIN;
    static constexpr int MAIN_STRIDE = MAIN * 16;
    static constexpr bool TSWZ = MAIN > 0;
    static constexpr int TAIL_STRIDE = TSWZ ? TAIL * 16 : TAIL * 16 + 16;
    // position of tail piece p of tile token t (an involution in p)
    static __device__ __forceinline__ constexpr int tail_pos(int p, int t) { return TSWZ ? p ^ (t & 7) : p; }
    static constexpr int TAIL_BASE = 32 * MAIN_STRIDE;
    static constexpr int TILE_BYTES = TAIL_BASE + 32 * TAIL_STRIDE;
    static constexpr int COPIES_PER_TOKEN = (MAIN ? 1 : 0) + 1;  // main row, tail
    static_assert(KS % NP == 0 && V % (32 * NP) == 0 && V <= QK, "shape family");
    static_assert(TAIL == 8, "the tail is one 8-lane copy of 128 bytes");
    static_assert(V <= 8 * (MAIN ? MAIN : TAIL), "value columns must lie in one row region");
};

// Position swizzle of the main rows: piece p of tile token t sits at position
// p ^ main_swizzle(t) (the low two bit pairs of t, exchanged).  Then a K
// operand read (16 tokens, one piece each) and a transposed V read (4 tokens x
// 4 consecutive pieces per 32 lanes) both touch 16 distinct 16-byte bank groups.
__device__ __forceinline__ constexpr int main_swizzle(int t) { return 4 * (t & 3) + ((t >> 2) & 3); }

// Row rho of a tile's S^T accumulator holds tile token row_token(rho) (bits 2
// and 3 swapped).  Then the two half-waves of a V^T operand read tokens 8
// apart, whose main rows sit 32 banks apart, while the K operand of 16
// consecutive rows still covers 16 distinct 16-byte bank groups.
__device__ __forceinline__ constexpr int row_token(int rho) { return (rho & ~12) | ((rho & 4) << 1) | ((rho & 8) >> 1); }

// Source of the copies of padding tokens: zeros, so that V of a slot that is
// weighted by P = 0 is finite.
__device__ __attribute__((aligned(16))) const uint8_t kZeroLatentRow[2048] = {};

__device__ __forceinline__ uint32_t lane_read(uint32_t v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
// l + the two bf16 values packed in w (each times 1.0)
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float l)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), __builtin_bit_cast(b2, 0x3F803F80u), l, false);
}


// Workgroup id -> logical block.  Workgroups are dealt to the 8 XCDs in turn
// (id mod 8); this map gives each XCD a contiguous range of logical blocks, so
// the blocks of one query row (its splits), which read the same query, share
// one L2.
__device__ __forceinline__ int xcd_block(int id, int n)
{
    const int q = n >> 3, rem = n & 7, x = id & 7;
    return x * q + min(x, rem) + (id >> 3);
}

// Compile-time choices of one wave's tile loop: its partner index and whether
// P goes to the MFMAs as a hi/lo pair.
template <int PX_, bool PREC_>
struct TileCfg {
    static constexpr int PX = PX_;
    static constexpr bool PREC = PREC_;
};

// 2 * HB waves per workgroup: wave w is partner x = w / HB of head block
// hb = w % HB.  A workgroup covers the 32 * HB heads of one head group; the
// one-dimensional grid has rows * splits * head groups workgroups.
template <int QK, int V, int HB>
__global__ __launch_bounds__(128 * HB, 1) void attend_kernel(const AttnArgs a)
{
    using S = AttnShape<QK, V, 2>;
    constexpr int KP = S::KP, VW = S::VW, NVT = S::NVT;
    constexpr int NW = 2 * HB, nthreads = 64 * NW;
    constexpr int NB = kAttnBuffers;
    static_assert(32 % NW == 0, "tokens per wave");
    constexpr int TOK_W = 32 / NW;  // tokens each wave copies per tile
    // The partners' partial S^T pass through the main rows of a spent tile
    // buffer (the rows the reading wave itself refills next), or through an
    // array of their own for rows without main rows.
    constexpr bool XIN = S::MAIN > 0 && TOK_W >= 4;
    constexpr int XN = XIN ? 1 : NW, XJ = XIN ? 1 : 4, XL = XIN ? 1 : 64;
    __shared__ __attribute__((aligned(1024))) uint8_t tile[NB][S::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) f32x4 xchs[XN][XJ][XL];
    __shared__ uint32_t rows[kAttnMaxSplitTokens];
    __shared__ uint32_t vbits[kAttnMaxSplitTokens / 32];
    __shared__ int first_tile, last_tile, overflow_flag;

    // the head groups of one (row, split) are consecutive logical blocks: they
    // gather the same latent rows, through one L2
    const int hgroups = (a.num_heads + 32 * HB - 1) / (32 * HB);
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int r = lb / (a.splits * hgroups), split = (lb / hgroups) % a.splits, hg = lb % hgroups;
    const int wave = wave_uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    __builtin_assume(wave >= 0 && wave < NW);  // lets copy kinds resolve at compile time
    const int hb = wave % HB, px = wave / HB;   // head block, partner index
    const int partner = px == 0 ? wave + HB : wave - HB;
    const int col = lane & 31, half = lane >> 5;
    int seq, limit;
    if (a.decode) {
        seq = r;
        limit = a.ctx_lens[r];
    } else {
        const int pc = map_piece(a.rows_map, r);
        seq = a.rows_map.bt_row[pc];
        limit = a.rows_map.pos0[pc] + (r - a.rows_map.row0[pc]) + 1;
    }
    const int j0 = split * a.tokens_per_split;
    const int cnt = max(0, min(a.tokens_per_split, a.k - j0));
    const int ntiles = (cnt + 31) / 32;
    const int32_t *sel = a.topk_idx + (int64_t)r * a.k + j0;
    const int32_t *tbl = a.block_table + (int64_t)seq * a.max_blocks;
    const int bmask = (1 << a.bs_log2) - 1;
    // block-uniform: the row keeps few keys, so P goes to the MFMAs as hi + lo
    const bool precise = min(limit, a.k) < kPreciseBelow;

    const int head = 32 * (HB * hg + hb) + col;
    const bool hok = head < a.num_heads;
    // Physical row of every kept token of this split (kNoRow = padding) and a
    // validity mask per 32-token tile.  Positions, then block-table entries, are
    // loaded 8 per thread at a time, so the look-ups cost two memory round trips.
    // The first round's positions are loaded before the queries below: memory
    // loads complete in issue order, so waiting for positions issued after the
    // queries would also wait for the queries (73 KB per workgroup), while this
    // way the queries arrive during the block-table round trip.
    auto load_positions = [&](int jb, int (&idx)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = jb + u * nthreads + threadIdx.x;
            idx[u] = j < cnt ? sel[j] : -1;
        }
    };
    auto look_up = [&](int jb, const int (&idx)[8]) {
        int blk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const bool ok = idx[u] >= 0 && idx[u] < limit;
            blk[u] = ok ? tbl[idx[u] >> a.bs_log2] : -1;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = jb + u * nthreads + threadIdx.x;
            const bool ok = blk[u] >= 0 && blk[u] < a.num_blocks;
            const uint32_t row = ok ? ((uint32_t)blk[u] << a.bs_log2) | (uint32_t)(idx[u] & bmask) : kNoRow;
            const uint64_t m = __ballot(row != kNoRow);
            if (j < ntiles * 32) rows[j] = row;
            const int w0 = (j - lane) >> 5;  // this wave's 64 tokens are tiles w0, w0 + 1
            if (lane == 0 && w0 < ntiles) vbits[w0] = (uint32_t)m;
            if (lane == 32 && w0 + 1 < ntiles) vbits[w0 + 1] = (uint32_t)(m >> 32);
        }
    };
    int idx0[8];
    load_positions(0, idx0);

    // q^T operand of step ks (of this partner's half) for this lane:
    // q[head][16(KP px + ks) + 8half .. +7].  Lanes of heads past num_heads load
    // the last head instead: their S^T columns feed only their own, never
    // stored, output columns.
    bf16x8 qb[KP];
    {
        const int qhead = hok ? head : a.num_heads - 1;
        const uint16_t *qp = a.q + ((int64_t)r * a.num_heads + qhead) * QK + 16 * KP * px + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) qb[ks] = as_bf16x8(load16(qp + 16 * ks));
    }

    if (ntiles > 0) look_up(0, idx0);  // (block-uniform)
    for (int jb = 8 * nthreads; jb < ntiles * 32; jb += 8 * nthreads) {  // (splits of more than 8 tokens per thread)
        int idx[8];
        load_positions(jb, idx);
        look_up(jb, idx);
    }
    if (threadIdx.x == 0) {
        first_tile = kAttnMaxSplitTokens;
        last_tile = -1;
        overflow_flag = 0;
    }
    f32x16 oacc[NVT];  // O^T tile vt: columns 32vt.. of this partner's value range
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) oacc[vt] = f32x16{};
    // m: reference max (log2 units); l: sum of the weights the MFMAs multiply
    // (output normaliser); le: sum of the unrounded weights (log-sum-exp)
    float m = -INFINITY, l = 0.0f, le = 0.0f;
    __syncthreads();
    for (int t = threadIdx.x; t < ntiles; t += nthreads)
        if (vbits[t]) {
            atomicMax(&last_tile, t);
            atomicMin(&first_tile, t);
        }
    __syncthreads();
    const int nt_eff = last_tile + 1;  // tiles after the last valid token are skipped
    const int t_ref = first_tile;      // the tile that fixes the reference max

    // Copies.  Wave w copies tokens w, w + NW, ... of a tile, TOK_W of them.
    // Per token: a buffer resource over its latent row (a zero row for padding
    // tokens and for tiles at or past nt_eff), then the main-row copy (64 lanes
    // x 16 bytes) and the tail copy (lanes 0..7 x 16 bytes), both buffer-form
    // LDS-DMA.  With packed tail rows (TLOAD), the tile loop moves the tails
    // differently: wave w loads those of tokens TOK_W w .. TOK_W w + TOK_W - 1
    // into registers, eight tokens per 64-lane load (lane L: token 8 j + L / 8,
    // position L % 8), and stores them into LDS one tile later; its copies then
    // move main rows only, so a tile costs TOK_W + TOK_W / 8 memory instructions
    // per wave instead of 2 TOK_W and the tails need no per-token lane mask.
    // Every wave's memory counter thus advances by DMA_W per loop tile (PDMA_W
    // per tile copied whole: the first three and the exact recompute's).
    constexpr bool TLOAD = S::TSWZ && TOK_W % 8 == 0;
    constexpr int NTL = TLOAD ? TOK_W / 8 : 0;
    constexpr int PDMA_W = TOK_W * S::COPIES_PER_TOKEN;
    constexpr int DMA_W = TLOAD ? TOK_W + NTL : PDMA_W;
    const uint64_t kv_addr = reinterpret_cast<uint64_t>(a.kv);
    uint64_t zero_addr = reinterpret_cast<uint64_t>(kZeroLatentRow);
    asm volatile("" : "+s"(zero_addr));  // keep the address in registers, out of the copy code
    // 64-bit address of the latent row of token lane % 32 of tile tn (the zero
    // row for padding and for tiles at or past nt_eff), computed for all 32
    // tokens at once; each copy then reads its token's address from a lane.
    // tile_row reads the tile's table entries (ahead of use), row_base forms the
    // addresses.
    auto tile_row = [&](int tn, int tok) -> uint32_t {
        return rows[max(0, min(tn, kAttnMaxSplitTokens / 32 - 1)) * 32 + tok];
    };
    auto row_base = [&](int tn, uint32_t v) -> uint64_t {
        const uint32_t row = tn >= 0 && tn < nt_eff ? v : kNoRow;
        return row != kNoRow ? kv_addr + (uint64_t)row * (QK * 2) : zero_addr;
    };
    auto tile_base = [&](int tn) -> uint64_t { return row_base(tn, tile_row(tn, lane & 31)); };
    auto buffer_base = [&](int buf) { return (SA_LDS uint8_t *)opaque_lds((SA_LDS uint8_t *)&tile[buf][0]); };
    auto copy_token = [&](uint64_t mybase, int n, SA_LDS uint8_t *dstb, auto with_tail) {
        const int ii = wave + NW * n;  // wave-uniform
        const uint64_t base = ((uint64_t)lane_read((uint32_t)(mybase >> 32), ii) << 32) | lane_read((uint32_t)mybase, ii);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(reinterpret_cast<const void *>(base), QK * 2);
        if constexpr (S::MAIN > 0)  // lane i fetches the piece stored at position i
            buf_dma16_to_lds(rs, (lane * 16) ^ (16 * main_swizzle(ii)), dstb + ii * S::MAIN_STRIDE);
        if constexpr (decltype(with_tail)::value)
            if (lane < 8)  // lane i fetches the tail piece stored at position i
                buf_dma16_to_lds(rs, S::MAIN * 16 + 16 * S::tail_pos(lane, ii),
                                 dstb + S::TAIL_BASE + ii * S::TAIL_STRIDE);
    };
    constexpr std::true_type kWithTail{};
    constexpr std::integral_constant<bool, !TLOAD> kLoopTail{};
    auto issue_tile = [&](int tn, int buf) {
        const uint64_t mybase = tile_base(tn);
        SA_LDS uint8_t *dstb = buffer_base(buf);
#pragma unroll
        for (int n = 0; n < TOK_W; ++n) copy_token(mybase, n, dstb, kWithTail);
    };
    // packed tails (TLOAD): table entry, source and LDS slot of load j
    auto tail_tok = [&](int j) { return TOK_W * wave + 8 * j + (lane >> 3); };
    auto tail_src = [&](int tn, uint32_t v) -> uint64_t {
        return row_base(tn, v) + S::MAIN * 16 + 16 * S::tail_pos(lane & 7, lane >> 3);
    };
    auto tail_slot = [&](int buf, int j) -> SA_LDS u32x4 * {
        return (SA_LDS u32x4 *)((SA_LDS uint8_t *)&tile[buf][0] + S::TAIL_BASE + (TOK_W * wave + 8 * j) * S::TAIL_STRIDE) +
               lane;
    };

    // Exchange slot j (of 4, 16 bytes per lane) of the partial that wave `reader`
    // reads, for a tile whose partials pass through buffer buf: with XIN, the
    // main row of the reader's own token reader + NW j, which the reader's next
    // copy into that buffer overwrites only after it has read the slot.
    auto xslot = [&](int buf, int reader, int j) -> SA_LDS f32x4 * {
        if constexpr (XIN)
            return (SA_LDS f32x4 *)((SA_LDS uint8_t *)&tile[buf][0] + (reader + NW * j) * S::MAIN_STRIDE) + lane;
        else
            return (SA_LDS f32x4 *)&xchs[reader][j][lane];
    };
    auto xch_write = [&](int buf, const f32x16 &s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) *xslot(buf, partner, j) = f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
    };

    // LDS byte offset of this lane's K operand of step ks (S row c holds token
    // row_token(c); the lane supplies its pieces 2ks + half).
    // (main pieces 2ks + hf at position (2ks + hf) ^ swizzle: the swizzle only
    // flips bits 0..3 of the piece index)
    auto k_offset = [&](int c, int hf, int ks) {
        const int tok = row_token(c);
        return 2 * ks < S::MAIN
                   ? tok * S::MAIN_STRIDE + ((32 * (ks & 7) + 16 * hf) ^ (16 * main_swizzle(tok))) + 256 * (ks >> 3)
                   : S::TAIL_BASE + tok * S::TAIL_STRIDE + 16 * S::tail_pos(2 * ks - S::MAIN + hf, tok);
    };
    constexpr int KPF = SA_ATTN_KPF, VPF = SA_ATTN_VPF;
    auto lane_id = [&]() { return lane; };
    // This partner's S^T of the tile in buffer buf (steps KP px .. KP px + KP - 1);
    // after MFMA step ks, fill(ks) places independent work (the previous tile's
    // softmax, the next tile's copies) in the MFMA's shadow.
    auto qk_half = [&](auto cfg, int buf, auto &&fill) -> f32x16 {
        const int ln = lane_id(), c = ln & 31, hf = ln >> 5;
        const uint8_t *tb = tile[buf];
        constexpr int ks0 = KP * decltype(cfg)::PX;
        bf16x8 kr[KP];
#pragma unroll
        for (int u = 0; u < KPF && u < KP; ++u)
            kr[u] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + k_offset(c, hf, ks0 + u)));
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) {
            if (ks + KPF < KP)
                kr[ks + KPF] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + k_offset(c, hf, ks0 + ks + KPF)));
            s = mfma_32x32x16(kr[ks], qb[ks], s);
            fill(ks);
            __builtin_amdgcn_sched_barrier(0);  // keeps the operand reads KPF steps ahead, no further
        }
        return s;
    };
    auto no_fill = [](int) {};
    // Weights of a tile from its S^T in kSmSteps small steps, so that they can
    // sit between the next tile's q.k MFMAs: step 0 sets the reference (on the
    // tile that fixes it: the max of the valid tokens over both half-waves),
    // 1-8 exponentiate, round and sum pair j = step - 1.  Register i of half hf
    // holds token 16(i/8) + 8hf + i%8.  The reference max is fixed by the first
    // tile with a valid token for this head (until then O and l are 0, so
    // nothing needs rescaling) and never moves afterwards: the output
    // accumulators are only ever touched by the MFMAs.  Weights are
    // exp2(s - m).  A head whose logits outgrow its reference by 64 or more
    // leaves a lane's sum of weights at 2^64 or more (+inf once a weight
    // overflows fp32, with inf or NaN in its accumulators); after the last tile
    // that recomputes the split exactly with its true max (below; a sum that
    // large from many smaller weights only costs a needless recompute).  P^T operand k2 (tokens 16k2 + 8hf .. +7) is w[k2] (and
    // wl[k2], the bf16 residues, for `precise` rows).
    struct SmState {
        f32x16 s;
        float mref;
        uint32_t vb;
        bool full, set_ref;  // (workgroup-uniform) every token valid; the tile fixes the reference
        u32x4 w[2], wl[2];
        float lt, let;       // the tile's sums of the rounded and of the unrounded weights
    };
    constexpr int kSmSteps = 9;
    auto sm_begin = [&](SmState &st, int t, bool set_ref) {
        const uint32_t bits = vbits[t];
        st.full = __builtin_amdgcn_readfirstlane(bits) == 0xFFFFFFFFu;
        st.set_ref = set_ref;
        st.vb = bits >> (8 * half);
        st.lt = 0.0f;
        st.let = 0.0f;
    };
    auto valid_bit = [&](uint32_t vb, int i) { return ((vb >> (16 * (i >> 3) + (i & 7))) & 1u) != 0; };
    // Weights of pair j (registers 2j, 2j + 1): exponentiated, rounded, summed
    // into the tile's sums; with `masked`, padding tokens weigh 0.  The
    // normaliser sums the same rounded weights the MFMA multiplies V by, so the
    // output is an exact weighted mean of the kept rows up to fp32 accumulation.
    auto sm_pair = [&](auto cfg, SmState &st, int j, bool masked) {
        float e[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) e[h] = exp2_hw(fmaf(st.s[2 * j + h], a.scale_log2, -st.mref));
        uint32_t hi = pack_bf16x2(e[0], e[1]);
        uint32_t keep = 0xFFFFFFFFu;
        if (masked) {
            const bool v0 = valid_bit(st.vb, 2 * j), v1 = valid_bit(st.vb, 2 * j + 1);
            keep = (v0 ? 0x0000FFFFu : 0u) | (v1 ? 0xFFFF0000u : 0u);
            e[0] = v0 ? e[0] : 0.0f;
            e[1] = v1 ? e[1] : 0.0f;
            hi &= keep;
        }
        st.w[j >> 2][j & 3] = hi;
        st.let += e[0] + e[1];
        if constexpr (decltype(cfg)::PREC) {
            const uint32_t lo = pack_bf16x2(e[0] - bf16_lo_to_f32(hi), e[1] - bf16_hi_to_f32(hi)) & keep;
            st.wl[j >> 2][j & 3] = lo;
            st.lt = add_bf16_pair(lo, st.lt);
        }
        st.lt = add_bf16_pair(hi, st.lt);
    };
    // Padding tokens have zero latent rows, so their logits are 0: the
    // reference max and the weights leave them out.
    auto sm_step = [&](auto cfg, SmState &st, int step) {
        if (step == 0) {
            // max over the two half-waves (they hold the other 16 tokens)
            auto halves_max = [](float x) {
                const uint32_t u = __float_as_uint(x);
                const auto rr = __builtin_amdgcn_permlane32_swap(u, u, false, false);
                return fmaxf(__uint_as_float(rr[0]), __uint_as_float(rr[1]));
            };
            if (st.set_ref) {
                // (each branch tests the bits of its own opaque copy of vb, so
                // that the tests stay inside the rarely taken branches)
                uint32_t vbx = st.vb;
                asm volatile("" : "+v"(vbx));
                float mv = -INFINITY;
#pragma unroll
                for (int i = 0; i < 16; ++i) mv = fmaxf(mv, valid_bit(vbx, i) ? st.s[i] : -INFINITY);
                m = halves_max(mv) * a.scale_log2;
            }
            st.mref = m == -INFINITY ? 0.0f : m;  // still no valid token: every weight is 0
        } else if (step < kSmSteps) {
            sm_pair(cfg, st, step - 1, false);
        }
    };
    // Steps 1..8 take every token as valid; sm_end redoes a tile holding
    // padding with the validity mask (one uniform branch per tile instead of
    // one per pair), then adds the tile's sums to the wave's.
    auto sm_end = [&](auto cfg, SmState &st) {
        if (!st.full) {
            uint32_t vbx = st.vb;  // (opaque: the bit tests stay inside this branch)
            asm volatile("" : "+v"(vbx));
            st.vb = vbx;
            st.lt = 0.0f;
            st.let = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) sm_pair(cfg, st, j, true);
        }
        l += st.lt;
        le += st.let;
    };
    // O^T += V^T P^T over the tile's two 16-token halves: step q = (k2, vt)
    // multiplies output tile vt (value columns 32vt..32vt+31 of this partner's
    // range) by token half k2.  The V^T operand of lane (c, hf) is column c of
    // tokens 16k2 + 8hf + 0..7, read as two transposed 4-token reads
    // (ds_read_b64_tr_b16: within each 16 lanes, lane 4a + b receives element b
    // of the 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12).  So lane
    // L addresses token 16k2 + 8hf + 4s + ((L >> 2) & 3), columns 32vt + 16((L >> 4)
    // & 1) + 4(L & 3)..+3.  The operands of step q + VPF are read while step q
    // multiplies.
    auto pv = [&](auto cfg, int buf, const SmState &st) {
        constexpr int PX = decltype(cfg)::PX;
        const int ln = lane_id();
        const int j = (ln >> 2) & 3, a4 = ln & 3, g1 = (ln >> 4) & 1, hfv = ln >> 5;
        const int xq = 2 * g1 + (a4 >> 1);  // piece within the 32-column tile
        SA_LDS uint8_t *tb = (SA_LDS uint8_t *)&tile[buf][0];
        // lane-constant part of the address, and the step part XORed into it
        int lb;
        if constexpr (S::MAIN > 0)
            lb = (8 * hfv + j) * S::MAIN_STRIDE + 8 * (a4 & 1) + 64 * j + 16 * (xq ^ (2 * hfv)) + 16 * (PX * VW / 8);
        else
            lb = S::TAIL_BASE + (8 * hfv + j) * S::TAIL_STRIDE + 8 * (a4 & 1) + 16 * xq + 16 * (PX * VW / 8);
        auto vaddr = [&](int k2, int sh, int vt) -> int {
            if constexpr (S::MAIN > 0)
                return (lb ^ (64 * (vt & 3) + 16 * sh)) + (16 * k2 + 4 * sh) * S::MAIN_STRIDE + 256 * (vt >> 2);
            else
                return lb + (16 * k2 + 4 * sh) * S::TAIL_STRIDE + 64 * vt;
        };
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        auto vread = [&](int q) -> bf16x8 {
            const int k2 = q / NVT, vt = q % NVT;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS s16x4 *)(tb + vaddr(k2, 0, vt)));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS s16x4 *)(tb + vaddr(k2, 1, vt)));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr int NQ = 2 * NVT;
        bf16x8 vd[NQ];
#pragma unroll
        for (int q = 0; q < VPF && q < NQ; ++q) vd[q] = vread(q);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q + VPF < NQ) vd[q + VPF] = vread(q + VPF);
            const int k2 = q / NVT, vt = q % NVT;
            oacc[vt] = mfma_32x32x16(vd[q], as_bf16x8(st.w[k2]), oacc[vt]);
            if constexpr (decltype(cfg)::PREC) oacc[vt] = mfma_32x32x16(vd[q], as_bf16x8(st.wl[k2]), oacc[vt]);
            __builtin_amdgcn_sched_barrier(0);  // keeps the operand reads VPF steps ahead, no further
        }
    };

    // Ring of NB = 4 tile buffers.  The prologue issues tiles 0, 1 and 2 and
    // computes this wave's partial S^T of tile 0.  Iteration t:
    //   barrier A: every wave is done with tile t-1 (its buffer now holds the
    //     partials of tile t for their readers), and tile t+1 has landed;
    //   read the partner's partial of tile t;
    //   partial S^T of tile t+1, with, between its MFMAs, the sum of tile t's
    //     partials, tile t's weights, and the copies of tile t+3 into the
    //     buffer of tile t-1 (each wave refills only rows it has just read);
    //   O += V P of tile t;
    //   wait for this wave's copies of tile t+2 (only tile t+3's main-row
    //     copies are younger: memory operations complete in order);
    //   with packed tails, store tile t+2's tails and load tile t+3's;
    //   barrier B: every wave is done with tile t, whose buffer then takes the
    //     partials of tile t+1.
    // Tiles of padding only are not computed (block-uniform); the last
    // iteration computes the (unused) partial of an all-padding tile.
    auto tiles = [&](auto cfg) {
        static_assert(NB == 4, "the ring below holds two read tiles and two in flight");
        // W1: the copies younger than tile t+2's at the ring wait (tile t+3's
        // main rows; its packed tails are loaded after that wait)
        constexpr int W1 = (TLOAD ? TOK_W : DMA_W) < 63 ? (TLOAD ? TOK_W : DMA_W) : 63;
        constexpr int P1 = PDMA_W < 63 ? PDMA_W : 63, P2 = 2 * PDMA_W < 63 ? 2 * PDMA_W : 63;
        issue_tile(0, 0);
        issue_tile(1, 1);
        issue_tile(2, 2);
        f32x16 sp = f32x16{};
        if (nt_eff > 0) {
            attn_wait_vmcnt<P2>();
            barrier_lds();
            sp = qk_half(cfg, 0, no_fill);
            xch_write(NB - 1, sp);
            attn_wait_vmcnt<P1>();
        }
        // table entries of the next tile to copy, read a tile ahead
        uint32_t vnext = tile_row(3, lane & 31), vtail[NTL > 0 ? NTL : 1];
        u32x4 tails[NTL > 0 ? NTL : 1];  // packed tails loaded in the previous iteration
#pragma unroll
        for (int j = 0; j < NTL; ++j) vtail[j] = tile_row(3, tail_tok(j));
        for (int t = 0; t < nt_eff; ++t) {
            barrier_lds();  // A
            const int xb = (t + NB - 1) % NB;
            f32x4 pr[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) pr[j] = *xslot(xb, wave, j);
            SmState st;
            sm_begin(st, t, t == t_ref);
            const uint64_t nbase = row_base(t + 3, vnext);
            vnext = tile_row(t + 4, lane & 31);
            SA_LDS uint8_t *dstb = buffer_base(xb);
            constexpr int kAdd = KP > 2 ? 2 : 0;  // q.k step after which the partials are summed
            f32x16 sn = qk_half(cfg, (t + 1) % NB, [&](int ks) {
                if (ks == kAdd) {
                    // S^T of tile t: partner 0's partial first, in both partners
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        st.s[i] = decltype(cfg)::PX == 0 ? sp[i] + pr[i >> 2][i & 3] : pr[i >> 2][i & 3] + sp[i];
                }
                // the copies of tile t+3, after the partials have been read
                if (ks > kAdd && ks - kAdd - 1 < TOK_W) copy_token(nbase, ks - kAdd - 1, dstb, kLoopTail);
                if (ks > kAdd && ks - kAdd - 1 < kSmSteps) sm_step(cfg, st, ks - kAdd - 1);
            });
            // (q.k steps too few to hold every copy or softmax step: the rest here)
#pragma unroll
            for (int n = KP - kAdd - 1; n < TOK_W; ++n) copy_token(nbase, n, dstb, kLoopTail);
#pragma unroll
            for (int step = KP - kAdd - 1; step < kSmSteps; ++step) sm_step(cfg, st, step);
            sm_end(cfg, st);
            pv(cfg, t % NB, st);
            sp = sn;
            attn_wait_vmcnt<W1>();
            // the packed tails of tile t+2 (loaded at the end of the previous
            // iteration; the first three tiles were copied whole) into its
            // buffer, read from the next iteration on; then the loads of tile
            // t+3's, which have a whole iteration to arrive
            if (t > 0) {
#pragma unroll
                for (int j = 0; j < NTL; ++j) *tail_slot((t + 2) % NB, j) = tails[j];
            }
#pragma unroll
            for (int j = 0; j < NTL; ++j) {
                tails[j] = load16_global(tail_src(t + 3, vtail[j]));
                vtail[j] = tile_row(t + 4, tail_tok(j));
            }
            barrier_lds();  // B
            xch_write(t % NB, sp);
        }
        attn_wait_vmcnt<0>();  // the last (zero) copies have landed

        // Exact recompute of the split when some head's logits outgrew its reference
        // max by more than 64 (never for logits within a few dozen of each other):
        // pass 1 finds every head's true max, pass 2 redoes the weighted sum with it.
        if (le >= 0x1p64f) overflow_flag = 1;
        __syncthreads();
        if (overflow_flag) {
            // S^T of tile t (both partners), through buffer 0 and the exchange
            // slots of buffer 1
            auto full_s = [&](int t) -> f32x16 {
                issue_tile(t, 0);
                attn_wait_vmcnt<0>();
                __syncthreads();
                const f32x16 mine = qk_half(cfg, 0, no_fill);
                xch_write(1, mine);
                __syncthreads();
                f32x16 s;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 o = *xslot(1, wave, j);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[4 * j + e] = decltype(cfg)::PX == 0 ? mine[4 * j + e] + o[e] : o[e] + mine[4 * j + e];
                }
                __syncthreads();
                return s;
            };
            float mt = -INFINITY;
            for (int t = 0; t < nt_eff; ++t) {
                const f32x16 s0 = full_s(t);
                const uint32_t vb = vbits[t] >> (8 * half);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (valid_bit(vb, i)) mt = fmaxf(mt, s0[i] * a.scale_log2);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            m = mt;
            l = 0.0f;
            le = 0.0f;
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) oacc[vt] = f32x16{};
            for (int t = 0; t < nt_eff; ++t) {
                SmState st;
                st.s = full_s(t);
                sm_begin(st, t, false);
#pragma unroll
                for (int step = 0; step < kSmSteps; ++step) sm_step(cfg, st, step);  // (s <= m now)
                sm_end(cfg, st);
                pv(cfg, 0, st);
                __syncthreads();
            }
        }
    };
    auto run = [&](auto pxc) {
        if (precise) tiles(TileCfg<decltype(pxc)::value, true>{});
        else tiles(TileCfg<decltype(pxc)::value, false>{});
    };
    if (px == 0) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});

    // both partners hold the same normaliser and weight sums (the same S^T)
    const float lt = l + __shfl_xor(l, 32);
    const float lte = le + __shfl_xor(le, 32);
    if (!hok) return;
    if (a.splits == 1) {
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int64_t obase = ((int64_t)r * a.num_heads + head) * V + px * VW;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const int v = 32 * vt + acc_row(i, half);  // registers i..i+3: columns v..v+3
                const f32x4 o = f32x4{oacc[vt][i], oacc[vt][i + 1], oacc[vt][i + 2], oacc[vt][i + 3]} * inv;
                if (a.out_bf16)
                    *reinterpret_cast<u32x2 *>(reinterpret_cast<uint16_t *>(a.out) + obase + v) =
                        u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                else
                    *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(a.out) + obase + v) = o;
            }
        if (a.lse && half == 0 && px == 0)
            a.lse[(int64_t)r * a.num_heads + head] = lt > 0.0f ? (m + log2f(lte)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t pbase = (((int64_t)r * a.splits + split) * a.num_heads + head);
        float *po = a.part_o + pbase * V + px * VW;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<f32x4 *>(po + 32 * vt + acc_row(i, half)) =
                    f32x4{oacc[vt][i], oacc[vt][i + 1], oacc[vt][i + 2], oacc[vt][i + 3]};
        if (half == 0 && px == 0) *reinterpret_cast<f32x4 *>(a.part_ml + pbase * 4) = f32x4{m, lt, lte, 0.0f};
    }
}

// Merge the split partials of one (row, head): with M the largest partial max,
// o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i and
// lse = (M + log2 sum_i 2^(m_i - M) le_i) ln 2.  The max and the sums run over
// the splits with one split per thread; the weights 2^(m_i - M) are kept in LDS,
// and the weighted sum loads four splits' partials at a time.  A split without a
// valid token has l_i = 0, weight 0 and a zero (finite) partial.
constexpr int kCombineWeights = 256;  // splits whose weights are kept in LDS

__device__ __forceinline__ float combine_block_reduce(float v, bool is_max, float *red)
{
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        const float o = __shfl_xor(v, d);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float t = red[0];
    for (int w = 1; w < nw; ++w) t = is_max ? fmaxf(t, red[w]) : t + red[w];
    __syncthreads();  // red is reused by the next call
    return t;
}

// HPB heads per workgroup, blockDim.x / HPB threads each (HPB > 1 only with
// at most 64 splits, where every wave works on its own).
template <int V, int HPB>
__global__ __launch_bounds__(128 * HPB) void combine_kernel(const float *__restrict__ part_o,
                                                            const float *__restrict__ part_ml, int splits,
                                                            int num_heads, void *__restrict__ out, int out_bf16,
                                                            float *__restrict__ lse)
{
    __shared__ float wgt[kCombineWeights];
    __shared__ float red[2];
    const int nt = blockDim.x / HPB, h = blockIdx.x * HPB + threadIdx.x / nt, r = blockIdx.y;
    const int tid = threadIdx.x % nt;
    const int64_t base = (int64_t)r * splits * num_heads + h;  // partial (r, split 0, h)
    auto ml_of = [&](int s) { return *reinterpret_cast<const f32x4 *>(part_ml + (base + (int64_t)s * num_heads) * 4); };
    const bool wave_path = splits <= 64;  // (block-uniform) every wave on its own, one split per lane
    float M, L, Le, wl = 0.0f;
    if (wave_path) {
        const int ln = tid & 63;
        const f32x4 ml = ln < splits ? ml_of(ln) : f32x4{-INFINITY, 0.0f, 0.0f, 0.0f};
        float mx = ml[1] > 0.0f ? ml[0] : -INFINITY;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) mx = fmaxf(mx, __shfl_xor(mx, d));
        M = mx;
        wl = ml[1] > 0.0f ? exp2f(ml[0] - M) : 0.0f;
        float ls = ml[1] * wl, les = ml[2] * wl;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            ls += __shfl_xor(ls, d);
            les += __shfl_xor(les, d);
        }
        L = ls;
        Le = les;
    } else {
        float mx = -INFINITY;
        for (int s = tid; s < splits; s += nt) {
            const f32x4 ml = ml_of(s);
            if (ml[1] > 0.0f) mx = fmaxf(mx, ml[0]);
        }
        M = combine_block_reduce(mx, true, red);
        float ls = 0.0f, les = 0.0f;
        for (int s = tid; s < splits; s += nt) {
            const f32x4 ml = ml_of(s);
            const float f = ml[1] > 0.0f ? exp2f(ml[0] - M) : 0.0f;
            if (s < kCombineWeights) wgt[s] = f;
            ls += ml[1] * f;
            les += ml[2] * f;
        }
        L = combine_block_reduce(ls, false, red);
        Le = combine_block_reduce(les, false, red);  // (its barriers also publish wgt)
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    // (wave path: split s's weight sits in lane s.  v_readlane reads it whatever
    // the exec mask, which matters below: for V < 4 * 64 only the first V / 4
    // lanes run the column loop, and a shuffle from an inactive lane reads 0.)
    auto w_of = [&](int s) -> float {
        if (wave_path) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), s));
        if (s < kCombineWeights) return wgt[s];
        const f32x4 ml = ml_of(s);
        return ml[1] > 0.0f ? exp2f(ml[0] - M) : 0.0f;
    };
    const int64_t obase = ((int64_t)r * num_heads + h) * V;
    for (int v = 4 * tid; v < V; v += 4 * nt) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        const float *po = part_o + base * V + v;
        const int64_t sstep = (int64_t)num_heads * V;
        int s = 0;
        for (; s + 4 <= splits; s += 4) {
            f32x4 x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const f32x4 *>(po + (s + u) * sstep);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += w_of(s + u) * x[u];
        }
        for (; s < splits; ++s) acc += w_of(s) * *reinterpret_cast<const f32x4 *>(po + s * sstep);
        acc *= inv;
        if (out_bf16) {
            uint32_t *ob = reinterpret_cast<uint32_t *>(out) + ((obase + v) >> 1);
            ob[0] = pack_bf16x2(acc[0], acc[1]);
            ob[1] = pack_bf16x2(acc[2], acc[3]);
        } else {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + obase + v) = acc;
        }
    }
    if (lse && tid == 0) lse[(int64_t)r * num_heads + h] = L > 0.0f ? (M + log2f(Le)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace sa
