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
// gfx950 mapping.  One workgroup = one (row, split, value half); wave w owns heads
// 32w..32w+31 and keeps their query rows in registers for the whole split.  Per
// tile of 32 kept tokens:
//   * the 32 latent rows are copied HBM -> LDS by buffer-form LDS-DMA, one
//     resource per token row: a 64-lane copy of its first 1 KiB and an 8-lane
//     copy of its 128-byte tail; the main rows' 16-byte pieces are XOR-swizzled
//     by token (through the copy's per-lane source offsets) so that MFMA
//     operand reads do not collide on LDS banks; a ring of 4 tile buffers
//     keeps 3 tiles' copies in flight while one tile is computed;
//   * the query of 32 heads (QK = 576: 144 registers per lane) and the 32 x 512
//     fp32 output accumulators (256 registers) of one wave do not fit in the
//     512-entry register file next to the q.k accumulator, so for V = 512 two
//     workgroups share a (row, split), each owning 256 value columns and each
//     computing the logits itself;
//   * S^T[token][head] = K . Q^T on 32x32x16 bf16 MFMAs (K from LDS, Q^T from
//     registers, contraction over QK in 16-wide steps);
//   * softmax in base 2 in fp32 against a per-head reference max taken from
//     the first tile with a valid token; it never moves, so the output
//     accumulators are touched only by MFMAs (a split whose logits outgrow the
//     reference by more than 64 is recomputed exactly with its true max);
//   * the S^T accumulator already has the register layout of the B operand of
//     O^T[v][head] += V^T[v][token] . P^T[token][head]: P is only rounded to bf16.
//     The softmax denominator sums the same rounded P.
//     The V^T operand comes straight from the token-major tile through
//     transposed LDS reads (ds_read_b64_tr_b16), four tokens per read.
#pragma once

#include "device_common.hpp"

namespace sa {

constexpr int kAttnMaxSplitTokens = 2048;
constexpr uint32_t kNoRow = 0xFFFFFFFFu;

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
};

#ifndef SA_ATTN_KPF
#define SA_ATTN_KPF 6  // K operand steps read ahead of their MFMA
#endif
#ifndef SA_ATTN_VPF
#define SA_ATTN_VPF 4  // V operand steps read ahead of their MFMAs
#endif
#ifndef SA_ATTN_FENCE
#define SA_ATTN_FENCE 1  // 1: a scheduling fence closes every MFMA step
#endif

constexpr int kAttnBuffers = 4;  // tile ring: kAttnBuffers - 1 tiles in flight while one is computed


template <int N>
__device__ __forceinline__ void attn_wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int QK, int V>
struct AttnShape {
    static constexpr int KS = QK / 16;                   // MFMA steps of q.k
    static constexpr int VSPLIT = V > 256 ? 2 : 1;       // workgroups sharing one (row, split), by v range
    static constexpr int VW = V / VSPLIT;                // v columns per workgroup
    static constexpr int NVT = VW / 32;                  // 32-column output tiles per wave
    static constexpr int PIECES = QK / 8;                // 16-byte pieces per latent row
    // LDS image of a 32-token tile.  Main rows: pieces 0..63 of each token
    // (one 1 KiB copy per token), MAIN_STRIDE bytes apart, piece p of token t
    // stored at position p ^ main_swizzle(t).  Tail: the remaining 8 pieces
    // (128 bytes) of each token, TAIL_STRIDE bytes apart (the extra 16 bytes
    // move consecutive tokens to different 16-byte bank groups).  Rows shorter
    // than 64 pieces live in the tail only.
    static constexpr int MAIN = PIECES >= 64 ? 64 : 0;
    static constexpr int TAIL = PIECES - MAIN;
    static constexpr int MAIN_STRIDE = MAIN * 16;
    static constexpr int TAIL_STRIDE = TAIL * 16 + 16;
    static constexpr int TAIL_BASE = 32 * MAIN_STRIDE;
    static constexpr int TILE_BYTES = TAIL_BASE + 32 * TAIL_STRIDE;
    static constexpr int COPIES_PER_TOKEN = (MAIN ? 1 : 0) + 1;  // main row, tail
    static_assert(QK % 16 == 0 && VW % 32 == 0 && V <= QK, "shape family");
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
// l + the two bf16 values packed in w (each times 1.0)
__device__ __forceinline__ float add_bf16_pair(uint32_t w, float l)
{
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, w), __builtin_bit_cast(b2, 0x3F803F80u), l, false);
}


// Workgroup id -> logical block.  Workgroups are dealt to the 8 XCDs in turn
// (id mod 8); this map gives each XCD a contiguous range of logical blocks, so
// the blocks of one query row (its splits and value halves), which read the
// same query and the same latent rows, share one L2.
__device__ __forceinline__ int xcd_block(int id, int n)
{
    const int q = n >> 3, rem = n & 7, x = id & 7;
    return x * q + min(x, rem) + (id >> 3);
}

// NW waves per workgroup, wave w owning heads 32w..32w+31 (NW = ceil(H / 32)).
// One-dimensional grid of rows * splits * VSPLIT workgroups.
template <int QK, int V, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attend_kernel(const AttnArgs a)
{
    using S = AttnShape<QK, V>;
    constexpr int KS = S::KS, VW = S::VW;
    __shared__ __attribute__((aligned(1024))) uint8_t tile[kAttnBuffers][S::TILE_BYTES];
    __shared__ uint32_t rows[kAttnMaxSplitTokens];
    __shared__ uint32_t vbits[kAttnMaxSplitTokens / 32];
    __shared__ int last_tile, overflow_flag;

    const int per_row = a.splits * S::VSPLIT;
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int r = lb / per_row, split = (lb % per_row) / S::VSPLIT, vh = lb % S::VSPLIT;
    constexpr int nthreads = 64 * NW;
    const int wave = wave_uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    __builtin_assume(wave >= 0 && wave < NW);  // lets copy kinds resolve at compile time
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

    const int head = 32 * wave + col;
    const bool hok = head < a.num_heads;
    // q^T operand of step ks for this lane: q[head][16ks + 8half .. +7]
    // (issued first: these loads overlap the row look-ups below).  Lanes of
    // heads past num_heads load the last head instead: their S^T columns feed
    // only their own, never stored, output columns.
    bf16x8 qb[KS];
    {
        const int qhead = hok ? head : a.num_heads - 1;
        const uint16_t *qp = a.q + ((int64_t)r * a.num_heads + qhead) * QK + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qb[ks] = as_bf16x8(load16(qp + 16 * ks));
    }

    // Physical row of every kept token of this split (kNoRow = padding) and a
    // validity mask per 32-token tile.  Positions, then block-table entries, are
    // loaded 8 per thread at a time, so the look-ups cost two memory round trips.
    for (int jb = 0; jb < ntiles * 32; jb += 8 * nthreads) {
        int idx[8], blk[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = jb + u * nthreads + threadIdx.x;
            idx[u] = j < cnt ? sel[j] : -1;
        }
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
    }
    if (threadIdx.x == 0) {
        last_tile = -1;
        overflow_flag = 0;
    }
    f32x16 oacc[S::NVT];  // O^T tile vt: columns 32vt.. of this block's value range
#pragma unroll
    for (int vt = 0; vt < S::NVT; ++vt) oacc[vt] = f32x16{};
    // m: reference max (log2 units); l: sum of the bf16-rounded weights (output
    // normaliser); le: sum of the unrounded weights (log-sum-exp)
    float m = -INFINITY, l = 0.0f, le = 0.0f;
    bool ovf = false;
    __syncthreads();
    for (int t = threadIdx.x; t < ntiles; t += nthreads)
        if (vbits[t]) atomicMax(&last_tile, t);
    __syncthreads();
    const int nt_eff = last_tile + 1;  // tiles after the last valid token are skipped

    // Copies.  Wave w copies tokens w, w + NW, ... of a tile, TOK_W of them (a
    // surplus repeats token 31, which writes the same bytes again).  Per token:
    // a buffer resource over its latent row (a zero row for padding tokens and
    // for tiles at or past nt_eff), then the main-row copy (64 lanes x 16 bytes)
    // and the tail copy (lanes 0..7 x 16 bytes), both buffer-form LDS-DMA.  The
    // memory counter of every wave thus advances by DMA_W per tile.  `myrow` is
    // the row of token lane % 32 of the tile.
    constexpr int TOK_W = (32 + NW - 1) / NW;
    constexpr int DMA_W = TOK_W * S::COPIES_PER_TOKEN;
    const uint64_t kv_addr = reinterpret_cast<uint64_t>(a.kv);
    uint64_t zero_addr = reinterpret_cast<uint64_t>(kZeroLatentRow);
    asm volatile("" : "+s"(zero_addr));  // keep the address in registers, out of the copy code
    auto tile_row = [&](int tn) -> uint32_t {
        const uint32_t v = rows[max(0, min(tn, kAttnMaxSplitTokens / 32 - 1)) * 32 + (lane & 31)];
        return tn >= 0 && tn < nt_eff ? v : kNoRow;
    };
    // `dstb`: the LDS base of the buffer, from opaque_lds (the tile reads that
    // follow use other buffers, and the ring waits order the rest)
    auto copy_token = [&](uint32_t myrow, int n, SA_LDS uint8_t *dstb) {
        const int ii = min(wave + NW * n, 31);  // wave-uniform
        const uint32_t row = lane_read(myrow, ii);
        // (a mask blend rather than a conditional, so no branch splits the q.k steps)
        const uint64_t keep = (uint64_t)0 - (uint64_t)(row != kNoRow);
        const uint64_t base = ((kv_addr + (uint64_t)row * (QK * 2)) & keep) | (zero_addr & ~keep);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(reinterpret_cast<const void *>(base), QK * 2);
        if constexpr (S::MAIN > 0)  // lane i fetches the piece stored at position i
            buf_dma16_to_lds(rs, (lane * 16) ^ (16 * main_swizzle(ii)), dstb + ii * S::MAIN_STRIDE);
        if (lane < 8) buf_dma16_to_lds(rs, S::MAIN * 16 + lane * 16, dstb + S::TAIL_BASE + ii * S::TAIL_STRIDE);
    };
    auto buffer_base = [&](int buf) { return (SA_LDS uint8_t *)opaque_lds((SA_LDS uint8_t *)&tile[buf][0]); };
    auto issue_tile = [&](int tn, int buf) {
        const uint32_t myrow = tile_row(tn);
        SA_LDS uint8_t *dstb = buffer_base(buf);
#pragma unroll
        for (int n = 0; n < TOK_W; ++n) copy_token(myrow, n, dstb);
    };

    // LDS byte offset of this lane's K operand of step ks (S row c holds token
    // row_token(c); the lane supplies its pieces 2ks + half).
    // (main pieces 2ks + hf at position (2ks + hf) ^ swizzle: the swizzle only
    // flips bits 0..3 of the piece index)
    auto k_offset = [&](int c, int hf, int ks) {
        const int tok = row_token(c);
        return 2 * ks < S::MAIN
                   ? tok * S::MAIN_STRIDE + ((32 * (ks & 7) + 16 * hf) ^ (16 * main_swizzle(tok))) + 256 * (ks >> 3)
                   : S::TAIL_BASE + tok * S::TAIL_STRIDE + 16 * (2 * ks - S::MAIN + hf);
    };

    // Per tile: S^T = K Q^T (qk), the softmax weights of S^T (softmax), then
    // O^T += V^T P^T (pv).  The loop below is software-pipelined across tiles:
    // iteration t computes S^T of tile t+1 while the weights of tile t are
    // formed (VALU beside the MFMAs), then multiplies tile t's values.  The
    // schedule is pinned so that LDS operand reads run ahead of the MFMAs that
    // use them: K operands KPF steps ahead, V operands VPF steps ahead.
    constexpr int KPF = SA_ATTN_KPF, VPF = SA_ATTN_VPF;
    auto lane_id = [&]() {
        // The lane id is made opaque per tile so that the lane-dependent values
        // derived from it are recomputed (a few ALU ops) instead of being hoisted
        // out of the tile loop, where they would compete with the accumulators.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        return ln;
    };
    // S^T of the tile in buffer buf; with_copies: the main copies of the tile
    // whose lane rows are `myrow` go into buffer nbuf between the q.k steps, and
    // after each MFMA a few VALU slots are left for independent work (the
    // previous tile's softmax)
    auto qk = [&](int buf, uint32_t myrow, int nbuf, auto with_copies, auto &&fill) -> f32x16 {
        const int ln = lane_id(), c = ln & 31, hf = ln >> 5;
        const uint8_t *tb = tile[buf];
        SA_LDS uint8_t *dstb = nullptr;
        if constexpr (decltype(with_copies)::value) dstb = buffer_base(nbuf);
        bf16x8 kr[KS];
#pragma unroll
        for (int u = 0; u < KPF && u < KS; ++u)
            kr[u] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + k_offset(c, hf, u)));
        f32x16 s = f32x16{};
        // Step ks: read the operand of step ks + KPF, multiply, issue this
        // step's copies, then the caller's VALU work.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + KPF < KS)
                kr[ks + KPF] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + k_offset(c, hf, ks + KPF)));
            s = mfma_32x32x16(kr[ks], qb[ks], s);
            if constexpr (decltype(with_copies)::value) {
                // tokens n with n * KS / TOK_W == ks
                const int n_lo = (ks * TOK_W + KS - 1) / KS, n_hi = ((ks + 1) * TOK_W + KS - 1) / KS;
#pragma unroll
                for (int n = n_lo; n < n_hi; ++n) copy_token(myrow, n, dstb);
            }
            fill(ks);
#if SA_ATTN_FENCE
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
        return s;
    };
    auto no_fill = [](int) {};
    // Weights of tile t from its S^T (branch-free).  Register i of half hf holds
    // token 16(i/8) + 8hf + i%8.  The reference max is fixed by the first tile
    // with a valid token for this head (until then O and l are 0, so nothing
    // needs rescaling) and never moves afterwards: the output accumulators are
    // only ever touched by the MFMAs.  Weights are exp2(min(s - m, 64)), finite
    // in fp32 and bf16; a head whose logits outgrow its reference by more than
    // 64 raises `ovf`, and the split is then recomputed exactly with its true
    // max (below).
    // The weights in kSmSteps small steps, so that the steps can sit between the
    // next tile's q.k MFMAs: steps 0-3 mask, 4-7 reduce the max, 8 crosses the
    // half-waves and sets the reference, 9-24 exponentiate, 25-32 round to bf16
    // and sum.  State lives in `SmState`.
    struct SmState {
        f32x16 s;
        float tmax, mref;
        float p[16];
        u32x4 w[2];
        uint32_t vb;
    };
    constexpr int kSmSteps = 33;
    auto sm_begin = [&](SmState &st, const f32x16 &s_in, int t) {
        st.s = s_in;
        st.vb = vbits[t] >> (8 * half);
    };
    auto sm_step = [&](SmState &st, int step) {
        if (step < 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * step + e;
                st.s[i] = ((st.vb >> (16 * (i >> 3) + (i & 7))) & 1u) ? st.s[i] : -INFINITY;
            }
        } else if (step < 8) {
            const int i0 = 4 * (step - 4);
            const float mx = fmaxf(fmaxf(st.s[i0], st.s[i0 + 1]), fmaxf(st.s[i0 + 2], st.s[i0 + 3]));
            st.tmax = step == 4 ? mx : fmaxf(st.tmax, mx);
        } else if (step == 8) {
            // max over the two half-waves (they hold the other 16 tokens)
            const uint32_t u = __float_as_uint(st.tmax);
            const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
            const float tmax = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])) * a.scale_log2;
            m = m == -INFINITY ? tmax : m;
            ovf |= tmax > m + 64.0f;
            st.mref = m == -INFINITY ? 0.0f : m;  // still no valid token: every s is -inf
        } else if (step < 25) {
            const int i = step - 9;
            st.p[i] = exp2_hw(fminf(fmaf(st.s[i], a.scale_log2, -st.mref), 64.0f));
        } else if (step < kSmSteps) {
            const int j = step - 25, k2 = j >> 2, jj = j & 3;
            const uint32_t w = pack_bf16x2(st.p[2 * j], st.p[2 * j + 1]);
            st.w[k2][jj] = w;
            // the normaliser sums the same bf16-rounded weights the MFMA
            // multiplies V by, so the output is an exact weighted mean of the
            // kept rows up to fp32 accumulation
            l = add_bf16_pair(w, l);
            le += st.p[2 * j] + st.p[2 * j + 1];
        }
    };
    auto sm_finish = [&](SmState &st, bf16x8 *pb) {
        pb[0] = as_bf16x8(st.w[0]);
        pb[1] = as_bf16x8(st.w[1]);
    };
    // the whole softmax of one tile, unpipelined
    auto softmax = [&](const f32x16 &s_in, int t, bf16x8 *pb) {
        SmState st;
        sm_begin(st, s_in, t);
#pragma unroll
        for (int step = 0; step < kSmSteps; ++step) sm_step(st, step);
        sm_finish(st, pb);
    };
    // O^T += V^T P^T over the tile's two 16-token halves: step q = (k2, vt)
    // multiplies output tile vt (value columns 32vt..32vt+31 of this block's
    // range) by token half k2.  The V^T operand of lane (c, hf) is column c of
    // tokens 16k2 + 8hf + 0..7, read as two transposed 4-token reads
    // (ds_read_b64_tr_b16: within each 16 lanes, lane 4a + b receives element b
    // of the 8-byte chunks addressed by lanes a, a + 4, a + 8, a + 12).  So lane
    // L addresses token 16k2 + 8hf + 4s + ((L >> 2) & 3), columns 32vt + 16((L >> 4)
    // & 1) + 4(L & 3)..+3.  The operands of step q + VPF are read while step q
    // multiplies.
    auto pv = [&](int buf, const bf16x8 *pb) {
        const int ln = lane_id();
        const int j = (ln >> 2) & 3, a4 = ln & 3, g1 = (ln >> 4) & 1, hfv = ln >> 5;
        const int xq = 2 * g1 + (a4 >> 1);  // piece within the 32-column tile
        SA_LDS uint8_t *tb = (SA_LDS uint8_t *)&tile[buf][0];
        // lane-constant part of the address, and the step part XORed into it
        int lb;
        if constexpr (S::MAIN > 0)
            lb = (8 * hfv + j) * S::MAIN_STRIDE + 8 * (a4 & 1) + 64 * j + 16 * (xq ^ (2 * hfv)) + 16 * (vh * VW / 8);
        else
            lb = S::TAIL_BASE + (8 * hfv + j) * S::TAIL_STRIDE + 8 * (a4 & 1) + 16 * xq + 16 * (vh * VW / 8);
        auto vaddr = [&](int k2, int sh, int vt) -> int {
            if constexpr (S::MAIN > 0)
                return (lb ^ (64 * (vt & 3) + 16 * sh)) + (16 * k2 + 4 * sh) * S::MAIN_STRIDE + 256 * (vt >> 2);
            else
                return lb + (16 * k2 + 4 * sh) * S::TAIL_STRIDE + 64 * vt;
        };
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        auto vread = [&](int q) -> bf16x8 {
            const int k2 = q / S::NVT, vt = q % S::NVT;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS s16x4 *)(tb + vaddr(k2, 0, vt)));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS s16x4 *)(tb + vaddr(k2, 1, vt)));
            return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        constexpr int NQ = 2 * S::NVT;
        bf16x8 vd[NQ];
#pragma unroll
        for (int q = 0; q < VPF && q < NQ; ++q) vd[q] = vread(q);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            if (q + VPF < NQ) vd[q + VPF] = vread(q + VPF);
            const int k2 = q / S::NVT, vt = q % S::NVT;
            oacc[vt] = mfma_32x32x16(vd[q], pb[k2], oacc[vt]);
#if SA_ATTN_FENCE
            __builtin_amdgcn_sched_barrier(0);
#endif
        }
    };

    // Ring of kAttnBuffers = 4 tile buffers, two tiles resident (t for its values,
    // t+1 for its q.k) and two in flight.  The prologue issues tiles 0..2;
    // iteration t (which computes S^T of tile t+1) issues tile t+3 into the buffer
    // of tile t-1 (zeros past nt_eff).  Copies complete in order and every wave
    // issues DMA_W per tile, so waiting for tile t+1 with only tile t+2 younger is
    // "at most DMA_W copies in flight" (before the loop: tile 0, two younger).
    // The barrier then makes every wave's share of tile t+1 visible and certifies
    // that every wave is done with tile t-1's buffer.  Tiles of padding only are
    // not computed (block-uniform).
    static_assert(kAttnBuffers == 4, "the ring below holds two resident and two in-flight tiles");
    constexpr int W2 = 2 * DMA_W < 63 ? 2 * DMA_W : 63;  // clamped: waiting for more is safe
    constexpr int W1 = DMA_W < 63 ? DMA_W : 63;
#pragma unroll
    for (int j = 0; j < kAttnBuffers - 1; ++j) issue_tile(j, j);
    f32x16 s_cur = f32x16{};
    if (nt_eff > 0) {
        attn_wait_vmcnt<W2>();
        barrier_no_fence();
        s_cur = qk(0, kNoRow, 0, std::false_type{}, no_fill);
    }
    for (int t = 0; t < nt_eff; ++t) {
        bf16x8 pb[2];
        f32x16 s_nxt = f32x16{};
        if (t + 1 < nt_eff) {  // (block-uniform)
            const uint32_t myrow = tile_row(t + 3);
            attn_wait_vmcnt<W1>();
            barrier_no_fence();
            SmState st;
            sm_begin(st, s_cur, t);
            // step ks of tile t's softmax after q.k step ks of tile t+1
            s_nxt = qk((t + 1) % kAttnBuffers, myrow, (t + 3) % kAttnBuffers, std::true_type{},
                       [&](int ks) { sm_step(st, ks); });
#pragma unroll
            for (int step = KS; step < kSmSteps; ++step) sm_step(st, step);
            sm_finish(st, pb);
        } else {
            softmax(s_cur, t, pb);
        }
        pv(t % kAttnBuffers, pb);
        s_cur = s_nxt;
    }
    attn_wait_vmcnt<0>();  // the last (zero) copies have landed

    // Exact recompute of the split when some head's logits outgrew its reference
    // max by more than 64 (never for logits within a few dozen of each other):
    // pass 1 finds every head's true max, pass 2 redoes the weighted sum with it.
    if (ovf) overflow_flag = 1;
    __syncthreads();
    if (overflow_flag) {
        float mt = -INFINITY;
        for (int t = 0; t < nt_eff; ++t) {
            issue_tile(t, 0);
            attn_wait_vmcnt<0>();
            __syncthreads();
            const f32x16 s0 = qk(0, kNoRow, 0, std::false_type{}, no_fill);
            const uint32_t vb = vbits[t] >> (8 * half);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((vb >> (16 * (i >> 3) + (i & 7))) & 1u) mt = fmaxf(mt, s0[i] * a.scale_log2);
            __syncthreads();
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        m = mt;
        l = 0.0f;
        le = 0.0f;
#pragma unroll
        for (int vt = 0; vt < S::NVT; ++vt) oacc[vt] = f32x16{};
        for (int t = 0; t < nt_eff; ++t) {
            issue_tile(t, 0);
            attn_wait_vmcnt<0>();
            __syncthreads();
            bf16x8 pb[2];
            softmax(qk(0, kNoRow, 0, std::false_type{}, no_fill), t, pb);  // s <= m now, so no weight is clamped
            pv(0, pb);
            __syncthreads();
        }
    }

    const float lt = l + __shfl_xor(l, 32);
    const float lte = le + __shfl_xor(le, 32);
    if (!hok) return;
    if (a.splits == 1) {
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int64_t obase = ((int64_t)r * a.num_heads + head) * V + vh * VW;
#pragma unroll
        for (int vt = 0; vt < S::NVT; ++vt)
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
        if (a.lse && half == 0 && vh == 0)
            a.lse[(int64_t)r * a.num_heads + head] = lt > 0.0f ? (m + log2f(lte)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t pbase = (((int64_t)r * a.splits + split) * a.num_heads + head);
        float *po = a.part_o + pbase * V + vh * VW;
#pragma unroll
        for (int vt = 0; vt < S::NVT; ++vt)
#pragma unroll
            for (int i = 0; i < 16; i += 4)
                *reinterpret_cast<f32x4 *>(po + 32 * vt + acc_row(i, half)) =
                    f32x4{oacc[vt][i], oacc[vt][i + 1], oacc[vt][i + 2], oacc[vt][i + 3]};
        if (half == 0 && vh == 0) *reinterpret_cast<f32x4 *>(a.part_ml + pbase * 4) = f32x4{m, lt, lte, 0.0f};
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
