// Sparse softmax attention with four partner waves per 32-head block (gfx950).
//
// Computes what attend_kernel computes (the pages' sparse attention operator:
// "Day-0 Model Adaptation Depends on the Compute Software Stack", Operator
// Library Abstraction; "Day-0 Adaptation: Running Trillion-Parameter Models on
// Domestic AI Accelerators", section 3.1; the tile loop of "Day-0 Adaptation for
// LLMs: Implementing Sparse Attention and Low-Precision Weights", section II),
// with the same tile ring, LDS-DMA gather and split partials, but at two waves
// per SIMD instead of one.
//
// Work split.  A workgroup covers 32 * HB heads of one (row, split) with 4 * HB
// waves: partner p = 0..3 of head block hb.  For q.k, partner p holds its 32
// heads' query over a quarter of the QK dims (QK = 576: 9 MFMA steps, 36
// registers) and computes a partial S^T[token][head] of the tile.  The four
// partials are reduce-scattered through LDS: partner p receives token chunk p
// (8 of the 32 tokens: accumulator registers 4p .. 4p + 3) from the other three
// and adds the four in partner order, so each logit is summed once and the same
// way everywhere.  Partner p then computes the softmax weights of its chunk
// only, rounds them to bf16 and publishes them; every partner reads the whole
// tile's P^T operand back and multiplies it into its own quarter of the value
// columns (128 columns: 64 accumulator registers).  So no logit, weight or
// product is computed twice, and a wave holds about half the registers of the
// two-partner kernel.
//
// LDS.  The ring of 4 tile buffers is the two-partner kernel's.  The partial
// chunks of tile t pass through the main rows of the buffer of tile t - 1 once
// every wave is done with it (reader r reads rows r, r + NW, r + 2 NW, which it
// refills itself right after); the bf16 weights of tile t pass through the rope
// rows (the tail) of tile t's own buffer, dead once every wave has taken its
// q.k; for rows that carry P as hi + lo, the lo half passes through the last
// main rows of the spent buffer, whose refill then waits for the third barrier.
//
// Per tile t, one wave:
//   barrier A: partials of tile t published;
//   read its three received chunks; q.k partial of tile t + 1 (9 MFMAs) with,
//     in their shadow, the sum of the chunks, the copies of tile t + 3 into the
//     spent buffer and the softmax of its chunk; publish its weights;
//   barrier B: weights published;
//   read the tile's P^T; O^T += V^T P^T over its value columns (8 MFMAs);
//   wait for its copies of tile t + 2;
//   barrier C: every wave is done with tile t;
//   publish the chunks of tile t + 1's partial into tile t's buffer.
#pragma once

#include "attention.hpp"

namespace sa {

template <int QK, int V, int HB>
__global__ __launch_bounds__(256 * HB, 1) void attend_p4_kernel(const AttnArgs a)
{
    constexpr int NP = 4;
    using S = AttnShape<QK, V, NP>;
    constexpr int KP = S::KP, VW = S::VW, NVT = S::NVT;
    constexpr int NW = NP * HB, nthreads = 64 * NW;
    constexpr int NB = kAttnBuffers;
    static_assert(NB == 4, "ring of two read tiles and two in flight");
    static_assert(32 % NW == 0, "tokens per wave");
    constexpr int TOK_W = 32 / NW;  // tokens each wave copies per tile
    static_assert(S::MAIN == 64 && TOK_W >= 3, "partials pass through three main rows the reader refills");
    // bf16 weights of one tile: [hb][k2][lane] 16 bytes, partner p filling bytes
    // 8 (p & 1) .. + 7 of k2 = p / 2
    constexpr int PBYTES = HB * 2 * 64 * 16;
    static_assert(PBYTES <= 32 * S::TAIL_STRIDE, "weights fit the tail rows");
    constexpr int PROW0 = 32 - PBYTES / S::MAIN_STRIDE;  // main rows that carry lo weights
    static_assert(3 * NW <= PROW0, "lo weights clear of the partials");
    __shared__ __attribute__((aligned(1024))) uint8_t tile[NB][S::TILE_BYTES];
    __shared__ uint32_t rows[kAttnMaxSplitTokens];
    __shared__ uint32_t vbits[kAttnMaxSplitTokens / 32];
    __shared__ float red[2][NW][32];
    __shared__ int first_tile, last_tile, overflow_flag;

    const int hgroups = (a.num_heads + 32 * HB - 1) / (32 * HB);
    const int lb = xcd_block(blockIdx.x, gridDim.x);
    const int r = lb / (a.splits * hgroups), split = (lb / hgroups) % a.splits, hg = lb % hgroups;
    const int wave = wave_uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    __builtin_assume(wave >= 0 && wave < NW);
    const int hb = wave % HB, px = wave / HB;  // head block, partner index
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
    const bool precise = min(limit, a.k) < kPreciseBelow;

    const int head = 32 * (HB * hg + hb) + col;
    const bool hok = head < a.num_heads;
    // Physical rows of the split's kept tokens, as in the two-partner kernel:
    // positions (loaded before the queries), then block-table entries.
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
            const int w0 = (j - lane) >> 5;
            if (lane == 0 && w0 < ntiles) vbits[w0] = (uint32_t)m;
            if (lane == 32 && w0 + 1 < ntiles) vbits[w0 + 1] = (uint32_t)(m >> 32);
        }
    };
    int idx0[8];
    load_positions(0, idx0);

    // q^T operand of step ks of this partner's quarter:
    // q[head][16 (KP px + ks) + 8 half .. + 7] (lanes past num_heads: the last head)
    bf16x8 qb[KP];
    {
        const int qhead = hok ? head : a.num_heads - 1;
        const uint16_t *qp = a.q + ((int64_t)r * a.num_heads + qhead) * QK + 16 * KP * px + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) qb[ks] = as_bf16x8(load16(qp + 16 * ks));
    }

    if (ntiles > 0) look_up(0, idx0);
    for (int jb = 8 * nthreads; jb < ntiles * 32; jb += 8 * nthreads) {
        int idx[8];
        load_positions(jb, idx);
        look_up(jb, idx);
    }
    if (threadIdx.x == 0) {
        first_tile = kAttnMaxSplitTokens;
        last_tile = -1;
        overflow_flag = 0;
    }
    f32x16 oacc[NVT];  // O^T tile vt: value columns VW px + 32 vt ..
#pragma unroll
    for (int vt = 0; vt < NVT; ++vt) oacc[vt] = f32x16{};
    // m: reference max (log2 units, the same in all four partners); l, le: this
    // lane's sums of the rounded and unrounded weights of its chunk's tokens
    float m = -INFINITY, l = 0.0f, le = 0.0f;
    __syncthreads();
    for (int t = threadIdx.x; t < ntiles; t += nthreads)
        if (vbits[t]) {
            atomicMax(&last_tile, t);
            atomicMin(&first_tile, t);
        }
    __syncthreads();
    const int nt_eff = last_tile + 1;
    const int t_ref = first_tile;

    // Copies: wave w copies tokens w + NW n of a tile (see attend_kernel).
    constexpr int DMA_W = TOK_W * S::COPIES_PER_TOKEN;
    const uint64_t kv_addr = reinterpret_cast<uint64_t>(a.kv);
    uint64_t zero_addr = reinterpret_cast<uint64_t>(kZeroLatentRow);
    asm volatile("" : "+s"(zero_addr));
    auto tile_base = [&](int tn) -> uint64_t {
        const uint32_t v = rows[max(0, min(tn, kAttnMaxSplitTokens / 32 - 1)) * 32 + (lane & 31)];
        const uint32_t row = tn >= 0 && tn < nt_eff ? v : kNoRow;
        return row != kNoRow ? kv_addr + (uint64_t)row * (QK * 2) : zero_addr;
    };
    auto buffer_base = [&](int buf) { return (SA_LDS uint8_t *)opaque_lds((SA_LDS uint8_t *)&tile[buf][0]); };
    auto copy_token = [&](uint64_t mybase, int n, SA_LDS uint8_t *dstb) {
        const int ii = wave + NW * n;
        const uint64_t base = ((uint64_t)lane_read((uint32_t)(mybase >> 32), ii) << 32) | lane_read((uint32_t)mybase, ii);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(reinterpret_cast<const void *>(base), QK * 2);
        buf_dma16_to_lds(rs, (lane * 16) ^ (16 * main_swizzle(ii)), dstb + ii * S::MAIN_STRIDE);
        if (lane < 8)
            buf_dma16_to_lds(rs, S::MAIN * 16 + 16 * S::tail_pos(lane, ii), dstb + S::TAIL_BASE + ii * S::TAIL_STRIDE);
    };
    auto issue_tile = [&](int tn, int buf) {
        const uint64_t mybase = tile_base(tn);
        SA_LDS uint8_t *dstb = buffer_base(buf);
#pragma unroll
        for (int n = 0; n < TOK_W; ++n) copy_token(mybase, n, dstb);
    };

    // Partial exchange.  Slot j of reader wave `reader` in buffer buf: main row
    // reader + NW j, 16 bytes per lane.  Sender partner p writes its chunk g
    // (g != p) to slot (p < g ? p : p - 1) of reader hb + HB g.
    auto xslot = [&](int buf, int reader, int j) -> SA_LDS f32x4 * {
        return (SA_LDS f32x4 *)((SA_LDS uint8_t *)&tile[buf][0] + (reader + NW * j) * S::MAIN_STRIDE) + lane;
    };
    auto chunk = [](const f32x16 &s, int g) { return f32x4{s[4 * g], s[4 * g + 1], s[4 * g + 2], s[4 * g + 3]}; };
    auto xch_write = [&](auto cfg, int buf, const f32x16 &s) {
        constexpr int PX = decltype(cfg)::PX;
#pragma unroll
        for (int g = 0; g < NP; ++g)
            if (g != PX) *xslot(buf, hb + HB * g, PX < g ? PX : PX - 1) = chunk(s, g);
    };
    // chunk PX of the tile's S^T: the four partners' chunks added in partner order
    auto xch_sum = [&](auto cfg, const f32x4 &own, const f32x4 (&pr)[NP - 1]) -> f32x4 {
        constexpr int PX = decltype(cfg)::PX;
        f32x4 s = PX == 0 ? own : pr[0];
#pragma unroll
        for (int p = 1; p < NP; ++p) s += p == PX ? own : pr[p < PX ? p : p - 1];
        return s;
    };
    // bf16 weights of a tile: hi in the tail rows of buffer hbuf, lo (rows that
    // carry hi + lo) in main rows PROW0 .. 31 of buffer lbuf
    auto p_slot = [&](int buf, int k2, bool lo) -> SA_LDS uint8_t * {
        return (SA_LDS uint8_t *)&tile[buf][0] + (lo ? PROW0 * S::MAIN_STRIDE : S::TAIL_BASE) +
               ((hb * 2 + k2) * 64 + lane) * 16;
    };

    auto k_offset = [&](int c, int hf, int ks) {
        const int tok = row_token(c);
        return 2 * ks < S::MAIN
                   ? tok * S::MAIN_STRIDE + ((32 * (ks & 7) + 16 * hf) ^ (16 * main_swizzle(tok))) + 256 * (ks >> 3)
                   : S::TAIL_BASE + tok * S::TAIL_STRIDE + 16 * S::tail_pos(2 * ks - S::MAIN + hf, tok);
    };
    constexpr int KPF = SA_ATTN_KPF < KP ? SA_ATTN_KPF : KP, VPF = SA_ATTN_VPF;
    auto lane_id = [&]() { return lane; };
    // This partner's partial S^T of the tile in buffer buf; fill(ks) after MFMA
    // step ks places independent work in its shadow.
    auto qk_part = [&](auto cfg, int buf, auto &&fill) -> f32x16 {
        const int ln = lane_id(), c = ln & 31, hf = ln >> 5;
        const uint8_t *tb = tile[buf];
        constexpr int ks0 = KP * decltype(cfg)::PX;
        bf16x8 kr[KP];
#pragma unroll
        for (int u = 0; u < KPF; ++u)
            kr[u] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + k_offset(c, hf, ks0 + u)));
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KP; ++ks) {
            if (ks + KPF < KP)
                kr[ks + KPF] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + k_offset(c, hf, ks0 + ks + KPF)));
            s = mfma_32x32x16(kr[ks], qb[ks], s);
            fill(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
        return s;
    };
    auto no_fill = [](int) {};

    // Softmax of this partner's chunk.  Register e of the chunk (accumulator
    // register 4 PX + e) of half hf holds tile token 16 (PX / 2) + 8 hf + 4 (PX & 1)
    // + e.  Weights exp2(s - m) against the reference max m, which the first
    // tile with a valid token fixes for good (the max over its valid tokens, from
    // all four partners' chunks); padding tokens weigh 0.
    auto valid_bit = [&](uint32_t vb, int i) { return ((vb >> (16 * (i >> 3) + (i & 7))) & 1u) != 0; };
    struct Chunk {
        f32x4 s;
        uint32_t hi[2], lo[2];
    };
    // the max over the valid tokens of chunk s of every partner of this head
    // block (the whole workgroup takes part: one barrier)
    auto ref_max = [&](auto cfg, const f32x4 &s, uint32_t vb) -> float {
        constexpr int PX = decltype(cfg)::PX;
        float mv = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) mv = fmaxf(mv, valid_bit(vb, 4 * PX + e) ? s[e] : -INFINITY);
        mv = fmaxf(mv, __shfl_xor(mv, 32));
        if (half == 0) red[0][wave][col] = mv;
        barrier_lds();
        float mx = red[0][hb][col];
#pragma unroll
        for (int p = 1; p < NP; ++p) mx = fmaxf(mx, red[0][hb + HB * p][col]);
        return mx;
    };
    // weights of pair j (registers 2j, 2j + 1 of the chunk) against mref
    auto sm_pair = [&](auto cfg, Chunk &ch, int j, float mref, uint32_t vb, bool full) {
        constexpr int PX = decltype(cfg)::PX;
        float e[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) e[h] = exp2_hw(fmaf(ch.s[2 * j + h], a.scale_log2, -mref));
        uint32_t hi = pack_bf16x2(e[0], e[1]);
        uint32_t keep = 0xFFFFFFFFu;
        if (!full) {
            const bool v0 = valid_bit(vb, 4 * PX + 2 * j), v1 = valid_bit(vb, 4 * PX + 2 * j + 1);
            keep = (v0 ? 0x0000FFFFu : 0u) | (v1 ? 0xFFFF0000u : 0u);
            e[0] = v0 ? e[0] : 0.0f;
            e[1] = v1 ? e[1] : 0.0f;
            hi &= keep;
        }
        ch.hi[j] = hi;
        le += e[0] + e[1];
        if constexpr (decltype(cfg)::PREC) {
            const uint32_t lo = pack_bf16x2(e[0] - bf16_lo_to_f32(hi), e[1] - bf16_hi_to_f32(hi)) & keep;
            ch.lo[j] = lo;
            l = add_bf16_pair(lo, l);
        }
        l = add_bf16_pair(hi, l);
    };
    auto p_write = [&](auto cfg, const Chunk &ch, int hbuf, int lbuf) {
        constexpr int PX = decltype(cfg)::PX;
        *(SA_LDS u32x2 *)(p_slot(hbuf, PX >> 1, false) + 8 * (PX & 1)) = u32x2{ch.hi[0], ch.hi[1]};
        if constexpr (decltype(cfg)::PREC)
            *(SA_LDS u32x2 *)(p_slot(lbuf, PX >> 1, true) + 8 * (PX & 1)) = u32x2{ch.lo[0], ch.lo[1]};
    };
    // O^T += V^T P^T over this partner's value columns for the tile in buffer
    // buf, with the P^T operands read from hbuf (and lbuf).  V^T operands come
    // through transposed LDS reads exactly as in attend_kernel.
    auto pv = [&](auto cfg, int buf, int hbuf, int lbuf) {
        constexpr int PX = decltype(cfg)::PX;
        u32x4 w[2], wl[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            w[k2] = *(SA_LDS u32x4 *)p_slot(hbuf, k2, false);
            if constexpr (decltype(cfg)::PREC) wl[k2] = *(SA_LDS u32x4 *)p_slot(lbuf, k2, true);
        }
        const int ln = lane_id();
        const int j = (ln >> 2) & 3, a4 = ln & 3, g1 = (ln >> 4) & 1, hfv = ln >> 5;
        const int xq = 2 * g1 + (a4 >> 1);
        SA_LDS uint8_t *tb = (SA_LDS uint8_t *)&tile[buf][0];
        const int lbv = (8 * hfv + j) * S::MAIN_STRIDE + 8 * (a4 & 1) + 64 * j + 16 * (xq ^ (2 * hfv)) +
                        16 * (PX * VW / 8);
        auto vaddr = [&](int k2, int sh, int vt) -> int {
            return (lbv ^ (64 * (vt & 3) + 16 * sh)) + (16 * k2 + 4 * sh) * S::MAIN_STRIDE + 256 * (vt >> 2);
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
            oacc[vt] = mfma_32x32x16(vd[q], as_bf16x8(w[k2]), oacc[vt]);
            if constexpr (decltype(cfg)::PREC) oacc[vt] = mfma_32x32x16(vd[q], as_bf16x8(wl[k2]), oacc[vt]);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    auto tiles = [&](auto cfg) {
        constexpr int PX = decltype(cfg)::PX;
        constexpr bool PREC = decltype(cfg)::PREC;
        // with hi + lo weights, the copy of this wave's token in rows PROW0..31 of
        // the spent buffer waits for barrier C (those rows carry the lo weights)
        constexpr int NLATE = PREC && (HB * PX + (HB - 1) + NW * (TOK_W - 1) >= PROW0) ? 1 : 0;
        static_assert(!PREC || HB * PX + NW * (TOK_W - 2) + HB - 1 < PROW0, "one late token per wave at most");
        constexpr int NEARLY = TOK_W - NLATE;
        constexpr int W1 = NEARLY * S::COPIES_PER_TOKEN;  // copies younger than tile t + 2's
        issue_tile(0, 0);
        issue_tile(1, 1);
        issue_tile(2, 2);
        f32x16 sp = f32x16{};
        if (nt_eff > 0) {
            attn_wait_vmcnt<2 * DMA_W < 63 ? 2 * DMA_W : 63>();
            barrier_lds();
            sp = qk_part(cfg, 0, no_fill);
            xch_write(cfg, NB - 1, sp);
            attn_wait_vmcnt<DMA_W>();
        }
        for (int t = 0; t < nt_eff; ++t) {
            barrier_lds();  // A
            const int xb = (t + NB - 1) % NB;
            f32x4 pr[NP - 1];
#pragma unroll
            for (int j = 0; j < NP - 1; ++j) pr[j] = *xslot(xb, wave, j);
            const f32x4 own = chunk(sp, PX);
            const uint32_t vbt = vbits[t];
            const bool full = __builtin_amdgcn_readfirstlane(vbt) == 0xFFFFFFFFu;
            const uint32_t vb = vbt >> (8 * half);
            Chunk ch;
            float mref = m == -INFINITY ? 0.0f : m;
            if (t == t_ref) {  // (block-uniform) the tile that fixes the reference max
                ch.s = xch_sum(cfg, own, pr);
                m = ref_max(cfg, ch.s, vb) * a.scale_log2;
                mref = m;
            }
            const uint64_t nbase = tile_base(t + 3);
            SA_LDS uint8_t *dstb = buffer_base(xb);
            const f32x16 sn = qk_part(cfg, (t + 1) % NB, [&](int ks) {
                if (ks == 0 && t != t_ref) ch.s = xch_sum(cfg, own, pr);
                // the early copies of tile t + 3, after the partials have been read
                if (ks >= 1 && ks - 1 < NEARLY) copy_token(nbase, ks - 1, dstb);
                if (ks == 2) sm_pair(cfg, ch, 0, mref, vb, full);
                if (ks == 4) sm_pair(cfg, ch, 1, mref, vb, full);
            });
#pragma unroll
            for (int n = KP - 1; n < NEARLY; ++n) copy_token(nbase, n, dstb);
            if constexpr (KP <= 2) sm_pair(cfg, ch, 0, mref, vb, full);
            if constexpr (KP <= 4) sm_pair(cfg, ch, 1, mref, vb, full);
            p_write(cfg, ch, t % NB, xb);
            barrier_lds();  // B
            pv(cfg, t % NB, t % NB, xb);
            attn_wait_vmcnt<W1>();
            barrier_lds();  // C
            if constexpr (NLATE > 0) copy_token(nbase, TOK_W - 1, dstb);
            xch_write(cfg, t % NB, sn);
            sp = sn;
        }
        attn_wait_vmcnt<0>();

        // Exact recompute when some head's logits outgrew its reference max (a
        // lane's sum of weights of 2^64 or more, +inf included): pass 1 finds the
        // true max, pass 2 redoes the weighted sum with it.  Not pipelined: tile t
        // in buffer 0, partials through buffer 1, weights through buffers 0 and 2.
        if (le >= 0x1p64f) overflow_flag = 1;
        __syncthreads();
        if (overflow_flag) {
            auto full_chunk = [&](int t) -> f32x4 {
                issue_tile(t, 0);
                attn_wait_vmcnt<0>();
                __syncthreads();
                const f32x16 mine = qk_part(cfg, 0, no_fill);
                xch_write(cfg, 1, mine);
                __syncthreads();
                f32x4 pr[NP - 1];
#pragma unroll
                for (int j = 0; j < NP - 1; ++j) pr[j] = *xslot(1, wave, j);
                return xch_sum(cfg, chunk(mine, PX), pr);
            };
            float mt = -INFINITY;
            for (int t = 0; t < nt_eff; ++t) {
                const f32x4 s = full_chunk(t);
                const uint32_t vb = vbits[t] >> (8 * half);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (valid_bit(vb, 4 * PX + e)) mt = fmaxf(mt, s[e] * a.scale_log2);
            }
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            __syncthreads();
            if (half == 0) red[0][wave][col] = mt;
            __syncthreads();
            m = red[0][hb][col];
#pragma unroll
            for (int p = 1; p < NP; ++p) m = fmaxf(m, red[0][hb + HB * p][col]);
            l = 0.0f;
            le = 0.0f;
#pragma unroll
            for (int vt = 0; vt < NVT; ++vt) oacc[vt] = f32x16{};
            for (int t = 0; t < nt_eff; ++t) {
                Chunk ch;
                ch.s = full_chunk(t);
                const uint32_t vb = vbits[t] >> (8 * half);
                const float mref = m == -INFINITY ? 0.0f : m;
                sm_pair(cfg, ch, 0, mref, vb, false);  // (s <= m now)
                sm_pair(cfg, ch, 1, mref, vb, false);
                p_write(cfg, ch, 0, 2);  // (buffer 0's tail: its q.k is done)
                __syncthreads();
                pv(cfg, 0, 0, 2);
                __syncthreads();
            }
        }
    };
    auto run = [&](auto pxc) {
        if (precise) tiles(TileCfg<decltype(pxc)::value, true>{});
        else tiles(TileCfg<decltype(pxc)::value, false>{});
    };
    switch (px) {
    case 0: run(std::integral_constant<int, 0>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    default: run(std::integral_constant<int, 3>{}); break;
    }

    // the head's sums over both lane halves and the four partners (partner order)
    const float lh = l + __shfl_xor(l, 32), leh = le + __shfl_xor(le, 32);
    __syncthreads();
    if (half == 0) {
        red[0][wave][col] = lh;
        red[1][wave][col] = leh;
    }
    __syncthreads();
    float lt = red[0][hb][col], lte = red[1][hb][col];
#pragma unroll
    for (int p = 1; p < NP; ++p) {
        lt += red[0][hb + HB * p][col];
        lte += red[1][hb + HB * p][col];
    }
    if (!hok) return;
    if (a.splits == 1) {
        const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
        const int64_t obase = ((int64_t)r * a.num_heads + head) * V + px * VW;
#pragma unroll
        for (int vt = 0; vt < NVT; ++vt)
#pragma unroll
            for (int i = 0; i < 16; i += 4) {
                const int v = 32 * vt + acc_row(i, half);
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

}  // namespace sa
