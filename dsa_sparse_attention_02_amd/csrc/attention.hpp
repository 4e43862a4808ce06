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
//   * the 32 latent rows are copied HBM -> LDS by the LDS-DMA path
//     (global_load_lds_dwordx4), 16-byte pieces XOR-swizzled by token so that
//     MFMA operand reads do not collide on LDS banks; a ring of 4 tile buffers
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
//     The V^T operand is gathered from LDS as dwords (two adjacent v of one
//     token) and split with byte permutes into an "even v" and an "odd v"
//     operand, so every LDS byte read is used.
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
    int decode;                  // 1: row r = sequence r, limit ctx_lens[r]; 0: sequence 0, limit limit_base + r + 1
    int limit_base;
    int tokens_per_split, splits, out_bf16;
    float scale_log2;            // softmax_scale * log2(e)
};

constexpr int kAttnBuffers = 4;  // tile ring: kAttnBuffers - 1 tiles in flight while one is computed

// s_barrier without the memory fence __syncthreads adds (which would wait for
// every LDS-DMA copy in flight); the asm memory clobber keeps the compiler from
// moving memory operations across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

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
    static constexpr int VP = VW / 64;                   // 64-wide v groups (even + odd tiles)
    static constexpr int PIECES = QK / 8;                // 16-byte pieces per latent row
    static constexpr int TILE_BYTES = 32 * PIECES * 16;
    static constexpr int DMA_PER_TILE = 32 * PIECES / 64;   // wave instructions per tile
    static_assert(QK % 16 == 0 && PIECES % 8 == 0 && VW % 64 == 0 && V <= QK, "shape family");
};

// LDS slot of 16-byte piece p of tile token t.  Rows are PIECES long (a
// multiple of 8); XOR-ing the low 3 bits with (t>>1)&7 puts the same piece of 16
// consecutive tokens on 16 distinct 16-byte bank groups.  The map is its own
// inverse and never leaves p's aligned group of 8.
__device__ __forceinline__ int tile_slot(int t, int p) { return p ^ ((t >> 1) & 7); }

// NW waves per workgroup, wave w owning heads 32w..32w+31 (NW = ceil(H / 32)).
template <int QK, int V, int NW>
__global__ __launch_bounds__(64 * NW, 1) void attend_kernel(const AttnArgs a)
{
    using S = AttnShape<QK, V>;
    constexpr int KS = S::KS, VP = S::VP, VW = S::VW, PIECES = S::PIECES;
    __shared__ __attribute__((aligned(1024))) uint8_t tile[kAttnBuffers][S::TILE_BYTES];
    __shared__ uint32_t rows[kAttnMaxSplitTokens];
    __shared__ uint32_t vbits[kAttnMaxSplitTokens / 32];
    __shared__ int last_tile, overflow_flag;

    const int split = blockIdx.x / S::VSPLIT, vh = blockIdx.x % S::VSPLIT, r = blockIdx.y;
    constexpr int nthreads = 64 * NW, nw = NW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int seq = a.decode ? r : 0;
    const int limit = a.decode ? a.ctx_lens[r] : a.limit_base + r + 1;
    const int j0 = split * a.tokens_per_split;
    const int cnt = max(0, min(a.tokens_per_split, a.k - j0));
    const int ntiles = (cnt + 31) / 32;
    const int32_t *sel = a.topk_idx + (int64_t)r * a.k + j0;
    const int32_t *tbl = a.block_table + (int64_t)seq * a.max_blocks;
    const int bmask = (1 << a.bs_log2) - 1;

    // physical row of every kept token of this split (kNoRow = padding), and a
    // validity bit mask per 32-token tile
    for (int jb = wave * 64; jb < ntiles * 32; jb += nthreads) {
        const int j = jb + lane;
        uint32_t row = kNoRow;
        if (j < cnt) {
            const int idx = sel[j];
            if (idx >= 0 && idx < limit) {
                const int blk = tbl[idx >> a.bs_log2];
                if (blk >= 0 && blk < a.num_blocks) row = ((uint32_t)blk << a.bs_log2) | (uint32_t)(idx & bmask);
            }
        }
        const uint64_t m = __ballot(row != kNoRow);
        if (j < ntiles * 32) rows[j] = row;
        if (lane == 0) vbits[jb >> 5] = (uint32_t)m;
        if (lane == 32 && jb + 32 < ntiles * 32) vbits[(jb >> 5) + 1] = (uint32_t)(m >> 32);
    }
    if (threadIdx.x == 0) {
        last_tile = -1;
        overflow_flag = 0;
    }
    // zero the tile buffers: slots of padding tokens are never copied into, and
    // they are multiplied by P = 0, so they must hold finite values
    for (int e = threadIdx.x; e < kAttnBuffers * S::TILE_BYTES / 16; e += nthreads)
        reinterpret_cast<u32x4 *>(&tile[0][0])[e] = u32x4{0, 0, 0, 0};

    const int head = 32 * wave + col;
    const bool hok = head < a.num_heads;
    // q^T operand of step ks for this lane: q[head][16ks + 8half .. +7]
    bf16x8 qb[KS];
    {
        const uint16_t *qp = a.q + ((int64_t)r * a.num_heads + head) * QK + 8 * half;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qb[ks] = hok ? as_bf16x8(load16(qp + 16 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
#pragma unroll
        for (int ks = KS; ks < KS; ++ks) asm volatile("" : "+a"(qb[ks]));
    }
    f32x16 oe[VP], oo[VP];
#pragma unroll
    for (int vp = 0; vp < VP; ++vp) {
        oe[vp] = f32x16{};
        oo[vp] = f32x16{};
    }
    // m: reference max (log2 units); l: sum of the bf16-rounded weights (output
    // normaliser); le: sum of the unrounded weights (log-sum-exp)
    float m = -INFINITY, l = 0.0f, le = 0.0f;
    bool ovf = false;
    __syncthreads();
    for (int t = threadIdx.x; t < ntiles; t += nthreads)
        if (vbits[t]) atomicMax(&last_tile, t);
    __syncthreads();
    const int nt_eff = last_tile + 1;  // tiles after the last valid token are skipped

    // A tile's copies.  Lane i first takes the row of token i % 32 (one LDS read
    // per tile); a copy instruction's lanes then pick their token's row from it:
    // with rows of >= 64 pieces an instruction spans at most two tokens, whose
    // rows come from v_readlane (no memory access); shorter rows use a lane
    // shuffle.  (LDS reads of rows[] could not overlap each other: none may pass
    // a copy into LDS.)
    constexpr int DMA_W = (S::DMA_PER_TILE + NW - 1) / NW;  // copies per wave per tile (at most)
    auto issue_tile = [&](int t, int buf) {
        const int myrow = (int)rows[t * 32 + (lane & 31)];
#pragma unroll 1
        for (int ii = wave; ii < S::DMA_PER_TILE; ii += NW) {
            const int L = ii * 64 + lane;
            const int tj = L / PIECES, p = tile_slot(tj, L % PIECES);
            int row;
            if constexpr (PIECES >= 64) {
                const int t0 = (ii * 64) / PIECES;  // wave-uniform
                const int ra = __builtin_amdgcn_readlane(myrow, t0);
                const int rb = __builtin_amdgcn_readlane(myrow, t0 + 1 < 32 ? t0 + 1 : 31);
                row = tj == t0 ? ra : rb;
            } else {
                row = __shfl(myrow, tj);
            }
            if ((uint32_t)row != kNoRow)
                dma16_to_lds(a.kv + (int64_t)(uint32_t)row * QK + p * 8, (SA_LDS void *)&tile[buf][ii * 1024]);
        }
    };

    auto compute = [&](int t, int buf) {
        // The lane id is made opaque per tile so that the lane-dependent values
        // below are recomputed (a few ALU ops) instead of being hoisted out of
        // the tile loop, where they would compete with the accumulators for
        // registers.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int c = ln & 31, hf = ln >> 5;
        // Per-lane LDS byte offsets of the operand reads.  With the swizzle only the
        // low 3 bits of a piece index move, so every read is one of these bases
        // plus a compile-time offset:
        //   K operand of step ks (token c, piece 2ks+hf):   koff[ks&3] + 128*(ks>>2)
        //   V dword of token 16k2+tj0(j), pair VW/2*vh + 32vp + c:
        //                                 voff[j] + 256*PIECES*k2 + 128*vp  (vh folded into voff)
        int koff[4], voff[8];
        {
            const int xk = (c >> 1) & 7;
#pragma unroll
            for (int j = 0; j < 4; ++j) koff[j] = (c * PIECES + ((2 * j + hf) ^ xk)) * 16;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tj0 = 8 * (j >> 2) + 4 * hf + (j & 3);
                voff[j] = (tj0 * PIECES + ((c >> 2) ^ ((tj0 >> 1) & 7))) * 16 + (c & 3) * 4 + vh * VW * 2;
            }
        }
        const uint8_t *tb = tile[buf];
        // two accumulators (even / odd steps) halve the dependent MFMA chain
        f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
        for (int g = 0; g < KS; g += 4) {
            bf16x8 ka[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (g + u < KS)
                    ka[u] = as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + koff[(g + u) & 3] + 128 * ((g + u) >> 2)));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int ks = g + u;
                if (ks >= KS) break;
                if (ks & 1) s1 = mfma_32x32x16(ka[u], qb[ks], s1);
                else s0 = mfma_32x32x16(ka[u], qb[ks], s0);
            }
        }
        f32x16 s = s0 + s1;
        const uint32_t vb = vbits[t] >> (4 * hf);  // bit acc_row(i, hf) - 4hf = 8(i/4) + i%4
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool ok = (vb >> (8 * (i >> 2) + (i & 3))) & 1u;
            s[i] = ok ? s[i] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[i]);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        // The reference max is fixed by the first tile with a valid token for this
        // head (until then O and l are 0, so nothing needs rescaling) and never
        // moves afterwards: the output accumulators are only ever touched by the
        // MFMAs.  Weights are exp2(min(s - m, 64)), finite in fp32 and bf16; a head
        // whose logits outgrow its reference by more than 64 raises `ovf`, and the
        // split is then recomputed exactly with its true max (below).
        if (m == -INFINITY) m = tmax;
        ovf |= tmax > m + 64.0f;
        bf16x8 pb[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            u32x4 w;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float x0 = s[8 * k2 + 2 * jj], x1 = s[8 * k2 + 2 * jj + 1];
                const float p0 = x0 == -INFINITY ? 0.0f : exp2f(fminf(x0 - m, 64.0f));
                const float p1 = x1 == -INFINITY ? 0.0f : exp2f(fminf(x1 - m, 64.0f));
                w[jj] = pack_bf16x2(p0, p1);
                // the normaliser sums the same bf16-rounded weights the MFMA
                // multiplies V by, so the output is an exact weighted mean of
                // the kept rows up to fp32 accumulation
                l += __uint_as_float(w[jj] << 16) + __uint_as_float(w[jj] & 0xFFFF0000u);
                le += p0 + p1;
            }
            pb[k2] = as_bf16x8(w);
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
            for (int vp = 0; vp < VP; ++vp) {
                uint32_t d[8];
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    d[j] = *reinterpret_cast<const uint32_t *>(tb + voff[j] + 256 * PIECES * k2 + 128 * vp);
                u32x4 ev, od;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    ev[jj] = __builtin_amdgcn_perm(d[2 * jj + 1], d[2 * jj], 0x05040100u);
                    od[jj] = __builtin_amdgcn_perm(d[2 * jj + 1], d[2 * jj], 0x07060302u);
                }
                oe[vp] = mfma_32x32x16(as_bf16x8(ev), pb[k2], oe[vp]);
                oo[vp] = mfma_32x32x16(as_bf16x8(od), pb[k2], oo[vp]);
            }
        }
    };

    // Ring of kAttnBuffers tiles.  Iteration t: wait until this wave's copies of
    // tile t have landed (at most the kAttnBuffers-2 younger tiles' copies still in
    // flight), barrier (every wave's share of tile t is in LDS, and every wave is
    // done reading tile t-1's buffer), refill that buffer with tile
    // t+kAttnBuffers-1, then compute tile t.  Tiles of padding only are neither
    // copied nor computed (block-uniform).  Each wave issues the same number of
    // copies per tile only when NW divides DMA_PER_TILE; otherwise the wait count
    // below is still an upper bound of the younger copies, so it only over-waits.
#pragma unroll
    for (int j = 0; j < kAttnBuffers - 1; ++j)
        if (j < nt_eff) issue_tile(j, j);
    for (int t = 0; t < nt_eff; ++t) {
        // (clamped to the counter's range: waiting for more copies is always safe)
        attn_wait_vmcnt<(DMA_W * (kAttnBuffers - 2) < 63 ? DMA_W * (kAttnBuffers - 2) : 63)>();
        barrier_no_fence();
        const int tn = t + kAttnBuffers - 1;
        if (tn < nt_eff) issue_tile(tn, tn % kAttnBuffers);
        compute(t, t % kAttnBuffers);
    }

    // Exact recompute of the split when some head's logits outgrew its reference
    // max by more than 64 (never for logits within a few dozen of each other):
    // pass 1 finds every head's true max, pass 2 redoes the weighted sum with it.
    if (ovf) overflow_flag = 1;
    __syncthreads();
    if (overflow_flag) {
        float mt = -INFINITY;
        for (int t = 0; t < nt_eff; ++t) {
            issue_tile(t, 0);
            __syncthreads();
            const uint8_t *tb = tile[0];
            f32x16 s0 = f32x16{};
            const int xk = (col >> 1) & 7;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int slot = 8 * (ks >> 2) + ((2 * (ks & 3) + half) ^ xk);
                s0 = mfma_32x32x16(as_bf16x8(*reinterpret_cast<const u32x4 *>(tb + (col * PIECES + slot) * 16)),
                                   qb[ks], s0);
            }
            const uint32_t vb = vbits[t] >> (4 * half);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if ((vb >> (8 * (i >> 2) + (i & 3))) & 1u) mt = fmaxf(mt, s0[i] * a.scale_log2);
            __syncthreads();
        }
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        m = mt;
        l = 0.0f;
        le = 0.0f;
#pragma unroll
        for (int vp = 0; vp < VP; ++vp) {
            oe[vp] = f32x16{};
            oo[vp] = f32x16{};
        }
        for (int t = 0; t < nt_eff; ++t) {
            issue_tile(t, 0);
            __syncthreads();
            compute(t, 0);  // s <= m now, so no weight is clamped
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
        for (int vp = 0; vp < VP; ++vp)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = 64 * vp + 2 * acc_row(i, half);
                const float e0 = oe[vp][i] * inv, e1 = oo[vp][i] * inv;
                if (a.out_bf16)
                    reinterpret_cast<uint32_t *>(a.out)[(obase + v) >> 1] = pack_bf16x2(e0, e1);
                else
                    *reinterpret_cast<f32x2 *>(reinterpret_cast<float *>(a.out) + obase + v) = f32x2{e0, e1};
            }
        if (a.lse && half == 0 && vh == 0)
            a.lse[(int64_t)r * a.num_heads + head] = lt > 0.0f ? (m + log2f(lte)) * 0.69314718055994531f : -INFINITY;
    } else {
        const int64_t pbase = (((int64_t)r * a.splits + split) * a.num_heads + head);
        float *po = a.part_o + pbase * V + vh * VW;
#pragma unroll
        for (int vp = 0; vp < VP; ++vp)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int v = 64 * vp + 2 * acc_row(i, half);
                *reinterpret_cast<f32x2 *>(po + v) = f32x2{oe[vp][i], oo[vp][i]};
            }
        if (half == 0 && vh == 0) *reinterpret_cast<f32x4 *>(a.part_ml + pbase * 4) = f32x4{m, lt, lte, 0.0f};
    }
}

// Merge the split partials of one (row, head): with M the largest partial max,
// o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i and
// lse = (M + log2 sum_i 2^(m_i - M) le_i) ln 2.
template <int V>
__global__ __launch_bounds__(128) void combine_kernel(const float *__restrict__ part_o,
                                                      const float *__restrict__ part_ml, int splits,
                                                      int num_heads, void *__restrict__ out, int out_bf16,
                                                      float *__restrict__ lse)
{
    const int h = blockIdx.x, r = blockIdx.y;
    const int64_t base = (int64_t)r * splits * num_heads + h;  // partial (r, split 0, h)
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) {
        const f32x4 ml = *reinterpret_cast<const f32x4 *>(part_ml + (base + (int64_t)s * num_heads) * 4);
        if (ml[1] > 0.0f) M = fmaxf(M, ml[0]);
    }
    float L = 0.0f, Le = 0.0f;
    for (int s = 0; s < splits; ++s) {
        const f32x4 ml = *reinterpret_cast<const f32x4 *>(part_ml + (base + (int64_t)s * num_heads) * 4);
        if (ml[1] > 0.0f) {
            const float f = exp2f(ml[0] - M);
            L += ml[1] * f;
            Le += ml[2] * f;
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int64_t obase = ((int64_t)r * num_heads + h) * V;
    for (int v = 4 * threadIdx.x; v < V; v += 4 * blockDim.x) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int s = 0; s < splits; ++s) {
            const int64_t ps = base + (int64_t)s * num_heads;
            const f32x4 ml = *reinterpret_cast<const f32x4 *>(part_ml + ps * 4);
            if (ml[1] > 0.0f) acc += exp2f(ml[0] - M) * *reinterpret_cast<const f32x4 *>(part_o + ps * V + v);
        }
        acc *= inv;
        if (out_bf16) {
            uint32_t *ob = reinterpret_cast<uint32_t *>(out) + ((obase + v) >> 1);
            ob[0] = pack_bf16x2(acc[0], acc[1]);
            ob[1] = pack_bf16x2(acc[2], acc[3]);
        } else {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + obase + v) = acc;
        }
    }
    if (lse && threadIdx.x == 0)
        lse[(int64_t)r * num_heads + h] = L > 0.0f ? (M + log2f(Le)) * 0.69314718055994531f : -INFINITY;
}

}  // namespace sa
