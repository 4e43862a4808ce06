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

#include "device_common.hpp"

namespace sa {

// ------------------------------------------------------------------ decode --
// Grid (ceil(max_ctx / (4*keys_per_wave)), batch), 256 threads.  Wave w of
// block x scans keys [(4x+w)*keys_per_wave, +keys_per_wave) of sequence
// blockIdx.y, clipped to its context length, in tiles of 32 keys loaded
// straight from the paged cache into MFMA operands (each key row is one
// contiguous read per lane pair), with the next tile's loads issued before the
// current tile's matrix work.
template <int IDX_DIM, int IDX_TILES>
__global__ __launch_bounds__(256) void idx_score_decode_kernel(
    const uint16_t *__restrict__ idx_k, const int32_t *__restrict__ block_table, int max_blocks,
    int bs_log2, const int32_t *__restrict__ ctx_lens, const uint16_t *__restrict__ idx_q,
    const float *__restrict__ idx_w, int idx_heads, int relu, float *__restrict__ scores,
    int64_t score_stride, int keys_per_wave)
{
    constexpr int KS = IDX_DIM / 16;
    const int b = blockIdx.y;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int ctx = ctx_lens[b];
    const int s_begin = (blockIdx.x * 4 + wave) * keys_per_wave;
    if (s_begin >= ctx) return;  // wave-uniform; the kernel has no barriers
    const int s_end = min(ctx, s_begin + keys_per_wave);

    bf16x8 qa[IDX_TILES][KS];
    float wr[IDX_TILES][16];
#pragma unroll
    for (int t = 0; t < IDX_TILES; ++t) {
        const int head = 32 * t + col;
        const uint16_t *qp = idx_q + ((int64_t)b * idx_heads + head) * IDX_DIM + half * (IDX_DIM / 2);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qa[t][ks] = head < idx_heads ? as_bf16x8(load16(qp + 8 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int hj = 32 * t + acc_row(i, half);
            wr[t][i] = hj < idx_heads ? idx_w[(int64_t)b * idx_heads + hj] : 0.0f;
        }
    }

    const int32_t *tbl = block_table + (int64_t)b * max_blocks;
    const int bmask = (1 << bs_log2) - 1;
    float *out = scores + (int64_t)b * score_stride;

    auto load_tile = [&](int s0, u32x4 (&kb)[KS]) {
        const int s = s0 + col;
        if (s < s_end) {
            const int64_t row = ((int64_t)tbl[s >> bs_log2] << bs_log2) | (s & bmask);
            const uint16_t *kp = idx_k + row * IDX_DIM + half * (IDX_DIM / 2);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kb[ks] = load16(kp + 8 * ks);
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kb[ks] = u32x4{0, 0, 0, 0};
        }
    };

    u32x4 cur[KS], nxt[KS];
    load_tile(s_begin, cur);
    for (int s0 = s_begin; s0 < s_end; s0 += 32) {
        if (s0 + 32 < s_end) load_tile(s0 + 32, nxt);
        f32x16 acc[IDX_TILES];
#pragma unroll
        for (int t = 0; t < IDX_TILES; ++t) acc[t] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int t = 0; t < IDX_TILES; ++t) acc[t] = mfma_32x32x16(qa[t][ks], as_bf16x8(cur[ks]), acc[t]);
        float part = 0.0f;
#pragma unroll
        for (int t = 0; t < IDX_TILES; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float d = acc[t][i];
                if (relu) d = fmaxf(d, 0.0f);
                part = fmaf(wr[t][i], d, part);
            }
        const float tot = part + __shfl_xor(part, 32);
        const int s = s0 + col;
        if (half == 0 && s < s_end) out[s] = tot + 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) cur[ks] = nxt[ks];
    }
}

// ----------------------------------------------------------------- prefill --
// One workgroup of 8 waves owns 16 consecutive query rows (2 per wave) and
// streams every key those rows can see, [0, last row's position], in tiles of
// 32 keys staged once in LDS and read by all 8 waves.  Each wave keeps both of
// its rows' indexer queries in registers, so every key tile feeds
// 2 rows x IDX_TILES x (IDX_DIM/16) MFMAs per wave.  Blocks run heaviest
// (last rows) first.
constexpr int kPrefillRowsPerBlock = 16;

template <int IDX_DIM, int IDX_TILES>
__global__ __launch_bounds__(512) void idx_score_prefill_kernel(
    const uint16_t *__restrict__ idx_k, const int32_t *__restrict__ block_table, int bs_log2,
    const uint16_t *__restrict__ idx_q, const float *__restrict__ idx_w, int idx_heads, int relu,
    int pos0, int nrows, float *__restrict__ scores, int64_t score_stride)
{
    constexpr int KS = IDX_DIM / 16;
    constexpr int ROW_BYTES = IDX_DIM * 2 + 16;  // +16: consecutive keys start 4 banks apart
    constexpr int CHUNKS = 32 * IDX_DIM * 2 / 16;  // 16-byte pieces per key tile
    constexpr int HP = 32 * IDX_TILES;
    __shared__ __attribute__((aligned(16))) uint8_t ktile[2][32 * ROW_BYTES];
    __shared__ __attribute__((aligned(16))) float wts[kPrefillRowsPerBlock][HP];

    const int g = gridDim.x - 1 - blockIdx.x;
    const int r0 = g * kPrefillRowsPerBlock;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int rows_here = min(kPrefillRowsPerBlock, nrows - r0);
    const int nkeys = pos0 + r0 + rows_here;  // keys visible to the block's last row
    const int bmask = (1 << bs_log2) - 1;

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

    // one 16-byte piece of a key tile per thread (threads past CHUNKS idle)
    const int pc = threadIdx.x;
    const int pkey = pc / (IDX_DIM / 8), ppart = pc % (IDX_DIM / 8);
    auto fetch = [&](int kt) -> u32x4 {
        const int s = kt * 32 + pkey;
        if (pc < CHUNKS && s < nkeys) {
            const int64_t row = ((int64_t)block_table[s >> bs_log2] << bs_log2) | (s & bmask);
            return load16(idx_k + row * IDX_DIM + ppart * 8);
        }
        return u32x4{0, 0, 0, 0};
    };
    auto stash = [&](int buf, u32x4 v) {
        if (pc < CHUNKS) *reinterpret_cast<u32x4 *>(&ktile[buf][pkey * ROW_BYTES + ppart * 16]) = v;
    };

    const int ntiles = (nkeys + 31) / 32;
    stash(0, fetch(0));
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        u32x4 nxt = u32x4{0, 0, 0, 0};
        if (kt + 1 < ntiles) nxt = fetch(kt + 1);
        const int s0 = kt * 32;
        if (s0 <= pos[0] || s0 <= pos[1]) {
            bf16x8 kb[KS];
            const uint8_t *kr = &ktile[buf][col * ROW_BYTES + half * IDX_DIM];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) kb[ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kr + 16 * ks));
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
#pragma unroll
                for (int t = 0; t < IDX_TILES; ++t)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&wts[lr][32 * t + 8 * q4 + 4 * half]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float d = acc[t][4 * q4 + e];
                            if (relu) d = fmaxf(d, 0.0f);
                            part = fmaf(w4[e], d, part);
                        }
                    }
                const float tot = part + __shfl_xor(part, 32);
                const int s = s0 + col;
                if (half == 0 && s <= pos[rr]) scores[(int64_t)(r0 + lr) * score_stride + s] = tot + 0.0f;
            }
        }
        if (kt + 1 < ntiles) stash(buf ^ 1, nxt);
        __syncthreads();
    }
}

}  // namespace sa
