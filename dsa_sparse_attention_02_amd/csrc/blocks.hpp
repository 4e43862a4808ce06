// Block-granular selection: the index selection keeps whole KV blocks per
// query block ("Day-0 Adaptation: Running Trillion-Parameter Models on
// Domestic AI Accelerators", 3.1: selection chooses the key-value blocks that
// take part for each query block, top-k of them, under a mask, with the same
// block mapping as the attention).  A KV block is a cache block of the
// sequence (logical tokens [j * bs, (j + 1) * bs)).  A query block is one
// decode row, or q_block consecutive prefill rows.
//
//   block score of KV block j for query block G =
//       max over rows i of G and tokens s of block j with s <= pos_i of the
//       token indexer score score_i(s)
//   candidates of G: blocks 0 .. last_G >> bs_log2 (last_G = G's last position)
//   kept: the k candidates of highest block score (ties: lower j), ascending
//   row i attends over the tokens s <= pos_i of its group's kept blocks
//
// The token scores come from the indexer kernels; the block scores feed the
// same top-k kernel as the token path (per-32-candidate score ranges and a
// candidate count per query block); the kept blocks are expanded to token
// positions for the attention kernel.
#pragma once

#include "device_common.hpp"

namespace sa {

constexpr int kBlockScoreThreads = 256;

// grid (query blocks of the launch, tiles of 32 candidate blocks); rows of the
// launch r = 0 .. nrows-1 at position ctx_lens[r] - 1 (decode, q_block = 1) or
// pos0 + r (prefill); query block g holds rows [g * q_block, (g + 1) * q_block).
// Writes ncand[g]; where ncand[g] > k, also the block scores of g's
// candidates (bscore, row stride bstride) and each 32-candidate tile's score
// range (bmm, row stride bmm_stride).  Where ncand[g] <= k every candidate is
// kept and the top-k reads no score, so none is computed.
__global__ __launch_bounds__(kBlockScoreThreads) void block_score_kernel(
    const float *__restrict__ scores, int64_t score_stride, const int32_t *__restrict__ ctx_lens, int pos0,
    int q_block, int nrows, int bs_log2, int k, float *__restrict__ bscore, int64_t bstride, f32x2 *__restrict__ bmm,
    int64_t bmm_stride, int32_t *__restrict__ ncand)
{
    __shared__ float tile[32];
    const int g = blockIdx.x, t = blockIdx.y;
    const int r0 = g * q_block, r1 = min(nrows, r0 + q_block);
    auto pos_of = [&](int r) { return ctx_lens ? ctx_lens[r] - 1 : pos0 + r; };
    const int last = pos_of(r1 - 1);  // rows of a group ascend in position
    const int n = last >= 0 ? (last >> bs_log2) + 1 : 0;
    if (t == 0 && threadIdx.x == 0) ncand[g] = n;
    const int j0 = t * 32;
    if (n <= k || j0 >= n) return;  // (block-uniform)
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int bs = 1 << bs_log2;
    for (int jj = wave; jj < 32; jj += kBlockScoreThreads / 64) {
        const int j = j0 + jj;
        float m = -INFINITY;
        if (j < n) {  // (wave-uniform)
            for (int r = r0; r < r1; ++r) {
                const int s_end = min(pos_of(r), j * bs + bs - 1);  // the row's last visible token of block j
                const float *sr = scores + (int64_t)r * score_stride;
                for (int s = j * bs + lane; s <= s_end; s += 64) m = fmaxf(m, sr[s]);
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d));
        }
        if (lane == 0) tile[jj] = m;
    }
    __syncthreads();
    if (threadIdx.x < 64) {  // wave 0
        const int j = j0 + lane;
        const bool ok = lane < 32 && j < n;
        const float v = ok ? tile[lane] : 0.0f;
        if (ok) bscore[(int64_t)g * bstride + j] = v;
        float lo = ok ? v : INFINITY, hi = ok ? v : -INFINITY;
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) {
            lo = fminf(lo, __shfl_xor(lo, d));
            hi = fmaxf(hi, __shfl_xor(hi, d));
        }
        if (lane == 0) bmm[(int64_t)g * bmm_stride + t] = f32x2{lo, hi};
    }
}

// Row r's token list for the attention: the kept blocks of its query block
// (k entries, ascending, -1 padded) expanded to k << bs_log2 positions,
// ascending; tokens past the row's position and padding blocks give -1, so
// the valid positions form a prefix.
__global__ __launch_bounds__(256) void expand_blocks_kernel(const int32_t *__restrict__ blocks, int k,
                                                            const int32_t *__restrict__ ctx_lens, int pos0,
                                                            int q_block, int bs_log2, int32_t *__restrict__ tokens)
{
    const int r = blockIdx.x;
    const int pos = ctx_lens ? ctx_lens[r] - 1 : pos0 + r;
    const int32_t *bl = blocks + (int64_t)(r / q_block) * k;
    const int kt = k << bs_log2, bmask = (1 << bs_log2) - 1;
    int32_t *o = tokens + (int64_t)r * kt;
    for (int i = threadIdx.x; i < kt; i += blockDim.x) {
        const int b = bl[i >> bs_log2];
        const int s = b >= 0 ? (b << bs_log2) + (i & bmask) : -1;
        o[i] = (s >= 0 && s <= pos) ? s : -1;
    }
}

}  // namespace sa
