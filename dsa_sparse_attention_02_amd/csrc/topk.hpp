// Per-row top-k selection (gfx950).
//
// Keeps, for every query row, the k keys that come first under (score
// descending, position ascending) among its n visible keys, and writes their
// positions in ascending order (all n positions when n <= k, -1 padded).  The
// pages ask for top-k over long rows that stays fast and stable at large k
// ("Day-0 Adaptation for LLMs: Implementing Sparse Attention and Low-Precision
// Weights", section III.1) and report that grouping the selection by row,
// buffering in on-chip shared memory and vectorised loads removed the thread
// divergence of the data-dependent selection ("Engineering Practices for Day-0
// Adaptation of Million-Token Context Models on Domestic AI Chips", Four Key
// Layers item 1).  On gfx950 that becomes one 1024-thread workgroup per row with
// LDS histograms and 16-byte score loads:
//
//  1. Radix select on order-preserving uint32 keys, 11 + 11 + 10 bits: each pass
//     histograms (in LDS) the next digit of the keys that match the prefix found
//     so far, and a suffix scan of the histogram picks the digit at which the
//     running count from the top reaches k.  After three passes the exact
//     threshold key T is known, with `gt` keys strictly above it and need = k - gt
//     keys equal to T still to take.
//  2. One ordered pass: a key is kept when key > T, or key == T and fewer than
//     `need` equal keys precede it.  With G and E the counts of greater and equal
//     keys before position s, a kept key lands at output slot G + min(E, need), so a
//     single block-wide exclusive scan of packed (G, E) counts yields ascending
//     output with the lowest-position tie-break, deterministically.
#pragma once

#include "device_common.hpp"

namespace sa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// inclusive scan over the block; returns the inclusive prefix, *total = block sum
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t *wsum, uint32_t *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(v, d);
        if (lane >= d) v += o;
    }
    if (lane == 63) wsum[wave] = v;
    __syncthreads();
    if (wave == 0) {
        uint32_t x = lane < kTopkWaves ? wsum[lane] : 0u;
#pragma unroll
        for (int d = 1; d < kTopkWaves; d <<= 1) {
            const uint32_t o = __shfl_up(x, d);
            if (lane >= d) x += o;
        }
        if (lane < kTopkWaves) wsum[lane] = x;  // inclusive wave totals
    }
    __syncthreads();
    const uint32_t before = wave ? wsum[wave - 1] : 0u;
    *total = wsum[kTopkWaves - 1];
    __syncthreads();  // wsum is reused by the next call
    return v + before;
}

// Rows r = blockIdx.x.  n = ctx_lens[r] when ctx_lens is non-null (decode),
// else n = n_base + r + 1 (prefill row at position n_base + r).
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(
    const float *__restrict__ scores, int64_t score_stride, const int32_t *__restrict__ ctx_lens,
    int n_base, int k, int32_t *__restrict__ out)
{
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[kTopkWaves];
    __shared__ uint32_t pick[2];

    const int r = blockIdx.x;
    const int n = ctx_lens ? ctx_lens[r] : n_base + r + 1;
    int32_t *o = out + (int64_t)r * k;
    const int tid = threadIdx.x;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
        return;
    }
    const float *sr = scores + (int64_t)r * score_stride;
    const int n4 = n & ~3;

    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < nbins; i += kTopkThreads) hist[i] = 0;
        if (tid == 0) {
            pick[0] = 0;
            pick[1] = 0;
        }
        __syncthreads();
        for (int i = 4 * tid; i < n4; i += 4 * kTopkThreads) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sr + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(v[e]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1u);
            }
        }
        for (int i = n4 + tid; i < n; i += kTopkThreads) {
            const uint32_t key = score_key(sr[i]);
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        // thread u owns bins [nbins-2-2u, nbins-1-2u] (2048 bins) or bin nbins-1-u
        // (1024 bins), so a prefix scan over u is a suffix scan over bins.
        const int per = nbins / kTopkThreads;
        const int hi_bin = nbins - 1 - per * tid;
        uint32_t mine = 0;
        for (int e = 0; e < per; ++e) mine += hist[hi_bin - e];
        uint32_t tot;
        const uint32_t incl = block_inclusive_scan(mine, wsum, &tot);
        uint32_t above = incl - mine;  // keys in bins above this thread's bins
        for (int e = 0; e < per; ++e) {
            const uint32_t c = hist[hi_bin - e];
            if (above < need && above + c >= need) {
                pick[0] = (uint32_t)(hi_bin - e);
                pick[1] = above;
            }
            above += c;
        }
        __syncthreads();
        const uint32_t digit = pick[0];
        need -= pick[1];
        prefix |= digit << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
        __syncthreads();  // pick[] and hist[] are rewritten next pass
    }
    const uint32_t T = prefix;

    // ordered compaction, 4 consecutive keys per thread per tile
    uint32_t base_g = 0, base_e = 0;
    for (int t0 = 0; t0 < n; t0 += 4 * kTopkThreads) {
        const int i0 = t0 + 4 * tid;
        uint32_t kk[4];
        if (i0 + 3 < n) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sr + i0);
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[e] = score_key(v[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) kk[e] = (i0 + e < n) ? score_key(sr[i0 + e]) : 0u;
        }
        uint32_t cg = 0, ce = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool valid = i0 + e < n;
            cg += (valid && kk[e] > T);
            ce += (valid && kk[e] == T);
        }
        const uint32_t packed = (cg << 16) | ce;
        uint32_t tot;
        const uint32_t excl = block_inclusive_scan(packed, wsum, &tot) - packed;
        uint32_t G = base_g + (excl >> 16), E = base_e + (excl & 0xFFFFu);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (i0 + e >= n) break;
            // slots stay below k by construction; the bound also holds if
            // inconsistent keys (NaN scores) ever broke the counting
            if (kk[e] > T) {
                const uint32_t slot = G + min(E, need);
                if (slot < (uint32_t)k) o[slot] = i0 + e;
                ++G;
            } else if (kk[e] == T) {
                if (E < need && G + E < (uint32_t)k) o[G + E] = i0 + e;
                ++E;
            }
        }
        base_g += tot >> 16;
        base_e += tot & 0xFFFFu;
    }
}

}  // namespace sa
