// Per-row top-k selection (gfx950).
//
// Keeps, for every query row, the k keys that come first under (score
// descending, position ascending) among its n visible keys, and writes their
// positions in ascending order (all n positions when n <= k, -1 padded).  The
// pages ask for top-k over long rows that stays fast and stable at large k
// ("Day-0 Adaptation for LLMs: Implementing Sparse Attention and Low-Precision
// Weights", section III.1), name sorting or threshold filtering as the two ways
// to select ("Day-0 Adaptation: Running Trillion-Parameter Models on Domestic
// AI Accelerators", section 3.1), and report that grouping the selection by row,
// buffering in on-chip shared memory and vectorised loads removed the thread
// divergence of the data-dependent selection ("Engineering Practices for Day-0
// Adaptation of Million-Token Context Models on Domestic AI Chips", Four Key
// Layers item 1).  On gfx950: one 1024-thread workgroup per row, LDS histograms
// and bitmaps, 16-byte score loads.
//
// Threshold path (rows up to kBitmapKeys keys):
//  1. The scoring kernels leave each 32-key tile's min and max; their reduction
//     gives the row's score range [lo, hi] without touching the scores.
//  2. Pass 1 histograms the scores into 2048 equal-width bins over [lo, hi]
//     (a monotone map, so whole bins are ordered) and a suffix scan finds the bin
//     T_bin holding the k-th largest score: `above` scores lie in higher bins,
//     need = k - above must come from T_bin.
//  3. Pass 2 marks every score of a higher bin in an LDS bitmap of positions and
//     collects T_bin's scores (few: the bin is 1/2048 of the range) as
//     (order-preserving key, position) pairs.
//  4. A bitonic sort of the candidates by (key descending, position ascending)
//     picks the `need` best; their bits join the bitmap.
//  5. Walking the bitmap in order writes exactly k positions, ascending.
// Radix path (longer rows, or more than kCandCap scores in T_bin, e.g. all
// scores equal): three LDS-histogram passes over the order-preserving keys
// (11 + 11 + 10 bits) pin the exact k-th key T; an ordered pass then keeps
// key > T and the first `need` keys equal to T.  With G and E the counts of
// greater and equal keys before a position, a kept key lands at slot
// G + min(E, need), so one block-wide scan of packed (G, E) counts yields
// ascending output with the lowest-position tie-break.
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

constexpr int kBitmapKeys = 1 << 18;  // rows up to 262144 keys take the threshold path
constexpr int kCandCap = 2048;          // candidates resolved in LDS
constexpr int kBins = 2048;

struct TopkShared {
    uint32_t hist[kBins];
    uint32_t wsum[kTopkWaves];
    uint32_t pick[4];
    float red[2][kTopkWaves];
    uint32_t bitmap[kBitmapKeys / 32];
    uint64_t cand[kCandCap];
};

// Finds the bin at which the count of keys in higher bins reaches `need`:
// returns (bin, keys strictly above that bin).  Thread u owns bins
// [nbins - per*(u+1), nbins - per*u) so a prefix scan over u is a suffix scan over bins.
__device__ __forceinline__ void pick_bin(TopkShared &sh, int nbins, uint32_t need, uint32_t &bin, uint32_t &above,
                                         uint32_t &count)
{
    const int tid = threadIdx.x;
    const int per = nbins / kTopkThreads;
    const int hi_bin = nbins - 1 - per * tid;
    if (tid == 0) {
        sh.pick[0] = 0;
        sh.pick[1] = 0;
    }
    uint32_t mine = 0;
    for (int e = 0; e < per; ++e) mine += sh.hist[hi_bin - e];
    uint32_t tot;
    const uint32_t incl = block_inclusive_scan(mine, sh.wsum, &tot);
    uint32_t ab = incl - mine;
    for (int e = 0; e < per; ++e) {
        const uint32_t c = sh.hist[hi_bin - e];
        if (ab < need && ab + c >= need) {
            sh.pick[0] = (uint32_t)(hi_bin - e);
            sh.pick[1] = ab;
            sh.pick[2] = c;
        }
        ab += c;
    }
    __syncthreads();
    bin = sh.pick[0];
    above = sh.pick[1];
    count = sh.pick[2];
    __syncthreads();  // pick[] and hist[] may be rewritten after this
}

// Radix path for one row: exact threshold key by three histogram passes, then
// ordered compaction with the lowest-position tie-break.
__device__ void topk_radix_row(TopkShared &sh, const float *__restrict__ sr, int n, int k, int32_t *__restrict__ o)
{
    const int tid = threadIdx.x;
    const int n4 = n & ~3;
    uint32_t prefix = 0, pmask = 0;
    uint32_t need = (uint32_t)k;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
        const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
        const int nbins = pass == 2 ? 1024 : 2048;
        for (int i = tid; i < nbins; i += kTopkThreads) sh.hist[i] = 0;
        __syncthreads();
        for (int i = 4 * tid; i < n4; i += 4 * kTopkThreads) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(sr + i);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t key = score_key(v[e]);
                if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nbins - 1)], 1u);
            }
        }
        for (int i = n4 + tid; i < n; i += kTopkThreads) {
            const uint32_t key = score_key(sr[i]);
            if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & (nbins - 1)], 1u);
        }
        __syncthreads();
        uint32_t digit, above, cnt;
        pick_bin(sh, nbins, need, digit, above, cnt);
        need -= above;
        prefix |= digit << shift;
        pmask |= (uint32_t)(nbins - 1) << shift;
    }
    const uint32_t T = prefix;

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
        const uint32_t excl = block_inclusive_scan(packed, sh.wsum, &tot) - packed;
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

// 5. The kept positions (set bits of the bitmap) in ascending order: contiguous
// words per thread, a block scan of their bit counts.
__device__ __forceinline__ void topk_emit(TopkShared &sh, int words, int k, int32_t *o, int tid)
{
    const int per = (words + kTopkThreads - 1) / kTopkThreads;
    const int w0 = tid * per, w1 = min(words, w0 + per);
    uint32_t cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sh.bitmap[w]);
    uint32_t tot;
    uint32_t pos = block_inclusive_scan(cnt, sh.wsum, &tot) - cnt;
    for (int w = w0; w < w1; ++w) {
        uint32_t bits = sh.bitmap[w];
        while (bits) {
            const int b = __builtin_ctz(bits);
            bits &= bits - 1;
            if (pos < (uint32_t)k) o[pos] = w * 32 + b;
            ++pos;
        }
    }
}

// Rows r = blockIdx.x.  n = ctx_lens[r] when ctx_lens is non-null (decode),
// else n = p + 1 for a prefill row at position p, found through the piece map
// (rows counted from the launch's first row).  tile_mm holds
// score ranges (min, max) at row stride mm_stride: one per 32-key tile
// (mm_per_row == 0) or mm_per_row entries covering the whole row.
__global__ __launch_bounds__(kTopkThreads) void topk_rows_kernel(
    const float *__restrict__ scores, int64_t score_stride, const f32x2 *__restrict__ tile_mm, int64_t mm_stride,
    int mm_per_row, const int32_t *__restrict__ ctx_lens, const SeqMap rows_map, int k, int32_t *__restrict__ out,
    const AppendArgs ap)
{
    __shared__ TopkShared sh;
    const int r = blockIdx.x;
    append_rows(ap, r, threadIdx.x, kTopkThreads);  // (decode row r = sequence r; before the attention reads it)
    int n;
    if (ctx_lens) {
        n = ctx_lens[r];
    } else {
        const int pc = map_piece(rows_map, r);
        n = rows_map.pos0[pc] + (r - rows_map.row0[pc]) + 1;
    }
    int32_t *o = out + (int64_t)r * k;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
        return;
    }
    const float *sr = scores + (int64_t)r * score_stride;
    if (n > kBitmapKeys) {
        topk_radix_row(sh, sr, n, k, o);
        return;
    }
    const int n4 = n & ~3;

    // 1. score range of the row
    float lo = INFINITY, hi = -INFINITY;
    const f32x2 *mm = tile_mm + (int64_t)r * mm_stride;
    const int nmm = mm_per_row ? mm_per_row : (n + 31) / 32;
    for (int t = tid; t < nmm; t += kTopkThreads) {
        const f32x2 v = mm[t];
        lo = fminf(lo, v[0]);
        hi = fmaxf(hi, v[1]);
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        lo = fminf(lo, __shfl_xor(lo, d));
        hi = fmaxf(hi, __shfl_xor(hi, d));
    }
    if (lane == 0) {
        sh.red[0][wv] = lo;
        sh.red[1][wv] = hi;
    }
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    lo = sh.red[0][0];
    hi = sh.red[1][0];
    for (int w = 1; w < kTopkWaves; ++w) {
        lo = fminf(lo, sh.red[0][w]);
        hi = fmaxf(hi, sh.red[1][w]);
    }
    const float span = hi - lo;
    const float scale = (span > 0.0f && span < INFINITY) ? (float)kBins / span : 0.0f;
    // monotone non-decreasing in the score (all steps are monotone in fp32)
    auto bin_of = [&](float x) -> uint32_t {
        const float f = fminf(fmaxf((x - lo) * scale, 0.0f), (float)(kBins - 1));
        return (uint32_t)f;
    };

    // 2. histogram of the bins (four 16-byte loads in flight per thread)
    constexpr int U = 4;
    const int nU = n & ~(4 * U * kTopkThreads - 1);
    for (int i = 4 * tid; i < nU; i += 4 * U * kTopkThreads) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const f32x4 *>(sr + i + u * 4 * kTopkThreads);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[bin_of(v[u][e])], 1u);
    }
    for (int i = nU + 4 * tid; i < n4; i += 4 * kTopkThreads) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(sr + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) atomicAdd(&sh.hist[bin_of(v[e])], 1u);
    }
    for (int i = n4 + tid; i < n; i += kTopkThreads) atomicAdd(&sh.hist[bin_of(sr[i])], 1u);
    __syncthreads();
    uint32_t tbin, above, m;
    pick_bin(sh, kBins, (uint32_t)k, tbin, above, m);
    const uint32_t need = (uint32_t)k - above;
    if (m > (uint32_t)kCandCap) {  // block-uniform
        topk_radix_row(sh, sr, n, k, o);
        return;
    }

    // 3. bitmap of the positions above T_bin; T_bin's candidates
    const int words = (n + 31) / 32;
    for (int i = tid; i < words; i += kTopkThreads) sh.bitmap[i] = 0;
    if (tid == 0) sh.pick[3] = 0;
    __syncthreads();
    // called by all 64 lanes of a wave together (the ballot needs every lane)
    auto visit = [&](float x, int i, bool valid) {
        const uint32_t bi = bin_of(x);
        if (valid && bi > tbin) atomicOr(&sh.bitmap[i >> 5], 1u << (i & 31));
        const bool c = valid && bi == tbin;
        const uint64_t mask = __ballot(c);
        if (mask) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&sh.pick[3], (uint32_t)__popcll(mask));
            base = __shfl(base, 0);
            if (c) {
                const uint32_t rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                                __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
                const uint32_t slot = base + rank;
                if (slot < (uint32_t)kCandCap)
                    sh.cand[slot] = ((uint64_t)score_key(x) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
            }
        }
    };
    // Wave-uniform loops: a wave covers U x 256 keys per iteration.  The main
    // loop's iterations lie wholly inside the row, so its U loads carry no
    // bounds checks and are all in flight together; the rest goes key by key.
    const int wEnd = n - 4 * (U - 1) * kTopkThreads - 4 * 64;  // last full iteration starts before this
    int wb = 4 * 64 * wv;
    for (; wb < wEnd; wb += 4 * U * kTopkThreads) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = *reinterpret_cast<const f32x4 *>(sr + wb + u * 4 * kTopkThreads + 4 * lane);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i0 = wb + u * 4 * kTopkThreads + 4 * lane;
#pragma unroll
            for (int e = 0; e < 4; ++e) visit(v[u][e], i0 + e, true);
        }
    }
    for (; wb < n; wb += 4 * U * kTopkThreads)
        for (int u = 0; u < U; ++u) {
            const int i0 = wb + u * 4 * kTopkThreads + 4 * lane;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool ok = i0 + e < n;
                visit(ok ? sr[i0 + e] : 0.0f, i0 + e, ok);
            }
        }
    __syncthreads();

    // 4. the need best candidates, by (key, -position) descending.  Up to 64 of
    // them: wave 0 ranks each against all (lane i holds candidate i); more: a
    // bitonic sort over the block.
    if (m <= 64) {  // block-uniform
        if (wv == 0) {
            const uint64_t mine = lane < (int)m ? sh.cand[lane] : 0;
            int rank = 0;  // candidates ahead of mine (keys are distinct: positions differ)
            for (int j = 0; j < (int)m; ++j) rank += __shfl(mine, j) > mine;
            if (lane < (int)m && rank < (int)need) {
                const int pos = (int)(0xFFFFFFFFu - (uint32_t)mine);
                atomicOr(&sh.bitmap[pos >> 5], 1u << (pos & 31));
            }
        }
        __syncthreads();
        topk_emit(sh, words, k, o, tid);
        return;
    }
    int P = 1;
    while (P < (int)m) P <<= 1;
    for (int i = (int)m + tid; i < P; i += kTopkThreads) sh.cand[i] = 0;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1)
        for (int j = size >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < P / 2; i += kTopkThreads) {
                const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1)), b = a | j;
                const uint64_t x = sh.cand[a], y = sh.cand[b];
                const bool desc = (a & size) == 0;  // the final pass (size == P) sorts descending
                if (desc ? (x < y) : (x > y)) {
                    sh.cand[a] = y;
                    sh.cand[b] = x;
                }
            }
            __syncthreads();
        }
    for (int i = tid; i < (int)need; i += kTopkThreads) {
        const int pos = (int)(0xFFFFFFFFu - (uint32_t)sh.cand[i]);
        atomicOr(&sh.bitmap[pos >> 5], 1u << (pos & 31));
    }
    __syncthreads();

    topk_emit(sh, words, k, o, tid);
}

// ------------------------------------------------- many workgroups per row --
// Exact top-k of long rows (a few rows of up to millions of keys) on many
// workgroups per row.  The k-th largest order-preserving score key T is found
// by radix select in three digit passes (key bits 31..21, 20..10, 9..0): each
// pass histograms, over chunks of kMbChunk keys, the next digit of the keys
// that match the digits fixed so far (LDS, then global atomics), and one
// workgroup per row picks the digit where the running count from the top
// reaches the remaining rank.  Afterwards the row keeps every key above T and
// the first `krem` keys equal to T in position order (lowest index first).  A
// count pass gives each chunk its numbers of both; the emit pass writes each
// chunk's kept positions, in ascending order, at the offset the counts of the
// chunks before it give.
constexpr int kMbChunk = 16384;  // keys per workgroup
constexpr int kMbBins = 2048;

struct MbRowState {
    uint32_t prefix, pmask, krem, pad;  // digits fixed so far, their mask, rank left within them
};

__global__ __launch_bounds__(256) void topk_mb_init_kernel(int k, MbRowState *__restrict__ st,
                                                           uint32_t *__restrict__ hist, const AppendArgs ap)
{
    const int r = blockIdx.x;
    append_rows(ap, r, threadIdx.x, 256);
    for (int i = threadIdx.x; i < 3 * kMbBins; i += 256) hist[(int64_t)r * 3 * kMbBins + i] = 0u;
    if (threadIdx.x == 0) st[r] = MbRowState{0u, 0u, (uint32_t)k, 0u};
}

// the four keys of positions i..i+3 of the chunk ending at c1 (zero keys past c1, never counted)
__device__ __forceinline__ void mb_keys4(const float *__restrict__ sr, int i, int c1, uint32_t *key)
{
    if (i + 3 < c1) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(sr + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[e] = score_key(v[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) key[e] = i + e < c1 ? score_key(sr[i + e]) : 0u;
    }
}

template <int PASS>
__global__ __launch_bounds__(kTopkThreads) void topk_mb_hist_kernel(
    const float *__restrict__ scores, int64_t score_stride, const int32_t *__restrict__ ctx_lens, int k,
    const MbRowState *__restrict__ st, uint32_t *__restrict__ hist)
{
    constexpr int SHIFT = PASS == 0 ? 21 : PASS == 1 ? 10 : 0;
    constexpr int NB = PASS == 2 ? 1024 : 2048;
    __shared__ uint32_t h[NB];
    const int r = blockIdx.y, n = ctx_lens[r], tid = threadIdx.x;
    const int c0 = blockIdx.x * kMbChunk;
    if (n <= k || c0 >= n) return;  // block-uniform
    const int c1 = min(n, c0 + kMbChunk);
    const MbRowState s = st[r];
    for (int i = tid; i < NB; i += kTopkThreads) h[i] = 0u;
    __syncthreads();
    const float *sr = scores + (int64_t)r * score_stride;
    for (int i = c0 + 4 * tid; i < c1; i += 4 * kTopkThreads) {
        uint32_t key[4];
        mb_keys4(sr, i, c1, key);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (i + e < c1 && (key[e] & s.pmask) == s.prefix) atomicAdd(&h[(key[e] >> SHIFT) & (NB - 1)], 1u);
    }
    __syncthreads();
    uint32_t *g = hist + ((int64_t)r * 3 + PASS) * kMbBins;
    for (int i = tid; i < NB; i += kTopkThreads)
        if (h[i]) atomicAdd(&g[i], h[i]);
}

template <int PASS>
__global__ __launch_bounds__(kTopkThreads) void topk_mb_pick_kernel(const int32_t *__restrict__ ctx_lens, int k,
                                                                      MbRowState *__restrict__ st,
                                                                      const uint32_t *__restrict__ hist)
{
    constexpr int SHIFT = PASS == 0 ? 21 : PASS == 1 ? 10 : 0;
    constexpr int NB = PASS == 2 ? 1024 : 2048;
    constexpr int PER = NB / kTopkThreads;
    __shared__ uint32_t wsum[kTopkWaves];
    const int r = blockIdx.x, tid = threadIdx.x;
    if (ctx_lens[r] <= k) return;
    const MbRowState s = st[r];
    const uint32_t *g = hist + ((int64_t)r * 3 + PASS) * kMbBins;
    // thread t owns bins NB-1-PER*t .. NB-PER*(t+1), visited from the top
    uint32_t cnt[PER], mine = 0u;
#pragma unroll
    for (int e = 0; e < PER; ++e) mine += cnt[e] = g[NB - 1 - (PER * tid + e)];
    uint32_t tot;
    uint32_t above = block_inclusive_scan(mine, wsum, &tot) - mine;  // keys in the bins above mine
    if (above < s.krem && s.krem <= above + mine) {  // exactly one thread
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            if (s.krem <= above + cnt[e]) {
                const uint32_t b = (uint32_t)(NB - 1 - (PER * tid + e));
                st[r] = MbRowState{s.prefix | (b << SHIFT), s.pmask | ((uint32_t)(NB - 1) << SHIFT), s.krem - above, 0u};
                break;
            }
            above += cnt[e];
        }
    }
}

// per chunk: keys above T, keys equal to T
__global__ __launch_bounds__(kTopkThreads) void topk_mb_count_kernel(
    const float *__restrict__ scores, int64_t score_stride, const int32_t *__restrict__ ctx_lens, int k,
    const MbRowState *__restrict__ st, uint32_t *__restrict__ counts, int chunks)
{
    __shared__ uint32_t wsum[kTopkWaves];
    const int r = blockIdx.y, n = ctx_lens[r], tid = threadIdx.x;
    const int c0 = blockIdx.x * kMbChunk;
    if (n <= k) return;
    uint32_t *cc = counts + ((int64_t)r * chunks + blockIdx.x) * 2;
    if (c0 >= n) {
        if (tid == 0) cc[0] = cc[1] = 0u;
        return;
    }
    const int c1 = min(n, c0 + kMbChunk);
    const uint32_t T = st[r].prefix;
    const float *sr = scores + (int64_t)r * score_stride;
    uint32_t a = 0u, e_ = 0u;
    for (int i = c0 + 4 * tid; i < c1; i += 4 * kTopkThreads) {
        uint32_t key[4];
        mb_keys4(sr, i, c1, key);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = i + e < c1;
            a += ok && key[e] > T;
            e_ += ok && key[e] == T;
        }
    }
    uint32_t ta, te;
    block_inclusive_scan(a, wsum, &ta);
    block_inclusive_scan(e_, wsum, &te);
    if (tid == 0) {
        cc[0] = ta;
        cc[1] = te;
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_mb_emit_kernel(
    const float *__restrict__ scores, int64_t score_stride, const int32_t *__restrict__ ctx_lens, int k,
    const MbRowState *__restrict__ st, const uint32_t *__restrict__ counts, int chunks, int32_t *__restrict__ out)
{
    __shared__ uint32_t wsum[kTopkWaves];
    __shared__ uint32_t base[2];  // this chunk's output offset, ties it keeps
    const int r = blockIdx.y, n = ctx_lens[r], tid = threadIdx.x;
    int32_t *o = out + (int64_t)r * k;
    if (n <= k) {  // the whole row, then padding; the row's workgroups share the k slots
        for (int i = blockIdx.x * kTopkThreads + tid; i < k; i += gridDim.x * kTopkThreads) o[i] = i < n ? i : -1;
        return;
    }
    const int c0 = blockIdx.x * kMbChunk;
    if (c0 >= n) return;
    const int c1 = min(n, c0 + kMbChunk);
    const uint32_t T = st[r].prefix, krem = st[r].krem;
    if (tid == 0) {
        // ties go to the chunks in position order, krem of them in all
        const uint32_t *cc = counts + (int64_t)r * chunks * 2;
        uint32_t off = 0u, ties = 0u;
        for (int c = 0; c < (int)blockIdx.x; ++c) {
            const uint32_t t = min(cc[2 * c + 1], krem > ties ? krem - ties : 0u);
            off += cc[2 * c] + t;
            ties += cc[2 * c + 1];
        }
        base[0] = off;
        base[1] = min(cc[2 * blockIdx.x + 1], krem > ties ? krem - ties : 0u);
    }
    __syncthreads();
    const uint32_t off0 = base[0], my_ties = base[1];
    const float *sr = scores + (int64_t)r * score_stride;
    uint32_t done = 0u, ties_seen = 0u;  // kept and tied keys of the chunk before this round
    for (int i0 = c0; i0 < c1; i0 += 4 * kTopkThreads) {  // block-uniform rounds of 4096 keys
        const int i = i0 + 4 * tid;
        uint32_t key[4] = {0u, 0u, 0u, 0u};
        if (i < c1) mb_keys4(sr, i, c1, key);
        uint32_t nt = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) nt += i + e < c1 && key[e] == T;
        uint32_t tt;
        uint32_t tie_rank = ties_seen + block_inclusive_scan(nt, wsum, &tt) - nt;
        bool keep[4];
        uint32_t nk = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = i + e < c1;
            bool kp = ok && key[e] > T;
            if (ok && key[e] == T) {
                kp = tie_rank < my_ties;
                ++tie_rank;
            }
            keep[e] = kp;
            nk += kp;
        }
        uint32_t tk;
        uint32_t rank = done + block_inclusive_scan(nk, wsum, &tk) - nk;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (keep[e]) {
                if (off0 + rank < (uint32_t)k) o[off0 + rank] = i + e;  // (always, by the counts)
                ++rank;
            }
        done += tk;
        ties_seen += tt;
    }
}

}  // namespace sa
