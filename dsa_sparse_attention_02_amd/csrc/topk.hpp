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
__device__ __forceinline__ void topk_radix_row(TopkShared &sh, const float *__restrict__ sr, int n, int k,
                                               int32_t *__restrict__ o)
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
    // exclusive block scan of cnt with one barrier (wsum is not used after this)
    const int lane = tid & 63, wave = tid >> 6;
    uint32_t incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t x = __shfl_up(incl, d);
        if (lane >= d) incl += x;
    }
    if (lane == 63) sh.wsum[wave] = incl;
    __syncthreads();
    uint32_t pos = incl - cnt;
    for (int w = 0; w < wave; ++w) pos += sh.wsum[w];
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

// The row's score range [lo, hi] from the (min, max) of its nmm tiles, in every
// thread.
__device__ __forceinline__ void row_range(TopkShared &sh, const f32x2 *__restrict__ mm, int nmm, float &lo, float &hi)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    lo = INFINITY;
    hi = -INFINITY;
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
    __syncthreads();
    lo = sh.red[0][0];
    hi = sh.red[1][0];
    for (int w = 1; w < kTopkWaves; ++w) {
        lo = fminf(lo, sh.red[0][w]);
        hi = fmaxf(hi, sh.red[1][w]);
    }
    __syncthreads();  // red is reused
}

// kBins equal-width bins over [lo, hi]: monotone non-decreasing in the score
// (every step is monotone in fp32); a zero or non-finite span puts every score
// in bin 0.
struct ScoreBins {
    float lo, scale;
    __device__ __forceinline__ ScoreBins(float lo_, float hi_)
    {
        lo = lo_;
        const float span = hi_ - lo_;
        scale = (span > 0.0f && span < INFINITY) ? (float)kBins / span : 0.0f;
    }
    __device__ __forceinline__ uint32_t operator()(float x) const
    {
        return (uint32_t)fminf(fmaxf((x - lo) * scale, 0.0f), (float)(kBins - 1));
    }
};

// (order-preserving key, position) as one 64-bit word: larger means kept first
__device__ __forceinline__ uint64_t cand_word(float x, int i)
{
    return ((uint64_t)score_key(x) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)i);
}

// 4. The need best of the m candidates in sh.cand, by (key, -position)
// descending, join the bitmap; 5. the bitmap's positions are written in order.
// Up to 64 candidates: wave 0 ranks each against all (lane i holds candidate
// i); more: a bitonic sort over the block.
__device__ __forceinline__ void resolve_emit(TopkShared &sh, int m, uint32_t need, int words, int k,
                                             int32_t *__restrict__ o)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (m <= 64) {  // block-uniform
        if (wv == 0) {
            const uint64_t mine = lane < m ? sh.cand[lane] : 0;
            int rank = 0;  // candidates ahead of mine (keys are distinct: positions differ)
            for (int j = 0; j < m; ++j) rank += __shfl(mine, j) > mine;
            if (lane < m && rank < (int)need) {
                const int pos = (int)(0xFFFFFFFFu - (uint32_t)mine);
                atomicOr(&sh.bitmap[pos >> 5], 1u << (pos & 31));
            }
        }
        __syncthreads();
        topk_emit(sh, words, k, o, tid);
        return;
    }
    int P = 1;
    while (P < m) P <<= 1;
    for (int i = m + tid; i < P; i += kTopkThreads) sh.cand[i] = 0;
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

// Steps 2-5 of the threshold path for a row of n keys (k < n <= kBitmapKeys)
// whose score range is [lo, hi].
__device__ __forceinline__ void threshold_row(TopkShared &sh, const float *__restrict__ sr, int n, int k,
                                              int32_t *__restrict__ o, float lo, float hi)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int n4 = n & ~3;
    const ScoreBins bin_of(lo, hi);
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();

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
                if (slot < (uint32_t)kCandCap) sh.cand[slot] = cand_word(x, i);
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
    resolve_emit(sh, (int)m, need, words, k, o);
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
    const int tid = threadIdx.x;
    if (n <= k) {
        for (int i = tid; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
        return;
    }
    const float *sr = scores + (int64_t)r * score_stride;
    if (n > kBitmapKeys) {
        topk_radix_row(sh, sr, n, k, o);
        return;
    }
    // 1. score range of the row
    float lo, hi;
    row_range(sh, tile_mm + (int64_t)r * mm_stride, mm_per_row ? mm_per_row : (n + 31) / 32, lo, hi);
    threshold_row(sh, sr, n, k, o, lo, hi);
}

// ------------------------------------------------- one pass for decode rows --
// Decode rows take one workgroup each, so a batch of long rows keeps one
// workgroup per row busy through both passes of the threshold path; there the
// per-key work (a histogram atomic per key, then a ballot per key) and the
// latency of each dependent step set the time.  This path reads each row once
// and does per-key work only on a small candidate set:
//  a. Estimate: the row's tile ranges and the keys of every 16th 32-key tile
//     (1/16 of the row) are loaded together; the sample is histogrammed into
//     the row's 2048 bins, and the bound T_f is set at the lower edge of the
//     bin above which the sample holds about 1.25 k/16 + 16 keys.
//  b. Gather: one pass over the row (GR 4 KB rounds per wave in flight)
//     writes the position of every key >= T_f to LDS (kCompCap at most).
//  c. If at least k and at most kCompCap keys were gathered, the top k of the
//     row are the top k of the gathered set (its k-th best key is >= T_f, so
//     every kept key was gathered): their scores are read back, and bins over
//     [T_f, hi], a suffix scan, a bitmap of the keys above the threshold bin
//     and a resolution of that bin's candidates give them, as in the threshold
//     path.  Otherwise (a sample that misjudged the row) the row takes the
//     threshold path from its scores.
// On MI355X a workgroup reads a row's scores at about 25 bytes per clock
// however many loads it keeps in flight, so this path gains on long rows with
// a small k / n (one pass instead of two) and loses on short ones (its fixed
// steps); which rows take it is a run-time choice (onepass_min).
// Either way the kept set is the exact top-k with the lowest-position
// tie-break; the sample only decides how much work finds it.
constexpr int kCompCap = 8192;  // positions gathered in LDS

constexpr int kSampleGap = 512;   // keys from one sample tile to the next

struct TopkGatherShared {
    TopkShared sh;
    int32_t cp[kCompCap];
    uint32_t ngather, ncand;
};

// pick_bin over kBins bins by wave 0 alone (lane l sums the 32 bins
// [kBins - 32 (l + 1), kBins - 32 l), a wave scan runs from the top bins down),
// then one barrier.  need <= the histogram's total.
template <class Shared>  // (TopkShared, or any with hist[kBins] and pick[3])
__device__ __forceinline__ void pick_bin_wave(Shared &sh, uint32_t need, uint32_t &bin, uint32_t &above,
                                              uint32_t &count)
{
    static_assert(kBins == 64 * 32, "32 bins per lane");
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid < 64) {
        const int base = kBins - 32 * (lane + 1);
        uint32_t c[32];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(&sh.hist[base + 4 * q]);
#pragma unroll
            for (int e = 0; e < 4; ++e) c[4 * q + e] = x[e];
        }
        uint32_t sum = 0;
#pragma unroll
        for (int e = 0; e < 32; ++e) sum += c[e];
        uint32_t incl = sum;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t x = __shfl_up(incl, d);
            if (lane >= d) incl += x;
        }
        if (lane == 0) {
            sh.pick[0] = 0;
            sh.pick[1] = 0;
            sh.pick[2] = 0;
        }
        uint32_t ab = incl - sum;
        if (ab < need && incl >= need) {  // (one lane)
            bool found = false;
#pragma unroll
            for (int e = 31; e >= 0; --e) {
                if (!found && ab + c[e] >= need) {
                    sh.pick[0] = (uint32_t)(base + e);
                    sh.pick[1] = ab;
                    sh.pick[2] = c[e];
                    found = true;
                }
                ab += c[e];
            }
        }
    }
    __syncthreads();
    bin = sh.pick[0];
    above = sh.pick[1];
    count = sh.pick[2];
}

// Rows of fewer than onepass_min keys take the threshold path.  GR: gather
// rounds whose loads are in flight together per wave (the loop's unroll).
template <int GR>
__global__ __launch_bounds__(kTopkThreads) void topk_decode_kernel(
    const float *__restrict__ scores, int64_t score_stride, const f32x2 *__restrict__ tile_mm, int64_t mm_stride,
    const int32_t *__restrict__ ctx_lens, int k, int onepass_min, int32_t *__restrict__ out, const AppendArgs ap)
{
    __shared__ TopkGatherShared g;
    TopkShared &sh = g.sh;
    const int r = blockIdx.x;
    append_rows(ap, r, threadIdx.x, kTopkThreads);  // (row r = sequence r; before the attention reads it)
    const int n = ctx_lens[r];
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
    const f32x2 *mm = tile_mm + (int64_t)r * mm_stride;
    const int nmm = (n + 31) / 32;
    if (n < onepass_min || n <= 2 * k || 2 * k > kCompCap) {  // (also where the gathered set would be large)
        float lo, hi;
        row_range(sh, mm, nmm, lo, hi);
        threshold_row(sh, sr, n, k, o, lo, hi);
        return;
    }

    // a. range and sample.  Sample tile j holds keys [512 j, 512 j + 32);
    // thread t takes 4 of them in tile (t >> 3) + 128 q, q < 4 (512 tiles cover
    // kBitmapKeys).  The first four tile ranges and the sample pieces of every
    // thread load together.  (A score row is allocated to a multiple of 64
    // keys, n64 here, so a 16-byte piece that starts below n is read whole;
    // keys at n and beyond are never counted.)
    const int wvu = __builtin_amdgcn_readfirstlane(wv);  // (wave-uniform, in a scalar register)
    const int n64 = (n + 63) & ~63;
    static_assert(4 * (kTopkThreads / 8) * kSampleGap >= kBitmapKeys, "one batch of sample loads");
    const int ns = (n + kSampleGap - 1) / kSampleGap;
    const int sx = 4 * (tid & 7);
    f32x2 mv[4];
    f32x4 sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int t = tid + kTopkThreads * q;
        mv[q] = t < nmm ? mm[t] : f32x2{INFINITY, -INFINITY};
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {  // (tiles past the last are read as the last one, and not counted)
        const int j = min((tid >> 3) + (kTopkThreads / 8) * q, ns - 1);
        sv[q] = *reinterpret_cast<const f32x4 *>(sr + kSampleGap * j + sx);
    }
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        lo = fminf(lo, mv[q][0]);
        hi = fmaxf(hi, mv[q][1]);
    }
    for (int t = tid + 4 * kTopkThreads; t < nmm; t += kTopkThreads) {  // (rows over 131072 keys)
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
    if (tid == 0) {
        g.ngather = 0;
        g.ncand = 0;
    }
    __syncthreads();
    lo = sh.red[0][0];
    hi = sh.red[1][0];
    for (int w = 1; w < kTopkWaves; ++w) {
        lo = fminf(lo, sh.red[0][w]);
        hi = fmaxf(hi, sh.red[1][w]);
    }
    const ScoreBins bin_of(lo, hi);
    auto sample_count = [&](const f32x4 &v, int j) {
        if (j < ns) {
            const int i0 = kSampleGap * j + sx;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i0 + e < n) atomicAdd(&sh.hist[bin_of(v[e])], 1u);
        }
    };
#pragma unroll
    for (int q = 0; q < 4; ++q) sample_count(sv[q], (tid >> 3) + (kTopkThreads / 8) * q);
    __syncthreads();
    // keys in the sample: 32 per sample tile, the last one cut at n
    const int nsamp = 32 * (ns - 1) + min(32, n - kSampleGap * (ns - 1));
    const uint32_t want = (uint32_t)min(nsamp, (int)ceilf(1.25f * (float)k * (float)nsamp / (float)n) + 16);
    uint32_t b, above, cnt;
    pick_bin_wave(sh, want, b, above, cnt);
    const float tf = bin_of.scale > 0.0f ? lo + (float)b / bin_of.scale : lo;

    // b. gather the positions of the keys >= T_f.  Round c covers keys
    // [1024 c, 1024 c + 1024): lane l the 16-byte pieces at 4 l + 256 u
    // (u < 4).  A wave scan of the lanes' counts (five ballots) places them;
    // one LDS atomic per round reserves the wave's slots.  GR rounds' loads are
    // in flight per wave.
    const int nch = (n + 1023) / 1024;
    auto load = [&](f32x4 (&v)[4], int c) {  // (pieces past the row's last one re-read it: never gathered)
        const int i0 = 1024 * c + 4 * lane;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4 *>(sr + min(i0 + 256 * u, n64 - 4));
    };
    auto gather_round = [&](const f32x4 (&v)[4], int c, auto full) {
        const int i0 = 1024 * c + 4 * lane;
        uint32_t bits = 0;  // bit 4 u + e: key i0 + 256 u + e is gathered
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                bits |= (v[u][e] >= tf && (decltype(full)::value || i0 + 256 * u + e < n)) ? 1u << (4 * u + e) : 0u;
        const uint32_t cnt = (uint32_t)__popc(bits);  // <= 16: five bits
        uint32_t pre = 0, tot = 0;
#pragma unroll
        for (int bt = 0; bt < 5; ++bt) {
            const uint64_t mb = __ballot((cnt >> bt) & 1u);
            pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u)) << bt;
            tot += (uint32_t)__popcll(mb) << bt;
        }
        if (tot == 0) return;  // (wave-uniform)
        uint32_t base = 0;
        if (lane == 0) base = atomicAdd(&g.ngather, tot);
        uint32_t slot = (uint32_t)__builtin_amdgcn_readfirstlane((int)base) + pre;
        while (bits) {
            const int j = __builtin_ctz(bits);
            bits &= bits - 1;
            if (slot < (uint32_t)kCompCap) g.cp[slot] = i0 + 256 * (j >> 2) + (j & 3);
            ++slot;
        }
    };
    for (int c = wvu; c < nch; c += GR * kTopkWaves) {
        f32x4 v[GR][4];
#pragma unroll
        for (int q = 0; q < GR; ++q)  // (a round past the last re-reads the last one, and is not gathered)
            load(v[q], min(c + q * kTopkWaves, nch - 1));
#pragma unroll
        for (int q = 0; q < GR; ++q) {
            const int cq = c + q * kTopkWaves;
            if (cq >= nch) break;  // (wave-uniform)
            if (1024 * cq + 1024 <= n) gather_round(v[q], cq, std::true_type{});
            else gather_round(v[q], cq, std::false_type{});
        }
    }
    __syncthreads();
    const int mc = (int)g.ngather;
    if (mc < k || mc > kCompCap) {  // (block-uniform) the sample misjudged the row
        threshold_row(sh, sr, n, k, o, lo, hi);
        return;
    }

    // c. the top k of the gathered keys
    constexpr int G = kCompCap / kTopkThreads;
    float xv[G];
    int pv[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        const int i = tid + kTopkThreads * q;
        pv[q] = i < mc ? g.cp[i] : 0;
        xv[q] = i < mc ? sr[pv[q]] : 0.0f;
    }
    const ScoreBins bin2(tf > lo ? tf : lo, hi);
    const int words = (n + 31) / 32;
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    for (int i = tid; i < words; i += kTopkThreads) sh.bitmap[i] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < G; ++q)
        if (tid + kTopkThreads * q < mc) atomicAdd(&sh.hist[bin2(xv[q])], 1u);
    __syncthreads();
    uint32_t tbin, m;
    pick_bin_wave(sh, (uint32_t)k, tbin, above, m);
    if (m > (uint32_t)kCandCap) {  // block-uniform
        topk_radix_row(sh, sr, n, k, o);
        return;
    }
#pragma unroll
    for (int q = 0; q < G; ++q) {
        if (tid + kTopkThreads * q >= mc) continue;
        const uint32_t bi = bin2(xv[q]);
        if (bi > tbin) {
            atomicOr(&sh.bitmap[pv[q] >> 5], 1u << (pv[q] & 31));
        } else if (bi == tbin) {
            const uint32_t slot = atomicAdd(&g.ncand, 1u);  // < m: the histogram counted them
            if (slot < (uint32_t)kCandCap) sh.cand[slot] = cand_word(xv[q], pv[q]);
        }
    }
    __syncthreads();
    resolve_emit(sh, (int)m, (uint32_t)k - above, words, k, o);
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

// ---------------------------------------------- one pass for very long rows --
// Rows over kBitmapKeys keys (with 2 k <= kLongCap, up to kMaxLongChunks
// chunks) in two launches instead of the many-workgroup radix select's nine:
//  1. per 16384-key chunk (topk_long_gather_kernel): the bound T_f of the row
//     is set from a sample, one 32-key tile in every kLongGap keys (1/64 of the
//     row), histogrammed over its own range, where about 1.25 k/64 + 16 sample
//     keys lie above it.  Every chunk of the row computes the same bound from
//     the same sample (chunk 0 stores it); its own keys are read meanwhile.
//     The chunk's keys >= T_f are then written, as (order-preserving key,
//     position) words in ascending position order, to the chunk's own segment
//     of kLongSeg words, with their count and largest key;
//  2. per row (topk_long_select_kernel): if the segments hold at least k and
//     at most kLongCap keys, the top k of the row are the top k of those keys
//     (the k-th best key of the row is >= T_f).  Each thread takes 8
//     consecutive ones of them into registers; they are binned over [T_f, max],
//     the threshold bin found by a suffix scan and its keys ranked exactly
//     (score, then the lower position); the kept keys are compacted in order
//     into the output, which is thus ascending without a sort.  Otherwise the
//     row takes the radix path of one workgroup (exact; slow on such rows, and
//     only where the sample misjudged the row or scores tie massively).
// The segments take 4 bytes per key of the row (8 per gathered key, room for
// half of each chunk), as much as its scores.
constexpr int kLongCap = 8192;        // gathered keys a row may select from
constexpr int kMaxLongChunks = 1024;  // 16384-key chunks a row may have (16M keys)
constexpr int kLongGap = 2048;        // keys from one sample tile to the next
constexpr int kLongSeg = kLongCap;    // gathered keys a chunk may hold (more than this: more than kLongCap)
constexpr int kLongPerThread = kLongCap / kTopkThreads;  // gathered keys per selecting thread

struct LongRowState {
    float tf;  // the bound
    uint32_t pad[3];
};

struct LongGatherShared {
    uint32_t hist[kBins];
    uint32_t pick[4];
    float red[2][kTopkWaves];
    uint32_t wtot[kTopkWaves], wmax[kTopkWaves];
};

// inverse of score_key
__device__ __forceinline__ float key_score(uint32_t key)
{
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// The bound T_f of a row of n > k keys (every thread gets it).  Sample tile j:
// keys [kLongGap j, kLongGap j + 32), tile entry kLongGap j / 32 of the ranges;
// thread t reads 4 keys of tile (t >> 3) + 128 q.  (A score row is allocated
// to a multiple of 64 keys, so a 16-byte piece of a tile that starts below n
// is read whole; keys at n and beyond are never counted.)
__device__ __forceinline__ float long_row_bound(LongGatherShared &sh, const float *__restrict__ sr,
                                                const f32x2 *__restrict__ mm, int n, int k)
{
    static_assert(kTopkThreads == 1024, "128 sample tiles per 4-load round");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int ns = (n + kLongGap - 1) / kLongGap;
    const int sx = 4 * (tid & 7), j0 = tid >> 3;
    // the first round's samples are read before the range is known (rows of up
    // to 512 tiles take one round; tiles past the last are read as the last one,
    // and not counted)
    f32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4 *>(sr + (int64_t)kLongGap * min(j0 + 128 * q, ns - 1) + sx);
    float lo = INFINITY, hi = -INFINITY;
    for (int j = tid; j < ns; j += kTopkThreads) {
        const f32x2 m = mm[(int64_t)j * (kLongGap / 32)];
        lo = fminf(lo, m[0]);
        hi = fmaxf(hi, m[1]);
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
    const ScoreBins bin_of(lo, hi);
    for (int jr = j0;;) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int j = jr + 128 * q, i0 = kLongGap * j + sx;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j < ns && i0 + e < n) atomicAdd(&sh.hist[bin_of(v[q][e])], 1u);
        }
        jr += 512;
        if (jr >= ns) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4 *>(sr + (int64_t)kLongGap * min(jr + 128 * q, ns - 1) + sx);
    }
    __syncthreads();
    const int nsamp = 32 * (ns - 1) + min(32, n - kLongGap * (ns - 1));
    const uint32_t want = (uint32_t)min(nsamp, (int)ceilf(1.25f * (float)k * (float)nsamp / (float)n) + 16);
    uint32_t b, above, cnt;
    pick_bin_wave(sh, want, b, above, cnt);
    return bin_of.scale > 0.0f ? lo + (float)b / bin_of.scale : lo;
}

// Chunk c of row r: keys [16384 c, 16384 c + 16384); wave w takes keys
// [1024 w, 1024 w + 1024) of it, lane l the 16 consecutive keys 16 l ..
// (four 16-byte loads), so lane order, then wave order, is position order.
// seg: [rows][chunks][kLongSeg] words; seg_info: [rows][chunks] (count, largest key).
// Chunk 0 of each row also writes the row's new cache entries (before the
// attention reads them) and the whole row's positions when it has <= k keys.
__global__ __launch_bounds__(kTopkThreads) void topk_long_gather_kernel(
    const float *__restrict__ scores, int64_t score_stride, const f32x2 *__restrict__ tile_mm, int64_t mm_stride,
    const int32_t *__restrict__ ctx_lens, int k, int32_t *__restrict__ out, LongRowState *__restrict__ state,
    uint64_t *__restrict__ seg, uint2 *__restrict__ seg_info, const AppendArgs ap)
{
    __shared__ LongGatherShared sh;
    const int r = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0) append_rows(ap, r, tid, kTopkThreads);
    const int n = ctx_lens[r];
    const int c0 = blockIdx.x * kMbChunk;
    if (n <= k) {  // (block-uniform) the whole row
        if (blockIdx.x == 0) {
            int32_t *o = out + (int64_t)r * k;
            for (int i = tid; i < k; i += kTopkThreads) o[i] = i < n ? i : -1;
        }
        return;
    }
    if (c0 >= n) return;  // (block-uniform)
    static_assert(kMbChunk == 1024 * kTopkWaves, "one 1024-key round per wave");
    const float *sr = scores + (int64_t)r * score_stride;
    const int n64 = (n + 63) & ~63;
    const int i0 = c0 + 1024 * wv + 16 * lane;
    f32x4 v[4];  // (pieces past the row's allocation re-read its last one: never gathered)
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const f32x4 *>(sr + min(i0 + 4 * u, n64 - 4));
    const float tf = long_row_bound(sh, sr, tile_mm + (int64_t)r * mm_stride, n, k);
    if (blockIdx.x == 0 && tid == 0) state[r] = LongRowState{tf, {0u, 0u, 0u}};
    uint32_t bits = 0, kmax = 0;  // gathered keys (bit j: key i0 + j); the largest one's order-preserving key
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool c = v[u][e] >= tf && i0 + 4 * u + e < n;
            bits |= c ? 1u << (4 * u + e) : 0u;
            kmax = c ? max(kmax, score_key(v[u][e])) : kmax;
        }
    const uint32_t cnt = (uint32_t)__popc(bits);  // <= 16: five bits
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bt = 0; bt < 5; ++bt) {
        const uint64_t mb = __ballot((cnt >> bt) & 1u);
        pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u)) << bt;
        tot += (uint32_t)__popcll(mb) << bt;
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, d));
    if (lane == 0) {
        sh.wtot[wv] = tot;
        sh.wmax[wv] = kmax;
    }
    __syncthreads();
    uint32_t slot = pre;
    for (int w = 0; w < wv; ++w) slot += sh.wtot[w];
    uint64_t *sg = seg + ((int64_t)r * gridDim.x + blockIdx.x) * kLongSeg;
    while (bits) {
        const int j = __builtin_ctz(bits);
        bits &= bits - 1;
        const int ju = j >> 2, je = j & 3;  // key j of the lane's 16, picked from registers
        float xu[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) xu[u] = je == 0 ? v[u][0] : je == 1 ? v[u][1] : je == 2 ? v[u][2] : v[u][3];
        const float x = ju == 0 ? xu[0] : ju == 1 ? xu[1] : ju == 2 ? xu[2] : xu[3];
        if (slot < (uint32_t)kLongSeg) sg[slot] = cand_word(x, i0 + j);
        ++slot;
    }
    if (tid == 0) {
        uint32_t all = 0, mx = 0;
        for (int w = 0; w < kTopkWaves; ++w) {
            all += sh.wtot[w];
            mx = max(mx, sh.wmax[w]);
        }
        seg_info[(int64_t)r * gridDim.x + blockIdx.x] = uint2{all, mx};
    }
}

__global__ __launch_bounds__(kTopkThreads) void topk_long_select_kernel(
    const float *__restrict__ scores, int64_t score_stride, const int32_t *__restrict__ ctx_lens, int k, int chunks,
    const LongRowState *__restrict__ state, const uint64_t *__restrict__ seg, const uint2 *__restrict__ seg_info,
    int32_t *__restrict__ out)
{
    __shared__ TopkShared sh;
    __shared__ uint32_t cstart[kMaxLongChunks];  // each chunk's first gathered key
    __shared__ uint32_t info[2], ncand;
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    // (the bound and the first chunk counts are read with n; rows of n <= k
    // have neither, and return)
    const float tf = state[r].tf;
    const uint2 ci0 = wv == 0 ? seg_info[(int64_t)r * chunks + min(lane, chunks - 1)] : uint2{0u, 0u};
    const int n = ctx_lens[r];
    if (n <= k) return;  // (written by the gathering launch)
    const float *sr = scores + (int64_t)r * score_stride;
    int32_t *o = out + (int64_t)r * k;
    const int nch = (n + kMbChunk - 1) / kMbChunk;  // chunks of this row (<= chunks)
    // chunk counts, their prefix and the largest key
    if (wv == 0) {
        uint32_t run = 0, mx = 0;
        for (int c0 = 0; c0 < nch; c0 += 64) {
            const int c = c0 + lane;
            uint2 ci = c0 == 0 ? ci0 : seg_info[(int64_t)r * chunks + min(c, chunks - 1)];
            if (c >= nch) ci = uint2{0u, 0u};
            uint32_t incl = ci.x;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const uint32_t x = __shfl_up(incl, d);
                if (lane >= d) incl += x;
            }
            if (c < nch) cstart[c] = run + incl - ci.x;
            run += __shfl(incl, 63);
            mx = max(mx, ci.y);
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, d));
        if (lane == 0) {
            info[0] = run;
            info[1] = mx;
            ncand = 0;
        }
    }
    for (int i = tid; i < kBins; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    const int mc = (int)info[0];
    if (mc < k || mc > kLongCap) {  // (block-uniform) the sample misjudged the row (no segment overflowed)
        topk_radix_row(sh, sr, n, k, o);
        return;
    }
    // gathered keys [8 t, 8 t + 8) of the row, in position order, to thread t:
    // the chunk holding key 8 t by a binary search of the chunk starts, then on
    static_assert(kLongPerThread == 8, "8 gathered keys per thread");
    const int s0 = kLongPerThread * tid;
    int c = 0;
    if (s0 < mc) {
        int hi = nch;  // the last chunk starting at or below s0 is in [c, hi)
        while (hi - c > 1) {
            const int mid = (c + hi) >> 1;
            if (cstart[mid] <= (uint32_t)s0) c = mid;
            else hi = mid;
        }
    }
    uint64_t w[kLongPerThread];
#pragma unroll
    for (int e = 0; e < kLongPerThread; ++e) {
        const int s = s0 + e;
        w[e] = 0;
        if (s < mc) {
            while (c + 1 < nch && cstart[c + 1] <= (uint32_t)s) ++c;
            w[e] = seg[((int64_t)r * chunks + c) * kLongSeg + (s - (int)cstart[c])];
        }
    }
    const ScoreBins bin2(tf, key_score(info[1]));
    uint32_t bi[kLongPerThread];
#pragma unroll
    for (int e = 0; e < kLongPerThread; ++e) {
        bi[e] = bin2(key_score((uint32_t)(w[e] >> 32)));
        if (s0 + e < mc) atomicAdd(&sh.hist[bi[e]], 1u);
    }
    __syncthreads();
    uint32_t tbin, above, m;
    pick_bin_wave(sh, (uint32_t)k, tbin, above, m);
    if (m > (uint32_t)kCandCap) {  // (block-uniform) massive ties in the threshold bin
        topk_radix_row(sh, sr, n, k, o);
        return;
    }
    // the threshold bin's keys, then the need-th best of them (words are
    // distinct: positions differ)
#pragma unroll
    for (int e = 0; e < kLongPerThread; ++e)
        if (s0 + e < mc && bi[e] == tbin) sh.cand[atomicAdd(&ncand, 1u)] = w[e];  // (< m)
    __syncthreads();
    const uint32_t need = (uint32_t)k - above;
    if (m <= 64) {  // (block-uniform) wave 0 ranks each candidate against all
        if (wv == 0) {
            const uint64_t mine = lane < (int)m ? sh.cand[lane] : 0;
            int rank = 0;
            for (int j = 0; j < (int)m; ++j) rank += __shfl(mine, j) > mine;
            if (lane < (int)m && rank == (int)need - 1) sh.cand[kCandCap - 1] = mine;  // (a slot past m <= 64)
        }
    } else {  // bitonic sort, descending, of the m (<= kCandCap) candidates padded to a power of two
        int P = 1;
        while (P < (int)m) P <<= 1;
        for (int i = (int)m + tid; i < P; i += kTopkThreads) sh.cand[i] = 0;
        __syncthreads();
        for (int size = 2; size <= P; size <<= 1)
            for (int j = size >> 1; j > 0; j >>= 1) {
                for (int i = tid; i < P / 2; i += kTopkThreads) {
                    const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1)), b2 = a | j;
                    const uint64_t x = sh.cand[a], y = sh.cand[b2];
                    if (((a & size) == 0) ? (x < y) : (x > y)) {
                        sh.cand[a] = y;
                        sh.cand[b2] = x;
                    }
                }
                __syncthreads();
            }
    }
    __syncthreads();
    const uint64_t tstar = m <= 64 ? sh.cand[kCandCap - 1] : sh.cand[need - 1];
    // kept: above the threshold bin, or in it and not below the need-th best
    uint32_t kb = 0;
#pragma unroll
    for (int e = 0; e < kLongPerThread; ++e)
        kb |= (s0 + e < mc && (bi[e] > tbin || (bi[e] == tbin && w[e] >= tstar))) ? 1u << e : 0u;
    const uint32_t cnt = (uint32_t)__popc(kb);  // <= 8: four bits
    uint32_t pre = 0, tot = 0;
#pragma unroll
    for (int bt = 0; bt < 4; ++bt) {
        const uint64_t mb = __ballot((cnt >> bt) & 1u);
        pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(mb >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mb, 0u)) << bt;
        tot += (uint32_t)__popcll(mb) << bt;
    }
    if (lane == 0) sh.wsum[wv] = tot;
    __syncthreads();
    uint32_t pos = pre;
    for (int v = 0; v < wv; ++v) pos += sh.wsum[v];
#pragma unroll
    for (int e = 0; e < kLongPerThread; ++e)
        if ((kb >> e) & 1u) {
            if (pos < (uint32_t)k) o[pos] = (int)(0xFFFFFFFFu - (uint32_t)w[e]);
            ++pos;
        }
}

}  // namespace sa
