// libsparse_attn: C ABI (include/sparse_attn.h) over the gfx950 kernels.
//
// Every check runs before the first HIP call; the library never allocates and
// never synchronises (the tuner aside, which measures); its one global state is
// the allocation-free decode's static scratch array and that array's address on
// each device.  Work is queued on the
// caller's stream in this order:
//   decode : indexer scan -> per-row top-k -> split attention -> split merge
//   prefill: per chunk of rows { indexer tile scan -> per-row top-k },
//            then attention over all rows (split + merge only when k > 2048);
//            the rows of one or several sequences, cut into pieces of one
//            sequence each (at most kMapPieces per launch)
// The decode/prefill separation over one cache and one index format follows
// "Day-0 Adaptation: Running Trillion-Parameter Models on Domestic AI
// Accelerators", sections 3.1 and 3.3.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/sparse_attn.h"
#include "attention.hpp"
#include "attention_p4.hpp"
#include "blocks.hpp"
#include "indexer.hpp"
#include "topk.hpp"

namespace {

using namespace sa;

constexpr int kMaxTopk = 16384;
constexpr int kTargetAttnBlocks = 256;        // one attention workgroup per CU of an MI355X
// Default split cap: past about 24 splits per row the merge of the partials
// costs more than the extra workgroups gain (batches of 1, 2 and 4 at long
// contexts ran 3-8% faster at 22 splits than at 32 or 64).
constexpr int kMaxDefaultSplits = 24;
#ifndef SA_COMBINE_HEADS
#define SA_COMBINE_HEADS 8
#endif
constexpr int kCombineHeads = SA_COMBINE_HEADS;  // heads per 512-thread merge workgroup (64 or 128 threads each)
#ifndef SA_TOPK_ONEPASS_MIN_PER_K
#define SA_TOPK_ONEPASS_MIN_PER_K 8
#endif
constexpr int kOnePassMinPerK = SA_TOPK_ONEPASS_MIN_PER_K;  // decode rows of >= this many keys per kept key: one-pass top-k
constexpr int kCUs = 256;                     // compute units of an MI355X
#ifndef SA_SCAN_BLOCKS_PER_CU
#define SA_SCAN_BLOCKS_PER_CU 1
#endif
constexpr int kScanBlocksPerCU = SA_SCAN_BLOCKS_PER_CU;  // persistent scan blocks per CU
constexpr size_t kPrefillScoreBudget = size_t(1) << 30;  // bytes of scores per prefill chunk (enough rows to fill every CU)
constexpr size_t kPrefillPartialBudget = size_t(256) << 20;
constexpr size_t kAlign = 256;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int ilog2(int x)
{
    int l = 0;
    while ((1 << l) < x) ++l;
    return l;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

sa_status check_params(const sa_params *p)
{
    if (!p) return SA_ERR_NULL;
    if (p->num_heads < 1 || p->qk_dim < 1 || p->v_dim < 1 || p->v_dim > p->qk_dim || p->idx_heads < 1 ||
        p->idx_dim < 1 || p->block_size < 1 || p->topk < 1 || !std::isfinite(p->softmax_scale) || !(p->softmax_scale > 0.0f) ||
        (p->idx_relu != 0 && p->idx_relu != 1) || (p->out_dtype != SA_OUT_F32 && p->out_dtype != SA_OUT_BF16))
        return SA_ERR_SHAPE;
    const bool attn_family = (p->qk_dim == 576 && p->v_dim == 512) || (p->qk_dim == 64 && p->v_dim == 64);
    const bool idx_family = p->idx_dim == 128 || p->idx_dim == 32;
    if (!attn_family || !idx_family || p->num_heads > 128 || p->idx_heads > 64 || !is_pow2(p->block_size) ||
        p->block_size > 1024 || p->topk > kMaxTopk)
        return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

sa_status check_cache(const sa_params *p, const sa_paged_cache *c, bool need_kv, bool need_idx, bool need_ctx)
{
    if (!c) return SA_ERR_NULL;
    if ((need_kv && !c->kv) || (need_idx && !c->idx_k) || !c->block_table || (need_ctx && !c->context_lens))
        return SA_ERR_NULL;
    if (c->num_blocks < 1 || c->max_blocks_per_seq < 1) return SA_ERR_SHAPE;
    if (c->num_blocks * (int64_t)p->block_size > INT32_MAX) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

// Attention launch shape: blocks of 32 heads (hb per workgroup), partners per
// block (waves that split the q.k contraction and the value columns) and head
// groups (workgroups per (row, split)).  The 576/512 family runs 64 heads per
// workgroup in 8 waves (4 partners), so a wave holds a quarter of its heads'
// query and of their outputs; the 64/64 family runs up to 128 heads with 2
// partners.  A block count of 3 runs as 4, with the last block's heads masked.
struct AttnLaunch {
    int hb, partners, waves, groups;
};

// Partner waves per 32-head block of the 576/512 attention: 2 (attend_kernel,
// one wave per SIMD) or 4 (attend_p4_kernel, two waves per SIMD).
#ifndef SA_DEFAULT_PARTNERS
#define SA_DEFAULT_PARTNERS 2
#endif
constexpr int kDefaultPartners = SA_DEFAULT_PARTNERS;

// SA_ATTN_PARTNERS_*: 0 takes the default
static bool valid_partners(int v)
{
    return v == SA_ATTN_PARTNERS_DEFAULT || v == SA_ATTN_PARTNERS_2 || v == SA_ATTN_PARTNERS_4;
}

AttnLaunch attn_launch(const sa_params *p, int partners = kDefaultPartners)
{
    AttnLaunch L{};
    L.hb = p->qk_dim == 576 ? (p->num_heads <= 32 ? 1 : 2) : (p->num_heads <= 32 ? 1 : p->num_heads <= 64 ? 2 : 4);
    L.partners = p->qk_dim == 576 && partners == 4 ? 4 : 2;
    L.waves = L.hb * L.partners;
    L.groups = (p->num_heads + 32 * L.hb - 1) / (32 * L.hb);
    return L;
}

// ------------------------------------------------------------------ plans --
struct DecodePlan {
    int64_t score_stride, mm_stride;  // floats per score row; tiles per min/max row
    int splits, tokens_per_split, scan_blocks;
    size_t off_scores, off_mm, off_part_o, off_part_ml, off_mb, total;
    int mb_chunks;  // > 0: rows too long for one top-k workgroup take the many-workgroup path
    int topk_path;  // SA_TOPK_*: which decode rows take the one-pass top-k, and its unroll
    int partners = kDefaultPartners;  // attention partner waves per head block
};

// want_splits > 0 asks for that many attention splits per row (clamped to
// what k allows); 0 takes one attention workgroup per CU over the batch
DecodePlan plan_decode(const sa_params *p, int batch, int max_ctx, int want_splits = 0, int topk_path = 0)
{
    DecodePlan d{};
    d.topk_path = topk_path;
    d.score_stride = round_up(max_ctx > 0 ? max_ctx : 1, 64);
    const int k = p->topk;
    const int groups = attn_launch(p).groups;  // attention workgroups per (row, split)
    int splits = want_splits > 0 ? want_splits
                                 : std::max(1, std::min(kMaxDefaultSplits, kTargetAttnBlocks / (batch * groups)));
    splits = std::max(1, std::min(splits, (k + 31) / 32));
    splits = std::max(splits, (k + kAttnMaxSplitTokens - 1) / kAttnMaxSplitTokens);
    int tps = (int)round_up((k + splits - 1) / splits, 32);
    tps = std::min(tps, kAttnMaxSplitTokens);
    splits = (k + tps - 1) / tps;
    d.splits = splits;
    d.tokens_per_split = tps;
    // persistent scan: one block of 4 waves per CU, fewer when there are few tiles
    const int64_t tiles = (int64_t)batch * ((std::max(max_ctx, 1) + 31) / 32);
    d.scan_blocks = (int)std::max<int64_t>(1, std::min<int64_t>(kScanBlocksPerCU * kCUs, (tiles + 31) / 32));
    size_t off = 0;
    d.off_scores = off;
    off = align_up(off + (size_t)batch * d.score_stride * 4, kAlign);
    d.mm_stride = d.score_stride / 32;
    d.off_mm = off;
    off = align_up(off + (size_t)batch * d.mm_stride * 8, kAlign);
    d.off_part_o = off;
    if (splits > 1) {
        off = align_up(off + (size_t)batch * splits * p->num_heads * p->v_dim * 4, kAlign);
        d.off_part_ml = off;
        off = align_up(off + (size_t)batch * splits * p->num_heads * 16, kAlign);
    } else {
        d.off_part_ml = off;
    }
    // many-workgroup top-k state: per row a MbRowState, 3 digit histograms and
    // two counts per chunk
    // (or, for k <= kLongCap / 2 and rows of at most kMaxLongChunks chunks, the
    // two-launch path's per-row state, per-chunk counts and key segments)
    d.off_mb = off;
    d.mb_chunks = max_ctx > kBitmapKeys ? (max_ctx + kMbChunk - 1) / kMbChunk : 0;
    if (d.mb_chunks > 0) {
        const size_t mb = (size_t)batch * (sizeof(MbRowState) + 3 * kMbBins * 4 + (size_t)d.mb_chunks * 8);
        const size_t lp = (size_t)batch * (sizeof(LongRowState) + (size_t)d.mb_chunks * (8 + (size_t)kLongSeg * 8));
        off = align_up(off + std::max(mb, lp), kAlign);
    }
    d.total = std::max(off, kAlign);
    return d;
}

struct PrefillPlan {
    int64_t score_stride, mm_stride;
    int chunk_rows;          // rows per indexer/top-k chunk
    int splits, tokens_per_split;
    int attn_chunk_rows;     // rows per attention launch when splits > 1
    size_t off_scores, off_mm, off_part_o, off_part_ml, off_mb, total;
    int mb_chunks;  // > 0: rows too long for one top-k workgroup take the many-workgroup path
    int partners = kDefaultPartners;  // attention partner waves per head block
};

// num_rows: query rows of the call; max_ctx: the most keys any row sees;
// chunks of rows are multiples of row_multiple (a power of two >= 16)
PrefillPlan plan_prefill(const sa_params *p, int num_rows, int64_t max_ctx, int row_multiple = kPrefillRowsPerBlock)
{
    PrefillPlan d{};
    d.score_stride = round_up(std::max<int64_t>(max_ctx, 1), 64);
    int64_t rows = (int64_t)(kPrefillScoreBudget / (size_t)(d.score_stride * 4));
    rows = std::max<int64_t>(row_multiple, rows / row_multiple * row_multiple);
    d.chunk_rows = (int)std::min<int64_t>(rows, round_up(num_rows, row_multiple));
    const int k = p->topk;
    d.splits = (k + kAttnMaxSplitTokens - 1) / kAttnMaxSplitTokens;
    d.tokens_per_split = (int)round_up((k + d.splits - 1) / d.splits, 32);
    size_t off = 0;
    d.off_scores = off;
    off = align_up(off + (size_t)d.chunk_rows * d.score_stride * 4, kAlign);
    d.mm_stride = d.score_stride / 32;
    d.off_mm = off;
    off = align_up(off + (size_t)d.chunk_rows * d.mm_stride * 8, kAlign);
    d.off_part_o = off;
    d.attn_chunk_rows = num_rows;
    if (d.splits > 1) {
        const size_t per_row = (size_t)d.splits * p->num_heads * (p->v_dim * 4 + 16);
        d.attn_chunk_rows = (int)std::max<size_t>(1, std::min<size_t>(num_rows, kPrefillPartialBudget / per_row));
        off = align_up(off + (size_t)d.attn_chunk_rows * d.splits * p->num_heads * p->v_dim * 4, kAlign);
        d.off_part_ml = off;
        off = align_up(off + (size_t)d.attn_chunk_rows * d.splits * p->num_heads * 16, kAlign);
    } else {
        d.off_part_ml = off;
    }
    d.total = std::max(off, kAlign);
    return d;
}

sa_status check_decode(const sa_params *p, const sa_paged_cache *c, int batch, int max_ctx, bool kv, bool idx)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!c) return SA_ERR_NULL;
    s = check_cache(p, c, kv, idx, true);
    if (s != SA_OK) return s;
    if (batch < 1 || max_ctx < 0 || (int64_t)max_ctx > (int64_t)c->max_blocks_per_seq * p->block_size)
        return SA_ERR_SHAPE;
    return SA_OK;
}

sa_status check_prefill(const sa_params *p, const sa_paged_cache *c, int num_rows, int q_start, bool kv, bool idx)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!c) return SA_ERR_NULL;
    s = check_cache(p, c, kv, idx, false);
    if (s != SA_OK) return s;
    if (num_rows < 1 || q_start < 0 ||
        (int64_t)q_start + num_rows > (int64_t)c->max_blocks_per_seq * p->block_size ||
        (int64_t)q_start + num_rows > INT32_MAX - 64)
        return SA_ERR_SHAPE;
    return SA_OK;
}

// A run of consecutive query rows of one sequence: rows [row0, row0 + n) of
// the call, at positions pos0 .. pos0 + n - 1, block-table row bt_row.
struct Piece {
    int64_t row0;
    int n, pos0, bt_row;
};

struct PrefillRows {
    std::vector<Piece> pieces;  // non-empty, in row order, covering rows [0, total)
    int total = 0;
    int64_t max_ctx = 0;
};

PrefillRows one_sequence(int num_rows, int q_start)
{
    PrefillRows r;
    r.pieces.push_back(Piece{0, num_rows, q_start, 0});
    r.total = num_rows;
    r.max_ctx = (int64_t)q_start + num_rows;
    return r;
}

// cu_seqlens/q_starts (host) of the varlen call; max_tokens = 0: no cache bound
sa_status varlen_rows(int num_seqs, const int32_t *cu, const int32_t *qs, int64_t max_tokens, PrefillRows *r)
{
    if (!cu || !qs) return SA_ERR_NULL;
    if (num_seqs < 1 || cu[0] != 0) return SA_ERR_SHAPE;
    r->pieces.clear();
    r->max_ctx = 0;
    for (int b = 0; b < num_seqs; ++b) {
        const int64_t n = (int64_t)cu[b + 1] - cu[b];
        if (n < 0 || qs[b] < 0) return SA_ERR_SHAPE;
        if (n == 0) continue;
        const int64_t end = (int64_t)qs[b] + n;
        if (end > INT32_MAX - 64 || (max_tokens > 0 && end > max_tokens)) return SA_ERR_SHAPE;
        r->pieces.push_back(Piece{cu[b], (int)n, qs[b], b});
        r->max_ctx = std::max(r->max_ctx, end);
    }
    if (cu[num_seqs] < 1 || (int64_t)cu[num_seqs] > INT32_MAX - 64) return SA_ERR_SHAPE;
    r->total = cu[num_seqs];
    return SA_OK;
}

// The pieces of rows [r0, r1), with r1 <= rmax as large as kMapPieces pieces
// allow.  `from` is the index of the first piece that may hold row r0.
int cut_rows(const PrefillRows &rows, size_t &from, int r0, int rmax, std::vector<Piece> &parts)
{
    parts.clear();
    while (from < rows.pieces.size() && rows.pieces[from].row0 + rows.pieces[from].n <= r0) ++from;
    int r1 = r0;
    for (size_t j = from; j < rows.pieces.size() && (int)parts.size() < kMapPieces && r1 < rmax; ++j) {
        const Piece &pc = rows.pieces[j];
        const int a = std::max<int64_t>(r0, pc.row0), b = std::min<int64_t>(rmax, pc.row0 + pc.n);
        parts.push_back(Piece{a, b - a, pc.pos0 + (int)(a - pc.row0), pc.bt_row});
        r1 = b;
    }
    return r1;
}

// Map of the parts for the top-k and attention launches: keyed by row, rows
// counted from r0.
SeqMap rows_map(const std::vector<Piece> &parts, int r0)
{
    SeqMap m{};
    m.npieces = (int)parts.size();
    for (int i = 0; i < m.npieces; ++i) {
        m.first[i] = m.row0[i] = (int)(parts[i].row0 - r0);
        m.nrows[i] = parts[i].n;
        m.pos0[i] = parts[i].pos0;
        m.bt_row[i] = parts[i].bt_row;
    }
    m.first[m.npieces] = (int)(parts.back().row0 + parts.back().n - r0);
    return m;
}

// Map for the prefill indexer: keyed by 16-row block, pieces ordered by their
// last position (the kernel runs the blocks from the last one, so the rows
// with the most keys start first).  Returns the block count.
int blocks_map(const std::vector<Piece> &parts, int r0, SeqMap *m)
{
    std::vector<int> order(parts.size());
    for (size_t i = 0; i < parts.size(); ++i) order[i] = (int)i;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        return parts[a].pos0 + parts[a].n < parts[b].pos0 + parts[b].n;
    });
    *m = SeqMap{};
    m->npieces = (int)parts.size();
    int nb = 0;
    for (int i = 0; i < m->npieces; ++i) {
        const Piece &pc = parts[order[i]];
        m->first[i] = nb;
        m->row0[i] = (int)(pc.row0 - r0);
        m->nrows[i] = pc.n;
        m->pos0[i] = pc.pos0;
        m->bt_row[i] = pc.bt_row;
        nb += (pc.n + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock;
    }
    m->first[m->npieces] = nb;
    return nb;
}

sa_status check_ws(const void *ws, size_t have, size_t need)
{
    if (!ws) return SA_ERR_NULL;
    if (have < need) return SA_ERR_WORKSPACE;
    return SA_OK;
}

void clear_hip_error() { (void)hipGetLastError(); }

sa_status launched()
{
    return hipGetLastError() == hipSuccess ? SA_OK : SA_ERR_HIP;
}

// Optional per-launch event marks (profiling entry points): marks[0] is recorded
// before the first launch and marks[i] after the i-th launch, while capacity lasts;
// `count` always advances so the caller learns how many marks a call takes.
struct StageMarks {
    void *const *events = nullptr;
    int capacity = 0;
    int count = 0;
    hipStream_t stream = nullptr;
    void mark()
    {
        if (events && count < capacity) (void)hipEventRecord((hipEvent_t)events[count], stream);
        ++count;
    }
};

// --------------------------------------------------------------- launches --
template <int D, int T>
void launch_idx_decode(const sa_params *p, const sa_paged_cache *c, int batch, const void *idx_q,
                       const float *idx_w, float *scores, int64_t stride, f32x2 *mm, int64_t mm_stride, int blocks,
                       const AppendArgs &ap, hipStream_t st)
{
    const dim3 grid(blocks), block(64 * kScanWavesPerBlock);
    if (p->block_size >= 32)
        hipLaunchKernelGGL((idx_score_decode_kernel<D, T, true>), grid, block, 0, st, (const uint16_t *)c->idx_k,
                           c->block_table, c->max_blocks_per_seq, ilog2(p->block_size), c->context_lens, batch,
                           (const uint16_t *)idx_q, idx_w, p->idx_heads, p->idx_relu, scores, stride, mm, mm_stride,
                           ap);
    else
        hipLaunchKernelGGL((idx_score_decode_kernel<D, T, false>), grid, block, 0, st, (const uint16_t *)c->idx_k,
                           c->block_table, c->max_blocks_per_seq, ilog2(p->block_size), c->context_lens, batch,
                           (const uint16_t *)idx_q, idx_w, p->idx_heads, p->idx_relu, scores, stride, mm, mm_stride,
                           ap);
}

void idx_decode(const sa_params *p, const sa_paged_cache *c, int batch, const void *idx_q, const float *idx_w,
                float *scores, int64_t stride, f32x2 *mm, int64_t mm_stride, int blocks, const AppendArgs &ap,
                hipStream_t st)
{
    const bool two = p->idx_heads > 32;
    if (p->idx_dim == 128) {
        if (two) launch_idx_decode<128, 2>(p, c, batch, idx_q, idx_w, scores, stride, mm, mm_stride, blocks, ap, st);
        else launch_idx_decode<128, 1>(p, c, batch, idx_q, idx_w, scores, stride, mm, mm_stride, blocks, ap, st);
    } else {
        if (two) launch_idx_decode<32, 2>(p, c, batch, idx_q, idx_w, scores, stride, mm, mm_stride, blocks, ap, st);
        else launch_idx_decode<32, 1>(p, c, batch, idx_q, idx_w, scores, stride, mm, mm_stride, blocks, ap, st);
    }
}

template <int D, int T>
void launch_idx_prefill(const sa_params *p, const sa_paged_cache *c, const uint16_t *idx_q, const float *idx_w,
                        const SeqMap &bm, int nblocks, float *scores, int64_t stride, f32x2 *mm, int64_t mm_stride,
                        hipStream_t st)
{
    dim3 grid(nblocks);
    if (p->block_size >= 32)
        hipLaunchKernelGGL((idx_score_prefill_kernel<D, T, true>), grid, dim3(512), 0, st, (const uint16_t *)c->idx_k,
                           c->block_table, c->max_blocks_per_seq, ilog2(p->block_size), idx_q, idx_w, p->idx_heads,
                           p->idx_relu, bm, scores, stride, mm, mm_stride);
    else
        hipLaunchKernelGGL((idx_score_prefill_kernel<D, T, false>), grid, dim3(512), 0, st,
                           (const uint16_t *)c->idx_k, c->block_table, c->max_blocks_per_seq, ilog2(p->block_size),
                           idx_q, idx_w, p->idx_heads, p->idx_relu, bm, scores, stride, mm, mm_stride);
}

void idx_prefill(const sa_params *p, const sa_paged_cache *c, const uint16_t *idx_q, const float *idx_w,
                 const SeqMap &bm, int nblocks, float *scores, int64_t stride, f32x2 *mm, int64_t mm_stride,
                 hipStream_t st)
{
    const bool two = p->idx_heads > 32;
    if (p->idx_dim == 128) {
        if (two) launch_idx_prefill<128, 2>(p, c, idx_q, idx_w, bm, nblocks, scores, stride, mm, mm_stride, st);
        else launch_idx_prefill<128, 1>(p, c, idx_q, idx_w, bm, nblocks, scores, stride, mm, mm_stride, st);
    } else {
        if (two) launch_idx_prefill<32, 2>(p, c, idx_q, idx_w, bm, nblocks, scores, stride, mm, mm_stride, st);
        else launch_idx_prefill<32, 1>(p, c, idx_q, idx_w, bm, nblocks, scores, stride, mm, mm_stride, st);
    }
}

void attend(const sa_params *p, AttnArgs a, int rows, hipStream_t st, StageMarks *mk)
{
    const AttnLaunch L = attn_launch(p, a.partners);
    dim3 grid(a.splits * rows * L.groups), block(64 * L.waves);
    if (p->qk_dim == 576 && L.partners == 4) {
        if (L.hb == 1) hipLaunchKernelGGL((attend_p4_kernel<576, 512, 1>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attend_p4_kernel<576, 512, 2>), grid, block, 0, st, a);
    } else if (p->qk_dim == 576) {
        if (L.hb == 1) hipLaunchKernelGGL((attend_kernel<576, 512, 1>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attend_kernel<576, 512, 2>), grid, block, 0, st, a);
    } else {
        switch (L.hb) {
        case 1: hipLaunchKernelGGL((attend_kernel<64, 64, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((attend_kernel<64, 64, 2>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((attend_kernel<64, 64, 4>), grid, block, 0, st, a); break;
        }
    }
    if (mk) mk->mark();
    if (a.splits > 1) {
        dim3 cg(p->num_heads, rows);
        // kCombineHeads heads per workgroup when that still makes a workgroup per
        // CU; else one head per workgroup (the 4 x 1M-key batch: 512 workgroups
        // instead of 64, its merge 2.4 us faster)
        if (p->v_dim == 512 && a.splits <= 64 && p->num_heads % kCombineHeads == 0 &&
            (int64_t)rows * p->num_heads >= (int64_t)kCombineHeads * kCUs)
            hipLaunchKernelGGL((combine_kernel<512, kCombineHeads>), dim3(p->num_heads / kCombineHeads, rows),
                               dim3(512), 0, st, a.part_o, a.part_ml, a.splits, p->num_heads, a.out, a.out_bf16,
                               a.lse);
        else if (p->v_dim == 512)
            hipLaunchKernelGGL((combine_kernel<512, 1>), cg, dim3(128), 0, st, a.part_o, a.part_ml, a.splits,
                               p->num_heads, a.out, a.out_bf16, a.lse);
        else
            hipLaunchKernelGGL((combine_kernel<64, 1>), cg, dim3(64), 0, st, a.part_o, a.part_ml, a.splits,
                               p->num_heads, a.out, a.out_bf16, a.lse);
        if (mk) mk->mark();
    }
}

AttnArgs attn_args(const sa_params *p, const sa_paged_cache *c, const void *q, const int32_t *topk_idx, void *out,
                   float *lse)
{
    AttnArgs a{};
    a.q = (const uint16_t *)q;
    a.kv = (const uint16_t *)c->kv;
    a.block_table = c->block_table;
    a.topk_idx = topk_idx;
    a.ctx_lens = c->context_lens;
    a.out = out;
    a.lse = lse;
    a.num_blocks = c->num_blocks;
    a.num_heads = p->num_heads;
    a.max_blocks = c->max_blocks_per_seq;
    a.bs_log2 = ilog2(p->block_size);
    a.k = p->topk;
    a.out_bf16 = p->out_dtype == SA_OUT_BF16;
    a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
    return a;
}

// No append (new_kv == nullptr).
AppendArgs no_append() { return AppendArgs{}; }

// Append of the current tokens new_kv / new_idx_k into the cache of c.
AppendArgs append_args(const sa_params *p, const sa_paged_cache *c, const void *new_kv, const void *new_idx_k)
{
    AppendArgs ap{};
    ap.new_kv = (const uint16_t *)new_kv;
    ap.new_idx_k = (const uint16_t *)new_idx_k;
    ap.kv = (uint16_t *)const_cast<void *>(c->kv);      // (the one call that writes the cache)
    ap.idx_k = (uint16_t *)const_cast<void *>(c->idx_k);
    ap.block_table = c->block_table;
    ap.ctx_lens = c->context_lens;
    ap.num_blocks = c->num_blocks;
    ap.max_blocks = c->max_blocks_per_seq;
    ap.bs_log2 = ilog2(p->block_size);
    ap.qk_dim = p->qk_dim;
    ap.idx_dim = p->idx_dim;
    return ap;
}

// Scan (when some row has more than topk keys), then top-k.  With an append,
// the scan scores each row's current token with its new indexer key and the
// top-k launch writes both new rows into the cache (before the attention).
void select_decode(const sa_params *p, const sa_paged_cache *c, int batch, int max_ctx, const void *idx_q,
                   const float *idx_w, int32_t *topk_idx, void *ws, const DecodePlan &d, hipStream_t st,
                   StageMarks *mk, const AppendArgs &ap = no_append())
{
    float *scores = (float *)((char *)ws + d.off_scores);
    f32x2 *mm = (f32x2 *)((char *)ws + d.off_mm);
    if (max_ctx > p->topk) {
        idx_decode(p, c, batch, idx_q, idx_w, scores, d.score_stride, mm, d.mm_stride, d.scan_blocks, ap, st);
        if (mk) mk->mark();
    }
    if (d.mb_chunks > 0 && 2 * p->topk <= kLongCap && d.mb_chunks <= kMaxLongChunks) {
        LongRowState *lst = (LongRowState *)((char *)ws + d.off_mb);
        uint64_t *seg = (uint64_t *)(lst + batch);  // (16-byte states keep these aligned)
        uint2 *seg_info = (uint2 *)(seg + (size_t)batch * d.mb_chunks * kLongSeg);
        const int32_t *cl = c->context_lens;
        hipLaunchKernelGGL(topk_long_gather_kernel, dim3(d.mb_chunks, batch), dim3(kTopkThreads), 0, st, scores,
                           d.score_stride, mm, d.mm_stride, cl, p->topk, topk_idx, lst, seg, seg_info, ap);
        hipLaunchKernelGGL(topk_long_select_kernel, dim3(batch), dim3(kTopkThreads), 0, st, scores, d.score_stride,
                           cl, p->topk, d.mb_chunks, (const LongRowState *)lst, (const uint64_t *)seg,
                           (const uint2 *)seg_info, topk_idx);
    } else if (d.mb_chunks > 0) {
        MbRowState *mst = (MbRowState *)((char *)ws + d.off_mb);
        uint32_t *hist = (uint32_t *)(mst + batch);
        uint32_t *counts = hist + (size_t)batch * 3 * kMbBins;
        const dim3 grid(d.mb_chunks, batch);
        const int32_t *cl = c->context_lens;
        hipLaunchKernelGGL(topk_mb_init_kernel, dim3(batch), dim3(256), 0, st, p->topk, mst, hist, ap);
        hipLaunchKernelGGL(topk_mb_hist_kernel<0>, grid, dim3(kTopkThreads), 0, st, scores, d.score_stride, cl, p->topk, mst, hist);
        hipLaunchKernelGGL(topk_mb_pick_kernel<0>, dim3(batch), dim3(kTopkThreads), 0, st, cl, p->topk, mst, hist);
        hipLaunchKernelGGL(topk_mb_hist_kernel<1>, grid, dim3(kTopkThreads), 0, st, scores, d.score_stride, cl, p->topk, mst, hist);
        hipLaunchKernelGGL(topk_mb_pick_kernel<1>, dim3(batch), dim3(kTopkThreads), 0, st, cl, p->topk, mst, hist);
        hipLaunchKernelGGL(topk_mb_hist_kernel<2>, grid, dim3(kTopkThreads), 0, st, scores, d.score_stride, cl, p->topk, mst, hist);
        hipLaunchKernelGGL(topk_mb_pick_kernel<2>, dim3(batch), dim3(kTopkThreads), 0, st, cl, p->topk, mst, hist);
        hipLaunchKernelGGL(topk_mb_count_kernel, grid, dim3(kTopkThreads), 0, st, scores, d.score_stride, cl, p->topk,
                           mst, counts, d.mb_chunks);
        hipLaunchKernelGGL(topk_mb_emit_kernel, grid, dim3(kTopkThreads), 0, st, scores, d.score_stride, cl, p->topk,
                           mst, counts, d.mb_chunks, topk_idx);
    } else {
        // rows of at least onepass_min keys take the one-pass top-k
        const int k = p->topk;
        const int onepass_min = d.topk_path == SA_TOPK_THRESHOLD ? INT_MAX
                                : d.topk_path == SA_TOPK_DEFAULT ? kOnePassMinPerK * k : 0;
        if (d.topk_path == SA_TOPK_ONEPASS_U4)
            hipLaunchKernelGGL(topk_decode_kernel<4>, dim3(batch), dim3(kTopkThreads), 0, st, scores, d.score_stride,
                               mm, d.mm_stride, c->context_lens, k, onepass_min, topk_idx, ap);
        else
            hipLaunchKernelGGL(topk_decode_kernel<2>, dim3(batch), dim3(kTopkThreads), 0, st, scores, d.score_stride,
                               mm, d.mm_stride, c->context_lens, k, onepass_min, topk_idx, ap);
    }
    if (mk) mk->mark();
}

void attend_decode(const sa_params *p, const sa_paged_cache *c, int batch, const void *q, const int32_t *topk_idx,
                   void *out, float *lse, void *ws, const DecodePlan &d, hipStream_t st, StageMarks *mk)
{
    AttnArgs a = attn_args(p, c, q, topk_idx, out, lse);
    a.decode = 1;
    a.tokens_per_split = d.tokens_per_split;
    a.splits = d.splits;
    a.partners = d.partners;
    a.part_o = (float *)((char *)ws + d.off_part_o);
    a.part_ml = (float *)((char *)ws + d.off_part_ml);
    attend(p, a, batch, st, mk);
}

// Scan (where some row has more than k keys) and top-k of the rows from r0 on,
// as many as one score chunk holds; returns the end of the chunk.
int select_prefill_chunk(const sa_params *p, const sa_paged_cache *c, const PrefillRows &rows, size_t &from, int r0,
                         const void *idx_q, const float *idx_w, int32_t *topk_idx, void *ws, const PrefillPlan &d,
                         hipStream_t st, StageMarks *mk)
{
    float *scores = (float *)((char *)ws + d.off_scores);
    f32x2 *mm = (f32x2 *)((char *)ws + d.off_mm);
    std::vector<Piece> parts;
    const int r1 = cut_rows(rows, from, r0, std::min(rows.total, r0 + d.chunk_rows), parts);
    // rows whose whole context fits in k need no scores
    bool scan = false;
    for (const Piece &pc : parts) scan |= (int64_t)pc.pos0 + pc.n > p->topk;
    if (scan) {
        SeqMap bm;
        const int nb = blocks_map(parts, r0, &bm);
        idx_prefill(p, c, (const uint16_t *)idx_q + (int64_t)r0 * p->idx_heads * p->idx_dim,
                    idx_w + (int64_t)r0 * p->idx_heads, bm, nb, scores, d.score_stride, mm, d.mm_stride, st);
        if (mk) mk->mark();
    }
    hipLaunchKernelGGL(topk_rows_kernel, dim3(r1 - r0), dim3(kTopkThreads), 0, st, scores, d.score_stride, mm,
                       d.mm_stride, 1, (const int32_t *)nullptr, rows_map(parts, r0), p->topk,
                       topk_idx + (int64_t)r0 * p->topk, no_append());
    if (mk) mk->mark();
    return r1;
}

void select_prefill(const sa_params *p, const sa_paged_cache *c, const PrefillRows &rows, const void *idx_q,
                    const float *idx_w, int32_t *topk_idx, void *ws, const PrefillPlan &d, hipStream_t st,
                    StageMarks *mk)
{
    size_t from = 0;
    for (int r0 = 0; r0 < rows.total;)
        r0 = select_prefill_chunk(p, c, rows, from, r0, idx_q, idx_w, topk_idx, ws, d, st, mk);
}

// attention of rows [ra, rb)
void attend_prefill_rows(const sa_params *p, const sa_paged_cache *c, const PrefillRows &rows, int ra, int rb,
                         const void *q, const int32_t *topk_idx, void *out, float *lse, void *ws, const PrefillPlan &d,
                         hipStream_t st, StageMarks *mk)
{
    std::vector<Piece> parts;
    size_t from = 0;
    for (int r0 = ra, r1; r0 < rb; r0 = r1) {
        r1 = cut_rows(rows, from, r0, std::min(rb, r0 + d.attn_chunk_rows), parts);
        AttnArgs a = attn_args(p, c, (const uint16_t *)q + (int64_t)r0 * p->num_heads * p->qk_dim,
                               topk_idx + (int64_t)r0 * p->topk,
                               (char *)out + (int64_t)r0 * p->num_heads * p->v_dim * (p->out_dtype ? 2 : 4),
                               lse ? lse + (int64_t)r0 * p->num_heads : nullptr);
        a.decode = 0;
        a.rows_map = rows_map(parts, r0);
        a.tokens_per_split = d.tokens_per_split;
        a.splits = d.splits;
        a.partners = d.partners;
        a.part_o = (float *)((char *)ws + d.off_part_o);
        a.part_ml = (float *)((char *)ws + d.off_part_ml);
        attend(p, a, r1 - r0, st, mk);
    }
}

void attend_prefill(const sa_params *p, const sa_paged_cache *c, const PrefillRows &rows, const void *q,
                    const int32_t *topk_idx, void *out, float *lse, void *ws, const PrefillPlan &d, hipStream_t st,
                    StageMarks *mk)
{
    attend_prefill_rows(p, c, rows, 0, rows.total, q, topk_idx, out, lse, ws, d, st, mk);
}

// The library's second stream on the current device (default priority,
// non-blocking), created on first use and kept until the process ends.
constexpr int kMaxDevices = 64;
static std::mutex g_side_mu;
static hipStream_t g_side[kMaxDevices];

static hipStream_t side_stream()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_side_mu);
    if (!g_side[dev] && hipStreamCreateWithFlags(&g_side[dev], hipStreamNonBlocking) != hipSuccess)
        g_side[dev] = nullptr;
    return g_side[dev];
}

// Index selection and attention pipelined by chunks of rows ("Day-0
// Adaptation for LLMs: Implementing Sparse Attention and Low-Precision
// Weights", section III item 3): the scan and top-k of chunk i + 1 run on the
// caller's stream while the attention of chunk i runs on the library's second
// stream, which waits for chunk i's top-k through an event; the caller's
// stream waits for the second stream's last launch at the end, so the call is
// ordered on the caller's stream as a serial one would be.  Returns false
// (having launched nothing) where it cannot run: one chunk, a stream under
// graph capture, or no second stream or events.
static bool prefill_pipelined(const sa_params *p, const sa_paged_cache *c, const PrefillRows &rows, const void *q,
                              const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                              void *ws, const PrefillPlan &d, hipStream_t st)
{
    if (d.chunk_rows >= rows.total) return false;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return false;
    hipStream_t side = side_stream();
    if (!side) return false;
    std::vector<int> ends;  // the chunks, as select_prefill_chunk cuts them
    {
        std::vector<Piece> parts;
        size_t from = 0;
        for (int r0 = 0; r0 < rows.total;) {
            r0 = cut_rows(rows, from, r0, std::min(rows.total, r0 + d.chunk_rows), parts);
            ends.push_back(r0);
        }
    }
    const int nchunks = (int)ends.size();
    std::vector<hipEvent_t> ev;
    auto drop = [&]() {
        for (hipEvent_t e : ev) (void)hipEventDestroy(e);  // (released once complete)
    };
    for (int i = 0; i < nchunks + 2; ++i) {
        hipEvent_t e = nullptr;
        if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
            drop();
            clear_hip_error();
            return false;
        }
        ev.push_back(e);
    }
    int ne = 0;
    (void)hipEventRecord(ev[ne], st);  // the side stream starts after the caller's earlier work
    (void)hipStreamWaitEvent(side, ev[ne++], 0);
    size_t from = 0;
    for (int i = 0, r0 = 0; i < nchunks; r0 = ends[i++]) {
        const int r1 = select_prefill_chunk(p, c, rows, from, r0, idx_q, idx_w, topk_idx, ws, d, st, nullptr);
        (void)hipEventRecord(ev[ne], st);
        (void)hipStreamWaitEvent(side, ev[ne++], 0);
        attend_prefill_rows(p, c, rows, r0, r1, q, topk_idx, out, lse, ws, d, side, nullptr);
    }
    (void)hipEventRecord(ev[ne], side);
    (void)hipStreamWaitEvent(st, ev[ne], 0);
    drop();
    return true;
}

// ------------------------------------------------ block-granular selection --
// p->topk = k counts KV blocks (cache blocks); the attention then runs over
// k * block_size token slots per row.
struct BlockPlan {
    sa_params pa;          // p with topk = k * block_size (the attention's view)
    int q_block, groups;   // rows per query block; query blocks per select chunk (decode: the batch)
    int64_t bstride, bmm_stride;
    size_t off_bscore, off_bmm, off_ncand, off_tokens, total;
};

sa_status check_blocks(const sa_params *p)
{
    if ((int64_t)p->topk * p->block_size > kMaxTopk) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

// the block-mode areas after `base` bytes: block scores and ranges of `groups`
// query blocks of at most max_ctx positions, candidate counts, and the
// expanded token lists of `rows` rows
void plan_block_areas(const sa_params *p, BlockPlan &b, size_t base, int groups, int64_t max_ctx, int rows)
{
    const int64_t nblk = (std::max<int64_t>(max_ctx, 1) + p->block_size - 1) / p->block_size;
    b.groups = groups;
    b.bstride = round_up(nblk, 64);
    b.bmm_stride = b.bstride / 32;
    size_t off = align_up(base, kAlign);
    b.off_bscore = off;
    off = align_up(off + (size_t)groups * b.bstride * 4, kAlign);
    b.off_bmm = off;
    off = align_up(off + (size_t)groups * b.bmm_stride * 8, kAlign);
    b.off_ncand = off;
    off = align_up(off + (size_t)groups * 4, kAlign);
    b.off_tokens = off;
    off = align_up(off + (size_t)rows * b.pa.topk * 4, kAlign);
    b.total = off;
}

BlockPlan plan_decode_blocks(const sa_params *p, int batch, int max_ctx, DecodePlan *dp)
{
    BlockPlan b{};
    b.pa = *p;
    b.pa.topk = p->topk * p->block_size;
    b.q_block = 1;
    *dp = plan_decode(&b.pa, batch, max_ctx);
    plan_block_areas(p, b, dp->total, batch, max_ctx, batch);
    return b;
}

BlockPlan plan_prefill_blocks(const sa_params *p, int num_rows, int q_start, int q_block, PrefillPlan *pp)
{
    BlockPlan b{};
    b.pa = *p;
    b.pa.topk = p->topk * p->block_size;
    b.q_block = q_block;
    *pp = plan_prefill(&b.pa, num_rows, (int64_t)q_start + num_rows, std::max(kPrefillRowsPerBlock, q_block));
    plan_block_areas(p, b, pp->total, pp->chunk_rows / q_block, (int64_t)q_start + num_rows, num_rows);
    return b;
}

// Block scores of `groups` query blocks, then the top-k over them into
// block_idx (k per query block).
void select_blocks(const sa_params *p, const BlockPlan &b, const float *scores, int64_t score_stride,
                   const int32_t *ctx_lens, int pos0, int nrows, int32_t *block_idx, void *ws, hipStream_t st)
{
    const int groups = (nrows + b.q_block - 1) / b.q_block;
    float *bscore = (float *)((char *)ws + b.off_bscore);
    f32x2 *bmm = (f32x2 *)((char *)ws + b.off_bmm);
    int32_t *ncand = (int32_t *)((char *)ws + b.off_ncand);
    hipLaunchKernelGGL(block_score_kernel, dim3(groups, (unsigned)(b.bstride / 32)), dim3(kBlockScoreThreads), 0, st,
                       scores, score_stride, ctx_lens, pos0, b.q_block, nrows, ilog2(p->block_size), p->topk, bscore,
                       b.bstride, bmm, b.bmm_stride, ncand);
    hipLaunchKernelGGL(topk_rows_kernel, dim3(groups), dim3(kTopkThreads), 0, st, (const float *)bscore, b.bstride,
                       (const f32x2 *)bmm, b.bmm_stride, 0, (const int32_t *)ncand, SeqMap{}, p->topk, block_idx,
                       no_append());
}

void decode_blocks_impl(const sa_params *p, const sa_paged_cache *c, int batch, int max_ctx, const void *q,
                        const void *idx_q, const float *idx_w, int32_t *block_idx, void *out, float *lse, void *ws,
                        const BlockPlan &b, const DecodePlan &d, hipStream_t st, StageMarks *mk)
{
    float *scores = (float *)((char *)ws + d.off_scores);
    f32x2 *mm = (f32x2 *)((char *)ws + d.off_mm);
    // token scores only where some sequence has more candidate blocks than k
    if ((int64_t)max_ctx > (int64_t)p->topk * p->block_size) {
        idx_decode(p, c, batch, idx_q, idx_w, scores, d.score_stride, mm, d.mm_stride, d.scan_blocks, no_append(),
                   st);
        if (mk) mk->mark();
    }
    select_blocks(p, b, scores, d.score_stride, c->context_lens, 0, batch, block_idx, ws, st);
    if (mk) mk->mark();
    int32_t *tokens = (int32_t *)((char *)ws + b.off_tokens);
    hipLaunchKernelGGL(expand_blocks_kernel, dim3(batch), dim3(256), 0, st, (const int32_t *)block_idx, p->topk,
                       c->context_lens, 0, 1, ilog2(p->block_size), tokens);
    attend_decode(&b.pa, c, batch, q, tokens, out, lse, ws, d, st, mk);
}

void prefill_blocks_impl(const sa_params *p, const sa_paged_cache *c, int num_rows, int q_start, const void *q,
                         const void *idx_q, const float *idx_w, int32_t *block_idx, void *out, float *lse, void *ws,
                         const BlockPlan &b, const PrefillPlan &d, hipStream_t st, StageMarks *mk)
{
    float *scores = (float *)((char *)ws + d.off_scores);
    f32x2 *mm = (f32x2 *)((char *)ws + d.off_mm);
    const PrefillRows rows = one_sequence(num_rows, q_start);
    std::vector<Piece> parts;
    size_t from = 0;
    for (int r0 = 0, r1; r0 < num_rows; r0 = r1) {  // chunks of whole query blocks
        r1 = cut_rows(rows, from, r0, std::min(num_rows, r0 + d.chunk_rows), parts);
        const int64_t last = (int64_t)q_start + r1 - 1;
        if ((last >> ilog2(p->block_size)) + 1 > p->topk) {
            SeqMap bm;
            const int nb = blocks_map(parts, r0, &bm);
            idx_prefill(p, c, (const uint16_t *)idx_q + (int64_t)r0 * p->idx_heads * p->idx_dim,
                        idx_w + (int64_t)r0 * p->idx_heads, bm, nb, scores, d.score_stride, mm, d.mm_stride, st);
            if (mk) mk->mark();
        }
        select_blocks(p, b, scores, d.score_stride, nullptr, q_start + r0, r1 - r0,
                      block_idx + (int64_t)(r0 / b.q_block) * p->topk, ws, st);
        if (mk) mk->mark();
    }
    int32_t *tokens = (int32_t *)((char *)ws + b.off_tokens);
    hipLaunchKernelGGL(expand_blocks_kernel, dim3(num_rows), dim3(256), 0, st, (const int32_t *)block_idx, p->topk,
                       (const int32_t *)nullptr, q_start, b.q_block, ilog2(p->block_size), tokens);
    attend_prefill(&b.pa, c, rows, q, tokens, out, lse, ws, d, st, mk);
}

}  // namespace

// ---------------------------------------------------------------- C ABI --
extern "C" {

int32_t sa_abi_version(void) { return SA_ABI_VERSION; }

const char *sa_status_string(sa_status s)
{
    switch (s) {
    case SA_OK: return "ok";
    case SA_ERR_NULL: return "required pointer is NULL";
    case SA_ERR_SHAPE: return "inconsistent or out-of-range sizes";
    case SA_ERR_UNSUPPORTED: return "parameters outside the compiled kernel families";
    case SA_ERR_WORKSPACE: return "workspace too small";
    case SA_ERR_HIP: return "HIP runtime reported a launch error";
    }
    return "unknown status";
}

sa_status sa_decode_workspace_size(const sa_params *p, int32_t batch, int32_t max_ctx, size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    if (batch < 1 || max_ctx < 0) return SA_ERR_SHAPE;
    *bytes = plan_decode(p, batch, max_ctx).total;
    return SA_OK;
}

sa_status sa_prefill_workspace_size(const sa_params *p, int32_t num_rows, int32_t q_start, size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    if (num_rows < 1 || q_start < 0 || (int64_t)q_start + num_rows > INT32_MAX - 64) return SA_ERR_SHAPE;
    *bytes = plan_prefill(p, num_rows, (int64_t)q_start + num_rows).total;
    return SA_OK;
}

sa_status sa_prefill_varlen_workspace_size(const sa_params *p, int32_t num_seqs, const int32_t *cu_seqlens,
                                           const int32_t *q_starts, size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    PrefillRows rows;
    if ((s = varlen_rows(num_seqs, cu_seqlens, q_starts, 0, &rows)) != SA_OK) return s;
    *bytes = plan_prefill(p, rows.total, rows.max_ctx).total;
    return SA_OK;
}

sa_status sparse_attn_select_decode(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                    const void *idx_q, const float *idx_w, int32_t *topk_idx, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    sa_status s = check_decode(p, c, batch, max_ctx, false, true);
    if (s != SA_OK) return s;
    if (!idx_q || !idx_w || !topk_idx) return SA_ERR_NULL;
    const DecodePlan d = plan_decode(p, batch, max_ctx);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    clear_hip_error();
    select_decode(p, c, batch, max_ctx, idx_q, idx_w, topk_idx, workspace, d, (hipStream_t)stream, nullptr);
    return launched();
}

sa_status sparse_attn_attend_decode(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                    const void *q, const int32_t *topk_idx, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    sa_status s = check_decode(p, c, batch, max_ctx, true, false);
    if (s != SA_OK) return s;
    if (!q || !topk_idx || !out) return SA_ERR_NULL;
    const DecodePlan d = plan_decode(p, batch, max_ctx);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    clear_hip_error();
    attend_decode(p, c, batch, q, topk_idx, out, lse, workspace, d, (hipStream_t)stream, nullptr);
    return launched();
}

static sa_status decode_impl(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                             const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream, StageMarks *mk,
                             const void *new_kv = nullptr, const void *new_idx_k = nullptr, int want_splits = 0,
                             int topk_path = 0, int partners = 0)
{
    sa_status s = check_decode(p, c, batch, max_ctx, true, true);
    if (s != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !topk_idx || !out) return SA_ERR_NULL;
    DecodePlan d = plan_decode(p, batch, max_ctx, want_splits, topk_path);
    if (partners) d.partners = partners;
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    clear_hip_error();
    if (mk) {
        mk->stream = st;
        mk->mark();
    }
    const AppendArgs ap = new_kv ? append_args(p, c, new_kv, new_idx_k) : no_append();
    select_decode(p, c, batch, max_ctx, idx_q, idx_w, topk_idx, workspace, d, st, mk, ap);
    attend_decode(p, c, batch, q, topk_idx, out, lse, workspace, d, st, mk);
    return launched();
}

sa_status sparse_attn_decode(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                             const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    return decode_impl(p, c, batch, max_ctx, q, idx_q, idx_w, topk_idx, out, lse, workspace, workspace_bytes, stream,
                       nullptr);
}

sa_status sparse_attn_decode_append(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                    const void *new_kv, const void *new_idx_k, const void *q, const void *idx_q,
                                    const float *idx_w, int32_t *topk_idx, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream)
{
    if (!new_kv || !new_idx_k) return SA_ERR_NULL;
    return decode_impl(p, c, batch, max_ctx, q, idx_q, idx_w, topk_idx, out, lse, workspace, workspace_bytes, stream,
                       nullptr, new_kv, new_idx_k);
}

sa_status sparse_attn_decode_profiled(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                      const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx,
                                      void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream,
                                      void *const *events, int32_t num_events, int32_t *num_marks)
{
    if (!num_marks || (num_events > 0 && !events)) return SA_ERR_NULL;
    StageMarks mk;
    mk.events = events;
    mk.capacity = num_events;
    const sa_status s = decode_impl(p, c, batch, max_ctx, q, idx_q, idx_w, topk_idx, out, lse, workspace,
                                    workspace_bytes, stream, &mk);
    *num_marks = mk.count;
    return s;
}

sa_status sparse_attn_select_prefill(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                                     const void *idx_q, const float *idx_w, int32_t *topk_idx, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    sa_status s = check_prefill(p, c, num_rows, q_start, false, true);
    if (s != SA_OK) return s;
    if (!idx_q || !idx_w || !topk_idx) return SA_ERR_NULL;
    const PrefillRows rows = one_sequence(num_rows, q_start);
    const PrefillPlan d = plan_prefill(p, rows.total, rows.max_ctx);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    clear_hip_error();
    select_prefill(p, c, rows, idx_q, idx_w, topk_idx, workspace, d, (hipStream_t)stream, nullptr);
    return launched();
}

sa_status sparse_attn_attend_prefill(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                                     const void *q, const int32_t *topk_idx, void *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    sa_status s = check_prefill(p, c, num_rows, q_start, true, false);
    if (s != SA_OK) return s;
    if (!q || !topk_idx || !out) return SA_ERR_NULL;
    const PrefillRows rows = one_sequence(num_rows, q_start);
    const PrefillPlan d = plan_prefill(p, rows.total, rows.max_ctx);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    clear_hip_error();
    attend_prefill(p, c, rows, q, topk_idx, out, lse, workspace, d, (hipStream_t)stream, nullptr);
    return launched();
}

static sa_status prefill_rows_impl(const sa_params *p, const sa_paged_cache *c, const PrefillRows &rows,
                                   const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx,
                                   void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream,
                                   StageMarks *mk, bool pipeline = false, int partners = 0)
{
    if (!q || !idx_q || !idx_w || !topk_idx || !out) return SA_ERR_NULL;
    PrefillPlan d = plan_prefill(p, rows.total, rows.max_ctx);
    if (partners) d.partners = partners;
    sa_status s = check_ws(workspace, workspace_bytes, d.total);
    if (s != SA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    clear_hip_error();
    if (mk) {
        mk->stream = st;
        mk->mark();
    }
    if (pipeline && !mk && prefill_pipelined(p, c, rows, q, idx_q, idx_w, topk_idx, out, lse, workspace, d, st))
        return launched();
    select_prefill(p, c, rows, idx_q, idx_w, topk_idx, workspace, d, st, mk);
    attend_prefill(p, c, rows, q, topk_idx, out, lse, workspace, d, st, mk);
    return launched();
}

static sa_status prefill_impl(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                              const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                              float *lse, void *workspace, size_t workspace_bytes, void *stream, StageMarks *mk)
{
    const sa_status s = check_prefill(p, c, num_rows, q_start, true, true);
    if (s != SA_OK) return s;
    return prefill_rows_impl(p, c, one_sequence(num_rows, q_start), q, idx_q, idx_w, topk_idx, out, lse, workspace,
                             workspace_bytes, stream, mk);
}

static sa_status prefill_varlen_impl(const sa_params *p, const sa_paged_cache *c, int32_t num_seqs,
                                     const int32_t *cu_seqlens, const int32_t *q_starts, const void *q,
                                     const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream, StageMarks *mk,
                                     bool pipeline = false, int partners = 0)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!c) return SA_ERR_NULL;
    if ((s = check_cache(p, c, true, true, false)) != SA_OK) return s;
    PrefillRows rows;
    if ((s = varlen_rows(num_seqs, cu_seqlens, q_starts, (int64_t)c->max_blocks_per_seq * p->block_size, &rows)) !=
        SA_OK)
        return s;
    return prefill_rows_impl(p, c, rows, q, idx_q, idx_w, topk_idx, out, lse, workspace, workspace_bytes, stream,
                             mk, pipeline, partners);
}

sa_status sparse_attn_prefill_varlen_cfg(const sa_params *p, const sa_paged_cache *c, int32_t num_seqs,
                                         const int32_t *cu_seqlens, const int32_t *q_starts,
                                         const sa_prefill_config *cfg, const void *q, const void *idx_q,
                                         const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                         void *workspace, size_t workspace_bytes, void *stream)
{
    if (cfg && ((cfg->pipeline != SA_PREFILL_SERIAL && cfg->pipeline != SA_PREFILL_PIPELINED) ||
                !valid_partners(cfg->attn_partners) || cfg->reserved[0] != 0 || cfg->reserved[1] != 0))
        return SA_ERR_SHAPE;
    return prefill_varlen_impl(p, c, num_seqs, cu_seqlens, q_starts, q, idx_q, idx_w, topk_idx, out, lse, workspace,
                               workspace_bytes, stream, nullptr, cfg && cfg->pipeline == SA_PREFILL_PIPELINED,
                               cfg ? cfg->attn_partners : 0);
}

sa_status sparse_attn_prefill_varlen(const sa_params *p, const sa_paged_cache *c, int32_t num_seqs,
                                     const int32_t *cu_seqlens, const int32_t *q_starts, const void *q,
                                     const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream)
{
    return prefill_varlen_impl(p, c, num_seqs, cu_seqlens, q_starts, q, idx_q, idx_w, topk_idx, out, lse, workspace,
                               workspace_bytes, stream, nullptr);
}

sa_status sparse_attn_prefill_varlen_profiled(const sa_params *p, const sa_paged_cache *c, int32_t num_seqs,
                                              const int32_t *cu_seqlens, const int32_t *q_starts, const void *q,
                                              const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                                              float *lse, void *workspace, size_t workspace_bytes, void *stream,
                                              void *const *events, int32_t num_events, int32_t *num_marks)
{
    if (!num_marks || (num_events > 0 && !events)) return SA_ERR_NULL;
    StageMarks mk;
    mk.events = events;
    mk.capacity = num_events;
    const sa_status s = prefill_varlen_impl(p, c, num_seqs, cu_seqlens, q_starts, q, idx_q, idx_w, topk_idx, out,
                                            lse, workspace, workspace_bytes, stream, &mk);
    *num_marks = mk.count;
    return s;
}

sa_status sparse_attn_prefill(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                              const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                              float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    return prefill_impl(p, c, num_rows, q_start, q, idx_q, idx_w, topk_idx, out, lse, workspace, workspace_bytes,
                        stream, nullptr);
}

sa_status sparse_attn_prefill_profiled(const sa_params *p, const sa_paged_cache *c, int32_t num_rows,
                                       int32_t q_start, const void *q, const void *idx_q, const float *idx_w,
                                       int32_t *topk_idx, void *out, float *lse, void *workspace,
                                       size_t workspace_bytes, void *stream, void *const *events,
                                       int32_t num_events, int32_t *num_marks)
{
    if (!num_marks || (num_events > 0 && !events)) return SA_ERR_NULL;
    StageMarks mk;
    mk.events = events;
    mk.capacity = num_events;
    const sa_status s = prefill_impl(p, c, num_rows, q_start, q, idx_q, idx_w, topk_idx, out, lse, workspace,
                                     workspace_bytes, stream, &mk);
    *num_marks = mk.count;
    return s;
}

// ------------------------------------------------------- run-time tuning --
static sa_status check_cfg(const sa_decode_config *cfg)
{
    if (cfg && (cfg->attn_splits < 0 || cfg->attn_splits > 1024)) return SA_ERR_SHAPE;
    if (cfg && (cfg->topk_path < SA_TOPK_DEFAULT || cfg->topk_path > SA_TOPK_ONEPASS_U4)) return SA_ERR_SHAPE;
    if (cfg && (!valid_partners(cfg->attn_partners) || cfg->reserved[0] != 0)) return SA_ERR_SHAPE;
    return SA_OK;
}

sa_status sa_decode_workspace_size_cfg(const sa_params *p, int32_t batch, int32_t max_ctx,
                                       const sa_decode_config *cfg, size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if ((s = check_cfg(cfg)) != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    if (batch < 1 || max_ctx < 0) return SA_ERR_SHAPE;
    *bytes = plan_decode(p, batch, max_ctx, cfg ? cfg->attn_splits : 0).total;
    return SA_OK;
}

sa_status sparse_attn_decode_cfg(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                 const sa_decode_config *cfg, const void *q, const void *idx_q, const float *idx_w,
                                 int32_t *topk_idx, void *out, float *lse, void *workspace, size_t workspace_bytes,
                                 void *stream)
{
    const sa_status s = check_cfg(cfg);
    if (s != SA_OK) return s;
    return decode_impl(p, c, batch, max_ctx, q, idx_q, idx_w, topk_idx, out, lse, workspace, workspace_bytes, stream,
                       nullptr, nullptr, nullptr, cfg ? cfg->attn_splits : 0, cfg ? cfg->topk_path : 0,
                       cfg ? cfg->attn_partners : 0);
}

// The split counts the tuner tries: every count the plan can realise (k is
// split into 32-token multiples of at most 2048 tokens), up to 64.
static std::vector<int> tune_candidates(const sa_params *p, int batch, int max_ctx)
{
    std::vector<int> out;
    for (int want = 1; want <= 64; ++want) {
        const int got = plan_decode(p, batch, max_ctx, want).splits;
        if (std::find(out.begin(), out.end(), got) == out.end()) out.push_back(got);
    }
    return out;
}

sa_status sa_decode_tune_workspace_size(const sa_params *p, int32_t batch, int32_t max_ctx, size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    if (batch < 1 || max_ctx < 0) return SA_ERR_SHAPE;
    size_t need = plan_decode(p, batch, max_ctx).total;
    for (int sp : tune_candidates(p, batch, max_ctx)) need = std::max(need, plan_decode(p, batch, max_ctx, sp).total);
    *bytes = need;
    return SA_OK;
}

sa_status sa_decode_tune(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx, const void *q,
                         const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                         void *workspace, size_t workspace_bytes, void *stream, int32_t reps,
                         sa_decode_config *best, float *best_us)
{
    sa_status s = check_decode(p, c, batch, max_ctx, true, true);
    if (s != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !topk_idx || !out || !best) return SA_ERR_NULL;
    if (reps < 1 || reps > 1000) return SA_ERR_SHAPE;
    size_t need = 0;
    if ((s = sa_decode_tune_workspace_size(p, batch, max_ctx, &need)) != SA_OK) return s;
    if ((s = check_ws(workspace, workspace_bytes, need)) != SA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return SA_ERR_HIP;
    }
    // one untimed call, then reps timed back to back; microseconds per call
    auto time_cfg = [&](int sp, int path, float &us, int partners = 0) -> sa_status {
        sa_status r = SA_OK;
        for (int i = 0; i <= reps && r == SA_OK; ++i) {
            if (i == 1 && hipEventRecord(e0, st) != hipSuccess) r = SA_ERR_HIP;
            if (r == SA_OK)
                r = decode_impl(p, c, batch, max_ctx, q, idx_q, idx_w, topk_idx, out, lse, workspace,
                                workspace_bytes, stream, nullptr, nullptr, nullptr, sp, path, partners);
        }
        float ms = 0.0f;
        if (r == SA_OK && (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
                           hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
            r = SA_ERR_HIP;
        us = ms * 1000.0f / reps;
        return r;
    };
    // the split count under the default top-k, then the top-k path under that
    // count, then (576/512 shape) the other attention kernel under both
    float best_t = INFINITY;
    int best_sp = 0, best_path = SA_TOPK_DEFAULT, best_partners = SA_ATTN_PARTNERS_DEFAULT;
    s = SA_OK;
    for (int sp : tune_candidates(p, batch, max_ctx)) {
        float us = 0.0f;
        if ((s = time_cfg(sp, SA_TOPK_DEFAULT, us)) != SA_OK) break;
        if (us < best_t) {
            best_t = us;
            best_sp = sp;
        }
    }
    for (int path = SA_TOPK_THRESHOLD; path <= SA_TOPK_ONEPASS_U4 && s == SA_OK; ++path) {
        float us = 0.0f;
        if ((s = time_cfg(best_sp, path, us)) != SA_OK) break;
        if (us < best_t) {
            best_t = us;
            best_path = path;
        }
    }
    if (p->qk_dim == 576 && s == SA_OK) {
        const int other = kDefaultPartners == 4 ? SA_ATTN_PARTNERS_2 : SA_ATTN_PARTNERS_4;
        float us = 0.0f;
        if ((s = time_cfg(best_sp, best_path, us, other)) == SA_OK && us < best_t) {
            best_t = us;
            best_partners = other;
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (s != SA_OK) return s;
    *best = sa_decode_config{};
    best->attn_splits = best_sp;
    best->topk_path = best_path;
    best->attn_partners = best_partners;
    if (best_us) *best_us = best_t;
    return SA_OK;
}

// ------------------------------------------------ block-granular selection --
static sa_status check_q_block(int q_block)
{
    if (q_block < 1) return SA_ERR_SHAPE;
    if (!is_pow2(q_block) || q_block > 128) return SA_ERR_UNSUPPORTED;
    return SA_OK;
}

sa_status sa_decode_blocks_workspace_size(const sa_params *p, int32_t batch, int32_t max_ctx, size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if ((s = check_blocks(p)) != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    if (batch < 1 || max_ctx < 0) return SA_ERR_SHAPE;
    DecodePlan d;
    *bytes = plan_decode_blocks(p, batch, max_ctx, &d).total;
    return SA_OK;
}

sa_status sparse_attn_decode_blocks(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                    const void *q, const void *idx_q, const float *idx_w, int32_t *block_idx,
                                    void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream)
{
    sa_status s = check_decode(p, c, batch, max_ctx, true, true);
    if (s != SA_OK) return s;
    if ((s = check_blocks(p)) != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !block_idx || !out) return SA_ERR_NULL;
    DecodePlan d;
    const BlockPlan b = plan_decode_blocks(p, batch, max_ctx, &d);
    if ((s = check_ws(workspace, workspace_bytes, b.total)) != SA_OK) return s;
    clear_hip_error();
    decode_blocks_impl(p, c, batch, max_ctx, q, idx_q, idx_w, block_idx, out, lse, workspace, b, d,
                       (hipStream_t)stream, nullptr);
    return launched();
}

sa_status sa_prefill_blocks_workspace_size(const sa_params *p, int32_t num_rows, int32_t q_start, int32_t q_block,
                                           size_t *bytes)
{
    sa_status s = check_params(p);
    if (s != SA_OK) return s;
    if ((s = check_blocks(p)) != SA_OK || (s = check_q_block(q_block)) != SA_OK) return s;
    if (!bytes) return SA_ERR_NULL;
    if (num_rows < 1 || q_start < 0 || (int64_t)q_start + num_rows > INT32_MAX - 64) return SA_ERR_SHAPE;
    PrefillPlan d;
    *bytes = plan_prefill_blocks(p, num_rows, q_start, q_block, &d).total;
    return SA_OK;
}

sa_status sparse_attn_prefill_blocks(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                                     int32_t q_block, const void *q, const void *idx_q, const float *idx_w,
                                     int32_t *block_idx, void *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    sa_status s = check_prefill(p, c, num_rows, q_start, true, true);
    if (s != SA_OK) return s;
    if ((s = check_blocks(p)) != SA_OK || (s = check_q_block(q_block)) != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !block_idx || !out) return SA_ERR_NULL;
    PrefillPlan d;
    const BlockPlan b = plan_prefill_blocks(p, num_rows, q_start, q_block, &d);
    if ((s = check_ws(workspace, workspace_bytes, b.total)) != SA_OK) return s;
    clear_hip_error();
    prefill_blocks_impl(p, c, num_rows, q_start, q, idx_q, idx_w, block_idx, out, lse, workspace, b, d,
                        (hipStream_t)stream, nullptr);
    return launched();
}

// ------------------------------------------------- allocation-free decode --
// The scratch memory of sparse_attn_decode_noalloc: one copy per device,
// alive until the process ends.  Host code never passes the array's name to a
// kernel (in host code it is a host-side stand-in): it uses the device address
// that hipGetSymbolAddress returns, looked up once per device.
static __device__ __align__(256) uint8_t scratch[SA_NOALLOC_SCRATCH_BYTES];

static std::mutex g_scratch_mu;
static void *g_scratch_addr[kMaxDevices];  // device address of `scratch`, by device id

// The address of `scratch` on the caller's current device (looked up on the
// first call for that device, with that device current).
static sa_status scratch_address(void **addr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SA_ERR_HIP;
        g_scratch_addr[dev] = ptr;
    }
    *addr = g_scratch_addr[dev];
    return SA_OK;
}

sa_status sparse_attn_decode_noalloc(const sa_params *p, const sa_paged_cache *c, int32_t batch, int32_t max_ctx,
                                     const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx,
                                     void *out, float *lse, void *stream)
{
    sa_status s = check_decode(p, c, batch, max_ctx, true, true);
    if (s != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !topk_idx || !out) return SA_ERR_NULL;
    if (plan_decode(p, batch, max_ctx).total > SA_NOALLOC_SCRATCH_BYTES) return SA_ERR_WORKSPACE;
    void *ws = nullptr;
    if ((s = scratch_address(&ws)) != SA_OK) return s;
    // every kernel of the decode writes the scratch it reads (the many-workgroup
    // top-k clears its histograms in its first launch; the long-row top-k's
    // select reads only the counts its gathering launch wrote), so the previous
    // call's contents need no clearing
    return decode_impl(p, c, batch, max_ctx, q, idx_q, idx_w, topk_idx, out, lse, ws, SA_NOALLOC_SCRATCH_BYTES,
                       stream, nullptr);
}

}  // extern "C"
