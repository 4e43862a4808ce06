// libsparse_attn: C ABI (include/sparse_attn.h) over the gfx950 kernels.
//
// Every check runs before the first HIP call; the library never allocates,
// never synchronises and keeps no mutable global state.  Work is queued on the
// caller's stream in this order:
//   decode : indexer scan -> per-row top-k -> split attention -> split merge
//   prefill: per chunk of rows { indexer tile scan -> per-row top-k },
//            then attention over all rows (split + merge only when k > 2048)
// The decode/prefill separation over one cache and one index format follows
// "Day-0 Adaptation: Running Trillion-Parameter Models on Domestic AI
// Accelerators", sections 3.1 and 3.3.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/sparse_attn.h"
#include "attention.hpp"
#include "indexer.hpp"
#include "topk.hpp"

namespace {

using namespace sa;

constexpr int kMaxTopk = 16384;
constexpr int kTargetAttnBlocks = 256;        // one attention workgroup per CU of an MI355X
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
        p->idx_dim < 1 || p->block_size < 1 || p->topk < 1 || !std::isfinite(p->softmax_scale) ||
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

// ------------------------------------------------------------------ plans --
struct DecodePlan {
    int64_t score_stride, mm_stride;  // floats per score row; tiles per min/max row
    int splits, tokens_per_split, scan_blocks;
    size_t off_scores, off_mm, off_part_o, off_part_ml, off_mb, total;
    int mb_chunks;  // > 0: rows too long for one top-k workgroup take the many-workgroup path
};

DecodePlan plan_decode(const sa_params *p, int batch, int max_ctx)
{
    DecodePlan d{};
    d.score_stride = round_up(max_ctx > 0 ? max_ctx : 1, 64);
    const int k = p->topk;
    const int vsplit = p->v_dim > 256 ? 2 : 1;  // value halves per (row, split), as in the attention kernel
    int splits = std::max(1, kTargetAttnBlocks / (batch * vsplit));
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
    d.off_mb = off;
    d.mb_chunks = max_ctx > kBitmapKeys ? (max_ctx + kMbChunk - 1) / kMbChunk : 0;
    if (d.mb_chunks > 0)
        off = align_up(off + (size_t)batch * (sizeof(MbRowState) + 3 * kMbBins * 4 + (size_t)d.mb_chunks * 8), kAlign);
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
};

PrefillPlan plan_prefill(const sa_params *p, int num_rows, int q_start)
{
    PrefillPlan d{};
    const int64_t ctx = (int64_t)q_start + num_rows;
    d.score_stride = round_up(ctx, 64);
    int64_t rows = (int64_t)(kPrefillScoreBudget / (size_t)(d.score_stride * 4));
    rows = std::max<int64_t>(kPrefillRowsPerBlock, rows / kPrefillRowsPerBlock * kPrefillRowsPerBlock);
    d.chunk_rows = (int)std::min<int64_t>(rows, round_up(num_rows, kPrefillRowsPerBlock));
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
                        int pos0, int nrows, float *scores, int64_t stride, f32x2 *mm, int64_t mm_stride,
                        hipStream_t st)
{
    dim3 grid((nrows + kPrefillRowsPerBlock - 1) / kPrefillRowsPerBlock);
    if (p->block_size >= 32)
        hipLaunchKernelGGL((idx_score_prefill_kernel<D, T, true>), grid, dim3(512), 0, st, (const uint16_t *)c->idx_k,
                           c->block_table, ilog2(p->block_size), idx_q, idx_w, p->idx_heads, p->idx_relu, pos0,
                           nrows, scores, stride, mm, mm_stride);
    else
        hipLaunchKernelGGL((idx_score_prefill_kernel<D, T, false>), grid, dim3(512), 0, st,
                           (const uint16_t *)c->idx_k, c->block_table, ilog2(p->block_size), idx_q, idx_w,
                           p->idx_heads, p->idx_relu, pos0, nrows, scores, stride, mm, mm_stride);
}

void idx_prefill(const sa_params *p, const sa_paged_cache *c, const uint16_t *idx_q, const float *idx_w, int pos0,
                 int nrows, float *scores, int64_t stride, f32x2 *mm, int64_t mm_stride, hipStream_t st)
{
    const bool two = p->idx_heads > 32;
    if (p->idx_dim == 128) {
        if (two) launch_idx_prefill<128, 2>(p, c, idx_q, idx_w, pos0, nrows, scores, stride, mm, mm_stride, st);
        else launch_idx_prefill<128, 1>(p, c, idx_q, idx_w, pos0, nrows, scores, stride, mm, mm_stride, st);
    } else {
        if (two) launch_idx_prefill<32, 2>(p, c, idx_q, idx_w, pos0, nrows, scores, stride, mm, mm_stride, st);
        else launch_idx_prefill<32, 1>(p, c, idx_q, idx_w, pos0, nrows, scores, stride, mm, mm_stride, st);
    }
}

void attend(const sa_params *p, AttnArgs a, int rows, hipStream_t st, StageMarks *mk)
{
    // waves of 32 heads; the 576-wide family runs 2 or 4 waves (a 1- or 3-wave
    // build would need more registers than the pipelined tile loop can spare),
    // waves past num_heads mask their heads
    int nw = (p->num_heads + 31) / 32;
    if (p->qk_dim == 576) nw = nw <= 2 ? 2 : 4;
    dim3 grid(a.splits * (p->v_dim > 256 ? 2 : 1) * rows), block(64 * nw);
    if (p->qk_dim == 576) {
        if (nw == 2) hipLaunchKernelGGL((attend_kernel<576, 512, 2>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attend_kernel<576, 512, 4>), grid, block, 0, st, a);
    } else {
        switch (nw) {
        case 1: hipLaunchKernelGGL((attend_kernel<64, 64, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((attend_kernel<64, 64, 2>), grid, block, 0, st, a); break;
        case 3: hipLaunchKernelGGL((attend_kernel<64, 64, 3>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((attend_kernel<64, 64, 4>), grid, block, 0, st, a); break;
        }
    }
    if (mk) mk->mark();
    if (a.splits > 1) {
        dim3 cg(p->num_heads, rows);
        if (p->v_dim == 512)
            hipLaunchKernelGGL((combine_kernel<512>), cg, dim3(128), 0, st, a.part_o, a.part_ml, a.splits,
                               p->num_heads, a.out, a.out_bf16, a.lse);
        else
            hipLaunchKernelGGL((combine_kernel<64>), cg, dim3(64), 0, st, a.part_o, a.part_ml, a.splits,
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
    if (d.mb_chunks > 0) {
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
        hipLaunchKernelGGL(topk_rows_kernel, dim3(batch), dim3(kTopkThreads), 0, st, scores, d.score_stride, mm,
                           d.mm_stride, 0, c->context_lens, 0, p->topk, topk_idx, ap);
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
    a.part_o = (float *)((char *)ws + d.off_part_o);
    a.part_ml = (float *)((char *)ws + d.off_part_ml);
    attend(p, a, batch, st, mk);
}

void select_prefill(const sa_params *p, const sa_paged_cache *c, int num_rows, int q_start, const void *idx_q,
                    const float *idx_w, int32_t *topk_idx, void *ws, const PrefillPlan &d, hipStream_t st,
                    StageMarks *mk)
{
    float *scores = (float *)((char *)ws + d.off_scores);
    f32x2 *mm = (f32x2 *)((char *)ws + d.off_mm);
    for (int r0 = 0; r0 < num_rows; r0 += d.chunk_rows) {
        const int nr = std::min(d.chunk_rows, num_rows - r0);
        const int pos0 = q_start + r0;
        // rows whose whole context fits in k need no scores
        if (pos0 + nr > p->topk) {
            idx_prefill(p, c, (const uint16_t *)idx_q + (int64_t)r0 * p->idx_heads * p->idx_dim,
                        idx_w + (int64_t)r0 * p->idx_heads, pos0, nr, scores, d.score_stride, mm, d.mm_stride, st);
            if (mk) mk->mark();
        }
        hipLaunchKernelGGL(topk_rows_kernel, dim3(nr), dim3(kTopkThreads), 0, st, scores, d.score_stride, mm,
                           d.mm_stride, 1, (const int32_t *)nullptr, pos0, p->topk, topk_idx + (int64_t)r0 * p->topk,
                           no_append());
        if (mk) mk->mark();
    }
}

void attend_prefill(const sa_params *p, const sa_paged_cache *c, int num_rows, int q_start, const void *q,
                    const int32_t *topk_idx, void *out, float *lse, void *ws, const PrefillPlan &d, hipStream_t st,
                    StageMarks *mk)
{
    for (int r0 = 0; r0 < num_rows; r0 += d.attn_chunk_rows) {
        const int nr = std::min(d.attn_chunk_rows, num_rows - r0);
        AttnArgs a = attn_args(p, c, (const uint16_t *)q + (int64_t)r0 * p->num_heads * p->qk_dim,
                               topk_idx + (int64_t)r0 * p->topk,
                               (char *)out + (int64_t)r0 * p->num_heads * p->v_dim * (p->out_dtype ? 2 : 4),
                               lse ? lse + (int64_t)r0 * p->num_heads : nullptr);
        a.decode = 0;
        a.limit_base = q_start + r0;
        a.tokens_per_split = d.tokens_per_split;
        a.splits = d.splits;
        a.part_o = (float *)((char *)ws + d.off_part_o);
        a.part_ml = (float *)((char *)ws + d.off_part_ml);
        attend(p, a, nr, st, mk);
    }
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
    *bytes = plan_prefill(p, num_rows, q_start).total;
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
                             const void *new_kv = nullptr, const void *new_idx_k = nullptr)
{
    sa_status s = check_decode(p, c, batch, max_ctx, true, true);
    if (s != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !topk_idx || !out) return SA_ERR_NULL;
    const DecodePlan d = plan_decode(p, batch, max_ctx);
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
    const PrefillPlan d = plan_prefill(p, num_rows, q_start);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    clear_hip_error();
    select_prefill(p, c, num_rows, q_start, idx_q, idx_w, topk_idx, workspace, d, (hipStream_t)stream, nullptr);
    return launched();
}

sa_status sparse_attn_attend_prefill(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                                     const void *q, const int32_t *topk_idx, void *out, float *lse, void *workspace,
                                     size_t workspace_bytes, void *stream)
{
    sa_status s = check_prefill(p, c, num_rows, q_start, true, false);
    if (s != SA_OK) return s;
    if (!q || !topk_idx || !out) return SA_ERR_NULL;
    const PrefillPlan d = plan_prefill(p, num_rows, q_start);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    clear_hip_error();
    attend_prefill(p, c, num_rows, q_start, q, topk_idx, out, lse, workspace, d, (hipStream_t)stream, nullptr);
    return launched();
}

static sa_status prefill_impl(const sa_params *p, const sa_paged_cache *c, int32_t num_rows, int32_t q_start,
                              const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                              float *lse, void *workspace, size_t workspace_bytes, void *stream, StageMarks *mk)
{
    sa_status s = check_prefill(p, c, num_rows, q_start, true, true);
    if (s != SA_OK) return s;
    if (!q || !idx_q || !idx_w || !topk_idx || !out) return SA_ERR_NULL;
    const PrefillPlan d = plan_prefill(p, num_rows, q_start);
    if ((s = check_ws(workspace, workspace_bytes, d.total)) != SA_OK) return s;
    hipStream_t st = (hipStream_t)stream;
    clear_hip_error();
    if (mk) {
        mk->stream = st;
        mk->mark();
    }
    select_prefill(p, c, num_rows, q_start, idx_q, idx_w, topk_idx, workspace, d, st, mk);
    attend_prefill(p, c, num_rows, q_start, q, topk_idx, out, lse, workspace, d, st, mk);
    return launched();
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

}  // extern "C"
