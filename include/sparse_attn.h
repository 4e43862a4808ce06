/*
 * sparse_attn.h -- C ABI of libsparse_attn.so: DSA-style sparse attention over a
 * paged latent KV cache for AMD Instinct MI355X (gfx950).
 *
 * The method has three stages per query row:
 *   1. an indexer scores every visible cached key,
 *   2. a per-query top-k keeps the k best keys under the causal limit
 *      (ties broken by the lower position),
 *   3. softmax attention runs over the gathered latent rows of the kept keys.
 * Sources: "Day-0 Adaptation for LLMs: Implementing Sparse Attention and
 * Low-Precision Weights" (section III.1 and the decode pseudocode: indexer ->
 * top-k -> gather -> attention); "Day-0 Adaptation: Running
 * Trillion-Parameter Models on Domestic AI Accelerators" (section 3.1: a
 * two-call interface, index selection followed by sparse attention, both over
 * one block table; section 3.3: separate prefill and decode paths over the same
 * cache and index structures); "Day-0 Model Adaptation Depends on the Compute
 * Software Stack" (Operator Library Abstraction: the sparse-attention operator
 * takes queries, keys/values and index lists and returns the context vectors).
 *
 * Conventions shared by every entry point
 * ----------------------------------------
 *  - Pointers marked (device) are HIP device pointers; everything else,
 *    including the two structs below, is host memory read only during the call.
 *  - bf16 tensors are raw bfloat16 bit patterns (uint16), row-major, densely
 *    packed in the layouts given below.
 *  - Ownership: the caller allocates and frees every buffer, including the
 *    workspace, whose size comes from the matching *_workspace_size call.  The
 *    library never allocates or frees device memory; calls on different
 *    streams with different workspaces may overlap.  Its only global state
 *    is the static scratch array of sparse_attn_decode_noalloc (below) and
 *    that array's device address, looked up once per device.
 *  - Streams: all work is queued on `stream` (a hipStream_t; NULL = the null
 *    stream).  No call synchronises (except sa_decode_tune, which measures);
 *    SA_OK means "queued".
 *  - Errors: every argument check runs before the first HIP call, so a
 *    rejected call touches no device state.  NULL required pointer ->
 *    SA_ERR_NULL; inconsistent sizes -> SA_ERR_SHAPE; a valid parameter set the
 *    compiled kernels do not cover -> SA_ERR_UNSUPPORTED; workspace too small ->
 *    SA_ERR_WORKSPACE; a launch failure reported by the HIP runtime ->
 *    SA_ERR_HIP.  Device-resident values (context lengths, block-table
 *    entries, indices) are not checked on the host; see the cache struct.
 *  - Outputs are fully overwritten.  Rows with an empty context yield indices
 *    -1, output 0 and lse -inf.
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 1

typedef enum {
    SA_OK = 0,
    SA_ERR_NULL = 1,
    SA_ERR_SHAPE = 2,
    SA_ERR_UNSUPPORTED = 3,
    SA_ERR_WORKSPACE = 4,
    SA_ERR_HIP = 5
} sa_status;

typedef enum { SA_OUT_F32 = 0, SA_OUT_BF16 = 1 } sa_out_dtype;

/*
 * Layer shape and method parameters.
 * Supported (compiled) families:
 *   qk_dim/v_dim in {576/512, 64/64}; idx_dim in {128, 32};
 *   1 <= num_heads <= 128; 1 <= idx_heads <= 64; block_size a power of two
 *   in [1, 1024]; 1 <= topk <= 16384.
 * The key of the attention is latent[0:qk_dim] and the value is
 * latent[0:v_dim] of one shared latent row per token (v_dim <= qk_dim).
 */
typedef struct {
    int32_t num_heads;      /* H: attention query heads */
    int32_t qk_dim;         /* D_qk: latent width used for q.k */
    int32_t v_dim;          /* D_v: leading latent width used as the value */
    int32_t idx_heads;      /* H_idx: indexer query heads */
    int32_t idx_dim;        /* D_idx: indexer q/k width (one key vector per token) */
    int32_t block_size;     /* tokens per cache block */
    int32_t topk;           /* k: keys kept per query row */
    float softmax_scale;    /* logits are softmax_scale * q.k; finite and > 0 */
    int32_t idx_relu;       /* 1: ReLU on each indexer head's dot product; 0: none */
    int32_t out_dtype;      /* sa_out_dtype of `out` */
} sa_params;

/*
 * Paged cache (section 3.2 of the page on domestic AI accelerators: fixed-size
 * blocks addressed through a block table).  Token s of sequence b lives in
 * physical block block_table[b * max_blocks_per_seq + s / block_size] at slot
 * s % block_size.
 *   kv          (device) bf16 [num_blocks][block_size][qk_dim]  latent rows
 *   idx_k       (device) bf16 [num_blocks][block_size][idx_dim] indexer keys
 *   block_table (device) int32 [num_seqs][max_blocks_per_seq]
 *   context_lens(device) int32 [num_seqs]  (decode only; may be NULL for prefill)
 * Contract on device-resident values: context_lens[b] <= max_ctx and
 * <= max_blocks_per_seq * block_size; the block-table entries that cover
 * tokens [0, context_lens[b]) are valid block ids < num_blocks.  Entries past a
 * sequence's last block are never read.  Slots past a sequence's length are
 * never read.
 */
typedef struct {
    const void *kv;
    const void *idx_k;
    int64_t num_blocks;
    const int32_t *block_table;
    int32_t max_blocks_per_seq;
    const int32_t *context_lens;
} sa_paged_cache;

int32_t sa_abi_version(void);
const char *sa_status_string(sa_status s);

/* ---------------------------------------------------------------- decode --
 * One query row per sequence b = 0..batch-1, at position context_lens[b]-1
 * (the cache already holds the current token); it sees keys [0, context_lens[b]).
 *   q       (device) bf16 [batch][num_heads][qk_dim]
 *   idx_q   (device) bf16 [batch][idx_heads][idx_dim]
 *   idx_w   (device) fp32 [batch][idx_heads]   indexer head weights
 *   topk_idx(device, out) int32 [batch][topk]: the kept logical positions in
 *           ascending order, -1 padded when fewer than topk keys are visible
 *   out     (device, out) fp32 or bf16 [batch][num_heads][v_dim]
 *   lse     (device, out, nullable) fp32 [batch][num_heads], natural-log
 *           log-sum-exp of the scaled logits over the kept keys
 * max_ctx is a host-side upper bound on every context_lens[b]; it sizes the
 * workspace and the launch grids.
 */
sa_status sa_decode_workspace_size(const sa_params *p, int32_t batch, int32_t max_ctx,
                                   size_t *bytes /* host, out */);
sa_status sparse_attn_decode(const sa_params *p, const sa_paged_cache *cache, int32_t batch,
                             int32_t max_ctx, const void *q, const void *idx_q,
                             const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream);
/* The two stages of sparse_attn_decode as separate calls over the same block
 * mapping (the index-select / sparse-attention pair of section 3.1).  The
 * select call writes topk_idx; the attend call reads it.  Attend treats any
 * index outside [0, context_lens[b]) as padding.  Both take the decode
 * workspace. */
sa_status sparse_attn_select_decode(const sa_params *p, const sa_paged_cache *cache,
                                    int32_t batch, int32_t max_ctx, const void *idx_q,
                                    const float *idx_w, int32_t *topk_idx, void *workspace,
                                    size_t workspace_bytes, void *stream);
sa_status sparse_attn_attend_decode(const sa_params *p, const sa_paged_cache *cache,
                                    int32_t batch, int32_t max_ctx, const void *q,
                                    const int32_t *topk_idx, void *out, float *lse,
                                    void *workspace, size_t workspace_bytes, void *stream);

/* sparse_attn_decode with the current token of every sequence appended to the
 * cache first: the cache update merged into the decode launches and the
 * block-level incremental update of the paged cache during decode
 * ("Engineering Practices for Day-0 Adaptation of Million-Token Context
 * Models on Domestic AI Chips", Four Key Layers items 2 and 3).
 *   new_kv     (device) bf16 [batch][qk_dim]:  latent row of each current token
 *   new_idx_k  (device) bf16 [batch][idx_dim]: its indexer key
 * Sequence b's current token is position context_lens[b] - 1 (context_lens
 * already counts it); its physical slot, block_table[b][pos / bs] * bs +
 * pos % bs, is overwritten in cache->kv and cache->idx_k (the one call that
 * writes through the cache pointers, declared const for the read-only calls).
 * Sequences with context_lens[b] == 0 append nothing.  As for every call, the
 * block-table entries that cover tokens [0, context_lens[b]), this position's
 * included, must be valid block ids (the cache struct's contract: the scan
 * reads that block).  The scores, indices,
 * output and lse are those of sparse_attn_decode on the updated cache; no
 * kernel is added: the indexer scan scores each current token with its new
 * key, and the top-k launch, which precedes the attention, writes both rows.
 * Other arguments and errors as for sparse_attn_decode; null new_kv or
 * new_idx_k -> SA_ERR_NULL.  Calls that overlap on one cache race. */
sa_status sparse_attn_decode_append(const sa_params *p, const sa_paged_cache *cache, int32_t batch,
                                    int32_t max_ctx, const void *new_kv, const void *new_idx_k,
                                    const void *q, const void *idx_q, const float *idx_w,
                                    int32_t *topk_idx, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* Profiling variant of sparse_attn_decode: identical work, and additionally
 * records caller-created HIP events (hipEvent_t handles in events[0 ..
 * num_events)) on `stream`: events[0] before the first kernel and events[i]
 * after the i-th kernel launch, while capacity lasts.  *num_marks (host, out)
 * receives the number of marks the call takes (kernels + 1), whether or not
 * they all fitted.  Kernel order: indexer scan (omitted when max_ctx <= topk),
 * top-k, attention, split merge (omitted when one split covers topk).  The
 * pages recommend profiling the time split across stages ("Day-0 Model
 * Adaptation Depends on the Compute Software Stack", From Adaptation to
 * Maturity).  events may be NULL when num_events is 0; num_marks is required. */
sa_status sparse_attn_decode_profiled(const sa_params *p, const sa_paged_cache *cache, int32_t batch,
                                      int32_t max_ctx, const void *q, const void *idx_q,
                                      const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream,
                                      void *const *events, int32_t num_events, int32_t *num_marks);

/* --------------------------------------------------------------- prefill --
 * num_rows query rows of sequence 0 (block_table row 0); row i sits at
 * position q_start + i and sees keys [0, q_start + i] (causal limit, itself
 * included).  The cache must hold at least q_start + num_rows tokens.
 * Layouts as for decode with batch replaced by num_rows.  Rows whose visible
 * key count is at most topk attend to all of their keys.  The workspace holds
 * the fp32 scores of a chunk of rows at a time (at most 1 GiB of them, at
 * least 16 rows), so it stays bounded however many rows the call covers.
 */
sa_status sa_prefill_workspace_size(const sa_params *p, int32_t num_rows, int32_t q_start,
                                    size_t *bytes /* host, out */);
sa_status sparse_attn_prefill(const sa_params *p, const sa_paged_cache *cache, int32_t num_rows,
                              int32_t q_start, const void *q, const void *idx_q,
                              const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                              void *workspace, size_t workspace_bytes, void *stream);
sa_status sparse_attn_select_prefill(const sa_params *p, const sa_paged_cache *cache,
                                     int32_t num_rows, int32_t q_start, const void *idx_q,
                                     const float *idx_w, int32_t *topk_idx, void *workspace,
                                     size_t workspace_bytes, void *stream);
/* Profiling variant of sparse_attn_prefill (marks as for the decode variant).
 * Kernel order: per chunk of rows, indexer tile scan (omitted while every row
 * of the chunk sees at most topk keys) then top-k; then the attention kernel
 * (and the split merge when topk > 2048), once per attention chunk. */
sa_status sparse_attn_prefill_profiled(const sa_params *p, const sa_paged_cache *cache,
                                       int32_t num_rows, int32_t q_start, const void *q,
                                       const void *idx_q, const float *idx_w, int32_t *topk_idx,
                                       void *out, float *lse, void *workspace, size_t workspace_bytes,
                                       void *stream, void *const *events, int32_t num_events,
                                       int32_t *num_marks);
/* Attend treats any index outside [0, q_start + i] of row i as padding. */
sa_status sparse_attn_attend_prefill(const sa_params *p, const sa_paged_cache *cache,
                                     int32_t num_rows, int32_t q_start, const void *q,
                                     const int32_t *topk_idx, void *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------- varlen prefill --
 * Prefill rows of several sequences in one call (section 3.3 of the page on
 * domestic AI accelerators: the prefill pathway over the shared paged cache;
 * the page on million-token context models names balancing the load of many
 * sequences at block level and pipelining the select and attention stages by
 * chunk).  Sequence s owns the packed query rows [cu_seqlens[s],
 * cu_seqlens[s+1]) of q, idx_q, idx_w, topk_idx, out and lse, and row s of the
 * block table; its row i sits at position q_starts[s] + i and sees keys
 * [0, q_starts[s] + i].  Each row gets exactly the result that
 * sparse_attn_prefill gives it when called for its sequence alone.
 *   cu_seqlens (host) int32 [num_seqs + 1]: cu_seqlens[0] = 0, non-decreasing
 *              (empty sequences are allowed), cu_seqlens[num_seqs] >= 1 rows
 *   q_starts   (host) int32 [num_seqs]: >= 0; the cache must hold
 *              q_starts[s] + (cu_seqlens[s+1] - cu_seqlens[s]) tokens of a
 *              non-empty sequence s, within max_blocks_per_seq * block_size
 *   the block table must have num_seqs rows (not checkable from here)
 * Both host arrays are read during the call only.  One launch of each kernel
 * covers up to 64 runs of rows of one sequence (more sequences take more
 * launches); the indexer launch starts the rows that see the most keys first.
 * Errors: SA_ERR_NULL for a missing host array, SA_ERR_SHAPE for any
 * violation of the rules above, otherwise as sparse_attn_prefill.
 */
sa_status sa_prefill_varlen_workspace_size(const sa_params *p, int32_t num_seqs, const int32_t *cu_seqlens,
                                           const int32_t *q_starts, size_t *bytes /* host, out */);
sa_status sparse_attn_prefill_varlen(const sa_params *p, const sa_paged_cache *cache, int32_t num_seqs,
                                     const int32_t *cu_seqlens, const int32_t *q_starts, const void *q,
                                     const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                                     float *lse, void *workspace, size_t workspace_bytes, void *stream);
/* Varlen prefill with a schedule choice (NULL = defaults).
 *   pipeline: SA_PREFILL_SERIAL (the default): every score chunk's scan and
 *             top-k, then the attention of all rows, on `stream`.
 *             SA_PREFILL_PIPELINED: the select and attention stages pipelined
 *             by chunk (section III item 3 of the page on implementing sparse
 *             attention and low-precision weights): the scan and top-k of
 *             chunk i + 1 run on `stream` while the attention of chunk i runs
 *             on a second stream that the library creates on first use (one
 *             per device, default priority, kept until the process ends); it
 *             waits for chunk i's top-k and for `stream`'s earlier work
 *             through events, and `stream` waits for its last launch, so the
 *             call is ordered on `stream` like any other.  It applies when the
 *             rows take more than one score chunk and `stream` is not being
 *             captured into a graph (otherwise the serial schedule runs).
 *             The results are the serial schedule's, bit for bit.  On MI355X
 *             it gains nothing at the shapes measured: an attention workgroup
 *             holds a compute unit's LDS, so the stages alternate on each unit
 *             rather than share it.
 *   attn_partners: the attention kernel (SA_ATTN_PARTNERS_*, below).
 * SA_ERR_SHAPE for another pipeline or attn_partners value or nonzero
 * reserved fields; otherwise as sparse_attn_prefill_varlen (same workspace). */
/* Attention kernel of the 576/512 shape family, both compiled in: each
 * 32-head block of a workgroup is worked by 2 partner waves (one wave per
 * SIMD; each partner takes half of the q.k dims and half of the value
 * columns, and both compute the tile's softmax) or by 4 (two waves per SIMD;
 * a quarter of the dims and columns each, the logits reduce-scattered and the
 * softmax split by token between the partners).  Both keep the same
 * selected keys and agree with the oracle to the same tolerance; their
 * outputs differ in rounding only.  Other shapes always take 2. */
#define SA_ATTN_PARTNERS_DEFAULT 0
#define SA_ATTN_PARTNERS_2 2
#define SA_ATTN_PARTNERS_4 4
#define SA_PREFILL_SERIAL 0
#define SA_PREFILL_PIPELINED 1
typedef struct {
    int32_t pipeline;
    int32_t attn_partners; /* SA_ATTN_PARTNERS_* */
    int32_t reserved[2];   /* zero */
} sa_prefill_config;
sa_status sparse_attn_prefill_varlen_cfg(const sa_params *p, const sa_paged_cache *cache, int32_t num_seqs,
                                         const int32_t *cu_seqlens, const int32_t *q_starts,
                                         const sa_prefill_config *cfg, const void *q, const void *idx_q,
                                         const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                         void *workspace, size_t workspace_bytes, void *stream);
/* Profiling variant (marks as for sparse_attn_prefill_profiled). */
sa_status sparse_attn_prefill_varlen_profiled(const sa_params *p, const sa_paged_cache *cache,
                                              int32_t num_seqs, const int32_t *cu_seqlens,
                                              const int32_t *q_starts, const void *q, const void *idx_q,
                                              const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                              void *workspace, size_t workspace_bytes, void *stream,
                                              void *const *events, int32_t num_events,
                                              int32_t *num_marks);

/* ----------------------------------------------------- run-time tuning --
 * Kernel tuning at run time (the page on the compute software stack names
 * auto-tuning of block sizes and unrolling at run time as the next step for
 * sparse attention operators).  Three tunables:
 *   attn_splits: the number of splits of each decode row's k keys across
 *                attention workgroups (merged afterwards).  0 = the library's
 *                choice (one attention workgroup per compute unit over the
 *                batch); otherwise requested splits per row, clamped to what k
 *                allows (32-token multiples of at most 2048 tokens per split).
 *                Results do not depend on it beyond floating-point rounding
 *                order.
 *   topk_path:   the decode top-k's algorithm and unroll for rows of at most
 *                262144 keys: SA_TOPK_DEFAULT (rows of at least 8 k keys take
 *                the one-pass path below, the rest the two-pass threshold
 *                path), SA_TOPK_THRESHOLD (every row two-pass: a histogram
 *                pass, then a marking pass), SA_TOPK_ONEPASS_U2 / _U4 (every
 *                row longer than 2 k one-pass: a 1/16 sample sets a bound, one
 *                pass gathers the keys above it, the top k of those are
 *                selected; 2 or 4 rounds of 4 KB loads in flight per wave, two
 *                compiled variants of the gather loop).  The kept indices are
 *                the same, bit for bit, on every path.
 *   attn_partners: the attention kernel (SA_ATTN_PARTNERS_*, above); results
 *                differ only in floating-point rounding.
 * The best choice depends on the context lengths, the batch and the cache's
 * placement, which only a run on the caller's data measures.
 */
#define SA_TOPK_DEFAULT 0
#define SA_TOPK_THRESHOLD 1
#define SA_TOPK_ONEPASS_U2 2
#define SA_TOPK_ONEPASS_U4 3
typedef struct {
    int32_t attn_splits;
    int32_t topk_path;     /* SA_TOPK_* */
    int32_t attn_partners; /* SA_ATTN_PARTNERS_* */
    int32_t reserved[1];   /* zero */
} sa_decode_config;

/* sparse_attn_decode with a configuration (NULL = defaults; attn_partners
 * picks the attention kernel, SA_ATTN_PARTNERS_*).  SA_ERR_SHAPE for
 * attn_splits outside [0, 1024], topk_path outside the SA_TOPK_* values,
 * attn_partners outside the SA_ATTN_PARTNERS_* values or nonzero reserved
 * fields; otherwise as sparse_attn_decode. */
sa_status sa_decode_workspace_size_cfg(const sa_params *p, int32_t batch, int32_t max_ctx,
                                       const sa_decode_config *cfg, size_t *bytes /* host, out */);
sa_status sparse_attn_decode_cfg(const sa_params *p, const sa_paged_cache *cache, int32_t batch,
                                 int32_t max_ctx, const sa_decode_config *cfg, const void *q,
                                 const void *idx_q, const float *idx_w, int32_t *topk_idx, void *out,
                                 float *lse, void *workspace, size_t workspace_bytes, void *stream);
/* Times sparse_attn_decode_cfg on the given inputs for every split count the
 * plan can realise (up to 64) under the default top-k, then every top-k path
 * under the fastest count, then (576/512 shape) the other attention kernel
 * under both: one untimed call, then `reps` (1..1000) calls
 * between two HIP events on `stream`, per configuration; writes the fastest
 * into *best (and its mean microseconds per call into *best_us when non-NULL).
 * Unlike every other call it creates two HIP events, waits for the stream
 * and leaves the outputs of the last call tried.  The workspace must hold
 * sa_decode_tune_workspace_size bytes (the largest of the candidates). */
sa_status sa_decode_tune_workspace_size(const sa_params *p, int32_t batch, int32_t max_ctx,
                                        size_t *bytes /* host, out */);
sa_status sa_decode_tune(const sa_params *p, const sa_paged_cache *cache, int32_t batch, int32_t max_ctx,
                         const void *q, const void *idx_q, const float *idx_w, int32_t *topk_idx,
                         void *out, float *lse, void *workspace, size_t workspace_bytes, void *stream,
                         int32_t reps, sa_decode_config *best /* host, out */,
                         float *best_us /* host, out, nullable */);

/* ------------------------------------------- block-granular selection --
 * The index selection keeps whole KV blocks per query block (section 3.1 of
 * the page on domestic AI accelerators: the selection operator chooses which
 * key-value blocks take part for each query block, keeps topk of them, under a
 * mask, with the block mapping the attention uses).  Here:
 *   - a KV block is a cache block: logical tokens [j*block_size, (j+1)*block_size)
 *   - a query block is one decode row, or q_block consecutive prefill rows
 *     (the last one may be shorter)
 *   - p->topk = K counts KV blocks; K * block_size <= 16384
 *   - block score of KV block j for query block G = max of the token indexer
 *     scores score_i(s) over rows i of G and tokens s of block j with
 *     s <= pos_i; the candidates are blocks 0 .. (last position of G) /
 *     block_size
 *   - kept: the K candidates of highest block score, equal scores keeping the
 *     lower block id; all candidates when there are at most K
 *   - row i attends (softmax, as in sparse_attn_decode) over the tokens
 *     s <= pos_i of its query block's kept blocks (the causal mask); a
 *     prefill row none of whose kept tokens is visible gets O = 0 and
 *     lse = -inf
 *   block_idx (device, out) int32 [query blocks][K]: kept block ids,
 *     ascending, -1 padded
 *   q, idx_q, idx_w, out, lse: as for the token-level calls
 * Errors as for the token-level calls; SA_ERR_UNSUPPORTED when K *
 * block_size > 16384 or q_block is not a power of two <= 128, SA_ERR_SHAPE
 * when q_block < 1.
 */
sa_status sa_decode_blocks_workspace_size(const sa_params *p, int32_t batch, int32_t max_ctx,
                                          size_t *bytes /* host, out */);
sa_status sparse_attn_decode_blocks(const sa_params *p, const sa_paged_cache *cache, int32_t batch,
                                    int32_t max_ctx, const void *q, const void *idx_q, const float *idx_w,
                                    int32_t *block_idx, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);
sa_status sa_prefill_blocks_workspace_size(const sa_params *p, int32_t num_rows, int32_t q_start,
                                           int32_t q_block, size_t *bytes /* host, out */);
sa_status sparse_attn_prefill_blocks(const sa_params *p, const sa_paged_cache *cache, int32_t num_rows,
                                     int32_t q_start, int32_t q_block, const void *q, const void *idx_q,
                                     const float *idx_w, int32_t *block_idx, void *out, float *lse,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------- allocation-free decode --
 * sparse_attn_decode for callers that cannot allocate device memory at all,
 * not even a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The inputs, outputs and their meaning are
 * those of sparse_attn_decode; the scratch memory (scores, split partials,
 * top-k state) is a static device array inside the library,
 * SA_NOALLOC_SCRATCH_BYTES (128 MiB) on every device the library runs on,
 * held until the process ends.  The call allocates and frees nothing.  Its
 * first call on a device (the caller's current device) looks the array's
 * device address up once and keeps it.
 *  - A batch whose decode workspace (sa_decode_workspace_size) exceeds
 *    SA_NOALLOC_SCRATCH_BYTES -> SA_ERR_WORKSPACE, before any HIP call.
 *    (Batch 64 at 128K keys needs about 69 MB, batch 4 at 1M keys about
 *    41 MB.)
 *  - All calls on one GPU share the array and it keeps the last call's
 *    contents: calls that overlap in time on one GPU (other streams, other
 *    threads) race and give wrong results; serialise them.
 *  - A failure to look up the array's address -> SA_ERR_HIP.
 * Other errors as for sparse_attn_decode. */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
sa_status sparse_attn_decode_noalloc(const sa_params *p, const sa_paged_cache *cache, int32_t batch,
                                     int32_t max_ctx, const void *q, const void *idx_q,
                                     const float *idx_w, int32_t *topk_idx, void *out, float *lse,
                                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
