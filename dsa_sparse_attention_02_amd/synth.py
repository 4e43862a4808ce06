"""Seeded synthetic workloads for DSA sparse attention over a paged latent KV cache.

This module only draws inputs and lays them out in the paged-cache format the
library consumes; it contains none of the method's arithmetic (no scoring, no
selection, no attention).  Both the CPU oracle and the HIP path are fed from it.

Workloads follow the shapes and value distributions the method is exercised on:
a lightweight indexer with small-integer query/key entries stored as bf16 (so
every indexer score is exactly representable and selected indices can be
compared bit for bit), per-head indexer weights drawn from a small set of powers
of two, bf16 N(0,1) queries and latent KV rows, and a paged cache whose block
table is a random permutation of a shared physical pool.  The paged layout (fixed
size blocks addressed through a logical->physical block table) is the one the
pages "Day-0 Adaptation: Running Trillion-Parameter Models on Domestic AI
Accelerators" (section 3.2, KV Cache Layout) and "Engineering Practices for Day-0
Adaptation of Million-Token Context Models on Domestic AI Chips" (Four Key
Layers, item 2) describe.

Random streams: every tensor is drawn from numpy's PCG64 seeded with
``SeedSequence([seed, tensor_id, part, chunk])`` so the values do not depend on
the number of worker threads.  Tensor ids: 0 q, 1 kv, 2 idx_q, 3 idx_k, 4 idx_w,
5 block-pool permutation, 6 context lengths.

Poisoned padding: cache slots that no sequence owns (the tail of each sequence's
last block and a few spare blocks) hold NaN in the latent cache and a large
value (64.0) in the indexer-key cache, and block-table entries past a
sequence's last block point at a spare block.  Any read outside the visible
range therefore corrupts either the selected indices or the output.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)
BF16_POISON_IDX = np.uint16(0x4280)  # 64.0 in bf16
SPARE_BLOCKS = 8

T_Q, T_KV, T_IDX_Q, T_IDX_K, T_IDX_W, T_PERM, T_CTX, T_NEW_KV, T_NEW_IDX_K = range(9)


@dataclass(frozen=True)
class Shape:
    """Head counts and dimensions of one attention layer plus the selection size."""
    num_heads: int          # H, query heads of the sparse attention
    qk_dim: int             # D_qk, latent row width used for logits (K = latent[:D_qk])
    v_dim: int              # D_v, value width (V = latent[:D_v])
    idx_heads: int          # H_idx, indexer query heads
    idx_dim: int            # D_idx, indexer key/query width (one key vector per token)
    block_size: int         # tokens per cache block
    topk: int               # k, keys kept per query
    softmax_scale: float
    idx_int_max: int        # indexer q/k integers are uniform in [-idx_int_max, idx_int_max]
    idx_w_set: tuple        # indexer head weights are drawn uniformly from this set
    idx_relu: int = 1


TINY = Shape(num_heads=8, qk_dim=64, v_dim=64, idx_heads=4, idx_dim=32, block_size=16,
             topk=64, softmax_scale=1.0 / 8.0, idx_int_max=3, idx_w_set=(0.25, 0.5, 1.0))
MLA = Shape(num_heads=128, qk_dim=576, v_dim=512, idx_heads=64, idx_dim=128, block_size=64,
            topk=2048, softmax_scale=1.0 / math.sqrt(576.0), idx_int_max=4,
            idx_w_set=(1.0, 0.5, 0.25, 0.125))


@dataclass(frozen=True)
class Spec:
    """One workload.  mode 'decode': `batch` sequences, query b sits at position
    ctx_b - 1.  mode 'prefill': one sequence of `rows` tokens, row i sits at
    position q_start + i and the cache holds q_start + rows tokens.  mode
    'varlen': sequence s has seq_rows[s] query rows (packed one sequence after
    another), its row i at position q_starts[s] + i, and the cache holds
    q_starts[s] + seq_rows[s] tokens of it."""
    name: str
    mode: str
    shape: Shape
    batch: int = 1
    ctx: Optional[Sequence[int]] = None      # explicit decode context lengths
    ctx_uniform: Optional[tuple] = None      # (lo, hi) inclusive, drawn per sequence
    rows: int = 0                            # prefill rows L
    q_start: int = 0
    seed: int = 1000
    seq_rows: Optional[Sequence[int]] = None   # varlen: query rows per sequence
    q_starts: Optional[Sequence[int]] = None   # varlen: position of each sequence's first row


WORKLOADS = {
    # 1 sequence, L=256, causal; indexer 4x32 ints in [-3,3]; 8 heads x 64 sharing one K/V of 64.
    "tiny_prefill_L256": Spec("tiny_prefill_L256", "prefill", TINY, rows=256, seed=1000),
    # decode, batch 32, every context 8192.
    "decode_b32_ctx8k": Spec("decode_b32_ctx8k", "decode", MLA, batch=32, ctx=[8192] * 32, seed=1001),
    # prefill, 1 sequence, L=32768.
    "prefill_L32k": Spec("prefill_L32k", "prefill", MLA, rows=32768, seed=1002),
    # mixed-length decode, batch 64, contexts uniform in [16384, 131072].
    "decode_b64_ctx16k_128k": Spec("decode_b64_ctx16k_128k", "decode", MLA, batch=64,
                                   ctx_uniform=(16384, 131072), seed=1003),
    # long-context decode, batch 4, each context 1,048,576.
    "decode_b4_ctx1m": Spec("decode_b4_ctx1m", "decode", MLA, batch=4, ctx=[1 << 20] * 4, seed=1004),
    # decode, batch 64, every context 131072: the mixed-length batch at its
    # longest context (a labelled supplementary of the 128K metric)
    "decode_b64_ctx128k_full": Spec("decode_b64_ctx128k_full", "decode", MLA, batch=64, ctx=[1 << 17] * 64,
                                    seed=1006),
    # chunked prefill of 8 sequences in one call: 4096 new rows each after cached
    # prefixes of 0, 4096, ..., 28672 tokens (the same 32768 rows and causal
    # pairs as the single 32K prefill, spread over 8 block-table rows).
    "prefill_varlen_8x4k": Spec("prefill_varlen_8x4k", "varlen", MLA, batch=8, seq_rows=[4096] * 8,
                                q_starts=[4096 * i for i in range(8)], seed=1005),
}


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bit patterns (inputs are finite)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(seed: int, ids: tuple, n: int) -> np.ndarray:
    return f32_to_bf16_bits(_rng(seed, *ids).standard_normal(n, dtype=np.float32))


def _ints_bf16(seed: int, ids: tuple, n: int, a: int) -> np.ndarray:
    v = _rng(seed, *ids).integers(-a, a, size=n, endpoint=True, dtype=np.int8)
    return f32_to_bf16_bits(v.astype(np.float32))


def context_lengths(spec: Spec) -> np.ndarray:
    if spec.mode == "prefill":
        return np.array([spec.q_start + spec.rows], dtype=np.int32)
    if spec.mode == "varlen":
        return (np.asarray(spec.q_starts, dtype=np.int64) + np.asarray(spec.seq_rows, dtype=np.int64)).astype(
            np.int32)
    if spec.ctx is not None:
        c = np.asarray(spec.ctx, dtype=np.int32)
        assert c.shape == (spec.batch,)
        return c
    lo, hi = spec.ctx_uniform
    return _rng(spec.seed, T_CTX).integers(lo, hi, size=spec.batch, endpoint=True).astype(np.int32)


CHUNK_TOKENS = 16384


def make(spec: Spec, keep_logical: bool = False, workers: Optional[int] = None) -> dict:
    """Draw every input of `spec`.  Returns a dict of numpy arrays (bf16 data as
    uint16 bit patterns) plus metadata.  With keep_logical, also returns each
    sequence's cache rows in logical order (`kv_logical[b]`, `idx_k_logical[b]`),
    which tests use to build references that never touch the block table."""
    sh = spec.shape
    seed = spec.seed
    bs = sh.block_size
    ctx = context_lengths(spec)
    nseq = len(ctx)
    nblk = [(int(c) + bs - 1) // bs for c in ctx]
    used = int(sum(nblk))
    pool = used + SPARE_BLOCKS
    perm = _rng(seed, T_PERM).permutation(pool).astype(np.int32)
    max_blocks = max(1, max(nblk))
    spare = perm[used:]
    table = np.empty((nseq, max_blocks), dtype=np.int32)
    off = 0
    for b in range(nseq):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        table[b, nblk[b]:] = spare[b % SPARE_BLOCKS]
        off += nblk[b]

    kv = np.empty((pool, bs, sh.qk_dim), dtype=np.uint16)
    idx_k = np.empty((pool, bs, sh.idx_dim), dtype=np.uint16)
    kv[spare] = BF16_NAN
    idx_k[spare] = BF16_POISON_IDX
    kv_log = [None] * nseq
    ik_log = [None] * nseq

    jobs = []
    for b in range(nseq):
        c = int(ctx[b])
        if keep_logical:
            kv_log[b] = np.empty((c, sh.qk_dim), dtype=np.uint16)
            ik_log[b] = np.empty((c, sh.idx_dim), dtype=np.uint16)
        for ci, t0 in enumerate(range(0, c, CHUNK_TOKENS)):
            jobs.append((b, ci, t0, min(c, t0 + CHUNK_TOKENS)))

    def fill(job):
        b, ci, t0, t1 = job
        n = t1 - t0
        kvc = _normal_bf16(seed, (T_KV, b, ci), n * sh.qk_dim).reshape(n, sh.qk_dim)
        ikc = _ints_bf16(seed, (T_IDX_K, b, ci), n * sh.idx_dim, sh.idx_int_max).reshape(n, sh.idx_dim)
        if keep_logical:
            kv_log[b][t0:t1] = kvc
            ik_log[b][t0:t1] = ikc
        # lay the logical rows out in their physical blocks (chunks are block aligned)
        j0 = t0 // bs
        full = n // bs
        if full:
            blocks = table[b, j0:j0 + full]
            kv[blocks] = kvc[:full * bs].reshape(full, bs, sh.qk_dim)
            idx_k[blocks] = ikc[:full * bs].reshape(full, bs, sh.idx_dim)
        rem = n - full * bs
        if rem:
            blk = table[b, j0 + full]
            kv[blk, :rem] = kvc[full * bs:]
            kv[blk, rem:] = BF16_NAN
            idx_k[blk, :rem] = ikc[full * bs:]
            idx_k[blk, rem:] = BF16_POISON_IDX

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(fill, jobs))

    if spec.mode == "decode":
        T = spec.batch
    elif spec.mode == "prefill":
        T = spec.rows
    else:
        T = int(sum(spec.seq_rows))
    # per-row streams so large prefill queries are drawn in parallel too
    q = np.empty((T, sh.num_heads, sh.qk_dim), dtype=np.uint16)
    rows_per = max(1, (1 << 22) // (sh.num_heads * sh.qk_dim))

    def fill_q(r0):
        r1 = min(T, r0 + rows_per)
        q[r0:r1] = _normal_bf16(seed, (T_Q, r0), (r1 - r0) * sh.num_heads * sh.qk_dim).reshape(
            r1 - r0, sh.num_heads, sh.qk_dim)

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(fill_q, range(0, T, rows_per)))

    idx_q = _ints_bf16(seed, (T_IDX_Q,), T * sh.idx_heads * sh.idx_dim, sh.idx_int_max).reshape(
        T, sh.idx_heads, sh.idx_dim)
    wset = np.asarray(sh.idx_w_set, dtype=np.float32)
    idx_w = wset[_rng(seed, T_IDX_W).integers(0, len(wset), size=(T, sh.idx_heads))]

    out = dict(spec=spec, shape=sh, mode=spec.mode, q=q, idx_q=idx_q, idx_w=idx_w,
               kv=kv, idx_k=idx_k, block_table=table, context_lens=ctx,
               num_blocks=pool, max_blocks=max_blocks, rows=T, q_start=spec.q_start)
    if spec.mode == "varlen":
        out["cu_seqlens"] = np.concatenate([[0], np.cumsum(spec.seq_rows)]).astype(np.int32)
        out["q_starts"] = np.asarray(spec.q_starts, dtype=np.int32)
    if keep_logical:
        out["kv_logical"] = kv_log
        out["idx_k_logical"] = ik_log
    return out


def new_tokens(w: dict):
    """The current token of each decode sequence, to be appended: its latent
    row (bf16 N(0,1), [B][qk_dim]) and indexer key (integers in
    [-idx_int_max, idx_int_max] as bf16, [B][idx_dim]), drawn like the cache
    rows from their own streams."""
    spec, sh = w["spec"], w["shape"]
    B = spec.batch
    new_kv = _normal_bf16(spec.seed, (T_NEW_KV,), B * sh.qk_dim).reshape(B, sh.qk_dim)
    new_idx_k = _ints_bf16(spec.seed, (T_NEW_IDX_K,), B * sh.idx_dim, sh.idx_int_max).reshape(B, sh.idx_dim)
    return new_kv, new_idx_k


def small_decode(name: str, shape: Shape, ctx: Sequence[int], seed: int = 7, **kw) -> Spec:
    return Spec(name, "decode", replace(shape, **kw) if kw else shape, batch=len(ctx), ctx=list(ctx), seed=seed)


def small_prefill(name: str, shape: Shape, rows: int, q_start: int = 0, seed: int = 7, **kw) -> Spec:
    return Spec(name, "prefill", replace(shape, **kw) if kw else shape, rows=rows, q_start=q_start, seed=seed)


def small_varlen(name: str, shape: Shape, seq_rows: Sequence[int], q_starts: Sequence[int], seed: int = 7,
                 **kw) -> Spec:
    assert len(seq_rows) == len(q_starts)
    return Spec(name, "varlen", replace(shape, **kw) if kw else shape, batch=len(seq_rows), seq_rows=list(seq_rows),
                q_starts=list(q_starts), seed=seed)
