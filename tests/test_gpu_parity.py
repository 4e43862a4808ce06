"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: selected indices bit-exact (the indexer inputs are small integers, so every
score is exact in fp32 on both sides); attention output within 2e-2 max-abs and
2e-3 mean-abs error, each query row's error measured relative to the RMS of that
row's oracle output (a prefill row that keeps one key outputs a V row, RMS ~1,
one that averages 2048 keys has RMS ~0.05, so one RMS for the whole tensor would
weigh rows by their scale); lse within 1e-3 absolute.  Full-size workloads run in the same launch configuration as the
benchmark and compare the rows the oracle can afford, one by one.
"""
import os
import sys
from dataclasses import replace

import numpy as np
import pytest

import oracle
from dsa_sparse_attention_02_amd import synth

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL, LSE_ABS = 2e-2, 2e-3, 1e-3


def say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dsa_sparse_attention_02_amd import sparse_attn as sa
    sa.lib()
    return torch, sa


def run_gpu(dev, w, out_bf16=False, staged=False):
    torch, sa = dev
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"], out_bf16=out_bf16)
    if w["mode"] == "decode":
        max_ctx = int(w["context_lens"].max())
        if staged:
            tk = sa.sparse_attn_select_decode(p, d["cache"], max_ctx, d["idx_q"], d["idx_w"])
            out, lse = sa.sparse_attn_attend_decode(p, d["cache"], max_ctx, d["q"], tk)
            res = (tk, out, lse)
        else:
            res = sa.sparse_attn_decode(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"])
    elif w["mode"] == "varlen":
        assert not staged
        res = sa.sparse_attn_prefill_varlen(p, d["cache"], w["cu_seqlens"], w["q_starts"], d["q"], d["idx_q"],
                                            d["idx_w"])
    else:
        if staged:
            tk = sa.sparse_attn_select_prefill(p, d["cache"], w["q_start"], d["idx_q"], d["idx_w"])
            out, lse = sa.sparse_attn_attend_prefill(p, d["cache"], w["q_start"], d["q"], tk)
            res = (tk, out, lse)
        else:
            res = sa.sparse_attn_prefill(p, d["cache"], w["q_start"], d["q"], d["idx_q"], d["idx_w"])
    torch.cuda.synchronize()
    return res


def compare(w, res, rows=None, tag=""):
    tk_all, out_all, lse_all = res[:3]
    ref = oracle.run_varlen(w, rows=rows) if w["mode"] == "varlen" else oracle.run(w, rows=rows)
    rows = ref["rows"]
    idx = __import__("torch").as_tensor(rows, device=tk_all.device)
    tk = tk_all.index_select(0, idx).cpu().numpy()
    out = out_all.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    lse = lse_all.index_select(0, idx).cpu().numpy().astype(np.float64)
    bad = np.nonzero(~np.all(tk == ref["topk"], axis=1))[0]
    assert len(bad) == 0, f"{tag}: indices differ on rows {rows[bad][:8]}"
    check_outputs(ref, out, lse, rows, tag)
    return ref


def check_outputs(ref, out, lse, rows, tag):
    """Outputs (float64 copies of the listed rows) against the oracle's."""
    assert np.isfinite(out).all(), f"{tag}: non-finite output"
    rms_all = float(np.sqrt(np.mean(ref["out"] ** 2)))
    rms = np.sqrt(np.mean(ref["out"] ** 2, axis=(1, 2), keepdims=True))
    rms = np.where(rms > 0, rms, 1.0)  # empty-context rows: output 0 on both sides
    err = np.abs(out - ref["out"]) / rms
    gerr = np.abs(out - ref["out"]) / rms_all
    empty = np.isneginf(ref["lse"])
    assert np.array_equal(np.isneginf(lse), empty), f"{tag}: empty-context rows disagree"
    lerr = np.abs(np.where(empty, 0, lse) - np.where(empty, 0, ref["lse"]))
    say(f"  {tag}: rows {len(rows)} out err/row-rms max {err.max():.3e} mean {err.mean():.3e}; "
        f"err/global-rms max {gerr.max():.3e} mean {gerr.mean():.3e} (rms {rms_all:.3f}); lse err max {lerr.max():.2e}")
    assert err.max() <= MAX_REL and err.mean() <= MEAN_REL, tag
    assert lerr.max() <= LSE_ABS, tag


MLA = synth.MLA
V64 = replace(MLA, num_heads=8, qk_dim=64, v_dim=64, softmax_scale=1.0 / 8.0)  # MLA indexer, small attention


CASES = {
    "tiny_prefill_L256": lambda: synth.WORKLOADS["tiny_prefill_L256"],
    "decode_ragged": lambda: synth.small_decode("decode_ragged", MLA,
                                                [0, 1, 31, 32, 33, 64, 2047, 2048, 2049, 3000, 5000, 9001], seed=101),
    "decode_k1": lambda: synth.small_decode("decode_k1", MLA, [1, 5, 700, 4099], seed=102, topk=1),
    "decode_k64_ties": lambda: synth.small_decode("decode_k64", MLA, [63, 64, 65, 4000, 12345], seed=103, topk=64,
                                                  idx_int_max=1),
    "decode_k3000_splits": lambda: synth.small_decode("decode_k3000", MLA, [2999, 3000, 3001, 7000], seed=104,
                                                      topk=3000),
    "decode_tiny_shape": lambda: synth.small_decode("decode_tiny", synth.TINY, [0, 3, 16, 64, 65, 300], seed=105),
    "prefill_2500": lambda: synth.small_prefill("prefill_2500", MLA, rows=2500, seed=106),
    "prefill_qstart": lambda: synth.small_prefill("prefill_qstart", MLA, rows=700, q_start=1900, seed=107),
    "prefill_tiny_qstart": lambda: synth.small_prefill("prefill_tiny_qs", synth.TINY, rows=100, q_start=37, seed=108),
    "prefill_k4100": lambda: synth.small_prefill("prefill_k4100", MLA, rows=300, q_start=4000, seed=109, topk=4100),
    # rows with exactly k, and more than k, 32-key tiles (the top-k's tile-maximum bound)
    "decode_k256_bound": lambda: synth.small_decode("decode_k256_bound", MLA, [8191, 8192, 8193, 20000, 65536],
                                                    seed=113, topk=256),
    # head counts that leave waves (or lanes of a wave) without a head
    "decode_h48": lambda: synth.small_decode("decode_h48", replace(MLA, num_heads=48), [1, 40, 2100, 5000], seed=110),
    "decode_h96": lambda: synth.small_decode("decode_h96", replace(MLA, num_heads=96), [2, 33, 2048, 6000], seed=111),
    "decode_tiny_h40": lambda: synth.small_decode("decode_tiny_h40", replace(synth.TINY, num_heads=40), [5, 64, 900],
                                                  seed=112),
    # value width 64 with 32 splits per row: the merge's column loop then runs on
    # 16 lanes of a wave while the split weights sit in lanes 0..31
    "decode_v64_splits": lambda: synth.small_decode("decode_v64_splits", V64, [3000, 2500, 4000, 2049, 5000, 2100],
                                                    seed=115),
}


@pytest.mark.parametrize("name", list(CASES))
def test_parity_small(dev, name):
    spec = CASES[name]()
    say(f"[gpu] parity {name}: mode {spec.mode} seed {spec.seed}")
    w = synth.make(spec)
    compare(w, run_gpu(dev, w), tag=name)


@pytest.mark.parametrize("name", ["decode_ragged", "prefill_2500", "tiny_prefill_L256"])
def test_staged_equals_fused_and_deterministic(dev, name):
    spec = CASES[name]()
    say(f"[gpu] staged/fused/determinism {name}")
    w = synth.make(spec)
    a = run_gpu(dev, w)
    b = run_gpu(dev, w)
    c = run_gpu(dev, w, staged=True)
    for x, y in ((a, b), (a, c)):
        assert np.array_equal(x[0].cpu().numpy(), y[0].cpu().numpy())
        assert np.array_equal(x[1].cpu().numpy(), y[1].cpu().numpy())
        assert np.array_equal(x[2].cpu().numpy(), y[2].cpu().numpy())


def test_block_relabelling_invariance_gpu(dev):
    spec = CASES["decode_ragged"]()
    say("[gpu] block relabelling invariance")
    w = synth.make(spec)
    pool = w["kv"].shape[0]
    perm = np.random.default_rng(17).permutation(pool)
    kv, ik = np.empty_like(w["kv"]), np.empty_like(w["idx_k"])
    kv[perm], ik[perm] = w["kv"], w["idx_k"]
    w2 = dict(w, kv=kv, idx_k=ik, block_table=perm[w["block_table"]].astype(np.int32))
    a, b = run_gpu(dev, w), run_gpu(dev, w2)
    for x, y in zip(a, b):
        assert np.array_equal(x.cpu().numpy(), y.cpu().numpy())


def test_bf16_output(dev):
    spec = CASES["decode_ragged"]()
    say("[gpu] bf16 output")
    w = synth.make(spec)
    compare(w, run_gpu(dev, w, out_bf16=True), tag="decode_ragged bf16 out")


# ------------------------------------------------------- full-size workloads --
FULL_ROWS = {
    "tiny_prefill_L256": None,                       # every row
    "decode_b32_ctx8k": None,                        # every row
    "decode_b64_ctx16k_128k": "ends",                # shortest, longest and a few more
    "decode_b4_ctx1m": [0, 3],
    "prefill_L32k": [0, 1, 2046, 2047, 2048, 2049, 4095, 16000, 31999, 32767],
    "prefill_varlen_8x4k": [0, 1, 2047, 4095, 4096, 8191, 12345, 20480, 28671, 28672, 30000, 32767],
}


@pytest.mark.parametrize("name", list(FULL_ROWS))
def test_parity_full_size(dev, name):
    spec = synth.WORKLOADS[name]
    say(f"[gpu] full-size parity {name}")
    w = synth.make(spec)
    rows = FULL_ROWS[name]
    if rows == "ends":
        ctx = w["context_lens"]
        rows = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 0, 17, 63})
    compare(w, run_gpu(dev, w), rows=rows, tag=name)


def test_parity_scan_score_bursts(dev):
    """About 6M visible keys: each of the scan's 2048 waves scores about 92
    32-key tiles, more than its 80-tile score buffer, so every wave writes a
    full burst mid-segment and a partial one at its end, and a few ranges cross
    a row boundary.  The attention part is kept small (8 heads of dim 64) so the
    cache stays near 2.3 GB; the indexer has the MLA shape."""
    shape = V64
    ctx = [1_000_003, 999_999, 1_000_000, 1_048_576, 1_000_037, 1_000_001]
    spec = synth.small_decode("decode_scan_bursts", shape, ctx, seed=114)
    say("[gpu] scan score bursts, 6 rows of ~1M keys")
    w = synth.make(spec)
    compare(w, run_gpu(dev, w), rows=[0, 3, 5], tag="decode_scan_bursts")


APPEND_CASES = {
    "append_ragged": lambda: synth.small_decode("append_ragged", MLA,
                                                [0, 1, 31, 32, 33, 64, 2047, 2048, 2049, 5000], seed=121),
    "append_k64_ties": lambda: synth.small_decode("append_k64", MLA, [63, 64, 65, 4000], seed=122, topk=64,
                                                  idx_int_max=1),
    "append_tiny": lambda: synth.small_decode("append_tiny", synth.TINY, [0, 3, 16, 64, 65, 300], seed=123),
    "append_decode_b32_ctx8k": lambda: synth.WORKLOADS["decode_b32_ctx8k"],
    # longer than 262144 keys: the many-workgroup top-k stores the new rows
    "append_long_mb": lambda: synth.small_decode("append_long", V64, [300_001, 262_145, 1, 0], seed=124),
}


@pytest.mark.parametrize("name", list(APPEND_CASES))
def test_decode_append_parity(dev, name):
    """sparse_attn_decode_append against the oracle: the cache pools after the
    call equal the oracle-appended pools bit for bit, and indices, output and
    lse are those of the oracle on the appended cache."""
    torch, sa = dev
    spec = APPEND_CASES[name]()
    say(f"[gpu] decode append {name}")
    w = synth.make(spec)
    new_kv, new_idx_k = synth.new_tokens(w)
    w2 = oracle.append(w, new_kv, new_idx_k)
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    nk = torch.from_numpy(new_kv).view(torch.bfloat16).cuda()
    ni = torch.from_numpy(new_idx_k).view(torch.bfloat16).cuda()
    res = sa.sparse_attn_decode_append(p, d["cache"], int(w["context_lens"].max()), nk, ni, d["q"], d["idx_q"],
                                       d["idx_w"])
    torch.cuda.synchronize()
    kv_after = d["cache"].kv.view(torch.int16).cpu().numpy().view(np.uint16)
    ik_after = d["cache"].idx_k.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(kv_after, w2["kv"]), f"{name}: kv pool differs after the append"
    assert np.array_equal(ik_after, w2["idx_k"]), f"{name}: idx_k pool differs after the append"
    rows = None if w["rows"] <= 64 else [0, 1, 15, 31]
    compare(w2, res, rows=rows, tag=f"{name} (appended)")


def _seventy_sequences():
    rng = np.random.default_rng(131)
    rows = [int(x) for x in rng.integers(0, 21, size=70)]
    rows[5] = 0
    assert sum(r > 0 for r in rows) > 64
    return synth.small_varlen("varlen_70", synth.TINY, rows, [int(x) for x in rng.integers(0, 301, size=70)],
                              seed=131)


VARLEN_CASES = {
    # ragged rows, an empty sequence, cached prefixes; some rows select, some keep every key
    "varlen_tiny_ragged": lambda: synth.small_varlen("varlen_tiny", synth.TINY, [3, 0, 17, 1, 40, 256],
                                                     [0, 5, 30, 63, 10, 700], seed=132),
    "varlen_mla_mixed": lambda: synth.small_varlen("varlen_mla", MLA, [1, 700, 0, 33, 1500], [0, 1800, 10, 3000, 0],
                                                   seed=133),
    # more sequences than one launch's 64 pieces: two launches per stage
    "varlen_70_sequences": _seventy_sequences,
    # k = 3000: attention in two splits plus the merge
    "varlen_k3000_splits": lambda: synth.small_varlen("varlen_k3000", MLA, [500, 2600], [2800, 0], seed=134,
                                                      topk=3000),
}


@pytest.mark.parametrize("name", list(VARLEN_CASES))
def test_prefill_varlen_parity(dev, name):
    """sparse_attn_prefill_varlen against the oracle's per-sequence prefill."""
    spec = VARLEN_CASES[name]()
    say(f"[gpu] varlen prefill {name}")
    w = synth.make(spec)
    compare(w, run_gpu(dev, w), tag=name)


def test_prefill_varlen_equals_one_call_per_sequence(dev):
    """Each packed row of the multi-sequence call gets bit for bit what the
    single-sequence prefill gives it for its own sequence alone (block-table
    row s passed as a one-row table)."""
    torch, sa = dev
    spec = VARLEN_CASES["varlen_mla_mixed"]()
    say("[gpu] varlen prefill = one call per sequence")
    w = synth.make(spec)
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    tk, out, lse = sa.sparse_attn_prefill_varlen(p, d["cache"], w["cu_seqlens"], w["q_starts"], d["q"], d["idx_q"],
                                                 d["idx_w"])
    cu, qs = w["cu_seqlens"], w["q_starts"]
    for s in range(len(qs)):
        a, b = int(cu[s]), int(cu[s + 1])
        if a == b:
            continue
        cache = sa.PagedCache(kv=d["cache"].kv, idx_k=d["cache"].idx_k,
                              block_table=d["cache"].block_table[s:s + 1].contiguous(),
                              context_lens=d["cache"].context_lens[s:s + 1].contiguous())
        tk1, out1, lse1 = sa.sparse_attn_prefill(p, cache, int(qs[s]), d["q"][a:b].contiguous(),
                                                 d["idx_q"][a:b].contiguous(), d["idx_w"][a:b].contiguous())
        torch.cuda.synchronize()
        assert torch.equal(tk[a:b], tk1), f"sequence {s}: indices differ"
        assert torch.equal(out[a:b], out1), f"sequence {s}: outputs differ"
        assert torch.equal(lse[a:b], lse1), f"sequence {s}: lse differs"


# ------------------------------------------------- block-granular selection --
BLOCK_CASES = {  # name: (spec, q_block, rows checked (None: all))
    "blk_decode_ragged": (lambda: synth.small_decode("blk_dec", replace(MLA, topk=32),
                                                     [0, 1, 63, 64, 65, 2048, 2049, 5000, 9001, 20000], seed=141),
                          1, None),
    "blk_decode_ties": (lambda: synth.small_decode("blk_ties", replace(MLA, topk=8, idx_int_max=1),
                                                   [600, 4000, 12345], seed=142), 1, None),
    "blk_decode_tiny": (lambda: synth.small_decode("blk_tiny", replace(synth.TINY, topk=4), [0, 3, 16, 64, 65, 300],
                                                   seed=143), 1, None),
    "blk_decode_k64_splits": (lambda: synth.small_decode("blk_k64", replace(MLA, topk=64), [5000, 9000], seed=144),
                              1, None),
    "blk_prefill_2500_q64": (lambda: synth.small_prefill("blk_p2500", replace(MLA, topk=16), rows=2500, seed=145),
                             64, [0, 1, 63, 64, 1000, 2047, 2048, 2499]),
    "blk_prefill_tiny_q16": (lambda: synth.small_prefill("blk_ptiny", replace(synth.TINY, topk=4), rows=256,
                                                         q_start=40, seed=146), 16, None),
    "blk_prefill_q1": (lambda: synth.small_prefill("blk_pq1", replace(MLA, topk=8), rows=300, q_start=1000,
                                                   seed=147), 1, [0, 1, 150, 299]),
    # last query block ragged (44 rows); early rows of a block may see none of its kept blocks
    "blk_prefill_q128": (lambda: synth.small_prefill("blk_pq128", replace(synth.TINY, topk=3), rows=300, seed=148),
                         128, None),
}


def run_blocks_gpu(dev, w, q_block):
    torch, sa = dev
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    if w["mode"] == "decode":
        res = sa.sparse_attn_decode_blocks(p, d["cache"], int(w["context_lens"].max()), d["q"], d["idx_q"],
                                           d["idx_w"])
    else:
        res = sa.sparse_attn_prefill_blocks(p, d["cache"], w["q_start"], q_block, d["q"], d["idx_q"], d["idx_w"])
    torch.cuda.synchronize()
    return res


def compare_blocks(w, res, q_block, rows=None, tag=""):
    torch = __import__("torch")
    blk, out_all, lse_all = res
    ref = oracle.run_blocks(w, q_block=q_block, rows=rows)
    got = blk.index_select(0, torch.as_tensor(ref["groups"], device=blk.device)).cpu().numpy()
    bad = np.nonzero(~np.all(got == ref["blocks"], axis=1))[0]
    assert len(bad) == 0, f"{tag}: kept blocks differ for query blocks {ref['groups'][bad][:8]}"
    idx = torch.as_tensor(ref["rows"], device=out_all.device)
    out = out_all.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    lse = lse_all.index_select(0, idx).cpu().numpy().astype(np.float64)
    check_outputs(ref, out, lse, ref["rows"], tag)


@pytest.mark.parametrize("name", list(BLOCK_CASES))
def test_block_selection_parity(dev, name):
    """Block-granular selection against the oracle's block path: kept block
    ids bit for bit, outputs and lse to the usual bar."""
    spec, qb, rows = BLOCK_CASES[name]
    say(f"[gpu] block selection {name}")
    w = synth.make(spec())
    compare_blocks(w, run_blocks_gpu(dev, w, qb), qb, rows=rows, tag=name)


def test_block_selection_full_size(dev):
    """The mixed-length decode batch (64 rows, contexts 16K-128K) keeping 32
    blocks of 64 tokens per row, on sampled rows."""
    spec = replace(synth.WORKLOADS["decode_b64_ctx16k_128k"], shape=replace(MLA, topk=32))
    say("[gpu] block selection, decode_b64_ctx16k_128k, 32 blocks")
    w = synth.make(spec)
    ctx = w["context_lens"]
    rows = sorted({int(np.argmin(ctx)), int(np.argmax(ctx)), 0, 17, 63})
    compare_blocks(w, run_blocks_gpu(dev, w, 1), 1, rows=rows, tag="blk_decode_b64")


# ------------------------------------------------------- run-time tuning --
@pytest.mark.parametrize("case,splits", [("decode_ragged", 1), ("decode_ragged", 3), ("decode_ragged", 7),
                                         ("decode_ragged", 64), ("decode_v64_splits", 32),
                                         ("decode_v64_splits", 64)])
def test_decode_split_counts(dev, case, splits):
    """The configured decode at several attention split counts matches the
    oracle; value width 64 with 32 and 64 splits drives the merge's
    partial-wave column loop with more splits than active lanes."""
    torch, sa = dev
    spec = CASES[case]()
    say(f"[gpu] {case} with {splits} attention splits")
    w = synth.make(spec)
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    res = sa.sparse_attn_decode_cfg(p, d["cache"], int(w["context_lens"].max()), splits, d["q"], d["idx_q"],
                                    d["idx_w"])
    torch.cuda.synchronize()
    compare(w, res, tag=f"{case} splits={splits}")


def test_decode_tune_then_run(dev):
    """The tuner returns a split count the plan realises; the configured call
    with it matches the oracle."""
    torch, sa = dev
    spec = CASES["decode_ragged"]()
    say("[gpu] decode tuning")
    w = synth.make(spec)
    d = sa.to_device(w)
    p = sa.Params.from_shape(w["shape"])
    max_ctx = int(w["context_lens"].max())
    splits, us = sa.decode_tune(p, d["cache"], max_ctx, d["q"], d["idx_q"], d["idx_w"], reps=3)
    say(f"  tuned: {splits} splits, {us:.1f} us per call")
    assert 1 <= splits <= 64 and us > 0
    res = sa.sparse_attn_decode_cfg(p, d["cache"], max_ctx, splits, d["q"], d["idx_q"], d["idx_w"])
    torch.cuda.synchronize()
    compare(w, res, tag=f"decode_ragged tuned splits={splits}")


def test_block_selection_prefill_chunks(dev):
    """Block-granular prefill over 32768 rows at up to 32K keys: the scores
    come in chunks of 8192 rows (1 GiB each), so query blocks of 64 rows in
    four chunks; rows sampled on both sides of the chunk boundaries."""
    spec = replace(synth.WORKLOADS["prefill_L32k"], shape=replace(MLA, topk=32))
    say("[gpu] block selection, prefill 32K rows in four chunks, query blocks of 64")
    w = synth.make(spec)
    rows = [0, 63, 8191, 8192, 16383, 16384, 20000, 32767]
    compare_blocks(w, run_blocks_gpu(dev, w, 64), 64, rows=rows, tag="blk_prefill_L32k_q64")


def test_decode_large_batch(dev):
    """512 rows of 2049-4000 keys: each persistent scan workgroup's pairs of
    tiles run across many row boundaries (a query and weight reload at each),
    and the attention runs one split per row with no merge."""
    rng = np.random.default_rng(151)
    ctx = [int(x) for x in rng.integers(2049, 4001, size=512)]
    spec = synth.small_decode("decode_b512", MLA, ctx, seed=151)
    say("[gpu] decode, 512 rows of 2049-4000 keys")
    w = synth.make(spec)
    compare(w, run_gpu(dev, w), rows=[0, 1, 2, 255, 256, 257, 400, 511], tag="decode_b512")
