"""Pins of the CPU oracle against facts fixed by mathematics, not by the oracle itself.

Each test below would fail on a plausible slip in the oracle: a dropped ReLU or
head weight, a transposed operand, a wrong paged address, a tie broken the wrong
way, a softmax over the wrong dimension, V taken from the wrong columns.

* exact integer closed form of the indexer (the inputs are small integers, so
  8 * score is an integer computed in int64 with no rounding at all);
* the rank definition of top-k checked by brute force on small rows;
* special cases of top-k (k >= n, k = 1 is the first argmax, all ties);
* dense brute-force attention on contiguous (never paged) K/V in float64,
  which the oracle must equal when k >= n;
* closed forms of softmax attention (zero query -> mean of V rows, k = 1 ->
  that V row, logit shift invariance);
* invariance of every result under a relabelling of physical blocks and under
  a change of the poisoned padding;
* a hand-worked example (tests/golden/handworked_decode.json).
"""
import json
import math
import os
from dataclasses import replace
from fractions import Fraction

import numpy as np
import pytest

import oracle
from dsa_sparse_attention_02_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MLA_SMALL = replace(synth.MLA, topk=2048)


def _logical_f32(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _int_scores_x(w, row, kind_scale):
    """kind_scale * score of every visible key, in exact int64 arithmetic."""
    sh = w["shape"]
    if w["mode"] == "decode":
        seq, n = row, int(w["context_lens"][row])
    else:
        seq, n = 0, w["q_start"] + row + 1
    iq = synth.bf16_bits_to_f32(w["idx_q"][row]).astype(np.int64)          # [Hidx][Didx]
    ik = synth.bf16_bits_to_f32(w["idx_k_logical"][seq][:n]).astype(np.int64)  # [n][Didx]
    d = ik @ iq.T                                                            # [n][Hidx]
    if sh.idx_relu:
        d = np.maximum(d, 0)
    wi = w["idx_w"][row].astype(np.float64) * kind_scale
    assert np.all(wi == np.round(wi))
    return d @ wi.astype(np.int64)


@pytest.mark.parametrize("which", ["mla_decode", "tiny_prefill"])
def test_indexer_exact_integer_closed_form(which):
    if which == "mla_decode":
        spec = synth.small_decode("pin_idx", MLA_SMALL, [1, 37, 700, 1500], seed=11)
        scale = 8  # weights are 1, 1/2, 1/4, 1/8
    else:
        spec = synth.small_prefill("pin_idx_tiny", synth.TINY, rows=96, seed=12)
        scale = 4  # weights are 1, 1/2, 1/4
    w = synth.make(spec, keep_logical=True)
    rows = list(range(w["rows"]))[:4] if which == "mla_decode" else [0, 1, 17, 63, 95]
    res = oracle.run(w, rows=rows, want_scores=True)
    for r, row in enumerate(rows):
        exact = _int_scores_x(w, row, scale)
        got = res["scores"][r][: len(exact)].astype(np.float64) * scale
        assert np.array_equal(got, exact.astype(np.float64)), (which, row)


def _rank_topk(scores, k):
    n = len(scores)
    keep = []
    for s in range(n):
        better = sum(1 for m in range(n) if scores[m] > scores[s] or (scores[m] == scores[s] and m < s))
        if better < k:
            keep.append(s)
    return keep


def test_topk_bruteforce_rank_definition():
    rng = np.random.default_rng(5)
    for trial in range(60):
        n = int(rng.integers(1, 400))
        k = int(rng.integers(1, 80))
        # few distinct values -> many exact ties at the threshold
        scores = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.5)
        got = oracle.topk(scores, k)
        want = _rank_topk(scores.tolist(), k)
        kept = got[got >= 0]
        assert list(kept) == want, (trial, n, k)
        assert np.all(got[len(kept):] == -1)
        assert np.all(np.diff(kept) > 0)


def test_topk_composability():
    """Under the strict order (score descending, position ascending), the top k
    of a row equal the top k of the union of its chunks' own top k (the property
    that lets a long row's selection run per chunk, then once over the
    survivors).  Chunks are contiguous ranges or arbitrary subsets; scores take
    few distinct values so ties cross chunk boundaries."""
    rng = np.random.default_rng(23)
    for trial in range(80):
        n = int(rng.integers(1, 600))
        k = int(rng.integers(1, 90))
        scores = rng.integers(-4, 5, size=n).astype(np.float32) * np.float32(0.25)
        if trial % 2 == 0:  # contiguous chunks
            cuts = np.sort(rng.choice(np.arange(1, max(n, 2)), size=min(n - 1, int(rng.integers(0, 6))), replace=False))
            parts = np.split(np.arange(n), cuts)
        else:  # arbitrary subsets
            lab = rng.integers(0, 4, size=n)
            parts = [np.nonzero(lab == c)[0] for c in range(4)]
        survivors = []
        for part in parts:
            if len(part) == 0:
                continue
            local = oracle.topk(scores[part], k)
            survivors.extend(part[local[local >= 0]].tolist())
        union = np.array(sorted(survivors), dtype=np.int64)  # ascending positions: array order = position order
        sel = oracle.topk(scores[union], k)
        got = union[sel[sel >= 0]]
        want = oracle.topk(scores, k)
        want = want[want >= 0]
        assert np.array_equal(got, want), (trial, n, k)


def test_topk_special_cases():
    rng = np.random.default_rng(9)
    s = rng.standard_normal(50).astype(np.float32)
    # k >= n keeps everything
    assert list(oracle.topk(s, 50)) == list(range(50))
    assert list(oracle.topk(s, 64)) == list(range(50)) + [-1] * 14
    # k = 1 is the first argmax
    t = rng.integers(0, 5, size=200).astype(np.float32)
    assert oracle.topk(t, 1)[0] == int(np.argmax(t))
    # all equal scores keep the lowest positions
    assert list(oracle.topk(np.full(300, 2.5, np.float32), 7)) == list(range(7))
    # -0 and +0 are the same score: ties broken by position
    z = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    assert list(oracle.topk(z, 2)) == [0, 1]
    # empty row
    assert list(oracle.topk(np.zeros(0, np.float32), 3)) == [-1, -1, -1]


def _dense_attention(q, kv_rows, sel, scale, v_dim):
    """Brute-force softmax attention in float64 on contiguous rows."""
    k = kv_rows[sel]                        # [n][Dqk]
    logits = scale * (q @ k.T)              # [H][n]
    m = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - m)
    z = e.sum(axis=1, keepdims=True)
    o = (e @ k[:, :v_dim]) / z
    return o, (m + np.log(z))[:, 0]


@pytest.mark.parametrize("which", ["tiny_prefill_k_eq_L", "mla_decode_short"])
def test_attention_equals_dense_when_k_covers_context(which):
    if which == "tiny_prefill_k_eq_L":
        spec = synth.small_prefill("pin_dense", synth.TINY, rows=256, seed=21, topk=256)
        rows = [0, 1, 15, 16, 100, 255]
    else:
        spec = synth.small_decode("pin_dense_mla", MLA_SMALL, [1, 64, 65, 300], seed=22)
        rows = [0, 1, 2, 3]
    w = synth.make(spec, keep_logical=True)
    sh = w["shape"]
    res = oracle.run(w, rows=rows)
    scale = float(np.float32(sh.softmax_scale))
    for r, row in enumerate(rows):
        if w["mode"] == "decode":
            seq, n = row, int(w["context_lens"][row])
        else:
            seq, n = 0, row + 1
        sel = np.arange(n)
        assert list(res["topk"][r][:n]) == list(sel)
        assert np.all(res["topk"][r][n:] == -1)
        o, lse = _dense_attention(_logical_f32(w["q"][row]), _logical_f32(w["kv_logical"][seq][:n]),
                                  sel, scale, sh.v_dim)
        np.testing.assert_allclose(res["out"][r], o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][r], lse, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    spec = synth.small_decode("pin_closed", MLA_SMALL, [3000, 2049, 5], seed=31)
    w = synth.make(spec, keep_logical=True)
    sh = w["shape"]
    base = oracle.run(w)

    # zero query: every logit is 0, so o is the mean of the kept V rows and lse = log(kept)
    wz = dict(w, q=np.zeros_like(w["q"]))
    rz = oracle.run(wz)
    for b in range(3):
        sel = rz["topk"][b][rz["topk"][b] >= 0]
        assert np.array_equal(sel, base["topk"][b][base["topk"][b] >= 0])
        v = _logical_f32(w["kv_logical"][b][sel])[:, : sh.v_dim]
        np.testing.assert_allclose(rz["out"][b], np.broadcast_to(v.mean(axis=0), rz["out"][b].shape),
                                   rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rz["lse"][b], math.log(len(sel)), rtol=1e-14)

    # k = 1: the output is exactly the V row of the first best-scoring key
    w1 = synth.make(replace(spec, shape=replace(MLA_SMALL, topk=1)), keep_logical=True)
    r1 = oracle.run(w1, want_scores=True)
    scale = float(np.float32(sh.softmax_scale))
    for b in range(3):
        n = int(w1["context_lens"][b])
        s = int(np.argmax(r1["scores"][b][:n]))
        assert r1["topk"][b][0] == s
        row = _logical_f32(w1["kv_logical"][b][s])
        np.testing.assert_array_equal(r1["out"][b], np.broadcast_to(row[: sh.v_dim], r1["out"][b].shape))
        np.testing.assert_allclose(r1["lse"][b], scale * (_logical_f32(w1["q"][b]) @ row), rtol=1e-12)

    # logit shift: make the non-V columns of every key equal, then change the
    # matching part of q.  All logits of a head move by one constant, so o stays
    # put and lse moves by exactly that constant.
    ws = synth.make(spec, keep_logical=True)
    c = synth.f32_to_bf16_bits(np.linspace(-1, 1, sh.qk_dim - sh.v_dim, dtype=np.float32))
    ws["kv"][:, :, sh.v_dim:] = c
    for b in range(3):
        ws["kv_logical"][b][:, sh.v_dim:] = c
    r_a = oracle.run(ws)
    q2 = ws["q"].copy()
    q2[:, :, sh.v_dim:] = synth.f32_to_bf16_bits(
        np.random.default_rng(3).standard_normal(q2[:, :, sh.v_dim:].shape).astype(np.float32))
    r_b = oracle.run(dict(ws, q=q2))
    np.testing.assert_allclose(r_b["out"], r_a["out"], rtol=1e-11, atol=1e-12)
    cf = _logical_f32(c)
    for b in range(3):
        shift = scale * (_logical_f32(q2[b][:, sh.v_dim:]) - _logical_f32(ws["q"][b][:, sh.v_dim:])) @ cf
        np.testing.assert_allclose(r_b["lse"][b] - r_a["lse"][b], shift, rtol=1e-9, atol=1e-9)


def _relabel_blocks(w, seed):
    """Move every physical block to a new slot and rewrite the block table to match."""
    pool = w["kv"].shape[0]
    perm = np.random.default_rng(seed).permutation(pool)
    kv = np.empty_like(w["kv"])
    ik = np.empty_like(w["idx_k"])
    kv[perm] = w["kv"]
    ik[perm] = w["idx_k"]
    return dict(w, kv=kv, idx_k=ik, block_table=perm[w["block_table"]].astype(np.int32))


@pytest.mark.parametrize("which", ["decode", "prefill"])
def test_block_relabelling_and_poison_invariance(which):
    if which == "decode":
        spec = synth.small_decode("pin_perm", replace(MLA_SMALL, topk=256), [1, 63, 64, 65, 2500], seed=41)
    else:
        spec = synth.small_prefill("pin_perm_p", synth.TINY, rows=200, seed=42)
    w = synth.make(spec)
    a = oracle.run(w)
    b = oracle.run(_relabel_blocks(w, 7))
    assert np.array_equal(a["topk"], b["topk"])
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["lse"], b["lse"])
    # different poison in every slot nobody owns: nothing changes
    wp = dict(w, kv=w["kv"].copy(), idx_k=w["idx_k"].copy())
    owned = np.zeros(w["kv"].shape[:2], dtype=bool)
    ctx = w["context_lens"]
    bs = w["shape"].block_size
    for s_ in range(len(ctx)):
        for t in range(int(ctx[s_])):
            owned[w["block_table"][s_, t // bs], t % bs] = True
    wp["kv"][~owned] = 0x3F80      # 1.0
    wp["idx_k"][~owned] = 0xC2C8   # -100.0
    c = oracle.run(wp)
    assert np.array_equal(a["topk"], c["topk"])
    assert np.array_equal(a["out"], c["out"])


def test_handworked_decode():
    g = json.load(open(os.path.join(GOLDEN, "handworked_decode.json")))
    s = g["shape"]
    sh = synth.Shape(num_heads=s["num_heads"], qk_dim=s["qk_dim"], v_dim=s["v_dim"],
                     idx_heads=s["idx_heads"], idx_dim=s["idx_dim"], block_size=s["block_size"],
                     topk=s["topk"], softmax_scale=s["softmax_scale"], idx_int_max=3,
                     idx_w_set=(1.0,), idx_relu=s["idx_relu"])
    bs, nb = sh.block_size, g["num_blocks"]
    table = np.array(g["block_table"], dtype=np.int32)
    kv = np.full((nb, bs, sh.qk_dim), synth.BF16_NAN, dtype=np.uint16)
    ik = np.full((nb, bs, sh.idx_dim), synth.BF16_POISON_IDX, dtype=np.uint16)
    lk = np.array(g["logical_idx_k"], dtype=np.float32)
    lv = np.array(g["logical_kv"], dtype=np.float32)
    for t in range(g["context_len"]):
        ik[table[0, t // bs], t % bs] = synth.f32_to_bf16_bits(lk[t])
        kv[table[0, t // bs], t % bs] = synth.f32_to_bf16_bits(lv[t])
    w = dict(shape=sh, mode="decode", rows=1, q_start=0, kv=kv, idx_k=ik, block_table=table,
             context_lens=np.array([g["context_len"]], dtype=np.int32),
             q=synth.f32_to_bf16_bits(np.array(g["q"], np.float32))[None],
             idx_q=synth.f32_to_bf16_bits(np.array(g["idx_q"], np.float32))[None],
             idx_w=np.array([g["idx_w"]], dtype=np.float32))
    res = oracle.run(w, want_scores=True)

    # expected values in exact rational arithmetic
    iq = [[Fraction(int(x)) for x in r] for r in g["idx_q"]]
    wt = [Fraction(x) for x in g["idx_w"]]
    exp_scores = []
    for key in g["logical_idx_k"]:
        sc = Fraction(0)
        for j in range(sh.idx_heads):
            d = sum(iq[j][c] * key[c] for c in range(sh.idx_dim))
            sc += wt[j] * max(d, 0)
        exp_scores.append(sc)
    assert [Fraction(float(x)) for x in res["scores"][0][:4]] == exp_scores
    order = sorted(range(4), key=lambda t: (-exp_scores[t], t))
    kept = sorted(order[: sh.topk])
    assert list(res["topk"][0]) == kept == [0, 1]
    q = g["q"][0]
    logits = [sum(q[c] * g["logical_kv"][t][c] for c in range(sh.qk_dim)) * s["softmax_scale"] for t in kept]
    e = [math.exp(x) for x in logits]
    o = [sum(e[i] * g["logical_kv"][t][v] for i, t in enumerate(kept)) / sum(e) for v in range(sh.v_dim)]
    np.testing.assert_allclose(res["out"][0][0], o, rtol=1e-15)
    np.testing.assert_allclose(res["lse"][0][0], math.log(sum(e)), rtol=1e-15)
    np.testing.assert_allclose(o, [math.e / (1 + math.e), (4 + 8 * math.e) / (1 + math.e)], rtol=1e-15)


def test_generator_is_thread_count_independent():
    spec = synth.small_decode("gen", MLA_SMALL, [20000, 5], seed=3)
    a = synth.make(spec, workers=1)
    b = synth.make(spec, workers=4)
    for key in ("kv", "idx_k", "q", "idx_q", "idx_w", "block_table", "context_lens"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("which", ["mla_decode_short", "tiny_decode"])
def test_append_writes_the_current_token(which):
    """The oracle's decode append, pinned to the logical view of the cache the
    generator keeps (never paged): after appending, dense brute-force attention
    and the exact integer indexer over the logical rows with row ctx - 1
    replaced by the new token equal the oracle's results on the appended
    (paged) workload; exactly one pool row per non-empty sequence changed."""
    if which == "mla_decode_short":
        spec = synth.small_decode("pin_append_mla", MLA_SMALL, [0, 1, 64, 65, 300], seed=41)
    else:
        spec = synth.small_decode("pin_append_tiny", replace(synth.TINY, topk=256), [0, 1, 15, 16, 17, 200],
                                  seed=42)
    w = synth.make(spec, keep_logical=True)
    sh = w["shape"]
    new_kv, new_idx_k = synth.new_tokens(w)
    w2 = oracle.append(w, new_kv, new_idx_k)
    ctx = w["context_lens"]
    live = [b for b in range(len(ctx)) if ctx[b] > 0]
    changed_kv = np.nonzero(np.any(w2["kv"].reshape(-1, sh.qk_dim) != w["kv"].reshape(-1, sh.qk_dim), axis=1))[0]
    changed_ik = np.nonzero(np.any(w2["idx_k"].reshape(-1, sh.idx_dim) != w["idx_k"].reshape(-1, sh.idx_dim),
                                   axis=1))[0]
    assert len(changed_kv) == len(live) and len(changed_ik) == len(live)
    new_rows = {tuple(new_kv[b]) for b in live}
    assert all(tuple(w2["kv"].reshape(-1, sh.qk_dim)[i]) in new_rows for i in changed_kv)
    # the logical view after the append
    kv_log = [np.array(a, copy=True) for a in w["kv_logical"]]
    ik_log = [np.array(a, copy=True) for a in w["idx_k_logical"]]
    for b in live:
        kv_log[b][ctx[b] - 1] = new_kv[b]
        ik_log[b][ctx[b] - 1] = new_idx_k[b]
    res = oracle.run(w2, want_scores=True)
    scale = float(np.float32(sh.softmax_scale))
    wl = dict(w2, idx_k_logical=ik_log)
    for b in range(len(ctx)):
        n = int(ctx[b])
        assert n <= sh.topk
        if n == 0:
            assert np.all(res["topk"][b] == -1) and np.all(res["out"][b] == 0)
            continue
        o, lse = _dense_attention(_logical_f32(w["q"][b]), _logical_f32(kv_log[b][:n]), np.arange(n), scale,
                                  sh.v_dim)
        np.testing.assert_allclose(res["out"][b], o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][b], lse, rtol=1e-12, atol=1e-12)
        x8 = _int_scores_x(wl, b, 8)
        assert np.array_equal((res["scores"][b][:n].astype(np.float64) * 8).astype(np.int64), x8)


def test_varlen_rows_follow_their_own_sequence():
    """Multi-sequence prefill in the oracle, pinned to the logical (never paged)
    rows the generator keeps: with k covering every context, each packed row
    equals dense brute-force attention over its own sequence's first
    q_starts[s] + i + 1 rows, and its indexer scores equal the exact integer
    closed form over that sequence's keys.  Ragged rows, an empty sequence and
    prefixes already in the cache."""
    spec = synth.small_varlen("pin_varlen", replace(synth.TINY, topk=256), [3, 0, 17, 1, 40], [0, 5, 30, 63, 10],
                              seed=51)
    w = synth.make(spec, keep_logical=True)
    sh = w["shape"]
    res = oracle.run_varlen(w, want_scores=True)
    scale = float(np.float32(sh.softmax_scale))
    cu, qs = w["cu_seqlens"], w["q_starts"]
    checked = 0
    for s in range(len(qs)):
        for i in range(int(cu[s + 1] - cu[s])):
            r = int(cu[s]) + i
            n = int(qs[s]) + i + 1
            assert list(res["topk"][r][:n]) == list(range(n)) and np.all(res["topk"][r][n:] == -1)
            o, lse = _dense_attention(_logical_f32(w["q"][r]), _logical_f32(w["kv_logical"][s][:n]), np.arange(n),
                                      scale, sh.v_dim)
            np.testing.assert_allclose(res["out"][r], o, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res["lse"][r], lse, rtol=1e-12, atol=1e-12)
            iq = synth.bf16_bits_to_f32(w["idx_q"][r]).astype(np.int64)
            ik = synth.bf16_bits_to_f32(w["idx_k_logical"][s][:n]).astype(np.int64)
            d = ik @ iq.T
            if sh.idx_relu:
                d = np.maximum(d, 0)
            wi = w["idx_w"][r].astype(np.float64) * 8
            x8 = d @ wi.astype(np.int64)
            assert np.array_equal((res["scores"][r][:n].astype(np.float64) * 8).astype(np.int64), x8)
            checked += 1
    assert checked == int(cu[-1])


def test_varlen_single_rows_equal_decode():
    """A multi-sequence prefill whose sequences each hold one row at position
    ctx - 1 is the decode of that batch: the oracle's varlen path (per-sequence
    prefill over its block-table row) and its decode path (row b over
    block-table row b, limit ctx_b) agree, with selection active (ctx > k)."""
    ctx = [1, 64, 65, 3000, 2049]
    vspec = synth.small_varlen("pin_varlen_dec", MLA_SMALL, [1] * len(ctx), [c - 1 for c in ctx], seed=52)
    w = synth.make(vspec)
    dec = dict(w, mode="decode", rows=len(ctx), q_start=0)
    a = oracle.run_varlen(w)
    b = oracle.run(dec)
    assert np.array_equal(a["topk"], b["topk"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-12, atol=1e-12)
    assert np.sum(a["topk"][3] >= 0) == MLA_SMALL.topk


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_blocks_of_one_token_are_tokens(mode):
    """Block-granular selection with one-token blocks and one-row query blocks
    is token selection: the oracle's block path (numpy block maxima, float64
    attention in numpy) gives the token path's indices (C oracle), and the
    same outputs."""
    shape = replace(synth.TINY, block_size=1, topk=8)
    if mode == "decode":
        spec = synth.small_decode("pin_blk1_dec", shape, [0, 1, 8, 9, 40, 200], seed=61)
    else:
        spec = synth.small_prefill("pin_blk1_pre", shape, rows=40, q_start=5, seed=62)
    w = synth.make(spec)
    a = oracle.run_blocks(w, q_block=1)
    b = oracle.run(w)
    assert np.array_equal(a["blocks"], b["topk"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_blocks_covering_the_context_are_dense(mode):
    """When every candidate block is kept, each row attends over its whole
    causal context: dense brute force over the logical rows."""
    if mode == "decode":
        spec = synth.small_decode("pin_blk_dense", replace(synth.TINY, topk=32), [0, 1, 15, 16, 17, 300], seed=63)
        qb = 1
    else:
        spec = synth.small_prefill("pin_blk_dense_p", replace(synth.TINY, topk=32), rows=100, q_start=200, seed=64)
        qb = 16
    w = synth.make(spec, keep_logical=True)
    sh = w["shape"]
    res = oracle.run_blocks(w, q_block=qb)
    scale = float(np.float32(sh.softmax_scale))
    for r in range(w["rows"]):
        seq, n = (r, int(w["context_lens"][r])) if mode == "decode" else (0, w["q_start"] + r + 1)
        if n == 0:
            assert np.all(res["out"][r] == 0) and np.all(np.isneginf(res["lse"][r]))
            continue
        o, lse = _dense_attention(_logical_f32(w["q"][r]), _logical_f32(w["kv_logical"][seq][:n]), np.arange(n),
                                  scale, sh.v_dim)
        np.testing.assert_allclose(res["out"][r], o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(res["lse"][r], lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode", ["decode", "prefill"])
def test_block_ranking_from_exact_integer_scores(mode):
    """The kept blocks follow from the exact integer indexer (int64 closed form
    over the logical keys): block maxima over the query block's rows and their
    visible tokens, ranked by score, ties to the lower block id."""
    if mode == "decode":
        spec = synth.small_decode("pin_blk_rank", replace(MLA_SMALL, topk=8), [1000, 3000, 700], seed=65)
        qb = 1
    else:
        spec = synth.small_prefill("pin_blk_rank_p", replace(synth.TINY, topk=3, idx_int_max=1), rows=64,
                                   q_start=100, seed=66)
        qb = 16
    w = synth.make(spec, keep_logical=True)
    sh = w["shape"]
    res = oracle.run_blocks(w, q_block=qb)
    bs = sh.block_size
    for gi, g in enumerate(res["groups"]):
        members = range(g * qb, min(w["rows"], (g + 1) * qb))
        best = {}
        for i in members:
            x8 = _int_scores_x(w, i, 8)            # 8 * score of every visible token, exact
            for s, v in enumerate(x8):
                best[s // bs] = max(best.get(s // bs, v), v)
        order = sorted(best, key=lambda j: (-best[j], j))
        want = sorted(order[:sh.topk])
        got = [int(j) for j in res["blocks"][gi] if j >= 0]
        assert got == want, (g, got, want)
