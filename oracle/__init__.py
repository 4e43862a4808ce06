"""ctypes front end of the plain-C CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke entry point and
the benchmark's CPU-baseline leg, never by the library.  It shares no code with
the HIP path; inputs come from the seeded generator.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (plain C11, OpenMP, no fused multiply-add)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC",
                               "-shared", "-D_POSIX_C_SOURCE=200809L", SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i64 = ctypes.c_int64
        L.oracle_rows.restype = ctypes.c_int
        L.oracle_rows.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i64, ctypes.c_int,
                                  ctypes.c_double, P, P, P, i64, P, i64, P, P, P, P, i64, P, P, P,
                                  P, i64, P]
        L.oracle_topk.restype = i64
        L.oracle_topk.argtypes = [P, i64, i64, P]
        L.oracle_append.restype = i64
        L.oracle_append.argtypes = [i64, i64, i64, i64, i64, P, P, P, i64, P, P, P]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of one row of fp32 scores: ascending positions, -1 padded."""
    s = np.ascontiguousarray(scores, dtype=np.float32)
    out = np.empty(k, dtype=np.int32)
    if lib().oracle_topk(_p(s), s.shape[0], k, _p(out)) < 0:
        raise RuntimeError("oracle_topk failed")
    return out


def run(w: dict, rows=None, want_scores: bool = False, stage_seconds=None):
    """Run the oracle on the listed query rows of workload `w` (a dict from
    the synth module).  Returns dict(topk, out, lse[, scores]) with one entry per
    listed row; out/lse are float64."""
    sh = w["shape"]
    mode = 0 if w["mode"] == "decode" else 1
    T = w["rows"]
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    nr = len(rows)
    tk = np.empty((nr, sh.topk), dtype=np.int32)
    o = np.empty((nr, sh.num_heads, sh.v_dim), dtype=np.float64)
    lse = np.empty((nr, sh.num_heads), dtype=np.float64)
    ctx = np.ascontiguousarray(w["context_lens"], dtype=np.int32)
    stride = int(ctx.max()) if len(ctx) else 1
    sc = np.full((nr, max(stride, 1)), np.nan, dtype=np.float32) if want_scores else None
    st = np.zeros(3, dtype=np.float64)
    rc = lib().oracle_rows(mode, sh.num_heads, sh.qk_dim, sh.v_dim, sh.idx_heads, sh.idx_dim,
                           sh.block_size, sh.topk, sh.idx_relu, float(np.float32(sh.softmax_scale)),
                           _p(w["kv"]), _p(w["idx_k"]), _p(w["block_table"]), w["block_table"].shape[1],
                           _p(ctx), w["q_start"], _p(w["q"]), _p(w["idx_q"]), _p(w["idx_w"]),
                           _p(rows), nr, _p(tk), _p(o), _p(lse),
                           _p(sc) if sc is not None else None, max(stride, 1), _p(st))
    if rc != 0:
        raise RuntimeError("oracle_rows failed")
    if stage_seconds is not None:
        stage_seconds += st
    res = dict(topk=tk, out=o, lse=lse, rows=rows)
    if sc is not None:
        res["scores"] = sc
    return res


def run_varlen(w: dict, rows=None, want_scores: bool = False) -> dict:
    """The oracle on a multi-sequence prefill workload (mode 'varlen' of the
    synth module): each packed row is a prefill row of its own sequence, at
    position q_starts[s] + i, over block-table row s; computed one sequence at
    a time with `run` on that sequence alone.  Returns run's dict for the
    listed packed rows."""
    cu = np.asarray(w["cu_seqlens"], dtype=np.int64)
    qs = np.asarray(w["q_starts"], dtype=np.int64)
    T = int(cu[-1])
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    seq_of = np.searchsorted(cu, rows, side="right") - 1
    parts = {}
    for s in np.unique(seq_of):
        s = int(s)
        sel = np.nonzero(seq_of == s)[0]
        a, b = int(cu[s]), int(cu[s + 1])
        sub = dict(w, mode="prefill", rows=b - a, q_start=int(qs[s]), q=w["q"][a:b], idx_q=w["idx_q"][a:b],
                   idx_w=w["idx_w"][a:b], block_table=w["block_table"][s:s + 1],
                   context_lens=np.asarray([qs[s] + b - a], dtype=np.int32))
        parts[s] = (sel, run(sub, rows=rows[sel] - a, want_scores=want_scores))
    sh = w["shape"]
    nr = len(rows)
    res = dict(topk=np.empty((nr, sh.topk), dtype=np.int32), out=np.empty((nr, sh.num_heads, sh.v_dim)),
               lse=np.empty((nr, sh.num_heads)), rows=rows)
    if want_scores:
        res["scores"] = np.full((nr, max(1, int(np.max(w["context_lens"])))), np.nan, dtype=np.float32)
    for sel, r in parts.values():
        for key in ("topk", "out", "lse"):
            res[key][sel] = r[key]
        if want_scores:
            res["scores"][sel, :r["scores"].shape[1]] = r["scores"]
    return res


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_blocks(w: dict, q_block: int = 1, rows=None) -> dict:
    """Block-granular selection ("Day-0 Adaptation: Running Trillion-Parameter
    Models on Domestic AI Accelerators", 3.1: the selection keeps the top-k
    key-value blocks for each query block, under a mask, with the attention's
    block mapping), read as follows.  K = shape.topk counts kept blocks; a KV
    block is a cache block (block_size logical tokens); a query block is one
    decode row, or q_block consecutive rows of a one-sequence prefill.
      1. token scores score_i(s) of each row of the query block G (the
         oracle's indexer, through `run`);
      2. block score of block j = max of score_i(s) over rows i of G and
         tokens s of block j with s <= pos_i; candidates j = 0 .. last_G // bs;
      3. kept = the K candidates of highest block score, ties to the lower j
         (the oracle's top-k on the block scores), ascending, -1 padded;
      4. row i: softmax(scale * q_i . k_s) over the kept tokens s <= pos_i,
         output the weighted latent rows' first v_dim entries, in float64
         (no visible kept token: output 0, lse -inf).
    Returns dict(groups, blocks [groups][K], out [rows][H][v_dim], lse
    [rows][H], rows) for the listed rows (all rows by default)."""
    sh = w["shape"]
    K, bs = sh.topk, sh.block_size
    T = int(w["rows"])
    decode = w["mode"] == "decode"
    qb = 1 if decode else int(q_block)
    rows = np.arange(T, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    ctx = np.asarray(w["context_lens"], dtype=np.int64)
    pos = (ctx - 1) if decode else (int(w["q_start"]) + np.arange(T, dtype=np.int64))
    groups = np.unique(rows // qb)
    blocks = np.full((len(groups), K), -1, dtype=np.int32)
    kept_of = {}
    for gi, g in enumerate(groups):
        members = np.arange(g * qb, min(T, (g + 1) * qb), dtype=np.int64)
        last = int(pos[members].max())
        n = last // bs + 1 if last >= 0 else 0
        if n <= K:
            kept = np.arange(n, dtype=np.int32)
        else:
            sc = run(w, rows=members, want_scores=True)["scores"]
            bscore = np.full(n, -np.inf, dtype=np.float32)
            for m, i in enumerate(members):
                p = int(pos[i])
                for j in range(min(n, p // bs + 1)):
                    bscore[j] = max(bscore[j], sc[m, j * bs:min(p, j * bs + bs - 1) + 1].max())
            kept = topk(bscore, K)
            kept = kept[kept >= 0]
        blocks[gi, :len(kept)] = kept
        kept_of[int(g)] = kept
    nr = len(rows)
    out = np.zeros((nr, sh.num_heads, sh.v_dim))
    lse = np.full((nr, sh.num_heads), -np.inf)
    scale = float(np.float32(sh.softmax_scale))
    for r, i in enumerate(rows):
        kept = kept_of[int(i // qb)]
        toks = (kept[:, None].astype(np.int64) * bs + np.arange(bs)[None, :]).ravel()
        toks = toks[toks <= pos[i]]
        if len(toks) == 0:
            continue
        seq = int(i) if decode else 0
        phys = w["block_table"][seq][toks // bs]
        kv = _bf16_to_f64(w["kv"][phys, toks % bs])          # [n][qk_dim]
        q = _bf16_to_f64(w["q"][i])                          # [H][qk_dim]
        logits = scale * (q @ kv.T)                          # [H][n]
        mx = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - mx)
        z = e.sum(axis=1, keepdims=True)
        out[r] = (e @ kv[:, :sh.v_dim]) / z
        lse[r] = (mx + np.log(z))[:, 0]
    return dict(groups=groups, blocks=blocks, out=out, lse=lse, rows=rows)


def append(w: dict, new_kv: np.ndarray, new_idx_k: np.ndarray) -> dict:
    """Decode workload `w` with each sequence's current token (position
    context_lens[b] - 1) replaced by new_kv[b] / new_idx_k[b] in copies of its
    cache pools.  Returns the new workload dict (the input is left as it was)."""
    sh = w["shape"]
    assert w["mode"] == "decode"
    out = dict(w)
    out["kv"] = np.array(w["kv"], dtype=np.uint16, copy=True, order="C")
    out["idx_k"] = np.array(w["idx_k"], dtype=np.uint16, copy=True, order="C")
    nk = np.ascontiguousarray(new_kv, dtype=np.uint16)
    ni = np.ascontiguousarray(new_idx_k, dtype=np.uint16)
    bt = np.ascontiguousarray(w["block_table"], dtype=np.int32)
    ctx = np.ascontiguousarray(w["context_lens"], dtype=np.int32)
    B = len(ctx)
    assert nk.shape == (B, sh.qk_dim) and ni.shape == (B, sh.idx_dim)
    lib().oracle_append(B, sh.qk_dim, sh.idx_dim, sh.block_size, out["kv"].shape[0], _p(out["kv"]),
                        _p(out["idx_k"]), _p(bt), bt.shape[1], _p(ctx), _p(nk), _p(ni))
    out.pop("kv_logical", None)
    out.pop("idx_k_logical", None)
    return out


def max_threads() -> int:
    return lib().oracle_max_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(n)
