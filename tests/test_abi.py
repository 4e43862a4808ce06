"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments with the documented status before
any HIP call (every pointer passed here is a dummy that must never be touched)."""
import ctypes
import os
import re

import pytest

from dsa_sparse_attention_02_amd import sparse_attn as sa
from dsa_sparse_attention_02_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sa.LIB_PATH):
        from dsa_sparse_attention_02_amd import build
        build.build()
    return sa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:sa_status|int32_t|const char \*)\s*\**\s*([a-z_][a-z0-9_]*)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(sa.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.sa_abi_version() == 1
    for s in range(6):
        assert len(sa.status_string(s)) > 0
    assert sa.status_string(99) == "unknown status"


def _params(**kw):
    return sa.Params.from_shape(synth.MLA).c() if not kw else sa.sa_params(**{**dict(
        num_heads=128, qk_dim=576, v_dim=512, idx_heads=64, idx_dim=128, block_size=64, topk=2048,
        softmax_scale=1.0 / 24, idx_relu=1, out_dtype=0), **kw})


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails or returns first


def _cache(**kw):
    base = dict(kv=FAKE.value, idx_k=FAKE.value, num_blocks=64, block_table=FAKE.value, max_blocks_per_seq=4,
                context_lens=FAKE.value)
    base.update(kw)
    return sa.sa_paged_cache(**base)


def _decode(L, p, c, batch=2, max_ctx=256, ws_bytes=1 << 40, **ptrs):
    args = dict(q=FAKE, idx_q=FAKE, idx_w=FAKE, topk=FAKE, out=FAKE, lse=None, ws=FAKE)
    args.update(ptrs)
    return L.sparse_attn_decode(ctypes.byref(p) if p is not None else None,
                                ctypes.byref(c) if c is not None else None, batch, max_ctx, args["q"],
                                args["idx_q"], args["idx_w"], args["topk"], args["out"], args["lse"], args["ws"],
                                ws_bytes, None)


def test_decode_validation(L):
    p, c = _params(), _cache()
    assert _decode(L, None, c) == sa.SA_ERR_NULL
    assert _decode(L, p, None) == sa.SA_ERR_NULL
    assert _decode(L, p, c, q=None) == sa.SA_ERR_NULL
    assert _decode(L, p, c, topk=None) == sa.SA_ERR_NULL
    assert _decode(L, p, _cache(context_lens=None)) == sa.SA_ERR_NULL
    assert _decode(L, p, _cache(kv=None)) == sa.SA_ERR_NULL
    assert _decode(L, p, c, ws=None) == sa.SA_ERR_NULL
    assert _decode(L, p, c, batch=0) == sa.SA_ERR_SHAPE
    assert _decode(L, p, c, max_ctx=-1) == sa.SA_ERR_SHAPE
    assert _decode(L, p, c, max_ctx=257) == sa.SA_ERR_SHAPE       # > max_blocks * block_size
    assert _decode(L, _params(topk=0), c) == sa.SA_ERR_SHAPE
    assert _decode(L, _params(v_dim=600), c) == sa.SA_ERR_SHAPE
    assert _decode(L, _params(out_dtype=7), c) == sa.SA_ERR_SHAPE
    assert _decode(L, _params(softmax_scale=float("nan")), c) == sa.SA_ERR_SHAPE
    # a zero or negative scale would make the padding slots' masked logits
    # meaningless (0 * -inf) and the reference max a minimum: rejected
    assert _decode(L, _params(softmax_scale=0.0), c) == sa.SA_ERR_SHAPE
    assert _decode(L, _params(softmax_scale=-0.125), c) == sa.SA_ERR_SHAPE
    assert _decode(L, _params(qk_dim=128, v_dim=128), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode(L, _params(idx_dim=64), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode(L, _params(num_heads=256), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode(L, _params(idx_heads=128), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode(L, _params(block_size=48), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode(L, _params(topk=16385), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode(L, p, c, ws_bytes=16) == sa.SA_ERR_WORKSPACE
    assert _decode(L, p, _cache(num_blocks=0)) == sa.SA_ERR_SHAPE


def test_prefill_and_staged_validation(L):
    p, c = _params(), _cache(context_lens=None)
    P = ctypes.byref
    assert L.sparse_attn_prefill(P(p), P(c), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) \
        == sa.SA_ERR_SHAPE
    assert L.sparse_attn_prefill(P(p), P(c), 200, 100, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 40, None) \
        == sa.SA_ERR_SHAPE  # 300 tokens > 4 blocks of 64
    assert L.sparse_attn_prefill(P(p), P(c), 8, 0, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None) \
        == sa.SA_ERR_NULL
    assert L.sparse_attn_prefill(P(p), P(c), 8, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 8, None) \
        == sa.SA_ERR_WORKSPACE
    # the select stage needs no latent cache, the attend stage no indexer cache
    assert L.sparse_attn_select_prefill(P(p), P(_cache(idx_k=None, context_lens=None)), 8, 0, FAKE, FAKE, FAKE,
                                        FAKE, 1 << 40, None) == sa.SA_ERR_NULL
    assert L.sparse_attn_attend_prefill(P(p), P(_cache(kv=None, context_lens=None)), 8, 0, FAKE, FAKE, FAKE, None,
                                        FAKE, 1 << 40, None) == sa.SA_ERR_NULL
    assert L.sparse_attn_select_decode(P(p), P(_cache()), 2, 256, FAKE, None, FAKE, FAKE, 1 << 40, None) \
        == sa.SA_ERR_NULL
    assert L.sparse_attn_attend_decode(P(p), P(_cache()), 2, 256, FAKE, FAKE, FAKE, None, FAKE, 3, None) \
        == sa.SA_ERR_WORKSPACE


def test_workspace_sizes(L):
    for name in ("decode_b32_ctx8k", "decode_b64_ctx16k_128k", "decode_b4_ctx1m"):
        spec = synth.WORKLOADS[name]
        p = sa.Params.from_shape(spec.shape)
        ctx = synth.context_lengths(spec)
        n = sa.decode_workspace_size(p, spec.batch, int(ctx.max()))
        # at least the fp32 score rows
        assert n >= spec.batch * int(ctx.max()) * 4
        assert n < (1 << 31)
    p = sa.Params.from_shape(synth.MLA)
    n = sa.prefill_workspace_size(p, 32768, 0)
    assert (1 << 20) < n <= (1 << 30) + (300 << 20)  # score rows are processed in chunks of at most 1 GiB
    with pytest.raises(sa.SparseAttnError):
        sa.decode_workspace_size(p, 0, 10)
    with pytest.raises(sa.SparseAttnError):
        sa.prefill_workspace_size(p, 10, -1)


def _decode_append(L, p, c, batch=2, max_ctx=256, ws_bytes=1 << 40, **ptrs):
    args = dict(new_kv=FAKE, new_idx_k=FAKE, q=FAKE, idx_q=FAKE, idx_w=FAKE, topk=FAKE, out=FAKE, lse=None, ws=FAKE)
    args.update(ptrs)
    return L.sparse_attn_decode_append(ctypes.byref(p) if p is not None else None,
                                       ctypes.byref(c) if c is not None else None, batch, max_ctx, args["new_kv"],
                                       args["new_idx_k"], args["q"], args["idx_q"], args["idx_w"], args["topk"],
                                       args["out"], args["lse"], args["ws"], ws_bytes, None)


def test_decode_append_validation(L):
    """The append call checks its two new-token pointers, then everything the
    decode call checks, before any HIP call."""
    p, c = _params(), _cache()
    assert _decode_append(L, p, c, new_kv=None) == sa.SA_ERR_NULL
    assert _decode_append(L, p, c, new_idx_k=None) == sa.SA_ERR_NULL
    assert _decode_append(L, None, c) == sa.SA_ERR_NULL
    assert _decode_append(L, p, c, q=None) == sa.SA_ERR_NULL
    assert _decode_append(L, p, _cache(kv=None)) == sa.SA_ERR_NULL
    assert _decode_append(L, p, c, batch=0) == sa.SA_ERR_SHAPE
    assert _decode_append(L, p, c, max_ctx=257) == sa.SA_ERR_SHAPE
    assert _decode_append(L, _params(idx_dim=64), c) == sa.SA_ERR_UNSUPPORTED
    assert _decode_append(L, p, c, ws_bytes=16) == sa.SA_ERR_WORKSPACE


def _i32(*v):
    return (ctypes.c_int32 * max(1, len(v)))(*v)


def _varlen(L, p, c, cu=(0, 3, 3, 10), qs=(0, 5, 200), ws_bytes=1 << 40, n=None, **ptrs):
    args = dict(q=FAKE, idx_q=FAKE, idx_w=FAKE, topk=FAKE, out=FAKE, lse=None, ws=FAKE)
    args.update(ptrs)
    cu_a = _i32(*cu) if cu is not None else None
    qs_a = _i32(*qs) if qs is not None else None
    return L.sparse_attn_prefill_varlen(ctypes.byref(p) if p is not None else None,
                                        ctypes.byref(c) if c is not None else None,
                                        (3 if qs is None else len(qs)) if n is None else n, cu_a, qs_a, args["q"], args["idx_q"],
                                        args["idx_w"], args["topk"], args["out"], args["lse"], args["ws"], ws_bytes,
                                        None)


def test_prefill_varlen_validation(L):
    """The multi-sequence prefill checks its host arrays (start at 0, never
    decrease, some row, every non-empty sequence within the cache), then what
    the single-sequence prefill checks, before any HIP call."""
    p, c = _params(), _cache()  # cache: 4 blocks per sequence of 64 tokens = 256 positions
    assert _varlen(L, p, c, cu=None) == sa.SA_ERR_NULL
    assert _varlen(L, p, c, qs=None) == sa.SA_ERR_NULL
    assert _varlen(L, None, c) == sa.SA_ERR_NULL
    assert _varlen(L, p, None) == sa.SA_ERR_NULL
    assert _varlen(L, p, c, q=None) == sa.SA_ERR_NULL
    assert _varlen(L, p, _cache(idx_k=None)) == sa.SA_ERR_NULL
    assert _varlen(L, p, c, n=0) == sa.SA_ERR_SHAPE
    assert _varlen(L, p, c, cu=(1, 3, 3, 10)) == sa.SA_ERR_SHAPE      # must start at 0
    assert _varlen(L, p, c, cu=(0, 3, 2, 10)) == sa.SA_ERR_SHAPE      # decreasing
    assert _varlen(L, p, c, cu=(0, 0, 0, 0)) == sa.SA_ERR_SHAPE       # no row at all
    assert _varlen(L, p, c, qs=(0, -1, 200)) == sa.SA_ERR_SHAPE       # negative start (empty sequence too)
    assert _varlen(L, p, c, qs=(0, 5, 250)) == sa.SA_ERR_SHAPE        # 250 + 7 rows > 256 positions
    # an empty sequence's start is not bounded by the cache: validation passes
    # and the workspace check stops the call (before any launch)
    assert _varlen(L, p, c, qs=(0, 300, 249), ws_bytes=16) == sa.SA_ERR_WORKSPACE
    assert _varlen(L, _params(idx_dim=64), c) == sa.SA_ERR_UNSUPPORTED
    assert _varlen(L, p, c, ws_bytes=16) == sa.SA_ERR_WORKSPACE
    # the workspace of the varlen call is that of one sequence of the same rows
    # and longest context
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.sa_prefill_varlen_workspace_size(ctypes.byref(p), 3, _i32(0, 3, 3, 10), _i32(0, 5, 200),
                                              ctypes.byref(a)) == sa.SA_OK
    assert L.sa_prefill_workspace_size(ctypes.byref(p), 10, 197, ctypes.byref(b)) == sa.SA_OK
    assert a.value == b.value > 0
    assert L.sa_prefill_varlen_workspace_size(ctypes.byref(p), 3, None, _i32(0, 5, 200),
                                              ctypes.byref(a)) == sa.SA_ERR_NULL


def test_decode_noalloc_validation(L):
    """The allocation-free decode checks what sparse_attn_decode checks, and
    rejects a batch whose workspace would exceed its static scratch array with
    SA_ERR_WORKSPACE, all before any HIP call."""
    p, c = _params(), _cache()
    f = L.sparse_attn_decode_noalloc
    ok = (FAKE,) * 5 + (None, None)
    assert f(None, ctypes.byref(c), 2, 256, *ok) == sa.SA_ERR_NULL
    assert f(ctypes.byref(p), None, 2, 256, *ok) == sa.SA_ERR_NULL
    assert f(ctypes.byref(p), ctypes.byref(c), 2, 256, None, *ok[1:]) == sa.SA_ERR_NULL
    assert f(ctypes.byref(p), ctypes.byref(c), 0, 256, *ok) == sa.SA_ERR_SHAPE
    assert f(ctypes.byref(_params(softmax_scale=0.0)), ctypes.byref(c), 2, 256, *ok) == sa.SA_ERR_SHAPE
    # 2048 rows of 64K keys need far more than 128 MiB of scores
    big = _cache(max_blocks_per_seq=1024)
    assert f(ctypes.byref(p), ctypes.byref(big), 2048, 65536, *ok) == sa.SA_ERR_WORKSPACE
    n = ctypes.c_size_t()
    assert L.sa_decode_workspace_size(ctypes.byref(p), 2048, 65536, ctypes.byref(n)) == sa.SA_OK
    assert n.value > (128 << 20)


def test_varlen_binding_host_array_errors(L):
    """The binding checks the host arrays of the multi-sequence prefill before
    it touches a tensor and raises SparseAttnError with SA_ERR_SHAPE: a
    cu_seqlens of the wrong length, and one that does not end at the row count
    of q (the tensors here live on the CPU, so the checks must come first)."""
    torch = pytest.importorskip("torch")
    p = sa.Params.from_shape(synth.MLA)
    q = torch.zeros((5, 1, 1), dtype=torch.bfloat16)
    for cu, qs in (([0, 5], [0, 0]), ([0, 2, 5, 5], [0, 0]), ([0, 3], [0])):
        with pytest.raises(sa.SparseAttnError) as e:
            sa.sparse_attn_prefill_varlen(p, None, cu, qs, q, q, q)
        assert e.value.status == sa.SA_ERR_SHAPE, (cu, qs)
    with pytest.raises(sa.SparseAttnError) as e:
        sa.prefill_varlen_workspace_size(p, [0, 2, 5, 7], [0, 0])
    assert e.value.status == sa.SA_ERR_SHAPE


def test_block_selection_validation(L):
    """The block-granular calls check K * block_size <= 16384 and q_block (a
    power of two <= 128) besides what the token calls check, before any HIP
    call."""
    p, c = _params(topk=32), _cache()
    F = FAKE

    def dec(pp=p, cc=c, batch=2, max_ctx=256, ws=1 << 40, q=F):
        return L.sparse_attn_decode_blocks(ctypes.byref(pp), ctypes.byref(cc), batch, max_ctx, q, F, F, F, F, None,
                                           F, ws, None)

    def pre(pp=p, cc=c, rows=100, q_start=0, qb=16, ws=1 << 40, q=F):
        return L.sparse_attn_prefill_blocks(ctypes.byref(pp), ctypes.byref(cc), rows, q_start, qb, q, F, F, F, F,
                                            None, F, ws, None)

    assert dec(q=None) == sa.SA_ERR_NULL and pre(q=None) == sa.SA_ERR_NULL
    assert dec(pp=_params(topk=257)) == sa.SA_ERR_UNSUPPORTED      # 257 * 64 > 16384
    assert pre(pp=_params(topk=257)) == sa.SA_ERR_UNSUPPORTED
    assert dec(batch=0) == sa.SA_ERR_SHAPE and dec(max_ctx=257) == sa.SA_ERR_SHAPE
    assert pre(qb=0) == sa.SA_ERR_SHAPE
    assert pre(qb=24) == sa.SA_ERR_UNSUPPORTED and pre(qb=256) == sa.SA_ERR_UNSUPPORTED
    assert pre(rows=200, q_start=100) == sa.SA_ERR_SHAPE            # 300 > 256 positions
    assert dec(ws=16) == sa.SA_ERR_WORKSPACE and pre(ws=16) == sa.SA_ERR_WORKSPACE
    n = ctypes.c_size_t()
    assert L.sa_decode_blocks_workspace_size(ctypes.byref(p), 2, 256, ctypes.byref(n)) == sa.SA_OK and n.value > 0
    assert L.sa_prefill_blocks_workspace_size(ctypes.byref(p), 100, 0, 128, ctypes.byref(n)) == sa.SA_OK
    assert L.sa_prefill_blocks_workspace_size(ctypes.byref(p), 100, 0, 3, ctypes.byref(n)) == sa.SA_ERR_UNSUPPORTED


def test_prefill_varlen_cfg_validation(L):
    """The configured varlen prefill checks its schedule before any HIP call."""
    p, c = _params(), _cache()
    F = FAKE
    cu = (ctypes.c_int32 * 2)(0, 4)
    qs = (ctypes.c_int32 * 1)(0)

    def call(cfg, ws=1 << 40):
        return L.sparse_attn_prefill_varlen_cfg(ctypes.byref(p), ctypes.byref(c), 1, cu, qs,
                                                ctypes.byref(cfg) if cfg is not None else None, F, F, F, F, F,
                                                None, F, ws, None)

    assert call(sa.sa_prefill_config(pipeline=2)) == sa.SA_ERR_SHAPE
    assert call(sa.sa_prefill_config(pipeline=-1)) == sa.SA_ERR_SHAPE
    bad = sa.sa_prefill_config()
    bad.reserved[1] = 1
    assert call(bad) == sa.SA_ERR_SHAPE
    for partners in (-1, 1, 3, 8):
        assert call(sa.sa_prefill_config(attn_partners=partners)) == sa.SA_ERR_SHAPE
    for partners in (sa.SA_ATTN_PARTNERS_2, sa.SA_ATTN_PARTNERS_4):
        assert call(sa.sa_prefill_config(attn_partners=partners), ws=16) == sa.SA_ERR_WORKSPACE
    assert call(sa.sa_prefill_config(pipeline=sa.SA_PREFILL_PIPELINED), ws=16) == sa.SA_ERR_WORKSPACE
    assert call(None, ws=16) == sa.SA_ERR_WORKSPACE


def test_decode_cfg_and_tune_validation(L):
    """The configured decode and the tuner check the configuration, the
    repetition count and the workspace before any HIP call."""
    p, c = _params(), _cache()
    F = FAKE

    def cfg_call(cfg, ws=1 << 40):
        return L.sparse_attn_decode_cfg(ctypes.byref(p), ctypes.byref(c), 2, 256,
                                        ctypes.byref(cfg) if cfg is not None else None, F, F, F, F, F, None, F, ws,
                                        None)

    assert cfg_call(sa.sa_decode_config(attn_splits=-1)) == sa.SA_ERR_SHAPE
    assert cfg_call(sa.sa_decode_config(attn_splits=2000)) == sa.SA_ERR_SHAPE
    assert cfg_call(sa.sa_decode_config(topk_path=-1)) == sa.SA_ERR_SHAPE
    assert cfg_call(sa.sa_decode_config(topk_path=sa.SA_TOPK_ONEPASS_U4 + 1)) == sa.SA_ERR_SHAPE
    bad = sa.sa_decode_config()
    bad.reserved[0] = 3
    assert cfg_call(bad) == sa.SA_ERR_SHAPE
    for partners in (-1, 1, 3, 8):
        assert cfg_call(sa.sa_decode_config(attn_partners=partners)) == sa.SA_ERR_SHAPE
    for partners in (sa.SA_ATTN_PARTNERS_2, sa.SA_ATTN_PARTNERS_4):
        assert cfg_call(sa.sa_decode_config(attn_partners=partners), ws=16) == sa.SA_ERR_WORKSPACE
    assert cfg_call(sa.sa_decode_config(topk_path=sa.SA_TOPK_ONEPASS_U4), ws=16) == sa.SA_ERR_WORKSPACE
    assert cfg_call(None, ws=16) == sa.SA_ERR_WORKSPACE
    assert cfg_call(sa.sa_decode_config(attn_splits=7), ws=16) == sa.SA_ERR_WORKSPACE
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.sa_decode_workspace_size_cfg(ctypes.byref(p), 2, 256, None, ctypes.byref(a)) == sa.SA_OK
    assert L.sa_decode_workspace_size(ctypes.byref(p), 2, 256, ctypes.byref(b)) == sa.SA_OK
    assert a.value == b.value
    for path in (sa.SA_TOPK_THRESHOLD, sa.SA_TOPK_ONEPASS_U2, sa.SA_TOPK_ONEPASS_U4):  # (the same workspace)
        cfg = sa.sa_decode_config(topk_path=path)
        assert L.sa_decode_workspace_size_cfg(ctypes.byref(p), 2, 256, ctypes.byref(cfg), ctypes.byref(b)) == sa.SA_OK
        assert b.value == a.value
    assert L.sa_decode_tune_workspace_size(ctypes.byref(p), 2, 256, ctypes.byref(b)) == sa.SA_OK
    assert b.value >= a.value
    best, us = sa.sa_decode_config(), ctypes.c_float()

    def tune(reps=5, ws=1 << 40, best_p=ctypes.byref(best)):
        return L.sa_decode_tune(ctypes.byref(p), ctypes.byref(c), 2, 256, F, F, F, F, F, None, F, ws, None, reps,
                                best_p, ctypes.byref(us))

    assert tune(best_p=None) == sa.SA_ERR_NULL
    assert tune(reps=0) == sa.SA_ERR_SHAPE
    assert tune(ws=16) == sa.SA_ERR_WORKSPACE
