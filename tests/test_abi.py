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
