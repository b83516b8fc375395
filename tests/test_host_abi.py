"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/qkv.h, sizes its arena by the closed-form layout and
rejects every invalid call before enqueuing anything.

Only calls that fail validation are made here (with a fake, never
dereferenced, device address), so nothing reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

import kv_cache_quantization_head_amd as qkv
from kv_cache_quantization_head_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000          # aligned fake device address, never dereferenced


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qkv_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = qkv.lib()
    names = _declared_functions()
    assert len(names) == 15, names
    for n in names:
        assert hasattr(L, n), n
    assert "qkv_encode_chunk" in names and "qkv_attend" in names


def _cfg(**kw):
    base = dict(n_layers=2, n_heads=12, head_dim=128, n_clusters=256, n_stages=2, bits=2,
                group_size=32, kmeans_iters=5, max_tokens=37440, max_chunk_tokens=32760,
                max_chunks=4, kv_dtype=B.QKV_BF16, max_query_tokens=4680)
    base.update(kw)
    return B.config(**base)


def _align(x, a=256):
    return (x + a - 1) // a * a


def test_workspace_bytes_matches_layout_closed_form():
    cfg = _cfg()
    H, d, T, S, C, G, K = 12, 128, 37440, 2, 256, 32, 4
    header = _align(8 + 4 * 257)
    codes = _align(S * H * T * d * 2 // 8)
    meta = _align(S * H * T * (d // G) * 4)
    ids = _align(H * T)
    cb = _align(K * H * C * d * 2)
    cn = _align(K * H * C * 4)
    stream = header + codes + meta + ids + cb + cn
    attn = _align(_align(8 * H * 4680 * d * 4) + 8 * H * 4680 * 4)
    assert qkv.workspace_bytes(cfg) == 2 * 2 * stream + attn


@pytest.mark.parametrize("field,value", [
    ("n_layers", 0), ("n_heads", 0), ("head_dim", 96), ("n_clusters", 0), ("n_clusters", 65536),
    ("n_stages", 0), ("n_stages", 5), ("bits", 3), ("group_size", 16), ("group_size", 128),
    ("kmeans_iters", -1), ("max_tokens", 0), ("max_tokens", 1 << 31), ("max_chunks", 0),
    ("max_chunks", 257), ("kv_dtype", 7), ("max_chunk_tokens", 40000), ("xlayer", 2),
    ("codebook_reuse", 2), ("xlayer_adapt", 1), ("outlier_channels", 2),
])
def test_invalid_config_rejected(field, value):
    cfg = _cfg(**{field: value})
    assert qkv.workspace_bytes(cfg) == 0
    ctx = ctypes.c_void_p()
    rc = qkv.lib().qkv_init(ctypes.byref(cfg), ctypes.c_void_p(FAKE), ctypes.c_size_t(1 << 40), None,
                            ctypes.byref(ctx))
    assert rc == B.QKV_E_INVAL and not ctx.value


def test_outlier_layout_closed_form():
    # meta gains one (sigma, z) entry per token and stage; one d-bit mask per
    # head and chunk; encode scratch holds [2L][H][64][d] fp64 channel sums
    cfg = _cfg(outlier_channels=1, max_query_tokens=0)
    H, d, T, S, C, G, K, L = 12, 128, 37440, 2, 256, 32, 4, 2
    header = _align(8 + 4 * 257)
    codes = _align(S * H * T * d * 2 // 8)
    meta = _align(S * H * T * (d // G + 1) * 4)
    ids = _align(H * T)
    cb = _align(K * H * C * d * 2)
    cn = _align(K * H * C * 4)
    mask = _align(K * H * d // 8)
    stream = header + codes + meta + ids + cb + cn + mask
    tiles = (32760 + 255) // 256
    units = 2 * L * H * tiles
    sort = _align(_align(units * 256) + units * (C + 1) * 2)
    chan = _align(2 * L * H * 64 * d * 8)
    assert qkv.workspace_bytes(cfg) == 2 * L * stream + sort + chan
    # not with the cross-layer mode
    assert qkv.workspace_bytes(_cfg(outlier_channels=1, xlayer=1, xlayer_rank=8)) == 0
    rc, ctx = _init(cfg)
    assert rc == B.QKV_OK
    try:
        d0 = B.qkv_layout_desc()
        assert qkv.lib().qkv_layout(ctx, 1, 1, ctypes.byref(d0)) == B.QKV_OK
        assert d0.meta_token_stride == (d // G + 1) * 4
        assert d0.chmask_off == 3 * stream + header + codes + meta + ids + cb + cn
        assert d0.chmask_chunk_stride == H * d // 8 and d0.chmask_head_stride == d // 8
    finally:
        qkv.lib().qkv_destroy(ctx)
    rc, ctx = _init(_cfg())
    try:
        d0 = B.qkv_layout_desc()
        assert qkv.lib().qkv_layout(ctx, 0, 0, ctypes.byref(d0)) == B.QKV_OK
        assert d0.chmask_off == 0 and d0.meta_token_stride == (d // G) * 4
    finally:
        qkv.lib().qkv_destroy(ctx)


def test_group_must_divide_and_xlayer_needs_bf16_and_rank():
    assert qkv.workspace_bytes(_cfg(head_dim=64, group_size=64)) > 0
    assert qkv.workspace_bytes(_cfg(xlayer=1, xlayer_rank=0)) == 0
    assert qkv.workspace_bytes(_cfg(xlayer=1, xlayer_rank=32, kv_dtype=B.QKV_F32)) == 0
    assert qkv.workspace_bytes(_cfg(xlayer=1, xlayer_rank=32)) > 0
    # the cross-layer read keeps one layer's bf16 K and V in blocks of the
    # chunk size (two blocks of 32760 tokens for 37440): only with attention
    H, d, T, M = 12, 128, 37440, 32760
    sweep = 2 * 2 * H * M * d * 2
    with_q = qkv.workspace_bytes(_cfg(xlayer=1, xlayer_rank=32))
    no_q = qkv.workspace_bytes(_cfg(xlayer=1, xlayer_rank=32, max_query_tokens=0))
    attn = _align(_align(8 * H * 4680 * d * 4) + 8 * H * 4680 * 4)
    assert with_q - no_q >= sweep and with_q - no_q <= sweep + attn


def _init(cfg, arena=FAKE, nbytes=None, predictor=None):
    ctx = ctypes.c_void_p()
    nb = qkv.workspace_bytes(cfg) if nbytes is None else nbytes
    rc = qkv.lib().qkv_init(ctypes.byref(cfg), ctypes.c_void_p(arena) if arena else None,
                            ctypes.c_size_t(nb), ctypes.c_void_p(predictor) if predictor else None,
                            ctypes.byref(ctx))
    return rc, ctx


def test_init_arena_checks():
    cfg = _cfg()
    assert _init(cfg, nbytes=qkv.workspace_bytes(cfg) - 1)[0] == B.QKV_E_ARENA
    assert _init(cfg, arena=FAKE + 128)[0] == B.QKV_E_ARENA
    assert _init(cfg, arena=0)[0] == B.QKV_E_INVAL
    assert _init(_cfg(xlayer=1, xlayer_rank=8))[0] == B.QKV_E_INVAL   # predictor missing
    rc, ctx = _init(cfg)
    assert rc == B.QKV_OK and ctx.value
    qkv.lib().qkv_destroy(ctx)


@pytest.fixture
def ctx():
    rc, c = _init(_cfg())
    assert rc == B.QKV_OK
    yield c
    qkv.lib().qkv_destroy(c)


def test_call_validation_before_enqueue(ctx):
    L = qkv.lib()
    p = ctypes.c_void_p(FAKE)
    # encode: bad layer range, null inputs, n < 1, chunk and capacity limits
    assert L.qkv_encode_chunk(ctx, -1, 1, p, p, 10, None) == B.QKV_E_INVAL
    assert L.qkv_encode_chunk(ctx, 1, 2, p, p, 10, None) == B.QKV_E_INVAL
    assert L.qkv_encode_chunk(ctx, 0, 1, None, p, 10, None) == B.QKV_E_INVAL
    assert L.qkv_encode_chunk(ctx, 0, 1, p, p, 0, None) == B.QKV_E_INVAL
    assert L.qkv_encode_chunk(ctx, 0, 1, p, p, 32761, None) == B.QKV_E_CAPACITY
    # attend / reconstruct before anything is encoded
    assert L.qkv_attend(ctx, 0, p, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_STATE
    assert L.qkv_attend(ctx, 0, p, 4681, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_CAPACITY
    assert L.qkv_attend(ctx, 2, p, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert L.qkv_attend(ctx, 0, p, 16, 5, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert L.qkv_attend(ctx, 0, None, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    # the no-allocation variant validates the same way before anything else
    N = L.qkv_attend_noalloc
    assert N(ctx, 0, p, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_STATE
    assert N(ctx, 0, p, 4681, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_CAPACITY
    assert N(ctx, 2, p, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert N(ctx, 0, None, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    # attention with a fresh chunk: nothing to attend to, capacity, arguments
    A = L.qkv_attend_with_chunk
    assert A(ctx, 0, p, 16, B.QKV_BF16, None, None, 0, p, B.QKV_F32, None, None) == B.QKV_E_STATE
    assert A(ctx, 0, p, 4681, B.QKV_BF16, p, p, 8, p, B.QKV_F32, None, None) == B.QKV_E_CAPACITY
    assert A(ctx, 2, p, 16, B.QKV_BF16, p, p, 8, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert A(ctx, 0, p, 16, B.QKV_BF16, None, p, 8, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert A(ctx, 0, p, 16, B.QKV_BF16, p, None, 8, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert A(ctx, 0, p, 16, B.QKV_BF16, p, p, -1, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert A(ctx, 0, None, 16, B.QKV_BF16, p, p, 8, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert A(ctx, 0, p, 16, B.QKV_BF16, p, p, 8, None, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert A(ctx, 0, p, 16, 9, p, p, 8, p, B.QKV_F32, None, None) == B.QKV_E_INVAL
    assert L.qkv_reconstruct(ctx, 0, 1, 0, 0, 10, p, B.QKV_F32, None) == B.QKV_E_STATE
    assert L.qkv_reconstruct(ctx, 0, 1, 2, 0, 10, p, B.QKV_F32, None) == B.QKV_E_INVAL
    assert L.qkv_reconstruct(ctx, 0, 1, 0, 5, 4, p, B.QKV_F32, None) == B.QKV_E_INVAL
    assert L.qkv_reconstruct(ctx, 0, 3, 0, 0, 1, p, B.QKV_F32, None) == B.QKV_E_INVAL
    # rewind beyond the encoded tokens
    assert L.qkv_rewind(ctx, 0, 1, 5, None) == B.QKV_E_STATE
    assert L.qkv_rewind(ctx, 0, 1, -1, None) == B.QKV_E_INVAL
    # layout / chunk table of an empty context
    d = B.qkv_layout_desc()
    assert L.qkv_layout(ctx, 1, 1, ctypes.byref(d)) == B.QKV_OK
    assert d.n_tokens == 0 and d.n_chunks == 0 and d.id_bytes == 1
    assert d.codes_off % 256 == 0 and d.meta_off % 256 == 0 and d.codebook_off % 256 == 0
    assert L.qkv_layout(ctx, 2, 0, ctypes.byref(d)) == B.QKV_E_INVAL
    assert L.qkv_chunk_starts(ctx, 0, None, 0) == 0


def test_cross_layer_attend_order():
    cfg = _cfg(xlayer=1, xlayer_rank=8)
    rc, c = _init(cfg, predictor=FAKE)
    assert rc == B.QKV_OK
    L = qkv.lib()
    p = ctypes.c_void_p(FAKE)
    # nothing encoded yet, and no layer swept: reading layer 1 is a state error
    assert L.qkv_attend(c, 1, p, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_STATE
    assert L.qkv_attend_with_chunk(c, 1, p, 16, B.QKV_BF16, None, None, 0, p, B.QKV_F32, None,
                                   None) == B.QKV_E_STATE
    assert L.qkv_attend_noalloc(c, 0, p, 16, B.QKV_BF16, p, B.QKV_F32, None, None) == B.QKV_E_STATE
    # layer 1 before layer 0 (no chain) is a state error
    assert L.qkv_encode_chunk(c, 1, 1, p, p, 100, None) == B.QKV_E_STATE
    L.qkv_destroy(c)


def test_status_strings():
    for s in (0, -1, -2, -3, -4, -5, -6, 99):
        assert isinstance(qkv.status_string(s), str)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with status 2 and a message."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_per_call_input_slice_must_stay_under_2gib():
    """One head's slice of one encode call (n * d * element bytes) is
    addressed with 32-bit offsets: 2^23 bf16 tokens of d = 128 are refused
    unless the calls are capped below that."""
    big = 1 << 23
    assert qkv.workspace_bytes(_cfg(max_tokens=big, max_chunk_tokens=0, max_query_tokens=0)) == 0
    assert qkv.workspace_bytes(_cfg(max_tokens=big, max_chunk_tokens=big - 1, max_query_tokens=0)) > 0
    assert qkv.workspace_bytes(_cfg(max_tokens=big, max_chunk_tokens=4096, max_query_tokens=0)) > 0


def test_codebook_reuse_keeps_one_snapshot():
    """With codebook reuse each stream holds one codebook snapshot: the
    snapshot strides are 0 and the arena shrinks by the other max_chunks - 1
    snapshots of every stream."""
    per_call, reused = _cfg(max_chunks=8), _cfg(max_chunks=8, codebook_reuse=1)
    H, C, d = 12, 256, 128
    saved = qkv.workspace_bytes(per_call) - qkv.workspace_bytes(reused)
    one = H * C * d * 2 + H * C * 4
    assert 2 * 2 * 7 * one <= saved <= 2 * 2 * (7 * one + 2 * 256)
    rc, c = _init(reused)
    assert rc == B.QKV_OK
    d_ = B.qkv_layout_desc()
    assert qkv.lib().qkv_layout(c, 1, 1, ctypes.byref(d_)) == B.QKV_OK
    assert d_.codebook_chunk_stride == 0 and d_.cnorm_chunk_stride == 0
    qkv.lib().qkv_destroy(c)


def test_adapted_mode_layout_and_readback():
    """xlayer_adapt needs the cross-layer mode; its re-fitted blocks live in
    the arena between the streams and the scratch region."""
    assert qkv.workspace_bytes(_cfg(xlayer_adapt=1)) == 0
    plain, adapted = _cfg(xlayer=1, xlayer_rank=8), _cfg(xlayer=1, xlayer_rank=8, xlayer_adapt=1)
    assert qkv.workspace_bytes(adapted) > qkv.workspace_bytes(plain) + 2 * 2 * 12 * 128 * 128 * 2
    rc, c = _init(adapted, predictor=FAKE)
    assert rc == B.QKV_OK
    L = qkv.lib()
    off1, off0 = ctypes.c_uint64(), ctypes.c_uint64()
    assert L.qkv_adapted_blocks(c, 1, ctypes.byref(off1)) == B.QKV_OK
    assert L.qkv_adapted_blocks(c, 0, ctypes.byref(off0)) == B.QKV_E_INVAL
    assert L.qkv_adapted_blocks(c, 2, ctypes.byref(off0)) == B.QKV_E_INVAL
    d = B.qkv_layout_desc()
    assert L.qkv_layout(c, 1, 1, ctypes.byref(d)) == B.QKV_OK
    assert off1.value % 256 >= 0 and off1.value > d.cnorm_off
    L.qkv_destroy(c)
    rc, c = _init(plain, predictor=FAKE)
    assert L.qkv_adapted_blocks(c, 1, ctypes.byref(off1)) == B.QKV_E_INVAL
    L.qkv_destroy(c)


def test_head_codes_addressable_with_32_bit_offsets():
    # the fused read addresses one head's codes of one stage with 32-bit
    # offsets: 2^26 tokens of INT4 codes at d = 128 (64 bytes per token) is
    # the first size refused; one token fewer is accepted
    T = 1 << 26
    ok = _cfg(n_layers=1, n_heads=1, bits=4, max_tokens=T - 1, max_chunk_tokens=4680, max_query_tokens=0)
    big = _cfg(n_layers=1, n_heads=1, bits=4, max_tokens=T, max_chunk_tokens=4680, max_query_tokens=0)
    assert qkv.workspace_bytes(ok) > 0
    assert qkv.workspace_bytes(big) == 0
    rc, ctx = _init(big, nbytes=1, arena=1)
    assert rc == B.QKV_E_INVAL and not ctx.value
