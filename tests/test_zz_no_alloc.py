"""qkv_attend_noalloc (the attention entry point that allocates nothing and
keeps its split partials in the library's fixed per-GPU array) against
qkv_attend, through the C-ABI: the same kernels on the same inputs, so the
outputs and log-sum-exps must be identical bit for bit.  Two calls in a row,
the second smaller (another layer with fewer tokens, fewer queries), both
large enough that query blocks are split over several blocks and the fixed
array holds partials; then a call whose partials exceed the array is
refused."""
import pytest
import torch

import kv_cache_quantization_head_amd as qkv
import synth
from kv_cache_quantization_head_amd import binding as B

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def test_noalloc_attend_matches_attend_on_two_calls():
    cfgs = synth.WAN_LAYER
    H, d, C = cfgs.n_heads, cfgs.head_dim, cfgs.n_clusters
    T0, T1 = cfgs.tokens, 5000
    cfg = qkv.config(2, H, d, C, cfgs.n_stages, cfgs.bits, cfgs.group, kmeans_iters=cfgs.iters,
                     max_tokens=T0, max_chunks=1, kv_dtype=qkv.QKV_BF16, max_query_tokens=4680)
    codec = qkv.Codec(cfg, device=DEV)
    _say("no-alloc attend: encode layer 0 (32760 tokens) and layer 1 (5000 tokens)")
    for layer, T in ((0, T0), (1, T1)):
        k = synth.kv_tokens(cfgs, layer, 0, 0, T, device=DEV)
        v = synth.kv_tokens(cfgs, layer, 1, 0, T, device=DEV)
        codec.encode_chunk(k, v, layer0=layer)
    for layer, nq, out_dtype in ((0, 4680, torch.float32), (1, 777, torch.bfloat16)):
        _say(f"no-alloc attend: layer {layer}, {nq} queries, out {out_dtype}")
        q = synth.queries(cfgs, layer, nq, device=DEV).contiguous()
        ref, ref_lse = codec.attend(layer, q, out_dtype=out_dtype)
        out = torch.full((H, nq, d), float("nan"), dtype=out_dtype, device=DEV)
        lse = torch.full((H, nq), float("nan"), dtype=torch.float32, device=DEV)
        codec.attend_noalloc(layer, q, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           ref.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_noalloc_attend_refuses_partials_beyond_the_array():
    # 64 heads x 4680 queries: the split partials of a long layer need more
    # than 128 MiB, so the call is refused before anything is enqueued
    H, d = 64, 128
    cfg = qkv.config(1, H, d, 16, 1, 2, 32, kmeans_iters=0, max_tokens=65536, max_chunks=1,
                     kv_dtype=qkv.QKV_BF16, max_query_tokens=4680)
    codec = qkv.Codec(cfg, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(5)
    k = torch.randn((H, 65536, d), generator=g, device=DEV).to(torch.bfloat16)
    codec.encode_chunk(k, k)
    q = torch.randn((H, 4680, d), generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty((H, 4680, d), dtype=torch.float32, device=DEV)
    with pytest.raises(qkv.QkvError) as e:
        codec.attend_noalloc(0, q, out)
    assert e.value.status == B.QKV_E_CAPACITY
