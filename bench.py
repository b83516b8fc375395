"""Benchmark of the hot path on one MI355X.

Default workload: the long-rollout cache, 30 layers x K,V bf16 [12 heads,
187200 tokens (120 latent frames x 1560), d=128] = 34.5 GB of bf16 K/V,
C=256 clusters, 5 k-means iterations, 3-stage INT2 with group 32.  Each
layer's cache is built untimed by 40 encode calls of 4680 tokens (three
latent frames), on device-generated seeded tokens.  One timed step is what a
generating model does per new 4680-token chunk, plus the whole-cache read
back:
  qkv_attend of a 4680-query bf16 chunk over each of the 30 packed layers
  (fused unpack -> dequant -> attention), qkv_encode_chunk of the chunk's
  new K/V into all 30 layers at once (k-means warm-started from each
  stream's last snapshot + PRQ + packing), qkv_reconstruct of every layer
  (K and V, all 191880 tokens, bf16 out), qkv_rewind back to 187200 tokens.
Inputs are resident in HBM before the timed region; each library call is
bracketed by HIP events on the stream it runs on.  After the timed steps, a
traced leg (the library's per-kernel HIP events) gives each kernel's time
for the per-kernel rooflines; then the oracle is timed on a bounded sample of
the same workload, and the one-layer Wan step (encode + reconstruct + attend
of one 32760-token layer) is timed for its own figures.

Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
# one fp32 vector operation per lane per clock: 256 CUs x 64 lanes x 2.4 GHz (the packed
# two-operation fp32 instructions behind the 157.3 TFLOP/s figure are not used)
ALU_PEAK_TOPS = 39.32
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--xlayer", action="store_true",
                    help="instead of the default step: time the cross-layer encode of one "
                         "wide-head layer (K and V [40, 62400, 128] bf16, rank 32, C = 512, "
                         "2-stage INT2, G = 64), predicted from the previous layer")
    ap.add_argument("--fresh", action="store_true",
                    help="instead of the default step: time a generated chunk on 4 wan_layer-shaped "
                         "layers (attention over the packed cache plus the chunk's fresh bf16 K/V for "
                         "every denoising step and layer, then the chunk's encode)")
    ap.add_argument("--denoise", type=int, default=4, help="denoising steps per chunk (--fresh)")
    ap.add_argument("--layers", type=int, default=None,
                    help="layers of the model (default step: 30; --fresh: 4; Wan2.1-1.3B has 30)")
    ap.add_argument("--no-wan-layer", action="store_true",
                    help="skip the one-layer Wan step that follows the default step")
    ap.add_argument("--reuse", action="store_true",
                    help="instead of the default step: encode a long-rollout layer (187200 tokens in 40 "
                         "calls) with codebook reuse and with per-call snapshots; time, reconstruction "
                         "error and storage cost of each")
    ap.add_argument("--outliers", action="store_true",
                    help="instead of the default step: the same wan_layer step with and without the "
                         "outlier-channel option; time of each call, reconstruction error and storage "
                         "cost of each mode")
    ap.add_argument("--wide", action="store_true",
                    help="instead of the default step: one wide-head layer (K,V bf16 [40, 62400, 128], C=512, "
                         "G=64) coded as 2-stage INT2 and as 1-stage INT4; encode and reconstruct time, "
                         "reconstruction error and storage cost of each")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (a known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def recorded_traffic(kernel_source):
    """HBM bytes of one qkv_attend call (attention kernel + merge) on a
    long-rollout layer, from the committed counter summary, or None when the
    attention source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_attend3_long_rollout_pmc.txt")
    try:
        fields = dict(line.split(":", 1) for line in open(path) if ":" in line)
    except OSError:
        return None
    digest = hashlib.sha256(open(kernel_source, "rb").read()).hexdigest()
    if fields.get("kernels_sha256", "").strip() != digest:
        return None
    try:
        return int(fields["traffic_bytes_per_launch"].strip())
    except (KeyError, ValueError):
        return None


def xlayer_main(args):
    """Cross-layer residual mode on the wide-head shape.  A step rewinds both
    layers, encodes layer 0 with SAS and then layer 1 from its prediction
    (projection, prediction, PRQ of the residual); each call is timed with HIP
    events on the current stream."""
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth

    dev = torch.device("cuda:0")
    cfgs = synth.scaled(synth.WIDE_HEAD, n_layers=2)
    H, T, d, C, r = cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.n_clusters, cfgs.xlayer_rank
    parts = []
    for kv in (0, 1):
        B, U, V = synth.predictor(cfgs, 0, kv, rank=r)
        parts += [B.reshape(-1), U.reshape(-1), V.reshape(-1)]
    Tq = 4680
    cfg = qkv.config(2, H, d, C, cfgs.n_stages, cfgs.bits, cfgs.group, kmeans_iters=cfgs.iters,
                     max_tokens=T, max_chunks=1, kv_dtype=qkv.QKV_BF16, max_query_tokens=Tq, xlayer=1,
                     xlayer_rank=r)
    blob = torch.cat(parts).to(dev)
    codec = qkv.Codec(cfg, device=dev, predictor=blob)
    cfg_a = qkv.config(2, H, d, C, cfgs.n_stages, cfgs.bits, cfgs.group, kmeans_iters=cfgs.iters,
                       max_tokens=T, max_chunks=1, kv_dtype=qkv.QKV_BF16, max_query_tokens=0, xlayer=1,
                       xlayer_rank=r, xlayer_adapt=1)
    codec_a = qkv.Codec(cfg_a, device=dev, predictor=blob)
    ks = torch.stack([synth.kv_tokens(cfgs, l, 0, 0, T, device=dev) for l in range(2)])
    vs = torch.stack([synth.kv_tokens(cfgs, l, 1, 0, T, device=dev) for l in range(2)])
    ev, ev_a = [], []
    q = synth.queries(cfgs, 1, Tq, device=dev)
    out = torch.empty((H, Tq, d), dtype=torch.bfloat16, device=dev)
    read_ev = []

    def step(record):
        for c, sink in ((codec, ev), (codec_a, ev_a)):
            c.rewind(0, 2, 0)
            m = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            m[0].record()
            c.encode_chunk(ks[:1], vs[:1], layer0=0)
            m[1].record()
            c.encode_chunk(ks[1:], vs[1:], layer0=1)
            m[2].record()
            if record:
                sink.append(m)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    sas = sum(m[0].elapsed_time(m[1]) for m in ev) / len(ev)
    xl = sum(m[1].elapsed_time(m[2]) for m in ev) / len(ev)
    xl_a = sum(m[1].elapsed_time(m[2]) for m in ev_a) / len(ev_a)

    # the read of the two layers in order (a model's forward pass): layer 0
    # (packed SAS read, its reconstruction kept as the rolling copy), then
    # layer 1 (prediction from that copy, reconstruction over it, bf16 read)
    def read(record):
        m = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        m[0].record()
        codec.attend(0, q, out=out, with_lse=False)
        m[1].record()
        codec.attend(1, q, out=out, with_lse=False)
        m[2].record()
        if record:
            read_ev.append(m)

    for _ in range(args.warmup):
        read(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        read(True)
    torch.cuda.synchronize()
    r0 = sum(m[0].elapsed_time(m[1]) for m in read_ev) / len(read_ev)
    r1 = sum(m[1].elapsed_time(m[2]) for m in read_ev) / len(read_ev)
    codec.trace(True)
    read(False)
    torch.cuda.synchronize()
    kt = codec.trace_read()
    codec.trace(False)
    sweep_bytes = 2 * H * T * d * 2
    # the prediction of layer 1's K and V in the read (one launch): per token,
    # head and tensor d*(d + r) fp64 fmas, on the fp64 matrix instruction
    xl_roofline = None
    if "k_xl_predict" in kt and kt["k_xl_predict"][0]:
        n_pred, tot_pred = kt["k_xl_predict"]
        flops = 2.0 * 2 * H * T * d * (d + r)
        tf = flops / (tot_pred / n_pred * 1e-3) / 1e12
        xl_roofline = {"kernel": "k_xl_predict", "bound": "fp64 matrix", "achieved": round(tf, 2),
                       "peak": 78.6, "unit": "TFLOP/s", "frac": round(tf / 78.6, 4),
                       "flops_per_launch": flops, "launch_ms": round(tot_pred / n_pred, 4)}

    def layer1_error(c):
        err = []
        for kv, x in ((0, ks[1]), (1, vs[1])):
            xf = x.float()
            rec = c.reconstruct(1, 1, kv, 0, T)[0]
            err.append(round(float(((rec - xf) ** 2).sum() / (xf ** 2).sum()), 6))
            del rec
        return err
    print(json.dumps({
        "metric": "cross-layer encode of one layer (K and V)", "value": round(xl, 4), "unit": "ms",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False,
        "dtype": "bf16 in, fp64 prediction", "data": "synthetic (seeded prototype/drift/outlier generator)",
        "config": {"workload": "wide_head layer: K,V bf16 [40, 62400, 128], C=512, 2-stage INT2 G=64, "
                               "cross-layer rank 32", "heads": H, "tokens": T, "rank": r},
        "sas_layer_ms": round(sas, 4), "layer1_rel_sq_error_kv": layer1_error(codec),
        "adapted_layer_ms_with_refit": round(xl_a, 4),
        "adapted_layer1_rel_sq_error_kv": layer1_error(codec_a),
        "read_q_tokens": Tq,
        "read_layer0_ms": round(r0, 4), "read_layer1_ms": round(r1, 4),
        "read_kernels": {k: {"launches": n, "avg_ms": round(tot / max(n, 1), 4)} for k, (n, tot) in kt.items()},
        "roofline": xl_roofline,
        "read_rolling_copy_bytes": sweep_bytes,
        "read_note": "layer 0: packed read + its reconstruction into the rolling bf16 copy; layer 1: "
                     "prediction from the copy (fp64), reconstruction over it, bf16 read"}), flush=True)


def fresh_main(args):
    """The read as a generating model issues it, on the wan_layer shape with
    --layers layers (4 by default): for each new 4680-token chunk, --denoise denoising steps each
    attend every layer's 4680 queries over its packed 32760-token cache plus
    the chunk's fresh bf16 K/V (qkv_attend_with_chunk), then the chunk is
    encoded into every layer's cache.  A step is one chunk; the cache is
    rewound to 32760 tokens before each step so every step sees the same
    sizes."""
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth

    dev = torch.device("cuda:0")
    L = args.layers or 4
    cfgs = synth.scaled(synth.WAN_LAYER, n_layers=L)
    H, T, d, Tq, n_new = cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.q_tokens, cfgs.q_tokens
    cfg = qkv.config(L, H, d, cfgs.n_clusters, cfgs.n_stages, cfgs.bits, cfgs.group, kmeans_iters=cfgs.iters,
                     max_tokens=T + n_new, max_chunk_tokens=T, max_chunks=2, kv_dtype=qkv.QKV_BF16,
                     max_query_tokens=Tq)
    codec = qkv.Codec(cfg, device=dev)
    ks = torch.stack([synth.kv_tokens(cfgs, l, 0, 0, T + n_new, device=dev) for l in range(L)])
    vs = torch.stack([synth.kv_tokens(cfgs, l, 1, 0, T + n_new, device=dev) for l in range(L)])
    codec.encode_chunk(ks[:, :, :T].contiguous(), vs[:, :, :T].contiguous())
    kn, vn = ks[:, :, T:].contiguous(), vs[:, :, T:].contiguous()
    qs = [synth.queries(cfgs, l, Tq, device=dev) for l in range(L)]
    out = torch.empty((H, Tq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, Tq), dtype=torch.float32, device=dev)
    ev = []

    def step(record):
        codec.rewind(0, L, T)
        m = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        m[0].record()
        for _ in range(args.denoise):
            for l in range(L):
                codec.attend_with_chunk(l, qs[l], kn[l], vn[l], out=out, lse=lse)
        m[1].record()
        codec.encode_chunk(kn, vn)
        m[2].record()
        if record:
            ev.append(m)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    att = sum(m[0].elapsed_time(m[1]) for m in ev) / len(ev)
    enc = sum(m[1].elapsed_time(m[2]) for m in ev) / len(ev)
    per_call = att / (args.denoise * L)
    flops = 4.0 * d * H * Tq * (T + n_new)
    print(json.dumps({
        "metric": "generated chunk: attention over packed cache + fresh chunk for every denoising step and "
                  "layer, then the chunk's encode", "value": round(att + enc, 4), "unit": "ms per chunk",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded prototype/drift/outlier generator)",
        "config": {"workload": f"wan_layer x {L} layers: packed cache 32760 + fresh 4680 tokens, 4680 bf16 "
                               f"queries, {args.denoise} denoising steps",
                   "layers": L, "heads": H, "cache_tokens": T, "fresh_tokens": n_new, "q_tokens": Tq,
                   "denoise_steps": args.denoise},
        "attend_with_chunk_ms": round(per_call, 4), "attend_with_chunk_TFLOPs": round(flops / per_call / 1e9, 1),
        "encode_chunk_ms": round(enc, 4)}), flush=True)


def reuse_main(args):
    """Codebook reuse against per-call snapshots on one long-rollout layer
    (12 heads, 187 200 tokens arriving as 40 calls of 4680, 3 INT2 stages,
    C = 256): a step encodes the whole layer from empty in each mode; after
    the timed steps the reconstruction error of each mode is measured over
    the layer, with the storage cost of each."""
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth
    from fractions import Fraction

    dev = torch.device("cuda:0")
    cfgs = synth.LONG_ROLLOUT
    H, T, d, C, S, b, G = (cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.n_clusters, cfgs.n_stages,
                           cfgs.bits, cfgs.group)
    n_call = 4680
    n_calls = T // n_call
    k = synth.kv_tokens(cfgs, 0, 0, 0, T, device=dev)
    v = synth.kv_tokens(cfgs, 0, 1, 0, T, device=dev)
    codecs = {}
    for reuse in (0, 1):
        cfg = qkv.config(1, H, d, C, S, b, G, kmeans_iters=cfgs.iters, max_tokens=T, max_chunk_tokens=n_call,
                         max_chunks=n_calls, kv_dtype=qkv.QKV_BF16, max_query_tokens=0, codebook_reuse=reuse)
        codecs[reuse] = qkv.Codec(cfg, device=dev)
    ks = [k[:, i * n_call:(i + 1) * n_call].contiguous() for i in range(n_calls)]
    vs = [v[:, i * n_call:(i + 1) * n_call].contiguous() for i in range(n_calls)]
    times = {0: [], 1: []}

    def step(record):
        for reuse, codec in codecs.items():
            codec.rewind(0, 1, 0)
            m = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            m[0].record()
            for i in range(n_calls):
                codec.encode_chunk(ks[i], vs[i])
            m[1].record()
            if record:
                times[reuse].append(m)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    res = {}
    for reuse, codec in codecs.items():
        ms = sum(m[0].elapsed_time(m[1]) for m in times[reuse]) / len(times[reuse])
        err = []
        for kv, x in ((0, k), (1, v)):
            xf = x.float()
            rec = codec.reconstruct(0, 1, kv, 0, T)[0]
            err.append(float(((rec - xf) ** 2).sum() / (xf ** 2).sum()))
            del rec
        cb_tokens = T if reuse else n_call
        fixed = Fraction(S * b) + Fraction(S * 32, G) + Fraction(8, d)
        bits = float(fixed + Fraction(8 * 2 * C, cb_tokens))
        res["reuse" if reuse else "per_call"] = {
            "layer_ms": round(ms, 4), "call_ms": round(ms / n_calls, 4),
            "rel_sq_error_k": round(err[0], 6), "rel_sq_error_v": round(err[1], 6),
            "bits_per_element": round(bits, 4)}
    print(json.dumps({
        "metric": "codebook reuse vs per-call snapshots: encode time of a long-rollout layer",
        "value": res["reuse"]["layer_ms"], "unit": "ms per layer (40 calls of 4680 tokens)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded prototype/drift/outlier generator)",
        "config": {"workload": "long_rollout layer: K,V bf16 [12, 187200, 128] in 40 calls of 4680, C=256, "
                               "5 iterations, 3-stage INT2, G=32", "heads": H, "tokens": T, "calls": n_calls},
        "modes": res}), flush=True)


def outliers_main(args):
    """The default wan_layer step (encode + reconstruct K and V in bf16 +
    4680-query attention) with the outlier-channel option on and off: HIP
    event time of each call averaged over the timed steps, then the
    reconstruction error of each mode over the layer and its storage cost."""
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth
    from fractions import Fraction

    dev = torch.device("cuda:0")
    cfgs = synth.WAN_LAYER
    H, T, d, C, S, b, G = (cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.n_clusters, cfgs.n_stages,
                           cfgs.bits, cfgs.group)
    k = synth.kv_tokens(cfgs, 0, 0, 0, T, device=dev)
    v = synth.kv_tokens(cfgs, 0, 1, 0, T, device=dev)
    q = synth.queries(cfgs, 0, cfgs.q_tokens, device=dev)
    codecs = {}
    for outl in (0, 1):
        cfg = qkv.config(1, H, d, C, S, b, G, kmeans_iters=cfgs.iters, max_tokens=T, max_chunks=1,
                         kv_dtype=qkv.QKV_BF16, max_query_tokens=cfgs.q_tokens, outlier_channels=outl)
        codecs[outl] = qkv.Codec(cfg, device=dev)
    names = ("qkv_encode_chunk", "qkv_reconstruct", "qkv_attend")
    times = {o: {n: [] for n in names} for o in codecs}
    rk = torch.empty((1, H, T, d), dtype=torch.bfloat16, device=dev)
    rv = torch.empty_like(rk)

    def step(record):
        for outl, codec in codecs.items():
            codec.rewind(0, 1, 0)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record()
            codec.encode_chunk(k, v)
            ev[1].record()
            codec.reconstruct(0, 1, 0, 0, T, out_dtype=torch.bfloat16, out=rk)
            codec.reconstruct(0, 1, 1, 0, T, out_dtype=torch.bfloat16, out=rv)
            ev[2].record()
            codec.attend(0, q)
            ev[3].record()
            if record:
                for i, n in enumerate(names):
                    times[outl][n].append((ev[i], ev[i + 1]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    res = {}
    for outl, codec in codecs.items():
        calls = {n: round(sum(a.elapsed_time(e) for a, e in times[outl][n]) / args.steps, 4) for n in names}
        err = []
        for kv, x in ((0, k), (1, v)):
            xf = x.float()
            rec = codec.reconstruct(0, 1, kv, 0, T)[0]
            err.append(float(((rec - xf) ** 2).sum() / (xf ** 2).sum()))
            del rec
        bits = Fraction(S * b) + Fraction(S * 32 * (d // G + outl), G * (d // G)) + Fraction(8, d) \
            + Fraction(8 * 2 * C, T) + (Fraction(1, T) if outl else 0)
        res["outliers" if outl else "plain"] = {
            "calls_ms": calls, "step_ms": round(sum(calls.values()), 4),
            "rel_sq_error_k": round(err[0], 7), "rel_sq_error_v": round(err[1], 7),
            "bits_per_element": round(float(bits), 4)}
    print(json.dumps({
        "metric": "outlier-channel option: wan_layer step time and reconstruction error, on and off",
        "value": res["outliers"]["step_ms"], "unit": "ms per step (encode + reconstruct + attend)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded prototype/drift/outlier generator)",
        "config": {"workload": "wan_layer: K,V bf16 [12, 32760, 128], C=256, 5 iterations, 2-stage INT2, "
                               "G=32; 4680 bf16 queries", "heads": H, "tokens": T},
        "modes": res}), flush=True)


def wide_main(args):
    """The wide-head comparison: one layer of 40 heads x 62400 tokens (C = 512,
    G = 64, 8 outlier channels x20) coded as INT2 x 2 stages and as INT4 x 1
    stage (equal code bits).  A step encodes the layer from empty and
    reconstructs K and V (bf16 out) in each variant; then the relative
    squared reconstruction error of each variant and its storage cost."""
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth
    from fractions import Fraction

    dev = torch.device("cuda:0")
    base = synth.WIDE_HEAD
    H, T, d, C, G = base.n_heads, base.tokens, base.head_dim, base.n_clusters, base.group
    k = synth.kv_tokens(base, 0, 0, 0, T, device=dev)
    v = synth.kv_tokens(base, 0, 1, 0, T, device=dev)
    rec = torch.empty((2, 1, H, T, d), dtype=torch.bfloat16, device=dev)
    codecs = {}
    for name, S, b, _ in [(n, s_, b_, g_) for n, s_, b_, g_ in base.variants]:
        cfg = qkv.config(1, H, d, C, S, b, G, kmeans_iters=base.iters, max_tokens=T, max_chunks=1,
                         kv_dtype=qkv.QKV_BF16, max_query_tokens=0)
        codecs[name] = (qkv.Codec(cfg, device=dev), S, b)
    times = {n: {"encode": [], "reconstruct": []} for n in codecs}

    def step(record):
        for name, (codec, _, _) in codecs.items():
            codec.rewind(0, 1, 0)
            m = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            m[0].record()
            codec.encode_chunk(k, v)
            m[1].record()
            codec.reconstruct(0, 1, 0, 0, T, out=rec[0])
            codec.reconstruct(0, 1, 1, 0, T, out=rec[1])
            m[2].record()
            if record:
                times[name]["encode"].append((m[0], m[1]))
                times[name]["reconstruct"].append((m[1], m[2]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    res = {}
    n_el = 2 * H * T * d
    for name, (codec, S, b) in codecs.items():
        err = []
        for kv, x in ((0, k), (1, v)):
            rec_f = codec.reconstruct(0, 1, kv, 0, T)[0]
            xf = x.float()
            err.append(float(((rec_f - xf) ** 2).sum() / (xf ** 2).sum()))
            del rec_f, xf
        fixed = Fraction(S * b) + Fraction(S * 32, G) + Fraction(16, d)      # codes, meta, u16 ids
        bits = float(fixed + Fraction(16 * C, T))
        enc = _avg_ms(times[name]["encode"])
        rc = _avg_ms(times[name]["reconstruct"])
        packed = n_el * (S * b / 8 + S * 4 / G) + 2 * H * T * 2
        res[name] = {"stages": S, "bits": b, "encode_ms": round(enc, 4), "reconstruct_k_and_v_ms": round(rc, 4),
                     "quantize_GBps_in_plus_out": round((n_el * 2 + packed) / (enc * 1e-3) / 1e9, 1),
                     "reconstruct_GBps": round((packed + n_el * 2) / (rc * 1e-3) / 1e9, 1),
                     "rel_sq_error_k": round(err[0], 7), "rel_sq_error_v": round(err[1], 7),
                     "bits_per_element": round(bits, 4)}
    print(json.dumps({
        "metric": "wide-head layer: 2-stage INT2 vs 1-stage INT4 (G=64), encode + reconstruct time, error, bits",
        "value": res["int2x2"]["encode_ms"], "unit": "ms (INT2 x 2 encode of one layer)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "dtype": "bf16",
        "data": "synthetic (seeded prototype/drift/outlier generator, device-generated)",
        "config": {"workload": "wide_head layer: K,V bf16 [40, 62400, 128], C=512, 5 iterations, G=64, "
                               "8 outlier channels x20", "heads": H, "tokens": T},
        "variants": res}), flush=True)


def _avg_ms(pairs):
    xs = [a.elapsed_time(b) for a, b in pairs]
    return sum(xs) / len(xs)


def wan_layer_step(args):
    """One Wan2.1-1.3B-shaped layer (K,V bf16 [12, 32760, 128], C=256, 2-stage
    INT2, G=32): encode of the whole layer from empty, reconstruct of K and V
    (bf16 out), attention of 4680 bf16 queries.  Returns its figures."""
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth

    dev = torch.device("cuda:0")
    cfgs = synth.WAN_LAYER
    H, T, d, Tq = cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.q_tokens
    S, b, G, C = cfgs.n_stages, cfgs.bits, cfgs.group, cfgs.n_clusters
    cfg = qkv.config(1, H, d, C, S, b, G, kmeans_iters=cfgs.iters, max_tokens=T, max_chunks=1,
                     kv_dtype=qkv.QKV_BF16, max_query_tokens=Tq)
    codec = qkv.Codec(cfg, device=dev)
    k = synth.kv_tokens(cfgs, 0, 0, 0, T, device=dev)
    v = synth.kv_tokens(cfgs, 0, 1, 0, T, device=dev)
    q = synth.queries(cfgs, 0, Tq, device=dev)
    rec = torch.empty((2, 1, H, T, d), dtype=torch.bfloat16, device=dev)
    out = torch.empty((H, Tq, d), dtype=torch.float32, device=dev)
    lse = torch.empty((H, Tq), dtype=torch.float32, device=dev)
    ev = {name: [] for name in ("encode", "reconstruct", "attend")}

    def step(record):
        codec.rewind(0, 1, 0)
        m = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        m[0].record()
        codec.encode_chunk(k, v)
        m[1].record()
        codec.reconstruct(0, 1, 0, 0, T, out=rec[0])
        codec.reconstruct(0, 1, 1, 0, T, out=rec[1])
        m[2].record()
        codec.attend(0, q, out=out, lse=lse)
        m[3].record()
        if record:
            for i, n in enumerate(ev):
                ev[n].append((m[i], m[i + 1]))

    for _ in range(2):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {n: _avg_ms(p) for n, p in ev.items()}
    n_el = 2 * H * T * d
    packed = n_el * (S * b / 8 + S * 4 / G) + 2 * H * T
    att_tflops = 4.0 * H * Tq * T * d / (ms["attend"] * 1e-3) / 1e12
    return {
        "workload": "wan_layer: K,V bf16 [12, 32760, 128], C=256, 5 iters, 2-stage INT2 G=32; 4680 bf16 queries",
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "calls_ms": {n: round(x, 4) for n, x in ms.items()},
        "encode_GBps": round((n_el * 2 + packed) / (ms["encode"] * 1e-3) / 1e9, 2),
        "reconstruct_GBps": round((packed + 2 * H * C * d * 2 + n_el * 2) / (ms["reconstruct"] * 1e-3) / 1e9, 2),
        "attend_q_tokens_per_s": round(Tq / (ms["attend"] * 1e-3), 1),
        "attend_TFLOPs": round(att_tflops, 2),
        "attend_frac_of_bf16_peak": round(att_tflops / BF16_PEAK_TFLOPS, 4),
    }


def rollout_cpu_baseline(cfgs, k_l0, v_l0, q_l0, n_layers, step_tokens, budget_s=14.0):
    """The oracle, as it stands, on a bounded sample of the long-rollout
    workload: head 0 of layer 0, its K and V streams encoded call after call
    (4680 tokens each, warm-started) for about two thirds of the budget, then
    the attention of 256 of that head's queries over the keys encoded so
    far.  The per-token encode time and the per-(query, key) attention time
    are scaled to the step's work (every layer and head: the chunk's encode,
    the 4680-query attention over the 187200-token cache) and reported as
    query tokens per second like the GPU line."""
    import numpy as np
    import torch
    from oracle import attend as o_attend
    from oracle import stream as o_stream

    n_call = cfgs.chunk_tokens
    H, T, d, Tq = cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.q_tokens
    streams = [o_stream.Stream(1, d, cfgs.n_clusters, cfgs.iters, cfgs.n_stages, cfgs.bits, cfgs.group, "bf16")
               for _ in range(2)]
    t = time.perf_counter()
    calls = 0
    while calls < T // n_call and time.perf_counter() - t < budget_s * 2 / 3:
        for s, x in zip(streams, (k_l0, v_l0)):
            s.encode(x[0:1, calls * n_call:(calls + 1) * n_call].float().cpu().numpy())
        calls += 1
    t_enc = time.perf_counter() - t
    nq = 256
    q = q_l0[0:1, :nq].float().cpu().numpy()
    t = time.perf_counter()
    o_attend.attend(q, streams[0].xhat(), streams[1].xhat())
    t_att = time.perf_counter() - t
    keys = calls * n_call
    enc_per_token = t_enc / (2 * keys)                 # per token of one stream
    att_per_pair = t_att / (nq * keys)
    step_s = enc_per_token * 2 * n_layers * H * step_tokens + att_per_pair * n_layers * H * Tq * T
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": round(n_layers * Tq / step_s, 6), "unit": "query tokens/s", "cores": cores,
            "blas_threads": torch.get_num_threads(), "kind": "oracle",
            "seconds": round(t_enc + t_att, 2),
            "sample": f"long_rollout layer 0, head 0: oracle encode of the first {calls} calls of 4680 tokens "
                      f"(K and V, warm-started; {t_enc:.1f} s), attention of {nq} queries over those {keys} keys "
                      f"({t_att:.2f} s); per-token encode and per-(query, key) attention times scaled to one "
                      f"step over {n_layers} layers x {H} heads (chunk encode + 4680-query attention over "
                      f"{T} keys)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU; the path would shard by heads and layers "
                          "with no exchange, and no multi-GPU run is made"}))
        sys.exit(2)
    if args.xlayer:
        xlayer_main(args)
        return
    if args.fresh:
        fresh_main(args)
        return
    if args.reuse:
        reuse_main(args)
        return
    if args.outliers:
        outliers_main(args)
        return
    if args.wide:
        wide_main(args)
        return
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth

    dev = torch.device("cuda:0")
    L = args.layers or 30
    cfgs = synth.scaled(synth.LONG_ROLLOUT, n_layers=L)
    H, T, d, Tq = cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.q_tokens
    S, b, G, C = cfgs.n_stages, cfgs.bits, cfgs.group, cfgs.n_clusters
    n_call = cfgs.chunk_tokens
    n_calls = T // n_call
    Tf = T + n_call
    cfg = qkv.config(L, H, d, C, S, b, G, kmeans_iters=cfgs.iters, max_tokens=Tf, max_chunk_tokens=n_call,
                     max_chunks=n_calls + 1, kv_dtype=qkv.QKV_BF16, max_query_tokens=Tq)
    codec = qkv.Codec(cfg, device=dev)
    # build the cache: 40 calls of 4680 tokens per layer (untimed)
    t_build = time.perf_counter()
    new_k = torch.empty((L, H, n_call, d), dtype=torch.bfloat16, device=dev)
    new_v = torch.empty_like(new_k)
    k0 = v0 = None
    for l in range(L):
        k = synth.kv_tokens(cfgs, l, 0, 0, Tf, device=dev)
        v = synth.kv_tokens(cfgs, l, 1, 0, Tf, device=dev)
        for i in range(n_calls):
            codec.encode_chunk(k[:, i * n_call:(i + 1) * n_call], v[:, i * n_call:(i + 1) * n_call], layer0=l)
        new_k[l].copy_(k[:, T:])
        new_v[l].copy_(v[:, T:])
        if l == 0:
            k0, v0 = k, v
        del k, v
    qs = torch.stack([synth.queries(cfgs, l, Tq, device=dev) for l in range(L)])
    torch.cuda.synchronize()
    print(f"# built {L} layers x {T} tokens in {time.perf_counter() - t_build:.1f} s", file=sys.stderr, flush=True)
    out = torch.empty((H, Tq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((H, Tq), dtype=torch.float32, device=dev)
    rec = torch.empty((L, H, Tf, d), dtype=torch.bfloat16, device=dev)
    ev = {name: [] for name in ("attend", "encode", "reconstruct", "rewind")}
    att_calls = []

    def step(record):
        m = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        a = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
        m[0].record()
        a[0].record()
        for l in range(L):
            codec.attend(l, qs[l], out=out, lse=lse)
            a[l + 1].record()
        m[1].record()
        codec.encode_chunk(new_k, new_v, layer0=0)
        m[2].record()
        codec.reconstruct(0, L, 0, 0, Tf, out=rec)
        codec.reconstruct(0, L, 1, 0, Tf, out=rec)
        m[3].record()
        codec.rewind(0, L, T)
        m[4].record()
        if record:
            for i, n in enumerate(ev):
                ev[n].append((m[i], m[i + 1]))
            att_calls.extend(zip(a[:-1], a[1:]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"# timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)
    ms = {n: _avg_ms(p) for n, p in ev.items()}
    ms_attend_call = _avg_ms(att_calls)
    att_sorted = sorted(x.elapsed_time(y) for x, y in att_calls)

    def pct(q):
        return round(att_sorted[min(len(att_sorted) - 1, int(q * len(att_sorted)))], 4)
    ms_step = wall * 1e3 / args.steps

    # traced leg (not timed): per-kernel HIP events of two more steps
    codec.trace(True)
    for _ in range(2):
        step(False)
    torch.cuda.synchronize()
    kt = codec.trace_read()
    codec.trace(False)

    def kernel_ms(name):
        n, tot = kt.get(name, (0, 0.0))
        return (tot / n, n) if n else (None, 0)

    # algorithmic work per launch
    id_b = 1
    tok_packed = S * d * b // 8 + S * (d // G) * 4 + id_b        # bytes per token of one stream
    enc_tokens = 2 * L * H * n_call                              # tokens of one encode call
    cb_bytes = C * d * 2
    quant_bytes = enc_tokens * (2 * d + tok_packed) + 2 * L * H * cb_bytes
    recon_tokens = L * H * Tf                                    # per reconstruct call (one tensor)
    recon_bytes = recon_tokens * (tok_packed + 2 * d) + L * H * (n_calls + 1) * cb_bytes
    assign_flops = enc_tokens * 2.0 * C * d
    assign_bytes = enc_tokens * (2 * d + id_b) + 2 * L * H * cb_bytes
    update_bytes = enc_tokens * 2 * d + 2 * L * H * cb_bytes
    att_flops = 4.0 * H * Tq * T * d
    hbm_ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)

    def hbm(name, nbytes, kernel):
        t, n = kernel_ms(kernel)
        if t is None:
            return None
        gbs = nbytes / (t * 1e-3) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "launch_ms": round(t, 4),
                "launches": n, "bytes_per_launch": int(nbytes)}

    rooflines = {}
    t_att, n_att = kernel_ms("k_attend3")
    if t_att:
        tf = att_flops / (t_att * 1e-3) / 1e12
        rooflines["attend"] = {"kernel": "k_attend3", "bound": "mfma", "achieved": round(tf, 2),
                               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                               "launch_ms": round(t_att, 4), "launches": n_att, "flops_per_launch": att_flops}
    rooflines["quantize"] = hbm("quantize", quant_bytes, "k_quantize")
    if rooflines["quantize"]:
        # the quantizer's own arithmetic: per element the base subtraction and,
        # per stage, the group's min and max search, subtract z, scale by 1/sigma,
        # round, clamp, multiply-add back, subtract (separately rounded fp32)
        ops = enc_tokens * d * (1 + 8 * S)
        tops = ops / (rooflines["quantize"]["launch_ms"] * 1e-3) / 1e12
        rooflines["quantize"]["alu"] = {"bound": "alu", "achieved": round(tops, 2), "peak": ALU_PEAK_TOPS,
                                        "unit": "Top/s (fp32 vector operations)",
                                        "frac": round(tops / ALU_PEAK_TOPS, 4), "ops_per_launch": ops}
    rooflines["reconstruct"] = hbm("reconstruct", recon_bytes, "k_reconstruct")
    rooflines["update"] = hbm("update", update_bytes, "k_update_sorted")
    t_as, n_as = kernel_ms("k_assign_mfma")
    if t_as:
        tf = assign_flops / (t_as * 1e-3) / 1e12
        cap = min(1.0, (assign_flops / assign_bytes) / hbm_ridge)
        rooflines["assign"] = {"kernel": "k_assign_mfma", "bound": "mfma", "achieved": round(tf, 2),
                               "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                               "hbm_cap_frac": round(cap, 4), "launch_ms": round(t_as, 4), "launches": n_as,
                               "flops_per_launch": assign_flops, "bytes_per_launch": int(assign_bytes)}
    kernels = {k: {"launches": n, "avg_ms": round(tot / n, 4)} for k, (n, tot) in kt.items()}

    att_tflops = att_flops / (ms_attend_call * 1e-3) / 1e12
    result = {
        "metric": "KV quantize+pack GB/s and fused dequant-attention tokens/s; % of HBM/MFMA peak",
        "value": round(L * Tq / (ms_step * 1e-3), 1),
        "unit": "query tokens/s (a 4680-token chunk through all 30 layers' packed caches, per whole step: "
                "attention + the chunk's encode + full reconstruct)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded prototype/drift/outlier generator, device-generated)",
        "config": {"workload": f"long_rollout: {L} layers x K,V bf16 [12, 187200, 128] (34.5 GB at 30 layers) "
                               "built by 40 calls of 4680 tokens per layer; C=256, 5 iters, 3-stage INT2 G=32; "
                               "step = 4680 bf16 queries attend each layer, the next 4680-token chunk is encoded "
                               "into all layers, every layer reconstructed (bf16)",
                   "layers": L, "heads": H, "tokens": T, "head_dim": d, "clusters": C, "stages": S, "bits": b,
                   "group": G, "q_tokens": Tq, "chunk_tokens": n_call},
        "calls_ms": {"attend_per_layer": round(ms_attend_call, 4),
                     "attend_per_layer_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
                     "attend_all_layers": round(ms["attend"], 4),
                     "encode_chunk_all_layers": round(ms["encode"], 4),
                     "reconstruct_all_layers_k_and_v": round(ms["reconstruct"], 4),
                     "rewind": round(ms["rewind"], 4)},
        "attend_q_tokens_per_s": round(L * Tq / (ms["attend"] * 1e-3), 1),
        "attend_TFLOPs": round(att_tflops, 2),
        "encode_GBps": round((enc_tokens * (2 * d + tok_packed)) / (ms["encode"] * 1e-3) / 1e9, 2),
        "reconstruct_GBps": round(2 * recon_bytes / (ms["reconstruct"] * 1e-3) / 1e9, 2),
        "roofline": {"kernel": "qkv_attend (k_attend3 + k_attend_merge), per layer", "bound": "mfma",
                     "achieved": round(att_tflops, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(os.path.join(ROOT, "kv_cache_quantization_head_amd",
                                                              "csrc", "attend.hip"))},
        "rooflines": rooflines,
        "kernels_traced": kernels,
    }
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = rollout_cpu_baseline(cfgs, k0, v0, qs[0], L, n_call)
    del codec, rec, k0, v0, qs, new_k, new_v
    torch.cuda.empty_cache()
    if not args.no_wan_layer:
        result["wan_layer"] = wan_layer_step(args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
