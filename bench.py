"""Benchmark of the hot path on one MI355X: encode + reconstruct + fused attention.

One step = one pass of the whole path over one Wan2.1-1.3B-shaped layer
(K and V bf16 [12 heads, 32760 tokens, d=128], C=256 clusters, 5 k-means
iterations, 2-stage INT2 with group 32):
  qkv_rewind to 0 (state reset, a one-thread kernel), qkv_encode_chunk of all
  32760 tokens (k-means + PRQ + packing, K and V), qkv_reconstruct of K and V
  (bf16 out), qkv_attend of a 4680-token bf16 query chunk over the packed
  cache.
Inputs are seeded synthetic tensors already resident in HBM.  Each library
call is also bracketed by HIP events on the stream it is launched on.

Prints ONE JSON line (see the repository's design notes for every field).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
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
    ap.add_argument("--layers", type=int, default=4,
                    help="layers of the model (--fresh; Wan2.1-1.3B has 30)")
    ap.add_argument("--reuse", action="store_true",
                    help="instead of the default step: encode a long-rollout layer (187200 tokens in 40 "
                         "calls) with codebook reuse and with per-call snapshots; time, reconstruction "
                         "error and storage cost of each")
    ap.add_argument("--outliers", action="store_true",
                    help="instead of the default step: the same wan_layer step with and without the "
                         "outlier-channel option; time of each call, reconstruction error and storage "
                         "cost of each mode")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy (a known-size "
                         "reference for HBM byte counters)")
    return ap.parse_args()


def cpu_baseline(cfgs, k_dev, v_dev, q_dev, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the same workload:
    whole heads of the layer, one after another, until about ``budget_s``
    seconds of CPU work are done.  Per head: full encode of K and V (k-means
    + PRQ), reconstruction, attention of all of that head's queries.  Scaled
    to the same GB/s unit as the GPU line (bf16 K+V bytes of the heads done
    per second)."""
    import numpy as np
    import torch
    from oracle import attend as o_attend
    from oracle import stream as o_stream

    threads = torch.get_num_threads()
    H = k_dev.shape[0]
    t = time.perf_counter()
    heads = 0
    while heads < H:
        k = k_dev[heads:heads + 1].float().cpu().numpy()
        v = v_dev[heads:heads + 1].float().cpu().numpy()
        q = q_dev[heads:heads + 1].float().cpu().numpy()
        xs = []
        for x in (k, v):
            s = o_stream.Stream(1, cfgs.head_dim, cfgs.n_clusters, cfgs.iters, cfgs.n_stages,
                                cfgs.bits, cfgs.group, "bf16")
            s.encode(x)
            xs.append(s.xhat())
        o_attend.attend(q, xs[0], xs[1])
        heads += 1
        if time.perf_counter() - t >= budget_s:
            break
    dt = time.perf_counter() - t
    sample_bytes = heads * 2 * k_dev.shape[1] * k_dev.shape[2] * 2     # bf16 K+V of the heads done
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": round(sample_bytes / dt / 1e9, 6), "unit": "GB/s", "cores": cores,
            "blas_threads": threads, "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"heads 0..{heads - 1} of {H} of the layer, K and V: full encode "
                      f"({cfgs.iters} k-means iterations + {cfgs.n_stages} PRQ stages), "
                      f"reconstruction, attention of all {q_dev.shape[1]} queries of each head"}


def recorded_traffic(kernel_source):
    """HBM bytes of one qkv_attend call (attention kernel + merge), from the
    committed counter summary, or None when the kernel source changed since
    it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "k_attend3_wan_layer_pmc.txt")
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
    cfg = qkv.config(2, H, d, C, cfgs.n_stages, cfgs.bits, cfgs.group, kmeans_iters=cfgs.iters,
                     max_tokens=T, max_chunks=1, kv_dtype=qkv.QKV_BF16, max_query_tokens=0, xlayer=1,
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
        "adapted_layer1_rel_sq_error_kv": layer1_error(codec_a)}), flush=True)


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
    L = args.layers
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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; the path shards by heads/layers "
                          "with no exchange (see the design notes), but no multi-GPU run exists"}))
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
    import torch
    import kv_cache_quantization_head_amd as qkv
    import synth

    dev = torch.device("cuda:0")
    cfgs = synth.WAN_LAYER
    H, T, d, Tq = cfgs.n_heads, cfgs.tokens, cfgs.head_dim, cfgs.q_tokens
    cfg = qkv.config(1, H, d, cfgs.n_clusters, cfgs.n_stages, cfgs.bits, cfgs.group,
                     kmeans_iters=cfgs.iters, max_tokens=T, max_chunks=1, kv_dtype=qkv.QKV_BF16,
                     max_query_tokens=Tq)
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
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if record else None
        if record: marks[0].record()
        codec.encode_chunk(k, v)
        if record: marks[1].record()
        codec.reconstruct(0, 1, 0, 0, T, out=rec[0])
        codec.reconstruct(0, 1, 1, 0, T, out=rec[1])
        if record: marks[2].record()
        codec.attend(0, q, out=out, lse=lse)
        if record:
            marks[3].record()
            ev["encode"].append((marks[0], marks[1]))
            ev["reconstruct"].append((marks[1], marks[2]))
            ev["attend"].append((marks[2], marks[3]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    print(f"# timed {args.steps} steps in {wall:.3f} s", file=sys.stderr, flush=True)

    def avg_ms(name):
        xs = [a.elapsed_time(b) for a, b in ev[name]]
        return sum(xs) / len(xs)

    ms = {n: avg_ms(n) for n in ev}
    ms_step = wall * 1e3 / args.steps
    n_el = 2 * H * T * d                                   # K + V elements
    kv_bytes = n_el * 2
    S, b, G = cfgs.n_stages, cfgs.bits, cfgs.group
    packed_bytes = n_el * (S * b / 8 + S * 4 / G) + 2 * H * T  # codes + meta + ids
    att_flops = 4.0 * H * Tq * T * d
    att_tflops = att_flops / (ms["attend"] * 1e-3) / 1e12
    codebook_bytes = 2 * H * cfgs.n_clusters * d * 2
    recon_gbs = (packed_bytes + codebook_bytes + n_el * 2) / (ms["reconstruct"] * 1e-3) / 1e9
    encode_gbs = (kv_bytes + packed_bytes) / (ms["encode"] * 1e-3) / 1e9
    result = {
        "metric": "KV quantize+pack GB/s and fused dequant-attention tokens/s; % of HBM/MFMA peak",
        "value": round(kv_bytes / (ms_step * 1e-3) / 1e9, 3),
        "unit": "GB/s (bf16 K+V cache bytes through encode + reconstruct + attend per step)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded prototype/drift/outlier generator)",
        "config": {"workload": "wan_layer: K,V bf16 [12, 32760, 128], C=256, 5 iters, 2-stage INT2 "
                               "G=32; 4680 bf16 queries", "heads": H, "tokens": T, "head_dim": d,
                   "clusters": cfgs.n_clusters, "stages": S, "bits": b, "group": G, "q_tokens": Tq},
        "calls_ms": {n: round(x, 4) for n, x in ms.items()},
        "encode_GBps": round(encode_gbs, 2),
        "reconstruct_GBps": round(recon_gbs, 2),
        "attend_q_tokens_per_s": round(Tq / (ms["attend"] * 1e-3), 1),
        "attend_TFLOPs": round(att_tflops, 2),
        "roofline": {"kernel": "qkv_attend (k_attend3 + k_attend_merge)", "bound": "mfma",
                     "achieved": round(att_tflops, 3), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(att_tflops / BF16_PEAK_TFLOPS, 4),
                     "traffic": recorded_traffic(os.path.join(ROOT, "kv_cache_quantization_head_amd",
                                                              "csrc", "kernels.hip"))},
    }
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.int16, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfgs, k, v, q)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
