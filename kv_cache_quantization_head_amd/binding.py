"""ctypes binding of libqkv.so: the C-ABI of include/qkv.h, same names.

Only argument marshalling lives here: tensors are passed as device pointers
with the caller's current HIP stream; the library fails loudly when it is
missing.  There is no fallback path.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(HERE, "libqkv.so")

QKV_F32, QKV_BF16 = 0, 1
QKV_OK, QKV_E_INVAL, QKV_E_CAPACITY, QKV_E_STATE, QKV_E_ARENA, QKV_E_HIP, QKV_E_UNSUPPORTED = \
    0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "QKV_OK", -1: "QKV_E_INVAL", -2: "QKV_E_CAPACITY", -3: "QKV_E_STATE",
                -4: "QKV_E_ARENA", -5: "QKV_E_HIP", -6: "QKV_E_UNSUPPORTED"}


class qkv_config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_clusters", ctypes.c_int32),
                ("n_stages", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("kmeans_iters", ctypes.c_int32),
                ("max_tokens", ctypes.c_int64), ("max_chunk_tokens", ctypes.c_int64),
                ("max_chunks", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("max_query_tokens", ctypes.c_int64), ("xlayer", ctypes.c_int32),
                ("xlayer_rank", ctypes.c_int32), ("codebook_reuse", ctypes.c_int32),
                ("xlayer_adapt", ctypes.c_int32), ("outlier_channels", ctypes.c_int32)]


class qkv_layout_desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "codes_off", "codes_stage_stride", "codes_head_stride", "codes_token_stride",
        "meta_off", "meta_stage_stride", "meta_head_stride", "meta_token_stride",
        "ids_off", "ids_head_stride", "id_bytes",
        "codebook_off", "codebook_chunk_stride", "codebook_head_stride",
        "cnorm_off", "cnorm_chunk_stride", "cnorm_head_stride")] + [
        ("n_tokens", ctypes.c_int64), ("n_chunks", ctypes.c_int32), ("reserved", ctypes.c_int32)] + [
        (n, ctypes.c_uint64) for n in ("chmask_off", "chmask_chunk_stride", "chmask_head_stride")]


class qkv_trace_entry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_lib = None


def lib_path():
    return _LIB_PATH


def lib():
    """Load libqkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m kv_cache_quantization_head_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    cfgp = ctypes.POINTER(qkv_config)
    L.qkv_workspace_bytes.argtypes = [cfgp]
    L.qkv_workspace_bytes.restype = ctypes.c_size_t
    L.qkv_init.argtypes = [cfgp, vp, ctypes.c_size_t, vp, ctypes.POINTER(vp)]
    L.qkv_init.restype = ctypes.c_int
    L.qkv_encode_chunk.argtypes = [vp, i32, i32, vp, vp, i64, vp]
    L.qkv_encode_chunk.restype = ctypes.c_int
    L.qkv_attend.argtypes = [vp, i32, vp, i64, i32, vp, i32, vp, vp]
    L.qkv_attend.restype = ctypes.c_int
    L.qkv_attend_noalloc.argtypes = [vp, i32, vp, i64, i32, vp, i32, vp, vp]
    L.qkv_attend_noalloc.restype = ctypes.c_int
    L.qkv_attend_with_chunk.argtypes = [vp, i32, vp, i64, i32, vp, vp, i64, vp, i32, vp, vp]
    L.qkv_attend_with_chunk.restype = ctypes.c_int
    L.qkv_reconstruct.argtypes = [vp, i32, i32, i32, i64, i64, vp, i32, vp]
    L.qkv_reconstruct.restype = ctypes.c_int
    L.qkv_rewind.argtypes = [vp, i32, i32, i64, vp]
    L.qkv_rewind.restype = ctypes.c_int
    L.qkv_layout.argtypes = [vp, i32, i32, ctypes.POINTER(qkv_layout_desc)]
    L.qkv_layout.restype = ctypes.c_int
    L.qkv_chunk_starts.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int64), i32]
    L.qkv_chunk_starts.restype = ctypes.c_int
    L.qkv_adapted_blocks.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_uint64)]
    L.qkv_adapted_blocks.restype = ctypes.c_int
    L.qkv_trace.argtypes = [vp, i32]
    L.qkv_trace.restype = ctypes.c_int
    L.qkv_trace_read.argtypes = [vp, ctypes.POINTER(qkv_trace_entry), i32]
    L.qkv_trace_read.restype = ctypes.c_int
    L.qkv_destroy.argtypes = [vp]
    L.qkv_destroy.restype = None
    L.qkv_status_string.argtypes = [vp, ctypes.c_int]
    L.qkv_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


class QkvError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def status_string(status, ctx=None):
    return lib().qkv_status_string(ctx, status).decode()


def config(n_layers, n_heads, head_dim, n_clusters, n_stages, bits, group_size, kmeans_iters=5,
           max_tokens=0, max_chunk_tokens=0, max_chunks=1, kv_dtype=QKV_BF16,
           max_query_tokens=0, xlayer=0, xlayer_rank=0, codebook_reuse=0, xlayer_adapt=0,
           outlier_channels=0):
    return qkv_config(n_layers, n_heads, head_dim, n_clusters, n_stages, bits, group_size,
                      kmeans_iters, max_tokens, max_chunk_tokens, max_chunks, kv_dtype,
                      max_query_tokens, xlayer, xlayer_rank, codebook_reuse, xlayer_adapt,
                      outlier_channels)


def workspace_bytes(cfg):
    return int(lib().qkv_workspace_bytes(ctypes.byref(cfg)))


def _dtype_code(t):
    if t == torch.float32:
        return QKV_F32
    if t == torch.bfloat16:
        return QKV_BF16
    raise ValueError(f"unsupported dtype {t}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, ctx=None):
    if status != QKV_OK:
        raise QkvError(status, status_string(status, ctx))


class Codec:
    """One qkv context over a device arena allocated with torch."""

    def __init__(self, cfg, device="cuda", predictor=None):
        self.cfg = cfg
        self.device = torch.device(device)
        L = lib()
        nbytes = workspace_bytes(cfg)
        if nbytes == 0:
            raise QkvError(QKV_E_INVAL, "invalid configuration")
        # torch's caching allocator returns blocks aligned well beyond 256 bytes
        self.arena = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.predictor = predictor
        ctx = ctypes.c_void_p()
        pred_ptr = ctypes.c_void_p(predictor.data_ptr()) if predictor is not None else None
        _check(L.qkv_init(ctypes.byref(cfg), ctypes.c_void_p(self.arena.data_ptr()),
                          ctypes.c_size_t(nbytes), pred_ptr, ctypes.byref(ctx)))
        self.ctx = ctx

    def __del__(self):
        if getattr(self, "ctx", None) and _lib is not None:
            _lib.qkv_destroy(self.ctx)
            self.ctx = None

    @property
    def kv_dtype(self):
        return torch.bfloat16 if self.cfg.kv_dtype == QKV_BF16 else torch.float32

    def encode_chunk(self, k, v, layer0=0):
        """k, v: [n_layers, H, n, d] (or [H, n, d]) device tensors in the cache dtype."""
        if k.dim() == 3:
            k, v = k.unsqueeze(0), v.unsqueeze(0)
        if k.shape != v.shape or k.dtype != self.kv_dtype or v.dtype != self.kv_dtype:
            raise ValueError("k and v must share shape and the cache dtype")
        if k.shape[1] != self.cfg.n_heads or k.shape[3] != self.cfg.head_dim:
            raise ValueError("k/v shape does not match the configuration")
        k, v = k.contiguous(), v.contiguous()
        _check(lib().qkv_encode_chunk(self.ctx, layer0, k.shape[0], ctypes.c_void_p(k.data_ptr()),
                                      ctypes.c_void_p(v.data_ptr()), k.shape[2], _stream()), self.ctx)

    def attend(self, layer, q, out_dtype=torch.float32, with_lse=True, out=None, lse=None):
        """q: [H, n_q, d] device tensor (bf16 or fp32).  Returns (out, lse)."""
        H, n_q, d = q.shape
        if H != self.cfg.n_heads or d != self.cfg.head_dim:
            raise ValueError("q shape does not match the configuration")
        q = q.contiguous()
        if out is None:
            out = torch.empty((H, n_q, d), dtype=out_dtype, device=q.device)
        if with_lse and lse is None:
            lse = torch.empty((H, n_q), dtype=torch.float32, device=q.device)
        lse_ptr = ctypes.c_void_p(lse.data_ptr()) if with_lse else None
        _check(lib().qkv_attend(self.ctx, layer, ctypes.c_void_p(q.data_ptr()), n_q,
                                _dtype_code(q.dtype), ctypes.c_void_p(out.data_ptr()),
                                _dtype_code(out.dtype), lse_ptr, _stream()), self.ctx)
        return out, lse

    def attend_noalloc(self, layer, q, out, lse=None):
        """qkv_attend_noalloc: out [H, n_q, d] and lse [H, n_q] are the caller's;
        the split partials live in the library's fixed per-GPU array."""
        H, n_q, d = q.shape
        if H != self.cfg.n_heads or d != self.cfg.head_dim or tuple(out.shape) != (H, n_q, d):
            raise ValueError("q / out shape does not match the configuration")
        if not q.is_contiguous() or not out.is_contiguous():
            raise ValueError("q and out must be contiguous")
        lse_ptr = ctypes.c_void_p(lse.data_ptr()) if lse is not None else None
        _check(lib().qkv_attend_noalloc(self.ctx, layer, ctypes.c_void_p(q.data_ptr()), n_q,
                                        _dtype_code(q.dtype), ctypes.c_void_p(out.data_ptr()),
                                        _dtype_code(out.dtype), lse_ptr, _stream()), self.ctx)
        return out, lse

    def attend_with_chunk(self, layer, q, k_new, v_new, out_dtype=torch.float32, with_lse=True, out=None,
                          lse=None):
        """Attention over the packed cache of `layer` followed by the fresh
        chunk k_new, v_new ([H, n_new, d] bf16 device tensors).  Returns
        (out, lse)."""
        H, n_q, d = q.shape
        if H != self.cfg.n_heads or d != self.cfg.head_dim:
            raise ValueError("q shape does not match the configuration")
        if k_new.shape != v_new.shape or k_new.dim() != 3 or k_new.shape[0] != H or k_new.shape[2] != d:
            raise ValueError("fresh K/V shape does not match the configuration")
        if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
            raise ValueError("fresh K/V must be bf16")
        q, k_new, v_new = q.contiguous(), k_new.contiguous(), v_new.contiguous()
        n_new = k_new.shape[1]
        if out is None:
            out = torch.empty((H, n_q, d), dtype=out_dtype, device=q.device)
        if with_lse and lse is None:
            lse = torch.empty((H, n_q), dtype=torch.float32, device=q.device)
        lse_ptr = ctypes.c_void_p(lse.data_ptr()) if with_lse else None
        kp = ctypes.c_void_p(k_new.data_ptr()) if n_new else None
        vp = ctypes.c_void_p(v_new.data_ptr()) if n_new else None
        _check(lib().qkv_attend_with_chunk(self.ctx, layer, ctypes.c_void_p(q.data_ptr()), n_q,
                                           _dtype_code(q.dtype), kp, vp, n_new,
                                           ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype), lse_ptr,
                                           _stream()), self.ctx)
        return out, lse

    def reconstruct(self, layer0, n_layers, kv, t0, t1, out_dtype=torch.float32, out=None):
        H, d = self.cfg.n_heads, self.cfg.head_dim
        if out is None:
            out = torch.empty((n_layers, H, t1 - t0, d), dtype=out_dtype, device=self.device)
        _check(lib().qkv_reconstruct(self.ctx, layer0, n_layers, kv, t0, t1,
                                     ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype),
                                     _stream()), self.ctx)
        return out

    def rewind(self, layer0, n_layers, n_tokens):
        _check(lib().qkv_rewind(self.ctx, layer0, n_layers, n_tokens, _stream()), self.ctx)

    def trace(self, enable=True):
        """Record HIP events around every kernel of later calls (qkv_trace)."""
        _check(lib().qkv_trace(self.ctx, 1 if enable else 0), self.ctx)

    def trace_read(self):
        """{kernel: (launches, total ms)} since the last read (synchronizes)."""
        buf = (qkv_trace_entry * 64)()
        n = lib().qkv_trace_read(self.ctx, buf, 64)
        if n < 0:
            _check(n, self.ctx)
        return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 64))}

    def layout(self, layer, kv):
        d = qkv_layout_desc()
        _check(lib().qkv_layout(self.ctx, layer, kv, ctypes.byref(d)), self.ctx)
        return {name: getattr(d, name) for name, _ in d._fields_}

    def chunk_starts(self, layer):
        n = lib().qkv_chunk_starts(self.ctx, layer, None, 0)
        if n < 0:
            _check(n, self.ctx)
        buf = (ctypes.c_int64 * max(n, 1))()
        lib().qkv_chunk_starts(self.ctx, layer, buf, n)
        return [int(buf[i]) for i in range(n)]

    def adapted_blocks(self, layer):
        """Re-fitted predictor blocks of the transition into `layer`: [2, H, d, d] bf16 view."""
        off = ctypes.c_uint64()
        _check(lib().qkv_adapted_blocks(self.ctx, layer, ctypes.byref(off)), self.ctx)
        H, d = self.cfg.n_heads, self.cfg.head_dim
        return self.arena[off.value:off.value + 2 * H * d * d * 2].view(torch.bfloat16).view(2, H, d, d)

    # ---- read-back views of the arena (for tests and inspection) ----
    def _view(self, off, nbytes):
        return self.arena[off:off + nbytes]

    def codes(self, layer, kv, stage):
        """[H, n_tokens, d*bits/8] uint8 packed codes of one stage."""
        lay = self.layout(layer, kv)
        H, T = self.cfg.n_heads, self.cfg.max_tokens
        tok = lay["codes_token_stride"]
        base = lay["codes_off"] + stage * lay["codes_stage_stride"]
        v = self._view(base, H * T * tok).view(H, T, tok)
        return v[:, :lay["n_tokens"]]

    def meta(self, layer, kv, stage):
        """[H, n_tokens, d/G (+1 with outlier channels), 2] uint16 fp16 bit patterns (sigma, z)."""
        lay = self.layout(layer, kv)
        H, T = self.cfg.n_heads, self.cfg.max_tokens
        ng = lay["meta_token_stride"] // 4
        base = lay["meta_off"] + stage * lay["meta_stage_stride"]
        v = self._view(base, H * T * ng * 4).view(torch.int16).view(H, T, ng, 2)
        return v[:, :lay["n_tokens"]]

    def ids(self, layer, kv):
        lay = self.layout(layer, kv)
        H, T = self.cfg.n_heads, self.cfg.max_tokens
        nb = lay["id_bytes"]
        v = self._view(lay["ids_off"], H * T * nb)
        v = v.view(H, T) if nb == 1 else v.view(torch.int16).view(H, T)
        return v[:, :lay["n_tokens"]]

    def channel_mask(self, layer, kv, chunk):
        """[H, d/32] int32 outlier-channel flags of one chunk (bit j%32 of word j/32)."""
        lay = self.layout(layer, kv)
        if not lay["chmask_off"]:
            raise ValueError("outlier_channels is off")
        H, d = self.cfg.n_heads, self.cfg.head_dim
        base = lay["chmask_off"] + chunk * lay["chmask_chunk_stride"]
        return self._view(base, H * d // 8).view(torch.int32).view(H, d // 32)

    def codebook(self, layer, kv, chunk):
        """[H, C, d] snapshot of one chunk, in the cache dtype."""
        lay = self.layout(layer, kv)
        H, C, d = self.cfg.n_heads, self.cfg.n_clusters, self.cfg.head_dim
        eb = 2 if self.cfg.kv_dtype == QKV_BF16 else 4
        base = lay["codebook_off"] + chunk * lay["codebook_chunk_stride"]
        v = self._view(base, H * C * d * eb)
        return v.view(self.kv_dtype).view(H, C, d)
