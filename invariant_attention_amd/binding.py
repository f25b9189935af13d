"""Thin ctypes binding over libinvattn.so: the C entry points under the same names.

Argument marshalling only -- tensors become device pointers, the stream
becomes a hipStream_t -- every step of the path runs in the library's HIP
kernels.  There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libinvattn.so")

IA_OK = 0
IA_ERR_INVALID_ARG = 1
IA_ERR_UNSUPPORTED_CONFIG = 2
IA_ERR_WORKSPACE_TOO_SMALL = 3
IA_ERR_OUT_OF_PAGES = 4
IA_ERR_PAGE_REFERENCED = 5
IA_ERR_HIP = 6
IA_ERR_INTERNAL = 7
IA_KV_BF16 = 0
IA_KV_FP8_E4M3 = 1
IA_SPLIT_FIXED = 0
IA_SPLIT_BY_COUNT = 1
IA_DECODE_AUTO = 0
IA_DECODE_SPLIT = 1
IA_DECODE_WIDE = 2
IA_DECODE_SPREAD = 3
IA_KV_HINT_AUTO = 0
IA_KV_HINT_STREAM = 1
IA_KV_HINT_CACHED = 2
IA_PREFILL_AUTO = 0
IA_PREFILL_FOLD = 1
IA_PREFILL_SPLIT = 2
IA_POOL_CONSTANT_HASH = 1

EXPORTS = [
    "ia_create", "ia_destroy", "ia_last_error", "ia_version", "ia_decode_workspace_bytes",
    "ia_prefill_workspace_bytes", "ia_kv_append", "ia_paged_attn_decode", "ia_paged_attn_prefill",
    "ia_pool_create", "ia_pool_destroy", "ia_seq_begin", "ia_seq_append_tokens", "ia_seq_reserve",
    "ia_seq_commit", "ia_seq_block_table", "ia_seq_len", "ia_seq_end", "ia_pool_evict", "ia_pool_page_refs",
    "ia_pool_page_published", "ia_pool_num_free", "ia_rmsnorm", "ia_gemm_bf16", "ia_validate_slots",
    "ia_validate_attention_args", "ia_paged_attn_decode_noalloc", "ia_decode_noalloc_scratch_bytes",
    "ia_stream_read", "ia_stream_read_sink_bytes",
]


class IAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"invattn status {status}: {msg}")
        self.status = status


class ia_config(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("split_tokens", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("split_policy", ctypes.c_int32), ("sm_scale", ctypes.c_float), ("sliding_window", ctypes.c_int32),
        ("decode_kernel", ctypes.c_int32), ("kv_cache_hint", ctypes.c_int32), ("prefill_grid", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Loads the in-tree library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with python -m invariant_attention_amd.build")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64p, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "ia_create": ([ctypes.POINTER(ia_config), ctypes.POINTER(vp)], ctypes.c_int),
        "ia_destroy": ([vp], None),
        "ia_last_error": ([], ctypes.c_char_p),
        "ia_version": ([], ctypes.c_char_p),
        "ia_decode_workspace_bytes": ([vp, i32, i32], sz),
        "ia_prefill_workspace_bytes": ([vp, i32, i32, i32, i32], sz),
        "ia_kv_append": ([vp, vp, vp, i64p, i32, vp, vp, i32, vp, vp, vp], ctypes.c_int),
        "ia_paged_attn_decode": ([vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, i32, i32, vp, vp, sz, vp], ctypes.c_int),
        "ia_paged_attn_prefill": ([vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, sz, vp],
                                  ctypes.c_int),
        "ia_pool_create": ([i32, i32, i32, ctypes.POINTER(vp)], ctypes.c_int),
        "ia_pool_destroy": ([vp], None),
        "ia_seq_begin": ([vp, vp, i32, ctypes.POINTER(vp), ctypes.POINTER(i32)], ctypes.c_int),
        "ia_seq_append_tokens": ([vp, vp, vp, i32], ctypes.c_int),
        "ia_seq_reserve": ([vp, vp, i32, vp], ctypes.c_int),
        "ia_seq_commit": ([vp, vp, i32], ctypes.c_int),
        "ia_seq_block_table": ([vp, vp, i32, ctypes.POINTER(i32)], ctypes.c_int),
        "ia_seq_len": ([vp], i32),
        "ia_seq_end": ([vp, vp], ctypes.c_int),
        "ia_pool_evict": ([vp, i32, ctypes.POINTER(i32)], ctypes.c_int),
        "ia_pool_page_refs": ([vp, i32], i32),
        "ia_pool_page_published": ([vp, i32], i32),
        "ia_pool_num_free": ([vp], i32),
        "ia_rmsnorm": ([vp, vp, i32, i32, ctypes.c_float, vp, vp], ctypes.c_int),
        "ia_gemm_bf16": ([vp, vp, i32, i32, i32, vp, vp], ctypes.c_int),
        "ia_validate_slots": ([vp, vp, i32, i32, i32], ctypes.c_int),
        "ia_validate_attention_args": ([vp, vp, i32, i32, vp, i32, i32, i32, i32], ctypes.c_int),
        "ia_paged_attn_decode_noalloc": ([vp, vp, vp, vp, i32, vp, vp, vp, i32, vp, i32, i32, vp, vp],
                                         ctypes.c_int),
        "ia_decode_noalloc_scratch_bytes": ([], sz),
        "ia_stream_read": ([vp, sz, vp, sz, vp], ctypes.c_int),
        "ia_stream_read_sink_bytes": ([], sz),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != IA_OK:
        raise IAError(status, load().ia_last_error().decode())


def _p(t):
    """Device (or host) pointer of a tensor / numpy array, None for None."""
    if t is None:
        return None
    if isinstance(t, torch.Tensor):
        assert t.is_contiguous(), "tensors passed to invattn must be contiguous"
        return ctypes.c_void_p(t.data_ptr())
    return t.ctypes.data_as(ctypes.c_void_p)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


# ------------------------------------------------------------------ context

class Context:
    """An immutable ia_ctx (frozen configuration)."""

    def __init__(self, cfg: ia_config):
        self.cfg = cfg
        self.handle = ia_create(cfg)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.ia_destroy(h)
            self.handle = None


def ia_create(cfg: ia_config) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load().ia_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h


def make_config(Hq: int, Hkv: int, d: int, *, page_size: int = 16, split_tokens: int = 2048,
                kv_dtype: int = IA_KV_BF16, split_policy: int = IA_SPLIT_FIXED, sm_scale: float | None = None,
                sliding_window: int = 0, decode_kernel: int = IA_DECODE_AUTO,
                kv_cache_hint: int = IA_KV_HINT_AUTO, prefill_grid: int = IA_PREFILL_AUTO) -> ia_config:
    scale = float(1.0 / d ** 0.5) if sm_scale is None else float(sm_scale)
    return ia_config(Hq, Hkv, d, page_size, split_tokens, kv_dtype, split_policy, scale, sliding_window,
                     decode_kernel, kv_cache_hint, prefill_grid)


def ia_last_error() -> str:
    return load().ia_last_error().decode()


def ia_version() -> str:
    return load().ia_version().decode()


def ia_decode_workspace_bytes(ctx: Context, batch: int, max_seq_len: int) -> int:
    return int(load().ia_decode_workspace_bytes(ctx.handle, batch, max_seq_len))


def ia_prefill_workspace_bytes(ctx: Context, B: int, total_q: int, max_q_len: int, max_seq_len: int) -> int:
    return int(load().ia_prefill_workspace_bytes(ctx.handle, B, total_q, max_q_len, max_seq_len))


def ia_kv_append(ctx: Context, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None,
                 stream=None) -> None:
    T = int(slot_mapping.shape[0])
    _check(load().ia_kv_append(ctx.handle, _p(k_new), _p(v_new), _p(slot_mapping), T, _p(k_cache), _p(v_cache),
                               int(k_cache.shape[0]), _p(k_scale), _p(v_scale), _stream(stream)))


def ia_paged_attn_decode(ctx: Context, q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, out,
                         workspace, k_scale=None, v_scale=None, stream=None) -> None:
    B = int(seq_lens.shape[0])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().ia_paged_attn_decode(ctx.handle, _p(q), _p(k_cache), _p(v_cache), int(k_cache.shape[0]),
                                       _p(k_scale), _p(v_scale), _p(block_table), int(block_table.shape[1]),
                                       _p(seq_lens), B, int(max_seq_len), _p(out), _p(workspace), ws_bytes,
                                       _stream(stream)))


def ia_paged_attn_decode_noalloc(ctx: Context, q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int,
                                 out, k_scale=None, v_scale=None, stream=None) -> None:
    B = int(seq_lens.shape[0])
    _check(load().ia_paged_attn_decode_noalloc(ctx.handle, _p(q), _p(k_cache), _p(v_cache), int(k_cache.shape[0]),
                                               _p(k_scale), _p(v_scale), _p(block_table), int(block_table.shape[1]),
                                               _p(seq_lens), B, int(max_seq_len), _p(out), _stream(stream)))


def ia_decode_noalloc_scratch_bytes() -> int:
    return int(load().ia_decode_noalloc_scratch_bytes())


def ia_paged_attn_prefill(ctx: Context, q, cu_q_lens, seq_lens, k_cache, v_cache, block_table, max_q_len: int,
                          max_seq_len: int, out, k_scale=None, v_scale=None, workspace=None,
                          stream=None) -> None:
    B = int(seq_lens.shape[0])
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().ia_paged_attn_prefill(ctx.handle, _p(q), _p(cu_q_lens), _p(seq_lens), _p(k_cache), _p(v_cache),
                                        int(k_cache.shape[0]), _p(k_scale), _p(v_scale), _p(block_table),
                                        int(block_table.shape[1]), B, int(q.shape[0]), int(max_q_len),
                                        int(max_seq_len), _p(out), _p(workspace), ws_bytes, _stream(stream)))


# ---------------------------------------------------------- layer operators

def ia_rmsnorm(x, weight, eps: float, out, stream=None) -> None:
    """out[m] = RMSNorm(x[m]) * weight for x, out [M][H] bf16 and weight [H] bf16."""
    M, H = int(x.shape[0]), int(x.shape[1])
    _check(load().ia_rmsnorm(_p(x), _p(weight), M, H, float(eps), _p(out), _stream(stream)))


def ia_gemm_bf16(a, w, out, stream=None) -> None:
    """out = a @ w^T for a [M][K], w [N][K], out [M][N] (bf16)."""
    M, K = int(a.shape[0]), int(a.shape[1])
    N = int(w.shape[0])
    _check(load().ia_gemm_bf16(_p(a), _p(w), M, N, K, _p(out), _stream(stream)))


# --------------------------------------------------------------- page pool

class Pool:
    """Host page table with exact prefix sharing (ia_pool_*)."""

    def __init__(self, num_pages: int, page_size: int = 16, flags: int = 0):
        h = ctypes.c_void_p()
        _check(load().ia_pool_create(num_pages, page_size, flags, ctypes.byref(h)))
        self.handle = h
        self.page_size = page_size

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _lib is not None:
            _lib.ia_pool_destroy(h)
            self.handle = None


def _i32(values):
    arr = (ctypes.c_int32 * max(1, len(values)))(*values)
    return arr


def ia_seq_begin(pool: Pool, tokens) -> tuple[ctypes.c_void_p, int]:
    toks = _i32(list(tokens))
    seq = ctypes.c_void_p()
    cached = ctypes.c_int32()
    _check(load().ia_seq_begin(pool.handle, toks, len(tokens), ctypes.byref(seq), ctypes.byref(cached)))
    return seq, int(cached.value)


def ia_seq_append_tokens(pool: Pool, seq, tokens) -> None:
    _check(load().ia_seq_append_tokens(pool.handle, seq, _i32(list(tokens)), len(tokens)))


def ia_seq_reserve(pool: Pool, seq, n_new: int) -> list[int]:
    out = (ctypes.c_int64 * max(1, n_new))()
    _check(load().ia_seq_reserve(pool.handle, seq, n_new, out))
    return list(out[:n_new])


def ia_seq_commit(pool: Pool, seq, n_done: int) -> None:
    _check(load().ia_seq_commit(pool.handle, seq, n_done))


def ia_seq_block_table(seq) -> list[int]:
    n = ctypes.c_int32()
    load().ia_seq_block_table(seq, None, 0, ctypes.byref(n))
    out = (ctypes.c_int32 * max(1, n.value))()
    _check(load().ia_seq_block_table(seq, out, n.value, ctypes.byref(n)))
    return list(out[:n.value])


def ia_seq_len(seq) -> int:
    return int(load().ia_seq_len(seq))


def ia_seq_end(pool: Pool, seq) -> None:
    _check(load().ia_seq_end(pool.handle, seq))


def ia_pool_evict(pool: Pool, want: int) -> int:
    n = ctypes.c_int32()
    _check(load().ia_pool_evict(pool.handle, want, ctypes.byref(n)))
    return int(n.value)


def ia_pool_page_refs(pool: Pool, page: int) -> int:
    return int(load().ia_pool_page_refs(pool.handle, page))


def ia_pool_page_published(pool: Pool, page: int) -> int:
    return int(load().ia_pool_page_published(pool.handle, page))


def ia_pool_num_free(pool: Pool) -> int:
    return int(load().ia_pool_num_free(pool.handle))


# ------------------------------------------------------------ host validators

def _host_array(x, dtype):
    import numpy as np
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=dtype))


def ia_validate_slots(pool, slot_mapping, num_pages: int, page_size: int) -> None:
    """Host check of a kv_append slot mapping (raises IAError with the first violation)."""
    import numpy as np
    sl = _host_array(slot_mapping, np.int64)
    _check(load().ia_validate_slots(pool.handle if pool is not None else None, _p(sl), int(sl.shape[0]),
                                    int(num_pages), int(page_size)))


def ia_validate_attention_args(cu_q_lens, seq_lens, block_table, num_pages: int, page_size: int,
                               max_seq_len: int, total_q: int | None = None) -> None:
    """Host check of an attention call's lengths and block table; cu_q_lens None for decode."""
    import numpy as np
    sl = _host_array(seq_lens, np.int32)
    bt = _host_array(block_table, np.int32)
    cu = None if cu_q_lens is None else _host_array(cu_q_lens, np.int32)
    B = int(sl.shape[0])
    tq = (int(cu[-1]) if cu is not None else B) if total_q is None else int(total_q)
    _check(load().ia_validate_attention_args(_p(cu), _p(sl), B, tq, _p(bt), int(bt.shape[1]) if bt.ndim == 2 else 0,
                                             int(num_pages), int(page_size), int(max_seq_len)))


# --------------------------------------------------------- measurement helper

def ia_stream_read_sink_bytes() -> int:
    return int(load().ia_stream_read_sink_bytes())


def ia_stream_read(buf, sink, stream=None) -> None:
    """Streams every byte of the device tensor buf (the achievable-HBM reference kernel)."""
    _check(load().ia_stream_read(_p(buf), buf.numel() * buf.element_size(), _p(sink),
                                 sink.numel() * sink.element_size(), _stream(stream)))
