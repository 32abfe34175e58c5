"""Python binding of the AbridgeKV attention hot-path library (``libabk.so``).

Argument marshalling only: every step of the path runs in the HIP library
behind the C ABI declared in ``include/abk.h``. Torch tensors are used for
device memory and streams; their data pointers are handed over as plain
pointers. If the library has not been built this module raises ImportError
(there is no fallback).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ABK_LIB") or os.path.join(_HERE, "libabk.so")

OK, INVALID_ARG, OUT_OF_PAGES, BAD_STATE, HIP_ERROR, UNSUPPORTED = range(6)
F32, BF16 = 0, 1

SYMBOLS = [
    "abk_pool_create", "abk_pool_destroy", "abk_seq_create", "abk_seq_release",
    "abk_write_prompt", "abk_append_kv", "abk_decode_attention", "abk_append_decode",
    "abk_compress_block",
    "abk_free_block", "abk_seq_query", "abk_export_layout", "abk_read_rows",
    "abk_pool_stats", "abk_budget_pool_stats", "abk_synth_fill", "abk_blockmask_attention",
    "abk_prefill_prompt", "abk_debug_fail_allocs", "abk_decode_attention_noalloc",
    "abk_last_error",
]


class AbkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"abk status {status}: {msg}")
        self.status = status


class PoolConfig(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("block_tokens", ctypes.c_int32), ("num_pause", ctypes.c_int32),
        ("layer_quota", ctypes.POINTER(ctypes.c_int32)),
        ("layer_pause", ctypes.POINTER(ctypes.c_int32)),
        ("page_rows", ctypes.c_int32), ("max_seqs", ctypes.c_int32),
        ("pool_bytes", ctypes.c_int64), ("max_position", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("rope_base", ctypes.c_double),
        ("compress", ctypes.c_int32), ("host_only", ctypes.c_int32),
        ("decode_split_rows", ctypes.c_int32),
        ("head_quota", ctypes.POINTER(ctypes.c_int32)),
        ("budget_pool_pages", ctypes.POINTER(ctypes.c_int64)),
    ]


class SeqInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("prompt_len", "generated", "blocks_done", "open_rows", "resident_rows", "n_pages")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run python -m long_reasoning_kv_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64
        ip = ctypes.POINTER(ctypes.c_int32)
        sig = {
            "abk_pool_create": [ctypes.POINTER(PoolConfig), vp, ctypes.POINTER(vp)],
            "abk_pool_destroy": [vp],
            "abk_seq_create": [vp, i32, ip],
            "abk_seq_release": [vp, i32],
            "abk_write_prompt": [vp, i32, i32, vp, vp],
            "abk_append_kv": [vp, i32, i32, ip, vp, vp],
            "abk_decode_attention": [vp, i32, i32, ip, vp, vp, vp],
            "abk_append_decode": [vp, i32, i32, ip, vp, vp, vp, vp, vp],
            "abk_compress_block": [vp, i32, i32, ip, vp, vp, vp, vp, vp],
            "abk_free_block": [vp, i32, ip],
            "abk_seq_query": [vp, i32, i32, ctypes.POINTER(SeqInfo)],
            "abk_export_layout": [vp, i32, i32, ip, i32, ip, i32],
            "abk_read_rows": [vp, i32, i32, i32, i32, vp, vp],
            "abk_pool_stats": [vp, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)],
            "abk_synth_fill": [vp, i32, i32, u64],
            "abk_blockmask_attention": [vp, i32, i32, i32, vp, vp, vp, vp, vp],
            "abk_prefill_prompt": [vp, i32, i32, vp, vp, vp, vp, vp],
            "abk_debug_fail_allocs": [vp, i32],
            "abk_decode_attention_noalloc": [vp, i32, i32, ip, vp, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.abk_last_error.argtypes = []
        L.abk_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise AbkError(status, lib().abk_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ids(seq_ids):
    ids = list(seq_ids)
    return len(ids), (ctypes.c_int32 * max(1, len(ids)))(*ids)


class Pool:
    """A paged AbridgeKV cache on one GPU (or host bookkeeping only)."""

    def __init__(self, *, num_layers, num_q_heads, num_kv_heads, head_dim, block_tokens,
                 num_pause, layer_quota, layer_pause=None, page_rows=64, max_seqs=64,
                 pool_bytes=1 << 30, max_position=40960, dtype="bf16", rope_base=1e6,
                 compress=True, host_only=False, decode_split_rows=0, head_quota=None,
                 budget_pool_pages=None, stream=None):
        """head_quota: optional per-(layer, KV head) quotas, [L][Hkv] nested or
        flat; then per-(sequence, layer) queries and layouts name the pair
        (l, h) as layer l * Hkv + h. budget_pool_pages: optional page counts
        of one pool per distinct quota value (ascending)."""
        self.L = num_layers
        self.Hq, self.Hkv, self.D = num_q_heads, num_kv_heads, head_dim
        self.C, self.page_rows = block_tokens, page_rows
        self.dtype = dtype
        self.quota = list(layer_quota)
        self.head_quota = None
        self._head_quota = None
        self._budget = (ctypes.c_int64 * len(budget_pool_pages))(*budget_pool_pages) \
            if budget_pool_pages is not None else None
        if head_quota is not None:
            flat = [int(x) for row in head_quota for x in (row if hasattr(row, "__iter__") else [row])]
            if len(flat) != num_layers * num_kv_heads:
                raise ValueError("head_quota needs num_layers x num_kv_heads entries")
            self.head_quota = [flat[l * num_kv_heads:(l + 1) * num_kv_heads] for l in range(num_layers)]
            self._head_quota = (ctypes.c_int32 * len(flat))(*flat)
        self.pause = list(layer_pause) if layer_pause is not None else [num_pause] * num_layers
        self._quota = (ctypes.c_int32 * num_layers)(*self.quota)
        self._pause = (ctypes.c_int32 * num_layers)(*layer_pause) if layer_pause is not None else None
        cfg = PoolConfig(
            num_layers, num_q_heads, num_kv_heads, head_dim, block_tokens, num_pause,
            ctypes.cast(self._quota, ctypes.POINTER(ctypes.c_int32)),
            ctypes.cast(self._pause, ctypes.POINTER(ctypes.c_int32)) if self._pause else None,
            page_rows, max_seqs, pool_bytes, max_position,
            {"f32": F32, "bf16": BF16}[dtype], rope_base, int(compress), int(host_only),
            decode_split_rows,
            ctypes.cast(self._head_quota, ctypes.POINTER(ctypes.c_int32)) if self._head_quota else None,
            ctypes.cast(self._budget, ctypes.POINTER(ctypes.c_int64)) if self._budget else None)
        if stream is None and not host_only:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        self.stream = stream
        h = ctypes.c_void_p()
        _check(lib().abk_pool_create(ctypes.byref(cfg), ctypes.c_void_p(stream or 0), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().abk_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def seq_create(self, prompt_len: int) -> int:
        sid = ctypes.c_int32()
        _check(lib().abk_seq_create(self._h, prompt_len, ctypes.byref(sid)))
        return sid.value

    def seq_release(self, sid: int):
        _check(lib().abk_seq_release(self._h, sid))

    def write_prompt(self, sid, layer, k, v):
        _check(lib().abk_write_prompt(self._h, sid, layer, _ptr(k), _ptr(v)))

    def append_kv(self, layer, seq_ids, k, v):
        n, ids = _ids(seq_ids)
        _check(lib().abk_append_kv(self._h, layer, n, ids, _ptr(k), _ptr(v)))

    def decode_attention(self, layer, seq_ids, q, out, lse):
        n, ids = _ids(seq_ids)
        _check(lib().abk_decode_attention(self._h, layer, n, ids, _ptr(q), _ptr(out), _ptr(lse)))

    def decode_attention_noalloc(self, layer, seq_ids, q, out, lse):
        """decode_attention with the split partials in the library's fixed
        per-GPU workspace: no device allocation; overlapping calls on one GPU
        race."""
        n, ids = _ids(seq_ids)
        _check(lib().abk_decode_attention_noalloc(self._h, layer, n, ids, _ptr(q), _ptr(out), _ptr(lse)))

    def append_decode(self, layer, seq_ids, k, v, q, out, lse):
        n, ids = _ids(seq_ids)
        _check(lib().abk_append_decode(self._h, layer, n, ids, _ptr(k), _ptr(v), _ptr(q), _ptr(out),
                                       _ptr(lse)))

    def compress_block(self, layer, seq_ids, q_pause, k_pause, v_pause, out, lse):
        n, ids = _ids(seq_ids)
        _check(lib().abk_compress_block(self._h, layer, n, ids, _ptr(q_pause), _ptr(k_pause),
                                        _ptr(v_pause), _ptr(out), _ptr(lse)))

    def free_block(self, seq_ids):
        n, ids = _ids(seq_ids)
        _check(lib().abk_free_block(self._h, n, ids))

    def seq_query(self, sid, layer) -> dict:
        info = SeqInfo()
        _check(lib().abk_seq_query(self._h, sid, layer, ctypes.byref(info)))
        return {n: getattr(info, n) for n, _ in SeqInfo._fields_}

    def export_layout(self, sid, layer):
        info = self.seq_query(sid, layer)
        npg, nr = max(1, info["n_pages"]), max(1, info["resident_rows"])
        pages = (ctypes.c_int32 * npg)()
        pos = (ctypes.c_int32 * nr)()
        _check(lib().abk_export_layout(self._h, sid, layer, pages, npg, pos, nr))
        return list(pages)[:info["n_pages"]], list(pos)[:info["resident_rows"]]

    def read_rows(self, sid, layer, row0, nrows, k_out, v_out):
        _check(lib().abk_read_rows(self._h, sid, layer, row0, nrows, _ptr(k_out), _ptr(v_out)))

    def budget_stats(self) -> list:
        """Per budget level: {quota, pages_used, pages_free} (one entry with
        quota -1 when the pool is shared)."""
        out, k, n = [], 0, 1
        while k < n:
            lv, q, u, f = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64(), ctypes.c_int64()
            _check(lib().abk_budget_pool_stats(self._h, k, ctypes.byref(lv), ctypes.byref(q), ctypes.byref(u),
                                               ctypes.byref(f)))
            n = lv.value
            out.append({"quota": q.value, "pages_used": u.value, "pages_free": f.value})
            k += 1
        return out

    def stats(self) -> dict:
        a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib().abk_pool_stats(self._h, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
        return {"pages_used": a.value, "pages_free": b.value, "resident_bytes": c.value}

    def blockmask_attention(self, layer, prompt_len, text_tokens, q, k, v, out, lse):
        _check(lib().abk_blockmask_attention(self._h, layer, prompt_len, text_tokens, _ptr(q), _ptr(k),
                                             _ptr(v), _ptr(out), _ptr(lse)))

    def prefill_prompt(self, sid, layer, q, k, v, out, lse):
        _check(lib().abk_prefill_prompt(self._h, sid, layer, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(lse)))

    def debug_fail_allocs(self, after: int):
        """Test support: the workspace growth after `after` more successful
        ones fails (-1: off)."""
        _check(lib().abk_debug_fail_allocs(self._h, after))

    def synth_fill(self, sid, generated, seed):
        _check(lib().abk_synth_fill(self._h, sid, generated, seed & 0xFFFFFFFFFFFFFFFF))
