"""AbridgeKV CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain fp64 reference for the attention hot path (positions, the block mask,
RoPE, softmax attention) plus an independent model of the page allocator. Only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it. The GPU library never loads it; the two share no
code. Inputs come from the caller (normally the ``synth`` generator).

The arithmetic lives in ``abk_oracle.c`` (compiled by :func:`build`); this
module marshals arguments and composes the steps in the order the method
states them:

* decode (one text query): visible keys by the mask -> cached keys
  RoPE(k) rounded to storage -> rotated query RoPE(q), rounded to storage the
  same way -> softmax attention (scale 1/sqrt(d) on the fp64 scores);
* compression of block b: every pause query PAUSE(b, j) with its own visible
  key set (prompt, retained code rows, the whole block, pause keys k <= j),
  then the code rows k < quota are what the layer keeps;
* per-head quotas: the same two steps for each KV head with its own quota,
  its query heads seeing that head only;
* block-mask prefill (training-forward attention): every token of a sequence
  laid out in training order (prompt, then each block's text followed by its
  pause tokens once the block is complete) as a query with its own visible set.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

PROMPT, TEXT, PAUSE = 0, 1, 2
F32, BF16 = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liborc.so")
# a build of the same source with other flags (the sanitizer test's) may stand in
_LOAD_PATH = os.environ.get("ABK_ORACLE_LIB") or _LIB_PATH
_lib = None


def build(verbose: bool = False) -> str:
    """Compile the oracle's C part (gcc, OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", "-o", _LIB_PATH + ".tmp",
           os.path.join(_HERE, "abk_oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


class _Layer(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int32), ("C", ctypes.c_int32), ("Kp", ctypes.c_int32),
                ("quota", ctypes.c_int32), ("compress", ctypes.c_int32)]


def lib():
    global _lib
    if _lib is None:
        if _LOAD_PATH == _LIB_PATH and not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LOAD_PATH)
        i64, i32, dbl, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_void_p
        lp = ctypes.POINTER(_Layer)
        L.orc_bitrev.argtypes = [i32, i32]
        L.orc_log2_exact.argtypes = [i32]
        L.orc_position.argtypes = [lp, i32, i64, i64]
        L.orc_position.restype = i64
        L.orc_creation_index.argtypes = [lp, i32, i64, i64]
        L.orc_creation_index.restype = i64
        L.orc_visible.argtypes = [lp, i32, i64, i64, i32, i64, i64]
        L.orc_visible_keys.argtypes = [lp, i64, i64, i32, i64, i64, vp, vp, vp, vp, i64]
        L.orc_visible_keys.restype = i64
        L.orc_round_bf16.argtypes = [dbl]
        L.orc_round_bf16.restype = dbl
        L.orc_round.argtypes = [dbl, i32]
        L.orc_round.restype = dbl
        L.orc_rope_rows.argtypes = [vp, vp, i64, i32, i32, dbl, i32, vp]
        L.orc_attention.argtypes = [vp, i32, i32, i32, i64, vp, vp, vp, vp]
        L.orc_attention_batch.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp, vp, vp]
        L.orc_num_threads.restype = i32
        L.orc_set_num_threads.argtypes = [i32]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


@dataclass(frozen=True)
class LayerView:
    """One layer's view of one sequence (the mask's parameters)."""
    P: int
    C: int
    Kp: int
    quota: int
    compress: bool = True

    def c(self) -> _Layer:
        return _Layer(self.P, self.C, self.Kp, self.quota, int(self.compress))


def bitrev(k: int, nbits: int) -> int:
    return lib().orc_bitrev(k, nbits)


def position(L: LayerView, kind: int, a: int, b: int = 0) -> int:
    return lib().orc_position(ctypes.byref(L.c()), kind, a, b)


def visible(L: LayerView, q, k) -> bool:
    """q, k: (kind, a, b) token identities."""
    return bool(lib().orc_visible(ctypes.byref(L.c()), q[0], q[1], q[2], k[0], k[1], k[2]))


def creation_index(L: LayerView, kind: int, a: int, b: int = 0) -> int:
    return lib().orc_creation_index(ctypes.byref(L.c()), kind, a, b)


def visible_keys(L: LayerView, G: int, nb: int, query):
    """Keys the mask shows to ``query`` when G text tokens exist and blocks < nb
    have their pause tokens. Returns (kind, a, b, pos) int arrays in creation
    order."""
    c = L.c()
    cap = L.P + G + (max(nb, query[1] + 1 if query[0] == PAUSE else 0) + 1) * max(L.Kp, 1) + 1
    kind = np.empty(cap, np.int32)
    a = np.empty(cap, np.int64)
    b = np.empty(cap, np.int64)
    pos = np.empty(cap, np.int64)
    n = lib().orc_visible_keys(ctypes.byref(c), G, nb, query[0], query[1], query[2],
                               _p(kind), _p(a), _p(b), _p(pos), cap)
    assert n <= cap
    return kind[:n].copy(), a[:n].copy(), b[:n].copy(), pos[:n].copy()


def round_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    f = np.vectorize(lambda t: lib().orc_round(float(t), dtype), otypes=[np.float64])
    return f(np.asarray(x, np.float64))


def rope_rows(x: np.ndarray, pos: np.ndarray, base: float, round_dtype: int = -1) -> np.ndarray:
    """x [n, H, d] doubles at positions pos[n] -> rotated (optionally rounded)."""
    x = np.ascontiguousarray(x, np.float64)
    n, H, d = x.shape
    pos = np.ascontiguousarray(pos, np.int64)
    y = np.empty_like(x)
    lib().orc_rope_rows(_p(x), _p(pos), n, H, d, base, round_dtype, _p(y))
    return y


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """q [Hq, d] (rotated), k/v [n, Hkv, d] -> out [Hq, d], lse [Hq]."""
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    Hq, d = q.shape
    n, Hkv, _ = k.shape
    out = np.empty((Hq, d))
    lse = np.empty(Hq)
    lib().orc_attention(_p(q), Hq, Hkv, d, n, _p(k), _p(v), _p(out), _p(lse))
    return out, lse


def attention_batch(q: np.ndarray, off: np.ndarray, k: np.ndarray, v: np.ndarray):
    """q [nq, Hq, d]; query r uses keys [off[r], off[r+1]) of k/v [N, Hkv, d]."""
    q = np.ascontiguousarray(q, np.float64)
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    off = np.ascontiguousarray(off, np.int64)
    nq, Hq, d = q.shape
    Hkv = k.shape[1]
    out = np.empty((nq, Hq, d))
    lse = np.empty((nq, Hq))
    lib().orc_attention_batch(_p(q), nq, Hq, Hkv, d, _p(off), _p(k), _p(v), _p(out), _p(lse))
    return out, lse


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


# ---- composed steps ----------------------------------------------------------

def decode(L: LayerView, G: int, nb: int, q_raw: np.ndarray, fetch, dtype: int, base: float):
    """Decode attention of text token G-1 at one layer.

    ``fetch(kind, a, b, which)`` returns raw (pre-RoPE) rows [n, Hkv, d] for
    token identities (arrays) and which in {'k', 'v'}. Returns (out [Hq, d],
    lse [Hq], keys) where keys = (kind, a, b, pos) of the rows attended to.
    """
    query = (TEXT, G - 1, 0)
    kind, a, b, pos = visible_keys(L, G, nb, query)
    k = rope_rows(fetch(kind, a, b, "k"), pos, base, dtype)
    v = fetch(kind, a, b, "v")
    qpos = np.array([position(L, *query)], np.int64)
    qr = rope_rows(q_raw[None], qpos, base, dtype)[0]  # rounded once, like stored keys
    out, lse = attention(qr, k, v)
    return out, lse, (kind, a, b, pos)


def compress(L: LayerView, G: int, nb: int, block: int, q_raw: np.ndarray, fetch, dtype: int,
             base: float, queries=None):
    """Pause-token attention of one compression of ``block`` at one layer.

    q_raw [Kp, Hq, d] are the pause queries (pre-RoPE). Returns (out [Kp,Hq,d],
    lse [Kp,Hq], code) where code = (kind, a, b, pos, k_cached, v) of the rows
    this layer keeps: pause k < quota, in k order. ``queries`` (optional) lists
    the pause indices to compute; out and lse then hold those rows, in order.
    """
    Kp = L.Kp
    queries = list(range(Kp)) if queries is None else [int(j) for j in queries]
    q_raw = np.asarray(q_raw)[queries]
    lists = [visible_keys(L, G, nb, (PAUSE, block, j)) for j in queries]
    kind = np.concatenate([t[0] for t in lists])
    a = np.concatenate([t[1] for t in lists])
    b = np.concatenate([t[2] for t in lists])
    pos = np.concatenate([t[3] for t in lists])
    off = np.zeros(len(queries) + 1, np.int64)
    off[1:] = np.cumsum([len(t[0]) for t in lists])
    k = rope_rows(fetch(kind, a, b, "k"), pos, base, dtype)
    v = fetch(kind, a, b, "v")
    qpos = np.array([position(L, PAUSE, block, j) for j in queries], np.int64)
    qr = rope_rows(q_raw, qpos, base, dtype)  # rounded once, like stored keys
    out, lse = attention_batch(qr, off, k, v)
    ck = np.arange(min(L.quota, Kp))
    cpos = np.array([position(L, PAUSE, block, j) for j in ck], np.int64)
    ckind = np.full(len(ck), PAUSE, np.int32)
    cb = np.full(len(ck), block, np.int64)
    code_k = rope_rows(fetch(ckind, cb, ck, "k"), cpos, base, dtype)
    code_v = fetch(ckind, cb, ck, "v")
    return out, lse, (ckind, cb, ck, cpos, code_k, code_v)


def _head_fetch(fetch, h: int):
    """fetch restricted to KV head h: rows [n, 1, d]."""
    return lambda kind, a, b, which: fetch(kind, a, b, which)[:, h:h + 1]


def decode_heads(Ls, G: int, nb: int, q_raw: np.ndarray, fetch, dtype: int, base: float):
    """Decode with a quota per (layer, KV head) (figure captions, Fig. 7: one
    head's quota halved or doubled; AI Radio transcript: a per-head schedule).
    Ls[h] is KV head h's view of the layer, with its own quota; the query heads
    of group h see KV head h only, with the visible set that quota gives.
    q_raw [Hq, d]. Returns (out [Hq, d], lse [Hq], keys per KV head)."""
    Hkv = len(Ls)
    g = q_raw.shape[0] // Hkv
    outs, lses, keys = [], [], []
    for h in range(Hkv):
        o, l, k = decode(Ls[h], G, nb, q_raw[h * g:(h + 1) * g], _head_fetch(fetch, h), dtype, base)
        outs.append(o)
        lses.append(l)
        keys.append(k)
    return np.concatenate(outs), np.concatenate(lses), keys


def compress_heads(Ls, G: int, nb: int, block: int, q_raw: np.ndarray, fetch, dtype: int, base: float,
                   queries=None):
    """Compression of ``block`` with a quota per (layer, KV head): every KV head
    h attends under its own view Ls[h] and keeps its own prefix k < quota.
    q_raw [Kp, Hq, d]. Returns (out [Kp, Hq, d], lse [Kp, Hq], code per KV
    head)."""
    Hkv = len(Ls)
    g = q_raw.shape[1] // Hkv
    outs, lses, codes = [], [], []
    for h in range(Hkv):
        o, l, c = compress(Ls[h], G, nb, block, q_raw[:, h * g:(h + 1) * g], _head_fetch(fetch, h), dtype,
                           base, queries)
        outs.append(o)
        lses.append(l)
        codes.append(c)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1), codes


def blockmask_prefill_heads(Ls, G: int, q_raw: np.ndarray, fetch, dtype: int, base: float, rows=None):
    """The block-mask prefill with a quota per (layer, KV head): KV head h's
    query heads under the mask of Ls[h] (its own kept code rows), seeing KV
    head h only. q_raw [T, Hq, d]. Returns (out [n, Hq, d], lse [n, Hq])."""
    Hkv = len(Ls)
    g = q_raw.shape[1] // Hkv
    outs, lses = [], []
    for h in range(Hkv):
        o, l = blockmask_prefill(Ls[h], G, np.asarray(q_raw)[:, h * g:(h + 1) * g], _head_fetch(fetch, h), dtype,
                                 base, rows)
        outs.append(o)
        lses.append(l)
    return np.concatenate(outs, axis=1), np.concatenate(lses, axis=1)


def training_tokens(L: LayerView, G: int):
    """Token identities (kind, a, b) of a sequence with G text tokens in
    training order (the creation order of Fig. 2(a) in the figure captions):
    the prompt, then per block its C text tokens, followed, when the block is
    complete and compression is on, by its Kp pause tokens."""
    kind, a, b = [PROMPT] * L.P, list(range(L.P)), [0] * L.P
    nb = G // L.C if L.compress else 0
    for blk in range((G + L.C - 1) // L.C):
        n = min(L.C, G - blk * L.C)
        kind += [TEXT] * n
        a += list(range(blk * L.C, blk * L.C + n))
        b += [0] * n
        if blk < nb:
            kind += [PAUSE] * L.Kp
            a += [blk] * L.Kp
            b += list(range(L.Kp))
    return np.array(kind, np.int32), np.array(a, np.int64), np.array(b, np.int64)


def blockmask_prefill(L: LayerView, G: int, q_raw: np.ndarray, fetch, dtype: int, base: float,
                      rows=None):
    """Attention of the tokens of a training-order sequence under the block mask
    (Fig. 2(a) of the figure captions), one layer.

    q_raw [T, Hq, d]: pre-RoPE queries of all T tokens in training order.
    ``fetch`` as in :func:`decode`. ``rows`` (optional) lists the token indices
    to compute. Each query attends to the keys the mask shows it among the
    tokens created before it, every key and query rotated at its own position
    and rounded once to the storage dtype. Returns (out [n, Hq, d], lse [n, Hq]).
    """
    kind, a, b = training_tokens(L, G)
    nb = G // L.C if L.compress else 0
    rows = list(range(len(kind))) if rows is None else [int(r) for r in rows]
    lists = [visible_keys(L, G, nb, (int(kind[r]), int(a[r]), int(b[r]))) for r in rows]
    kk = np.concatenate([t[0] for t in lists])
    ka = np.concatenate([t[1] for t in lists])
    kb = np.concatenate([t[2] for t in lists])
    kpos = np.concatenate([t[3] for t in lists])
    off = np.zeros(len(rows) + 1, np.int64)
    off[1:] = np.cumsum([len(t[0]) for t in lists])
    k = rope_rows(fetch(kk, ka, kb, "k"), kpos, base, dtype)
    v = fetch(kk, ka, kb, "v")
    qpos = np.array([position(L, int(kind[r]), int(a[r]), int(b[r])) for r in rows], np.int64)
    qr = rope_rows(np.asarray(q_raw)[rows], qpos, base, dtype)
    return attention_batch(qr, off, k, v)
