"""Shared GPU-test plumbing: pools, seeded inputs from ``synth``, histories
driven through the C ABI, and the matching oracle references."""
from __future__ import annotations

import numpy as np
import torch

import long_reasoning_kv_amd as abk
import oracle
import synth
from oracle import PAUSE, PROMPT, TEXT, LayerView

TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}
ORC_DT = {"f32": oracle.F32, "bf16": oracle.BF16}


def seq_seed(base: int, i: int) -> int:
    return (base * 1000003 + i * 7919 + 17) & 0xFFFFFFFFFFFFFFFF


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Doubles exactly representable in dtype -> contiguous device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(TORCH_DT[dtype]).cuda().contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Run:
    """A pool plus the seeds of its sequences, so every input can be
    regenerated on the host for the oracle."""

    def __init__(self, *, L, Hq, Hkv, D, C, Kp, quota, pause=None, pr, dtype="bf16",
                 compress=True, max_seqs=64, pool_bytes=None, max_position=40960,
                 split_rows=0, base=1e6, seed=0, head_quota=None, budget_pool_pages=None):
        self.L, self.Hq, self.Hkv, self.D, self.C = L, Hq, Hkv, D, C
        self.pause_q_scale = 1.0  # multiplies the pause queries' normals (both sides)
        self.quota = list(quota)
        self.head_quota = [list(r) for r in head_quota] if head_quota is not None else None
        self.pause = list(pause) if pause is not None else [Kp] * L
        self.pr, self.dtype, self.compress, self.base = pr, dtype, compress, base
        esize = 4 if dtype == "f32" else 2
        if pool_bytes is None:
            pool_bytes = 64 << 20
        self.pool = abk.Pool(num_layers=L, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                             block_tokens=C, num_pause=Kp, layer_quota=quota, layer_pause=pause,
                             page_rows=pr, max_seqs=max_seqs, pool_bytes=pool_bytes,
                             max_position=max_position, dtype=dtype, rope_base=base,
                             compress=compress, decode_split_rows=split_rows, head_quota=head_quota,
                             budget_pool_pages=budget_pool_pages)
        self.page_bytes = (1 if head_quota is not None else Hkv) * pr * D * esize
        self.seed = seed
        self.seeds = {}   # sid -> synth seed
        self.P = {}       # sid -> prompt length
        self.G = {}       # sid -> generated tokens (all layers)
        self.nb = {}      # sid -> blocks compressed and freed

    # -- inputs ---------------------------------------------------------------
    def rows(self, sid, layer, kind, a, b, which, heads=None, scale=1.0):
        heads = heads or (self.Hq if which == synth.WHICH_Q else self.Hkv)
        return synth.rows(self.seeds[sid], layer, kind, a, b, which, heads, self.D, self.dtype, scale)

    def fetch(self, sid, layer):
        def f(kind, a, b, which):
            w = synth.WHICH_K if which == "k" else synth.WHICH_V
            out = np.empty((len(kind), self.Hkv, self.D))
            for kd in (PROMPT, TEXT, PAUSE):
                m = kind == kd
                if m.any():
                    out[m] = self.rows(sid, layer, kd, a[m], b[m], w)
            return out
        return f

    def view(self, sid, layer) -> LayerView:
        return LayerView(self.P[sid], self.C, self.pause[layer], self.quota[layer], self.compress)

    def views(self, sid, layer):
        """Per-KV-head views of a pool with per-head quotas."""
        return [LayerView(self.P[sid], self.C, self.pause[layer], q, self.compress)
                for q in self.head_quota[layer]]

    # -- histories through the ABI --------------------------------------------
    def new_seq(self, P, idx):
        sid = self.pool.seq_create(P)
        self.seeds[sid] = seq_seed(self.seed, idx)
        self.P[sid], self.G[sid], self.nb[sid] = P, 0, 0
        return sid

    def write_prompts(self, sid):
        P = self.P[sid]
        for l in range(self.L):
            if P:
                k = dev(self.rows(sid, l, PROMPT, np.arange(P), 0, synth.WHICH_K), self.dtype)
                v = dev(self.rows(sid, l, PROMPT, np.arange(P), 0, synth.WHICH_V), self.dtype)
            else:
                k = v = torch.empty(0, device="cuda", dtype=TORCH_DT[self.dtype])
            self.pool.write_prompt(sid, l, k, v)

    def pause_inputs(self, sids, layer):
        Kp = self.pause[layer]
        ks = np.arange(Kp)
        q = np.stack([self.rows(s, layer, PAUSE, np.full(Kp, self.nb[s]), ks, synth.WHICH_Q,
                                scale=self.pause_q_scale) for s in sids])
        k = np.stack([self.rows(s, layer, PAUSE, np.full(Kp, self.nb[s]), ks, synth.WHICH_K) for s in sids])
        v = np.stack([self.rows(s, layer, PAUSE, np.full(Kp, self.nb[s]), ks, synth.WHICH_V) for s in sids])
        return q, k, v

    def compress_layer(self, sids, layer):
        q, k, v = self.pause_inputs(sids, layer)
        Kp = self.pause[layer]
        out = torch.empty((len(sids), Kp, self.Hq, self.D), device="cuda", dtype=TORCH_DT[self.dtype])
        lse = torch.empty((len(sids), Kp, self.Hq), device="cuda", dtype=torch.float32)
        self.pool.compress_block(layer, sids, dev(q, self.dtype), dev(k, self.dtype), dev(v, self.dtype),
                                 out, lse)
        return out, lse

    def append_token(self, sids):
        for l in range(self.L):
            k = np.stack([self.rows(s, l, TEXT, [self.G[s]], 0, synth.WHICH_K)[0] for s in sids])
            v = np.stack([self.rows(s, l, TEXT, [self.G[s]], 0, synth.WHICH_V)[0] for s in sids])
            self.pool.append_kv(l, sids, dev(k, self.dtype), dev(v, self.dtype))
        for s in sids:
            self.G[s] += 1

    def grow(self, targets: dict):
        """Drive every sequence to targets[sid] generated tokens through the
        ABI, compressing and freeing each block once the next token needs it."""
        while True:
            active = [s for s, g in targets.items() if self.G[s] < g]
            if not active:
                break
            if self.compress:
                full = [s for s in active if self.G[s] > 0 and self.G[s] - self.nb[s] * self.C == self.C]
                if full:
                    for l in range(self.L):
                        self.compress_layer(full, l)
                    self.pool.free_block(full)
                    for s in full:
                        self.nb[s] += 1
            self.append_token(active)

    def fill(self, sid, G):
        self.pool.synth_fill(sid, G, self.seeds[sid])
        self.G[sid] = G
        self.nb[sid] = (G - 1) // self.C if (self.compress and G > 0) else 0

    # -- decode -------------------------------------------------------------------
    def decode_query(self, sid, layer, scale=1.0):
        return self.rows(sid, layer, TEXT, [self.G[sid] - 1], 0, synth.WHICH_Q, scale=scale)[0]

    def decode(self, sids, layer, q=None):
        if q is None:
            q = np.stack([self.decode_query(s, layer) for s in sids])
        out = torch.empty((len(sids), self.Hq, self.D), device="cuda", dtype=TORCH_DT[self.dtype])
        lse = torch.empty((len(sids), self.Hq), device="cuda", dtype=torch.float32)
        self.pool.decode_attention(layer, sids, dev(q, self.dtype), out, lse)
        torch.cuda.synchronize()
        return host(out), host(lse), q

    def step_fused(self, sids):
        """One token of every sequence through abk_append_decode at every layer;
        returns [(out, lse, q)] per layer."""
        res = []
        for l in range(self.L):
            k = np.stack([self.rows(s, l, TEXT, [self.G[s]], 0, synth.WHICH_K)[0] for s in sids])
            v = np.stack([self.rows(s, l, TEXT, [self.G[s]], 0, synth.WHICH_V)[0] for s in sids])
            q = np.stack([self.rows(s, l, TEXT, [self.G[s]], 0, synth.WHICH_Q)[0] for s in sids])
            out = torch.empty((len(sids), self.Hq, self.D), device="cuda", dtype=TORCH_DT[self.dtype])
            lse = torch.empty((len(sids), self.Hq), device="cuda", dtype=torch.float32)
            self.pool.append_decode(l, sids, dev(k, self.dtype), dev(v, self.dtype), dev(q, self.dtype),
                                    out, lse)
            torch.cuda.synchronize()
            res.append((host(out), host(lse), q))
        for s in sids:
            self.G[s] += 1
        return res

    def step_separate(self, sids):
        """The same step as step_fused through abk_append_kv + abk_decode_attention."""
        self.append_token(sids)
        return [self.decode(sids, l) for l in range(self.L)]

    def compress_and_free(self, sids):
        for l in range(self.L):
            self.compress_layer(sids, l)
        self.pool.free_block(sids)
        for s in sids:
            self.nb[s] += 1

    def oracle_decode(self, sid, layer, q):
        if self.head_quota is not None:
            out, lse, keys = oracle.decode_heads(self.views(sid, layer), self.G[sid], self.nb[sid], q,
                                                 self.fetch(sid, layer), ORC_DT[self.dtype], self.base)
            return out, lse, keys
        return oracle.decode(self.view(sid, layer), self.G[sid], self.nb[sid], q, self.fetch(sid, layer),
                             ORC_DT[self.dtype], self.base)

    def oracle_compress(self, sid, layer):
        """Oracle of compressing block nb[sid] (its open block, full)."""
        b = self.nb[sid]
        Kp = self.pause[layer]
        q = self.rows(sid, layer, PAUSE, np.full(Kp, b), np.arange(Kp), synth.WHICH_Q, scale=self.pause_q_scale)
        if self.head_quota is not None:
            return oracle.compress_heads(self.views(sid, layer), self.G[sid], b, b, q, self.fetch(sid, layer),
                                         ORC_DT[self.dtype], self.base)
        return oracle.compress(self.view(sid, layer), self.G[sid], b, b, q, self.fetch(sid, layer),
                               ORC_DT[self.dtype], self.base)

