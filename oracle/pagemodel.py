"""Independent model of the paged AbridgeKV cache -- TEST INFRASTRUCTURE ONLY.

Tracks, per (sequence, layer), which logical rows are resident and on which
pages, under the allocation policy the library promises. It exists to check
the library's page tables, positions and row counts bit for bit; it shares no
code with the library.

What it follows:
 - Fig. 1(a)/(b) captions of 2610.20641: rows of a block accumulate while it is
   open; when it completes its pause tokens write code rows and its raw rows
   are freed, so a sequence's cache rises through a block and falls at each
   compression.
 - The AI Radio transcript: the resident cache is the prompt, the code rows of
   finished blocks and the open block; each layer has a fixed budget and rows a
   layer does not keep are never allocated.

Policy (the library's contract, restated here independently):
 - One global pool of pages; a page holds ``page_rows`` rows of one
   (sequence, layer) for all KV heads. Allocation always takes the lowest free
   page id; sequence ids are the lowest free slot.
 - Per (sequence, layer) two page lists. Persistent: the prompt, then code rows
   in (block, k) order, packed across page boundaries (in full-KV mode the
   generated rows are packed here too). Open: the open block's raw rows, on
   pages of their own, so that freeing the block frees whole pages.
 - Batched calls validate everything first and change nothing on failure.
 - Allocation order inside a call: sequences in the order given; for creation
   and fills, layers in ascending order (persistent pages before open pages).
"""
from __future__ import annotations

import heapq

from . import PAUSE, PROMPT, TEXT, LayerView, position

OK, INVALID_ARG, OUT_OF_PAGES, BAD_STATE = 0, 1, 2, 3


class PoolError(Exception):
    def __init__(self, status: int, msg: str = ""):
        super().__init__(f"status {status}: {msg}")
        self.status = status


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


class _Layer:
    def __init__(self):
        self.G = 0                 # generated rows appended at this layer
        self.pers_ids = []         # identities (kind, a, b) of persistent rows
        self.pers_pages = []
        self.open_pages = []
        self.compressed = False    # current block compressed, not yet freed
        self.prompt_written = False


class _Seq:
    def __init__(self, P: int, L: int):
        self.P = P
        self.nb = 0                # blocks compressed and freed
        self.layers = [_Layer() for _ in range(L)]


class PageModel:
    def __init__(self, num_pages: int, page_rows: int, num_layers: int, C: int, quotas,
                 pauses=None, max_seqs: int = 64, compress: bool = True, budget_pages=None):
        self.num_pages = num_pages
        self.pr = page_rows
        self.L = num_layers
        self.C = C
        self.quota = list(quotas)
        self.Kp = list(pauses) if pauses is not None else [max(self.quota)] * num_layers
        self.max_seqs = max_seqs
        self.compress_on = compress
        # separate pools per budget level (the AI Radio transcript: one page
        # pool per budget level): level k = k-th smallest distinct quota, its
        # pages the k-th consecutive id range; otherwise one pool
        if budget_pages is None:
            self.level_quota = [-1]
            bounds = [0, num_pages]
            self.level_of = [0] * num_layers
        else:
            self.level_quota = sorted(set(self.quota))
            assert len(budget_pages) == len(self.level_quota) and sum(budget_pages) <= num_pages
            bounds = [0]
            for n in budget_pages:
                bounds.append(bounds[-1] + n)
            self.level_of = [self.level_quota.index(q) for q in self.quota]
        self._bounds = bounds
        self._free = [list(range(bounds[k], bounds[k + 1])) for k in range(len(bounds) - 1)]
        for h in self._free:
            heapq.heapify(h)
        self._slots = list(range(max_seqs))
        heapq.heapify(self._slots)
        self.seqs = {}

    # -- helpers --------------------------------------------------------------
    def view(self, sid: int, l: int) -> LayerView:
        return LayerView(self.seqs[sid].P, self.C, self.Kp[l], self.quota[l], self.compress_on)

    def _alloc(self, n: int, l: int):
        h = self._free[self.level_of[l]]
        return [heapq.heappop(h) for _ in range(n)]

    def _release(self, pages):
        for p in pages:
            k = max(i for i in range(len(self._free)) if self._bounds[i] <= p)
            heapq.heappush(self._free[k], p)

    def _need(self, need: dict):
        """need: layer -> pages; every budget level must hold its layers' sum."""
        per = {}
        for l, n in need.items():
            per[self.level_of[l]] = per.get(self.level_of[l], 0) + n
        for k, n in per.items():
            if n > len(self._free[k]):
                raise PoolError(OUT_OF_PAGES, f"need {n} pages in level {k}, {len(self._free[k])} free")

    def level_free(self, k: int) -> int:
        return len(self._free[k])

    def _check_ids(self, sids):
        if len(set(sids)) != len(sids):
            raise PoolError(INVALID_ARG, "duplicate sequence id")
        for s in sids:
            if s not in self.seqs:
                raise PoolError(INVALID_ARG, f"unknown sequence {s}")

    def _check_layer(self, l):
        if not 0 <= l < self.L:
            raise PoolError(INVALID_ARG, "bad layer")

    def open_rows(self, sid: int, l: int) -> int:
        s = self.seqs[sid]
        return s.layers[l].G - s.nb * self.C if self.compress_on else 0

    def pers_rows(self, sid: int, l: int) -> int:
        return len(self.seqs[sid].layers[l].pers_ids)

    def resident_rows(self, sid: int, l: int) -> int:
        return self.pers_rows(sid, l) + self.open_rows(sid, l)

    def pages_free(self) -> int:
        return sum(len(h) for h in self._free)

    # -- operations -----------------------------------------------------------
    def seq_create(self, P: int) -> int:
        if P < 0:
            raise PoolError(INVALID_ARG, "negative prompt")
        if not self._slots:
            raise PoolError(OUT_OF_PAGES, "no free sequence slot")
        self._need({l: _cdiv(P, self.pr) for l in range(self.L)})
        sid = heapq.heappop(self._slots)
        s = _Seq(P, self.L)
        for l, lay in enumerate(s.layers):
            lay.pers_pages = self._alloc(_cdiv(P, self.pr), l)
            lay.pers_ids = [(PROMPT, i, 0) for i in range(P)]
        self.seqs[sid] = s
        return sid

    def write_prompt(self, sid: int, l: int):
        self._check_ids([sid])
        self._check_layer(l)
        lay = self.seqs[sid].layers[l]
        if lay.G != 0:
            raise PoolError(BAD_STATE, "prompt rewritten after generation began")
        lay.prompt_written = True

    def append(self, l: int, sids):
        self._check_layer(l)
        self._check_ids(sids)
        need = 0
        for sid in sids:
            s = self.seqs[sid]
            lay = s.layers[l]
            if not lay.prompt_written:
                raise PoolError(BAD_STATE, "prompt not written")
            if lay.G != min(x.G for x in s.layers):
                raise PoolError(BAD_STATE, "layer ahead of the current token")
            if self.compress_on:
                op = self.open_rows(sid, l)
                if op >= self.C:
                    raise PoolError(BAD_STATE, "open block full: compress and free it first")
                need += op % self.pr == 0
            else:
                need += len(lay.pers_ids) % self.pr == 0
        self._need({l: need})
        for sid in sids:
            s = self.seqs[sid]
            lay = s.layers[l]
            if self.compress_on:
                if self.open_rows(sid, l) % self.pr == 0:
                    lay.open_pages += self._alloc(1, l)
            else:
                if len(lay.pers_ids) % self.pr == 0:
                    lay.pers_pages += self._alloc(1, l)
                lay.pers_ids.append((TEXT, lay.G, 0))
            lay.G += 1

    def check_decode(self, l: int, sids):
        self._check_layer(l)
        self._check_ids(sids)
        for sid in sids:
            s = self.seqs[sid]
            lay = s.layers[l]
            if not lay.prompt_written or lay.G == 0 or lay.G != max(x.G for x in s.layers):
                raise PoolError(BAD_STATE, "current token not appended at this layer")
            if lay.compressed:
                raise PoolError(BAD_STATE, "block compressed but not freed")

    def compress(self, l: int, sids):
        self._check_layer(l)
        self._check_ids(sids)
        if not self.compress_on:
            raise PoolError(BAD_STATE, "compression is off")
        need = 0
        q = self.quota[l]
        for sid in sids:
            lay = self.seqs[sid].layers[l]
            if self.open_rows(sid, l) != self.C or lay.compressed:
                raise PoolError(BAD_STATE, "block not complete or already compressed")
            r = len(lay.pers_ids)
            need += _cdiv(r + q, self.pr) - _cdiv(r, self.pr)
        self._need({l: need})
        for sid in sids:
            s = self.seqs[sid]
            lay = s.layers[l]
            r = len(lay.pers_ids)
            lay.pers_pages += self._alloc(_cdiv(r + q, self.pr) - _cdiv(r, self.pr), l)
            lay.pers_ids += [(PAUSE, s.nb, k) for k in range(q)]
            lay.compressed = True

    # -- per-head quotas: the layers of one model layer's KV heads together ----
    # With a quota per (layer, KV head) (figure captions, Fig. 7), the model's
    # layer l is this model's layers l*hs .. l*hs + hs - 1 (one per KV head).
    # A call checks every (sequence, head) first; then allocation runs
    # sequence by sequence, heads in ascending order within a sequence.
    def append_heads(self, l: int, hs: int, sids):
        lays = [l * hs + j for j in range(hs)]
        for lv in lays:
            self._check_layer(lv)
        self._check_ids(sids)
        need = {lv: 0 for lv in lays}
        for sid in sids:
            s = self.seqs[sid]
            g0 = min(x.G for x in s.layers)
            for lv in lays:
                lay = s.layers[lv]
                if not lay.prompt_written:
                    raise PoolError(BAD_STATE, "prompt not written")
                if lay.G != g0:
                    raise PoolError(BAD_STATE, "layer ahead of the current token")
                if self.compress_on:
                    op = self.open_rows(sid, lv)
                    if op >= self.C:
                        raise PoolError(BAD_STATE, "open block full: compress and free it first")
                    need[lv] += op % self.pr == 0
                else:
                    need[lv] += len(lay.pers_ids) % self.pr == 0
        self._need(need)
        for sid in sids:
            s = self.seqs[sid]
            for lv in lays:
                lay = s.layers[lv]
                if self.compress_on:
                    if self.open_rows(sid, lv) % self.pr == 0:
                        lay.open_pages += self._alloc(1, lv)
                else:
                    if len(lay.pers_ids) % self.pr == 0:
                        lay.pers_pages += self._alloc(1, lv)
                    lay.pers_ids.append((TEXT, lay.G, 0))
                lay.G += 1

    def check_decode_heads(self, l: int, hs: int, sids):
        for j in range(hs):
            self.check_decode(l * hs + j, sids)

    def compress_heads(self, l: int, hs: int, sids):
        lays = [l * hs + j for j in range(hs)]
        for lv in lays:
            self._check_layer(lv)
        self._check_ids(sids)
        if not self.compress_on:
            raise PoolError(BAD_STATE, "compression is off")
        need = {lv: 0 for lv in lays}
        for sid in sids:
            for lv in lays:
                lay = self.seqs[sid].layers[lv]
                if self.open_rows(sid, lv) != self.C or lay.compressed:
                    raise PoolError(BAD_STATE, "block not complete or already compressed")
                r = len(lay.pers_ids)
                need[lv] += _cdiv(r + self.quota[lv], self.pr) - _cdiv(r, self.pr)
        self._need(need)
        for sid in sids:
            s = self.seqs[sid]
            for lv in lays:
                lay = s.layers[lv]
                q = self.quota[lv]
                r = len(lay.pers_ids)
                lay.pers_pages += self._alloc(_cdiv(r + q, self.pr) - _cdiv(r, self.pr), lv)
                lay.pers_ids += [(PAUSE, s.nb, k) for k in range(q)]
                lay.compressed = True

    def free_block(self, sids):
        self._check_ids(sids)
        if not self.compress_on:
            raise PoolError(BAD_STATE, "compression is off")
        for sid in sids:
            if not all(x.compressed for x in self.seqs[sid].layers):
                raise PoolError(BAD_STATE, "not every layer compressed")
        for sid in sids:
            s = self.seqs[sid]
            for lay in s.layers:
                self._release(lay.open_pages)
                lay.open_pages = []
                lay.compressed = False
            s.nb += 1

    def release(self, sid: int):
        self._check_ids([sid])
        s = self.seqs.pop(sid)
        for lay in s.layers:
            self._release(lay.pers_pages)
            self._release(lay.open_pages)
        heapq.heappush(self._slots, sid)

    def fill(self, sid: int, G: int):
        """Bulk-build the state after G generated tokens (compressing every
        completed block except the one holding the last token)."""
        self._check_ids([sid])
        s = self.seqs[sid]
        if G < 0:
            raise PoolError(INVALID_ARG, "negative length")
        if any(x.G or x.prompt_written for x in s.layers):
            raise PoolError(BAD_STATE, "fill needs a fresh sequence")
        nb = (G - 1) // self.C if (self.compress_on and G > 0) else 0
        opn = G - nb * self.C if self.compress_on else 0
        plan = []
        for l in range(self.L):
            r0 = s.P
            r1 = s.P + (nb * self.quota[l] if self.compress_on else G)
            plan.append((_cdiv(r1, self.pr) - _cdiv(r0, self.pr), _cdiv(opn, self.pr)))
        self._need({l: a + b for l, (a, b) in enumerate(plan)})
        for l, lay in enumerate(s.layers):
            lay.pers_pages += self._alloc(plan[l][0], l)
            lay.open_pages += self._alloc(plan[l][1], l)
            if self.compress_on:
                lay.pers_ids += [(PAUSE, b, k) for b in range(nb) for k in range(self.quota[l])]
            else:
                lay.pers_ids += [(TEXT, j, 0) for j in range(G)]
            lay.G = G
            lay.prompt_written = True
        s.nb = nb

    # -- inspection -----------------------------------------------------------
    def snapshot(self):
        """Plain nested copy of the whole state (for equality checks)."""
        seqs = {sid: (s.P, s.nb, [(x.G, tuple(x.pers_ids), tuple(x.pers_pages),
                                   tuple(x.open_pages), x.compressed, x.prompt_written)
                                  for x in s.layers])
                for sid, s in self.seqs.items()}
        return sorted(p for h in self._free for p in h), sorted(self._slots), seqs

    def layout(self, sid: int, l: int):
        """(page ids: persistent then open, positions of resident rows,
        identities of resident rows)."""
        s = self.seqs[sid]
        lay = s.layers[l]
        v = self.view(sid, l)
        ids = list(lay.pers_ids)
        ids += [(TEXT, s.nb * self.C + i, 0) for i in range(self.open_rows(sid, l))]
        pos = [position(v, *t) for t in ids]
        return lay.pers_pages + lay.open_pages, pos, ids
