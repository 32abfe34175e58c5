"""CPU tests of the C-ABI library: symbols, configuration checks, and the
host-only pool's bookkeeping against the oracle's independent page model
(page ids, positions and row counts bit-exact; errors leave state unchanged)."""
import ctypes
import os
import re

import pytest

import long_reasoning_kv_amd as abk
from oracle.pagemodel import PageModel, PoolError
from tests.conftest import ROOT


def _header_symbols():
    with open(os.path.join(ROOT, "include", "abk.h")) as f:
        txt = f.read()
    return sorted(set(re.findall(r"^\s*(?:abk_status|const char\s*\*)\s*(abk_\w+)\s*\(", txt, re.M)))


def test_library_exports_every_declared_symbol():
    L = abk.lib()
    declared = _header_symbols()
    assert len(declared) >= 15
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(abk.SYMBOLS) == declared


def _pool(**kw):
    base = dict(num_layers=3, num_q_heads=4, num_kv_heads=2, head_dim=16, block_tokens=8,
                num_pause=4, layer_quota=[4, 2, 1], page_rows=4, max_seqs=4,
                pool_bytes=0, max_position=4096, dtype="f32", host_only=True)
    base.update(kw)
    if base["pool_bytes"] == 0:
        page_bytes = base["num_kv_heads"] * base["page_rows"] * base["head_dim"] * 4
        base["pool_bytes"] = 2 * page_bytes * kw.pop("_pages", 300)
    base.pop("_pages", None)
    return abk.Pool(**base)


@pytest.mark.parametrize("bad", [
    dict(num_q_heads=6),                 # group 3
    dict(head_dim=24),                   # unsupported d
    dict(block_tokens=10),               # not a multiple of page_rows
    dict(num_pause=3),                   # not a power of two
    dict(layer_quota=[4, 8, 1]),         # quota above pause count
    dict(page_rows=128, block_tokens=128),
    dict(rope_base=-1.0),
    dict(max_seqs=0),
])
def test_config_errors(bad):
    with pytest.raises(abk.AbkError) as e:
        _pool(**bad)
    assert e.value.status == abk.INVALID_ARG


def _compare(pool, pm, sid):
    for l in range(pm.L):
        info = pool.seq_query(sid, l)
        pages, pos = pool.export_layout(sid, l)
        mp, mpos, _ = pm.layout(sid, l)
        assert pages == mp and pos == mpos, (sid, l)
        assert info["resident_rows"] == pm.resident_rows(sid, l)
        assert info["open_rows"] == pm.open_rows(sid, l)
        assert info["n_pages"] == len(mp)


def _both(pool, pm, fpool, fmodel):
    """Run the op on both; they must succeed together or fail with one status."""
    err = None
    try:
        r1 = fpool()
    except abk.AbkError as e:
        err = e.status
    try:
        r2 = fmodel()
    except PoolError as e:
        assert err == e.status, (err, e.status)
        return None
    assert err is None, err
    assert r1 == r2
    return r1


def _append_then_decode(pm, l, sids):
    pm.append(l, sids)
    return pm.check_decode(l, sids)


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("compress", [True, False])
def test_host_pool_matches_page_model(compress, fused):
    pool = _pool(compress=compress, _pages=160)
    pm = PageModel(num_pages=160, page_rows=4, num_layers=3, C=8, quotas=[4, 2, 1],
                   pauses=[4, 4, 4], max_seqs=4, compress=compress)
    sids = [_both(pool, pm, lambda P=P: pool.seq_create(P), lambda P=P: pm.seq_create(P))
            for P in (2, 5, 0)]
    for s in sids:
        for l in range(3):
            _both(pool, pm, lambda s=s, l=l: pool.write_prompt(s, l, None, None),
                  lambda s=s, l=l: pm.write_prompt(s, l))
    for t in range(30):
        for l in range(3):
            if fused:
                # abk_append_decode: the append's bookkeeping, then the decode's checks
                _both(pool, pm, lambda l=l: pool.append_decode(l, sids, None, None, None, None, None),
                      lambda l=l: _append_then_decode(pm, l, sids))
                continue
            _both(pool, pm, lambda l=l: pool.append_kv(l, sids, None, None),
                  lambda l=l: pm.append(l, sids))
            _both(pool, pm, lambda l=l: pool.decode_attention(l, sids, None, None, None),
                  lambda l=l: pm.check_decode(l, sids))
        if compress:
            done = [s for s in sids if pm.open_rows(s, 0) == 8]
            if done:
                # a free before every layer is compressed is refused by both
                _both(pool, pm, lambda: pool.free_block(done), lambda: pm.free_block(done))
                for l in range(3):
                    _both(pool, pm, lambda l=l: pool.compress_block(l, done, None, None, None, None, None),
                          lambda l=l: pm.compress(l, done))
                _both(pool, pm, lambda: pool.free_block(done), lambda: pm.free_block(done))
        for s in sids:
            _compare(pool, pm, s)
    st = pool.stats()
    assert st["pages_free"] == pm.pages_free()
    assert st["pages_used"] + st["pages_free"] == 160
    # release and reuse: lowest slot and lowest pages
    _both(pool, pm, lambda: pool.seq_release(sids[1]), lambda: pm.release(sids[1]))
    s3 = _both(pool, pm, lambda: pool.seq_create(9), lambda: pm.seq_create(9))
    assert s3 == sids[1]
    _compare(pool, pm, s3)
    pool.close()


def test_host_pool_exhaustion_and_protocol_errors_match():
    pool = _pool(_pages=14)
    pm = PageModel(num_pages=14, page_rows=4, num_layers=3, C=8, quotas=[4, 2, 1],
                   pauses=[4, 4, 4], max_seqs=4)
    s = _both(pool, pm, lambda: pool.seq_create(4), lambda: pm.seq_create(4))
    _both(pool, pm, lambda: pool.seq_create(30), lambda: pm.seq_create(30))  # out of pages
    _both(pool, pm, lambda: pool.append_kv(0, [s], None, None), lambda: pm.append(0, [s]))  # no prompt
    for l in range(3):
        _both(pool, pm, lambda l=l: pool.write_prompt(s, l, None, None), lambda l=l: pm.write_prompt(s, l))
    _both(pool, pm, lambda: pool.append_kv(0, [s, s], None, None), lambda: pm.append(0, [s, s]))
    _both(pool, pm, lambda: pool.append_kv(0, [3], None, None), lambda: pm.append(0, [3]))
    _both(pool, pm, lambda: pool.decode_attention(0, [s], None, None, None), lambda: pm.check_decode(0, [s]))
    for t in range(8):
        for l in range(3):
            _both(pool, pm, lambda l=l: pool.append_kv(l, [s], None, None), lambda l=l: pm.append(l, [s]))
    _compare(pool, pm, s)
    # block full: appending is refused until compressed and freed
    _both(pool, pm, lambda: pool.append_kv(0, [s], None, None), lambda: pm.append(0, [s]))
    for l in range(3):
        _both(pool, pm, lambda l=l: pool.compress_block(l, [s], None, None, None, None, None),
              lambda l=l: pm.compress(l, [s]))
    _both(pool, pm, lambda: pool.compress_block(0, [s], None, None, None, None, None),
          lambda: pm.compress(0, [s]))  # twice
    _both(pool, pm, lambda: pool.decode_attention(1, [s], None, None, None), lambda: pm.check_decode(1, [s]))
    _both(pool, pm, lambda: pool.free_block([s]), lambda: pm.free_block([s]))
    _compare(pool, pm, s)
    pool.close()


def test_host_pool_fill_matches_page_model():
    pool = _pool(_pages=400, max_seqs=8)
    pm = PageModel(num_pages=400, page_rows=4, num_layers=3, C=8, quotas=[4, 2, 1],
                   pauses=[4, 4, 4], max_seqs=8)
    for P, G in [(3, 1), (0, 8), (5, 9), (2, 29), (7, 40)]:
        s = _both(pool, pm, lambda P=P: pool.seq_create(P), lambda P=P: pm.seq_create(P))
        _both(pool, pm, lambda s=s, G=G: pool.synth_fill(s, G, 1), lambda s=s, G=G: pm.fill(s, G))
        _compare(pool, pm, s)
        _both(pool, pm, lambda s=s: pool.synth_fill(s, 3, 1), lambda s=s: pm.fill(s, 3))  # not fresh
    pool.close()


def test_null_and_range_arguments():
    pool = _pool()
    L = abk.lib()
    assert L.abk_seq_create(pool._h, 3, None) == abk.INVALID_ARG
    assert L.abk_seq_query(pool._h, 99, 0, ctypes.byref(abk.SeqInfo())) == abk.INVALID_ARG
    assert L.abk_append_kv(pool._h, 0, 1, None, None, None) == abk.INVALID_ARG
    assert L.abk_pool_destroy(None) == abk.OK
    assert L.abk_pool_stats(None, None, None, None) == abk.INVALID_ARG
    pool.close()


def test_blockmask_attention_argument_checks():
    """Checks before any launch: bad layer, negative or too long sequences,
    unsupported shapes; an empty sequence is a no-op."""
    pool = _pool()  # fp32, d = 16: no block-mask prefill kernel
    L = abk.lib()
    assert L.abk_blockmask_attention(pool._h, 5, 0, 8, None, None, None, None, None) == abk.INVALID_ARG
    assert L.abk_blockmask_attention(pool._h, 0, -1, 8, None, None, None, None, None) == abk.INVALID_ARG
    assert L.abk_blockmask_attention(pool._h, 0, 0, 5000, None, None, None, None, None) == abk.INVALID_ARG
    assert L.abk_blockmask_attention(pool._h, 0, 2, 8, None, None, None, None, None) == abk.UNSUPPORTED
    pool.close()
    bf = _pool(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128, page_rows=4,
               pool_bytes=2 * 2 * 4 * 128 * 2 * 40)
    assert L.abk_blockmask_attention(bf._h, 0, 0, 0, None, None, None, None, None) == abk.OK
    assert L.abk_blockmask_attention(bf._h, 0, 3, 17, None, None, None, None, None) == abk.OK  # host-only
    bf.close()


def test_prefill_prompt_checks_before_writing():
    L = abk.lib()
    pool = _pool()  # fp32: no prompt prefill kernel
    s = pool.seq_create(3)
    assert L.abk_prefill_prompt(pool._h, 7, 0, None, None, None, None, None) == abk.INVALID_ARG
    assert L.abk_prefill_prompt(pool._h, s, 9, None, None, None, None, None) == abk.INVALID_ARG
    assert L.abk_prefill_prompt(pool._h, s, 0, None, None, None, None, None) == abk.UNSUPPORTED
    # nothing was written: appending is still refused for want of a prompt
    with pytest.raises(abk.AbkError) as e:
        pool.append_kv(0, [s], None, None)
    assert e.value.status == abk.BAD_STATE
    pool.close()
    bf = _pool(dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128, page_rows=4,
               pool_bytes=2 * 2 * 4 * 128 * 2 * 40)
    s = bf.seq_create(3)
    bf.prefill_prompt(s, 0, None, None, None, None, None)  # host-only: bookkeeping only
    bf.append_kv(0, [s], None, None)                       # the prompt counts as written
    with pytest.raises(abk.AbkError) as e:
        bf.prefill_prompt(s, 0, None, None, None, None, None)
    assert e.value.status == abk.BAD_STATE                 # generation has started
    bf.close()
    # 32 KV heads (one pool layer per head): above the block-mask prefill's 16,
    # refused before the prompt is written
    wide = _pool(dtype="bf16", num_layers=1, num_q_heads=128, num_kv_heads=32, head_dim=128,
                 page_rows=4, layer_quota=[4], head_quota=[[4] * 32], pool_bytes=2 * 4 * 128 * 2 * 400)
    s = wide.seq_create(3)
    with pytest.raises(abk.AbkError) as e:
        wide.prefill_prompt(s, 0, None, None, None, None, None)
    assert e.value.status == abk.UNSUPPORTED
    with pytest.raises(abk.AbkError) as e:
        wide.append_kv(0, [s], None, None)
    assert e.value.status == abk.BAD_STATE                 # no prompt was written
    wide.close()


# ---- per-head quotas (figure captions, Fig. 7: a quota per (layer, KV head)) ----

HEAD_Q = [[4, 1], [2, 0], [1, 4]]  # [layer][KV head]


def test_per_head_host_pool_matches_page_model():
    # the pool keeps one row set per (layer, KV head): the page model with one
    # layer per pair, a model layer's heads handled together in each call
    hs = 2
    pool = _pool(head_quota=HEAD_Q, _pages=400)
    pm = PageModel(num_pages=400 * 2, page_rows=4, num_layers=3 * hs, C=8,
                   quotas=[q for row in HEAD_Q for q in row], pauses=[4] * 6, max_seqs=4)
    assert pool.stats()["pages_free"] == 800  # pages of one KV head: twice as many
    sids = [_both(pool, pm, lambda P=P: pool.seq_create(P), lambda P=P: pm.seq_create(P))
            for P in (2, 5, 0)]
    for s in sids:
        for l in range(3):
            _both(pool, pm, lambda s=s, l=l: pool.write_prompt(s, l, None, None),
                  lambda s=s, l=l: [pm.write_prompt(s, l * hs + j) for j in range(hs)] and None)
    for t in range(27):
        for l in range(3):
            _both(pool, pm, lambda l=l: pool.append_kv(l, sids, None, None),
                  lambda l=l: pm.append_heads(l, hs, sids))
            _both(pool, pm, lambda l=l: pool.decode_attention(l, sids, None, None, None),
                  lambda l=l: pm.check_decode_heads(l, hs, sids))
        done = [s for s in sids if pm.open_rows(s, 0) == 8]
        if done:
            _both(pool, pm, lambda: pool.free_block(done), lambda: pm.free_block(done))
            for l in range(3):
                _both(pool, pm, lambda l=l: pool.compress_block(l, done, None, None, None, None, None),
                      lambda l=l: pm.compress_heads(l, hs, done))
            _both(pool, pm, lambda: pool.free_block(done), lambda: pm.free_block(done))
        for s in sids:
            for lv in range(3 * hs):
                info = pool.seq_query(s, lv)
                assert info["resident_rows"] == pm.resident_rows(s, lv), (s, lv)
                pages, pos = pool.export_layout(s, lv)
                mp, mpos, _ = pm.layout(s, lv)
                assert pages == mp and pos == mpos, (s, lv)
    # every (layer, head) kept its own quota per finished block
    s = sids[0]
    for l in range(3):
        for h in range(hs):
            info = pool.seq_query(s, l * hs + h)
            assert info["resident_rows"] == 2 + info["blocks_done"] * HEAD_Q[l][h] + info["open_rows"]
    assert pool.stats()["pages_free"] == pm.pages_free()
    pool.close()


def test_per_head_config_and_call_checks():
    with pytest.raises(abk.AbkError) as e:
        _pool(head_quota=[[4, 8], [2, 0], [1, 4]])  # above the pause count
    assert e.value.status == 1
    with pytest.raises(ValueError):
        _pool(head_quota=[[4, 1], [2, 0]])  # not L x Hkv
    pool = _pool(head_quota=HEAD_Q)
    s = pool.seq_create(3)
    with pytest.raises(abk.AbkError) as e:
        pool.append_kv(3, [s], None, None)  # model layers are 0..2
    assert e.value.status == 1
    # the pool's (layer, head) pairs are 0..5 for inspection
    assert pool.seq_query(s, 5)["prompt_len"] == 3
    with pytest.raises(abk.AbkError):
        pool.seq_query(s, 6)
    with pytest.raises(abk.AbkError) as e:
        pool.blockmask_attention(3, 4, 8, None, None, None, None, None)  # model layers only
    assert e.value.status == 1
    with pytest.raises(abk.AbkError) as e:
        pool.blockmask_attention(0, 4, 8, None, None, None, None, None)  # f32, d = 16: no MFMA prefill
    assert e.value.status == 5
    pool.close()


# ---- separate page pools per budget level (AI Radio transcript) ----------------

def _drive(pool, pm, sids, steps, hs=1):
    for t in range(steps):
        for l in range(3):
            if hs == 1:
                _both(pool, pm, lambda l=l: pool.append_kv(l, sids, None, None), lambda l=l: pm.append(l, sids))
            else:
                _both(pool, pm, lambda l=l: pool.append_kv(l, sids, None, None),
                      lambda l=l: pm.append_heads(l, hs, sids))
        done = [s for s in sids if pm.open_rows(s, 0) == 8]
        if done:
            for l in range(3):
                if hs == 1:
                    _both(pool, pm, lambda l=l: pool.compress_block(l, done, None, None, None, None, None),
                          lambda l=l: pm.compress(l, done))
                else:
                    _both(pool, pm, lambda l=l: pool.compress_block(l, done, None, None, None, None, None),
                          lambda l=l: pm.compress_heads(l, hs, done))
            _both(pool, pm, lambda: pool.free_block(done), lambda: pm.free_block(done))


@pytest.mark.parametrize("per_head", [False, True])
def test_budget_pools_match_page_model(per_head):
    # one pool per distinct quota (levels ascending), each with its own page id
    # range; every (sequence, layer) allocates from its level only
    hs = 2 if per_head else 1
    quotas = [q for row in HEAD_Q for q in row] if per_head else [4, 2, 1]
    levels = sorted(set(quotas))
    budget = [12 + 2 * k for k in range(len(levels))]
    kw = dict(head_quota=HEAD_Q) if per_head else {}
    pool = _pool(budget_pool_pages=budget, _pages=400, **kw)
    pm = PageModel(num_pages=400 * hs, page_rows=4, num_layers=3 * hs, C=8, quotas=quotas,
                   pauses=[4] * (3 * hs), max_seqs=4, budget_pages=budget)
    st = pool.budget_stats()
    assert [x["quota"] for x in st] == levels
    assert [x["pages_free"] for x in st] == budget
    sids = [_both(pool, pm, lambda P=P: pool.seq_create(P), lambda P=P: pm.seq_create(P)) for P in (2, 5)]
    for s in sids:
        for l in range(3):
            _both(pool, pm, lambda s=s, l=l: pool.write_prompt(s, l, None, None),
                  lambda s=s, l=l: [pm.write_prompt(s, l * hs + j) for j in range(hs)] and None)
    # grow until some level runs out; both refuse the same call
    _drive(pool, pm, sids, 60, hs)
    for s in sids:
        for lv in range(3 * hs):
            pages, pos = pool.export_layout(s, lv)
            mp, mpos, _ = pm.layout(s, lv)
            assert pages == mp and pos == mpos, (s, lv)
            k = levels.index(quotas[lv])
            lo = sum(budget[:k])
            assert all(lo <= pg < lo + budget[k] for pg in pages), (s, lv)
    st = pool.budget_stats()
    assert [x["pages_free"] for x in st] == [pm.level_free(k) for k in range(len(levels))]
    assert any(x["pages_free"] < 4 for x in st)  # some level was driven to its end
    pool.close()


def test_budget_pool_config_checks():
    with pytest.raises(abk.AbkError) as e:
        _pool(budget_pool_pages=[10, 10, 10 ** 6])  # more pages than pool_bytes gives
    assert e.value.status == 1
    with pytest.raises(abk.AbkError) as e:
        _pool(budget_pool_pages=[10, -1, 10])
    assert e.value.status == 1
    pool = _pool()
    st = pool.budget_stats()
    assert len(st) == 1 and st[0]["quota"] == -1 and st[0]["pages_free"] == 300
    pool.close()
