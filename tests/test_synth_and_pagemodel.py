"""CPU checks of the input generator and of the oracle's page model."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import PAUSE, PROMPT, TEXT
from oracle.pagemodel import BAD_STATE, INVALID_ARG, OUT_OF_PAGES, PageModel, PoolError
from tests.conftest import golden_lines


# ---- synth --------------------------------------------------------------------

def test_splitmix64_reference_vectors():
    for line in golden_lines("splitmix64.txt"):
        seed, *outs = map(int, line.split())
        got = [int(x) for x in synth.splitmix64_stream(seed, len(outs))]
        assert got == outs


def test_normals_are_standard_normal():
    z = synth.normals_from_keys(synth.row_keys(7, 0, synth.TEXT, np.arange(4000), 0, 0, 0), 128)
    z = z.ravel()
    assert abs(z.mean()) < 0.01 and abs(z.var() - 1) < 0.01
    # fourth moment of N(0,1) is 3
    assert abs((z ** 4).mean() - 3) < 0.05


def test_rows_are_keyed_by_identity():
    a = synth.rows(1, 0, synth.TEXT, [5, 6], 0, synth.WHICH_K, 2, 16, "bf16")
    b = synth.rows(1, 0, synth.TEXT, [6], 0, synth.WHICH_K, 2, 16, "bf16")
    np.testing.assert_array_equal(a[1], b[0])
    c = synth.rows(1, 0, synth.TEXT, [6], 0, synth.WHICH_V, 2, 16, "bf16")
    assert not np.array_equal(b, c)
    d = synth.rows(2, 0, synth.TEXT, [6], 0, synth.WHICH_K, 2, 16, "bf16")
    assert not np.array_equal(b, d)


@pytest.mark.parametrize("dtype,scale", [("bf16", 1.0), ("f32", 1.0), ("bf16", 8.0)])
def test_c_and_numpy_generators_agree(dtype, scale):
    a = np.arange(3000) * 7 + 1
    for kind, which, heads in [(synth.TEXT, synth.WHICH_K, 8), (synth.PAUSE, synth.WHICH_Q, 32)]:
        x = synth.rows(99, 5, kind, a, 3, which, heads, 128, dtype, scale)
        y = synth.rows_numpy(99, 5, kind, a, 3, which, heads, 128, dtype, scale)
        mism = np.count_nonzero(x != y)
        # libm may differ by an ulp in rare cases; after storage rounding that
        # almost never shows
        assert mism <= 2, mism


def test_bf16_storage_matches_torch():
    x = np.random.default_rng(0).standard_normal(10000)
    got = synth.to_storage(x, "bf16")
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(got, want)


# ---- page model -----------------------------------------------------------------

def _decode_ready(pm, sid):
    return all(pm.seqs[sid].layers[l].G == pm.seqs[sid].layers[0].G for l in range(pm.L))


def _check_layout_against_mask(pm, sid):
    """The page model's resident rows must equal the keys the mask shows a
    decode query (two independent derivations of the same set)."""
    s = pm.seqs[sid]
    for l in range(pm.L):
        G = s.layers[l].G
        if G == 0 or s.layers[l].compressed or (pm.compress_on and pm.open_rows(sid, l) == 0):
            continue  # no current query: between a free and the next append
        pages, pos, ids = pm.layout(sid, l)
        kind, a, b, kpos = oracle.visible_keys(pm.view(sid, l), G, s.nb, (TEXT, G - 1, 0))
        assert ids == list(zip(kind.tolist(), a.tolist(), b.tolist()))
        assert pos == kpos.tolist()
        npers = len(s.layers[l].pers_ids)
        assert len(s.layers[l].pers_pages) == -(-npers // pm.pr)
        assert len(s.layers[l].open_pages) == -(-pm.open_rows(sid, l) // pm.pr)
        q = pm.quota[l]
        if pm.compress_on:
            assert len(ids) == s.P + s.nb * q + (G - s.nb * pm.C)


def _step(pm, sids):
    """One generated token for every sequence; compress+free completed blocks."""
    for l in range(pm.L):
        pm.append(l, sids)
        pm.check_decode(l, sids)
    if pm.compress_on:
        done = [s for s in sids if pm.open_rows(s, 0) == pm.C]
        if done:
            for l in range(pm.L):
                pm.compress(l, done)
            pm.free_block(done)


@pytest.mark.parametrize("compress", [True, False])
def test_pagemodel_history_matches_mask(compress):
    pm = PageModel(num_pages=400, page_rows=4, num_layers=3, C=8, quotas=[4, 2, 1],
                   pauses=[4, 4, 4], max_seqs=4, compress=compress)
    sids = [pm.seq_create(P) for P in (2, 5, 0)]
    assert sids == [0, 1, 2]
    for s in sids:
        for l in range(3):
            pm.write_prompt(s, l)
    for t in range(41):
        _step(pm, sids)
        for s in sids:
            _check_layout_against_mask(pm, s)
    used = sum(len(x.pers_pages) + len(x.open_pages) for s in sids for x in pm.seqs[s].layers)
    assert used + pm.pages_free() == 400


def test_pagemodel_fill_equals_history_rows():
    kw = dict(num_pages=400, page_rows=4, num_layers=2, C=8, quotas=[4, 2], pauses=[4, 4])
    for G in (1, 7, 8, 9, 16, 17, 30):
        a = PageModel(**kw)
        s = a.seq_create(3)
        for l in range(2):
            a.write_prompt(s, l)
        for _ in range(G):
            _step(a, [s])
        # a history that just completed a block has compressed and freed it in
        # _step; fill keeps the last token's block open, so compare before that
        b = PageModel(**kw)
        t = b.seq_create(3)
        b.fill(t, G)
        if G % 8 == 0:
            continue
        for l in range(2):
            assert a.layout(s, l)[1:] == b.layout(t, l)[1:]


def test_pagemodel_lowest_free_page_and_slot():
    pm = PageModel(num_pages=64, page_rows=4, num_layers=1, C=8, quotas=[2], pauses=[2])
    s0 = pm.seq_create(4)      # page 0
    s1 = pm.seq_create(4)      # page 1
    assert pm.layout(s0, 0)[0] == [0] and pm.layout(s1, 0)[0] == [1]
    pm.release(s0)
    s2 = pm.seq_create(8)      # reuses slot 0 and pages 0, 2
    assert s2 == 0 and pm.layout(s2, 0)[0] == [0, 2]


def test_pagemodel_errors_leave_state_unchanged():
    pm = PageModel(num_pages=6, page_rows=4, num_layers=2, C=8, quotas=[2, 2], pauses=[2, 2])
    s = pm.seq_create(4)       # pages 0 (layer 0), 1 (layer 1)
    for l in range(2):
        pm.write_prompt(s, l)
    snap = pm.snapshot()
    with pytest.raises(PoolError) as e:
        pm.seq_create(13)      # needs 2 layers x 4 pages
    assert e.value.status == OUT_OF_PAGES and pm.snapshot() == snap
    with pytest.raises(PoolError) as e:
        pm.compress(0, [s])    # block not complete
    assert e.value.status == BAD_STATE and pm.snapshot() == snap
    with pytest.raises(PoolError) as e:
        pm.append(0, [s, s])
    assert e.value.status == INVALID_ARG and pm.snapshot() == snap
    with pytest.raises(PoolError) as e:
        pm.check_decode(0, [s])  # nothing appended yet
    assert e.value.status == BAD_STATE
    pm.append(0, [s])
    with pytest.raises(PoolError) as e:
        pm.append(0, [s])      # layer 0 is ahead of layer 1
    assert e.value.status == BAD_STATE
    with pytest.raises(PoolError) as e:
        pm.check_decode(1, [s])
    assert e.value.status == BAD_STATE
    with pytest.raises(PoolError) as e:
        pm.free_block([s])
    assert e.value.status == BAD_STATE
