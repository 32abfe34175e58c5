"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (Fig. 2(b) positions), the textual mask rules drawn for the Fig.
2(a) case, closed forms of softmax attention, RoPE's defining identities, a
library SDPA in float64, and the resident-row count the pages state.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import PAUSE, PROMPT, TEXT, LayerView
from tests.conftest import golden_lines

RNG = np.random.default_rng(12345)


# ---- positions: Fig. 2(b) -----------------------------------------------------

def test_fig2b_positions_golden():
    for line in golden_lines("fig2b_positions.txt"):
        C, K, *offs = map(int, line.split())
        L = LayerView(P=0, C=C, Kp=K, quota=K)
        got = [oracle.position(L, PAUSE, 0, k) for k in range(K)]
        assert got == offs


def test_positions_inside_replaced_block():
    # pause k of block b lies inside [P + b*C, P + (b+1)*C)
    for K in (1, 2, 4, 8, 64, 256):
        L = LayerView(P=37, C=512, Kp=K, quota=K)
        for b in (0, 3):
            pos = [oracle.position(L, PAUSE, b, k) for k in range(K)]
            assert len(set(pos)) == K
            assert min(pos) == 37 + b * 512 and max(pos) < 37 + (b + 1) * 512


def test_bitrev_involution_and_prefix_property():
    for nbits in range(0, 9):
        K = 1 << nbits
        for k in range(K):
            assert oracle.bitrev(oracle.bitrev(k, nbits), nbits) == k
        # any prefix q (power of two) of the K pause tokens is evenly spread:
        # {bitrev_K(k) * C/K : k < q} == {j * C/q : j < q}
        C = 512
        L = LayerView(P=0, C=C, Kp=K, quota=K)
        q = 1
        while q <= K:
            got = sorted(oracle.position(L, PAUSE, 0, k) for k in range(q))
            assert got == [j * C // q for j in range(q)]
            # and equal to the positions a layer running only q pause tokens gets
            Lq = LayerView(P=0, C=C, Kp=q, quota=q)
            assert [oracle.position(Lq, PAUSE, 0, k) for k in range(q)] == \
                [oracle.position(L, PAUSE, 0, k) for k in range(q)]
            q *= 2


def test_text_and_prompt_positions():
    L = LayerView(P=5, C=8, Kp=4, quota=4)
    assert [oracle.position(L, PROMPT, i) for i in range(5)] == list(range(5))
    assert oracle.position(L, TEXT, 0) == 5
    assert oracle.position(L, TEXT, 20) == 25


# ---- the block mask: Fig. 2(a) ------------------------------------------------

def _fig2a_tokens(P, C, K, nblocks):
    toks = [(PROMPT, i, 0) for i in range(P)]
    for b in range(nblocks):
        toks += [(TEXT, b * C + i, 0) for i in range(C)]
        toks += [(PAUSE, b, k) for k in range(K)]
    return toks


def test_fig2a_mask_golden():
    lines = list(golden_lines("fig2a_mask.txt"))
    want = np.array([[int(x) for x in ln.split()[1:15]] for ln in lines])
    want_pos = [int(ln.split()[15]) for ln in lines]
    L = LayerView(P=2, C=4, Kp=2, quota=2)
    toks = _fig2a_tokens(2, 4, 2, 2)
    assert len(toks) == 14
    got = np.array([[int(oracle.visible(L, q, k)) for k in toks] for q in toks])
    np.testing.assert_array_equal(got, want)
    assert [oracle.position(L, *t) for t in toks] == want_pos
    # creation order is the training layout of the figure
    assert [oracle.creation_index(L, *t) for t in toks] == list(range(14))


def test_mask_quota_truncates_earlier_code_rows():
    # a layer keeping q < K rows sees only pause k < q of earlier blocks
    L = LayerView(P=2, C=4, Kp=2, quota=1)
    assert oracle.visible(L, (TEXT, 4, 0), (PAUSE, 0, 0))
    assert not oracle.visible(L, (TEXT, 4, 0), (PAUSE, 0, 1))
    # ...but all pause tokens of its own block still see each other causally
    assert oracle.visible(L, (PAUSE, 1, 1), (PAUSE, 1, 0))
    assert oracle.visible(L, (PAUSE, 1, 1), (PAUSE, 1, 1))
    assert not oracle.visible(L, (PAUSE, 1, 0), (PAUSE, 1, 1))


def test_mask_compression_off_is_causal():
    L = LayerView(P=3, C=4, Kp=2, quota=2, compress=False)
    toks = [(PROMPT, i, 0) for i in range(3)] + [(TEXT, j, 0) for j in range(13)]
    for qi, q in enumerate(toks):
        for ki, k in enumerate(toks):
            assert oracle.visible(L, q, k) == (ki <= qi)


@pytest.mark.parametrize("P,C,K,q", [(2, 4, 2, 2), (5, 8, 4, 2), (0, 8, 4, 4), (7, 16, 8, 1)])
def test_resident_rows_closed_form(P, C, K, q):
    # resident cache = prompt + q code rows per finished block + open rows
    L = LayerView(P=P, C=C, Kp=K, quota=q)
    for G in range(1, 6 * C):
        nb = (G - 1) // C
        kind, a, b, pos = oracle.visible_keys(L, G, nb, (TEXT, G - 1, 0))
        opn = G - nb * C
        assert len(kind) == P + nb * q + opn
        # and they are, in creation order: prompt, code rows (block, k), open rows
        want = [(PROMPT, i, 0) for i in range(P)]
        want += [(PAUSE, bb, k) for bb in range(nb) for k in range(q)]
        want += [(TEXT, nb * C + i, 0) for i in range(opn)]
        assert list(zip(kind.tolist(), a.tolist(), b.tolist())) == want


def test_pause_query_key_counts():
    # pause j of block b sees prompt + b*q retained rows + C block rows + j+1 pause rows
    P, C, K, q = 3, 8, 4, 2
    L = LayerView(P=P, C=C, Kp=K, quota=q)
    for b in range(4):
        G = (b + 1) * C
        for j in range(K):
            kind, *_ = oracle.visible_keys(L, G, b, (PAUSE, b, j))
            assert len(kind) == P + b * q + C + j + 1


# ---- RoPE ---------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = RNG.standard_normal((5, 3, 16))
    y = oracle.rope_rows(x, np.zeros(5, np.int64), 1e6)
    np.testing.assert_array_equal(x, y)


def test_rope_preserves_pair_norms_and_pairs_rotate_half():
    d = 16
    x = RNG.standard_normal((7, 2, d))
    pos = RNG.integers(0, 40000, 7)
    y = oracle.rope_rows(x, pos, 1e6)
    h = d // 2
    np.testing.assert_allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2,
                               rtol=1e-12)
    # a vector with a single nonzero at i only mixes into i + d/2
    e = np.zeros((1, 1, d))
    e[0, 0, 3] = 1.0
    ye = oracle.rope_rows(e, np.array([11]), 1e6)
    nz = set(np.nonzero(np.abs(ye[0, 0]) > 1e-15)[0].tolist())
    assert nz <= {3, 3 + h}


def test_rope_relative_position_property():
    # <RoPE(q, m), RoPE(k, n)> depends on m - n only
    d = 32
    q = RNG.standard_normal((1, 1, d))
    k = RNG.standard_normal((1, 1, d))
    ref = None
    for m, n in [(100, 40), (60, 0), (1060, 1000), (30060, 30000)]:
        qm = oracle.rope_rows(q, np.array([m]), 1e6)
        kn = oracle.rope_rows(k, np.array([n]), 1e6)
        dot = float((qm * kn).sum())
        if ref is None:
            ref = dot
        assert abs(dot - ref) < 1e-9


def test_rope_against_complex_rotation():
    # pair i rotated by angle pos * base^(-2i/d), written as multiplication by
    # exp(1j * angle) on the complex number x_i + 1j x_{i+d/2}
    d, base = 8, 1e6
    x = RNG.standard_normal((4, 1, d))
    pos = np.array([0, 1, 517, 32767])
    y = oracle.rope_rows(x, pos, base)
    h = d // 2
    ang = pos[:, None] * base ** (-np.arange(h) * 2.0 / d)[None, :]
    z = (x[:, 0, :h] + 1j * x[:, 0, h:]) * np.exp(1j * ang)
    np.testing.assert_allclose(y[:, 0, :h], z.real, atol=1e-12)
    np.testing.assert_allclose(y[:, 0, h:], z.imag, atol=1e-12)


# ---- storage rounding ---------------------------------------------------------

def test_round_bf16_against_torch_and_ties():
    x32 = RNG.standard_normal(20000).astype(np.float32).astype(np.float64)
    x32 = np.concatenate([x32, x32 * 1e-30, x32 * 1e30, x32 * 1e-39])
    x32 = x32.astype(np.float32).astype(np.float64)  # fp32-exact: torch rounds via float
    want = torch.from_numpy(x32).float().to(torch.bfloat16).double().numpy()
    got = oracle.round_storage(x32, oracle.BF16)
    np.testing.assert_array_equal(got, want)
    # ties go to even; the second rounding of an fp32 value is not needed
    assert oracle.lib().orc_round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle.lib().orc_round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert oracle.lib().orc_round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7


def test_round_f32_matches_numpy():
    x = RNG.standard_normal(1000) * 3
    np.testing.assert_array_equal(oracle.round_storage(x, oracle.F32),
                                  x.astype(np.float32).astype(np.float64))


# ---- attention closed forms -----------------------------------------------------

def test_attention_zero_query_is_mean():
    n, d = 37, 16
    k = RNG.standard_normal((n, 1, d))
    v = RNG.standard_normal((n, 1, d))
    out, lse = oracle.attention(np.zeros((2, d)), k, v)
    np.testing.assert_allclose(lse, math.log(n), rtol=1e-14)
    np.testing.assert_allclose(out, np.broadcast_to(v[:, 0].mean(0), (2, d)), atol=1e-14)


def test_attention_single_key_and_permutation():
    d = 16
    q = RNG.standard_normal((4, d))
    k1 = RNG.standard_normal((1, 2, d))
    v1 = RNG.standard_normal((1, 2, d))
    out, lse = oracle.attention(q, k1, v1)
    for h in range(4):
        np.testing.assert_allclose(out[h], v1[0, h // 2], atol=1e-15)
        assert abs(lse[h] - q[h] @ k1[0, h // 2] / math.sqrt(d)) < 1e-12
    n = 50
    k = RNG.standard_normal((n, 2, d))
    v = RNG.standard_normal((n, 2, d))
    perm = RNG.permutation(n)
    o1, l1 = oracle.attention(q, k, v)
    o2, l2 = oracle.attention(q, k[perm], v[perm])
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)


def test_attention_matches_torch_sdpa_gqa():
    Hq, Hkv, n, d = 8, 2, 300, 32
    q = RNG.standard_normal((Hq, d)) * 3
    k = RNG.standard_normal((n, Hkv, d))
    v = RNG.standard_normal((n, Hkv, d))
    out, lse = oracle.attention(q, k, v)
    tq = torch.from_numpy(q)[:, None, :]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0].numpy()
    np.testing.assert_allclose(out, ref, atol=1e-12)
    s = torch.einsum("hd,hnd->hn", torch.from_numpy(q), tk) / math.sqrt(d)
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), atol=1e-12)


# ---- composed decode: compression off equals causal SDPA ----------------------

def test_decode_compression_off_equals_causal_sdpa():
    P, C, Hq, Hkv, d, base = 3, 4, 4, 2, 16, 1e6
    Gmax = 11
    L = LayerView(P=P, C=C, Kp=2, quota=2, compress=False)
    kraw = RNG.standard_normal((P + Gmax, Hkv, d))
    vraw = RNG.standard_normal((P + Gmax, Hkv, d))
    qraw = RNG.standard_normal((P + Gmax, Hq, d))

    def fetch(kind, a, b, which):
        idx = np.where(kind == PROMPT, a, P + a)
        return (kraw if which == "k" else vraw)[idx]

    # the library SDPA over the whole sequence, causal, on rotated q and k
    pos = np.arange(P + Gmax)
    qr = oracle.rope_rows(qraw, pos, base)
    kr = oracle.rope_rows(kraw, pos, base)
    tq = torch.from_numpy(qr).permute(1, 0, 2)
    tk = torch.from_numpy(kr).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    tv = torch.from_numpy(vraw).permute(1, 0, 2).repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    for G in range(1, Gmax + 1):
        out, lse, keys = oracle.decode(L, G, 0, qraw[P + G - 1], fetch, dtype=-1, base=base)
        assert len(keys[0]) == P + G
        np.testing.assert_allclose(out, ref[:, P + G - 1].numpy(), atol=1e-12)


@pytest.mark.parametrize("q", [2, 4])
def test_decode_compressed_equals_attention_over_resident_rows(q):
    # with compression on, decode equals plain attention over exactly the rows
    # the pages say stay resident: prompt, q code rows per block, open block
    P, C, K, Hq, Hkv, d, base = 2, 8, 4, 2, 1, 16, 1e6
    L = LayerView(P=P, C=C, Kp=K, quota=q)
    G = 29
    nb = (G - 1) // C
    data = {}

    def row(t, which):
        key = (t, which)
        if key not in data:
            data[key] = RNG.standard_normal((Hkv, d))
        return data[key]

    def fetch(kind, a, b, which):
        return np.stack([row((int(x), int(y), int(z)), which) for x, y, z in zip(kind, a, b)])

    qraw = RNG.standard_normal((Hq, d))
    out, lse, keys = oracle.decode(L, G, nb, qraw, fetch, dtype=-1, base=base)
    res = [(PROMPT, i, 0) for i in range(P)]
    res += [(PAUSE, bb, k) for bb in range(nb) for k in range(q)]
    res += [(TEXT, j, 0) for j in range(nb * C, G)]
    kk = np.stack([row(t, "k") for t in res])
    vv = np.stack([row(t, "v") for t in res])
    pos = np.array([P + bb * C + [0, 4, 2, 6][k] for bb in range(nb) for k in range(q)])
    pos = np.concatenate([np.arange(P), pos, P + np.arange(nb * C, G)])
    kr = oracle.rope_rows(kk, pos, base)
    qr = oracle.rope_rows(qraw[None], np.array([P + G - 1]), base)[0]
    o2, l2 = oracle.attention(qr, kr, vv)
    np.testing.assert_allclose(out, o2, atol=1e-14)
    np.testing.assert_allclose(lse, l2, atol=1e-14)
    assert len(keys[0]) == len(res) == P + nb * q + (G - nb * C)
    if q == K:
        assert len(res) == 19  # the tiny case: 2 prompt + 3 blocks x 4 + 5 open


def test_quota_table_golden():
    rows = [tuple(map(int, ln.split())) for ln in golden_lines("quotas.txt")]
    table, (C, mean) = rows[:3], rows[3]
    assert sum(n for _, n in table) == 36
    total = sum(r * n for r, n in table)
    assert total == 36 * mean and C // mean == 4


def test_compress_query_subset_equals_full():
    """Sampling pause queries selects rows of the full computation unchanged."""
    Lv = LayerView(3, 8, 4, 2)
    G, nb = 24, 2
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 2, 16))

    def fetch(kind, a, b, which):
        # any deterministic rows keyed by identity
        key = kind * 100000 + a * 100 + b + (7 if which == "k" else 0)
        return np.sin(key[:, None, None] * 0.37 + np.arange(16)[None, None, :] * 0.11) * np.ones((1, 1, 16))

    full = oracle.compress(Lv, G, nb, nb, q, fetch, oracle.F32, 1e6)
    part = oracle.compress(Lv, G, nb, nb, q, fetch, oracle.F32, 1e6, queries=[3, 0])
    np.testing.assert_array_equal(part[0], full[0][[3, 0]])
    np.testing.assert_array_equal(part[1], full[1][[3, 0]])


# ---- block-mask prefill (training-forward attention) ---------------------------

def test_training_tokens_follow_creation_order():
    for comp in (True, False):
        L = LayerView(P=3, C=4, Kp=2, quota=1, compress=comp)
        kind, a, b = oracle.training_tokens(L, 10)
        idx = [oracle.creation_index(L, int(k), int(x), int(y)) for k, x, y in zip(kind, a, b)]
        assert idx == list(range(len(kind)))
        assert len(kind) == 3 + 10 + (2 * 2 if comp else 0)


def test_blockmask_prefill_fig2a_golden():
    """Zero queries weigh every visible key equally; one-hot values then make
    each output row the mask row of Fig. 2(a) divided by its count."""
    lines = list(golden_lines("fig2a_mask.txt"))
    want = np.array([[int(t) for t in ln.split()[1:15]] for ln in lines], np.float64)
    L = LayerView(P=2, C=4, Kp=2, quota=2)
    kind, a, b = oracle.training_tokens(L, 8)
    T = len(kind)
    assert T == 14
    rng = np.random.default_rng(0)

    def fetch(kk, ka, kb, which):
        if which == "k":
            return rng.standard_normal((len(kk), 1, 16))
        out = np.zeros((len(kk), 1, 16))
        for n, (x, y, z) in enumerate(zip(kk, ka, kb)):
            out[n, 0, oracle.creation_index(L, int(x), int(y), int(z))] = 1.0
        return out

    out, lse = oracle.blockmask_prefill(L, 8, np.zeros((T, 1, 16)), fetch, oracle.F32, 1e6)
    cnt = want.sum(1)
    np.testing.assert_allclose(out[:, 0, :14] * cnt[:, None], want, atol=1e-12)
    np.testing.assert_allclose(out[:, 0, 14:], 0.0)
    np.testing.assert_allclose(lse[:, 0], np.log(cnt), atol=1e-12)


def test_blockmask_prefill_compression_off_is_causal_sdpa():
    L = LayerView(P=5, C=8, Kp=4, quota=2, compress=False)
    G, Hq, Hkv, d = 19, 4, 2, 16
    T = L.P + G
    rng = np.random.default_rng(1)
    q = rng.standard_normal((T, Hq, d))
    k = rng.standard_normal((T, Hkv, d))
    v = rng.standard_normal((T, Hkv, d))
    kind, a, b = oracle.training_tokens(L, G)
    idx = {(int(x), int(y), int(z)): i for i, (x, y, z) in enumerate(zip(kind, a, b))}

    def fetch(kk, ka, kb, which):
        src = k if which == "k" else v
        return src[[idx[(int(x), int(y), int(z))] for x, y, z in zip(kk, ka, kb)]]

    out, lse = oracle.blockmask_prefill(L, G, q, fetch, oracle.F32, 1e6)
    pos = np.arange(T)
    qr = torch.from_numpy(oracle.rope_rows(q, pos, 1e6, oracle.F32)).transpose(0, 1)
    kr = torch.from_numpy(oracle.rope_rows(k, pos, 1e6, oracle.F32)).transpose(0, 1)
    vv = torch.from_numpy(v).transpose(0, 1)
    kr = kr.repeat_interleave(Hq // Hkv, 0)
    vv = vv.repeat_interleave(Hq // Hkv, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qr, kr, vv, is_causal=True)
    np.testing.assert_allclose(out, ref.transpose(0, 1).numpy(), atol=1e-10)


def test_blockmask_prefill_rows_equal_decode_and_compression():
    """A text row is the decode of that token right after it is written; a
    pause row is that pause token's query in the compression of its block."""
    L = LayerView(P=3, C=8, Kp=4, quota=2)
    G, Hq, Hkv, d = 21, 2, 1, 16
    kind, a, b = oracle.training_tokens(L, G)
    T = len(kind)
    rng = np.random.default_rng(2)
    q = rng.standard_normal((T, Hq, d))
    kv = {w: rng.standard_normal((T, Hkv, d)) for w in ("k", "v")}
    idx = {(int(x), int(y), int(z)): i for i, (x, y, z) in enumerate(zip(kind, a, b))}

    def fetch(kk, ka, kb, which):
        return kv[which][[idx[(int(x), int(y), int(z))] for x, y, z in zip(kk, ka, kb)]]

    out, lse = oracle.blockmask_prefill(L, G, q, fetch, oracle.BF16, 1e6)
    for r in range(T):
        if kind[r] == oracle.TEXT:
            g = int(a[r]) + 1
            o2, l2, _ = oracle.decode(L, g, (g - 1) // L.C, q[r], fetch, oracle.BF16, 1e6)
        elif kind[r] == oracle.PAUSE:
            blk = int(a[r])
            qb = q[[idx[(oracle.PAUSE, blk, j)] for j in range(L.Kp)]]
            o2, l2, _ = oracle.compress(L, (blk + 1) * L.C, blk, blk, qb, fetch, oracle.BF16, 1e6,
                                        queries=[int(b[r])])
            o2, l2 = o2[0], l2[0]
        else:
            continue
        np.testing.assert_allclose(out[r], o2, atol=1e-12)
        np.testing.assert_allclose(lse[r], l2, atol=1e-12)


# ---- per-head quotas (figure captions, Fig. 7: a quota per (layer, KV head)) ----

def _keyed_rows(Hkv, d, seed):
    data = {}
    rng = np.random.default_rng(seed)

    def row(t, which):
        key = (t, which)
        if key not in data:
            data[key] = rng.standard_normal((Hkv, d))
        return data[key]

    def fetch(kind, a, b, which):
        return np.stack([row((int(x), int(y), int(z)), which) for x, y, z in zip(kind, a, b)])

    return row, fetch


@pytest.mark.parametrize("quotas", [(4, 1), (2, 0), (4, 4)])
def test_decode_per_head_equals_attention_over_each_heads_rows(quotas):
    # KV head h keeps the pause prefix k < quotas[h] of every finished block;
    # its two query heads attend over exactly the prompt, those code rows and
    # the open block, and see no other KV head
    P, C, K, g, d, base = 3, 8, 4, 2, 16, 1e6
    Hkv = len(quotas)
    G = 29
    nb = (G - 1) // C
    row, fetch = _keyed_rows(Hkv, d, 11)
    qraw = RNG.standard_normal((g * Hkv, d))
    Ls = [LayerView(P=P, C=C, Kp=K, quota=q) for q in quotas]
    out, lse, keys = oracle.decode_heads(Ls, G, nb, qraw, fetch, dtype=-1, base=base)
    for h, q in enumerate(quotas):
        res = [(PROMPT, i, 0) for i in range(P)]
        res += [(PAUSE, bb, k) for bb in range(nb) for k in range(q)]
        res += [(TEXT, j, 0) for j in range(nb * C, G)]
        kk = np.stack([row(t, "k")[h:h + 1] for t in res])
        vv = np.stack([row(t, "v")[h:h + 1] for t in res])
        pos = np.array([P + bb * C + [0, 4, 2, 6][k] for bb in range(nb) for k in range(q)], dtype=np.int64)
        pos = np.concatenate([np.arange(P), pos, P + np.arange(nb * C, G)])
        kr = oracle.rope_rows(kk, pos, base)
        qr = oracle.rope_rows(qraw[None, h * g:(h + 1) * g], np.array([P + G - 1]), base)[0]
        o2, l2 = oracle.attention(qr, kr, vv)
        np.testing.assert_allclose(out[h * g:(h + 1) * g], o2, atol=1e-14)
        np.testing.assert_allclose(lse[h * g:(h + 1) * g], l2, atol=1e-14)
        assert len(keys[h][0]) == P + nb * q + (G - nb * C)


def test_per_head_with_equal_quotas_equals_per_layer():
    # one quota for every head is the per-layer case: decode and compression
    # of all heads at once (the attention routine's GQA path) give the same
    P, C, K, q, g, Hkv, d = 5, 8, 4, 2, 2, 3, 16
    G = 24
    nb = 2
    _, fetch = _keyed_rows(Hkv, d, 12)
    L = LayerView(P=P, C=C, Kp=K, quota=q)
    qd = RNG.standard_normal((g * Hkv, d))
    o1, l1, _ = oracle.decode(L, G + 1, nb, qd, fetch, oracle.F32, 1e6)
    o2, l2, _ = oracle.decode_heads([L] * Hkv, G + 1, nb, qd, fetch, oracle.F32, 1e6)
    np.testing.assert_allclose(o2, o1, atol=1e-14)
    np.testing.assert_allclose(l2, l1, atol=1e-14)
    qc = RNG.standard_normal((K, g * Hkv, d))
    c1 = oracle.compress(L, G, nb, nb, qc, fetch, oracle.F32, 1e6)
    c2 = oracle.compress_heads([L] * Hkv, G, nb, nb, qc, fetch, oracle.F32, 1e6)
    np.testing.assert_allclose(c2[0], c1[0], atol=1e-14)
    np.testing.assert_allclose(c2[1], c1[1], atol=1e-14)
    for h in range(Hkv):
        np.testing.assert_array_equal(c2[2][h][5], c1[2][5][:, h:h + 1])
        np.testing.assert_array_equal(c2[2][h][4], c1[2][4][:, h:h + 1])
