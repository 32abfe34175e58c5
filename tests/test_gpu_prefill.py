"""GPU parity of the block-mask prefill (abk_blockmask_attention) against the
oracle: every token of a training-order sequence attending under the block
mask at one layer.

- Small shapes, every row: 64-token blocks with 16 pause tokens, per-layer
  quotas, ragged prompts, a trailing partial block, no prompt, and
  compression off (plain causal).
- The Fig. 9 shape (16K text tokens, C = 512, K = 256 pause tokens, quotas
  64 / 128 / 256), sampled rows of every kind across the sequence.

Bars as everywhere: out max-abs 2e-2, lse 1e-3.
"""
import numpy as np
import pytest
import torch

import long_reasoning_kv_amd as abk
import oracle
import synth
from oracle import LayerView
from tests.harness import dev, host

pytestmark = pytest.mark.gpu

HQ, HKV, D = 32, 8, 128


def _close(name, got, want, tol):
    err = float(np.abs(np.asarray(got) - np.asarray(want)).max())
    print(f"[parity] {name}: max-abs {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: max-abs {err} > {tol}"


def _pool(C, Kp, quotas, compress=True, max_position=4096, pr=16):
    return abk.Pool(num_layers=len(quotas), num_q_heads=HQ, num_kv_heads=HKV, head_dim=D,
                    block_tokens=C, num_pause=Kp, layer_quota=quotas, page_rows=pr, max_seqs=2,
                    pool_bytes=2 * HKV * pr * D * 2 * 64, max_position=max_position, dtype="bf16",
                    rope_base=1e6, compress=compress)


def _synth_inputs(L, G, layer, seed):
    """q/k/v of every training-order token from the seeded generator."""
    kind, a, b = oracle.training_tokens(L, G)
    rows = {w: np.empty((len(kind), HQ if w == synth.WHICH_Q else HKV, D))
            for w in (synth.WHICH_Q, synth.WHICH_K, synth.WHICH_V)}
    for kd in (oracle.PROMPT, oracle.TEXT, oracle.PAUSE):
        m = kind == kd
        if m.any():
            for w, arr in rows.items():
                arr[m] = synth.rows(seed, layer, kd, a[m], b[m], w, arr.shape[1], D, "bf16", 1.0)
    return kind, a, b, rows[synth.WHICH_Q], rows[synth.WHICH_K], rows[synth.WHICH_V]


def _fetcher(L, G, k, v):
    kind, a, b = oracle.training_tokens(L, G)
    idx = {(int(x), int(y), int(z)): i for i, (x, y, z) in enumerate(zip(kind, a, b))}

    def fetch(kk, ka, kb, which):
        src = k if which == "k" else v
        return src[[idx[(int(x), int(y), int(z))] for x, y, z in zip(kk, ka, kb)]]
    return fetch


@pytest.mark.parametrize("P,G,compress", [(37, 3 * 64 + 45, True), (0, 4 * 64, True),
                                          (64, 2 * 64, True), (5, 0, True), (29, 150, False)])
def test_blockmask_prefill_every_row(P, G, compress):
    C, Kp, quotas = 64, 16, [16, 8]
    pool = _pool(C, Kp, quotas, compress)
    for layer in range(2):
        L = LayerView(P, C, Kp, quotas[layer], compress)
        kind, a, b, q, k, v = _synth_inputs(L, G, layer, seed=11 + layer)
        T = len(kind)
        out = torch.empty((T, HQ, D), device="cuda", dtype=torch.bfloat16)
        lse = torch.empty((T, HQ), device="cuda", dtype=torch.float32)
        pool.blockmask_attention(layer, P, G, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.blockmask_prefill(L, G, q, _fetcher(L, G, k, v), oracle.BF16, 1e6)
        _close(f"prefill out P{P} G{G} c{int(compress)} L{layer} ({T} rows)", host(out), o_ref, 2e-2)
        _close(f"prefill lse P{P} G{G} c{int(compress)} L{layer}", host(lse), l_ref, 1e-3)
    pool.close()


@pytest.mark.parametrize("P,G", [(37, 3 * 64 + 45), (0, 4 * 64)])
def test_blockmask_prefill_peaky_queries(P, G):
    """Queries eight times larger (a power of two: the bf16 values stay exact):
    scores spread over about 11 log2 units, so running maxima move on later
    tiles too, not only on each column's first tile."""
    C, Kp, quotas = 64, 16, [16, 8]
    pool = _pool(C, Kp, quotas, True)
    for layer in range(2):
        L = LayerView(P, C, Kp, quotas[layer], True)
        kind, a, b, q, k, v = _synth_inputs(L, G, layer, seed=21 + layer)
        q = q * 8.0
        T = len(kind)
        out = torch.empty((T, HQ, D), device="cuda", dtype=torch.bfloat16)
        lse = torch.empty((T, HQ), device="cuda", dtype=torch.float32)
        pool.blockmask_attention(layer, P, G, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.blockmask_prefill(L, G, q, _fetcher(L, G, k, v), oracle.BF16, 1e6)
        _close(f"peaky prefill out P{P} G{G} L{layer} ({T} rows)", host(out), o_ref, 2e-2)
        _close(f"peaky prefill lse P{P} G{G} L{layer}", host(lse), l_ref, 1e-3)
    pool.close()


@pytest.mark.parametrize("C,Kp,quotas", [(512, 256, [64, 128, 256]), (256, 128, [32, 64, 128])])
def test_blockmask_prefill_fig9_shape_sampled(C, Kp, quotas):
    """16K text tokens after a 256-token prompt, three layers, at the bench's
    two block sizes (4:1 mean quota at each): C = 512, K = 256 and C = 256,
    K = 128, both T = 24,832 rows."""
    P, G = 256, 16384
    pool = _pool(C, Kp, quotas, max_position=P + G, pr=64)
    gen = torch.Generator().manual_seed(9)
    for layer in range(3):
        L = LayerView(P, C, Kp, quotas[layer])
        kind, a, b = oracle.training_tokens(L, G)
        T = len(kind)
        assert T == P + G + (G // C) * Kp
        q = torch.randn((T, HQ, D), generator=gen).to(torch.bfloat16)
        k = torch.randn((T, HKV, D), generator=gen).to(torch.bfloat16)
        v = torch.randn((T, HKV, D), generator=gen).to(torch.bfloat16)
        out = torch.empty((T, HQ, D), device="cuda", dtype=torch.bfloat16)
        lse = torch.empty((T, HQ), device="cuda", dtype=torch.float32)
        pool.blockmask_attention(layer, P, G, q.cuda(), k.cuda(), v.cuda(), out, lse)
        torch.cuda.synchronize()
        per, nb = C + Kp, G // C
        rows = [0, P - 1,                                                  # prompt
                P, P + C // 2 + 44, P + C - 1,                             # block 0 text
                P + C, P + C + Kp // 3, P + per - 1,                       # block 0 pause
                P + 15 * per + 17, P + 15 * per + C + Kp // 2 - 28,        # block 15
                P + (nb - 1) * per + C - 1, P + (nb - 1) * per + C, T - 1]  # last block
        qn, kn, vn = (x.float().numpy().astype(np.float64) for x in (q, k, v))
        o_ref, l_ref = oracle.blockmask_prefill(L, G, qn, _fetcher(L, G, kn, vn), oracle.BF16, 1e6,
                                                rows=rows)
        _close(f"fig9 prefill out C{C} L{layer} q{quotas[layer]}", host(out[rows]), o_ref, 2e-2)
        _close(f"fig9 prefill lse C{C} L{layer} q{quotas[layer]}", host(lse[rows]), l_ref, 1e-3)
        assert np.isfinite(host(out)).all() and np.isfinite(host(lse)).all()
    pool.close()


def test_prefill_prompt_writes_the_rows_and_attends():
    """abk_prefill_prompt: the prompt's causal attention against the oracle, the
    pool rows bit-equal to abk_write_prompt's, and a later decode over them
    against the oracle."""
    from tests.harness import Run
    C, Kp, quotas = 64, 16, [16, 8]
    runs = [Run(L=2, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=Kp, quota=quotas, pr=16, dtype="bf16", max_seqs=4,
                seed=21) for _ in range(2)]
    for P in (37, 1, 0):
        sids = [r.new_seq(P, P) for r in runs]
        for l in range(2):
            L = LayerView(P, C, Kp, quotas[l])
            # the harness regenerates prompt rows from the sequence's seed at each layer
            kind, a, b, q, k, v = _synth_inputs(L, 0, l, seed=runs[0].seeds[sids[0]])
            kd, vd = dev(k, "bf16"), dev(v, "bf16")
            out = torch.empty((P, HQ, D), device="cuda", dtype=torch.bfloat16)
            lse = torch.empty((P, HQ), device="cuda", dtype=torch.float32)
            runs[0].pool.prefill_prompt(sids[0], l, dev(q, "bf16"), kd, vd, out, lse)
            runs[1].pool.write_prompt(sids[1], l, kd, vd)
            torch.cuda.synchronize()
            if P:
                o_ref, l_ref = oracle.blockmask_prefill(L, 0, q, _fetcher(L, 0, k, v), oracle.BF16, 1e6)
                _close(f"prompt prefill out P{P} L{l}", host(out), o_ref, 2e-2)
                _close(f"prompt prefill lse P{P} L{l}", host(lse), l_ref, 1e-3)
                kk = [torch.empty((P, HKV, D), device="cuda", dtype=torch.bfloat16) for _ in range(4)]
                runs[0].pool.read_rows(sids[0], l, 0, P, kk[0], kk[1])
                runs[1].pool.read_rows(sids[1], l, 0, P, kk[2], kk[3])
                torch.cuda.synchronize()
                assert torch.equal(kk[0], kk[2]) and torch.equal(kk[1], kk[3])
        # a few tokens later the decode sees the prompt rows as written
        runs[0].G[sids[0]] = 0
        runs[0].grow({sids[0]: 5})
        for l in range(2):
            out, lse, q = runs[0].decode([sids[0]], l)
            o_ref, l_ref, _ = runs[0].oracle_decode(sids[0], l, q[0])
            _close(f"decode after prompt prefill P{P} L{l}", out[0], o_ref, 2e-2)
            _close(f"decode lse after prompt prefill P{P} L{l}", lse[0], l_ref, 1e-3)
    for r in runs:
        r.pool.close()


@pytest.mark.parametrize("P,G", [(37, 3 * 64 + 45), (0, 2 * 64)])
def test_blockmask_prefill_per_head_quotas(P, G):
    # a quota per (layer, KV head) (figure captions, Fig. 7): each KV head's
    # query heads see that head's own kept code rows of earlier blocks
    C, Kp = 64, 16
    hq = [[16, 0, 4, 8, 1, 16, 2, 8], [8, 8, 1, 2, 16, 0, 4, 16]]
    pool = abk.Pool(num_layers=2, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_tokens=C,
                    num_pause=Kp, layer_quota=[16, 16], page_rows=16, max_seqs=2,
                    pool_bytes=2 * 16 * D * 2 * 1024, max_position=4096, dtype="bf16", rope_base=1e6,
                    head_quota=hq)
    for layer in range(2):
        Ls = [LayerView(P, C, Kp, q) for q in hq[layer]]
        kind, a, b, q, k, v = _synth_inputs(Ls[0], G, layer, seed=21 + layer)
        T = len(kind)
        out = torch.empty((T, HQ, D), device="cuda", dtype=torch.bfloat16)
        lse = torch.empty((T, HQ), device="cuda", dtype=torch.float32)
        pool.blockmask_attention(layer, P, G, dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), out, lse)
        torch.cuda.synchronize()
        o_ref, l_ref = oracle.blockmask_prefill_heads(Ls, G, q, _fetcher(Ls[0], G, k, v), oracle.BF16, 1e6)
        _close(f"per-head prefill out P{P} G{G} L{layer} ({T} rows)", host(out), o_ref, 2e-2)
        _close(f"per-head prefill lse P{P} G{G} L{layer}", host(lse), l_ref, 1e-3)
    pool.close()
