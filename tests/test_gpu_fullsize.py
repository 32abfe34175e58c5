"""GPU parity at the benchmark's full sizes, in the launch configuration that
bench.py times (bf16, d = 128, 32 q / 8 KV heads, 64-row pages, C = 512, the
automatic decode schedule), on outputs the oracle computes one by one.

- The 36-layer per-layer-quota decode step: 22 sequences, prompts U[128, 512],
  U[4096, 32768] generated tokens, quotas 6x256 / 12x64 / 18x128 (seeded).
- The block-compression event: 64 sequences completing a block at once, all
  36 layers, K = 256 pause tokens; and one or two sequences alone (the
  context-split schedule).
- The serving mix's shape: more sequences than one launch takes, fused calls,
  blocks completing between steps; AbridgeKV and full-KV modes; and the mix at
  its benchmarked size (the 200 GiB pool of bench.py's admitted sequences).

Bars as everywhere: out max-abs 2e-2, lse 1e-3; stored values and rotated keys
bit-exact (both sides round the same fp64 rotation once); row counts and
positions bit-exact.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from oracle import PAUSE, TEXT
from tests.harness import Run, host

pytestmark = pytest.mark.gpu

L, HQ, HKV, D, C, PR, KP = 36, 32, 8, 128, 512, 64, 256


def _close(name, got, want, tol):
    err = float(np.abs(np.asarray(got) - np.asarray(want)).max())
    print(f"[parity] {name}: max-abs {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: max-abs {err} > {tol}"


def _pool_bytes(P, Gmax, quotas, compressed_blocks=None):
    page_bytes = HKV * PR * D * 2
    pages = 0
    for q in quotas:
        nb = (Gmax - 1) // C if compressed_blocks is None else compressed_blocks
        R = P + nb * q + C
        pages += int(np.sum(np.ceil(R / PR) + 2 + C // PR))
    return 2 * page_bytes * pages


def _sample_layers(quotas):
    """Two layers of each quota class."""
    out = []
    for q in (64, 128, 256):
        out += [int(l) for l in np.where(quotas == q)[0][:2]]
    return out


@pytest.mark.parametrize("fused", [False, True])
def test_36_layer_quota_decode_step_sampled(fused):
    quotas, P, G = bench.decode_workload(2)
    B = len(P)
    run = Run(L=L, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=int(quotas.max()), quota=quotas.tolist(), pr=PR,
              dtype="bf16", max_seqs=B, pool_bytes=_pool_bytes(P, G + 1, quotas),
              max_position=33792, seed=2)
    sids = [run.new_seq(int(P[i]), i) for i in range(B)]
    for s, g in zip(sids, G):
        run.fill(s, int(g))
    layers = _sample_layers(quotas)
    seqs = (0, 11, 21)
    if fused:
        # the step through abk_append_decode, as bench.py runs it (a full open
        # block is compressed and freed first)
        full = [s for s in sids if run.G[s] - run.nb[s] * C == C]
        if full:
            run.compress_and_free(full)
        results = run.step_fused(sids)
    else:
        run.grow({s: int(g) + 1 for s, g in zip(sids, G)})
        results = None
    print(f"[fullsize] 36-layer step: {B} sequences filled and appended (fused={fused})", flush=True)
    for l in range(L):
        out, lse, q = results[l] if fused else run.decode(sids, l)
        assert np.isfinite(out).all() and np.isfinite(lse).all(), l
        for i, s in enumerate(sids):
            nb = run.nb[s]
            want = int(P[i]) + nb * int(quotas[l]) + (run.G[s] - nb * C)
            assert run.pool.seq_query(s, l)["resident_rows"] == want, (i, l)
        if l in layers:
            for i in seqs:
                o_ref, l_ref, keys = run.oracle_decode(sids[i], l, q[i])
                _close(f"36L decode out seq{i} L{l} q{quotas[l]}", out[i], o_ref, 2e-2)
                _close(f"36L decode lse seq{i} L{l} q{quotas[l]}", lse[i], l_ref, 1e-3)
    # positions of one sampled (sequence, layer), bit-exact
    s, l = sids[11], layers[-1]
    pos = run.pool.export_layout(s, l)[1]
    want = oracle.visible_keys(run.view(s, l), run.G[s], run.nb[s], (TEXT, run.G[s] - 1, 0))[3]
    assert pos == want.tolist()


def test_block_compression_event_sampled():
    rng = np.random.default_rng(3)
    quotas = bench.layer_quotas(2)
    B = 64
    P = rng.integers(128, 512, B, endpoint=True)
    b = rng.integers(0, 62, B, endpoint=True)
    G = (b + 1) * C
    run = Run(L=L, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=KP, quota=quotas.tolist(), pr=PR, dtype="bf16",
              max_seqs=B, pool_bytes=_pool_bytes(P, G, quotas, compressed_blocks=b + 1),
              max_position=33792, seed=3)
    sids = [run.new_seq(int(P[i]), i) for i in range(B)]
    for s, g in zip(sids, G):
        run.fill(s, int(g))
    print("[fullsize] compression event: 64 sequences filled", flush=True)
    layers = _sample_layers(quotas)
    seqs = (0, 31, 63)
    queries = [0, 1, 100, 150, 255]  # every 64-pause query tile
    kept = {}
    before = {(i, l): run.pool.seq_query(sids[i], l)["resident_rows"] for i in seqs for l in layers}
    for l in range(L):
        out, lse = run.compress_layer(sids, l)
        if l in layers:
            kept[l] = (host(out[list(seqs)][:, queries]), host(lse[list(seqs)][:, queries]))
    torch.cuda.synchronize()
    for l in layers:
        q_l = int(quotas[l])
        for n, i in enumerate(seqs):
            s = sids[i]
            qraw = run.rows(s, l, PAUSE, np.full(KP, b[i]), np.arange(KP), synth.WHICH_Q)
            o_ref, l_ref, code = oracle.compress(run.view(s, l), run.G[s], run.nb[s], run.nb[s], qraw,
                                                 run.fetch(s, l), oracle.BF16, run.base, queries=queries)
            _close(f"event out seq{i} L{l} q{q_l}", kept[l][0][n], o_ref, 2e-2)
            _close(f"event lse seq{i} L{l} q{q_l}", kept[l][1][n], l_ref, 1e-3)
            # the layer's new code rows: values and rotated keys bit-exact
            rows = run.pool.seq_query(s, l)["resident_rows"]
            assert rows == before[(i, l)] + q_l
            r0 = rows - C - q_l
            k = torch.empty((q_l, HKV, D), device="cuda", dtype=torch.bfloat16)
            v = torch.empty_like(k)
            run.pool.read_rows(s, l, r0, q_l, k, v)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(v), code[5])
            np.testing.assert_array_equal(host(k), code[4])
            pos = run.pool.export_layout(s, l)[1]
            assert pos[r0:r0 + q_l] == code[3].tolist()
    run.pool.free_block(sids)
    for i, s in enumerate(sids):
        for l in (0, L - 1):
            assert run.pool.seq_query(s, l)["resident_rows"] == int(P[i]) + (int(b[i]) + 1) * int(quotas[l])


def test_compression_of_few_sequences_splits_the_context():
    """One or two sequences completing a block: the context of each query tile
    is split over several workgroups and merged; same bars as above."""
    quotas = [256, 64]
    for Ps, bs in (([300], [20]), ([130, 500], [3, 41])):
        run = Run(L=2, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=KP, quota=quotas, pr=PR, dtype="bf16",
                  max_seqs=4, pool_bytes=1 << 30, max_position=33792, seed=5)
        sids = [run.new_seq(P, i) for i, P in enumerate(Ps)]
        for s, b in zip(sids, bs):
            run.fill(s, (b + 1) * C)
        queries = [0, 5, 128, 255]
        for l in range(2):
            out, lse = run.compress_layer(sids, l)
            out, lse = host(out), host(lse)
            for n, s in enumerate(sids):
                b = run.nb[s]
                qraw = run.rows(s, l, PAUSE, np.full(KP, b), np.arange(KP), synth.WHICH_Q)
                o_ref, l_ref, code = oracle.compress(run.view(s, l), run.G[s], b, b, qraw, run.fetch(s, l),
                                                     oracle.BF16, run.base, queries=queries)
                _close(f"split compress out P{Ps[n]} b{b} L{l}", out[n][queries], o_ref, 2e-2)
                _close(f"split compress lse P{Ps[n]} b{b} L{l}", lse[n][queries], l_ref, 1e-3)
                q_l = quotas[l]
                r0 = run.pool.seq_query(s, l)["resident_rows"] - C - q_l
                k = torch.empty((q_l, HKV, D), device="cuda", dtype=torch.bfloat16)
                v = torch.empty_like(k)
                run.pool.read_rows(s, l, r0, q_l, k, v)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(host(v), code[5])
                np.testing.assert_array_equal(host(k), code[4])
        run.pool.close()


@pytest.mark.parametrize("compress", [True, False])
def test_serving_mix_more_sequences_than_one_launch(compress):
    """The serving mix's shape at a size the oracle checks: 300 sequences (two
    launches per call, split at 256) of one fused append + decode call per layer
    per step, with blocks completing between the steps (compressed at every
    layer and freed, as in serving). Sampled sequences on both sides of the
    launch split against the oracle; row counts of every sequence exact."""
    rng = np.random.default_rng(4)
    B, steps = 300, 3
    quotas = [256, 64]
    P = rng.integers(128, 512, B, endpoint=True)
    G = rng.integers(1024, 4096, B, endpoint=True)
    # a few sequences reach a block boundary during the steps
    G[::23] = (G[::23] // C) * C + C - rng.integers(0, steps, len(G[::23]))
    if compress:
        pool_bytes = _pool_bytes(P, G + steps + 1, np.array(quotas))
    else:
        pool_bytes = 2 * HKV * PR * D * 2 * 2 * int(np.sum(np.ceil((P + G + steps) / PR) + 1))
    run = Run(L=2, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=KP, quota=quotas, pr=PR, dtype="bf16",
              compress=compress, max_seqs=B, pool_bytes=pool_bytes, max_position=33792, seed=4)
    sids = [run.new_seq(int(P[i]), i) for i in range(B)]
    for s, g in zip(sids, G):
        run.fill(s, int(g))
    print(f"[fullsize] serving mix (compress={compress}): {B} sequences filled", flush=True)
    crossed = set()
    for t in range(steps):
        if compress:
            full = [s for s in sids if run.G[s] - run.nb[s] * C == C]
            if full:
                run.compress_and_free(full)
                crossed.update(full)
        results = run.step_fused(sids)
    if compress:
        assert crossed, "no sequence completed a block"
    check = sorted(set([0, 137, 255, 256, 299] + sorted(crossed)[:2]))
    for l in range(2):
        out, lse, q = results[l]
        assert np.isfinite(out).all() and np.isfinite(lse).all()
        for i, s in enumerate(sids):
            nb = run.nb[s]
            want = int(P[i]) + (nb * quotas[l] + (run.G[s] - nb * C) if compress else run.G[s])
            assert run.pool.seq_query(s, l)["resident_rows"] == want, (i, l)
        for s in check:
            i = sids.index(s)
            o_ref, l_ref, _ = run.oracle_decode(s, l, q[i])
            _close(f"mix out seq{i} L{l}", out[i], o_ref, 2e-2)
            _close(f"mix lse seq{i} L{l}", lse[i], l_ref, 1e-3)
    run.pool.close()


def test_serving_mix_full_size_sampled():
    """The saturated serving mix at the size bench.py times: the 200 GiB pool
    holding the sequences bench.py admits (prompts U[128, 512], U[1024, 32768]
    generated tokens, the 36-layer quotas), fused steps up to and past the
    first block that completes (compressed at every layer and freed inside the
    step, as in serving). Row counts of every sequence exact; sampled
    (sequence, layer) outputs of the last step against the oracle, the
    compressed sequence among them."""
    torch.cuda.empty_cache()
    quotas = bench.layer_quotas(2)
    pool_bytes = 200 << 30
    P, G, _ = bench.serving_mix_admit(quotas, 66, True, pool_bytes // (2 * HKV * PR * D * 2))
    B = len(P)
    first = bench.traced_sequence(G, 0)
    steps = (-int(G[first])) % C + 2  # it compresses in the step before the last
    run = Run(L=L, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=int(quotas.max()), quota=quotas.tolist(), pr=PR,
              dtype="bf16", max_seqs=B, pool_bytes=pool_bytes, max_position=33792, seed=4)
    sids = [run.new_seq(int(P[i]), i) for i in range(B)]
    for s, g in zip(sids, G):
        run.fill(s, int(g))
    print(f"[fullsize] serving mix: {B} sequences filled, {steps} steps", flush=True)
    crossed = set()
    for t in range(steps):
        full = [s for s in sids if run.G[s] - run.nb[s] * C == C]
        if full:
            run.compress_and_free(full)
            crossed.update(full)
        results = run.step_fused(sids)
    assert sids[first] in crossed
    layers = _sample_layers(quotas)[::2]  # one layer of each quota class
    seqs = sorted({first, 0, B - 1})
    for l in range(L):
        out, lse, q = results[l]
        assert np.isfinite(out).all() and np.isfinite(lse).all(), l
        for i, s in enumerate(sids):
            nb = run.nb[s]
            want = int(P[i]) + nb * int(quotas[l]) + (run.G[s] - nb * C)
            assert run.pool.seq_query(s, l)["resident_rows"] == want, (i, l)
        if l in layers:
            for i in seqs:
                o_ref, l_ref, _ = run.oracle_decode(sids[i], l, q[i])
                _close(f"mix200 out seq{i} L{l} q{quotas[l]}", out[i], o_ref, 2e-2)
                _close(f"mix200 lse seq{i} L{l} q{quotas[l]}", lse[i], l_ref, 1e-3)
    run.pool.close()
    torch.cuda.empty_cache()


def test_36_layer_per_head_decode_step_sampled():
    # the bench's per-head step (quotas per (layer, KV head), bench.head_quotas):
    # one fused call per layer over the 22 filled sequences, sampled against
    # the oracle's per-head composition
    quotas, P, G = bench.decode_workload(2)
    hq = bench.head_quotas(quotas, 2)
    B = len(P)
    pool_bytes = 0
    for l in range(L):
        for q in hq[l]:
            R = P + ((G + 1 - 1) // C) * q + C
            pool_bytes += int(np.sum(np.ceil(R / PR) + 2 + C // PR)) * 2 * PR * D * 2
    run = Run(L=L, Hq=HQ, Hkv=HKV, D=D, C=C, Kp=KP, quota=quotas.tolist(), pr=PR, dtype="bf16",
              max_seqs=B, pool_bytes=pool_bytes, max_position=33792, seed=2, head_quota=hq)
    sids = [run.new_seq(int(P[i]), i) for i in range(B)]
    for s, g in zip(sids, G):
        run.fill(s, int(g))
    full = [s for s in sids if run.G[s] - run.nb[s] * C == C]
    if full:
        run.compress_and_free(full)
    results = run.step_fused(sids)
    print(f"[fullsize] 36-layer per-head step: {B} sequences", flush=True)
    layers = _sample_layers(quotas)
    for l in range(L):
        out, lse, q = results[l]
        assert np.isfinite(out).all() and np.isfinite(lse).all(), l
        if l in layers:
            for i in (0, 11, 21):
                s = sids[i]
                o_ref, l_ref, keys = run.oracle_decode(s, l, q[i])
                _close(f"36L per-head decode out seq{i} L{l}", out[i], o_ref, 2e-2)
                _close(f"36L per-head decode lse seq{i} L{l}", lse[i], l_ref, 1e-3)
                for h in range(HKV):
                    assert run.pool.seq_query(s, l * HKV + h)["resident_rows"] == len(keys[h][0]), (i, l, h)
