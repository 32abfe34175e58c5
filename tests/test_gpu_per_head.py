"""GPU parity with per-(layer, KV head) quotas (figure captions, Fig. 7: a
quota per (layer, KV head); AI Radio transcript: a per-head schedule). Every
(layer, KV head) holds its own rows and page table; each KV head is checked
against the oracle's per-head composition, with the bars of the other parity
tests: bf16 max-abs 2e-2 on outputs and 1e-3 on lse, fp32 1e-5; kept code rows
and row counts exact."""
import numpy as np
import pytest
import torch

from tests.harness import Run, host

pytestmark = pytest.mark.gpu

TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-5)}

# quotas per (layer, KV head): every power of two up to the pause count, and 0
HQ_BF16 = [[64, 0, 16, 32, 8, 64, 1, 2], [4, 8, 16, 32, 64, 0, 64, 16]]


def _close(name, got, want, tol):
    err = float(np.abs(np.asarray(got) - np.asarray(want)).max()) if np.size(want) else 0.0
    print(f"[parity] {name}: max-abs {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: max-abs {err} > {tol}"


def _check_decode(run, sids, layer, out, lse, q):
    to, tl = TOL[run.dtype]
    for i, s in enumerate(sids):
        o_ref, l_ref, keys = run.oracle_decode(s, layer, q[i])
        _close(f"decode out seq{s} L{layer}", out[i], o_ref, to)
        _close(f"decode lse seq{s} L{layer}", lse[i], l_ref, tl)
        for h in range(run.Hkv):
            info = run.pool.seq_query(s, layer * run.Hkv + h)
            assert info["resident_rows"] == len(keys[h][0]), (s, layer, h)
            assert info["resident_rows"] == (run.P[s] + run.nb[s] * run.head_quota[layer][h]
                                             + run.G[s] - run.nb[s] * run.C)


def _check_compress(run, sids, layer, out, lse):
    to, tl = TOL[run.dtype]
    out, lse = host(out), host(lse)
    dt = torch.bfloat16 if run.dtype == "bf16" else torch.float32
    for i, s in enumerate(sids):
        o_ref, l_ref, codes = run.oracle_compress(s, layer)
        _close(f"compress out seq{s} L{layer}", out[i], o_ref, to)
        _close(f"compress lse seq{s} L{layer}", lse[i], l_ref, tl)
        for h in range(run.Hkv):
            q = run.head_quota[layer][h]
            lv = layer * run.Hkv + h
            r0 = run.pool.seq_query(s, lv)["resident_rows"] - run.C - q
            assert r0 == run.P[s] + run.nb[s] * q
            if q == 0:
                continue
            k = torch.empty((q, 1, run.D), device="cuda", dtype=dt)
            v = torch.empty_like(k)
            run.pool.read_rows(s, lv, r0, q, k, v)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host(v), codes[h][5])
            np.testing.assert_array_equal(host(k), codes[h][4])


def _run(**kw):
    args = dict(L=2, Hq=32, Hkv=8, D=128, C=128, Kp=64, quota=[64, 64], pr=64, dtype="bf16",
                pool_bytes=256 << 20, max_position=4096, head_quota=HQ_BF16)
    args.update(kw)
    return Run(**args)


@pytest.mark.parametrize("fused", [False, True])
def test_per_head_quotas_compress_then_decode(fused):
    run = _run(seed=31)
    sids = [run.new_seq(P, i) for i, P in enumerate([5, 64, 30])]
    for s in sids:
        run.write_prompts(s)
    run.grow({s: 2 * run.C for s in sids})  # one block freed, the second full
    outs = [run.compress_layer(sids, l) for l in range(run.L)]
    torch.cuda.synchronize()
    for l, (out, lse) in enumerate(outs):
        _check_compress(run, sids, l, out, lse)
    run.pool.free_block(sids)
    for s in sids:
        run.nb[s] += 1
    # the next token at every layer, then decode
    res = run.step_fused(sids) if fused else run.step_separate(sids)
    for l, (out, lse, q) in enumerate(res):
        _check_decode(run, sids, l, out, lse, q)


@pytest.mark.parametrize("split_rows", [0, 128])
def test_per_head_quotas_filled_histories(split_rows):
    # long synthetic histories (fill keys rows by the model's layer and KV
    # head) under the automatic schedule and fixed splits
    run = _run(seed=32, split_rows=split_rows, pool_bytes=1 << 30, max_position=40960)
    Gs = [1, 128, 129, 3000, 9001]
    sids = [run.new_seq(P, i) for i, P in enumerate([0, 17, 200, 64, 333])]
    for s, G in zip(sids, Gs):
        run.fill(s, G)
    for l in range(run.L):
        out, lse, q = run.decode(sids, l)
        _check_decode(run, sids, l, out, lse, q)


def test_per_head_quotas_fp32_generic_kernels():
    # fp32, d = 16: the generic compression and split decode kernels
    hq = [[4, 1], [2, 0]]
    run = Run(L=2, Hq=4, Hkv=2, D=16, C=8, Kp=4, quota=[4, 4], pr=4, dtype="f32", head_quota=hq, seed=33,
              max_position=1024)
    sids = [run.new_seq(P, i) for i, P in enumerate([2, 0, 7])]
    for s in sids:
        run.write_prompts(s)
    for blk in range(3):
        run.grow({s: (blk + 1) * run.C for s in sids})
        outs = [run.compress_layer(sids, l) for l in range(run.L)]
        torch.cuda.synchronize()
        for l, (out, lse) in enumerate(outs):
            _check_compress(run, sids, l, out, lse)
        run.pool.free_block(sids)
        for s in sids:
            run.nb[s] += 1
    run.grow({s: 3 * run.C + 5 for s in sids})
    for l in range(run.L):
        out, lse, q = run.decode(sids, l)
        _check_decode(run, sids, l, out, lse, q)


@pytest.mark.parametrize("per_head", [False, True])
def test_budget_pools_compress_then_decode(per_head):
    # one page pool per budget level (AI Radio transcript): results as with one
    # pool; every (sequence, layer) holds pages of its level's id range only
    kw = dict(head_quota=HQ_BF16) if per_head else dict(head_quota=None, quota=[64, 16])
    quotas = [q for row in HQ_BF16 for q in row] if per_head else [64, 16]
    levels = sorted(set(quotas))
    budget = [400] * len(levels)
    run = _run(seed=34, budget_pool_pages=budget, **kw)
    sids = [run.new_seq(P, i) for i, P in enumerate([5, 64, 30])]
    for s in sids:
        run.write_prompts(s)
    run.grow({s: 2 * run.C for s in sids})
    outs = [run.compress_layer(sids, l) for l in range(run.L)]
    torch.cuda.synchronize()
    if per_head:
        for l, (out, lse) in enumerate(outs):
            _check_compress(run, sids, l, out, lse)
    run.pool.free_block(sids)
    for s in sids:
        run.nb[s] += 1
    res = run.step_fused(sids)
    to, tl = TOL[run.dtype]
    for l, (out, lse, q) in enumerate(res):
        if per_head:
            _check_decode(run, sids, l, out, lse, q)
        else:
            for i, s in enumerate(sids):
                o_ref, l_ref, _ = run.oracle_decode(s, l, q[i])
                _close(f"decode out seq{s} L{l}", out[i], o_ref, to)
                _close(f"decode lse seq{s} L{l}", lse[i], l_ref, tl)
    for s in sids:
        for lv in range(len(quotas)):
            pages, _ = run.pool.export_layout(s, lv)
            k = levels.index(quotas[lv])
            assert all(sum(budget[:k]) <= p < sum(budget[:k + 1]) for p in pages), (s, lv)


@pytest.mark.parametrize("Hq,Hkv,D,dtype,pr", [(16, 2, 64, "bf16", 16), (8, 8, 64, "bf16", 32),
                                               (16, 2, 128, "bf16", 32), (2, 1, 16, "f32", 4)])
def test_per_head_quotas_other_shapes(Hq, Hkv, D, dtype, pr):
    # group sizes 8 and 1, d = 64 and 16, 16- and 32-row pages, fp32: the
    # generic decode and compression kernels over per-head pools
    C, Kp = 64, 16
    rng = np.random.default_rng(Hq * 100 + Hkv)
    hq = [[int(x) for x in rng.choice([0, 1, 2, 4, 8, 16], Hkv)] for _ in range(2)]
    run = Run(L=2, Hq=Hq, Hkv=Hkv, D=D, C=C, Kp=Kp, quota=[Kp, Kp], pr=pr, dtype=dtype, head_quota=hq,
              seed=35, max_position=4096, pool_bytes=64 << 20)
    sids = [run.new_seq(P, i) for i, P in enumerate([3, 0, 20])]
    for s in sids:
        run.write_prompts(s)
    for blk in range(2):
        run.grow({s: (blk + 1) * C for s in sids})
        outs = [run.compress_layer(sids, l) for l in range(run.L)]
        torch.cuda.synchronize()
        for l, (out, lse) in enumerate(outs):
            _check_compress(run, sids, l, out, lse)
        run.pool.free_block(sids)
        for s in sids:
            run.nb[s] += 1
    run.grow({s: 2 * C + 7 for s in sids})
    for l in range(run.L):
        out, lse, q = run.decode(sids, l)
        _check_decode(run, sids, l, out, lse, q)
