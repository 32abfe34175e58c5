"""The allocation-free decode entry point (abk_decode_attention_noalloc)
against abk_decode_attention through the C ABI: the same outputs on two calls
in a row, the second with fewer sequences (the shared per-GPU workspace keeps
the first call's partials), on each decode path; the oracle as well; and a
call whose partials exceed the fixed workspace refused before anything is
enqueued."""
import numpy as np
import pytest
import torch

import long_reasoning_kv_amd as abk
from tests.harness import Run, dev, host

pytestmark = pytest.mark.gpu

# (pool shape, sequences (prompt, generated)): the MFMA decode (bf16, d = 128,
# four query heads per KV head, 64-row pages), the SIMT stream-K decode (32-row
# pages), the fixed-split decode (split_rows > 0) and the generic fp32 one
CASES = {
    "mfma": (dict(L=2, Hq=32, Hkv=8, D=128, C=512, Kp=128, quota=[128, 64], pr=64, dtype="bf16"),
             [(300, 9001), (17, 4100), (128, 700), (0, 1), (511, 6000)]),
    "stream": (dict(L=1, Hq=32, Hkv=8, D=128, C=512, Kp=128, quota=[128], pr=32, dtype="bf16"),
               [(200, 5000), (33, 1200), (1, 513), (90, 2048)]),
    "split": (dict(L=1, Hq=32, Hkv=8, D=128, C=512, Kp=128, quota=[128], pr=64, dtype="bf16",
                   split_rows=256), [(64, 3000), (7, 900), (250, 2500)]),
    "fp32": (dict(L=1, Hq=8, Hkv=2, D=64, C=64, Kp=16, quota=[8], pr=16, dtype="f32"),
             [(5, 300), (40, 129), (0, 64)]),
}


def _outputs(run, call, sids, layer, q):
    out = torch.empty((len(sids), run.Hq, run.D), device="cuda", dtype=q.dtype)
    lse = torch.empty((len(sids), run.Hq), device="cuda", dtype=torch.float32)
    call(layer, sids, q, out, lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_decode_equals_decode_attention(case):
    kw, seqs = CASES[case]
    run = Run(max_seqs=len(seqs), pool_bytes=512 << 20, max_position=16384, seed=21, **kw)
    print(f"[noalloc] {case}: filling {len(seqs)} sequences", flush=True)
    sids = [run.new_seq(P, i) for i, (P, _) in enumerate(seqs)]
    for s, (_, G) in zip(sids, seqs):
        run.fill(s, G)
    # call 1: every sequence; call 2: fewer
    for ids in (sids, sids[:2]):
        for layer in range(run.L):
            qn = np.stack([run.decode_query(s, layer) for s in ids])
            q = dev(qn, run.dtype)
            oa, la = _outputs(run, run.pool.decode_attention, ids, layer, q)
            ob, lb = _outputs(run, run.pool.decode_attention_noalloc, ids, layer, q)
            print(f"[noalloc] {case}: {len(ids)} sequences, layer {layer}", flush=True)
            assert torch.equal(oa, ob) and torch.equal(la, lb), (case, len(ids), layer)
            to, tl = (2e-2, 1e-3) if run.dtype == "bf16" else (1e-5, 1e-5)
            o_ref, l_ref, _ = run.oracle_decode(ids[-1], layer, qn[-1])
            assert float(np.abs(host(ob)[-1] - o_ref).max()) <= to
            assert float(np.abs(host(lb)[-1] - l_ref).max()) <= tl
    run.pool.close()


def test_noalloc_decode_refuses_partials_above_its_workspace():
    """40 sequences of 4,000 rows in 64-row splits leave 40 x 63 partials of 8
    heads: 42 MB, above the 32 MiB workspace. The call is refused and changes
    nothing; abk_decode_attention serves the same call, and a smaller one still
    fits."""
    run = Run(L=1, Hq=32, Hkv=8, D=128, C=512, Kp=128, quota=[128], pr=64, dtype="bf16", compress=False,
              split_rows=64, max_seqs=40, pool_bytes=1 << 30, max_position=8192, seed=22)
    sids = [run.new_seq(100, i) for i in range(40)]
    for s in sids:
        run.fill(s, 3900)
    q = dev(np.stack([run.decode_query(s, 0) for s in sids]), "bf16")
    before = [run.pool.seq_query(s, 0) for s in sids]
    out = torch.full((40, 32, 128), 7.0, device="cuda", dtype=torch.bfloat16)
    lse = torch.full((40, 32), 7.0, device="cuda", dtype=torch.float32)
    with pytest.raises(abk.AbkError) as e:
        run.pool.decode_attention_noalloc(0, sids, q, out, lse)
    assert e.value.status == abk.UNSUPPORTED
    torch.cuda.synchronize()
    assert [run.pool.seq_query(s, 0) for s in sids] == before
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())  # nothing was enqueued
    oa, la = _outputs(run, run.pool.decode_attention, sids[:8], 0, q[:8])
    ob, lb = _outputs(run, run.pool.decode_attention_noalloc, sids[:8], 0, q[:8])
    assert torch.equal(oa, ob) and torch.equal(la, lb)
    run.pool.close()
