"""CPU checks of bench.py's accounting: the workload sizes and algorithmic
counts its roofline figures divide by, against the oracle's own enumeration."""
import numpy as np
import pytest

import bench
import oracle
from oracle import LayerView


@pytest.mark.parametrize("P,G,C,Kp,q,comp", [(3, 21, 8, 4, 2, True), (0, 16, 8, 4, 4, True),
                                             (5, 7, 4, 2, 1, True), (4, 9, 8, 4, 2, False)])
def test_prefill_key_count_matches_oracle(P, G, C, Kp, q, comp):
    """The prefill's algorithmic flops are 4 d Hq times the keys every token
    sees under the block mask."""
    L = LayerView(P, C, Kp, q, comp)
    kind, a, b = oracle.training_tokens(L, G)
    nb = G // C if comp else 0
    tot = sum(len(oracle.visible_keys(L, G, nb, (int(x), int(y), int(z)))[0])
              for x, y, z in zip(kind, a, b))
    assert bench.blockmask_visible_keys(P, G, C, Kp, q, comp) == tot


def test_decode_resident_rows_match_oracle():
    """Rows a decode step reads per (sequence, layer), as bench.py counts them
    (C = 512), equal the size of the oracle's visible set."""
    rng = np.random.default_rng(0)
    for _ in range(12):
        P = int(rng.integers(0, 600))
        q = int(rng.choice([64, 128, 256]))
        G = int(rng.integers(1, 3000))
        L = LayerView(P, bench.C, 256, q)
        keys = oracle.visible_keys(L, G, (G - 1) // bench.C, (oracle.TEXT, G - 1, 0))[0]
        assert int(bench.resident_rows(np.array([P]), np.array([G]), q)[0]) == len(keys)
        L0 = LayerView(P, bench.C, 256, q, compress=False)
        keys0 = oracle.visible_keys(L0, G, 0, (oracle.TEXT, G - 1, 0))[0]
        assert int(bench.resident_rows(np.array([P]), np.array([G]), q, compress=False)[0]) == len(keys0)


def test_serving_mix_admission_fits_the_pool():
    quotas = bench.layer_quotas(2)
    pages = 50_000
    for comp in (True, False):
        P, G, used = bench.serving_mix_admit(quotas, 64, comp, pages)
        assert len(P) > 0 and used <= pages


def test_head_quotas_keep_layer_totals():
    """The per-head decode workload keeps each layer's rows: its 8 head quotas
    sum to 8 x the layer quota, are powers of two at most the pause count (256),
    and vary within every layer below 256."""
    quotas = bench.layer_quotas(2)
    hq = bench.head_quotas(quotas, 2)
    assert len(hq) == bench.L
    for q, row in zip(quotas, hq):
        assert len(row) == bench.HKV and sum(row) == bench.HKV * int(q)
        assert all(x > 0 and (x & (x - 1)) == 0 and x <= 256 for x in row)
        assert (len(set(row)) > 1) == (int(q) < 256)


def test_budget_pool_split_covers_the_admitted_needs():
    """The serving mix's per-level pools hold every admitted sequence's largest
    footprint at its level and together no more than the pool."""
    quotas = bench.layer_quotas(2)
    pages = 200 * 2 ** 30 // (2 * bench.HKV * bench.PR * bench.D * 2)
    by = {}
    P, G, used = bench.serving_mix_admit(quotas, 64, True, pages, by_quota=by)
    assert sum(by.values()) == used
    qs, split = bench.budget_pool_split(by, pages)
    assert qs == sorted(set(int(q) for q in quotas))
    assert all(n >= by[q] for q, n in zip(qs, split)) and sum(split) <= pages


def test_traced_sequence_compresses_first():
    """The serving mix traces the sequence whose block completes earliest at
    or after the warmup: brute force over the steps of the compression rule."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        G = rng.integers(1, 40000, int(rng.integers(1, 50)))
        warm = int(rng.integers(0, 4))
        first = [next(t for t in range(warm, warm + bench.C + 1) if (int(x) + t) % bench.C == 0) for x in G]
        assert first[bench.traced_sequence(G, warm)] == min(first)


def test_occupancy_summary_finds_the_drop():
    """A trace that grows by one row per layer and falls at a compression
    step reports that step, its sizes and the closed-form drop it carries."""
    tr = {"sequence": 3, "seq_kv_mb": [10.0, 10.147, 2.0, 2.147], "seq_generated": [511, 512, 513, 514],
          "drop_closed_form_mb": 8.1}
    s = bench.occupancy_summary(tr)
    assert s["sequence"] == 3 and s["generated_at_first_step"] == 511
    assert s["drops"] == [{"step": 2, "generated": 513, "from_mb": 10.147, "to_mb": 2.0}]
    assert s["kv_mb"] == [10.0, 10.1, 2.0, 2.1] and s["drop_closed_form_mb"] == 8.1
