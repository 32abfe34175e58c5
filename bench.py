#!/usr/bin/env python3
"""Benchmark of the AbridgeKV attention hot path on one MI355X.

Default workload (the metric's configuration): one decode step across all 36
layers of a Qwen3-4B-shaped cache (32 query / 8 KV heads, d = 128, bf16) for 22
sequences with prompts U[128, 512] and U[4096, 32768] generated tokens, blocks
of C = 512 compressed to per-layer quotas (6 layers keep 256 rows per block, 12
keep 64, 18 keep 128; which layers is a seeded permutation). A step is, per
layer, one call that appends the current token (RoPE + write) and runs the
split-KV decode attention over the resident rows (abk_append_decode); any
sequence whose block completes is compressed at every layer and its raw pages
freed inside the step, as in serving. Inputs are synthetic and already
resident in HBM when timing starts.

Prints one JSON line: tokens/s, achieved HBM GB/s of the decode call against
MI355X's 8 TB/s (HIP events around every call in the timed region), the CPU
oracle on a bounded sample, the block-compression event (64 sequences x 36
layers) and the block-mask prefill at the Fig. 9 shape, each with its MFMA
rate, and a bounded run of the saturated serving mix (200 GiB pool, AbridgeKV
against full KV through the same kernels, `--mix-steps` steps each).
`--serving-mix` runs only the serving mix, with its occupancy trace;
`--profile-summary DIR` writes profiles/ from rocprofv3 runs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
L, HQ, HKV, D, C, PR = 36, 32, 8, 128, 512, 64
METRIC = "decode-attn tokens/s + achieved HBM GB/s over AbridgeKV cache (36L quotas)"


def layer_quotas(seed: int):
    """Seeded permutation of the 36 layers: first 6 keep 256, next 12 keep 64,
    the remaining 18 keep 128 (mean 128 rows per 512-token block)."""
    perm = np.random.default_rng(seed).permutation(L)
    q = np.empty(L, np.int32)
    q[perm[:6]] = 256
    q[perm[6:18]] = 64
    q[perm[18:]] = 128
    return q


def head_quotas(quotas, seed: int = 2):
    """Per-(layer, KV head) quotas with each layer's total kept: a layer of
    quota q <= 128 gives its 8 KV heads a seeded permutation of {2q, q/2, q/2,
    q, q, q, q, q} (one head doubled, two halved, as in Fig. 7's single-head
    moves); a layer at the pause count (256) keeps 256 on every head."""
    rng = np.random.default_rng(seed + 1000)
    out = []
    for q in quotas:
        q = int(q)
        row = [2 * q, q // 2, q // 2] + [q] * (HKV - 3) if 2 * q <= 256 else [q] * HKV
        out.append([int(x) for x in rng.permutation(row)])
    return out


def decode_workload(seed: int = 2, batch: int = 22):
    rng = np.random.default_rng(seed)
    P = rng.integers(128, 512, batch, endpoint=True)
    G = rng.integers(4096, 32768, batch, endpoint=True)
    return layer_quotas(seed), P.astype(int), G.astype(int)


def resident_rows(P, G, q, compress=True):
    if not compress:
        return P + G
    nb = (G - 1) // C
    return P + nb * q + (G - nb * C)


KERNEL_SOURCES = {
    "decode_mfma": ("decode.hip", "common.h", "kernels.h"),
    "compress_attn_mfma": ("compress.hip", "attn_mfma.h", "common.h", "kernels.h"),
    "blockmask_attn_mfma": ("prefill.hip", "attn_mfma.h", "common.h", "kernels.h"),
}


def kernel_source_hash(kernel: str):
    """Hash of the sources a kernel family is built from: counters taken on
    other sources no longer describe it."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "long_reasoning_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, launches_bytes: float):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/*.json),
    or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(kernel):
        return None
    return t.get("bytes_per_launch")


# ---- rocprofv3 summaries ----------------------------------------------------------

NUM_XCD, NUM_CU, SIMD_PER_CU = 8, 256, 4


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _find(d, suffix):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    return None


def _cmd(d, name):
    path = os.path.join(d, name + ".cmd")
    return open(path).read().strip() if os.path.exists(path) else "(command not recorded)"


def _counters(d, name, counter, match):
    """Per-dispatch values of one counter for kernels whose name contains ``match``."""
    path = _find(os.path.join(d, name), "counter_collection.csv")
    if path is None:
        return []
    return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in _csv_rows(path)
            if r["Counter_Name"] == counter and match in r["Kernel_Name"]]


def _calibration(d):
    """KiB that FETCH_SIZE / WRITE_SIZE read for one plain device copy of known
    size: the scale from counter units to HBM bytes."""
    info = os.path.join(d, "copy_fetch.json")
    n = json.load(open(info))["copy_bytes"] if os.path.exists(info) else 1 << 30
    out = {"copy_bytes": n}
    for which, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        vals = sorted(v for _, v in _counters(d, "copy_" + which, counter, "copyBuffer"))[-3:]
        kib = float(np.mean(vals)) if vals else float("nan")
        out[which + "_kib_per_copy"] = kib
        out[which + "_scale"] = (n / 1024.0) / kib if vals else float("nan")
    return out


def _stats_table(d, name, match):
    path = _find(os.path.join(d, name), "kernel_stats.csv")
    lines = []
    for r in _csv_rows(path) if path else []:
        if any(m in r["Name"] for m in match):
            lines.append(f"  {r['Name'][:60]:60s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.1f} "
                         f"{float(r['MinNs']) / 1e3:9.1f} {float(r['MaxNs']) / 1e3:9.1f} "
                         f"{float(r['TotalDurationNs']) / 1e6:10.2f}")
    head = f"  {'kernel':60s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_ms':>10s}"
    return [head] + lines, path


SQ_PASSES = {
    "sq": ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_WAVES"),
    "stall": ("SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_ANY",
              "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_COEXEC_CYCLES"),
    "lds": ("SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_ADDR_CONFLICT", "SQ_LDS_UNALIGNED_STALL",
            "SQ_LDS_IDX_ACTIVE", "SQ_LDS_DATA_FIFO_FULL", "SQ_LDS_CMD_FIFO_FULL"),
    "grbm": ("GRBM_GUI_ACTIVE",),
}


def sq_summary(d, prefix, match):
    """Lines on where an MFMA kernel's time goes, from the SQ counter passes
    <prefix>_sq, _stall, _lds and _grbm (means per dispatch)."""
    v = {}
    for pas, names in SQ_PASSES.items():
        for c in names:
            r = _counters(d, f"{prefix}_{pas}", c, match)
            if r:
                v[c] = float(np.mean([x for _, x in r]))
    if "GRBM_GUI_ACTIVE" not in v or "SQ_VALU_MFMA_BUSY_CYCLES" not in v:
        return []
    gui = v["GRBM_GUI_ACTIVE"] / NUM_XCD
    simd = gui * NUM_CU * SIMD_PER_CU
    out = [f"SQ counters, mean per dispatch (GRBM_GUI_ACTIVE summed over {NUM_XCD} XCDs: "
           f"{gui:.4g} cycles each):"]
    for c in sorted(v):
        out.append(f"  {c:28s} {v[c]:.4g}")
    out.append(f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x {NUM_CU} CUs x {SIMD_PER_CU} SIMDs) = "
               f"{100 * v['SQ_VALU_MFMA_BUSY_CYCLES'] / simd:.1f}%")
    if "SQ_BUSY_CU_CYCLES" in v:
        out.append(f"CU busy = SQ_BUSY_CU_CYCLES / (cycles x {NUM_CU}) = "
                   f"{100 * v['SQ_BUSY_CU_CYCLES'] / (gui * NUM_CU):.1f}%")
    if "SQ_INSTS_VALU" in v and "SQ_INSTS_MFMA" in v:
        out.append(f"VALU instructions (MFMA included) per MFMA: {v['SQ_INSTS_VALU'] / v['SQ_INSTS_MFMA']:.2f}")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in v:
        out.append(f"cycles with a VALU instruction issued while the MFMA unit is busy: "
                   f"{100 * v['SQ_VALU_MFMA_COEXEC_CYCLES'] / v['SQ_VALU_MFMA_BUSY_CYCLES']:.1f}% of MFMA-busy cycles")
    if "SQ_WAVE_CYCLES" in v:
        w = v["SQ_WAVE_CYCLES"]
        out.append(f"wave time: issuing {100 * v['SQ_ACTIVE_INST_ANY'] / w:.1f}%, waiting to issue "
                   f"(dependency or busy unit) {100 * v['SQ_WAIT_INST_ANY'] / w:.1f}%, waiting on a counter "
                   f"or barrier {100 * v['SQ_WAIT_ANY'] / w:.1f}%; VALU issue {100 * v['SQ_ACTIVE_INST_VALU'] / w:.1f}%, "
                   f"LDS issue {100 * v['SQ_ACTIVE_INST_LDS'] / w:.1f}%, waiting for LDS issue "
                   f"{100 * v['SQ_WAIT_INST_LDS'] / w:.1f}%")
    if "SQ_LDS_IDX_ACTIVE" in v:
        out.append(f"LDS: bank conflicts {v['SQ_LDS_BANK_CONFLICT']:.0f}, address conflicts "
                   f"{v['SQ_LDS_ADDR_CONFLICT']:.0f}, unaligned stalls {v['SQ_LDS_UNALIGNED_STALL']:.0f}; "
                   f"FIFO-full cycles summed over the counters' instances: data {v['SQ_LDS_DATA_FIFO_FULL']:.3g}, "
                   f"command {v['SQ_LDS_CMD_FIFO_FULL']:.3g} (against {gui:.3g} cycles per XCD)")
    for pas in SQ_PASSES:
        out.append(f"  {pas} pass: {_cmd(d, f'{prefix}_{pas}')}")
    return out


def profile_summary(d):
    """Write profiles/*.txt and profiles/*_traffic.json from a directory of
    rocprofv3 runs (one sub-directory per pass, ``<pass>.cmd`` holding the
    command of each pass, ``<pass>.json`` the JSON line bench printed)."""
    cal = _calibration(d)
    prof = os.path.join(ROOT, "profiles")
    os.makedirs(prof, exist_ok=True)
    cal_lines = [
        f"calibration: a plain device copy of {cal['copy_bytes']} B reads FETCH_SIZE "
        f"{cal['fetch_kib_per_copy']:.1f} KiB and WRITE_SIZE {cal['write_kib_per_copy']:.1f} KiB per "
        f"dispatch -> scale {cal['fetch_scale']:.3f} (fetch), {cal['write_scale']:.3f} (write)",
        f"  fetch pass: {_cmd(d, 'copy_fetch')}",
        f"  write pass: {_cmd(d, 'copy_write')}",
    ]
    for fam, tag, trace, prefix, match, what in (
            ("decode_mfma", "decode_mfma_36L_22seq", "dec_trace", "dec", "decode_",
             "decode step of the 36-layer per-layer-quota workload, 22 sequences, bf16, d = 128, "
             "32 q / 8 KV heads, 64-row pages (bench.py default workload)"),
            ("compress_attn_mfma", "compress_attn_mfma_64seq_36L", "cmp_trace", "cmp",
             "compress_attn_mfma",
             "block compression event: 64 sequences x 36 layers, K = 256 pause tokens, bf16, "
             "d = 128, 32 q / 8 KV heads (bench.py compression event)"),
            ("blockmask_attn_mfma", "blockmask_attn_mfma_fig9_36L", "pre_trace", "pre",
             "blockmask_",
             "block-mask prefill at the Fig. 9 shape: 256-token prompt + 16,384 text tokens, "
             "C = 512, K = 256, 36 layers, bf16, d = 128, 32 q / 8 KV heads (bench.py prefill)")):
        if not os.path.isdir(os.path.join(d, prefix + "_fetch")):
            continue
        table, _ = _stats_table(d, trace, [match, "append_kernel", "pause_rope"])
        fetch = _counters(d, prefix + "_fetch", "FETCH_SIZE", match)
        write = _counters(d, prefix + "_write", "WRITE_SIZE", match)
        by = {}
        for nm, v in fetch:
            by.setdefault(nm, [[], []])[0].append(v)
        for nm, v in write:
            by.setdefault(nm, [[], []])[1].append(v)
        # one call = one dispatch of each kernel of the family
        per_call = 0.0
        cnt_lines = [f"  {'kernel':60s} {'dispatches':>10s} {'FETCH KiB':>12s} {'WRITE KiB':>12s} "
                     f"{'HBM MB':>10s}"]
        fetch_kib = write_kib = 0.0
        for nm, (fv, wv) in sorted(by.items()):
            f_, w_ = float(np.mean(fv)), float(np.mean(wv))
            mb = (f_ * cal["fetch_scale"] + w_ * cal["write_scale"]) * 1024 / 1e6
            per_call += mb * 1e6
            fetch_kib += f_
            write_kib += w_
            cnt_lines.append(f"  {nm[:60]:60s} {len(fv):10d} {f_:12.1f} {w_:12.1f} {mb:10.2f}")
        bench_json = os.path.join(d, trace + ".json")
        bj = json.load(open(bench_json)) if os.path.exists(bench_json) else None
        extra = []
        if fam == "decode_mfma" and bj:
            rf = bj["roofline"]
            extra = [f"bench.py in the traced run: {rf['avg_launch_us']:.1f} us per decode call "
                     f"(HIP events around each step's fused calls, per call), algorithmic "
                     f"{rf['algorithmic_bytes_per_launch'] / 1e6:.1f} MB per call, "
                     f"{rf['achieved']:.0f} GB/s = {100 * rf['frac']:.1f}% of 8 TB/s",
                     f"counted HBM bytes / algorithmic bytes: "
                     f"{per_call / rf['algorithmic_bytes_per_launch']:.3f}"]
        if fam == "blockmask_attn_mfma" and bj and bj.get("prefill"):
            pf = bj["prefill"]
            extra = [f"bench.py in the traced run: {pf['ms_per_forward']:.1f} ms per 36-layer forward, "
                     f"{pf['roofline']['achieved']:.0f} TFLOP/s algorithmic = "
                     f"{100 * pf['roofline']['frac']:.1f}% of 2.5 PFLOP/s bf16"]
        if fam in ("compress_attn_mfma", "blockmask_attn_mfma"):
            extra += sq_summary(d, prefix, "compress_attn_mfma" if prefix == "cmp" else "blockmask_attn")
        if fam == "compress_attn_mfma" and bj and bj.get("compress"):
            c = bj["compress"]
            extra.append(f"bench.py in the traced run: {c['ms_per_event']:.1f} ms per event, "
                         f"{c['roofline']['achieved']:.0f} TFLOP/s algorithmic = "
                         f"{100 * c['roofline']['frac']:.1f}% of 2.5 PFLOP/s bf16")
        text = [f"{fam} -- {what}", "",
                "Commands (run from the repository root with TMPDIR=/tmp; "
                "the library built in-tree beforehand):",
                f"  trace pass: {_cmd(d, trace)}",
                f"  fetch pass: {_cmd(d, prefix + '_fetch')}",
                f"  write pass: {_cmd(d, prefix + '_write')}", "",
                "rocprofv3 --kernel-trace --stats (durations in us):"] + table + [
                "", "Counters, mean per dispatch (FETCH_SIZE and WRITE_SIZE in KiB, scaled to HBM "
                "bytes with the copy calibration):"] + cnt_lines + [
                f"HBM bytes per call (one dispatch of each kernel above): {per_call / 1e6:.2f} MB", ""
                ] + cal_lines + ([""] + extra if extra else [])
        with open(os.path.join(prof, tag + ".txt"), "w") as f:
            f.write("\n".join(text) + "\n")
        rec = {"kernel": fam, "kernel_source_hash": kernel_source_hash(fam),
               "bytes_per_launch": per_call, "fetch_kib_per_launch": fetch_kib,
               "write_kib_per_launch": write_kib, "fetch_scale": cal["fetch_scale"],
               "write_scale": cal["write_scale"], "summary": f"profiles/{tag}.txt"}
        with open(os.path.join(prof, fam + "_traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        print(f"wrote profiles/{tag}.txt and profiles/{fam}_traffic.json")
    if os.path.isdir(os.path.join(d, "mix_trace")):
        mix_summary(d, prof)


def mix_summary(d, prof):
    """profiles/serving_mix_200GiB.txt: the kernel table of a traced serving-mix
    run beside the bench lines of that run and of an untraced full run."""
    table, _ = _stats_table(d, "mix_trace", ["decode_", "compress", "pause_rope", "free_kernel"])
    lines = ["serving mix -- 200 GiB paged pool, 36 layers, quotas 6x256/12x64/18x128, "
             "P ~ U[128,512], G ~ U[1024,32768]; AbridgeKV, then full KV through the same kernels", "",
             "Commands (run from the repository root with TMPDIR=/tmp; the library built in-tree beforehand):",
             f"  trace pass: {_cmd(d, 'mix_trace')}", "",
             "rocprofv3 --kernel-trace --stats of the traced run (durations in us; both modes):"] + table
    for name, what in (("mix_trace", "traced run"), ("mix_full", "untraced run")):
        path = os.path.join(d, name + ".json")
        if not os.path.exists(path):
            continue
        j = json.load(open(path))
        lines += ["", f"bench.py line of the {what}" + (f" ({_cmd(d, name)})" if name == "mix_full" else "") + ":"]
        for mode in ("abridgekv", "full_kv"):
            m = j[mode]
            lines.append(f"  {mode:9s}: {m['sequences_resident']} sequences, {m['steps']} steps, "
                         f"{m['tokens_per_s']:.0f} tokens/s, {m['ms_per_step']:.2f} ms/step, "
                         f"{m['compressions_in_timed_steps']} compressions, "
                         f"{m['kv_gbps_incl_compression']:.0f} GB/s of K/V read")
        lines.append(f"  ratios: sequences x{j['sequences_ratio']:.2f}, tokens/s x{j['tokens_per_s_ratio']:.2f}")
        if name == "mix_full":
            tr = j["abridgekv"]["occupancy_trace"]
            kv = tr["seq_kv_mb"]
            lines += ["", f"occupancy (untraced run, AbridgeKV): sequence {tr['sequence']}'s resident K/V in MB, "
                          "every 16th step, with its generated count:",
                      "  " + ", ".join(f"{g}:{x:.0f}" for g, x in
                                       list(zip(tr["seq_generated"], kv))[::16]),
                      "pool pages by layer budget (rows kept per block) every 32 steps:"]
            for q, v in tr["pages_by_quota"].items():
                lines.append(f"  {q:>3s}-row layers: " + ", ".join(str(x) for x in v))
    with open(os.path.join(prof, "serving_mix_200GiB.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/serving_mix_200GiB.txt")


# ---------------------------------------------------------------------------------

def run_decode(args, torch, abk):
    quotas, P, G = decode_workload(args.seed)
    B = len(P)
    Kp = int(quotas.max())
    hq = head_quotas(quotas, args.seed) if args.per_head else [[int(q)] * HKV for q in quotas]
    # warmup, then the timed steps twice: alone (value, ms_per_step), then with
    # HIP events for the roofline's per-call durations: around each step's 36
    # fused calls (after the step's compressions), or with --separate-append
    # around every decode call (the appends between them excluded)
    total_steps = args.warmup + 2 * args.steps
    # pool: resident rows now plus growth over the run, in whole pages, with slack
    pages = 0
    for l in range(L):
        for qh in (hq[l] if args.per_head else [quotas[l]]):
            R = resident_rows(P, G + total_steps, qh)
            pages += int(np.sum(np.ceil(R / PR) + 2 + C // PR))
    page_bytes = (1 if args.per_head else HKV) * PR * D * 2
    pool = abk.Pool(num_layers=L, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_tokens=C,
                    num_pause=Kp, layer_quota=quotas.tolist(), page_rows=PR, max_seqs=B,
                    pool_bytes=2 * page_bytes * pages, max_position=33792, dtype="bf16",
                    rope_base=1e6, decode_split_rows=args.split_rows,
                    head_quota=hq if args.per_head else None)
    sids = []
    for i in range(B):
        s = pool.seq_create(int(P[i]))
        pool.synth_fill(s, int(G[i]), (args.seed * 1000003 + i * 7919 + 17))
        sids.append(s)
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda")
    gen.manual_seed(args.seed)
    bf = torch.bfloat16
    q_in = torch.randn((total_steps, L, B, HQ, D), device="cuda", dtype=bf, generator=gen)
    k_in = torch.randn((total_steps, L, B, HKV, D), device="cuda", dtype=bf, generator=gen)
    v_in = torch.randn((total_steps, L, B, HKV, D), device="cuda", dtype=bf, generator=gen)
    qp = torch.randn((B, Kp, HQ, D), device="cuda", dtype=bf, generator=gen)
    kp = torch.randn((B, Kp, HKV, D), device="cuda", dtype=bf, generator=gen)
    vp = torch.randn((B, Kp, HKV, D), device="cuda", dtype=bf, generator=gen)
    out = torch.empty((B, HQ, D), device="cuda", dtype=bf)
    lse = torch.empty((B, HQ), device="cuda", dtype=torch.float32)
    cout = torch.empty((B, Kp, HQ, D), device="cuda", dtype=bf)
    clse = torch.empty((B, Kp, HQ), device="cuda", dtype=torch.float32)

    # host mirror of generated counts for the compress/free schedule and bytes
    g = G.copy()
    nb = (g - 1) // C
    # per-layer views and events made before the timed region, so that the host
    # stays well ahead of the GPU inside it
    views = [[(q_in[t, l], k_in[t, l], v_in[t, l]) for l in range(L)] for t in range(total_steps)]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(L)] for _ in range(args.steps)]
    cev = []

    ncomp = [0, 0]  # blocks compressed in the first (value) and second (events) timed pass

    def step(t, rec):
        full = [i for i in range(B) if g[i] - nb[i] * C == C]
        if full and t >= args.warmup:
            ncomp[0 if rec is None else 1] += len(full)
        if full:
            ids = [sids[i] for i in full]
            for l in range(L):
                if rec is not None:
                    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    c0.record()
                pool.compress_block(l, ids, qp[:len(ids)], kp[:len(ids)], vp[:len(ids)],
                                    cout[:len(ids)], clse[:len(ids)])
                if rec is not None:
                    c1.record()
                    cev.append((c0, c1))
            pool.free_block(ids)
            for i in full:
                nb[i] += 1
        for l in range(L):
            q, k, v = views[t][l]
            if args.separate_append:
                # the events bracket the decode call alone
                pool.append_kv(l, sids, k, v)
                if rec is not None:
                    rec[l][0].record()
                pool.decode_attention(l, sids, q, out, lse)
                if rec is not None:
                    rec[l][1].record()
            else:
                if rec is not None and l == 0:
                    rec[0][0].record()
                pool.append_decode(l, sids, k, v, q, out, lse)
                if rec is not None and l == L - 1:
                    rec[0][1].record()
        if rec is not None:
            # resident (row, KV head) pairs each call reads
            rows_log.append([sum(int((P + nb * qh + (g + 1 - nb * C)).sum()) for qh in hq[l]) for l in range(L)])
        g[:] += 1

    rows_log = []
    for t in range(args.warmup):
        step(t, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, args.warmup + args.steps):
        step(t, None)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    for t in range(args.warmup + args.steps, total_steps):
        step(t, ev[t - args.warmup - args.steps])
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t1
    # algorithmic bytes of one decode call: every resident K and V row once,
    # plus q, out (bf16) and lse (fp32); a fused call also reads the new k, v
    # and writes them as the new row
    row_bytes = 2 * HKV * D * 2
    io_bytes = B * (2 * HQ * D * 2 + HQ * 4) + (0 if args.separate_append else B * 2 * row_bytes)
    if args.separate_append:
        dec_ms = [e0.elapsed_time(e1) for evs in ev for e0, e1 in evs]
    else:
        # one bracket per step: its calls' mean duration, once per call
        dec_ms = [evs[0][0].elapsed_time(evs[0][1]) / L for evs in ev for _ in range(L)]
    dec_bytes = [rh * (2 * D * 2) + io_bytes for rl in rows_log for rh in rl]
    achieved = sum(dec_bytes) / (sum(dec_ms) * 1e-3) / 1e9
    comp_ms = sum(a.elapsed_time(b) for a, b in cev)
    tokens = B * args.steps
    # every sequence compresses one block per C generated tokens: the measured
    # cost of a block (all layers), spread over the C steps that lead to it
    amortized = None
    if ncomp[1] > 0:
        per_step_ms = wall * 1e3 / args.steps + B / C * comp_ms / ncomp[1]
        amortized = {"value": B / (per_step_ms * 1e-3), "ms_per_step": per_step_ms,
                     "ms_per_block": comp_ms / ncomp[1]}
    resident = pool.stats()["resident_bytes"]
    full_kv_rows = int(sum(resident_rows(P, g, quotas[l], compress=False).sum() for l in range(L)))
    res = {
        "value": tokens / wall,
        "ms_per_step": wall * 1e3 / args.steps,
        "ms_per_step_with_events": wall_ev * 1e3 / args.steps,
        "hbm_gbps": achieved,
        "decode_ms_per_step": sum(dec_ms) / args.steps,
        "compress_ms_in_event_steps": comp_ms,
        "blocks_compressed": {"value_steps": ncomp[0], "event_steps": ncomp[1]},
        "with_compression_amortized": amortized,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic_from_profiles("decode_mfma", float(np.mean(dec_bytes))),
            "kernel": ("decode_mfma_kernel (+ decode_stream_merge_kernel)" if args.separate_append else
                       "decode_mfma_kernel with fused append (+ decode_stream_merge_kernel)"),
            "timing": ("HIP events around every decode call" if args.separate_append else
                       "HIP events around each step's 36 fused calls, divided by 36"),
            "algorithmic_bytes_per_launch": float(np.mean(dec_bytes)),
            "avg_launch_us": float(np.mean(dec_ms)) * 1e3,
        },
        "config": {
            "workload": "36-layer " + ("per-(layer, KV head)" if args.per_head else "per-layer") +
                        "-quota decode step (append + split-KV decode per "
                        "layer, " + ("two calls" if args.separate_append else "one fused call") +
                        " each; compress+free when a block completes), 22 sequences",
            "layers": L, "batch": B, "q_heads": HQ, "kv_heads": HKV, "head_dim": D,
            "block_tokens": C, "pause_tokens": Kp,
            "quotas": ("per (layer, KV head): each layer's 8 heads a seeded permutation of "
                       "{2q, q/2, q/2, q x 5} of the layer quota q (6x256/12x64/18x128, seeded; 256: "
                       "every head)" if args.per_head else "6x256/12x64/18x128 (seeded)"),
            "prompt": "U[128,512]", "generated": "U[4096,32768]", "page_rows": PR,
            "resident_kv_gb": resident / 1e9,
            "full_kv_equivalent_gb": full_kv_rows * row_bytes / 1e9,
        },
    }
    pool.close()
    del q_in, k_in, v_in
    return res, (quotas, P, G)


def run_decode_1layer(args, torch, abk, reps: int = 50):
    """The one-layer decode call: 16 sequences, prompt 256, 7,900 generated
    tokens (15 compressed blocks + 220 open rows), quota = K = 128: 2,396
    resident rows per sequence. Each timed call follows a 1 GiB write, so the
    157 MB it reads cannot be served from the last-level cache: a 1 GiB buffer
    is read (not written, which would leave dirty lines to drain during the
    call) before each timed call. The median over `reps` calls, HIP events on
    the library's stream."""
    B, P0, G0, q = 16, 256, 7900, 128
    rows = P0 + ((G0 - 1) // C) * q + (G0 - ((G0 - 1) // C) * C)
    pool = abk.Pool(num_layers=1, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_tokens=C,
                    num_pause=q, layer_quota=[q], page_rows=PR, max_seqs=B, pool_bytes=1 << 30,
                    max_position=8192, dtype="bf16", rope_base=1e6)
    sids = []
    for i in range(B):
        s = pool.seq_create(P0)
        pool.synth_fill(s, G0, 1 * 1000003 + i * 7919 + 17)
        sids.append(s)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    qd = torch.randn((B, HQ, D), device="cuda", dtype=torch.bfloat16, generator=gen)
    out = torch.empty((B, HQ, D), device="cuda", dtype=torch.bfloat16)
    lse = torch.empty((B, HQ), device="cuda", dtype=torch.float32)
    flush = torch.ones(1 << 28, device="cuda", dtype=torch.int32)  # 1 GiB
    acc = torch.zeros((), device="cuda", dtype=torch.int64)
    times, warm = [], []
    for r in range(reps + 3):
        acc += flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pool.decode_attention(0, sids, qd, out, lse)
        e1.record()
        torch.cuda.synchronize()
        if r >= 3:
            times.append(e0.elapsed_time(e1) * 1e3)
    # back to back, no flush between calls (the cache then holds part of the rows)
    for r in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pool.decode_attention(0, sids, qd, out, lse)
        e1.record()
        torch.cuda.synchronize()
        warm.append(e0.elapsed_time(e1) * 1e3)
    pool.close()
    del flush
    torch.cuda.empty_cache()
    nbytes = B * rows * 2 * HKV * D * 2 + B * (2 * HQ * D * 2 + HQ * 4)
    us = float(np.median(times))
    return {"metric": "one-layer decode call, 16 sequences x 2,396 resident rows",
            "us_per_call": us, "tokens_per_s": B / (us * 1e-6),
            "algorithmic_bytes": nbytes, "gbps": nbytes / (us * 1e-6) / 1e9,
            "frac_of_8tbs": nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "us_per_call_no_flush": float(np.median(warm)),
            "config": {"workload": "1 layer, 16 sequences, P = 256, G = 7,900, quota = K = 128, bf16, "
                                   "64-row pages; 1 GiB read before each timed call", "reps": reps}}


def compress_event(args, torch, abk, layer_pause=None, single_sequence=True):
    """One block-compression event: 64 sequences complete a 512-token block at
    once; pause-token attention + code-row scatter at all 36 layers, then the
    raw pages are freed. layer_pause None: every layer runs 256 pause tokens
    and keeps its quota's prefix; else layer l runs layer_pause[l]."""
    rng = np.random.default_rng(3)
    quotas = layer_quotas(2)
    B = 64
    P = rng.integers(128, 512, B, endpoint=True)
    b = rng.integers(0, 62, B, endpoint=True)
    G = (b + 1) * C
    Kp = 256
    kps = [Kp] * L if layer_pause is None else [int(x) for x in layer_pause]
    pages = 0
    for l in range(L):
        pages += int(np.sum(np.ceil((P + (b + 1) * quotas[l]) / PR) + 1 + C // PR))
    page_bytes = HKV * PR * D * 2
    pool = abk.Pool(num_layers=L, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_tokens=C,
                    num_pause=Kp, layer_quota=quotas.tolist(), layer_pause=layer_pause, page_rows=PR,
                    max_seqs=B, pool_bytes=2 * page_bytes * pages, max_position=33792, dtype="bf16",
                    rope_base=1e6)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3)
    bf = torch.bfloat16
    qp = [torch.randn((B, kps[l], HQ, D), device="cuda", dtype=bf, generator=gen) for l in range(L)]
    kp = [torch.randn((B, kps[l], HKV, D), device="cuda", dtype=bf, generator=gen) for l in range(L)]
    vp = [torch.randn((B, kps[l], HKV, D), device="cuda", dtype=bf, generator=gen) for l in range(L)]
    out = torch.empty((B, Kp, HQ, D), device="cuda", dtype=bf)
    lse = torch.empty((B, Kp, HQ), device="cuda", dtype=torch.float32)
    times = []
    for rep in range(args.compress_reps + 1):
        sids = []
        for i in range(B):
            s = pool.seq_create(int(P[i]))
            pool.synth_fill(s, int(G[i]), 3 * 1000003 + i)
            sids.append(s)
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(L + 1)]
        e[0].record()
        for l in range(L):
            pool.compress_block(l, sids, qp[l], kp[l], vp[l], out, lse)
            e[l + 1].record()
        pool.free_block(sids)
        torch.cuda.synchronize()
        if rep > 0:
            times.append([e[l].elapsed_time(e[l + 1]) for l in range(L)])
        for s in sids:
            pool.seq_release(s)
    # one sequence completing its last block alone (the common serving case):
    # the context of each query tile is split over several workgroups
    single = []
    for rep in range(args.compress_reps + 1 if single_sequence else 0):
        s = pool.seq_create(int(P[0]))
        pool.synth_fill(s, 63 * C, 3 * 1000003 + 999)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for l in range(L):
            pool.compress_block(l, [s], qp[l][:1], kp[l][:1], vp[l][:1], out[:1], lse[:1])
        e1.record()
        pool.free_block([s])
        torch.cuda.synchronize()
        if rep > 0:
            single.append(e0.elapsed_time(e1))
        pool.seq_release(s)
    pool.close()
    ms = float(np.mean([sum(t) for t in times]))
    # algorithmic flops: QK^T and PV over context N_l plus the causal pause part
    flops = 0.0
    nbytes = 0.0
    for l in range(L):
        N = P + b * quotas[l] + C
        flops += float(np.sum(4.0 * HQ * kps[l] * D * (N + (kps[l] + 1) / 2.0)))
        nbytes += float(np.sum(N)) * 2 * HKV * D * 2 + B * kps[l] * (2 * HQ + 2 * HKV) * D * 2
    return {"ms": ms, "flops": flops, "nbytes": nbytes, "B": B, "P0": int(P[0]),
            "single_ms": float(np.mean(single)) if single else None}


def run_compress(args, torch, abk):
    """The compression event under the default pause reading (256 pause tokens
    at every layer, each layer keeping its quota's prefix), then the same event
    with as many pause tokens per layer as its quota."""
    ev = compress_event(args, torch, abk, single_sequence=not args.no_single_sequence)
    ms, flops, nbytes, B = ev["ms"], ev["flops"], ev["nbytes"], ev["B"]
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": "block compressions/s (64 sequences x 36 layers per event)",
        "events_per_s": 1e3 / ms, "ms_per_event": ms,
        "blocks_per_s": B * 1e3 / ms,
        "tflop_per_event": flops / 1e12, "gb_per_event": nbytes / 1e9,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / BF16_PEAK_TFLOPS,
                     # HBM bytes per launch (one layer of the event), from the counters
                     "traffic": traffic_from_profiles("compress_attn_mfma", nbytes / L)},
        "config": {"workload": "block compression, 64 sequences, 36 layers, K=256 pause tokens "
                               "(layer keeps quota prefix)", "prompt": "U[128,512]",
                   "block_index": "U{0..62}"},
        "single_sequence_ms": ev["single_ms"],
        "single_sequence": f"one sequence (prompt {ev['P0']}) compressing block 62 alone, 36 layers",
    }
    if not args.no_pause_per_layer:
        a = compress_event(args, torch, abk, layer_pause=layer_quotas(2).tolist(), single_sequence=False)
        ta = a["flops"] / (a["ms"] * 1e-3) / 1e12
        res["pause_per_layer"] = {
            "workload": "the same event with K_l = the layer's quota pause tokens (64/128/256)",
            "ms_per_event": a["ms"], "blocks_per_s": a["B"] * 1e3 / a["ms"],
            "tflop_per_event": a["flops"] / 1e12, "achieved_tflops": ta,
            "frac": ta / BF16_PEAK_TFLOPS}
    return res


def blockmask_visible_keys(P: int, G: int, C: int, Kp: int, q: int, compress: bool = True):
    """Keys each token of a training-order sequence attends to under the block
    mask, summed over the sequence (compression off: causal, T(T+1)/2)."""
    if not compress:
        T = P + G
        return T * (T + 1) // 2
    tot = P * (P + 1) // 2
    nb = G // C
    for blk in range((G + C - 1) // C):
        n = min(C, G - blk * C)
        base = P + blk * q
        tot += n * base + n * (n + 1) // 2           # text: prefix + causal in block
        if blk < nb:
            tot += Kp * (base + C) + Kp * (Kp + 1) // 2  # pause: prefix + block + causal
    return tot


def run_prefill(args, torch, abk):
    """Block-mask prefill at the Fig. 9 shape: one sequence of 16,384 text
    tokens after a 256-token prompt, C = 512, K = 256 pause tokens per block,
    every one of the 36 layers (its own quota); the same kernel with
    compression off (plain causal attention over the same text) beside it,
    and the same text at C = 256 (K = 128, every quota halved: 4:1 as well),
    the block size Fig. 9 reports as costlier from partly filled tiles."""
    P, G = 256, 16384
    bf = torch.bfloat16

    def forward(Cb, Kp, quotas, comp):
        """ms per 36-layer forward (mean of two after a warmup), flops, rows"""
        pool = abk.Pool(num_layers=L, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_tokens=Cb,
                        num_pause=Kp, layer_quota=quotas.tolist(), page_rows=PR, max_seqs=1,
                        pool_bytes=2 * HKV * PR * D * 2 * 16, max_position=P + G, dtype="bf16",
                        rope_base=1e6, compress=comp)
        T = P + G + ((G // Cb) * Kp if comp else 0)
        gen = torch.Generator(device="cuda")
        gen.manual_seed(5)
        q = torch.randn((T, HQ, D), device="cuda", dtype=bf, generator=gen)
        k = torch.randn((T, HKV, D), device="cuda", dtype=bf, generator=gen)
        v = torch.randn((T, HKV, D), device="cuda", dtype=bf, generator=gen)
        out = torch.empty((T, HQ, D), device="cuda", dtype=bf)
        lse = torch.empty((T, HQ), device="cuda", dtype=torch.float32)
        times = []
        for rep in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for l in range(L):
                pool.blockmask_attention(l, P, G, q, k, v, out, lse)
            e1.record()
            torch.cuda.synchronize()
            if rep > 0:
                times.append(e0.elapsed_time(e1))
        pool.close()
        del q, k, v, out, lse
        keys = sum(blockmask_visible_keys(P, G, Cb, Kp, int(qq), comp) for qq in quotas)
        return float(np.mean(times)), 4.0 * D * HQ * keys, T

    quotas = layer_quotas(2)
    ms, flops, T = forward(C, 256, quotas, True)
    ms_c, flops_c = float("nan"), float("nan")
    if not args.no_prefill_causal:
        ms_c, flops_c, _ = forward(C, 256, quotas, False)
    b256 = None
    if not args.no_prefill_c256:
        ms_b, flops_b, T_b = forward(256, 128, quotas // 2, True)
        tf_b = flops_b / (ms_b * 1e-3) / 1e12
        b256 = {"ms_per_forward": ms_b, "rows": T_b, "tflop_per_forward": flops_b / 1e12,
                "achieved_tflops": tf_b, "frac": tf_b / BF16_PEAK_TFLOPS, "time_vs_c512": ms_b / ms,
                "config": {"workload": "the same 256-token prompt + 16,384 text tokens at C = 256, "
                                       "K = 128 pause tokens per block, quotas 6x128/12x32/18x64 "
                                       "(4:1 mean quota), 36 layers"}}
    tflops = flops / (ms * 1e-3) / 1e12
    # algorithmic bytes per launch (one layer): q, out and lse of every row, k
    # and v of every row once
    nbytes = T * (2 * HQ * D * 2 + HQ * 4 + 2 * HKV * D * 2)
    return {
        "metric": "block-mask prefill (training-forward attention), 36 layers of one sequence",
        "ms_per_forward": ms, "rows": T, "tflop_per_forward": flops / 1e12,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / BF16_PEAK_TFLOPS,
                     # HBM bytes per launch (one layer), from the counters
                     "traffic": traffic_from_profiles("blockmask_attn_mfma", nbytes)},
        "causal_ms_per_forward": ms_c, "causal_tflop_per_forward": flops_c / 1e12,
        "causal_tflops": flops_c / (ms_c * 1e-3) / 1e12, "time_vs_causal": ms / ms_c,
        "block_size_256": b256,
        "config": {"workload": "Fig. 9 shape: 256-token prompt + 16,384 text tokens, C = 512, "
                               "K = 256 pause tokens per block (4:1 mean quota), 36 layers with "
                               "quotas 6x256/12x64/18x128; causal: the same kernel with "
                               "compression off over the 16,640 prompt + text tokens"},
    }


def serving_mix_admit(quotas, steps: int, compress: bool, pool_pages: int, seed: int = 4, by_quota=None):
    """Admit sequences (P ~ U[128, 512], G ~ U[1024, 32768], seeded) while the
    pool holds each one's largest footprint over the run: its persistent rows
    after the blocks it completes during the run, plus a whole open block per
    layer (compressed before its pages are freed), or in full-KV mode all its
    rows at the end. Both modes draw the same sequence stream. by_quota (a
    dict, optional) receives the admitted footprint's pages per quota value."""
    rng = np.random.default_rng(seed)
    Ps, Gs, used = [], [], 0
    while True:
        P = int(rng.integers(128, 512, endpoint=True))
        G = int(rng.integers(1024, 32768, endpoint=True))
        if compress:
            nb_end = (G + steps - 1) // C
            need = int(sum(-(-(P + nb_end * int(q)) // PR) + C // PR for q in quotas))
        else:
            need = L * (-(-(P + G + steps) // PR))
        if used + need > pool_pages:
            break
        Ps.append(P)
        Gs.append(G)
        used += need
        if by_quota is not None and compress:
            for q in quotas:
                by_quota[int(q)] = by_quota.get(int(q), 0) + -(-(P + ((G + steps - 1) // C) * int(q)) // PR) + C // PR
    return np.array(Ps, dtype=np.int64), np.array(Gs, dtype=np.int64), used


def budget_pool_split(by_quota: dict, pool_pages: int):
    """Pages of one pool per budget level (quota value, ascending): each level's
    admitted footprint plus the free rest shared in proportion to it."""
    qs = sorted(by_quota)
    used = sum(by_quota.values())
    rest = pool_pages - used
    pages = [by_quota[q] + rest * by_quota[q] // used for q in qs]
    return qs, pages


def traced_sequence(G, warm: int) -> int:
    """Index of the sequence whose block completes first at or after step
    `warm` (in step t a sequence with G generated tokens before the first step
    compresses when G + t is a multiple of C)."""
    return int(np.argmin([(-(int(x) + warm)) % C for x in G]))


def run_serving_mix(args, torch, abk, compress: bool):
    """The saturated serving mix: a 200 GiB pool filled with as many sequences
    as fit, then `steps` decode steps of all of them (one fused append + decode
    call per layer); a sequence whose block completes is compressed at every
    layer and freed inside the step. Full-KV mode runs the same kernels with
    compression off. With args.budget_pools (AbridgeKV mode), the pages form one
    pool per budget level, sized by the admitted sequences' needs."""
    steps, warm = args.serving_mix_steps, 2
    quotas = layer_quotas(2)
    Kp = int(quotas.max())
    page_bytes = HKV * PR * D * 2
    pool_bytes = 200 << 30
    pool_pages = pool_bytes // (2 * page_bytes)
    by_quota = {}
    P, G, used = serving_mix_admit(quotas, steps + warm, compress, pool_pages, by_quota=by_quota)
    B = len(P)
    split = budget_pool_split(by_quota, pool_pages) if (compress and args.budget_pools) else None
    pool = abk.Pool(num_layers=L, num_q_heads=HQ, num_kv_heads=HKV, head_dim=D, block_tokens=C,
                    num_pause=Kp, layer_quota=quotas.tolist(), page_rows=PR, max_seqs=B,
                    pool_bytes=pool_bytes, max_position=33792, dtype="bf16", rope_base=1e6,
                    compress=compress, budget_pool_pages=split[1] if split else None)
    sids = []
    for i in range(B):
        s = pool.seq_create(int(P[i]))
        pool.synth_fill(s, int(G[i]), 4 * 1000003 + i * 7919 + 17)
        sids.append(s)
    torch.cuda.synchronize()
    print(f"[bench] serving mix ({'AbridgeKV' if compress else 'full KV'}): {B} sequences, "
          f"{used} of {pool_pages} pages at their largest", file=sys.stderr, flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    bf = torch.bfloat16
    nsets = 2  # step inputs alternate between two random sets (values do not affect timing)
    q_in = torch.randn((nsets, L, B, HQ, D), device="cuda", dtype=bf, generator=gen)
    k_in = torch.randn((nsets, L, B, HKV, D), device="cuda", dtype=bf, generator=gen)
    v_in = torch.randn((nsets, L, B, HKV, D), device="cuda", dtype=bf, generator=gen)
    g = G.copy()
    nb = (g - 1) // C if compress else np.zeros_like(g)
    full_max = 1
    if compress:
        for t in range(steps + warm):
            full_max = max(full_max, int(np.sum((g + t) - ((g + t - 1) // C) * C == C)))
    qp = torch.randn((full_max, Kp, HQ, D), device="cuda", dtype=bf, generator=gen)
    kp = torch.randn((full_max, Kp, HKV, D), device="cuda", dtype=bf, generator=gen)
    vp = torch.randn((full_max, Kp, HKV, D), device="cuda", dtype=bf, generator=gen)
    cout = torch.empty((full_max, Kp, HQ, D), device="cuda", dtype=bf)
    clse = torch.empty((full_max, Kp, HQ), device="cuda", dtype=torch.float32)
    out = torch.empty((B, HQ, D), device="cuda", dtype=bf)
    lse = torch.empty((B, HQ), device="cuda", dtype=torch.float32)
    views = [[(q_in[t, l], k_in[t, l], v_in[t, l]) for l in range(L)] for t in range(nsets)]
    stats = {"compressions": 0, "rows": 0}
    # occupancy trace (host bookkeeping only, no GPU synchronisation): one
    # sequence's resident K/V summed over layers after every timed step, and
    # the pool's pages by budget class (layers keeping 64 / 128 / 256 rows per
    # block) every 32 steps. The traced sequence is the one whose block
    # completes earliest in the timed steps (in step t a sequence compresses
    # when G + t is a multiple of C), so that its drop falls inside the trace.
    row_bytes = 2 * HKV * D * 2
    ti = traced_sequence(G, warm + 1)  # a drop after the first timed step shows in the trace
    trace = {"sequence": ti, "seq_kv_mb": [], "seq_generated": [], "budget_steps": [],
             "pages_by_quota": {str(q): [] for q in sorted(set(quotas.tolist()))}, "pages_used": [],
             # a compression step: each layer's C open rows become q_l code rows,
             # then the step's token adds one row per layer
             "drop_closed_form_mb": round(sum(C - int(q) - 1 for q in quotas) * row_bytes / 1e6, 3)
             if compress else None}

    def record(t):
        rows = sum(pool.seq_query(sids[ti], l)["resident_rows"] for l in range(L))
        trace["seq_kv_mb"].append(round(rows * row_bytes / 1e6, 3))
        trace["seq_generated"].append(int(g[ti]))
        if t % 32 == 0:
            by = {q: 0 for q in trace["pages_by_quota"]}
            if split:
                # each budget pool's own count
                for x in pool.budget_stats():
                    by[str(x["quota"])] = x["pages_used"]
            else:
                for s in sids:
                    for l in range(L):
                        by[str(int(quotas[l]))] += pool.seq_query(s, l)["n_pages"]
            trace["budget_steps"].append(t)
            for q in by:
                trace["pages_by_quota"][q].append(by[q])
            trace["pages_used"].append(pool.stats()["pages_used"])

    def step(t, count):
        if compress:
            full = [i for i in range(B) if g[i] - nb[i] * C == C]
            if full:
                ids = [sids[i] for i in full]
                m = len(ids)
                for l in range(L):
                    pool.compress_block(l, ids, qp[:m], kp[:m], vp[:m], cout[:m], clse[:m])
                pool.free_block(ids)
                for i in full:
                    nb[i] += 1
                if count:
                    stats["compressions"] += m
        if count:
            # resident rows the step's decode reads (the current token included)
            stats["rows"] += int(sum(resident_rows(P, g + 1, int(q), compress).sum() for q in quotas))
        for l in range(L):
            q, k, v = views[t % nsets][l]
            pool.append_decode(l, sids, k, v, q, out, lse)
        g[:] += 1

    for t in range(warm):
        step(t, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(steps):
        step(warm + t, True)
        record(t)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    st = pool.stats()
    budget = pool.budget_stats() if split else None
    pool.close()
    del q_in, k_in, v_in
    torch.cuda.empty_cache()
    if budget:
        for x, n in zip(budget, split[1]):
            x["pages"] = n
    return {"sequences_resident": B, "tokens_per_s": B * steps / dt, "ms_per_step": 1e3 * dt / steps,
            "budget_pools": budget,
            "steps": steps, "compressions_in_timed_steps": stats["compressions"],
            "decode_kv_gb_per_step": stats["rows"] * row_bytes / steps / 1e9,
            "kv_gbps_incl_compression": stats["rows"] * row_bytes / dt / 1e9,
            "pool_pages_used_at_end": st["pages_used"], "pool_pages": int(pool_pages),
            "occupancy_trace": trace}


def occupancy_summary(tr: dict) -> dict:
    """The traced sequence's resident K/V per timed step (MB, one decimal) and
    the steps where it drops, beside the closed-form drop of one compression."""
    kv = tr["seq_kv_mb"]
    drops = [{"step": t, "generated": tr["seq_generated"][t], "from_mb": kv[t - 1], "to_mb": kv[t]}
             for t in range(1, len(kv)) if kv[t] < kv[t - 1]]
    return {"sequence": tr["sequence"], "generated_at_first_step": tr["seq_generated"][0] if kv else None,
            "kv_mb": [round(x, 1) for x in kv], "drops": drops,
            "drop_closed_form_mb": tr["drop_closed_form_mb"]}


def serving_mix_leg(a: dict, f: dict) -> dict:
    """The serving mix's two modes as the default bench line reports them, each
    with its traced sequence's occupancy (the pool's per-budget page counts
    are left to the long form)."""
    keys = ("sequences_resident", "tokens_per_s", "ms_per_step", "steps", "compressions_in_timed_steps",
            "decode_kv_gb_per_step", "kv_gbps_incl_compression", "pool_pages_used_at_end", "pool_pages")
    return {"metric": "serving mix: decode tokens/s and sequences resident, AbridgeKV vs full KV",
            "unit": "tokens/s",
            "config": {"workload": "saturated serving mix: 200 GiB paged pool, 36 layers, quotas "
                                   "6x256/12x64/18x128, P ~ U[128,512], G ~ U[1024,32768], one fused "
                                   "append+decode call per layer per step, compress+free at block "
                                   "boundaries inside the steps; full KV: the same kernels, compression off"},
            "abridgekv": {**{k: a[k] for k in keys}, "occupancy": occupancy_summary(a["occupancy_trace"])},
            "full_kv": {**{k: f[k] for k in keys}, "occupancy": occupancy_summary(f["occupancy_trace"])},
            "tokens_per_s_ratio": a["tokens_per_s"] / f["tokens_per_s"],
            "sequences_ratio": a["sequences_resident"] / f["sequences_resident"]}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(workload, budget_s: float):
    """The CPU oracle as it stands, on a bounded sample of the decode step:
    (sequence, layer) pairs until the time budget is spent; cost scales with
    resident rows, so the whole step's time is extrapolated by rows. Timed
    with every host thread, then on one thread for a third of the budget."""
    import oracle
    import synth
    from oracle import TEXT, LayerView
    quotas, P, G = workload
    B = len(P)
    # (sequence, layer) pairs in a seeded order: the oracle decodes them one by
    # one until it has spent the budget
    pairs = [(si, l) for si in range(B) for l in range(L)]
    order = np.random.default_rng(12345).permutation(len(pairs))
    pairs = [pairs[k] for k in order]

    def sample(budget):
        sampled_rows, secs, npairs = 0, 0.0, 0
        for si, l in pairs:
            Lv = LayerView(int(P[si]), C, int(quotas.max()), int(quotas[l]))
            g, nb = int(G[si]), (int(G[si]) - 1) // C
            seed = 2 * 1000003 + si * 7919 + 17
            # inputs of the rows the mask shows (generation is not timed)
            kind, ka, kb, _ = oracle.visible_keys(Lv, g, nb, (TEXT, g - 1, 0))
            rows = {}
            for which, w in (("k", synth.WHICH_K), ("v", synth.WHICH_V)):
                out = np.empty((len(kind), HKV, D))
                for kd in (0, 1, 2):
                    m = kind == kd
                    if m.any():
                        out[m] = synth.rows(seed, l, kd, ka[m], kb[m], w, HKV, D, "bf16")
                rows[which] = out

            def fetch(kind_, a_, b_, which, rows=rows):
                return rows[which]

            q = synth.rows(seed, l, TEXT, [g - 1], 0, synth.WHICH_Q, HQ, D, "bf16")[0]
            t0 = time.perf_counter()
            _, _, keys = oracle.decode(Lv, g, nb, q, fetch, oracle.BF16, 1e6)
            secs += time.perf_counter() - t0
            sampled_rows += len(keys[0])
            npairs += 1
            if secs > budget:
                break
        return sampled_rows, secs, npairs

    total_rows = sum(int(resident_rows(P, G, quotas[l]).sum()) for l in range(L))
    threads = oracle.num_threads()
    sampled_rows, secs, npairs = sample(budget_s)
    oracle.set_num_threads(1)
    rows1, secs1, npairs1 = sample(budget_s / 3)
    oracle.set_num_threads(threads)
    return {"value": B / (secs * total_rows / sampled_rows), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{npairs} (sequence, layer) pairs of the step in a seeded random order "
                      f"({sampled_rows} resident rows, {secs:.2f} s of oracle time); "
                      f"extrapolated by rows to the 22-sequence 36-layer step ({total_rows} rows)",
            "single_core_value": B / (secs1 * total_rows / rows1),
            "single_core_sample": f"the first {npairs1} pairs of the same order on one thread "
                                  f"({rows1} rows, {secs1:.2f} s)",
            "cpu_model": _cpu_model()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--split-rows", type=int, default=0, help="rows per split-KV work item (0: library default)")
    ap.add_argument("--per-head", action="store_true",
                    help="decode step with quotas per (layer, KV head) of the same layer totals")
    ap.add_argument("--no-per-head", action="store_true",
                    help="skip the per-head decode step reported beside the main line")
    ap.add_argument("--separate-append", action="store_true",
                    help="append and decode as two calls per layer (default: abk_append_decode)")
    ap.add_argument("--compress-reps", type=int, default=2)
    ap.add_argument("--no-pause-per-layer", action="store_true",
                    help="skip the compression event with K_l = quota pause tokens per layer")
    ap.add_argument("--no-compress", action="store_true",
                    help="skip the compression event and the one-layer decode call (the decode "
                         "step alone, as the decode profile runs it)")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-prefill-c256", action="store_true",
                    help="skip the prefill leg at block size C = 256")
    ap.add_argument("--no-prefill-causal", action="store_true",
                    help="skip the plain-causal comparison of the prefill (profiled runs)")
    ap.add_argument("--no-single-sequence", action="store_true",
                    help="skip the single-sequence compression latency (profiled runs of the event)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--serving-mix", action="store_true",
                    help="only run the saturated serving mix (200 GiB pool, AbridgeKV and full KV)")
    ap.add_argument("--serving-mix-steps", type=int, default=512)
    ap.add_argument("--mix-steps", type=int, default=64,
                    help="steps of each mode of the serving-mix leg of the default run (0: skip it)")
    ap.add_argument("--budget-pools", action="store_true",
                    help="serving mix: one page pool per budget level (AbridgeKV mode)")
    ap.add_argument("--profile-summary", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 runs under DIR (no GPU needed)")
    args = ap.parse_args()
    if args.profile_summary:
        profile_summary(args.profile_summary)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration_mib:
        # a plain copy of known size: reads and writes exactly n bytes each
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    import long_reasoning_kv_amd as abk
    if args.serving_mix:
        mix = {"abridgekv": run_serving_mix(args, torch, abk, True),
               "full_kv": run_serving_mix(args, torch, abk, False)}
        a, f = mix["abridgekv"], mix["full_kv"]
        print(json.dumps({
            "metric": "serving mix: decode tokens/s and sequences resident, AbridgeKV vs full KV",
            "unit": "tokens/s", "n_gpus": 1, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "saturated serving mix: 200 GiB paged pool, 36 layers, quotas "
                                   "6x256/12x64/18x128, P ~ U[128,512], G ~ U[1024,32768], one fused "
                                   "append+decode call per layer per step, compress+free at block "
                                   "boundaries inside the steps"},
            "abridgekv": a, "full_kv": f,
            "tokens_per_s_ratio": a["tokens_per_s"] / f["tokens_per_s"],
            "sequences_ratio": a["sequences_resident"] / f["sequences_resident"]}), flush=True)
        return
    print(f"[bench] decode workload: 36 layers, 22 sequences, {args.warmup}+{args.steps} steps",
          file=sys.stderr, flush=True)
    res, workload = run_decode(args, torch, abk)
    per_head = None
    if not args.per_head and not args.no_per_head:
        # the same step with quotas per (layer, KV head) of the same layer totals
        print("[bench] decode step with per-head quotas", file=sys.stderr, flush=True)
        ph, _ = run_decode(argparse.Namespace(**{**vars(args), "per_head": True}), torch, abk)
        per_head = {"metric": "decode tokens/s with quotas per (layer, KV head)", "value": ph["value"],
                    "unit": "tokens/s", "ms_per_step": ph["ms_per_step"],
                    "vs_per_layer": ph["value"] / res["value"],
                    "avg_launch_us": ph["roofline"]["avg_launch_us"],
                    "hbm_gbps": ph["roofline"]["achieved"],
                    "config": {"workload": ph["config"]["workload"], "quotas": ph["config"]["quotas"],
                               "resident_kv_gb": ph["config"]["resident_kv_gb"]}}
    one = None
    if not args.no_compress:
        print("[bench] one-layer decode call: 16 sequences, 2,396 rows each", file=sys.stderr, flush=True)
        one = run_decode_1layer(args, torch, abk)
    comp = None
    if not args.no_compress:
        print("[bench] compression event: 64 sequences x 36 layers", file=sys.stderr, flush=True)
        comp = run_compress(args, torch, abk)
    pre = None
    if not args.no_prefill:
        print("[bench] block-mask prefill: 16K text tokens, 36 layers", file=sys.stderr, flush=True)
        pre = run_prefill(args, torch, abk)
    mix = None
    if args.mix_steps > 0:
        print(f"[bench] serving mix: 200 GiB pool, {args.mix_steps} steps per mode", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()  # the earlier legs' cached blocks: the pool takes 200 GiB
        margs = argparse.Namespace(**{**vars(args), "serving_mix_steps": args.mix_steps})
        mix = serving_mix_leg(run_serving_mix(margs, torch, abk, True), run_serving_mix(margs, torch, abk, False))
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline (bounded sample)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(workload, args.cpu_budget_s)
    line = {
        "metric": METRIC, "value": res["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": res["config"], "hbm_gbps": res["hbm_gbps"],
        "ms_per_step_with_events": res["ms_per_step_with_events"],
        "decode_ms_per_step": res["decode_ms_per_step"],
        "compress_ms_in_event_steps": res["compress_ms_in_event_steps"],
        "blocks_compressed": res["blocks_compressed"],
        "with_compression_amortized": res["with_compression_amortized"],
        "roofline": res["roofline"], "cpu_baseline": cpu, "compress": comp, "prefill": pre,
        "per_head": per_head, "decode_1layer": one, "serving_mix": mix,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
