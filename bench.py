#!/usr/bin/env python3
"""Benchmark of the DSA layer hot path on one MI355X.

A step is one dsa_forward (lightning indexer -> top-k -> sparse MQA-mode MLA)
over a decode batch of 64 sequences at 131072 tokens of context, k = 2048,
inputs (FP8 index-key cache, bf16 latent cache, queries) already resident in
HBM.  Prints one JSON line: decode queries/s, with the indexer's roofline
(HBM-bound; stage time from HIP events recorded on the library's stream inside
the timed region) and the CPU oracle timed on a bounded sample of the same
workload.  Per-stage figures and a causal-prefill measurement (16384 tokens)
ride along under "stages" and "prefill".

    python bench.py [--steps K] [--warmup W]
                    [--workload decode|prefill|decode1x4k|decode16x32k|ragged|crossover|kl]
                    [--no-prefill] [--no-configs] [--no-cpu-baseline] [--cpu-sample N] [--copy-calib]

The default line also carries, under "configs", the other decode workloads:
one query over 4096 positions (microseconds per call), 16 sequences of 32768
(planted keys) and the ragged paged batch of 128 sequences (log-uniform lengths
1024..131072, 64-token blocks in a random physical order) beside the same
lengths in contiguous caches; and, under "prefill", the 16384-token causal
prefill with its own sampled CPU-oracle baseline.  --workload <name> makes one
of them the measured line (used to profile it on its own).  --copy-calib runs,
after the timed steps, a plain 1 GiB device-to-device elementwise copy whose
HBM counter readings give the scale for the counter-based traffic figure.
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA, published
FP8_PEAK_TFLOPS = 5000.0       # dense fp8 MFMA, published
IDX_BYTES_PER_KEY = 128 + 4 + 4  # FP8 key row + key scale read, fp32 score written
CALIB_BYTES = 1 << 30           # size of the calibration copy (read and written)

# HBM traffic of one indexer launch on the decode workload, from two rocprofv3
# --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
# same counter reads for the 1 GiB calibration copy.  Valid only for the kernel
# source it was measured on: the figure is dropped when indexer.hip changes.
INDEXER_TRAFFIC = {
    "source_sha": "c6c67e20879b8327",
    "fetch_kib": 543112, "write_kib": 35887,          # raw counter readings
    "calib_fetch_kib": 524295, "calib_write_kib": 1048576,  # the 1 GiB copy
    "bytes_per_launch": (543112 * 2 + 35887) * 1024,
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sparse_long_context_dsa_amd", "csrc", name)
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def calibration_copy(reps=3):
    """A plain elementwise copy of CALIB_BYTES, for scaling HBM counters."""
    n = CALIB_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def indexer_units(nvis, k):
    """Keys scored in one launch (queries with n_vis <= k are bypassed)."""
    return int(sum(int(n) for n in nvis if n > k))


def mla_work(counts):
    rows = int(sum(int(c) for c in counts))
    flops = rows * 128 * (576 + 512) * 2
    gather = rows * 1152
    return rows, flops, gather


def decode_bytes(wl):
    """Algorithmic bytes (and the attention's flops) of one dsa_forward on a
    decode-style workload: the indexer reads each scored key row (128 B), its
    scale (4 B) and writes its score (4 B), plus q, w and q_scale per scored
    query; the top-k reads the scores and writes k positions per query; the
    attention gathers 1152 B per selected row and reads q (144 KiB), writes
    out (256 KiB) and reads k positions per query."""
    nv = wl.q_nvis.cpu().numpy()
    k = wl.k
    units = indexer_units(nv, k)
    scored = int((nv > k).sum())
    rows, flops, gather = mla_work(np.minimum(nv, k))
    return {"indexer": units * IDX_BYTES_PER_KEY + scored * (64 * 128 + 64 * 8),
            "topk": units * 4 + wl.nq * k * 4,
            "mla": gather + wl.nq * (128 * 576 * 2 + 128 * 512 * 4 + k * 4),
            "mla_flops": flops, "mla_gather": gather, "keys_scored": units, "rows_attended": rows}


def planted_in_topk(wl, idx):
    """How many of each sequence's planted key positions the forward selected
    (decode: query i is sequence i)."""
    if not wl.planted:
        return None
    idx_h = idx.cpu().numpy()
    q_seq = wl.q_seq.cpu().numpy()
    hits, per_seq = [], []
    for s, pos in sorted(wl.planted.items()):
        qi = int(np.nonzero(q_seq == s)[0][-1])
        sel = idx_h[qi][idx_h[qi] >= 0]
        hits.append(int(np.isin(pos, sel).sum()))
        per_seq.append(len(pos))
    hits = np.asarray(hits)
    return {"planted_per_sequence": int(np.max(per_seq)), "selected_per_sequence_mean": float(hits.mean()),
            "selected_min": int(hits.min()), "selected_max": int(hits.max()),
            "share_of_planted_selected": float(hits.sum() / max(1, int(np.sum(per_seq)))),
            "share_of_topk_that_is_planted": float(hits.mean() / wl.k)}


def flush_caches(buf):
    """Evicts L2 and the 256 MB Infinity Cache: writes a 1 GiB buffer."""
    buf.fill_(1.0)


def prepare(wl):
    import sparse_long_context_dsa_amd as dsa
    nq, rows = wl.nq, wl.rows
    q8 = torch.empty((nq, 64, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((nq, 64), dtype=torch.float32, device="cuda")
    k8 = torch.empty((rows, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty((rows,), dtype=torch.float32, device="cuda")
    dsa.dsa_quantize_fp8(wl.q_idx.view(nq * 64, 128), q8.view(nq * 64, 128), qs.view(nq * 64))
    dsa.dsa_quantize_fp8(wl.k_idx, k8, ks)
    queries = dsa.Queries(wl.q_seq, wl.q_nvis, wl.max_nvis)
    if wl.block_size:
        layout = dsa.KvLayout(wl.num_seqs, rows, block_table=wl.block_table, block_size=wl.block_size)
    else:
        layout = dsa.KvLayout(wl.num_seqs, rows, seq_row0=wl.row0)
    out = torch.empty((nq, 128, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((nq, 128), dtype=torch.float32, device="cuda")
    idx = torch.empty((nq, wl.k), dtype=torch.int32, device="cuda")
    ws = dsa.workspace(dsa.DSA_OP_FORWARD, queries, wl.k)
    return dict(q8=q8, qs=qs, k8=k8, ks=ks, queries=queries, layout=layout, out=out, lse=lse, idx=idx, ws=ws)


def time_forward(wl, p, steps, warmup):
    """Times `steps` dsa_forward steps twice, after `warmup` untimed ones.

    The first pass is the measurement: plain dsa_forward calls, bracketed by a
    synchronize on both sides; it gives the wall time.  The second pass runs
    the same steps through dsa_forward_profiled, which records HIP events on
    the library's stream between the stages; it gives the per-stage times.
    The event records themselves idle the GPU for a few microseconds each, so
    they stay out of the first pass.

    Returns (wall seconds of the first pass, per-stage mean ms, wall seconds
    of the second pass)."""
    import sparse_long_context_dsa_amd as dsa

    def step(ev=None):
        dsa.dsa_forward(p["queries"], p["layout"], p["q8"], p["qs"], wl.w, p["k8"], p["ks"], wl.q_mla, wl.kv,
                        wl.k, wl.softmax_scale, p["out"], p["lse"], p["idx"], ws=p["ws"], events=ev)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    # Five events per step: before the first kernel, before the indexer (after
    # the top-k's histogram clear), after the indexer, after the top-k, after
    # the attention; the top-k stage is the clear plus the selection.
    E = 5
    ev = dsa.HipEvents(E * steps)
    ptr = ctypes.sizeof(ctypes.c_void_p)
    base = ctypes.addressof(ev.handles)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step((ctypes.c_void_p * E).from_address(base + E * i * ptr))
    torch.cuda.synchronize()
    wall_ev = time.perf_counter() - t0
    st = {"indexer": [], "topk": [], "mla": []}
    for i in range(steps):
        b = E * i
        st["indexer"].append(ev.elapsed_ms(b + 1, b + 2))
        st["topk"].append(ev.elapsed_ms(b, b + 1) + ev.elapsed_ms(b + 2, b + 3))
        st["mla"].append(ev.elapsed_ms(b + 3, b + 4))
    ev.close()
    return wall, {k: float(np.mean(v)) for k, v in st.items()}, wall_ev


def time_forward_cold(wl, p, steps):
    """Mean ms of one dsa_forward with L2 and the Infinity Cache flushed before
    each step: torch events around each step on the stream the library
    launches on (the current stream), the flush outside them."""
    import sparse_long_context_dsa_amd as dsa
    buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        flush_caches(buf)
        e0.record()
        dsa.dsa_forward(p["queries"], p["layout"], p["q8"], p["qs"], wl.w, p["k8"], p["ks"], wl.q_mla, wl.kv,
                        wl.k, wl.softmax_scale, p["out"], p["lse"], p["idx"], ws=p["ws"])
        e1.record()
    torch.cuda.synchronize()
    ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    del buf
    return ms


def measure_decode(wl, steps, warmup, cold=False):
    """One decode workload: warm steps (wall clock, then HIP events between
    the stages), optionally cold steps, the HBM fractions of each stage and of
    the whole step, and the planted-key diagnostic."""
    p = prepare(wl)
    torch.cuda.synchronize()
    wall, st, wall_ev = time_forward(wl, p, steps, warmup)
    b = decode_bytes(wl)
    ms = 1e3 * wall / steps
    total = b["indexer"] + b["topk"] + b["mla"]
    res = {
        "workload": wl.name, "batch": wl.nq, "context_max": int(wl.q_nvis.max().item()),
        "context_mean": float(wl.q_nvis.float().mean().item()), "k": wl.k,
        "paged_block_size": wl.block_size or None,
        "queries_per_s": wl.nq * steps / wall, "ms_per_step": ms, "us_per_step": 1e3 * ms,
        "events_pass_ms_per_step": 1e3 * wall_ev / steps,
        "indexer_ms": st["indexer"], "topk_ms": st["topk"], "mla_ms": st["mla"],
        "algorithmic_bytes": {kk: b[kk] for kk in ("indexer", "topk", "mla")},
        "step_gbs": total / (ms * 1e-3) / 1e9, "step_frac_hbm": total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline_queries_per_s": wl.nq / (total / (HBM_PEAK_GBS * 1e9)),
        "mla_tflops_bf16": b["mla_flops"] / (st["mla"] * 1e-3) / 1e12,
    }
    for stage in ("indexer", "topk", "mla"):
        if st[stage] > 0 and b[stage] > 0:
            res[f"{stage}_frac_hbm"] = b[stage] / (st[stage] * 1e-3) / 1e9 / HBM_PEAK_GBS
    if cold:
        cms = time_forward_cold(wl, p, steps)
        res["cold_ms_per_step"] = cms
        res["cold_us_per_step"] = 1e3 * cms
        res["cold_queries_per_s"] = wl.nq / (cms * 1e-3)
    res["planted"] = planted_in_topk(wl, p["idx"])
    del p
    torch.cuda.empty_cache()
    return res


def extra_decode_configs(steps, warmup):
    """The decode workloads beside the headline: 1 x 4096 (latency), 16 x 32768
    (planted) and the ragged paged batch, the latter also with the same
    lengths in contiguous caches (the cost of paging)."""
    from workloads import make_config, make_custom
    out = {}
    for cfg, key, cold in ((0, "decode_1x4096", True), (1, "decode_16x32768_planted", True),
                           (4, "ragged_paged_128", True)):
        log(f"config: {key}")
        wl = make_config(cfg, device="cuda")
        out[key] = measure_decode(wl, steps, warmup, cold=cold)
        if cfg == 4:
            lens = wl.seq_len.tolist()
            del wl
            torch.cuda.empty_cache()
            log("config: the same ragged lengths, contiguous caches")
            wl = make_custom(seq_lens=lens, device="cuda", seed=20260004, name="ragged contiguous 128")
            c = measure_decode(wl, steps, warmup, cold=True)
            out["ragged_contiguous_128"] = c
            pg = out[key]
            out[key]["paging_cost"] = {"warm": pg["ms_per_step"] / c["ms_per_step"] - 1.0,
                                       "cold": pg["cold_ms_per_step"] / c["cold_ms_per_step"] - 1.0}
        del wl
        torch.cuda.empty_cache()
    return out


def key_scale_formats(wl, p, steps):
    """The standalone indexer (no histogram) on the same workload with fp32 key
    scales and with E8M0 key scales (one byte per key, from
    dsa_quantize_fp8_e8m0): mean launch time over `steps` launches, each between
    torch CUDA events on the stream the library launches on."""
    import sparse_long_context_dsa_amd as dsa
    nq, rows = wl.nq, wl.rows
    k8e = torch.empty((rows, 128), dtype=torch.uint8, device="cuda")
    kb = torch.empty((rows,), dtype=torch.uint8, device="cuda")
    dsa.dsa_quantize_fp8_e8m0(wl.k_idx, k8e, kb)
    ld = (wl.max_nvis + 63) // 64 * 64
    scores = torch.empty((nq, ld), dtype=torch.float32, device="cuda")
    units = indexer_units(wl.q_nvis.cpu().numpy(), -1)
    res = {}
    for name, call, per_key in (
            ("fp32_key_scales", lambda: dsa.dsa_indexer_scores(p["queries"], p["layout"], p["q8"], p["qs"], wl.w,
                                                               p["k8"], p["ks"], scores), 128 + 4 + 4),
            ("e8m0_key_scales", lambda: dsa.dsa_indexer_scores_e8m0(p["queries"], p["layout"], p["q8"], p["qs"],
                                                                    wl.w, k8e, kb, scores), 128 + 1 + 4)):
        for _ in range(3):
            call()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record()
            call()
            e1.record()
        torch.cuda.synchronize()
        ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
        nbytes = units * per_key + nq * (64 * 128 + 64 * 8)
        res[name] = {"us": 1e3 * ms, "bytes_per_launch": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
                     "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del k8e, kb, scores
    return res


def cpu_baseline(wl, sample, k):
    """The oracle (NumPy float64) on the first `sample` queries of the workload.
    Its inputs (FP8 codes from its own quantiser, bf16 rows) are prepared
    outside the timed region, as the GPU's are."""
    import oracle
    from oracle.bf16 import bf16_decode  # noqa: F401  (same package, decoding happens inside the timed calls)
    qseq = wl.q_seq.cpu().numpy()
    nv = wl.q_nvis.cpu().numpy()
    row0 = wl.row0.cpu().numpy() if wl.row0 is not None else None
    bt = wl.block_table.cpu().numpy() if wl.block_table is not None else None
    inputs = []
    for i in range(sample):
        rows = oracle.phys_rows(int(qseq[i]), np.arange(int(nv[i])), row0=row0, block_table=bt,
                                block_size=wl.block_size)
        rt = torch.from_numpy(rows).cuda()
        q8, qs = oracle.quantize_rows(wl.q_idx[i].cpu().numpy())
        k8, ks = oracle.quantize_rows(wl.k_idx[rt].cpu().numpy())
        kv = wl.kv[rt].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        qm = wl.q_mla[i].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        inputs.append((q8, qs, wl.w[i].cpu().numpy(), k8, ks, qm, kv))
        log(f"cpu baseline: prepared query {i + 1}/{sample}")
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    for (q8, qs, w, k8, ks, qm, kv) in inputs:
        oracle.forward_query(q8, qs, w, k8, ks, qm, kv, k, wl.softmax_scale)
    dt = time.perf_counter() - t0
    return {"value": sample / dt, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"first {sample} of the 64 decode queries at 131072 context (full indexer, top-k and "
                      f"attention per query), {dt:.1f} s"}


def prefill_cpu_baseline(wl, k, n_random=250, seed=5):
    """The oracle on a stratified sample of the causal prefill's queries: the
    positions t = 1, 2, 2048, 2049, 2050 and 16383 (0-based, n_vis = t) plus
    n_random seeded random positions, each a whole indexer -> top-k -> sparse
    attention query.  The full prefill's oracle time is extrapolated from the
    sample by flop share (indexer 2*64*128 flop per scored key, attention
    2*128*1088 flop per attended row) and reported as tokens/s, labelled as
    extrapolated.  Inputs are prepared outside the timed region."""
    import oracle
    nv = wl.q_nvis.cpu().numpy()
    n = wl.nq
    fixed = [t for t in (1, 2, 2048, 2049, 2050, n - 1) if t < n]
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(n), fixed)
    sample = sorted(set(fixed) | set(rng.choice(rest, min(n_random, rest.size), replace=False).tolist()))
    log(f"prefill cpu baseline: preparing {len(sample)} queries")
    k8_all, ks_all = oracle.quantize_rows(wl.k_idx.cpu().numpy())
    kv_all = wl.kv.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    row0 = int(wl.row0[0].item())

    def flops(t):
        t = int(t)
        return (2 * 64 * 128 * t if t > k else 0) + 2 * 128 * 1088 * min(k, t)

    inputs = []
    for i in sample:
        t = int(nv[i])
        q8, qs = oracle.quantize_rows(wl.q_idx[i].cpu().numpy())
        qm = wl.q_mla[i].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        inputs.append((q8, qs, wl.w[i].cpu().numpy(), k8_all[row0:row0 + t], ks_all[row0:row0 + t], qm,
                       kv_all[row0:row0 + t]))
    try:
        from threadpoolctl import threadpool_info
        cores = max([int(x.get("num_threads", 1)) for x in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    for args in inputs:
        oracle.forward_query(*args, k, wl.softmax_scale)
    dt = time.perf_counter() - t0
    share = sum(flops(nv[i]) for i in sample) / sum(flops(t) for t in nv)
    est = dt / share
    return {"value": n / est, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(sample)} of the {n} causal prefill queries (t = {fixed} and {len(sample) - len(fixed)} "
                      f"seeded random t; full indexer, top-k and attention per query) in {dt:.1f} s, "
                      f"extrapolated to the whole prefill by flop share ({share:.4f} of its flops): "
                      f"{est:.0f} s estimated"}


def run_prefill(steps, warmup, cpu=False):
    from workloads import make_config
    log("prefill: generating 16384-token causal workload")
    wl = make_config(3, device="cuda")
    p = prepare(wl)
    torch.cuda.synchronize()
    log("prefill: timing dsa_forward")
    wall, st, wall_ev = time_forward(wl, p, steps, warmup)
    nv = wl.q_nvis.cpu().numpy()
    cnt = np.minimum(nv, wl.k)
    pairs = indexer_units(nv, wl.k)
    idx_flops = pairs * 64 * 128 * 2
    rows, flops, gather = mla_work(cnt)
    res = {
        "workload": "prefill 16384 tokens, causal, k=2048",
        "ms_per_step": 1e3 * wall / steps,
        "tokens_per_s": wl.nq * steps / wall,
        "events_pass_ms_per_step": 1e3 * wall_ev / steps,
        "indexer_ms": st["indexer"], "topk_ms": st["topk"], "mla_ms": st["mla"],
        "indexer_tflops_fp8": idx_flops / (st["indexer"] * 1e-3) / 1e12,
        "indexer_frac_fp8_peak": idx_flops / (st["indexer"] * 1e-3) / 1e12 / FP8_PEAK_TFLOPS,
        "mla_tflops_bf16": flops / (st["mla"] * 1e-3) / 1e12,
        "mla_frac_bf16_peak": flops / (st["mla"] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        "mla_gather_gbs": gather / (st["mla"] * 1e-3) / 1e9,
        "topk_gbs": (pairs * 4 + wl.nq * wl.k * 4) / (st["topk"] * 1e-3) / 1e9 if st["topk"] > 0 else None,
    }
    del p
    torch.cuda.empty_cache()
    if cpu:
        log("prefill: timing the CPU oracle on a stratified sample")
        res["cpu_baseline"] = prefill_cpu_baseline(wl, wl.k)
    del wl
    return res


def common_fields(args):
    return {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "fp8+bf16", "data": "synthetic"}


def prefill_result(args):
    pf = run_prefill(args.steps, args.warmup, cpu=not args.no_cpu_baseline)
    mla_achieved = pf["mla_tflops_bf16"]
    result = {"metric": "DSA layer prefill tokens/s (16384-token causal sequence)",
              "value": pf["tokens_per_s"], "unit": "tokens/s"}
    result.update(common_fields(args))
    result.update({
        "ms_per_step": pf["ms_per_step"],
        "config": {"workload": pf["workload"], "tokens": 16384, "k": 2048, "indexer_heads": 64,
                   "indexer_dim": 128, "heads": 128, "latent": 576},
        "roofline": {"bound": "mfma", "kernel": "sparse_mla", "achieved": mla_achieved,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": mla_achieved / BF16_PEAK_TFLOPS,
                     "traffic": None},
        "stages": pf,
    })
    if "cpu_baseline" in pf:
        result["cpu_baseline"] = pf.pop("cpu_baseline")
    return result


def config_result(args, cfg, key):
    """One of the other decode workloads as the measured line."""
    from workloads import make_config
    log(f"config: {key}")
    wl = make_config(cfg, device="cuda")
    r = measure_decode(wl, args.steps, args.warmup, cold=True)
    result = {"metric": f"DSA layer decode queries/s ({r['workload']})", "value": r["queries_per_s"],
              "unit": "queries/s"}
    result.update(common_fields(args))
    result.update({
        "ms_per_step": r["ms_per_step"],
        "config": {"workload": r["workload"], "batch": r["batch"], "context": r["context_max"], "k": r["k"],
                   "indexer_heads": 64, "indexer_dim": 128, "heads": 128, "latent": 576},
        "roofline": {"bound": "hbm", "kernel": "indexer", "achieved": r["algorithmic_bytes"]["indexer"] /
                     (r["indexer_ms"] * 1e-3) / 1e9 if r["indexer_ms"] > 0 else None, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": r.get("indexer_frac_hbm"), "traffic": None},
        "stages": r})
    return result


def decode_result(args):
    import sparse_long_context_dsa_amd as dsa  # noqa: F401
    from workloads import make_config
    log("generating decode workload 64 x 131072 (planted keys)")
    wl = make_config(2, device="cuda")
    p = prepare(wl)
    torch.cuda.synchronize()
    log("timing dsa_forward")
    wall, st, wall_ev = time_forward(wl, p, args.steps, args.warmup)
    log("timed regions done")
    nv = wl.q_nvis.cpu().numpy()
    units = indexer_units(nv, wl.k)
    idx_bytes = units * IDX_BYTES_PER_KEY + wl.nq * (64 * 128 + 64 * 8)
    achieved = idx_bytes / (st["indexer"] * 1e-3) / 1e9
    traffic = None
    if INDEXER_TRAFFIC is not None and INDEXER_TRAFFIC["source_sha"] == source_sha("indexer.hip"):
        traffic = INDEXER_TRAFFIC["bytes_per_launch"] / (st["indexer"] * 1e-3) / 1e9
    topk_bytes = units * 4 + wl.nq * wl.k * 4
    rows, flops, gather = mla_work(np.minimum(nv, wl.k))
    mla_bytes = gather + wl.nq * (128 * 576 * 2 + 128 * 512 * 4 + wl.k * 4)
    result = {
        "metric": "DSA layer decode queries/s @128K ctx; indexer HBM TB/s; sparse-MLA TFLOPs",
        "value": wl.nq * args.steps / wall,
        "unit": "queries/s",
    }
    result.update(common_fields(args))
    result.update({
        "ms_per_step": 1e3 * wall / args.steps,
        "config": {"workload": wl.name, "batch": wl.nq, "context": int(nv.max()), "k": wl.k,
                   "indexer_heads": 64, "indexer_dim": 128, "heads": 128, "latent": 576},
        "roofline": {"bound": "hbm", "kernel": "indexer", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": idx_bytes},
        "stages": {
            "timing": "HIP events on the library's stream between the stages, in a second pass of the "
                      "same steps (dsa_forward_profiled); value and ms_per_step come from the first pass "
                      "(plain dsa_forward, no events)",
            "events_pass_ms_per_step": 1e3 * wall_ev / args.steps,
            "indexer_ms": st["indexer"], "topk_ms": st["topk"], "mla_ms": st["mla"],
            "indexer_gbs": achieved,
            "topk_gbs": topk_bytes / (st["topk"] * 1e-3) / 1e9,
            "topk_frac_hbm": topk_bytes / (st["topk"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mla_tflops_bf16": flops / (st["mla"] * 1e-3) / 1e12,
            "mla_gbs": mla_bytes / (st["mla"] * 1e-3) / 1e9,
            "mla_gather_gbs": gather / (st["mla"] * 1e-3) / 1e9,
        },
    })
    if traffic is not None:
        result["roofline"]["traffic_bytes_per_launch"] = INDEXER_TRAFFIC["bytes_per_launch"]
    result["stages"]["planted"] = planted_in_topk(wl, p["idx"])
    log("standalone indexer: fp32 vs E8M0 key scales")
    result["indexer_key_scales"] = key_scale_formats(wl, p, args.steps)
    if args.copy_calib:
        log("calibration copy")
        calibration_copy()
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample, wl.k)
    del p
    del wl
    torch.cuda.empty_cache()
    if not args.no_configs:
        result["configs"] = extra_decode_configs(args.steps, args.warmup)
    if not args.no_prefill:
        result["prefill"] = run_prefill(max(2, args.steps // 4), 2, cpu=not args.no_cpu_baseline)
    return result


def crossover_result(args):
    """Sparse path (dsa_forward: indexer, top-k, attention over k rows) against
    the dense mode (dsa_dense_mla over the whole history) on decode batches of
    64 queries, as the history grows.  Each side: `warmup` untimed calls, then
    `steps` timed ones between two synchronizes."""
    import sparse_long_context_dsa_amd as dsa
    from workloads import make_custom
    rows = []
    for L in (1024, 2048, 2560, 3072, 4096, 6144, 8192, 16384, 32768):
        log(f"crossover: context {L}")
        wl = make_custom(seq_lens=[L] * 64, device="cuda", seed=70 + L % 97, plant=True)
        p = prepare(wl)
        wall, _, _ = time_forward(wl, p, args.steps, args.warmup)
        dws = dsa.workspace(dsa.DSA_OP_MLA_DENSE, p["queries"], 1)

        def dense():
            dsa.dsa_dense_mla(p["queries"], p["layout"], wl.q_mla, wl.kv, wl.softmax_scale, p["out"], p["lse"],
                              ws=dws)

        for _ in range(args.warmup):
            dense()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dense()
        torch.cuda.synchronize()
        dwall = time.perf_counter() - t0
        rows.append({"context": L, "sparse_ms": 1e3 * wall / args.steps, "dense_ms": 1e3 * dwall / args.steps})
        del p, wl, dws
        torch.cuda.empty_cache()
    cross = next((r["context"] for r in rows if r["sparse_ms"] < r["dense_ms"]), None)
    result = {"metric": "shortest decode history where the sparse path beats dense attention (batch 64, k=2048)",
              "value": cross, "unit": "positions"}
    result.update(common_fields(args))
    result.update({"higher_is_better": False,
                   "config": {"workload": "decode 64 x L, L from 1024 to 32768", "batch": 64, "k": 2048},
                   "rows": rows})
    return result


def kl_result(args):
    """The indexer's KL loss on the 16384-token causal prefill (the training
    shape): the sparse stage over each query's top-k set (from dsa_forward,
    with the attention's lse) and the dense warm-up over every visible
    position (lse from dsa_dense_mla).  Indexer scores for every position come
    from dsa_indexer_scores.  Each call: `warmup` untimed, then `steps` timed
    between two synchronizes.  The dominant kernel recomputes the attention
    logits (128 heads x 576 x 2 flop per member of a set) on bf16 MFMA; its rate
    is quoted over the whole call (target, loss and sum kernels), so it is a
    lower bound on the target kernel's own."""
    import oracle
    import sparse_long_context_dsa_amd as dsa
    from workloads import make_config
    log("kl: generating the 16384-token causal workload")
    wl = make_config(3, device="cuda")
    p = prepare(wl)
    nq = wl.nq
    dsa.dsa_forward(p["queries"], p["layout"], p["q8"], p["qs"], wl.w, p["k8"], p["ks"], wl.q_mla, wl.kv, wl.k,
                    wl.softmax_scale, p["out"], p["lse"], p["idx"], ws=p["ws"])
    ld = (wl.max_nvis + 63) // 64 * 64
    scores = torch.empty((nq, ld), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_scores(p["queries"], p["layout"], p["q8"], p["qs"], wl.w, p["k8"], p["ks"], scores)
    kl = torch.empty((nq,), dtype=torch.float32, device="cuda")
    loss = torch.empty((1,), dtype=torch.float32, device="cuda")
    grad_s = torch.empty((nq, wl.k), dtype=torch.float32, device="cuda")
    nv = wl.q_nvis.cpu().numpy()
    members_s = int(np.minimum(nv, wl.k).sum())
    members_d = int(nv.sum())

    def timed(call):
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / args.steps

    log("kl: sparse stage")
    t_s = timed(lambda: dsa.dsa_indexer_kl_sparse(p["queries"], p["layout"], wl.q_mla, wl.kv, p["idx"], None, wl.k,
                                                  p["lse"], wl.softmax_scale, scores, grad_s, kl, loss=loss))
    loss_s = float(loss.item())
    # Backward through the indexer score, from the sparse stage's dL/dI.
    dq = torch.empty((nq, 64, 128), dtype=torch.float32, device="cuda")
    dw = torch.empty((nq, 64), dtype=torch.float32, device="cuda")
    dk = torch.zeros((wl.rows, 128), dtype=torch.float32, device="cuda")
    log("kl: indexer backward, sparse stage")
    tb_s = timed(lambda: dsa.dsa_indexer_backward(p["queries"], p["layout"], p["q8"], p["qs"], wl.w, p["k8"], p["ks"],
                                                  p["idx"], None, wl.k, grad_s, dq, dw, dk))
    del grad_s
    log("kl: dense warm-up")
    lse_d = torch.empty((nq, 128), dtype=torch.float32, device="cuda")
    dws = dsa.workspace(dsa.DSA_OP_MLA_DENSE, p["queries"], 1)
    dsa.dsa_dense_mla(p["queries"], p["layout"], wl.q_mla, wl.kv, wl.softmax_scale, p["out"], lse_d, ws=dws)
    grad_d = torch.empty((nq, ld), dtype=torch.float32, device="cuda")
    t_d = timed(lambda: dsa.dsa_indexer_kl_dense(p["queries"], p["layout"], wl.q_mla, wl.kv, lse_d, wl.softmax_scale,
                                                 scores, grad_d, kl, loss=loss))
    loss_d = float(loss.item())
    log("kl: indexer backward, dense warm-up")
    tb_d = timed(lambda: dsa.dsa_indexer_backward(p["queries"], p["layout"], p["q8"], p["qs"], wl.w, p["k8"], p["ks"],
                                                  None, None, 0, grad_d, dq, dw, dk))
    del dq, dw, dk
    flop_member = 128 * 576 * 2
    # Backward per (query, key) pair: the 64 x 128 FP8 dot products, then the
    # dq and dk contractions (64 x 128 multiply-adds each).
    bwd_flop = 3 * 64 * 128 * 2
    tf_s = members_s * flop_member / t_s / 1e12
    tf_d = members_d * flop_member / t_d / 1e12
    cpu = None
    if not args.no_cpu_baseline:
        log("kl: timing the CPU oracle on a bounded sample")
        idx_h = p["idx"].cpu().numpy()
        sc_h = scores.cpu().numpy()
        sample = [int(i) for i in np.linspace(nq - 64, nq - 1, 16)]
        inputs = []
        for i in sample:
            c = int(min(nv[i], wl.k))
            pos = idx_h[i, :c]
            rows = int(wl.row0[0].item()) + pos
            kvr = wl.kv[torch.from_numpy(rows).cuda()].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            qm = wl.q_mla[i].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            inputs.append((qm, kvr, sc_h[i, pos].astype(np.float64)))
        t0 = time.perf_counter()
        for qm, kvr, x in inputs:
            oracle.indexer_kl_query(qm, kvr, x, wl.softmax_scale)
        dt = time.perf_counter() - t0
        cpu = {"value": len(sample) / dt, "unit": "queries/s", "cores": len(os.sched_getaffinity(0)),
               "kind": "oracle", "sample": f"{len(sample)} of the last 64 queries (2048-member sets), sparse stage, "
                                           f"{dt:.2f} s"}
    result = {"metric": "indexer KL loss, sparse stage: queries/s (16384-token causal prefill, k=2048)",
              "value": nq / t_s, "unit": "queries/s"}
    result.update(common_fields(args))
    result.update({
        "dtype": "bf16", "ms_per_step": 1e3 * t_s,
        "config": {"workload": "prefill 16384 tokens, causal, k=2048: indexer KL loss", "tokens": nq, "k": wl.k,
                   "heads": 128, "latent": 576},
        "roofline": {"bound": "mfma", "kernel": "kl_target", "achieved": tf_s, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf_s / BF16_PEAK_TFLOPS, "traffic": None},
        "sparse": {"members": members_s, "ms": 1e3 * t_s, "tflops_bf16": tf_s, "loss": loss_s},
        "dense_warmup": {"members": members_d, "ms": 1e3 * t_d, "tflops_bf16": tf_d,
                         "frac_bf16_peak": tf_d / BF16_PEAK_TFLOPS, "loss": loss_d},
        "indexer_backward": {
            "flop_per_pair": bwd_flop,
            "sparse": {"pairs": members_s, "ms": 1e3 * tb_s, "tflops": members_s * bwd_flop / tb_s / 1e12},
            "dense_warmup": {"pairs": members_d, "ms": 1e3 * tb_d, "tflops": members_d * bwd_flop / tb_d / 1e12}},
    })
    if cpu:
        result["cpu_baseline"] = cpu
    return result


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks settle only after some tens of milliseconds of steady
    # work: 5 warm-up steps (about 1.6 ms) left the timed decode steps 7-10%
    # slower than 50 do; 50 and 100 give the same figure.
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", choices=("decode", "prefill", "decode1x4k", "decode16x32k", "ragged", "crossover",
                                           "kl"), default="decode")
    ap.add_argument("--cpu-sample", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--copy-calib", action="store_true")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(decode shards by sequence with no exchange; see the design notes). "
              f"Got --gpus {args.gpus}, WORLD_SIZE {world}.", file=sys.stderr)
        sys.exit(2)

    import sparse_long_context_dsa_amd as dsa
    dsa._lib.lib()  # fail loudly if the HIP library is missing
    log(f"library {dsa.lib_path()}")
    if args.workload == "crossover":
        result = crossover_result(args)
    elif args.workload == "kl":
        result = kl_result(args)
    elif args.workload in ("decode1x4k", "decode16x32k", "ragged"):
        cfg, key = {"decode1x4k": (0, "decode_1x4096"), "decode16x32k": (1, "decode_16x32768_planted"),
                    "ragged": (4, "ragged_paged_128")}[args.workload]
        result = config_result(args, cfg, key)
    elif args.workload == "prefill":
        result = prefill_result(args)
        if args.copy_calib:
            log("calibration copy")
            calibration_copy()
    else:
        result = decode_result(args)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
