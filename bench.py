#!/usr/bin/env python3
"""Decode throughput of one CSA2 layer group on one MI355X.

Default workload: the decoder's first group at 64K context, batch 32 -- a Full
layer (quantise the 32 new tokens' main-KV rows to FP4, scan all 65,536
indexer keys per sequence, pool of 2,048 blocks, Top-512) followed by three
Reuse layers (own Q and 128-row SWA window, same Top-512).  One step = the
whole group over one batch; inputs are synthetic, seeded, and resident in HBM
before timing starts.

Prints one JSON line: query-tokens/s, achieved HBM GB/s of the group, the
roofline of the dominant kernel (the indexer scan; for a prefill chunk the
attention against the fp16 MFMA peak, with the scan against the int8 peak
beside it) and of the attention kernel, from HIP events recorded around them
inside the timed region, and the FP64 oracle timed on the host.

Timing: every timed step starts with a cold last-level cache -- a 512 MiB
device write (twice the MI355X's 256 MB Infinity Cache) runs between steps,
outside the step's own event pair -- and the line reports the median step
(with p10 / p90); back-to-back steps, which find the previous step's rows and
windows still cached, are reported beside it as "warm".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak (AMD spec)
PEAK_F16_TFLOPS = 2500.0       # MI355X dense fp16 / bf16 MFMA peak (AMD spec)
PEAK_I8_TOPS = 5000.0          # MI355X dense int8 MFMA peak (AMD spec)

# HBM bytes per k_index_scan launch measured with rocprofv3 FETCH_SIZE and
# WRITE_SIZE (each scaled by what the counter reads for a plain 1 GiB copy) on
# the workloads and kernel sources named here; reported only while they match.
SCAN_TRAFFIC = {"source_sha256": "cb0cdfd54593cc3524fc7bea46fac9cdb8c4791efb497dcf86067602f648ac52",   # csrc/index.hip + csrc/common.h
                "bytes": {"decode_group_full_reuse3_b32_t65536": 268804505 + 9437286,
                          "decode_group_full_reuse3_b32_t65536_idx8": 278864076 + 9437900,
                          "verify_group_full_reuse3_b8_q6_t1m": 1074306662 + 25168281}}


def scan_traffic(w):
    import hashlib
    h = hashlib.sha256()
    for name in ("index.hip", "common.h"):                  # the scan kernel's sources
        with open(os.path.join(ROOT, "fp4_kv_cache_e4m3_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    sha = h.hexdigest()
    if sha == SCAN_TRAFFIC["source_sha256"]:
        return SCAN_TRAFFIC["bytes"].get(w.name)
    return None


def group_bytes(w) -> dict:
    """Algorithmic bytes of one group step (what the method must move)."""
    nq, T = w.nq, w.kv_len
    row = w.dim // 2 + w.dim // 16                         # FP4 row: codes + scales
    f8 = 4 if w.idx_fp8 else 0                             # fp32 scale per key position / query head
    scan = w.batch * T * (w.idx_dim + f8) + nq * w.idx_heads * (w.idx_dim + 4 + f8)
    select = nq * ((0 if w.encoder else 2048 * 4) + 512 * 4)   # pool (decoder groups) + topk written
    quant = w.batch * w.new_per_seq * (w.dim * 4 + row)
    bt = 512 * 4 if w.page_size else 0                     # paged: one block-table entry per Top-K entry
    swa_new = nq * (w.dim * 2 + w.dim + 4) if w.swa8 else 0  # 8-bit windows: the step's new rows quantised
    attn_layer = (nq * (512 * row + w.heads * w.dim * 2 + w.heads * w.dim * 4 + 512 * 4 + bt)
                  + w.batch * w.swa_rows * (w.dim + 4 if w.swa8 else w.dim * 2) + swa_new)
    reindex = nq * (2048 * 4 + 16384 * (w.idx_dim + f8) + w.idx_heads * (w.idx_dim + 4 + f8) + 512 * 4)
    n_full, n_rx = w.layers.count("full"), w.layers.count("reindex")
    total = n_full * (quant + scan + select) + n_rx * reindex + len(w.layers) * attn_layer
    return dict(scan=scan, select=select, quant=quant, attn_layer=attn_layer, reindex=reindex,
                total=total)


def host_cores() -> int:
    """Cores this process may run on (the affinity mask), else the count."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(w, max_queries: int, min_seconds: float = 10.0, threads: int | None = None) -> dict:
    """The FP64 oracle on the first max_queries query tokens of the same
    workload (one full group step each: new-entry quantisation of their
    sequences, Full index over all T positions, every layer's attention),
    repeated until at least min_seconds of wall time have been timed.
    Input generation is not timed.  threads: the BLAS thread-pool size to run
    with (None: the pool as numpy set it up)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from fp4_kv_cache_e4m3_amd import synth
    from oracle import attention as oattn
    from oracle import indexer as oidx
    from oracle import quant as oquant

    T, qn = w.kv_len, w.q_per_seq
    nqs = min(w.nq, max_queries)
    n_seq = (nqs + qn - 1) // qn
    iq, iw = synth.index_q(w)[:nqs], synth.index_w(w)[:nqs]
    ik = [synth.index_k(w, b) for b in range(n_seq)]
    newr = synth.new_rows(w)[:n_seq * w.new_per_seq]
    qs = [synth.bf16_bits_to_f32(synth.attn_q_bf16(w, l)[:nqs]).astype(np.float64)
          for l in range(len(w.layers))]
    sws = [synth.bf16_bits_to_f32(synth.swa_bf16(w, l)[:n_seq]).astype(np.float64)
           for l in range(len(w.layers))]
    new_sw = None
    if w.swa8:                                          # the window as its 8-bit rows hold it
        from oracle import swa8 as oswa8
        sws = [oswa8.swa_values(*oswa8.quantize_swa_rows(s.reshape(-1, w.dim))).reshape(s.shape) for s in sws]
        new_sw = [synth.bf16_bits_to_f32(synth.new_swa_rows(w, l)[:n_seq * qn]).astype(np.float64)
                  for l in range(len(w.layers))]
    srcs = [synth.kv_source(w, b) for b in range(n_seq)]
    f8 = w.idx_fp8
    qsc = (lambda l, src=False: synth.index_q_scale(w, l, src)[:nqs]) if f8 else (lambda l, src=False: None)
    sq = qsc(0)
    sk = [synth.index_k_scale(w, b) for b in range(n_seq)] if f8 else None
    rx = {l: (synth.index_q(w, l)[:nqs], synth.index_w(w, l)[:nqs], qsc(l))
          for l, m in enumerate(w.layers) if m == "reindex" and l > 0}
    if w.layers[0] == "reindex":
        rx[0] = (iq, iw, sq)
        iq, iw = synth.index_q(w, 0, pool_source=True)[:nqs], synth.index_w(w, 0, pool_source=True)[:nqs]
        sq = qsc(0, True)
    if f8:
        from oracle import indexer_fp8 as o8

        def full_q(qi, b):
            return o8.full_query(iq[qi], sq[qi], iw[qi], ik[b], sk[b], T)

        def rx_q(l, qi, b, pool):
            return o8.reindex_query(rx[l][0][qi], rx[l][2][qi], rx[l][1][qi], ik[b], sk[b], pool, T)[0]
    else:
        def full_q(qi, b):
            return oidx.full_query(iq[qi], iw[qi], ik[b], T)

        def rx_q(l, qi, b, pool):
            return oidx.reindex_query(rx[l][0][qi], rx[l][1][qi], ik[b], pool, T)

    def one_pass():
        if w.layers[0] == "full":
            oquant.quantize_rows(newr)
        if new_sw is not None:                          # the step's new 8-bit window rows
            for l in range(len(w.layers)):
                v = oswa8.swa_values(*oswa8.quantize_swa_rows(new_sw[l]))
                sws[l][:, w.swa_rows - qn:] = v.reshape(n_seq, qn, w.dim)
        for qi in range(nqs):
            b = qi // qn
            pool, pos, _ = full_q(qi, b)
            for l, m in enumerate(w.layers):
                if m == "reindex":
                    pos = rx_q(l, qi, b, pool)
                if m in ("full", "reindex"):
                    codes, scales = oquant.quantize_rows(srcs[b][pos])     # the selected cache rows
                keys = oattn.query_entries(qi % qn, qn, len(pos), np.arange(len(pos)), codes, scales,
                                           sws[l][b:b + 1], w.window)
                oattn.attend(qs[l][qi], keys, 1.0 / np.sqrt(w.dim))

    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        reps = 0
        t0 = time.perf_counter()
        while True:
            one_pass()
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= min_seconds:
                break
    return {"value": reps * nqs / dt, "unit": "query-tokens/s", "cores": used, "kind": "oracle",
            "sample": f"first {nqs} of {w.nq} query tokens ({n_seq} of {w.batch} sequences), full group "
                      f"step ({'+'.join(w.layers)}), T={T}, repeated {reps}x; {dt:.2f} s wall"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="decode_group_full_reuse3_b32_t65536")
    ap.add_argument("--cpu-queries", type=int, default=32, help="query tokens in the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "reference for scaling HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "only --gpus 1 is supported: the path runs on one GPU and "
                                   "its multi-GPU sharding is not implemented", "n_gpus": args.gpus}))
        return 2

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), flush=True)
        return 0

    import fp4_kv_cache_e4m3_amd as csa2
    from fp4_kv_cache_e4m3_amd import synth

    w = synth.WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    csa2.load()
    g = csa2.DecodeGroup(w)
    stream = torch.cuda.current_stream()
    nl = len(w.layers)
    full = w.layers[0] == "full"
    # the step's library calls in order (the Full layer's index call split into
    # its scan and select so that the scan can be timed on its own)
    calls = g.calls(stream, split_full=True)
    roof_stage = "index_scan" if full else "reindex"
    roof_i = next(i for i, (st, _) in enumerate(calls) if st == roof_stage)

    attn_i = next(i for i, (st, _) in enumerate(calls) if st == "attention")

    def step(ev=None, at=None):
        # ev / at: event pairs recorded around the first scan (or reindex) call
        # and the first attention call (timing only; no sync)
        for i, (_, call) in enumerate(calls):
            if ev is not None and i == roof_i: ev[0].record(stream)
            if at is not None and i == attn_i: at[0].record(stream)
            call()
            if ev is not None and i == roof_i: ev[1].record(stream)
            if at is not None and i == attn_i: at[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    def pair():
        return [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    # timed region: K cold steps.  Before each, a 512 MiB write evicts the
    # last-level cache (outside the step's event pair); the scan and the
    # first attention call are bracketed by their own events on alternate
    # sampled steps (every event on the stream costs a few microseconds)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    step_ev = [pair() for _ in range(args.steps)]
    scan_ev = {k: pair() for k in range(args.steps) if k % 5 == 0}
    attn_ev = {k: pair() for k in range(args.steps) if k % 5 == 2}
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for k in range(args.steps):
        flush.fill_(k & 0xFF)
        step_ev[k][0].record(stream)
        step(scan_ev.get(k), attn_ev.get(k))
        step_ev[k][1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = sorted(e[0].elapsed_time(e[1]) for e in step_ev)
    pct = lambda f: step_ms[min(len(step_ms) - 1, int(round(f * (len(step_ms) - 1))))]
    ms = pct(0.5)
    scan_ms = sorted(e[0].elapsed_time(e[1]) for e in scan_ev.values())[len(scan_ev) // 2]
    attn_ms = sorted(e[0].elapsed_time(e[1]) for e in attn_ev.values())[len(attn_ev) // 2]

    # warm: K steps back to back between two events
    start, stop = pair()
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    warm_ms = start.elapsed_time(stop) / args.steps

    # per-stage breakdown: a separate warm pass of K steps, one event after
    # every call
    bev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        bev[k][0].record(stream)
        for i, (_, call) in enumerate(calls):
            call()
            bev[k][i + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {}
    for k in range(args.steps):
        for i, (st, _) in enumerate(calls):
            stage_ms[st] = stage_ms.get(st, 0.0) + bev[k][i].elapsed_time(bev[k][i + 1]) / args.steps

    # the device's achievable HBM read rate (every byte of 1 GiB read once by
    # csa2_read_rate), the reference beside the 8 TB/s spec peak
    del flush
    rbuf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    rsink = torch.empty(csa2.READ_RATE_SINK_WORDS, dtype=torch.int32, device="cuda")
    for _ in range(3):
        csa2.read_rate(rbuf, rsink, stream)
    rev = [pair() for _ in range(10)]
    for a, b_ in rev:
        a.record(stream)
        csa2.read_rate(rbuf, rsink, stream)
        b_.record(stream)
    torch.cuda.synchronize()
    read_ms = sorted(a.elapsed_time(b_) for a, b_ in rev)[len(rev) // 2]
    read_gbs = (1 << 30) / (read_ms / 1e3) / 1e9
    del rbuf, rsink

    nbytes = group_bytes(w)
    value = w.nq / (ms / 1e3)
    scan_bytes = nbytes["scan"] if full else nbytes["reindex"]
    group = "group" if nl <= 6 else f"{nl}-layer decoder step"
    achieved = scan_bytes / (scan_ms / 1e3) / 1e9
    attn_achieved = nbytes["attn_layer"] / (attn_ms / 1e3) / 1e9
    # the library runs the one-workgroup-per-query kernel for many query tokens
    wide = w.dim == 512 and not w.swa8 and w.nq * ((w.heads + 63) // 64) >= 96
    attn_kernel = "k_attn_wide" if wide else "k_attn"
    # matrix work of one attention layer: QK^T and PV over the Top-512 and window entries
    attn_tflop = 4.0 * w.nq * w.heads * (512 + w.window) * w.dim / 1e12
    # integer work of the indexer scan: every score row against every position
    scan_tops = 2.0 * w.nq * w.idx_heads * w.kv_len * w.idx_dim / 1e12
    out = {
        "metric": f"decode query-tokens/s per CSA2 layer {group} at 64K ctx + achieved HBM GB/s",
        "value": round(value, 1),
        "unit": "query-tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp4e2m1+e4m3/{}/fp16-mfma".format("fp8e4m3" if w.idx_fp8 else "int8"),
        "data": "synthetic (seeded numpy; N(0,1) KV/Q/SWA, {} indexer inputs)".format(
            "E4M3 + fp32-scale" if w.idx_fp8 else "integer"),
        "config": {"workload": w.name, "batch": w.batch, "q_per_seq": w.q_per_seq,
                   "kv_len": w.kv_len, "dim": w.dim, "heads": w.heads, "window": w.window,
                   "idx_heads": w.idx_heads, "idx_dim": w.idx_dim, "layers": list(w.layers),
                   "idx_fp8": w.idx_fp8, "swa8": w.swa8, "page_size": w.page_size, "swa_ring": w.swa_ring},
        "timing": "cold last-level cache (512 MiB write between steps, outside the events); "
                  "median of the per-step event times",
        "ms_per_step_p10": round(pct(0.1), 4), "ms_per_step_p90": round(pct(0.9), 4),
        "warm": {"ms_per_step": round(warm_ms, 4), "value": round(w.nq / (warm_ms / 1e3), 1),
                 "hbm_frac_group": round(nbytes["total"] / (warm_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                 "timing": "steps back to back between two events"},
        "hbm_gbs_group": round(nbytes["total"] / (ms / 1e3) / 1e9, 1),
        "hbm_frac_group": round(nbytes["total"] / (ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
        "breakdown_ms": dict({"pass": "separate, one event after every call (sums per stage)"},
                             **{st: round(v, 4) for st, v in stage_ms.items()}),
        "roofline": {"kernel": "k_index_scan" if full else "k_reindex_score+k_select_reindex",
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "bytes_per_launch": scan_bytes, "traffic": scan_traffic(w) if full else None},
        "roofline_attn": {"kernel": attn_kernel, "bound": "hbm", "achieved": round(attn_achieved, 1),
                          "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(attn_achieved / PEAK_HBM_GBS, 4),
                          "bytes_per_launch": nbytes["attn_layer"], "ms": round(attn_ms, 4)},
        "wall_s_timed": round(t_wall, 3),
        "hbm_read_achievable": {"kernel": "k_read_rate", "gbs": round(read_gbs, 1),
                                "frac_of_peak": round(read_gbs / PEAK_HBM_GBS, 4), "bytes": 1 << 30,
                                "timing": "median of 10 event pairs, every byte read once"},
    }
    if w.encoder:
        # a prefill chunk is matrix work: the attention (the step's dominant
        # kernel) against the fp16 MFMA peak, the scan against the int8 one
        a_tf = attn_tflop / (attn_ms / 1e3)
        out["roofline"] = {"kernel": attn_kernel, "bound": "mfma", "achieved": round(a_tf, 1),
                           "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(a_tf / PEAK_F16_TFLOPS, 4),
                           "flop_per_launch": attn_tflop * 1e12, "ms": round(attn_ms, 4), "traffic": None}
        s_tops = scan_tops / (scan_ms / 1e3)
        out["roofline_scan"] = {"kernel": "k_index_scan", "bound": "mfma", "achieved": round(s_tops, 1),
                                "peak": PEAK_I8_TOPS, "unit": "TOP/s", "frac": round(s_tops / PEAK_I8_TOPS, 4),
                                "ops_per_launch": scan_tops * 1e12, "ms": round(scan_ms, 4)}
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, args.cpu_queries)
        one = cpu_baseline(w, args.cpu_queries, threads=1)
        cb["host_cores"] = host_cores()
        cb["value_1thread"] = one["value"]
        cb["sample_1thread"] = one["sample"]
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
