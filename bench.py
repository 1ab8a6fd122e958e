"""Throughput of the long-context causal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-long] [--no-cpu-baseline]

A step runs every step of the hot path once, each on its own synthetic workload, with inputs already resident in HBM:
  dense   causal GQA prefill, B1 Hq32 Hkv4 D128 N32768, Q/K/V i.i.d. N(0,1) (the headline workload)
  sparse  block-mask build + block-sparse prefill, N32768 block 64, planted outliers, centroid budget 10%, rescue
          alpha 1
  decode  split-KV paged decode, B32 Hq64 Hkv8 D64, lengths U[1024, 32768], page 16, 512-token chunks
`value` is the dense prefill's TFLOP/s: the causal count 2*B*Hq*N^2*D over the kernel's own mean duration, taken with
HIP events recorded around each call on the stream it is launched on. `ms_per_step` is the wall time of a whole step
(all three paths); `headline_kernel_ms` is the dense call's mean event time alone.
After the timed steps, further lines go under `paths`, each timed over at least 20 calls: dense prefill at N=4096 and
at 128K; the decode workload timed cold and over an fp8 (E4M3) copy of its cache; chunked prefill over a paged
cache (a 4K chunk closing a 32K sequence; a 128-token-window chunk over 8 sequences); the 128K mask + sparse pass
(speedup over the library's own dense kernel at the same length); and at 32K and 128K the mask built with the
query-aware rescue (rescue_mode 1) and from fp8 keys. The fp64 CPU oracle is timed on the host (cpu_baseline) on
seeded sampled rows of the headline workload, with the full workload's time extrapolated from its rate. One JSON
line goes to stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "prefill attention TFLOP/s (dense-equiv) + % bf16 MFMA peak; decode HBM GB/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(key, source):
    """HBM bytes per launch recorded in profiles/traffic.txt from rocprofv3 FETCH_SIZE/WRITE_SIZE runs (scaled by a
    plain-copy calibration), or None when absent or when the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.txt")
    src = os.path.join(ROOT, "long_context_attention_causal_amd", "csrc", source)
    try:
        kv = dict(l.split("=", 1) for l in open(path) if "=" in l and not l.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get(f"{key}.source_sha256") != hashlib.sha256(open(src, "rb").read()).hexdigest():
            return None
        return float(kv[f"{key}.fetch_bytes"]) + float(kv[f"{key}.write_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def device_peak():
    """The bf16 MFMA peak the device itself implies: compute units x 4096 flop per clock x the peak engine clock the
    HIP runtime reports (hipDeviceAttributeClockRate, kHz), beside the nominal figure the fractions use. The runtime
    is the one torch already loaded (found in this process's mappings), so no second copy is opened."""
    import ctypes
    import torch
    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count,
           "peak_clock_mhz": None, "bf16_peak_from_props_tflops": None}
    try:
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l and l.split()[-1].startswith("/"))
        hip = ctypes.CDLL(path)
        v = ctypes.c_int(0)
        kHipDeviceAttributeClockRate = 5   # position in hipDeviceAttribute_t (hip_runtime_api.h)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), kHipDeviceAttributeClockRate, torch.cuda.current_device()) == 0:
            out["peak_clock_mhz"] = v.value / 1e3
            out["bf16_peak_from_props_tflops"] = props.multi_processor_count * 4096 * v.value * 1e3 / 1e12
    except (StopIteration, OSError, AttributeError):
        pass
    return out


def dense_flops(B, Hq, N, D):
    return 2.0 * B * Hq * N * N * D


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-long", action="store_true", help="skip the 32K/128K dense and 128K sparse lines")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--long-reps", type=int, default=20)
    ap.add_argument("--cpu-rows", type=int, default=3200,
                    help="query rows per head the CPU oracle computes for cpu_baseline")
    ap.add_argument("--only", choices=["dense", "dense32k", "sparse", "sparse128k", "decode", "decode8", "paged",
                                       "copy"],
                    default=None,
                    help="run one path alone (for profiler runs); prints a short JSON line with its mean time")
    ap.add_argument("--selector-sweep", action="store_true",
                    help="selector footprint and block-size sweep (N 32K..256K, blocks 64/128/256, both rescue "
                         "modes); prints one JSON document instead of the bench line")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (each GPU would run an "
              f"independent share: see the sharding notes in DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_attention_causal_amd as lca
    import workloads as W

    lca.load()
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.only:
        run_only(args, lca, W, torch, np, to_dev, dev)
        return
    if args.selector_sweep:
        selector_sweep(lca, W, torch, np, to_dev, dev)
        return

    # ---------------------------------------------------------------------------------------- inputs
    log("generating the headline dense workload (N=32768, plain N(0,1))")
    wh = W.WORKLOADS["dense_bf16_n32k"]
    ch = W.make("dense_bf16_n32k")
    qh, kh, vh = to_dev(ch.q), to_dev(ch.k), to_dev(ch.v)
    oh = torch.empty_like(qh)

    log("generating the 32K block-sparse workload")
    w3 = W.WORKLOADS["c3_sparse_bf16_n32k"]
    c3 = W.make("c3_sparse_bf16_n32k")
    q3, k3, v3 = to_dev(c3.q), to_dev(c3.k), to_dev(c3.v)
    o3 = torch.empty_like(q3)
    m3 = lca.block_mask_build(q3, k3, w3["block"], w3["keep_permille"], w3["alpha"], w3["q_lo_pct"], w3["q_hi_pct"],
                              scale=c3.scale, want_radius_stats=False)

    log("generating the paged decode workload")
    w5 = W.WORKLOADS["c5_decode_paged_bf16"]
    c5 = W.make("c5_decode_paged_bf16")
    q5, kc5, vc5 = to_dev(c5.q), to_dev(c5.k_cache), to_dev(c5.v_cache)
    bt5 = torch.from_numpy(c5.block_table).to(dev)
    sl5 = torch.from_numpy(c5.seq_lens).to(dev)
    maxlen5 = int(w5["len_hi"])
    o5 = torch.empty_like(q5)
    ws5 = torch.zeros(lca.decode_workspace_bytes(q5, kc5, bt5, maxlen5, w5["chunk"]), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)

    def step(rec):
        e = [ev() for _ in range(5)]
        e[0].record()
        lca.prefill_dense(qh, kh, vh, scale=ch.scale, out=oh, return_lse=False)
        e[1].record()
        lca.block_mask_build(q3, k3, w3["block"], w3["keep_permille"], w3["alpha"], w3["q_lo_pct"], w3["q_hi_pct"],
                             scale=c3.scale, outputs=m3)
        e[2].record()
        lca.prefill_block_sparse(q3, k3, v3, m3.kv_count, m3.kv_index, w3["block"], scale=c3.scale, out=o3,
                                 return_lse=False)
        e[3].record()
        lca.decode_paged(q5, kc5, vc5, bt5, sl5, maxlen5, w5["chunk"], scale=c5.scale, out=o5, return_lse=False,
                         workspace=ws5)
        e[4].record()
        rec.append(e)

    log(f"warmup {args.warmup}, timed {args.steps} steps")
    junk = []
    for _ in range(args.warmup):
        step(junk)
    torch.cuda.synchronize()
    recs = []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(recs)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([[r[i].elapsed_time(r[i + 1]) for i in range(4)] for r in recs])   # ms per part
    t_head, t_mask3, t_sparse3, t_dec = (float(x) for x in per.mean(axis=0))

    def spread(x):   # median and the 10th / 90th percentiles of per-call times, ms
        x = np.asarray(x, dtype=np.float64)
        return {"ms_median": float(np.median(x)), "ms_p10": float(np.percentile(x, 10)),
                "ms_p90": float(np.percentile(x, 90)), "calls": int(x.size)}

    def time_calls(fn, reps):
        fn()
        torch.cuda.synchronize()
        es = []
        for _ in range(reps):
            a, b = ev(), ev()
            a.record()
            fn()
            b.record()
            es.append((a, b))
        torch.cuda.synchronize()
        x = [a.elapsed_time(b) for a, b in es]
        return float(np.mean(x)), spread(x)

    # decode timed cold as well: 1 GiB read between calls evicts L2 and the 256 MB last-level cache (a read rather than
    # a write, whose dirty lines would be written back during the decode and charge it for the eviction)
    log("paged decode, cold (1 GiB read between calls)")
    junk = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cold = []
    for i in range(args.steps + 2):
        junk.sum()
        a_, b_ = ev(), ev()
        a_.record()
        lca.decode_paged(q5, kc5, vc5, bt5, sl5, maxlen5, w5["chunk"], scale=c5.scale, out=o5, return_lse=False,
                         workspace=ws5)
        b_.record()
        if i >= 2:
            cold.append((a_, b_))
    torch.cuda.synchronize()
    cold_ms = [a_.elapsed_time(b_) for a_, b_ in cold]
    del junk
    torch.cuda.empty_cache()

    # the same decode workload over the fp8 (E4M3) cache: back to back, then cold like the bf16 line
    log("generating the fp8 paged decode workload")
    c8 = W.make("c5_decode_paged_fp8")
    q8 = to_dev(c8.q)
    k8, v8 = torch.from_numpy(c8.k_cache).to(dev), torch.from_numpy(c8.v_cache_t).to(dev)
    bt8, sl8 = torch.from_numpy(c8.block_table).to(dev), torch.from_numpy(c8.seq_lens).to(dev)
    o8 = torch.empty_like(q8)
    dec8 = lambda: lca.decode_paged_fp8(q8, k8, v8, c8.k_scale, c8.v_scale, bt8, sl8, maxlen5, w5["chunk"],
                                        scale=c8.scale, out=o8, return_lse=False, workspace=ws5)
    log("paged decode over the fp8 cache")
    dec8()
    torch.cuda.synchronize()
    warm8 = []
    for _ in range(args.steps + 30):
        a_, b_ = ev(), ev()
        a_.record()
        dec8()
        b_.record()
        warm8.append((a_, b_))
    junk = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cold8 = []
    for i in range(args.steps + 2):
        junk.sum()
        a_, b_ = ev(), ev()
        a_.record()
        dec8()
        b_.record()
        if i >= 2:
            cold8.append((a_, b_))
    torch.cuda.synchronize()
    warm8_ms = [a_.elapsed_time(b_) for a_, b_ in warm8]
    cold8_ms = [a_.elapsed_time(b_) for a_, b_ in cold8]
    L8 = c8.seq_lens.astype(np.int64)
    dec8_bytes = float(L8.sum() * w5["Hkv"] * w5["D"] * 2 + w5["B"] * w5["Hq"] * w5["D"] * 2 * 2
                       + ((L8 + 15) // 16).sum() * 4)
    del junk, q8, k8, v8, bt8, sl8, o8, c8
    torch.cuda.empty_cache()

    B, Hq, N, D = ch.q.shape
    fl_head = dense_flops(B, Hq, N, D)
    tf_head = fl_head / (t_head * 1e-3) / 1e12

    # sparse accounting from the mask the GPU built
    cnt3 = m3.kv_count.cpu().numpy().astype(np.int64)
    b3 = w3["block"]
    D3 = w3["D"]
    exec3 = float(((cnt3 - 1) * 4.0 * b3 * b3 * D3 + 2.0 * b3 * (b3 + 1) * D3).sum())
    causal_pairs3 = w3["Hq"] * (w3["N"] // b3) * (w3["N"] // b3 + 1) / 2
    density3 = float(cnt3.sum() / causal_pairs3)
    dense_eq3 = dense_flops(1, w3["Hq"], w3["N"], D3)

    # decode algorithmic bytes: K and V rows of every cached token, q, o and the block-table entries read
    L5 = c5.seq_lens.astype(np.int64)
    Hkv5, D5, Hq5, B5 = w5["Hkv"], w5["D"], w5["Hq"], w5["B"]
    kv_bytes = float(L5.sum() * Hkv5 * D5 * 2 * 2)
    dec_bytes = kv_bytes + B5 * Hq5 * D5 * 2 * 2 + float(((L5 + 15) // 16).sum() * 4)
    dec_gbs = dec_bytes / (t_dec * 1e-3) / 1e9

    # mask stats pass: reads Q and K once
    mask_read3 = float((w3["Hq"] + w3["Hkv"]) * w3["N"] * D3 * 2)

    paths = {
        "dense_prefill_n32768": {"ms": t_head, **spread(per[:, 0]), "tflops": tf_head,
                                 "pct_bf16_peak": 100 * tf_head / PEAK_BF16_TFLOPS,
                                 "tokens_per_s": B * N / (t_head * 1e-3), "note": "the headline (value) line"},
        "mask_build_n32768_b64": {"ms": t_mask3, **spread(per[:, 1]), "stats_read_bytes": mask_read3,
                                  "stats_read_gbs_over_whole_build": mask_read3 / (t_mask3 * 1e-3) / 1e9,
                                  "density": density3},
        "sparse_prefill_n32768_b64": {"ms": t_sparse3, **spread(per[:, 2]), "executed_tflop": exec3 / 1e12,
                                      "executed_tflops": exec3 / (t_sparse3 * 1e-3) / 1e12,
                                      "pct_bf16_peak_executed": 100 * exec3 / (t_sparse3 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                      "dense_equiv_tflops_incl_mask": dense_eq3 / ((t_sparse3 + t_mask3) * 1e-3) / 1e12,
                                      "speedup_vs_dense_kernel_only": t_head / t_sparse3,
                                      "speedup_vs_dense_incl_mask": t_head / (t_sparse3 + t_mask3),
                                      "planted_kept": None},
        "decode_paged_c5": {"ms": t_dec, **spread(per[:, 3]), "algorithmic_bytes": dec_bytes, "gbs": dec_gbs,
                            "cold_ms": float(np.mean(cold_ms)), "cold_ms_median": float(np.median(cold_ms)),
                            "cold_gbs": dec_bytes / (float(np.mean(cold_ms)) * 1e-3) / 1e9,
                            "cold_pct_hbm_peak": 100 * dec_bytes / (float(np.mean(cold_ms)) * 1e-3) / 1e9 / PEAK_HBM_GBS,
                            "measured_hbm_bytes": (lambda a, b: None if a is None or b is None else a + b)(
                                measured_traffic("decode_split_c5", "decode.hip"),
                                measured_traffic("decode_combine_c5", "decode.hip")),
                            "pct_hbm_peak": 100 * dec_gbs / PEAK_HBM_GBS, "tokens_per_s": B5 / (t_dec * 1e-3),
                            "tflops": 4.0 * D5 * Hq5 * float(L5.sum()) / (t_dec * 1e-3) / 1e12},
    }

    t8 = float(np.mean(warm8_ms))
    paths["decode_paged_c5_fp8"] = {
        "ms": t8, **spread(warm8_ms), "algorithmic_bytes": dec8_bytes, "gbs": dec8_bytes / (t8 * 1e-3) / 1e9,
        "pct_hbm_peak": 100 * dec8_bytes / (t8 * 1e-3) / 1e9 / PEAK_HBM_GBS, "tokens_per_s": w5["B"] / (t8 * 1e-3),
        "cold_ms": float(np.mean(cold8_ms)), "cold_ms_median": float(np.median(cold8_ms)),
        "cold_gbs": dec8_bytes / (float(np.mean(cold8_ms)) * 1e-3) / 1e9,
        "cold_pct_hbm_peak": 100 * dec8_bytes / (float(np.mean(cold8_ms)) * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "speedup_vs_bf16_cold": float(np.mean(cold_ms)) / float(np.mean(cold8_ms)),
        "measured_hbm_bytes": (lambda a, b: None if a is None or b is None else a + b)(
            measured_traffic("decode_split_fp8_c5", "decode.hip"), measured_traffic("decode_combine_fp8_c5", "decode.hip"))}

    def planted_kept(mask, planted, block):
        """How many planted key blocks the mask keeps in the row of the query they were planted for."""
        if not planted:
            return None
        idx = torch.tensor([[b, h, t // block, j] for (b, g, j, u, h, t) in planted], device=mask.device).T
        return {"kept": int(mask[idx[0], idx[1], idx[2], idx[3]].sum().item()), "planted": len(planted)}

    def query_aware(q, k, v, o, w, scale, t_dense_same_n, planted, reps):
        """Mask build with the query-aware rescue (rescue_mode 1) and the sparse pass over its lists."""
        blk, nbq = w["block"], w["N"] // w["block"]
        mk = lambda out=None: lca.block_mask_build(q, k, blk, w["keep_permille"], w["alpha"], w["q_lo_pct"],
                                                   w["q_hi_pct"], scale=scale, want_radius_stats=False,
                                                   outputs=out, rescue_mode=1)
        m = mk()
        tm, stm = time_calls(lambda: mk(m), reps)
        ts, sts = time_calls(lambda: lca.prefill_block_sparse(q, k, v, m.kv_count, m.kv_index, blk, scale=scale,
                                                              out=o, return_lse=False), reps)
        cnt = m.kv_count.cpu().numpy().astype(np.int64)
        ex = float(((cnt - 1) * 4.0 * blk * blk * w["D"] + 2.0 * blk * (blk + 1) * w["D"]).sum())
        return {"mask_ms": tm, "mask_ms_median": stm["ms_median"], "sparse_ms": ts, "sparse_ms_median": sts["ms_median"],
                "density": float(cnt.sum() / (w["Hq"] * nbq * (nbq + 1) / 2)),
                "executed_tflops": ex / (ts * 1e-3) / 1e12,
                "speedup_vs_dense_kernel_only": t_dense_same_n / ts,
                "speedup_vs_dense_incl_mask": t_dense_same_n / (ts + tm),
                "planted_kept": planted_kept(m.mask, planted, blk)}

    # chunked prefill over a paged cache: a 4K chunk closing a 32K sequence, and a windowed chunk over 8 sequences
    def paged_line(name, reps):
        w = W.WORKLOADS[name]
        log(f"generating {name}")
        p = W.make(name)
        c = p.cache
        qp, kp, vp = to_dev(p.q), to_dev(c.k_cache), to_dev(c.v_cache)
        btp, slp = torch.from_numpy(c.block_table).to(dev), torch.from_numpy(c.seq_lens).to(dev)
        op = torch.empty_like(qp)
        wsb = lca.prefill_paged_workspace_bytes(qp, kp, btp, window=w["window"])
        wsp = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        log(f"paged prefill {name} (workspace {wsb} bytes)")
        t, sp = time_calls(lambda: lca.prefill_paged(qp, kp, vp, btp, slp, window=w["window"], scale=p.scale, out=op,
                                                     return_lse=False, workspace=wsp), reps)
        Lp = c.seq_lens.astype(np.int64)
        Nq = w["Nq"]
        pos = (Lp[:, None] - Nq) + np.arange(Nq)[None, :]
        keys = np.minimum(pos + 1, w["window"]) if w["window"] > 0 else pos + 1
        fl = 4.0 * w["D"] * w["Hq"] * float(keys.sum())
        # algorithmic bytes: the chunk's q read and o written, and every cached K/V row some query of the chunk sees
        lo = np.maximum(pos[:, 0] - w["window"] + 1, 0) if w["window"] > 0 else np.zeros_like(Lp)
        kv_rows = float((Lp - lo).sum())
        nbytes = 2.0 * w["B"] * w["Hq"] * Nq * w["D"] * 2 + kv_rows * w["Hkv"] * w["D"] * 2 * 2
        ai = fl / nbytes
        line = {"ms": t, **sp, "key_range_split": wsb > 0, "tflops": fl / (t * 1e-3) / 1e12,
                "pct_bf16_peak": 100 * fl / (t * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "new_tokens_per_s": w["B"] * Nq / (t * 1e-3), "flop": fl, "algorithmic_bytes": nbytes,
                "flop_per_byte": ai, "gbs": nbytes / (t * 1e-3) / 1e9}
        # below the ridge (about 315 flop/B) the bound is HBM: report the fraction of that roofline too
        if ai < PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9):
            line["bound"] = "hbm"
            line["pct_hbm_peak"] = 100 * nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS
        else:
            line["bound"] = "mfma"
        return line

    # dense prefill at N=4096 (the shorter dense workload)
    log("dense prefill at N=4096")
    c2 = W.make("c2_dense_bf16_n4k")
    q2, k2, v2 = to_dev(c2.q), to_dev(c2.k), to_dev(c2.v)
    o2 = torch.empty_like(q2)
    t2, s2 = time_calls(lambda: lca.prefill_dense(q2, k2, v2, scale=c2.scale, out=o2, return_lse=False),
                        max(args.long_reps, 20))
    B2, Hq2, N2, D2 = c2.q.shape
    tf2 = dense_flops(B2, Hq2, N2, D2) / (t2 * 1e-3) / 1e12
    paths["dense_prefill_n4096"] = {"ms": t2, **s2, "tflops": tf2, "pct_bf16_peak": 100 * tf2 / PEAK_BF16_TFLOPS,
                                    "tokens_per_s": N2 / (t2 * 1e-3),
                                    "measured_hbm_bytes": measured_traffic("prefill_dense_c2", "prefill.hip")}
    del q2, k2, v2, o2, c2

    paths["paged_prefill_c6_chunk4k_of_32k"] = paged_line("c6_paged_prefill_chunk", 20)
    paths["paged_prefill_c7_window128"] = paged_line("c7_paged_prefill_window", 20)

    def fp8_key_mask(q, k_bits, w, scale, m_bf16, planted, reps):
        """The same mask built from per-tensor E4M3 codes of the keys: its time, density, planted recall and its
        Jaccard overlap with the bf16-key mask (kept pairs in both over kept pairs in either)."""
        codes, ksc = W.e4m3_keys(k_bits)
        kc = torch.from_numpy(codes).to(dev)
        blk, nbq = w["block"], w["N"] // w["block"]
        mk = lambda out=None: lca.block_mask_build(q, kc, blk, w["keep_permille"], w["alpha"], w["q_lo_pct"],
                                                   w["q_hi_pct"], scale=scale, want_radius_stats=False, outputs=out,
                                                   k_scale=ksc)
        m = mk()
        t, st = time_calls(lambda: mk(m), reps)
        inter = int((m.mask & m_bf16.mask).sum().item())
        union = int((m.mask | m_bf16.mask).sum().item())
        cnt = m.kv_count.cpu().numpy().astype(np.int64)
        return {"mask_ms": t, "mask_ms_median": st["ms_median"], "k_scale": ksc,
                "density": float(cnt.sum() / (w["Hq"] * nbq * (nbq + 1) / 2)),
                "jaccard_vs_bf16_keys": inter / union, "planted_kept": planted_kept(m.mask, planted, blk)}

    if not args.no_long:
        paths["sparse_prefill_n32768_b64"]["planted_kept"] = planted_kept(m3.mask, c3.planted, w3["block"])
        log("query-aware rescue at 32K")
        paths["sparse_prefill_n32768_b64"]["query_aware_rescue"] = query_aware(
            q3, k3, v3, o3, w3, c3.scale, t_head, c3.planted, args.long_reps)
        log("mask from fp8 keys at 32K")
        paths["mask_build_n32768_b64"]["fp8_keys"] = fp8_key_mask(q3, c3.k, w3, c3.scale, m3, c3.planted,
                                                                  args.long_reps)
        del q3, k3, v3, o3, m3
        torch.cuda.empty_cache()
        log("generating the 128K block-sparse workload")
        w4 = W.WORKLOADS["c4_sparse_bf16_n128k"]
        c4 = W.make("c4_sparse_bf16_n128k")
        q4, k4, v4 = to_dev(c4.q), to_dev(c4.k), to_dev(c4.v)
        o4 = torch.empty_like(q4)
        planted4 = c4.planted
        k4_bits = c4.k
        del c4
        log("dense prefill at 128K")
        t128, s128 = time_calls(lambda: lca.prefill_dense(q4, k4, v4, scale=1 / math.sqrt(128), out=o4,
                                                          return_lse=False), args.long_reps)
        fl128 = dense_flops(1, w4["Hq"], w4["N"], w4["D"])
        tf128 = fl128 / (t128 * 1e-3) / 1e12
        paths["dense_prefill_n131072"] = {"ms": t128, **s128, "tflops": tf128,
                                          "pct_bf16_peak": 100 * tf128 / PEAK_BF16_TFLOPS}
        log("mask build + sparse prefill at 128K")
        m4 = lca.block_mask_build(q4, k4, w4["block"], w4["keep_permille"], w4["alpha"], w4["q_lo_pct"],
                                  w4["q_hi_pct"], scale=1 / math.sqrt(128), want_radius_stats=False)
        tm4, _ = time_calls(lambda: lca.block_mask_build(q4, k4, w4["block"], w4["keep_permille"], w4["alpha"],
                                                         w4["q_lo_pct"], w4["q_hi_pct"], scale=1 / math.sqrt(128),
                                                         outputs=m4), args.long_reps)
        ts4, sts4 = time_calls(lambda: lca.prefill_block_sparse(q4, k4, v4, m4.kv_count, m4.kv_index, w4["block"],
                                                                scale=1 / math.sqrt(128), out=o4, return_lse=False),
                               args.long_reps)
        cnt4 = m4.kv_count.cpu().numpy().astype(np.int64)
        b4 = w4["block"]
        exec4 = float(((cnt4 - 1) * 4.0 * b4 * b4 * w4["D"] + 2.0 * b4 * (b4 + 1) * w4["D"]).sum())
        nb4 = w4["N"] // b4
        paths["sparse_prefill_n131072_b128"] = {
            "mask_ms": tm4, "sparse_ms": ts4, "sparse_ms_median": sts4["ms_median"], "density": float(cnt4.sum() / (w4["Hq"] * nb4 * (nb4 + 1) / 2)),
            "executed_tflops": exec4 / (ts4 * 1e-3) / 1e12,
            "pct_bf16_peak_executed": 100 * exec4 / (ts4 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "dense_equiv_tflops_incl_mask": fl128 / ((ts4 + tm4) * 1e-3) / 1e12,
            "speedup_vs_dense_kernel_only": t128 / ts4,
            "speedup_vs_dense_incl_mask": t128 / (ts4 + tm4),
            "planted_kept": planted_kept(m4.mask, planted4, b4)}
        log("mask from fp8 keys at 128K")
        paths["sparse_prefill_n131072_b128"]["fp8_keys_mask"] = fp8_key_mask(q4, k4_bits, w4, 1 / math.sqrt(128), m4,
                                                                              planted4, args.long_reps)
        del m4, k4_bits
        log("query-aware rescue at 128K")
        paths["sparse_prefill_n131072_b128"]["query_aware_rescue"] = query_aware(
            q4, k4, v4, o4, w4, 1 / math.sqrt(128), t128, planted4, args.long_reps)
        del q4, k4, v4, o4
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import attention as A
        rows = W.sample_rows(wh["seed"], N, Hq, args.cpu_rows)
        log(f"timing the fp64 oracle on the host ({rows.shape[1]} seeded rows per head of the headline workload)")
        cores = len(os.sched_getaffinity(0))
        G = Hq // ch.k.shape[1]
        t_cpu = 0.0
        sample_flop = 0.0
        for h in range(Hq):
            g = h // G
            # widening the inputs to fp64 is preparation, not timed; the oracle's attention over the rows is
            kf = W.f64_from_bf16_bits(ch.k[:, g:g + 1])
            vf = W.f64_from_bf16_bits(ch.v[:, g:g + 1])
            qf = np.zeros((B, 1, N, D))
            qf[:, 0, rows[h]] = W.f64_from_bf16_bits(ch.q[:, h, rows[h]])
            t0 = time.perf_counter()
            A.causal_attention(qf, kf, vf, ch.scale, rows=rows[h])
            t_cpu += time.perf_counter() - t0
            sample_flop += 4.0 * D * float((rows[h] + 1).sum()) * B   # causal: row t sees t + 1 keys
        rate = sample_flop / t_cpu
        blas = "unknown"
        try:
            blas = str(np.show_config(mode="dicts")["Build Dependencies"]["blas"].get("name", "unknown"))
        except Exception:
            pass
        cpu = {"value": rate / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
               "sample": f"fp64 numpy oracle ({blas} BLAS, {os.environ.get('OMP_NUM_THREADS', 'default')} BLAS "
                         f"threads) on {rows.size} seeded query rows ({rows.shape[1]} per head, all {Hq} heads, "
                         f"rows 0 and N-1 included) of the headline workload: {sample_flop / 1e9:.1f} GFLOP of "
                         f"causal work in {t_cpu:.2f} s; the full workload extrapolated at that rate",
               "rows": int(rows.size), "seconds": t_cpu, "gflops": rate / 1e9,
               "extrapolated_full_s": fl_head / rate, "blas": blas}

    line = {
        "metric": METRIC, "value": tf_head, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "headline_kernel_ms": t_head,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "dense_bf16_n32k: dense causal GQA prefill B1 Hq32 Hkv4 D128 N32768, Q/K/V i.i.d. "
                               "N(0,1) in bf16 (value); a step also runs the N32768 block-64 mask build and "
                               "block-sparse prefill and the paged decode (B32 Hq64 Hkv8 D64)",
                   "global_batch": 1, "seq_len": N, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": tf_head, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf_head / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("prefill_dense_n32k", "prefill.hip"),
                     "kernel": "prefill_dense_kernel<128>", "per_launch_flop": fl_head,
                     "algorithmic_bytes": float((B * Hq + 2 * ch.k.shape[1]) * N * D * 2 + B * Hq * N * D * 2)},
        "cpu_baseline": cpu,
        "device": device_peak(),
        "paths": paths,
    }
    print(json.dumps(line), flush=True)


def selector_sweep(lca, W, torch, np, to_dev, dev):
    """Selector footprint and block-size sweep on the planted workload shape (B1 Hq32 Hkv4 D128): for N of 32K,
    64K, 128K and 256K and blocks of 64, 128 and 256 keys (up to 4096 blocks), in both rescue modes, the mask
    build's workspace and output bytes, its measured peak device memory beyond the inputs, its time, the mask
    density, the planted blocks kept in their query's row, and the sparse pass's time over the mask. The centroid
    budget is 10% at 32K and 5% above, rescue alpha 1. Q/K/V are drawn once per N; the outliers are planted
    afresh for each block size."""
    Hq, Hkv, D = 32, 4, 128
    scale = 1.0 / math.sqrt(D)
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    rows = []
    for N in (32768, 65536, 131072, 262144):
        seed = 100 + N // 32768
        keep = 100 if N <= 32768 else 50
        log(f"selector sweep: generating N={N}")
        base = W.dense_inputs(seed, 1, Hq, Hkv, N, D, "bf16")
        k_clean = base.k.copy()
        q, v = to_dev(base.q), to_dev(base.v)
        o = torch.empty_like(q)
        for block in (64, 128, 256):
            nb = N // block
            if nb > 4096:
                continue
            base.k[...] = k_clean
            W.plant_outliers(base, seed, block)
            k = to_dev(base.k)
            for mode in (0, 1):
                log(f"selector sweep: N={N} block={block} rescue_mode={mode}")
                ws = lca.block_mask_workspace_bytes(q, k, block, keep, 1.0, scale=scale, rescue_mode=mode)
                out_bytes = Hq * nb * nb * (1 + 4) + Hq * nb * 4
                torch.cuda.synchronize()
                torch.cuda.empty_cache()
                torch.cuda.reset_peak_memory_stats()
                before = torch.cuda.memory_allocated()
                m = lca.block_mask_build(q, k, block, keep, 1.0, scale=scale, want_radius_stats=False,
                                         rescue_mode=mode)
                torch.cuda.synchronize()
                peak = torch.cuda.max_memory_allocated() - before
                t_mask = timed(lambda: lca.block_mask_build(q, k, block, keep, 1.0, scale=scale, outputs=m,
                                                            rescue_mode=mode), 5)
                t_sparse = timed(lambda: lca.prefill_block_sparse(q, k, v, m.kv_count, m.kv_index, block,
                                                                  scale=scale, out=o, return_lse=False), 3)
                cnt = m.kv_count.cpu().numpy().astype(np.int64)
                idx = torch.tensor([[b, h, t // block, j] for (b, g, j, u, h, t) in base.planted], device=dev).T
                kept = int(m.mask[idx[0], idx[1], idx[2], idx[3]].sum().item())
                rows.append({"N": N, "block": block, "rescue_mode": mode, "keep_permille": keep,
                             "workspace_bytes": ws, "output_bytes": out_bytes, "peak_bytes_measured": int(peak),
                             "mask_ms": t_mask, "sparse_ms": t_sparse,
                             "density": float(cnt.sum() / (Hq * nb * (nb + 1) / 2)),
                             "planted_kept": kept, "planted": len(base.planted)})
                print(json.dumps(rows[-1]), file=sys.stderr, flush=True)
                del m
            del k
        del q, v, o, base, k_clean
        torch.cuda.empty_cache()
    print(json.dumps({"selector_sweep": rows}), flush=True)


def run_only(args, lca, W, torch, np, to_dev, dev):
    """One path, args.warmup + args.steps calls, for kernel-level profiler runs. `copy` is a plain 1 GiB
    device-to-device copy, the reference for scaling the profiler's HBM byte counters."""
    if args.only == "copy":
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        fn = lambda: dst.copy_(src)
    elif args.only in ("dense", "dense32k"):
        name = "c2_dense_bf16_n4k" if args.only == "dense" else "dense_bf16_n32k"
        c = W.make(name)
        q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
        o = torch.empty_like(q)
        fn = lambda: lca.prefill_dense(q, k, v, scale=c.scale, out=o, return_lse=False)
    elif args.only in ("sparse", "sparse128k"):
        name = "c3_sparse_bf16_n32k" if args.only == "sparse" else "c4_sparse_bf16_n128k"
        w = W.WORKLOADS[name]
        c = W.make(name)
        q, k, v = to_dev(c.q), to_dev(c.k), to_dev(c.v)
        o = torch.empty_like(q)
        m = lca.block_mask_build(q, k, w["block"], w["keep_permille"], w["alpha"], w["q_lo_pct"], w["q_hi_pct"],
                                 scale=c.scale, want_radius_stats=False)

        def fn():
            lca.block_mask_build(q, k, w["block"], w["keep_permille"], w["alpha"], w["q_lo_pct"], w["q_hi_pct"],
                                 scale=c.scale, outputs=m)
            lca.prefill_block_sparse(q, k, v, m.kv_count, m.kv_index, w["block"], scale=c.scale, out=o,
                                     return_lse=False)
    elif args.only == "paged":
        w = W.WORKLOADS["c6_paged_prefill_chunk"]
        p = W.make("c6_paged_prefill_chunk")
        q, kc, vc = to_dev(p.q), to_dev(p.cache.k_cache), to_dev(p.cache.v_cache)
        bt, sl = torch.from_numpy(p.cache.block_table).to(dev), torch.from_numpy(p.cache.seq_lens).to(dev)
        o = torch.empty_like(q)
        wsb = lca.prefill_paged_workspace_bytes(q, kc, bt, window=w["window"])
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
        fn = lambda: lca.prefill_paged(q, kc, vc, bt, sl, window=w["window"], scale=p.scale, out=o, return_lse=False,
                                       workspace=ws)
    elif args.only == "decode8":
        w = W.WORKLOADS["c5_decode_paged_fp8"]
        c = W.make("c5_decode_paged_fp8")
        q = to_dev(c.q)
        kc, vc = torch.from_numpy(c.k_cache).to(dev), torch.from_numpy(c.v_cache_t).to(dev)
        bt, sl = torch.from_numpy(c.block_table).to(dev), torch.from_numpy(c.seq_lens).to(dev)
        o = torch.empty_like(q)
        ws = torch.empty(lca.decode_workspace_bytes(q, kc, bt, w["len_hi"], w["chunk"]), dtype=torch.uint8, device=dev)
        fn = lambda: lca.decode_paged_fp8(q, kc, vc, c.k_scale, c.v_scale, bt, sl, w["len_hi"], w["chunk"],
                                          scale=c.scale, out=o, return_lse=False, workspace=ws)
    else:
        w = W.WORKLOADS["c5_decode_paged_bf16"]
        c = W.make("c5_decode_paged_bf16")
        q, kc, vc = to_dev(c.q), to_dev(c.k_cache), to_dev(c.v_cache)
        bt, sl = torch.from_numpy(c.block_table).to(dev), torch.from_numpy(c.seq_lens).to(dev)
        o = torch.empty_like(q)
        ws = torch.empty(lca.decode_workspace_bytes(q, kc, bt, w["len_hi"], w["chunk"]), dtype=torch.uint8, device=dev)
        fn = lambda: lca.decode_paged(q, kc, vc, bt, sl, w["len_hi"], w["chunk"], scale=c.scale, out=o,
                                      return_lse=False, workspace=ws)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(args.steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    print(json.dumps({"only": args.only, "calls": args.steps, "ms_per_call": a.elapsed_time(b) / args.steps}),
          flush=True)


if __name__ == "__main__":
    main()
