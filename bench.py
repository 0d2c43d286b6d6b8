"""Benchmark of the FP4 lightning-indexer hot path on one MI355X.

A step is one pass of the whole path over one batch: the fused K writer for
the step's new compressed tokens, the index-Q pack, the paged FP4 logits over
every cached token of every row, and the per-row top-k.  The default workload
is the decode batch of 64 requests (1 query row each, contexts U[1024, 16384]
compressed tokens, random page tables, top-k 2048).

Inputs are synthetic and seeded; the page pool is filled before timing by the
library's own K writer.  Every timed step reads a different copy of the
inputs (copies total well above the 256 MB last-level cache), so the HBM
figures are HBM, not cache.  A timed step is three launches in sequence (the
K write and Q pack together in one launch, the logits, the top-k), issued as
prepared library calls (arguments marshalled once per input copy, one ctypes
call per launch: about 10 us of host time per step, below the GPU time) or,
with `--launch graph`, as a replay of a HIP graph captured per input copy
(slower on this stack: hipGraphLaunch costs more host time than the three
calls).  Per-kernel durations come from a second pass over the
same K steps, launched eagerly with the two encoders as separate kernels,
where each kernel carries HIP events that its own dispatch stamps with its
start and end times (fp4idx_time_next_call -> hipExtLaunchKernel); they feed
the roofline figures.

The same step is also timed with the logits and the top-k as one fused call
(fp4idx_mqa_logits_topk, no logits in memory; extras.fused_logits_topk) and
on the FP8 indexer cache (132-byte fused tokens,
the layout the FP4 cache replaces) and reported under extras.fp8_cache; the
headline value is the FP4 path's.

Prints one JSON line (rank 0).
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

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E
MFMA_FP4_PEAK_TFLOPS = 10100.0  # dense MXFP4
# fp32 VALU lane-ops/s with packed fp32 off: 256 CUs x 4 SIMDs x 16 lanes per clock x
# 2.4 GHz = 39.3 T (the published 157.3 TFLOP/s fp32 vector rate counts an FMA as two flop
# and a packed instruction as two FMAs per lane); fp4idx_peak_valu_fp32 measures it
VALU_PEAK_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
CACHE_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Digest of everything the kernels are compiled from (HIP sources, headers, build flags)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_fp4_fp4idx_amd", "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files += [os.path.join(ROOT, "sparse_attention_fp4_fp4idx_amd", "build.py"), os.path.join(ROOT, "include", "fp4idx.h")]
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.basename(f).encode())
            h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(workload_key)
    except Exception:
        return None
    if not rec or rec.get("source_sha") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index (1 = decode batch 64)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache comparison leg")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused logits + top-k leg")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak microbenchmarks")
    ap.add_argument("--launch", choices=("prepared", "graph"), default="prepared",
                    help="timed steps as prepared library calls (default) or as HIP graph replays")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = enough to defeat the cache)")
    ap.add_argument("--source-sha", action="store_true", help="print the kernel-source digest and exit")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MB",
                    help="also run a plain device copy of MB mebibytes (a known-size reference for HBM counters)")
    args = ap.parse_args()
    if args.source_sha:
        print(kernel_source_hash())
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} (WORLD_SIZE {world}) is not "
              "supported. The path shards by request or by context across GPUs; see DESIGN.md.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_fp4_fp4idx_amd import fp4idx as F
    from sparse_attention_fp4_fp4idx_amd import workloads as W

    F.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def b16(a):
        return t(a.view(np.int16)).view(torch.bfloat16)

    t0 = time.time()
    wl = W.make(args.config)
    log(f"[bench] workload: {wl.name}: rows {wl.n_rows} reqs {wl.n_reqs} scores {wl.scores} pages {wl.num_pages} "
        f"new tokens {wl.k_new.shape[0]} ({time.time() - t0:.1f}s)")
    tab = b16(W.rope_table(wl.max_pos))
    norm_w = b16(wl.norm_w)

    # ---- fill the pool with encoded cached tokens (untimed)
    payload = torch.zeros(wl.num_pages * 4096, dtype=torch.uint8, device=dev)
    scale = torch.zeros(wl.num_pages * 256, dtype=torch.uint8, device=dev)
    if wl.cached_slots.size:
        kc = wl.cached_k()
        for a in range(0, kc.shape[0], 1 << 20):
            F.write_k(b16(kc[a:a + (1 << 20)]), t(wl.cached_pos[a:a + (1 << 20)]), t(wl.cached_slots[a:a + (1 << 20)]),
                      norm_w, wl.eps, tab, payload, scale)
        del kc
    torch.cuda.synchronize()
    log(f"[bench] pool filled ({time.time() - t0:.1f}s)")

    # ---- measured peaks (the library's microbenchmarks): FP4 MFMA and streaming HBM read
    measured = None
    if not args.no_peaks:
        sink_f = torch.zeros(1, dtype=torch.float32, device=dev)
        sink_u = torch.zeros(1, dtype=torch.int32, device=dev)
        big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        big.fill_(1)
        pev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
        for a_, b_ in pev:
            a_.record(stream)
            b_.record(stream)
        F.peak_mfma_fp4(64, sink_f, stream=stream)
        F.peak_read(big, sink_u, stream=stream)
        torch.cuda.synchronize()
        vev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
        for a_, b_ in vev:
            a_.record(stream)
            b_.record(stream)
        F.peak_valu_fp32(64, sink_f, stream=stream)
        mev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
               for _ in range(3)]
        for row in mev:
            for a_, b_ in row:
                a_.record(stream)
                b_.record(stream)
        for m in range(3):
            F.peak_mfma_valu(m, 16, sink_f, stream=stream)
        flop = [0] * 4
        nbytes = [0] * 4
        lops = [0] * 4
        for i in range(4):
            F.time_next_call(*pev[i])
            flop[i] = F.peak_mfma_fp4(2048, sink_f, stream=stream)
            F.time_next_call(*pev[4 + i])
            nbytes[i] = F.peak_read(big, sink_u, stream=stream)
            F.time_next_call(*vev[i])
            lops[i] = F.peak_valu_fp32(4096, sink_f, stream=stream)
            for m in range(3):
                F.time_next_call(*mev[m][i])
                F.peak_mfma_valu(m, 1024, sink_f, stream=stream)
        torch.cuda.synchronize()
        mf = float(np.median([flop[i] / (pev[i][0].elapsed_time(pev[i][1]) * 1e-3) / 1e12 for i in range(4)]))
        rd = float(np.median([nbytes[i] / (pev[4 + i][0].elapsed_time(pev[4 + i][1]) * 1e-3) / 1e9
                              for i in range(4)]))
        va = float(np.median([lops[i] / (vev[i][0].elapsed_time(vev[i][1]) * 1e-3) / 1e12 for i in range(4)]))
        # MFMA alone, fp32 FMAs alone, both interleaved: overlap 1 = the pipes run in
        # parallel (mix = the longer part), 0 = they take turns (mix = the sum)
        tm = [float(np.median([mev[m][i][0].elapsed_time(mev[m][i][1]) * 1e3 for i in range(4)])) for m in range(3)]
        overlap = (tm[0] + tm[1] - tm[2]) / min(tm[0], tm[1])
        measured = {"mfma_fp4_TFLOPs": round(mf, 1), "hbm_read_GBs": round(rd, 1), "valu_fp32_Tlane_ops": round(va, 1),
                    "mfma_valu_overlap": round(overlap, 3),
                    "mfma_valu_us": {"mfma": round(tm[0], 1), "valu": round(tm[1], 1), "both": round(tm[2], 1)},
                    "note": "fp4idx_peak_mfma_fp4 (4,096 waves of dependent-free 16x16x128 FP4 MFMA chains), "
                            "fp4idx_peak_read (1 GiB streaming read), fp4idx_peak_valu_fp32 (4,096 waves of "
                            "16 independent fp32 FMA chains) and fp4idx_peak_mfma_valu (the MFMA and FMA chains "
                            "alone and interleaved; overlap = (alone + alone - both) / shorter alone, 1 = the "
                            "pipes overlap, 0 = they take turns), dispatch-stamped, median of 4"}
        del big
        log(f"[bench] measured peaks: FP4 MFMA {mf:.0f} TFLOP/s, HBM read {rd:.0f} GB/s, "
            f"fp32 VALU {va:.1f} T lane-ops/s, MFMA/VALU overlap {overlap:.2f} ({time.time() - t0:.1f}s)")

    T, H, k = wl.n_rows, wl.heads, wl.topk
    pos_new, slot_new = t(wl.pos_new), t(wl.slot_new)
    pos_q, indptr, ctx, bt = t(wl.pos_q), t(wl.req_row_indptr), t(wl.row_ctx), t(wl.block_table)
    names = ("write_k", "pack_q", "mqa_logits", "topk")

    def run_cache(fp8: bool, pools: dict, fused: bool = False):
        """Time the step on one cache format: rotating input copies, the timed
        prepared calls (or graph replays), then the per-kernel event pass.
        With fused, the logits and the top-k are one fp4idx_mqa_logits_topk
        call (FP4 cache).  Returns (ms_per_step, per-kernel ms, copies)."""
        qcode_b = 128 if fp8 else 64
        base = dict(pools, q=b16(wl.q), w=t(wl.w), k_new=b16(wl.k_new))
        step_bytes = sum(v.numel() * v.element_size() for v in base.values()) + T * wl.max_ctx * 4 * 2
        copies = args.copies or max(2, int(np.ceil(2 * CACHE_BYTES / step_bytes)))
        copies = min(copies, max(2, int(0.5 * torch.cuda.mem_get_info()[0] // step_bytes)))
        sets = []
        for c in range(copies):
            s = {n: (v if c == 0 else v.clone()) for n, v in base.items()}
            s["logits"] = torch.empty((T, wl.max_ctx), dtype=torch.float32, device=dev)
            s["q_code"] = torch.empty((T, H, qcode_b), dtype=torch.uint8, device=dev)
            s["q_scale"] = (torch.empty((T, H), dtype=torch.float32, device=dev) if fp8
                            else torch.empty((T, H, 4), dtype=torch.uint8, device=dev))
            s["w_out"] = torch.empty((T, H), dtype=torch.float32, device=dev)
            s["top"] = torch.empty((T, k), dtype=torch.int32, device=dev)
            sets.append(s)
        log(f"[bench] {'fp8' if fp8 else 'fp4'}: {copies} input copies of {step_bytes / 1e6:.1f} MB "
            f"({time.time() - t0:.1f}s)")

        def pool_args(s):
            return (s["pool"],) if fp8 else (s["payload"], s["scale"])

        def step(s, strm, ev=None):
            """One pass of the path on stream strm.  The timed steps encode the
            step's K tokens and query rows in one launch (write_k_pack_q); the
            kernel-timing pass (ev given) launches the two encoders separately
            so that each component kernel gets its own duration."""
            def arm(i):   # events stamped with kernel i's own start / end (hipExtLaunchKernel)
                if ev is not None:
                    F.time_next_call(ev[i][0], ev[i][1])
            if ev is None:
                (F.write_k_pack_q_fp8 if fp8 else F.write_k_pack_q)(
                    s["k_new"], pos_new, slot_new, norm_w, wl.eps, tab, *pool_args(s), s["q"], pos_q, s["w"],
                    wl.w_scale, s["q_code"], s["q_scale"], s["w_out"], stream=strm)
            else:
                arm(0)
                (F.write_k_fp8 if fp8 else F.write_k)(s["k_new"], pos_new, slot_new, norm_w, wl.eps, tab,
                                                      *pool_args(s), stream=strm)
                arm(1)
                (F.pack_q_fp8 if fp8 else F.pack_q)(s["q"], pos_q, tab, s["w"], wl.w_scale, s["q_code"],
                                                    s["q_scale"], s["w_out"], stream=strm)
            arm(2)
            if fused:
                F.mqa_logits_topk(s["q_code"], s["q_scale"], s["w_out"], indptr, ctx, bt, *pool_args(s), k,
                                  wl.max_rows_per_req, wl.max_ctx, out_idx=s["top"], stream=strm)
                return
            (F.mqa_logits_fp8 if fp8 else F.mqa_logits)(s["q_code"], s["q_scale"], s["w_out"], indptr, ctx, bt,
                                                        *pool_args(s), wl.max_rows_per_req, wl.max_ctx,
                                                        logits=s["logits"], stream=strm)
            arm(3)
            F.topk(s["logits"], ctx, k, wl.max_ctx, out_idx=s["top"], stream=strm)

        for i in range(args.warmup):
            step(sets[i % copies], stream)
        torch.cuda.synchronize()

        # the timed steps: per input copy either three prepared library calls
        # (arguments marshalled once, one ctypes call each) or one captured HIP graph
        runners = []
        if args.launch == "graph":
            cap = torch.cuda.Stream()
            for c in range(copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    step(sets[c], torch.cuda.current_stream())
                runners.append(g.replay)
                sets[c]["graph"] = g
        else:
            for c in range(copies):
                s_ = sets[c]
                pw, _ = (F.prepare_write_k_pack_q_fp8 if fp8 else F.prepare_write_k_pack_q)(
                    s_["k_new"], pos_new, slot_new, norm_w, wl.eps, tab, *pool_args(s_), s_["q"], pos_q, s_["w"],
                    wl.w_scale, s_["q_code"], s_["q_scale"], s_["w_out"], stream=stream)
                if fused:
                    pl, _ = F.prepare_mqa_logits_topk(s_["q_code"], s_["q_scale"], s_["w_out"], indptr, ctx, bt,
                                                      *pool_args(s_), k, wl.max_rows_per_req, wl.max_ctx,
                                                      out_idx=s_["top"], stream=stream)
                    pt = lambda: None  # noqa: E731
                else:
                    pl, _ = (F.prepare_mqa_logits_fp8 if fp8 else F.prepare_mqa_logits)(
                        s_["q_code"], s_["q_scale"], s_["w_out"], indptr, ctx, bt, *pool_args(s_),
                        wl.max_rows_per_req, wl.max_ctx, logits=s_["logits"], stream=stream)
                    pt, _ = F.prepare_topk(s_["logits"], ctx, k, wl.max_ctx, out_idx=s_["top"], stream=stream)

                def run(pw=pw, pl=pl, pt=pt):
                    pw()
                    pl()
                    pt()
                runners.append(run)
        for c in range(copies):
            runners[c]()
        torch.cuda.synchronize()

        # timed region: K steps, bracketed by synchronize
        torch.cuda.synchronize()
        start = time.perf_counter()
        for i in range(args.steps):
            runners[i % copies]()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - start

        # kernel durations: the same K steps launched eagerly on the launch stream, each kernel carrying
        # HIP events that its own dispatch stamps with its start and end times (no marker packets in between)
        evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in names]
               for _ in range(args.steps)]
        for row in evs:          # create the HIP events (torch creates them on first record)
            for a, b in row:
                a.record(stream)
                b.record(stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(sets[i % copies], stream, evs[i])
        torch.cuda.synchronize()
        used = names[:3] if fused else names
        times = {n: [evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(args.steps)] for j, n in enumerate(used)}
        if fused:
            times = {"write_k": times["write_k"], "pack_q": times["pack_q"], "mqa_logits_topk": times["mqa_logits"]}
        per_kernel = {n: float(np.mean(v)) for n, v in times.items()}
        # median and minimum over the K steps as well (the mean feeds the roofline)
        per_kernel_stats = {n: (float(np.median(v)), float(np.min(v))) for n, v in times.items()}
        del sets, runners
        return elapsed * 1e3 / args.steps, per_kernel, copies, per_kernel_stats

    if args.calib_copy:
        # reference for rocprofv3 FETCH_SIZE / WRITE_SIZE: reads and writes exactly MB MiB
        csrc = torch.empty(args.calib_copy << 20, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        torch.cuda.synchronize()
        del csrc, cdst

    ms_per_step, per_kernel_ms, copies, per_kernel_stats = run_cache(False, dict(payload=payload, scale=scale))
    scores = wl.scores
    value = scores / (ms_per_step * 1e-3)

    # ---- roofline of the dominant kernel (algorithmic bytes per launch)
    uniq_tokens = int(np.sum([int(np.max(wl.row_ctx[wl.req_row_indptr[b]:wl.req_row_indptr[b + 1]], initial=0))
                              for b in range(wl.n_reqs)]))
    logits_bytes = 68 * uniq_tokens + 4 * scores + 4608 * T + 4 * ((uniq_tokens + 63) // 64)
    alg = {"mqa_logits": logits_bytes,
           "topk": 4 * scores + 4 * k * T,
           "write_k": 460 * wl.k_new.shape[0] + 256,
           "pack_q": 21380 * T}
    dom = max(per_kernel_ms, key=per_kernel_ms.get)
    dom_ms = per_kernel_ms[dom]
    # the dominant kernel against each resource it uses; the binding one is the
    # resource with the largest fraction of its peak (the roofline's limit):
    # HBM bytes; FP4 MFMA flop (2*128*heads per score); fp32 VALU lane-ops
    # (ReLU + FMA per head per score, 2*heads; packed fp32 is off)
    fractions = {"hbm": alg[dom] / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    serial = None
    if dom == "mqa_logits":
        fractions["mfma"] = 2 * 128 * H * scores / (dom_ms * 1e-3) / 1e12 / MFMA_FP4_PEAK_TFLOPS
        fractions["alu"] = 2 * H * scores / (dom_ms * 1e-3) / 1e12 / VALU_PEAK_TOPS
        # on gfx950 a SIMD's matrix and vector work do not overlap (measured), so the
        # contraction and its ReLU/weight epilogue bound the kernel together: their
        # times at peak, summed, over the kernel's time
        serial = fractions["mfma"] + fractions["alu"]
    bound = max(fractions, key=fractions.get)
    peak, unit = {"hbm": (HBM_PEAK_GBS, "GB/s"), "mfma": (MFMA_FP4_PEAK_TFLOPS, "TFLOP/s"),
                  "alu": (VALU_PEAK_TOPS, "T lane-ops/s")}[bound]
    traffic = measured_traffic(f"config{args.config}:{dom}")
    roofline = {"kernel": dom, "bound": bound, "achieved": round(fractions[bound] * peak, 1), "peak": peak,
                "unit": unit, "frac": round(fractions[bound], 4), "traffic": traffic,
                "alg_bytes_per_launch": alg[dom], "avg_launch_us": round(dom_ms * 1e3, 2),
                "fractions": {k: round(v, 4) for k, v in fractions.items()}}
    if serial is not None:
        roofline["frac_mfma_plus_alu"] = round(serial, 4)
    if measured:
        # the same achieved figures against the measured peaks
        mp = {"hbm": measured["hbm_read_GBs"], "mfma": measured["mfma_fp4_TFLOPs"],
              "alu": measured["valu_fp32_Tlane_ops"]}
        vendor = {"hbm": HBM_PEAK_GBS, "mfma": MFMA_FP4_PEAK_TFLOPS, "alu": VALU_PEAK_TOPS}
        fm = {r: fractions[r] * vendor[r] / mp[r] for r in mp if r in fractions}
        roofline["frac_vs_measured_peak"] = {r: round(v, 4) for r, v in fm.items()}
        if serial is not None:
            roofline["frac_vs_measured_peak"]["mfma_plus_alu"] = round(fm["mfma"] + fm["alu"], 4)
        roofline["measured_peaks"] = measured

    # ---- split-pool reader: every cached token of the workload back to fp32, one launch (not part of the step)
    extras = {}
    if wl.cached_slots.size:
        rslots = t(wl.cached_slots)
        rout = torch.empty((rslots.numel(), 128), dtype=torch.float32, device=dev)
        rev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a, b in rev:
            a.record(stream)
            b.record(stream)
        F.read_k(payload, scale, rslots, out=rout, stream=stream)      # warm-up
        torch.cuda.synchronize()
        for a, b in rev:
            F.time_next_call(a, b)
            F.read_k(payload, scale, rslots, out=rout, stream=stream)
        torch.cuda.synchronize()
        r_ms = float(np.median([a.elapsed_time(b) for a, b in rev]))
        r_bytes = 584 * rslots.numel()   # 64 code + 4 scale + 4 slot bytes read, 512 bytes written per token
        extras["read_k"] = {"tokens": int(rslots.numel()), "us": round(r_ms * 1e3, 2),
                            "GB/s": round(r_bytes / (r_ms * 1e-3) / 1e9, 1),
                            "hbm_frac": round(r_bytes / (r_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        del rout

    # ---- the FP8 indexer cache on the same workload (132-byte fused tokens): same step, same timing
    if not args.no_fp8:
        pool8 = torch.zeros(wl.num_pages * W.FP8_PAGE_BYTES, dtype=torch.uint8, device=dev)
        if wl.cached_slots.size:
            kc = wl.cached_k()
            for a in range(0, kc.shape[0], 1 << 20):
                F.write_k_fp8(b16(kc[a:a + (1 << 20)]), t(wl.cached_pos[a:a + (1 << 20)]),
                              t(wl.cached_slots[a:a + (1 << 20)]), norm_w, wl.eps, tab, pool8)
            del kc
        torch.cuda.synchronize()
        ms8, pk8, copies8, _ = run_cache(True, dict(pool=pool8))
        del pool8
        l8 = 132 * uniq_tokens + 4 * scores + 8704 * T + 4 * ((uniq_tokens + 63) // 64)
        a8 = l8 / (pk8["mqa_logits"] * 1e-3) / 1e9
        extras["fp8_cache"] = {
            "ms_per_step": round(ms8, 4), "scores_per_s": round(scores / (ms8 * 1e-3), 1),
            "kernels_us": {n: round(v * 1e3, 2) for n, v in pk8.items()},
            "logits_roofline": {"bound": "hbm", "achieved": round(a8, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": round(a8 / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": l8,
                                "traffic": measured_traffic(f"config{args.config}:fp8_mqa_logits")},
            "bytes_per_cached_token": 132, "input_copies": copies8,
            "fp4_vs_fp8_step_speedup": round(ms8 / ms_per_step, 3)}
        log(f"[bench] fp8 cache: {ms8 * 1e3:.1f} us/step, logits {pk8['mqa_logits'] * 1e3:.1f} us "
            f"({time.time() - t0:.1f}s)")

    # ---- the fused logits + top-k call on the same workload (FP4 cache, no logits in memory)
    if not args.no_fused and wl.heads <= 64 and wl.max_ctx <= F.FUSED_MAX_CTX:
        msf, pkf, copiesf, _ = run_cache(False, dict(payload=payload, scale=scale), fused=True)
        extras["fused_logits_topk"] = {
            "ms_per_step": round(msf, 4), "scores_per_s": round(scores / (msf * 1e-3), 1),
            "kernels_us": {n: round(v * 1e3, 2) for n, v in pkf.items()},
            "two_call_logits_plus_topk_us": round((per_kernel_ms["mqa_logits"] + per_kernel_ms["topk"]) * 1e3, 2),
            "step_speedup_vs_two_calls": round(ms_per_step / msf, 3), "input_copies": copiesf}
        log(f"[bench] fused logits+top-k: {msf * 1e3:.1f} us/step, kernel {pkf['mqa_logits_topk'] * 1e3:.1f} us "
            f"({time.time() - t0:.1f}s)")

    # ---- CPU baseline: the oracle on the same workload (bounded sample)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as orc
        tabn = W.rope_table(wl.max_pos)
        budget_scores = 8_000_000
        rows = np.arange(T)
        if scores > budget_scores:   # whole requests, taken in order, up to the budget
            acc, last = 0, 0
            for b in range(wl.n_reqs):
                acc += int(wl.row_ctx[wl.req_row_indptr[b]:wl.req_row_indptr[b + 1]].sum())
                last = b + 1
                if acc >= budget_scores:
                    break
            rows = np.arange(wl.req_row_indptr[last])
        n_rows_s = rows.size
        s_scores = int(wl.row_ctx[rows].sum())
        nb = int(np.searchsorted(wl.req_row_indptr, n_rows_s, side="left"))
        ind = wl.req_row_indptr[:nb + 1].copy()
        # the oracle's own pool, from the same generator inputs (untimed set-up)
        pay_np = np.zeros(wl.num_pages * 4096, np.uint8)
        sc_np = np.zeros(wl.num_pages * 256, np.uint8)
        if wl.cached_slots.size:
            kc = wl.cached_k()
            pages_used = set(np.unique(wl.block_table[:nb][wl.block_table[:nb] >= 0]).tolist())
            keep = np.isin(wl.cached_slots // 64, np.fromiter(pages_used, np.int64))
            orc.write_k(kc[keep], wl.cached_pos[keep], wl.cached_slots[keep], wl.norm_w, wl.eps, tabn, pay_np, sc_np)
            del kc
        # timed: the sampled step on the oracle, repeated until about 10 s of CPU wall time
        secs = np.zeros(4)
        reps = 0
        while reps < 200 and (reps == 0 or secs.sum() < 10.0):
            c0 = time.perf_counter()
            orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tabn, pay_np, sc_np)
            c1 = time.perf_counter()
            qf, qs, wo = orc.pack_q(wl.q[rows], wl.pos_q[rows], tabn, wl.w[rows], wl.w_scale)
            c2 = time.perf_counter()
            lg = orc.logits(qf, qs, wo, ind, wl.row_ctx[rows], wl.block_table[:nb], pay_np, sc_np,
                            logits_stride=wl.max_ctx)
            c3 = time.perf_counter()
            orc.topk(np.nan_to_num(lg), wl.row_ctx[rows], k)
            c4 = time.perf_counter()
            secs += (c1 - c0, c2 - c1, c3 - c2, c4 - c3)
            reps += 1
        secs /= reps
        cpu_s = secs[0] * (n_rows_s / T) + secs[1:].sum()
        # the same sampled step once more on one host thread
        threads = orc.get_threads()
        orc.set_threads(1)
        c0 = time.perf_counter()
        orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tabn, pay_np, sc_np)
        c1 = time.perf_counter()
        qf, qs, wo = orc.pack_q(wl.q[rows], wl.pos_q[rows], tabn, wl.w[rows], wl.w_scale)
        lg1 = orc.logits(qf, qs, wo, ind, wl.row_ctx[rows], wl.block_table[:nb], pay_np, sc_np,
                         logits_stride=wl.max_ctx)
        orc.topk(np.nan_to_num(lg1), wl.row_ctx[rows], k)
        c2 = time.perf_counter()
        orc.set_threads(threads)
        cpu1_s = (c1 - c0) * (n_rows_s / T) + (c2 - c1)
        del lg1
        cpu = {"value": round(s_scores / cpu_s, 1), "unit": "scores/s", "cores": orc.get_threads(), "kind": "oracle",
               "sample": f"{n_rows_s} of {T} rows ({s_scores} scores): the step's K write (pro rata), pack_q, "
                         f"logits and top-k on the oracle, run {reps} times ({reps * cpu_s:.1f}s of CPU wall time); "
                         f"value = scores / mean time per run",
               "seconds_per_run": {n: round(float(v), 4) for n, v in zip(names, secs)},
               "single_thread": {"value": round(s_scores / cpu1_s, 1), "cores": 1,
                                 "sample": "the same sampled step, run once on one host thread"}}
        del pay_np, sc_np, lg

    out = {
        "metric": "indexer scores/sec (q-row x token) + K-write tokens/sec; % HBM / FP4-MFMA peak",
        "value": round(value, 1),
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1, fp32 accumulate); fp32 encoders",
        "data": "synthetic",
        "config": {"workload": wl.name, "launch": ("prepared calls" if args.launch == "prepared" else "hip graph per step")
                   + ": write_k+pack_q in one launch, logits, top-k", "requests": wl.n_reqs, "rows": T, "heads": H, "head_dim": 128,
                   "scores_per_step": scores, "k_write_tokens_per_step": int(wl.k_new.shape[0]), "topk": k,
                   "pool_pages": wl.num_pages, "input_copies": copies},
        "k_write_tokens_per_s": round(wl.k_new.shape[0] / (per_kernel_ms["write_k"] * 1e-3), 1),
        "kernels_us": {n: round(v * 1e3, 2) for n, v in per_kernel_ms.items()},
        "kernels_us_median_min": {n: [round(a * 1e3, 2), round(b * 1e3, 2)] for n, (a, b) in per_kernel_stats.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
