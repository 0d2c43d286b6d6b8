"""Benchmark of the FP4 lightning-indexer hot path on one MI355X.

A step is one pass of the whole path over one batch: the fused K writer for
the step's new compressed tokens, the index-Q pack, the paged FP4 logits over
every cached token of every row, and the per-row top-k.  The headline
workload (the JSON line's value, config and roofline) is the prefill batch:
one request of 4,096 query rows with causal limits over 16,384 cached
compressed tokens plus a fused K write of 1,024 new ones, top-k 2048.  The
other four workloads (tiny decode, decode batch 64, decode 256 x 6, the mixed
agentic batch with its 65,536-token bulk K write) are timed the same way and
reported under extras.configs, each with its own roofline fraction.

Inputs are synthetic and seeded; the page pool is filled before timing by the
library's own K writer.  Every timed step reads a different copy of the
inputs (copies total well above the 256 MB last-level cache), so the HBM
figures are HBM, not cache.  A timed step is three launches in sequence (the
K write and Q pack together in one launch, the logits, the top-k), issued as
prepared library calls (arguments marshalled once per input copy, one ctypes
call per launch) or, with `--launch graph`, as a replay of a HIP graph
captured per input copy.  Per-kernel durations come from a second pass over
the same K steps, launched eagerly with the two encoders as separate
kernels, where each kernel carries HIP events that its own dispatch stamps
with its start and end times (fp4idx_time_next_call -> hipExtLaunchKernel).

The first tens of milliseconds of a heavy step after idle run below the
GPU's steady clock (its power management dips, then recovers over about a
hundred prefill steps), and the W + K steps fall inside that transient.  So
each workload's record also holds a `sustained` rate: the same K steps timed
again after at least 60 ms of further untimed steps, and then K steps with
the logits schedule built once and reused (one plan serves every
compressed-attention layer of a step).  The JSON line's value is the K steps
right after the W warm-up steps, the schedule built in every step.

Roofline of a kernel: its algorithmic bytes at 8 TB/s and its FP4 MFMA flop
at 10.1 PFLOP/s give a roofline time max(bytes / BW, flop / P); the fraction
is that time over the measured time, and the bound is the larger term.  The
fp32 VALU work of the logits epilogue is reported beside it (secondary).

For the headline workload the same step is also timed with the logits and
the top-k as one fused call (extras.fused_logits_topk) and on the FP8
indexer cache (extras.fp8_cache).  The oracle is timed on a bounded row
sample of the headline step on the host's cores (cpu_baseline).

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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
HEADLINE = 3
NAMES = ("write_k", "pack_q", "plan", "mqa_logits", "topk")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _strip_c_comments(text: str) -> str:
    """C/C++ source without its comments (string and character literals kept
    whole): each comment replaced by one space, trailing spaces and blank
    lines dropped."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return "\n".join(line.rstrip() for line in "".join(out).split("\n") if line.strip())


def kernel_source_hash() -> str:
    """Digest of everything the kernels are compiled from (HIP sources and
    headers without their comments, build flags): the key of the stored
    counter readings, which a change of the compiled code makes stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_fp4_fp4idx_amd", "csrc")
    files = [os.path.join(csrc, f) for f in sorted(os.listdir(csrc))]
    files += [os.path.join(ROOT, "sparse_attention_fp4_fp4idx_amd", "build.py"), os.path.join(ROOT, "include", "fp4idx.h")]
    for f in files:
        if os.path.isfile(f):
            h.update(os.path.basename(f).encode())
            data = open(f, "rb").read()
            if f.endswith((".hip", ".hpp", ".h")):
                data = _strip_c_comments(data.decode()).encode()
            h.update(data)
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def unique_k_tokens(wl) -> int:
    """K tokens the logits must read once: for every physical page any
    request's rows reach, the most tokens of it any of those requests needs
    (a prefix page shared through several block tables counts once)."""
    need = {}
    for b in range(wl.n_reqs):
        c = int(np.max(wl.row_ctx[wl.req_row_indptr[b]:wl.req_row_indptr[b + 1]], initial=0))
        for p in range((c + 63) // 64):
            pid = int(wl.block_table[b, p])
            need[pid] = max(need.get(pid, 0), min(64, c - 64 * p))
    return int(sum(need.values()))


def algorithmic(wl) -> dict:
    """Per kernel of one step: (HBM bytes, FP4 MFMA flop, fp32 VALU lane-ops)."""
    T, H, k, S = wl.n_rows, wl.heads, wl.topk, wl.scores
    uk = unique_k_tokens(wl)
    pages = (uk + 63) // 64
    return {"write_k": (460 * wl.k_new.shape[0] + 256, 0, 0),
            "pack_q": (21380 * T * H // 64, 0, 0),
            "mqa_logits": (68 * uk + 4 * S + 4608 * T * H // 64 + 4 * pages, 2 * 128 * H * S, 2 * H * S),
            "topk": (4 * S + 4 * k * T, 0, 0),
            "unique_k_tokens": uk}


def roofline_of(kernel, alg, us, measured=None, traffic=None):
    """The kernel against HBM and FP4 MFMA: roofline time = max(bytes / BW,
    flop / peak), fraction = roofline time / measured time; the bound is the
    larger term.  The fp32 VALU epilogue (logits) is a secondary figure."""
    nbytes, flop, lops = alg[kernel]
    t = us * 1e-6
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = flop / (MFMA_FP4_PEAK_TFLOPS * 1e12)
    bound = "mfma" if t_mfma > t_hbm else "hbm"
    frac = max(t_hbm, t_mfma) / t
    rec = {"kernel": kernel, "bound": bound,
           "achieved": round(flop / t / 1e12 if bound == "mfma" else nbytes / t / 1e9, 1),
           "peak": MFMA_FP4_PEAK_TFLOPS if bound == "mfma" else HBM_PEAK_GBS,
           "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(frac, 4), "traffic": traffic,
           "alg_bytes_per_launch": int(nbytes), "mfma_flop_per_launch": int(flop), "avg_launch_us": round(us, 2),
           "fractions": {"hbm": round(t_hbm / t, 4), "mfma": round(t_mfma / t, 4)}}
    if lops:
        t_alu = lops / (VALU_PEAK_TOPS * 1e12)
        rec["secondary"] = {"alu": round(t_alu / t, 4), "mfma_plus_alu": round((t_mfma + t_alu) / t, 4),
                            "note": "fp32 VALU epilogue (ReLU + FMA per head and score) at 39.3 T lane-ops/s; "
                                    "mfma_plus_alu = (MFMA time + VALU time at peak) / measured time, the two "
                                    "pipes of a SIMD largely taking turns"}
        if measured:
            tm = flop / (measured["mfma_fp4_TFLOPs"] * 1e12)
            ta = lops / (measured["valu_fp32_Tlane_ops"] * 1e12)
            th = nbytes / (measured["hbm_read_GBs"] * 1e9)
            rec["secondary"]["vs_measured_peaks"] = {"hbm": round(th / t, 4), "mfma": round(tm / t, 4),
                                                     "alu": round(ta / t, 4), "mfma_plus_alu": round((tm + ta) / t, 4)}
    elif measured:
        rec["frac_vs_measured_hbm_read"] = round(nbytes / (measured["hbm_read_GBs"] * 1e9) / t, 4)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=HEADLINE, help="headline workload index (3 = prefill)")
    ap.add_argument("--only", action="store_true", help="time the headline workload only (no extras.configs)")
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
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported. Across GPUs "
              "the path shards by request (no exchange) or, for long rows, by context (one all-gather of each "
              "row's local top-k candidates before a final selection).", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_fp4_fp4idx_amd import fp4idx as F
    from sparse_attention_fp4_fp4idx_amd import workloads as W

    F.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    t0 = time.time()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def b16(a):
        return t(a.view(np.int16)).view(torch.bfloat16)

    def event_pairs(n):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a_, b_ in ev:   # torch creates the HIP events on first record
            a_.record(stream)
            b_.record(stream)
        return ev

    if args.calib_copy:
        # reference for rocprofv3 FETCH_SIZE / WRITE_SIZE: reads and writes exactly MB MiB
        csrc = torch.empty(args.calib_copy << 20, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        for _ in range(3):
            cdst.copy_(csrc)
        torch.cuda.synchronize()
        del csrc, cdst

    # ---- measured peaks (the library's microbenchmarks): FP4 MFMA, streaming HBM read, fp32 VALU
    measured = None
    if not args.no_peaks:
        sink_f = torch.zeros(1, dtype=torch.float32, device=dev)
        sink_u = torch.zeros(1, dtype=torch.int32, device=dev)
        big = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        big.fill_(1)
        pev, vev = event_pairs(8), event_pairs(4)
        mev = [event_pairs(4) for _ in range(3)]
        F.peak_mfma_fp4(64, sink_f, stream=stream)
        F.peak_read(big, sink_u, stream=stream)
        F.peak_valu_fp32(64, sink_f, stream=stream)
        for m in range(3):
            F.peak_mfma_valu(m, 16, sink_f, stream=stream)
        torch.cuda.synchronize()
        flop, nbytes, lops = [0] * 4, [0] * 4, [0] * 4
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

    def bench_config(idx: int, headline: bool):
        """Time one workload: the FP4 step (prepared calls or graph replays),
        then the dispatch-stamped kernel pass; for the headline workload also
        the fused and FP8 legs and the reader.  Returns (record, wl, pool)."""
        wl = W.make(idx)
        log(f"[bench] workload {idx}: {wl.name}: rows {wl.n_rows} reqs {wl.n_reqs} scores {wl.scores} "
            f"pages {wl.num_pages} new tokens {wl.k_new.shape[0]} ({time.time() - t0:.1f}s)")
        tab = b16(W.rope_table(wl.max_pos))
        norm_w = b16(wl.norm_w)
        payload = torch.zeros(wl.num_pages * 4096, dtype=torch.uint8, device=dev)
        scale = torch.zeros(wl.num_pages * 256, dtype=torch.uint8, device=dev)
        if wl.cached_slots.size:   # fill the pool with encoded cached tokens (untimed)
            kc = wl.cached_k()
            for a in range(0, kc.shape[0], 1 << 20):
                F.write_k(b16(kc[a:a + (1 << 20)]), t(wl.cached_pos[a:a + (1 << 20)]),
                          t(wl.cached_slots[a:a + (1 << 20)]), norm_w, wl.eps, tab, payload, scale)
            del kc
        torch.cuda.synchronize()
        T, H, k = wl.n_rows, wl.heads, wl.topk
        pos_new, slot_new = t(wl.pos_new), t(wl.slot_new)
        pos_q, indptr, ctx, bt = t(wl.pos_q), t(wl.req_row_indptr), t(wl.row_ctx), t(wl.block_table)

        def run_cache(fp8: bool, pools: dict, fused: bool = False):
            """Rotating input copies, the timed steps, then the per-kernel
            event pass.  Returns (ms_per_step, per-kernel ms, copies, stats)."""
            qcode_b = 128 if fp8 else 64
            base = dict(pools, q=b16(wl.q), w=t(wl.w), k_new=b16(wl.k_new))
            step_bytes = sum(v.numel() * v.element_size() for v in base.values()) + T * wl.max_ctx * 4 * 2
            copies = args.copies or max(2, int(np.ceil(2 * CACHE_BYTES / step_bytes)))
            copies = min(copies, max(2, int(0.5 * torch.cuda.mem_get_info()[0] // step_bytes)))
            sets = []
            for c in range(copies):
                s = {n: (v if c == 0 else v.clone()) for n, v in base.items()}
                s["logits"] = torch.empty((T, wl.max_ctx), dtype=torch.float32, device=dev)
                s["ws"] = F.new_workspace(T, wl.n_reqs, wl.max_ctx, dev)
                s["q_code"] = torch.empty((T, H, qcode_b), dtype=torch.uint8, device=dev)
                s["q_scale"] = (torch.empty((T, H), dtype=torch.float32, device=dev) if fp8
                                else torch.empty((T, H, 4), dtype=torch.uint8, device=dev))
                s["w_out"] = torch.empty((T, H), dtype=torch.float32, device=dev)
                s["top"] = torch.empty((T, k), dtype=torch.int32, device=dev)
                sets.append(s)

            def pool_args(s):
                return (s["pool"],) if fp8 else (s["payload"], s["scale"])

            def step(s, strm, ev=None):
                """One pass of the path on stream strm.  The timed steps encode
                the step's K tokens and query rows in one launch and the FP4
                logits as one call (its schedule, then the scheduled kernel);
                the kernel pass (ev given) launches the two encoders, and the
                schedule and the logits kernel, separately so that each kernel
                gets its own duration, and times the host-bounded logits call
                after the step for comparison."""
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
                if fused:
                    arm(3)
                    F.mqa_logits_topk(s["q_code"], s["q_scale"], s["w_out"], indptr, ctx, bt, *pool_args(s), k,
                                      wl.max_rows_per_req, wl.max_ctx, out_idx=s["top"], stream=strm)
                    return
                if fp8:
                    arm(3)
                    F.mqa_logits_fp8(s["q_code"], s["q_scale"], s["w_out"], indptr, ctx, bt, *pool_args(s),
                                     wl.max_rows_per_req, wl.max_ctx, logits=s["logits"], stream=strm)
                elif ev is None:
                    F.mqa_logits(s["q_code"], s["q_scale"], s["w_out"], indptr, ctx, bt, *pool_args(s),
                                 logits=s["logits"], workspace=s["ws"], stream=strm)
                else:
                    plan = F.LogitsPlan(H, indptr, ctx, wl.max_ctx, workspace=s["ws"], stream=strm)
                    arm(2)
                    plan.build()
                    arm(3)
                    plan.run(s["q_code"], s["q_scale"], s["w_out"], bt, *pool_args(s), logits=s["logits"],
                             stream=strm)
                arm(4)
                F.topk(s["logits"], ctx, k, wl.max_ctx, out_idx=s["top"], stream=strm)
                if ev is not None and not fp8:
                    arm(5)
                    F.mqa_logits_bounded(s["q_code"], s["q_scale"], s["w_out"], indptr, ctx, bt, *pool_args(s),
                                         wl.max_rows_per_req, wl.max_ctx, logits=s["logits"], stream=strm)

            for i in range(args.warmup):
                step(sets[i % copies], stream)
            torch.cuda.synchronize()
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
                prepared = []
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
                        if fp8:
                            pl, _ = F.prepare_mqa_logits_fp8(s_["q_code"], s_["q_scale"], s_["w_out"], indptr, ctx,
                                                             bt, *pool_args(s_), wl.max_rows_per_req, wl.max_ctx,
                                                             logits=s_["logits"], stream=stream)
                        else:
                            pl, _ = F.prepare_mqa_logits(s_["q_code"], s_["q_scale"], s_["w_out"], indptr, ctx, bt,
                                                         *pool_args(s_), logits=s_["logits"], workspace=s_["ws"],
                                                         stream=stream)
                        pt, _ = F.prepare_topk(s_["logits"], ctx, k, wl.max_ctx, out_idx=s_["top"], stream=stream)

                    def run(pw=pw, pl=pl, pt=pt):
                        pw()
                        pl()
                        pt()
                    runners.append(run)
                    prepared.append((pw, pt))
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

            # Sustained rate: the GPU's power management slows the first tens of
            # milliseconds of a heavy step after idle (a dip below, then a slow
            # recovery to, its steady clock), so the same steps are timed again after
            # at least 60 ms (at most 400 steps) of further untimed steps; then with
            # the schedule built once per input copy and reused (one plan serves every
            # layer of a step), timed in the same regime.
            sustained = None
            if args.launch == "prepared" and not fp8 and not fused:
                n_more = int(min(400, max(args.steps, np.ceil(60.0 / max(elapsed * 1e3 / args.steps, 1e-3)))))
                for i in range(n_more):
                    runners[i % copies]()
                torch.cuda.synchronize()
                start = time.perf_counter()
                for i in range(args.steps):
                    runners[i % copies]()
                torch.cuda.synchronize()
                sustained = {"ms_per_step": (time.perf_counter() - start) * 1e3 / args.steps,
                             "untimed_steps_before": args.warmup + copies + args.steps + n_more}
                reused = []
                for c in range(copies):
                    s_ = sets[c]
                    plan = F.LogitsPlan(H, indptr, ctx, wl.max_ctx, workspace=s_["ws"], stream=stream).build()
                    pr, _ = plan.prepare_run(s_["q_code"], s_["q_scale"], s_["w_out"], bt, *pool_args(s_),
                                             logits=s_["logits"], stream=stream)
                    pw, pt = prepared[c]

                    def run_reused(pw=pw, pr=pr, pt=pt):
                        pw()
                        pr()
                        pt()
                    reused.append(run_reused)
                for c in range(copies):
                    reused[c]()
                torch.cuda.synchronize()
                start = time.perf_counter()
                for i in range(args.steps):
                    reused[i % copies]()
                torch.cuda.synchronize()
                sustained["plan_reused_ms_per_step"] = (time.perf_counter() - start) * 1e3 / args.steps
                del reused

            # kernel durations: the same K steps launched eagerly, each kernel carrying
            # HIP events its own dispatch stamps (no marker packets in between)
            evs = [event_pairs(len(NAMES) + 1) for _ in range(args.steps)]
            torch.cuda.synchronize()
            for i in range(args.steps):
                step(sets[i % copies], stream, evs[i])
            torch.cuda.synchronize()
            if fused:
                used = {"write_k": 0, "pack_q": 1, "mqa_logits_topk": 3}
            elif fp8:
                used = {"write_k": 0, "pack_q": 1, "mqa_logits": 3, "topk": 4}
            else:
                used = {"write_k": 0, "pack_q": 1, "plan": 2, "mqa_logits": 3, "topk": 4, "mqa_logits_bounded": 5}
            times = {n: [evs[i][j][0].elapsed_time(evs[i][j][1]) for i in range(args.steps)] for n, j in used.items()}
            per_kernel = {n: float(np.mean(v)) for n, v in times.items()}
            stats = {n: (float(np.median(v)), float(np.min(v))) for n, v in times.items()}
            del sets, runners
            return elapsed * 1e3 / args.steps, per_kernel, copies, stats, sustained

        ms, pk, copies, stats, sustained = run_cache(False, dict(payload=payload, scale=scale))
        alg = algorithmic(wl)
        kus = {n: v * 1e3 for n, v in pk.items()}
        bounded_us = kus.pop("mqa_logits_bounded")   # not part of the step
        dom = max((n for n in kus if n in alg), key=kus.get)   # the schedule's own kernel has no roofline
        key = f"config{idx}:{dom}"
        rec = {"workload": wl.name, "ms_per_step": round(ms, 4), "scores_per_step": wl.scores,
               "scores_per_s": round(wl.scores / (ms * 1e-3), 1), "rows": T, "requests": wl.n_reqs,
               "k_write_tokens_per_step": int(wl.k_new.shape[0]),
               "kernels_us": {n: round(v, 2) for n, v in kus.items()},
               "kernels_us_median_min": {n: [round(a * 1e3, 2), round(b * 1e3, 2)] for n, (a, b) in stats.items()},
               "roofline": roofline_of(dom, alg, kus[dom], measured, measured_traffic(key)),
               "k_write": {"tokens": int(wl.k_new.shape[0]),
                           "tokens_per_s": round(wl.k_new.shape[0] / (kus["write_k"] * 1e-6), 1),
                           "roofline": roofline_of("write_k", alg, kus["write_k"], measured)},
               "unique_k_tokens": alg["unique_k_tokens"], "input_copies": copies,
               "logits_host_bounded_us": round(bounded_us, 2)}
        if sustained is not None:
            sm, rm = sustained["ms_per_step"], sustained["plan_reused_ms_per_step"]
            rec["sustained"] = {
                "ms_per_step": round(sm, 4), "scores_per_s": round(wl.scores / (sm * 1e-3), 1),
                "plan_reused_ms_per_step": round(rm, 4), "plan_reused_scores_per_s": round(wl.scores / (rm * 1e-3), 1),
                "untimed_steps_before": sustained["untimed_steps_before"],
                "note": "the same K steps timed again after further untimed steps (at least 60 ms of them), past "
                        "the power-management transient of the first steps after idle; then K steps with the "
                        "schedule built once and reused (one plan serves every compressed-attention layer of a "
                        "step). ms_per_step and value above are the K steps right after the W warm-up steps"}
        if dom != "mqa_logits":
            rec["logits_roofline"] = roofline_of("mqa_logits", alg, kus["mqa_logits"], measured,
                                                 measured_traffic(f"config{idx}:mqa_logits"))
        rec["topk_roofline"] = roofline_of("topk", alg, kus["topk"], measured)
        log(f"[bench] workload {idx}: {ms * 1e3:.1f} us/step, kernels " +
            ", ".join(f"{n} {v:.1f}" for n, v in kus.items()) + f" us ({time.time() - t0:.1f}s)")
        if sustained is not None:
            log(f"[bench] workload {idx}: sustained {sustained['ms_per_step'] * 1e3:.1f} us/step after "
                f"{sustained['untimed_steps_before']} untimed steps, "
                f"{sustained['plan_reused_ms_per_step'] * 1e3:.1f} us/step with the schedule reused")

        if headline:
            extras = {}
            if wl.cached_slots.size:   # the split-pool reader over every cached token, one launch
                rslots = t(wl.cached_slots)
                rout = torch.empty((rslots.numel(), 128), dtype=torch.float32, device=dev)
                rev = event_pairs(5)
                F.read_k(payload, scale, rslots, out=rout, stream=stream)      # warm-up
                torch.cuda.synchronize()
                for a, b in rev:
                    F.time_next_call(a, b)
                    F.read_k(payload, scale, rslots, out=rout, stream=stream)
                torch.cuda.synchronize()
                r_ms = float(np.median([a.elapsed_time(b) for a, b in rev]))
                r_bytes = 584 * rslots.numel()   # 64 code + 4 scale + 4 slot bytes read, 512 written per token
                extras["read_k"] = {"tokens": int(rslots.numel()), "us": round(r_ms * 1e3, 2),
                                    "GB/s": round(r_bytes / (r_ms * 1e-3) / 1e9, 1),
                                    "hbm_frac": round(r_bytes / (r_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
                del rout
            if not args.no_fp8:   # the FP8 indexer cache (132-byte fused tokens): same step, same timing
                pool8 = torch.zeros(wl.num_pages * W.FP8_PAGE_BYTES, dtype=torch.uint8, device=dev)
                if wl.cached_slots.size:
                    kc = wl.cached_k()
                    for a in range(0, kc.shape[0], 1 << 20):
                        F.write_k_fp8(b16(kc[a:a + (1 << 20)]), t(wl.cached_pos[a:a + (1 << 20)]),
                                      t(wl.cached_slots[a:a + (1 << 20)]), norm_w, wl.eps, tab, pool8)
                    del kc
                torch.cuda.synchronize()
                ms8, pk8, copies8, _, _ = run_cache(True, dict(pool=pool8))
                del pool8
                uk = alg["unique_k_tokens"]
                l8 = 132 * uk + 4 * wl.scores + 8704 * T + 4 * ((uk + 63) // 64)
                t8 = pk8["mqa_logits"] * 1e-3
                extras["fp8_cache"] = {
                    "ms_per_step": round(ms8, 4), "scores_per_s": round(wl.scores / (ms8 * 1e-3), 1),
                    "kernels_us": {n: round(v * 1e3, 2) for n, v in pk8.items()},
                    "logits_roofline": {
                        "hbm": round(l8 / t8 / 1e9 / HBM_PEAK_GBS, 4),
                        "mfma_fp8": round(2 * 128 * H * wl.scores / t8 / 1e12 / (MFMA_FP4_PEAK_TFLOPS / 2), 4),
                        "alg_bytes_per_launch": l8,
                        "note": "FP8 MFMA at half the FP4 rate (5.05 PFLOP/s dense)",
                        "traffic": measured_traffic(f"config{idx}:fp8_mqa_logits")},
                    "bytes_per_cached_token": 132, "input_copies": copies8,
                    # both legs timed past the power transient: the FP4 sustained step
                    "fp4_vs_fp8_step_speedup": round(ms8 / (sustained["ms_per_step"] if sustained else ms), 3)}
                log(f"[bench] fp8 cache: {ms8 * 1e3:.1f} us/step, logits {pk8['mqa_logits'] * 1e3:.1f} us "
                    f"({time.time() - t0:.1f}s)")
            if not args.no_fused and wl.heads <= 64 and wl.max_ctx <= F.FUSED_MAX_CTX:
                msf, pkf, copiesf, _, _ = run_cache(False, dict(payload=payload, scale=scale), fused=True)
                extras["fused_logits_topk"] = {
                    "ms_per_step": round(msf, 4), "scores_per_s": round(wl.scores / (msf * 1e-3), 1),
                    "kernels_us": {n: round(v * 1e3, 2) for n, v in pkf.items()},
                    "two_call_logits_plus_topk_us": round(kus["mqa_logits"] + kus["topk"], 2),
                    "step_speedup_vs_two_calls": round((sustained["ms_per_step"] if sustained else ms) / msf, 3),
                    "input_copies": copiesf}
                log(f"[bench] fused logits+top-k: {msf * 1e3:.1f} us/step, kernel "
                    f"{pkf['mqa_logits_topk'] * 1e3:.1f} us ({time.time() - t0:.1f}s)")
            rec["extras"] = extras
        del payload, scale
        torch.cuda.empty_cache()
        return rec, wl

    head, wl = bench_config(args.config, True)
    configs = {}
    if not args.only:
        for idx in range(5):
            if idx != args.config:
                configs[f"config{idx}"] = bench_config(idx, False)[0]

    # ---- CPU baseline: the oracle on a bounded row sample of the headline step
    cpu = None
    if not args.no_cpu_baseline:
        import oracle as orc
        tabn = W.rope_table(wl.max_pos)
        T, k = wl.n_rows, wl.topk
        # rows spread over the batch (every request keeps its block table row), about 1.5 M scores
        n_s = int(min(T, max(1, 1_500_000 * T // max(1, wl.scores))))
        rows = np.unique(np.linspace(0, T - 1, n_s).astype(np.int64))
        req = np.searchsorted(wl.req_row_indptr, rows, side="right") - 1
        reqs = np.unique(req)
        ind = np.concatenate([[0], np.cumsum([np.sum(req == b) for b in reqs])]).astype(np.int32)
        bts = wl.block_table[reqs]
        s_ctx = wl.row_ctx[rows]
        s_scores = int(s_ctx.astype(np.int64).sum())
        # the oracle's own pool, from the same generator inputs (untimed set-up)
        pay_np = np.zeros(wl.num_pages * 4096, np.uint8)
        sc_np = np.zeros(wl.num_pages * 256, np.uint8)
        if wl.cached_slots.size:
            kc = wl.cached_k()
            used = np.unique(bts[bts >= 0])
            keep = np.isin(wl.cached_slots // 64, used)
            orc.write_k(kc[keep], wl.cached_pos[keep], wl.cached_slots[keep], wl.norm_w, wl.eps, tabn, pay_np, sc_np)
            del kc
        secs = np.zeros(4)
        reps = 0
        while reps < 100 and (reps == 0 or secs.sum() < 10.0):   # about 10 s of host time
            c0 = time.perf_counter()
            orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tabn, pay_np, sc_np)
            c1 = time.perf_counter()
            qf, qs, wo = orc.pack_q(wl.q[rows], wl.pos_q[rows], tabn, wl.w[rows], wl.w_scale)
            c2 = time.perf_counter()
            lg = orc.logits(qf, qs, wo, ind, s_ctx, bts, pay_np, sc_np, logits_stride=wl.max_ctx)
            c3 = time.perf_counter()
            orc.topk(np.nan_to_num(lg), s_ctx, k)
            c4 = time.perf_counter()
            secs += (c1 - c0, c2 - c1, c3 - c2, c4 - c3)
            reps += 1
        secs /= reps
        # per sampled step: the K write pro rata to the sampled rows, the rest as measured
        cpu_s = secs[0] * (rows.size / T) + secs[1:].sum()
        # the same sampled step once more on one host thread
        n_thr = orc.get_threads()
        orc.set_threads(1)
        try:
            c0 = time.perf_counter()
            orc.write_k(wl.k_new, wl.pos_new, wl.slot_new, wl.norm_w, wl.eps, tabn, pay_np, sc_np)
            c1 = time.perf_counter()
            qf, qs, wo = orc.pack_q(wl.q[rows], wl.pos_q[rows], tabn, wl.w[rows], wl.w_scale)
            lg = orc.logits(qf, qs, wo, ind, s_ctx, bts, pay_np, sc_np, logits_stride=wl.max_ctx)
            orc.topk(np.nan_to_num(lg), s_ctx, k)
            c2 = time.perf_counter()
        finally:
            orc.set_threads(n_thr)
        one_s = (c1 - c0) * (rows.size / T) + (c2 - c1)
        cpu = {"value": round(s_scores / cpu_s, 1), "unit": "scores/s", "cores": orc.get_threads(), "kind": "oracle",
               "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
               "sample": f"{rows.size} of {T} rows spread evenly over the batch ({s_scores} scores, "
                         f"{reps} runs, {reps * cpu_s:.1f} s of host wall time): the step's K write pro rata, "
                         f"pack_q, logits and top-k of those rows on the oracle; value = sampled scores / "
                         f"mean time per run",
               "seconds_per_run": {n: round(float(v), 4)
                                   for n, v in zip(("write_k", "pack_q", "mqa_logits", "topk"), secs)},
               "single_thread": {"value": round(s_scores / one_s, 1), "cores": 1,
                                 "sample": "the same sampled step, run once on one host thread"}}
        log(f"[bench] cpu baseline: {cpu['value'] / 1e6:.2f} M scores/s on {cpu['cores']} threads, "
            f"{cpu['single_thread']['value'] / 1e6:.2f} M on one ({time.time() - t0:.1f}s)")
        del pay_np, sc_np, lg

    out = {
        "metric": "indexer scores/sec (q-row x token) + K-write tokens/sec; % HBM / FP4-MFMA peak",
        "value": head["scores_per_s"],
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4 (e2m1 x e2m1, fp32 accumulate); fp32 encoders",
        "data": "synthetic",
        "config": {"workload": head["workload"],
                   "launch": ("prepared calls" if args.launch == "prepared" else "hip graph per step")
                   + ": write_k+pack_q in one launch, logits, top-k",
                   "requests": head["requests"], "rows": head["rows"], "heads": wl.heads, "head_dim": 128,
                   "scores_per_step": head["scores_per_step"], "k_write_tokens_per_step": head["k_write_tokens_per_step"],
                   "topk": wl.topk, "pool_pages": wl.num_pages, "input_copies": head["input_copies"]},
        "k_write_tokens_per_s": head["k_write"]["tokens_per_s"],
        "kernels_us": head["kernels_us"],
        "kernels_us_median_min": head["kernels_us_median_min"],
        "roofline": dict(head["roofline"], measured_peaks=measured),
        "cpu_baseline": cpu,
        "extras": dict(head.get("extras", {}), configs=configs,
                       headline_topk_roofline=head["topk_roofline"], headline_k_write=head["k_write"],
                       headline_sustained=head.get("sustained")),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
