"""Throughput of the ShadowKV sparse decode step on one MI355X.

A step is one decode step of the model: every layer's shadowkv_decode_step
(score landmarks, group score, select top-k chunks, set-difference cache
update, host-V fetch of the misses, MFMA key rebuild + RoPE + logits, PV and
combine) for all b sequences, one token each.  The metric is
layer-steps/s (one layer-step = one shadowkv_decode_step call) with the
effective HBM bandwidth (algorithmic bytes / time) and the equivalent
bandwidth (dense K+V bytes / time, the review page's B~ measured).

Inputs are seeded synthetic arrays with the workload's shapes, generated on
the device; the low-rank factors, prefill metadata and the pinned host V are
built before the timed region (prefill is not part of the metric).  Queries
for every timed step are resident in HBM before timing starts.  The host-V
fetch over PCIe is a step of the method itself (Algorithm 2 step 3), so it is
inside the timed region.

Output: one JSON line on stdout (progress goes to stderr).

Traffic counters: run the bench twice under `rocprofv3 --pmc FETCH_SIZE`
and `--pmc WRITE_SIZE` (CSV output) with --copy-calibration, which adds a
device copy of known size; `bench.py --ingest-counters FETCH.csv WRITE.csv`
then writes profiles/traffic_score_<workload>.json (bytes per launch of the
scoring kernel, each counter scaled by what it reads for the copy), which
later bench lines report as roofline.traffic while the kernel sources are
unchanged.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12       # bytes/s, MI355X HBM3E
PEAK_PCIE = 64.0e9      # bytes/s per direction, PCIe Gen5 x16


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(wl) -> dict:
    """Bytes one layer-step must move at minimum, by kernel (bf16: 2 B)."""
    E = 2 if wl.bf16 else 4
    bh = wl.b * wl.h_kv
    return {
        "landmarks": bh * wl.n * wl.d * E,                    # score: all of L
        "q": wl.b * wl.h_q * wl.d * E,
        "a_rows": bh * wl.k * wl.c * wl.r * E,                # rebuild: gathered A rows
        "b_factor": bh * wl.r * wl.d * E,
        "outlier_kv": 2 * bh * wl.o * wl.c * wl.d * E,
        "local_kv": 2 * bh * wl.w * wl.d * E,
        "selected_v": bh * wl.k * wl.c * wl.d * E,
        "out": wl.b * wl.h_q * wl.d * E,
    }


# The sources a kernel's traffic record depends on: the kernel function's
# own text and its launcher (cut from the file at these markers), plus the
# device helpers it uses.
TRAFFIC_KERNELS = {
    "score": ("score_mfma_kernel", "select.hip", ("void score_mfma_kernel(", "hipError_t launch_score(")),
    "attn": ("attn_mfma_kernel", "attend.hip", ("void attn_mfma_kernel(", "static hipError_t attn_t(")),
}


def kernel_source_hash(which: str = "score"):
    """Hash of the kernel's text (from its template line to the end of the
    function) and of its launcher's, plus the device helpers; None when the
    markers are not found (then no traffic record matches)."""
    _, fname, markers = TRAFFIC_KERNELS[which]
    csrc = os.path.join(ROOT, "sparse_kv_cache_step_amd", "csrc")
    text = open(os.path.join(csrc, fname)).read()
    h = hashlib.sha256()
    for m in markers:
        i = text.find(m)
        if i < 0:
            return None
        t = text.rfind("template <", 0, i)
        if t >= 0 and text.count("\n}\n", t, i) == 0:  # the template line of this function
            i = t
        h.update(text[i:text.index("\n}\n", i)].encode())
    with open(os.path.join(csrc, "skv_device.h"), "rb") as fh:
        h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, which: str = "score"):
    """HBM bytes per launch of a kernel from committed rocprofv3 counter
    runs, if they were taken on the kernel's current sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{which}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = kernel_source_hash(which)
    if h is None or rec.get("source_hash") != h:
        return None
    return rec.get("bytes_per_launch")


COPY_BYTES = 256 << 20  # the calibration copy


def ingest_counters(fetch_csv: str, write_csv: str, workload: str, command: str) -> int:
    """HBM bytes per launch of the scoring and fused attention kernels from
    two rocprofv3 counter CSVs, each counter scaled by what it reads for the
    calibration copy."""
    import csv

    def per_kernel(path, counter, kname):
        vals, names = {}, {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            vals[d] = vals.get(d, 0.0) + float(r["Counter_Value"])
            names[d] = r["Kernel_Name"]
        score = sorted(d for d in vals if "score_mfma_kernel" in names[d])
        mine = sorted(d for d in vals if kname in names[d])
        # the calibration copy is the last copy dispatched before the first
        # scoring launch (bench.py runs it right before the warmup)
        copies = [d for d in vals if "copyBuffer" in names[d] and score and d < score[0]]
        if not mine or not copies:
            return None
        return sum(vals[d] for d in mine) / len(mine), vals[max(copies)], len(mine)

    done = 0
    for which, (kname, _, _) in TRAFFIC_KERNELS.items():
        f = per_kernel(fetch_csv, "FETCH_SIZE", kname)
        w = per_kernel(write_csv, "WRITE_SIZE", kname)
        if f is None or w is None:
            print(f"no counter values for {kname} (or the calibration copy)", file=sys.stderr)
            continue
        (f_kib, f_copy_kib, nf), (w_kib, w_copy_kib, nw) = f, w
        f_scale = COPY_BYTES / (f_copy_kib * 1024.0)
        w_scale = COPY_BYTES / (w_copy_kib * 1024.0)
        fetch_b = f_kib * 1024.0 * f_scale
        write_b = w_kib * 1024.0 * w_scale
        rec = {"workload": workload, "kernel": kname, "source_hash": kernel_source_hash(which),
               "fetch_bytes_per_launch": int(fetch_b), "write_bytes_per_launch": int(write_b),
               "bytes_per_launch": int(fetch_b + write_b),
               "raw_KiB": {"FETCH_SIZE": f_kib, "WRITE_SIZE": w_kib, "copy_FETCH_SIZE": f_copy_kib,
                           "copy_WRITE_SIZE": w_copy_kib},
               "copy_scale": {"FETCH_SIZE": f_scale, "WRITE_SIZE": w_scale}, "dispatches": [nf, nw],
               "command": command}
        out = os.path.join(ROOT, "profiles", f"traffic_{which}_{workload}.json")
        with open(out, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec))
        done += 1
    return 0 if done else 1


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo), or the
    platform's processor string where that file is missing."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default="llama3-8b-128k-b8")
    ap.add_argument("--layers", type=int, default=None, help="default: the workload's layer count")
    ap.add_argument("--host-v-share", type=int, default=0,
                    help="layers share this many pinned host-V buffers (0: one per layer)")
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probes", action="store_true",
                    help="skip the device-ceiling probes (for profiler runs that count every dispatch)")
    ap.add_argument("--kernel-events", choices=["on", "off"], default="on")
    ap.add_argument("--overlap", choices=["on", "off"], default="off",
                    help="fetch beside the key rebuild (on) or before it (off)")
    ap.add_argument("--batch", type=int, default=None, help="sequences per layer override")
    ap.add_argument("--chunk", type=int, default=None,
                    help="chunk size override (top-k and outlier chunks scaled to keep their token budgets)")
    ap.add_argument("--top-k", type=int, default=None, help="selected chunks per KV head (budget) override")
    ap.add_argument("--rank", type=int, default=None, help="rank of the key factors override")
    ap.add_argument("--outlier-chunks", type=int, default=None, help="outlier chunks override")
    ap.add_argument("--append", action="store_true",
                    help="generation loop: each layer-step also appends the generated token to the local block "
                         "(no oracle baseline in this mode)")
    ap.add_argument("--snapkv", default=None, metavar="W,POOL",
                    help="SnapKV-style fixed selection: after the prefill each layer selects once from a window "
                         "of W queries with average pooling over POOL chunks; the timed steps keep that "
                         "selection (no oracle baseline in this mode)")
    ap.add_argument("--cache-chunks", type=int, default=0,
                    help="V chunks resident in HBM per (sequence, KV head): 0 = top-k, the set-difference cache; "
                         "larger keeps the most recently selected chunks too (least recently used)")
    ap.add_argument("--sweep", action="store_true",
                    help="run chunk-size / budget / rank variants of the workload, one JSON line each")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a device copy of 256 MiB (traffic-counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_score_<workload>.json from rocprofv3 counter CSVs and exit")
    ap.add_argument("--counter-command", default="",
                    help="with --ingest-counters: the command that produced the CSVs (recorded)")
    args = ap.parse_args()
    if args.ingest_counters:
        return ingest_counters(args.ingest_counters[0], args.ingest_counters[1], args.workload,
                               args.counter_command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sparse_kv_cache_step_amd import binding as skv
    from sparse_kv_cache_step_amd import synth

    if not os.path.exists(skv.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    base = synth.WORKLOADS[args.workload]
    snap = None
    if args.snapkv:
        w_obs, pool = (int(x) for x in args.snapkv.split(","))
        snap = (w_obs, pool)

    def variant(wl, chunk=None, top_k=None, rank=None, outliers=None):
        """The workload with another chunk size (top-k and outlier chunks
        scaled to keep their token budgets), budget or rank."""
        kw, tags = {}, []
        if chunk and chunk != wl.c:
            kw.update(c=chunk, k=max(1, wl.k * wl.c // chunk), o=wl.o * wl.c // chunk)
            tags.append(f"c={chunk}")
        if top_k:
            kw["k"] = top_k
            tags.append(f"k={top_k}")
        if rank:
            kw["r"] = rank
            tags.append(f"r={rank}")
        if outliers is not None:
            kw["o"] = outliers
            tags.append(f"o={outliers}")
        if not kw:
            return wl
        return wl.with_(name=f"{wl.name}[{','.join(tags)}]", **kw)

    def run_one(wl) -> dict:
        layers = args.layers or wl.layers
        wl = wl.with_(layers=layers)
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        dt = torch.bfloat16 if wl.bf16 else torch.float32
        nq = args.warmup + args.steps
        # the per-kernel pass decodes the K steps after the timed ones (fresh
        # queries, so a cache larger than the selection is not replayed warm)
        nq_all = nq + (args.steps if args.kernel_events == "on" else 0)
        log(f"bench: {wl.name} b={wl.b} s={wl.s} h_q={wl.h_q} h_kv={wl.h_kv} d={wl.d} r={wl.r} o={wl.o} k={wl.k} "
            f"w={wl.w} layers={layers} steps={args.steps} warmup={args.warmup}")

        # ---- setup (untimed): data, factors, prefill, pinned host V ----------------
        t0 = time.time()
        n_host = layers if args.host_v_share <= 0 else min(layers, args.host_v_share)
        host_bufs = []
        Ls, qs = [], []
        keep = {}  # inputs of the spot-checked layer, for the oracle
        new_kv = []  # decode-token append: (keys, values) per layer
        q_obs = []  # SnapKV-style selection: each layer's window queries
        spot_layer = layers - 1
        prefill_ms = {"factorize": 0.0, "prefill_meta": 0.0}
        for l in range(layers):
            k_pre = synth.k_pre_torch(wl, l, dev)
            v = synth.v_torch(wl, l, dev)
            torch.cuda.synchronize()
            ts = time.perf_counter()
            A, B = skv.factorize(k_pre, wl.r)
            torch.cuda.synchronize()
            prefill_ms["factorize"] += (time.perf_counter() - ts) * 1e3
            lay = skv.Layer(batch=wl.b, heads_q=wl.h_q, heads_kv=wl.h_kv, head_dim=wl.d, seq_len=wl.s, chunk=wl.c,
                            rank=wl.r, n_outlier=wl.o, top_k=wl.k, local_window=wl.w, rope_base=wl.rope_base,
                            bf16=wl.bf16, max_new=nq_all if args.append else 0,
                            cache_chunks=args.cache_chunks)
            if l < n_host:
                host_bufs.append(lay.host_buffer())
            torch.cuda.synchronize()
            ts = time.perf_counter()
            lay.prefill_meta(k_pre, v, A, B, host_bufs[l % n_host])
            torch.cuda.synchronize()
            prefill_ms["prefill_meta"] += (time.perf_counter() - ts) * 1e3
            if snap:
                # the observation window's queries come before the decoded ones
                q_all = synth.queries_torch(wl, l, dev, steps=snap[0] + nq_all)
                q_obs.append(q_all[:snap[0]].permute(1, 2, 0, 3).contiguous())
                qs.append(q_all[snap[0]:].contiguous())
                del q_all
            else:
                qs.append(synth.queries_torch(wl, l, dev, steps=nq_all))
            if args.append:
                # the generated tokens' pre-RoPE keys and values, one per step
                g = torch.Generator(device=dev)
                g.manual_seed(1000003 * (l + 1) + wl.wid)
                new_kv.append((torch.randn((nq_all, wl.b, wl.h_kv, wl.d), generator=g, device=dev).to(dt),
                               torch.randn((nq_all, wl.b, wl.h_kv, wl.d), generator=g, device=dev).to(dt)))
            torch.cuda.synchronize()
            if l == spot_layer and not args.no_cpu_baseline and not args.append and not snap:
                sample = [0, wl.b // 2] if wl.b > 1 else [0]
                keep = {"seqs": sample, "k_pre": k_pre[sample].float().cpu(), "v": v[sample].float().cpu()}
            del k_pre, v, A, B
            lay.set_overlap(args.overlap == "on")
            Ls.append(lay)
            if l % 4 == 3 or l == layers - 1:
                log(f"  setup: {l + 1}/{layers} layers ready ({time.time() - t0:.0f}s)")
        torch.cuda.empty_cache()
        outs = [torch.empty((wl.b, wl.h_q, wl.d), dtype=dt, device=dev) for _ in range(layers)]
        stream = torch.cuda.current_stream()

        def run_steps(t_begin, t_count):
            for t in range(t_begin, t_begin + t_count):
                for l in range(layers):
                    Ls[l].decode_step(qs[l][t], outs[l], stream)
                    if args.append:  # the generated token joins the local block
                        Ls[l].append(new_kv[l][0][t], new_kv[l][1][t], stream)

        if args.copy_calibration:
            src = torch.ones(COPY_BYTES, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst

        snap_us = None
        if snap:
            # one selection per layer (timed on its own), then decode with it
            torch.cuda.synchronize()
            s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for l in range(layers):
                Ls[l].snapkv_select(q_obs[l], snap[1], stream)
            s1.record(stream)
            torch.cuda.synchronize()
            snap_us = s0.elapsed_time(s1) * 1e3 / layers
            log(f"snapkv selection: {snap_us:.1f} us per layer (w_obs={snap[0]}, pool={snap[1]})")
            del q_obs[:]

        # ---- warmup ---------------------------------------------------------------
        run_steps(0, args.warmup)
        torch.cuda.synchronize()
        for lay in Ls:
            lay.reset_stats()

        # ---- timed region ---------------------------------------------------------
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        e0.record(stream)
        run_steps(args.warmup, args.steps)
        e1.record(stream)
        torch.cuda.synchronize()
        last_out = outs[spot_layer].clone()  # output and selection of the last timed step
        last_sel = Ls[spot_layer].read(skv.SKV_T_SELECTION)
        wall = time.perf_counter() - wall0
        elapsed = e0.elapsed_time(e1) / 1e3
        log(f"timed: {args.steps} steps x {layers} layers in {elapsed * 1e3:.2f} ms (host wall {wall * 1e3:.2f} ms)")
        stats = [lay.stats() for lay in Ls]
        hits = sum(s["hits"] for s in stats)
        misses = sum(s["misses"] for s in stats)
        alpha = hits / max(1, hits + misses)
        h2d_bytes = sum(s["bytes_h2d"] for s in stats)

        # ---- per-kernel durations: the next K steps with HIP events --------------
        kern_ms = {name: 0.0 for name in skv.KERNELS}
        kern_steps = 0
        if args.kernel_events == "on":
            for lay in Ls:
                lay.set_timing(True)
            run_steps(nq, args.steps)
            torch.cuda.synchronize()
            for lay in Ls:
                ms, st = lay.get_timing()
                lay.set_timing(False)
                kern_steps += st
                for kname, v_ms in ms.items():
                    kern_ms[kname] += v_ms
        per_launch_us = {k: (v * 1e3 / kern_steps if kern_steps else None) for k, v in kern_ms.items()}

        # ---- a cold step: every layer's cache emptied, one more step timed ------
        cold_us = None
        if not snap and not args.append:
            for lay in Ls:
                lay.reset_cache(stream)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record(stream)
            run_steps(nq - 1, 1)
            c1.record(stream)
            torch.cuda.synchronize()
            cold_us = c0.elapsed_time(c1) * 1e3 / layers

        # ---- the device's own ceilings, measured in this run --------------------
        peaks = {}
        try:
            if args.no_probes:
                raise RuntimeError("--no-probes")
            nb = 1 << 30
            src = torch.empty(nb, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            hsrc = torch.empty(nb // 4, dtype=torch.uint8, pin_memory=True)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            dst.copy_(src)
            ev[0].record(stream)
            dst.copy_(src)
            ev[1].record(stream)
            dst[: nb // 4].copy_(hsrc, non_blocking=True)
            ev[2].record(stream)
            dst[: nb // 4].copy_(hsrc, non_blocking=True)
            ev[3].record(stream)
            torch.cuda.synchronize()
            peaks = {"hbm_copy_TBps": round(2 * nb / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e12, 3),
                     "pcie_h2d_pinned_GBps": round((nb // 4) / (ev[2].elapsed_time(ev[3]) * 1e-3) / 1e9, 2)}
            # a plain streaming read of the 1 GiB buffer (4x the last-level
            # cache): the ceiling a read-only kernel reaches on this device
            src.fill_(1)
            peaks["hbm_read_TBps"] = round(skv.shadowkv_probe_hbm_read(src.data_ptr(), nb, 5, stream.cuda_stream)
                                           / 1e3, 3)
            # the host-issued alternative to the device-initiated fetch: about a
            # step's misses (half the selection) as 2 KB chunks scattered over
            # the pinned buffer, one hipMemcpyAsync each, then one batch
            chunk_b = wl.c * wl.d * (2 if wl.bf16 else 4)
            n_cp = max(1, wl.k * wl.b * wl.h_kv // 2)
            rng = np.random.default_rng(0)
            picks = rng.choice(hsrc.numel() // chunk_b, size=min(n_cp, hsrc.numel() // chunk_b), replace=False)
            each, batch = skv.shadowkv_probe_host_copies(hsrc.data_ptr(), hsrc.numel(), dst.data_ptr(), chunk_b,
                                                         [int(x) for x in picks], 2, stream.cuda_stream)
            peaks["host_copies_per_chunk_GBps"] = round(each, 2)
            peaks["host_copies_batch_GBps"] = round(batch, 2)
            peaks["host_copies_chunks"] = int(len(picks))
            del src, dst, hsrc
        except RuntimeError as e:  # not enough memory for the probes: leave them out
            log(f"device peaks skipped: {e}")

        layer_steps = args.steps * layers
        ab = algorithmic_bytes(wl)
        if snap:
            del ab["landmarks"]  # a fixed selection reads no landmarks
        alg_total = sum(ab.values())
        t_ls = elapsed / layer_steps
        dense_kv = 2 * wl.b * wl.h_kv * wl.s * wl.d * (2 if wl.bf16 else 4)

        roofline = None
        kernels = {}
        if kern_steps:
            score_bytes = ab.get("landmarks", 0) + ab["q"]
            qk_bytes = ab["a_rows"] + ab["b_factor"] + ab["outlier_kv"] // 2 + ab["local_kv"] // 2 + ab["q"]
            pv_bytes = ab["selected_v"] + ab["outlier_kv"] // 2 + ab["local_kv"] // 2 + ab["out"]
            fetch_bytes = h2d_bytes / max(1, layer_steps)
            for name, nbytes, peak in (("score", score_bytes, PEAK_HBM), ("qk", qk_bytes, PEAK_HBM),
                                       ("pv", pv_bytes, PEAK_HBM), ("attn", qk_bytes + pv_bytes, PEAK_HBM),
                                       ("fetch", fetch_bytes, PEAK_PCIE)):
                us = per_launch_us[name]
                if not us:
                    continue  # not run in this mode (a fixed selection scores and fetches nothing)
                gbs = nbytes / (us * 1e-6) / 1e9 if us else None
                kernels[name] = {"us_per_launch": round(us, 3), "bytes_per_launch": int(nbytes),
                                 "GBps": round(gbs, 1) if gbs else None, "peak_GBps": peak / 1e9,
                                 "frac": round(gbs * 1e9 / peak, 4) if gbs else None}
            if per_launch_us["select"]:
                kernels["select"] = {"us_per_launch": round(per_launch_us["select"], 3)}
            # scoring and attention together: the two HBM streams of the step
            att = "attn" if "attn" in kernels else None
            if "score" in kernels and (att or ("qk" in kernels and "pv" in kernels)):
                parts = [kernels["score"]] + ([kernels[att]] if att else [kernels["qk"], kernels["pv"]])
                nb_sa = sum(k_["bytes_per_launch"] for k_ in parts)
                us_sa = sum(k_["us_per_launch"] for k_ in parts)
                gbs_sa = nb_sa / (us_sa * 1e-6) / 1e9
                kernels["score_plus_attn"] = {"us_per_launch": round(us_sa, 3), "bytes_per_launch": int(nb_sa),
                                              "GBps": round(gbs_sa, 1), "peak_GBps": PEAK_HBM / 1e9,
                                              "frac": round(gbs_sa * 1e9 / PEAK_HBM, 4)}
            if snap:
                # a fixed selection runs no scoring: attention dominates
                fused = "attn" in kernels
                sc = kernels["attn" if fused else "qk"]
                roofline = {"kernel": "attn_mfma_kernel + combine_kernel (rebuild, logits, PV, merge)" if fused
                            else "qk_mfma_kernel (key rebuild + static keys, logits)",
                            "bound": "hbm", "achieved": sc["GBps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                            "frac": sc["frac"], "traffic": measured_traffic(wl.name, "attn") if fused else None,
                            "bytes_per_launch": sc["bytes_per_launch"],
                            "us_per_launch": sc["us_per_launch"]}
            else:
                sc = kernels["score"]
                traffic = measured_traffic(wl.name)
                roofline = {"kernel": "score_mfma_kernel (landmark scoring)", "bound": "hbm",
                            "achieved": sc["GBps"], "peak": PEAK_HBM / 1e9, "unit": "GB/s", "frac": sc["frac"],
                            "traffic": traffic, "bytes_per_launch": sc["bytes_per_launch"],
                            "us_per_launch": sc["us_per_launch"]}

        # the same fractions against the read ceiling measured in this run
        read_ceiling = peaks.get("hbm_read_TBps")
        if read_ceiling:
            for kk in kernels.values():
                if kk.get("GBps") and kk.get("peak_GBps") == PEAK_HBM / 1e9:
                    kk["frac_of_read_ceiling"] = round(kk["GBps"] / (read_ceiling * 1e3), 4)
            if roofline:
                roofline["frac_of_read_ceiling"] = round(roofline["achieved"] / (read_ceiling * 1e3), 4)
                roofline["read_ceiling_GBps"] = round(read_ceiling * 1e3, 1)

        fetch_gbs = kernels.get("fetch", {}).get("GBps") if kernels else None
        closed_form = None
        if fetch_gbs:
            closed_form = skv.shadowkv_equiv_bandwidth(wl.s, wl.c, wl.k, wl.o, alpha, PEAK_HBM, fetch_gbs * 1e9) / 1e12

        # ---- oracle on the host, bounded sample of the same workload --------------
        cpu_baseline = None
        parity = None
        if not args.no_cpu_baseline and keep:
            import oracle
            from oracle import Shape
            seqs = keep["seqs"]
            shape = Shape(b=len(seqs), h_q=wl.h_q, h_kv=wl.h_kv, d=wl.d, s=wl.s, c=wl.c, r=wl.r, o=wl.o, k=wl.k,
                          w=wl.w, rope_base=wl.rope_base, bf16=wl.bf16)
            kp = keep["k_pre"].double().numpy()
            vv = keep["v"].double().numpy()
            log(f"cpu baseline: oracle prefill + SVD for sequences {seqs} of layer {spot_layer} (untimed)")
            meta = oracle.prefill(shape, kp, vv)
            A_o, B_o = oracle.svd_factors(shape, kp)
            q_all = qs[spot_layer][:, seqs].float().cpu().double().numpy()
            # decode steps 0, 1, ..., nq - 1 (the GPU's output at the last timed
            # step is spot-checked there), then again from step 0 until the time
            # budget is spent; the oracle's decode does not depend on the cache
            t_last = args.warmup + args.steps - 1
            t_start = time.perf_counter()
            n_done, res, res_last = 0, None, None
            while True:
                t = n_done % nq
                res = oracle.decode(shape, q_all[t], meta, A_o, B_o, vv)
                if t == t_last:
                    res_last = res
                n_done += 1
                if n_done >= nq and time.perf_counter() - t_start > args.cpu_baseline_seconds:
                    break
            cpu_s = time.perf_counter() - t_start
            per_seq_step = cpu_s / (n_done * len(seqs))
            threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
            cores = min(threads, os.cpu_count() or 1, len(seqs) * wl.h_kv)
            cpu_baseline = {"value": round(1.0 / (per_seq_step * wl.b), 4), "unit": "layer-steps/s", "cores": cores,
                            "kind": "oracle", "cpu_model": cpu_model(), "nproc": os.cpu_count(),
                            "omp_threads": threads,
                            "sample": f"{n_done} decode steps (steps 0..{nq - 1}, cycled) of sequences {seqs} "
                                      f"(of {wl.b}) of layer {spot_layer}; {cpu_s:.1f} s of CPU time; "
                                      f"scaled to all {wl.b} sequences"}
            if res_last is not None:
                gpu_out = last_out[seqs].float().cpu().double().numpy()
                gpu_sel = last_sel[seqs].cpu().numpy()
                parity = {"layer": spot_layer, "step": t_last, "sequences": seqs,
                          "selection_equal": bool(np.array_equal(gpu_sel, res_last["sel"])),
                          "max_abs_err_vs_oracle": float(np.max(np.abs(gpu_out - res_last["out"]))),
                          "tolerance": 2e-2 if wl.bf16 else 1e-4}
            log(f"cpu baseline: {cpu_baseline['value']} layer-steps/s on {cores} threads")

        value = layer_steps / elapsed
        line = {
            "metric": "sparse decode layer-steps/sec + effective & equivalent HBM TB/s at 128K, 1 GPU",
            "value": round(value, 2), "unit": "layer-steps/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(elapsed / args.steps * 1e3, 4), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.bf16 else "f32", "data": "synthetic",
            "config": {"workload": wl.name, "batch": wl.b, "seq_len": wl.s, "heads_q": wl.h_q, "heads_kv": wl.h_kv,
                       "head_dim": wl.d, "chunk": wl.c, "rank": wl.r, "outlier_chunks": wl.o, "top_k": wl.k,
                       "local_window": wl.w, "layers": layers, "host_v_buffers": n_host,
                       "cache_chunks": args.cache_chunks or wl.k,
                       **({"append": True} if args.append else {}),
                       **({"snapkv": {"w_obs": snap[0], "pool": snap[1]}} if snap else {})},
            "us_per_layer_step": round(t_ls * 1e6, 3),
            "effective_TBps": round(alg_total / t_ls / 1e12, 4),
            "equivalent_TBps": round(dense_kv / t_ls / 1e12, 4),
            "alpha": None if snap else round(alpha, 4),
            "h2d_GB": round(h2d_bytes / 1e9, 4),
            "closed_form_equiv_TBps": round(closed_form, 3) if closed_form else None,
            "roofline": roofline,
            "kernels": kernels,
            "cpu_baseline": cpu_baseline,
            "parity_spot_check": parity,
            "setup_s": round(time.time() - t0, 1),
            "prefill_ms_per_layer": {k: round(v / layers, 2) for k, v in prefill_ms.items()},
            "tokens_per_s_attention_only": round(value * wl.b / layers, 1),
            "cold_step_us_per_layer": round(cold_us, 2) if cold_us else None,
            "device_peaks": peaks,
        }
        if snap:
            line["snapkv_select_us_per_layer"] = round(snap_us, 2)
        for lay in Ls:
            lay.close()
        for hb in host_bufs:
            hb.free()
        torch.cuda.empty_cache()
        return line

    if args.sweep:
        # chunk size, budget and rank around the workload, every kernel reused;
        # one JSON line per configuration
        n8 = base.s // 8
        grid = [dict(), dict(chunk=4), dict(chunk=16), dict(top_k=n8 // 128), dict(top_k=n8 // 32),
                dict(rank=96), dict(rank=128), dict(rank=192)]
        for g in grid:
            print(json.dumps(run_one(variant(base, **g))), flush=True)
        return 0
    if args.batch:
        base = base.with_(name=f"{base.name}[b={args.batch}]", b=args.batch)
    line = run_one(variant(base, args.chunk, args.top_k, args.rank, args.outlier_chunks))
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
