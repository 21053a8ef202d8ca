#!/usr/bin/env python3
"""Benchmark of the TurboQuant packed-KV hot path on one MI355X.

One step = one pass of the whole path over one workload, by default the
batched decode workload, the largest of the five that the metric names no
single one of (64 sequences with lengths uniform in [1024, 32768], 32 query
heads / 8 KV heads, d = 128, bf16 K/V, K 4-bit records, V 2-bit tiles, the
first 128 tokens of every sequence raw bf16, V skipped below weight 1e-6);
--workload selects another of the five:
  quantize all K vectors, quantize all V vectors, one decode-attention step.
Inputs are resident in HBM before timing.  Four copies of the inputs and of
the packed cache rotate between steps, and a step attends over a cache copy
written three steps earlier, so reads are not served from the 256 MB
Infinity Cache.  Timing uses HIP events on the launch stream.  Per-kernel
durations (the roofline figures and `value`) come from a second timed pass
in which each phase is launched back to back, decode over ten cache copies.

Prints one JSON line.  `value` is the decode-attention throughput in GB/s of
algorithmic bytes (packed K and V records, norms, q and out).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "packed-KV decode-attention GB/s (% HBM peak) + quantize Mvec/s at d=128"
WORKLOAD = "batched_ragged"
COPIES = 4
ATT_COPIES = 10
KERNEL_SOURCES = ["compressed_kv_cache_tq_amd/csrc/quantize.hip",
                  "compressed_kv_cache_tq_amd/csrc/attend_split.h+compressed_kv_cache_tq_amd/csrc/attend.hip"]


def source_hash(paths: str) -> str:
    """sha256 (first 16 hex digits) of the '+'-joined source files, concatenated."""
    h = hashlib.sha256()
    for path in paths.split("+"):
        with open(os.path.join(ROOT, path), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(workload: str, name: str):
    """Per-call HBM bytes measured with rocprofv3 --pmc for a step phase of a
    workload, or None if the summary is missing or the kernel source changed
    since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    src = kv.get("source")
    if not src or kv.get("source_sha256_16") != source_hash(src):
        return None
    return float(kv["hbm_bytes_per_call"])


CALIB_BYTES = 512 << 20
STEP_SOURCES = {"quantize_k": KERNEL_SOURCES[0], "quantize_v": KERNEL_SOURCES[0], "attend": KERNEL_SOURCES[1]}


def step_kernels(wname: str) -> dict:
    """Kernels of one bench step of a workload (default options), by the name
    rocprofv3 reports ('*' stands for a template argument the launch picks:
    the quantize's tiles per chunk, by size; the decode's softmax form, by
    group size and splits): the traffic of a phase is the sum over its
    kernels."""
    from compressed_kv_cache_tq_amd import workloads
    wl = workloads.WORKLOADS[wname]
    f32 = "true" if wl.dtype == "f32" else "false"
    k, v = wl.k, wl.v
    # (kernel, dispatches per call)
    if k.qjl_m:  # the sketch kernel launches once per 32 sequences
        qk = [(f"quantize_kernel<{k.bits_lo}, {k.bits_hi}, {2 if wl.dtype == 'f32' else 1}, false, true>",
               -(-wl.batch // 32))]
    else:
        qk = [(f"rotq_kernel<{k.bits_lo}, {k.bits_hi}, {f32}, false, *, false, false>", 1)]
    qv = [(f"rotq_kernel<{v.bits_lo}, {v.bits_hi}, {f32}, true, *, false, false>", 1)]
    if wl.lens_range:  # ragged lengths: the last, partly written value tile of each sequence
        qv.append((f"rotq_kernel<{v.bits_lo}, {v.bits_hi}, {f32}, true, 2, true, false>", 1))
    at = [(f"split_kernel<{k.bits_lo}, {k.bits_hi}, {v.bits_lo}, {v.bits_hi}, {'true' if k.qjl_m else 'false'}, "
           f"false, false, *>", 1)]
    if not wl.lens_range:
        at.append(("combine_kernel", 1))
    return {"quantize_k": qk, "quantize_v": qv, "attend": at}


def _pmc_per_dispatch(run_dir: str, counter: str):
    """{dispatch_id: (kernel_name, counter value summed over instances)} of a rocprofv3 run."""
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(run_dir, "**", "*.db"), recursive=True)
    if len(dbs) != 1:
        raise SystemExit(f"expected one rocprofv3 database under {run_dir}, found {len(dbs)}")
    con = sqlite3.connect(dbs[0])
    per = {}
    for did, name, cname, v in con.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        if cname != counter:
            continue
        n, tot = per.get(did, (name, 0.0))
        per[did] = (n, tot + float(v))
    if not per:
        raise SystemExit(f"no {counter} values in {dbs[0]}")
    return per


def traffic_summary(fetch_dir: str, write_dir: str, wname: str, command: str = "") -> int:
    """HBM bytes per call of each bench phase: FETCH_SIZE and WRITE_SIZE (KiB
    per dispatch, summed over the phase's kernels) scaled by the factor that
    maps the same counter of the calibration copy onto its known CALIB_BYTES
    read and written."""
    STEP_KERNELS = step_kernels(wname)
    out = {}
    for counter, run_dir in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = _pmc_per_dispatch(run_dir, counter)
        calib = [v for _, (n, v) in sorted(per.items()) if "neg_kernel" in n][-5:]
        if len(calib) < 5:
            raise SystemExit(f"{run_dir}: the calibration kernel (--copy-calibration) is missing")
        factor = CALIB_BYTES / (1024.0 * float(np.median(calib)))
        for key, names in STEP_KERNELS.items():
            tot, raw = 0.0, 0.0
            for kname, mult in names:
                pat = re.compile(re.escape(kname).replace(r"\*", r"\w+"))
                vals = [v for n, v in per.values() if pat.search(n.replace("(anonymous namespace)::", ""))]
                if not vals:
                    raise SystemExit(f"{run_dir}: no dispatch of {kname}")
                tot += mult * float(np.mean(vals)) * 1024.0 * factor
                raw += mult * float(np.mean(vals))
            out.setdefault(key, {})[counter] = (tot, factor, raw, float(np.median(calib)))
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    for key, d in out.items():
        fetch, ff, fraw, fcal = d["FETCH_SIZE"]
        write, fw, wraw, wcal = d["WRITE_SIZE"]
        src = STEP_SOURCES[key]
        path = os.path.join(ROOT, "profiles", f"traffic_{wname}_{key}.txt")
        with open(path, "w") as f:
            kl = ", ".join(f"{n}{f' x {m}' if m > 1 else ''}" for n, m in STEP_KERNELS[key])
            f.write(f"# HBM traffic per call of {kl} ({wname} bench step),\n")
            f.write("# from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE, each scaled by the factor that maps\n")
            f.write(f"# the counter of a {CALIB_BYTES >> 20} MiB fp32 streaming kernel onto its known bytes.\n")
            if command:
                f.write(f"# command: {command}\n")
            f.write(f"source = {src}\n")
            f.write(f"source_sha256_16 = {source_hash(src)}\n")
            f.write(f"fetch_size_kib_raw = {fraw:.1f}\n")
            f.write(f"write_size_kib_raw = {wraw:.1f}\n")
            f.write(f"calibration_fetch_kib_raw = {fcal:.1f}\n")
            f.write(f"calibration_write_kib_raw = {wcal:.1f}\n")
            f.write(f"fetch_factor = {ff:.4f}\n")
            f.write(f"write_factor = {fw:.4f}\n")
            f.write(f"fetch_bytes_per_call = {fetch:.0f}\n")
            f.write(f"write_bytes_per_call = {write:.0f}\n")
            f.write(f"hbm_bytes_per_call = {fetch + write:.0f}\n")
        print(open(path).read())
    return 0


def stats_summary(csv_path: str, out_path: str, title: str = "", command: str = "") -> int:
    """Kernel statistics of a rocprofv3 --kernel-trace --stats run (its
    kernel_stats.csv, durations in ns) as a short text table in microseconds."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    with open(out_path, "w") as f:
        if title:
            f.write(f"# {title}\n")
        if command:
            f.write(f"# command: {command}\n")
        f.write("# source: rocprofv3 kernel_stats.csv; durations in microseconds\n")
        f.write(f"{'kernel':<80} {'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'stddev':>8}\n")
        for r in rows:
            name = r["Name"].replace("(anonymous namespace)::", "")
            name = name[:80]
            f.write(f"{name:<80} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>9.2f} "
                    f"{float(r['MinNs']) / 1e3:>9.2f} {float(r['MaxNs']) / 1e3:>9.2f} "
                    f"{float(r['StdDev']) / 1e3:>8.2f}\n")
    print(open(out_path).read())
    return 0


def counter_summary(run_dirs, out_path: str, title: str = "", command: str = "") -> int:
    """Per-kernel averages (per dispatch) of the counters of rocprofv3 --pmc
    runs of this script (csv or database output).  The per-wave cycle
    counters (SQ_WAIT_*, SQ_ACTIVE_INST_*) are also given as a fraction of
    SQ_WAVE_CYCLES, the cycles that waves were resident."""
    import csv
    import glob
    import sqlite3
    per = {}  # (kernel, counter) -> {dispatch: value}
    for run_dir in run_dirs:
        csvs = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
        rows = []
        if csvs:
            for path in csvs:
                for r in csv.DictReader(open(path)):
                    rows.append((r["Dispatch_Id"], r["Kernel_Name"], r["Counter_Name"], r["Counter_Value"]))
        else:
            for db in glob.glob(os.path.join(run_dir, "**", "*.db"), recursive=True):
                con = sqlite3.connect(db)
                rows += list(con.execute(
                    "select dispatch_id, kernel_name, counter_name, value from counters_collection"))
        if not rows:
            raise SystemExit(f"no counter values under {run_dir}")
        for did, name, cname, v in rows:
            name = re.sub(r"\(anonymous namespace\)::", "", name)
            d = per.setdefault((name, cname), {})
            d[(run_dir, did)] = d.get((run_dir, did), 0.0) + float(v)
    kernels = sorted({k for k, _ in per})
    with open(out_path, "w") as f:
        if title:
            f.write(f"# {title}\n")
        if command:
            f.write(f"# command: {command}\n")
        f.write("# per-dispatch averages of rocprofv3 --pmc counters (summed over the counter's instances);\n")
        f.write("# '(x of wave cycles)' = counter / SQ_WAVE_CYCLES of the same kernel\n")
        for k in kernels:
            cnames = sorted(c for kk, c in per if kk == k)
            vals = {c: float(np.mean(list(per[(k, c)].values()))) for c in cnames}
            ndisp = max(len(per[(k, c)]) for c in cnames)
            f.write(f"\nkernel {k[:160]}\n")
            f.write(f"  dispatches averaged: {ndisp}\n")
            wc = vals.get("SQ_WAVE_CYCLES")
            for c in cnames:
                extra = ""
                if wc and c.startswith(("SQ_WAIT", "SQ_ACTIVE_INST")):
                    extra = f"  ({vals[c] / wc:.3f} of wave cycles)"
                f.write(f"  {c:<28} {vals[c]:>18.1f}{extra}\n")
    print(open(out_path).read())
    return 0


def _oracle_spec(spec):
    from oracle import quantize as oqz
    return oqz.Spec(bits_lo=spec.bits_lo, bits_hi=spec.bits_lo if spec.bits_hi is None else spec.bits_hi,
                    split=spec.split, qjl_m=spec.qjl_m, rot_seed=spec.rot_seed, qjl_seed=spec.qjl_seed,
                    rotation="haar" if spec.rotation == 0 else "hadamard", norm_f16=bool(spec.norm_f16))


def cpu_baseline(inp, wl, kspec, vspec, kc, vc, comp_h, sample, tok_bytes, n_quant=65536):
    """The float64 oracle on the host, on a bounded sample of the step: one
    decode step of the sampled sequences (all their KV and query heads) read
    from the GPU's packed cache (unpacking included, median of 3 runs), and
    quantize + pack of the first n_quant key vectors of the first sampled
    sequence.  Also the oracle's exact V-skip count on that decode sample."""
    from compressed_kv_cache_tq_amd import tq
    from oracle import attend as oat
    from oracle import pack as opk
    from oracle import quantize as oqz
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    ks, vs = _oracle_spec(kspec), _oracle_spec(vspec)
    Hkv, S = wl.hkv, wl.sink
    kcb = tq.code_bytes(kspec)
    nbk, nbv = tq.cache_code_bytes(kspec, kc.cap), tq.cache_code_bytes(vspec, vc.cap)
    m8 = kspec.qjl_m // 8
    raw = []  # per sampled sequence, per kv head: the packed arrays as stored on the GPU
    for b in sample:
        n = int(comp_h[b])
        rows = []
        for h in range(Hkv):
            st = b * Hkv + h
            r = {"k": kc.codes[st * nbk: st * nbk + n * kcb].cpu().numpy().reshape(n, kcb),
                 "v": vc.codes[st * nbv:(st + 1) * nbv].cpu().numpy(),
                 "kn": kc.norms[st * kc.cap: st * kc.cap + n].cpu().numpy(),
                 "vn": vc.norms[st * vc.cap: st * vc.cap + n].cpu().numpy()}
            if m8:
                r["z"] = kc.qjl_signs[st * kc.cap * m8:(st * kc.cap + n) * m8].cpu().numpy().reshape(n, m8)
                r["g"] = kc.qjl_rnorms[st * kc.cap: st * kc.cap + n].cpu().numpy()
            rows.append(r)
        raw.append(rows)
    lens = np.asarray(inp.seq_lens)[sample]
    q = inp.q[sample]
    sk = sv = None
    if S:
        sk = [[inp.k[b][h, :S] for h in range(Hkv)] for b in sample]
        sv = [[inp.v[b][h, :S] for h in range(Hkv)] for b in sample]

    def unpack():
        K, Kn, V, Vn, Z, R = ([] for _ in range(6))
        for i, b in enumerate(sample):
            n = int(comp_h[b])
            K.append([opk.unpack_records(r["k"], kspec.widths) for r in raw[i]])
            V.append([opk.unpack_tiled(r["v"], vspec.widths, n) for r in raw[i]])
            Kn.append([r["kn"] for r in raw[i]])
            Vn.append([r["vn"] for r in raw[i]])
            if m8:
                Z.append([opk.unpack_sign_bits(r["z"]) for r in raw[i]])
                R.append([r["g"] for r in raw[i]])
        return K, Kn, V, Vn, (Z if m8 else None), (R if m8 else None)

    def decode_once():
        t0 = time.perf_counter()
        K, Kn, V, Vn, Z, R = unpack()
        oat.attend(q, ks, vs, lens, K, Kn, V, Vn, k_bits=Z, k_gamma=R, sink_k=sk, sink_v=sv, sink=S,
                   v_skip=wl.v_skip)
        return time.perf_counter() - t0

    t_dec = float(np.median([decode_once() for _ in range(3)]))
    n_tok = int(np.sum(comp_h[sample]))
    dec_bytes = Hkv * n_tok * tok_bytes + Hkv * int(np.minimum(lens, S).sum()) * 2 * 128 * 2 + \
        2 * len(sample) * wl.hq * 128 * 4
    res = {"value": round(dec_bytes / t_dec / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
           "decode_seconds": round(t_dec, 3)}
    # the oracle's exact V-skip rule (final weight below the threshold) on the decode sample
    skipped = total = 0
    if wl.v_skip > 0:
        K, Kn, V, Vn, Z, R = unpack()
        G = wl.hq // Hkv
        for i in range(len(sample)):
            for h in range(Hkv):
                _, det = oat.attend_group(q[i, h * G:(h + 1) * G], ks, K[i][h], Kn[i][h], vs, V[i][h], Vn[i][h],
                                          k_bits=None if Z is None else Z[i][h],
                                          k_gamma=None if R is None else R[i][h],
                                          sink_k=None if sk is None else sk[i][h],
                                          sink_v=None if sv is None else sv[i][h], v_skip=wl.v_skip,
                                          return_details=True)
                for _, keep, _ in det:
                    skipped += int(np.sum(~keep))
                    total += keep.size
        res["v_skip_rate_oracle"] = round(skipped / max(total, 1), 6)
    b0 = sample[0]
    nq = min(n_quant, int(comp_h[b0]) * Hkv)
    xs = inp.k[b0][:, S:S + int(comp_h[b0])].reshape(-1, 128)[:nq].astype(np.float64)
    t1 = time.perf_counter()
    qq = oqz.quantize(xs, ks)
    opk.pack_records(qq.idx, kspec.widths)
    t_q = time.perf_counter() - t1
    res["quantize_Mvec_s"] = round(nq / t_q / 1e6, 5)
    res["sample"] = (f"decode: one step of sequences {list(map(int, sample))} ({n_tok} compressed tokens x {Hkv} "
                     f"KV heads, {wl.hq} query heads each) read from the GPU's packed cache, unpacking "
                     f"included, median of 3; quantize + pack: {nq} key vectors of sequence {int(b0)}")
    return res


def kspec_bytes(spec) -> int:
    from compressed_kv_cache_tq_amd import tq
    return tq.code_bytes(spec)


def bench_search(args) -> int:
    """Inner-product search: scores of the search workload's queries against
    its packed database, back to back (prep + scores launches per call)."""
    import torch
    from compressed_kv_cache_tq_amd import tq, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wl = workloads.SEARCH
    rot = tq.ROT_HAAR if args.rotation == "haar" else tq.ROT_HADAMARD
    spec = tq.Spec(wl.bits, qjl_m=wl.qjl_m, layout=tq.LAYOUT_RECORD, rotation=rot)
    tab = tq.device_tables(spec)
    xd = torch.from_numpy(workloads.bf16_bits(workloads.search_database(wl)).view(np.int16)).cuda().view(torch.bfloat16)
    cache = tq.alloc_cache(spec, wl.streams, wl.n_tok)
    tq.quantize_kv(spec, tab, xd, cache)
    del xd
    # five database copies (5 x 58.7 MB) so back-to-back calls read HBM, not
    # the 256 MB Infinity Cache
    caches = [cache] + [tq.clone_cache(cache) for _ in range(4)]
    q = torch.from_numpy(workloads.search_queries(wl)).cuda()
    N = wl.streams * wl.n_tok
    scores = torch.empty((wl.nq, N), dtype=torch.float32, device="cuda")
    ws = tq.alloc_ip_workspace()
    stream = torch.cuda.current_stream()

    def call(i):
        tq.ip_scores(spec, tab, caches[i % len(caches)], q, n_streams=wl.streams, n_tok=wl.n_tok, scores=scores,
                     workspace=ws)

    for i in range(max(args.warmup, len(caches))):
        call(i)
    torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for i in range(args.steps):
        call(i)
    eb.record(stream)
    torch.cuda.synchronize()
    ms = ea.elapsed_time(eb) / args.steps
    per_vec = tq.code_bytes(spec) + 4 + (wl.qjl_m // 8 + 4 if wl.qjl_m else 0)
    db_bytes = N * per_vec + wl.nq * 128 * 4
    out_bytes = wl.nq * N * 4
    gbs = (db_bytes + out_bytes) / (ms * 1e-3) / 1e9
    res = {
        "metric": "packed inner-product search GB/s (% HBM peak)", "value": round(gbs, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": wl.name, "database": N, "streams": wl.streams, "queries": wl.nq, "d": 128,
                   "bits": wl.bits, "qjl": bool(wl.qjl_m), "rotation": args.rotation},
        "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "call_us": round(ms * 1e3, 2),
        "gscores_s": round(wl.nq * N / (ms * 1e-3) / 1e9, 2),
        "bytes": {"database_and_queries": db_bytes, "scores": out_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": f"ip_kernel<{wl.bits},{wl.bits}{',qjl' if wl.qjl_m else ''}> + ipq_prep_kernel",
                     "algorithmic_bytes_per_launch": db_bytes + out_bytes, "avg_launch_us": round(ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_search(wl, spec, cache, q)
    print(json.dumps(res), flush=True)
    return 0


def cpu_baseline_search(wl, spec, cache, q):
    """The float64 oracle on the host: estimates of all queries against the
    first stream of the GPU's packed database (median of 3 runs)."""
    from oracle import pack as opk
    from oracle import quantize as oqz
    from oracle import search as osr
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    n = wl.n_tok
    os_ = oqz.Spec(bits_lo=wl.bits, bits_hi=wl.bits, split=128, qjl_m=wl.qjl_m,
                   rotation="haar" if spec.rotation == 0 else "hadamard")
    rb = kspec_bytes(spec)
    raw = cache.codes[:n * rb].cpu().numpy().reshape(n, rb)
    norms = cache.norms[:n].cpu().numpy()
    signs = cache.qjl_signs[:n * wl.qjl_m // 8].cpu().numpy().reshape(n, wl.qjl_m // 8) if wl.qjl_m else None
    gamma = cache.qjl_rnorms[:n].cpu().numpy() if wl.qjl_m else None
    qh = q.cpu().numpy()

    def once():
        t0 = time.perf_counter()
        idx = opk.unpack_records(raw, spec.widths)
        bits = opk.unpack_sign_bits(signs) if wl.qjl_m else None
        osr.ip_scores(qh, idx, norms, os_, bits=bits, gamma=gamma)
        return time.perf_counter() - t0

    t = float(np.median([once() for _ in range(3)]))
    per_vec = rb + 4 + (wl.qjl_m // 8 + 4 if wl.qjl_m else 0)
    nbytes = n * per_vec + wl.nq * 128 * 4 + wl.nq * n * 4
    return {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"estimates of the {wl.nq} queries against the first stream ({n} vectors) of the GPU's "
                      f"packed database, median of 3", "seconds": round(t, 3)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD,
                    help="workload to time (default: batched_ragged, the largest single-GPU configuration)")
    ap.add_argument("--rotation", choices=("haar", "hadamard", "hadamard_fwht"), default="haar",
                    help="how the rotation is drawn (the workloads are specified with the Haar rotation); "
                         "hadamard_fwht: the Hadamard matrix applied by butterflies in the key quantize")
    ap.add_argument("--kbits", type=int, choices=(8,), default=None,
                    help="keys at 8 bits (uniform, no sketch: the K8 of a K8/V3 policy) instead of the workload's")
    ap.add_argument("--norms", choices=("f32", "f16"), default="f32",
                    help="how key and value norms are stored (f16: binary16, 2 bytes per token and tensor)")
    ap.add_argument("--paged", action="store_true",
                    help="caches in a pool of 64-token pages, each sequence's pages in a seeded random order")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run a plain 512 MiB fp32 streaming kernel (out = -in) 5 times; "
                         "its byte counts calibrate rocprofv3's FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: turn two rocprofv3 --pmc runs of this script on --workload (FETCH_SIZE, then "
                         "WRITE_SIZE, with --copy-calibration) into profiles/traffic_<workload>_*.txt")
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_CSV", "OUT"),
                    help="no GPU: turn the kernel_stats.csv of a rocprofv3 --kernel-trace --stats run into a "
                         "short text summary (with --command and --title)")
    ap.add_argument("--counter-summary", nargs="+", metavar="PATH",
                    help="no GPU: RUN_DIR [RUN_DIR ...] OUT: per-kernel counter averages of rocprofv3 --pmc runs "
                         "of this script, written to OUT (with --command and --title)")
    ap.add_argument("--title", default="", help="first line of the --stats-summary / --counter-summary file")
    ap.add_argument("--command", default="", help="command line recorded by --traffic-summary")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary, args.workload, command=args.command)
    if args.stats_summary:
        return stats_summary(*args.stats_summary, title=args.title, command=args.command)
    if args.counter_summary:
        if len(args.counter_summary) < 2:
            ap.error("--counter-summary needs RUN_DIR [RUN_DIR ...] OUT")
        return counter_summary(args.counter_summary[:-1], args.counter_summary[-1], title=args.title,
                               command=args.command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); every box here has a single "
              f"MI355X and this path is not sharded across GPUs.", file=sys.stderr)
        return 2
    if args.workload == "ip_search":
        return bench_search(args)
    import torch
    from compressed_kv_cache_tq_amd import tq, workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    wname = args.workload
    wl = workloads.WORKLOADS[wname]
    inp = workloads.generate(wname)
    B, Hkv, Hq, S = len(inp.k), wl.hkv, wl.hq, wl.sink
    lens_h = np.asarray(inp.seq_lens, dtype=np.int64)
    comp_h = np.maximum(lens_h - S, 0)
    T = int(lens_h.max())
    cap = max(32, -(-int(comp_h.max()) // 32) * 32)
    uniform = bool(np.all(lens_h == lens_h[0]))
    f32 = wl.dtype == "f32"
    rot = {"haar": tq.ROT_HAAR, "hadamard": tq.ROT_HADAMARD, "hadamard_fwht": tq.ROT_HADAMARD_FWHT}[args.rotation]
    kspec = tq.Spec(wl.k.bits_lo, wl.k.bits_hi, split=wl.k.split, qjl_m=wl.k.qjl_m, layout=tq.LAYOUT_RECORD,
                    rot_seed=wl.k.rot_seed, qjl_seed=wl.k.qjl_seed, rotation=rot)
    if args.kbits == 8:
        kspec = tq.Spec(8, layout=tq.LAYOUT_RECORD, rot_seed=wl.k.rot_seed, rotation=rot)
    nf16 = 1 if args.norms == "f16" else 0
    kspec = dataclasses.replace(kspec, norm_f16=nf16)
    kb = (kspec.bits_lo, kspec.bits_lo if kspec.bits_hi is None else kspec.bits_hi)
    vspec = tq.Spec(wl.v.bits_lo, wl.v.bits_hi, split=wl.v.split, layout=tq.LAYOUT_TILED, rot_seed=wl.v.rot_seed,
                    rotation=rot, norm_f16=nf16)
    ktab, vtab = tq.device_tables(kspec), tq.device_tables(vspec)

    def device_input(parts):
        """[B * Hkv, cap, 128] zero-padded compressed tokens (bf16 bits or fp32)."""
        host = np.zeros((B * Hkv, cap, 128), dtype=np.float32 if f32 else np.uint16)
        for b in range(B):
            n = int(comp_h[b])
            if n:
                src = parts[b][:, S:S + n]
                host[b * Hkv:(b + 1) * Hkv, :n] = src if f32 else workloads.bf16_bits(src)
        t = torch.from_numpy(host if f32 else host.view(np.int16)).cuda()
        return t if f32 else t.view(torch.bfloat16)

    xk = [device_input(inp.k)]
    xv = [device_input(inp.v)]
    for _ in range(COPIES - 1):
        xk.append(xk[0].clone())
        xv.append(xv[0].clone())
    if args.paged:
        # every sequence's compressed tokens on its own pages of one pool, the
        # pool's pages handed out in a seeded random order
        npg = -(-comp_h // tq.PAGE_TOKENS)
        n_pages, max_pages = int(npg.sum()), max(1, int(npg.max()))
        perm = np.random.default_rng(7).permutation(n_pages).astype(np.int32)
        btab_h = np.full((B, max_pages), -1, dtype=np.int32)
        at = 0
        for b in range(B):
            btab_h[b, :npg[b]] = perm[at:at + npg[b]]
            at += int(npg[b])
        btab = torch.from_numpy(btab_h).cuda()
        kc = [tq.alloc_page_pool(kspec, n_pages, Hkv) for _ in range(COPIES)]
        vc = [tq.alloc_page_pool(vspec, n_pages, Hkv) for _ in range(COPIES)]
    else:
        kc = [tq.alloc_cache(kspec, B * Hkv, cap) for _ in range(COPIES)]
        vc = [tq.alloc_cache(vspec, B * Hkv, cap) for _ in range(COPIES)]
    sink_k = sink_v = None
    if S:
        sk = np.stack([inp.k[b][:, :S] for b in range(B)])
        sv = np.stack([inp.v[b][:, :S] for b in range(B)])
        sink_k = torch.from_numpy(workloads.bf16_bits(sk).view(np.int16)).cuda()
        sink_v = torch.from_numpy(workloads.bf16_bits(sv).view(np.int16)).cuda()
    q = torch.from_numpy(np.ascontiguousarray(inp.q, dtype=np.float32)).cuda()
    lens = torch.from_numpy(lens_h.astype(np.int32)).cuda()
    out = torch.empty_like(q)
    ws = tq.alloc_attend_workspace(B, Hq, Hkv, S, T)
    stream = torch.cuda.current_stream()

    def quantize(spec, tab, x, cache):
        if args.paged:
            tq.quantize_kv_paged(spec, tab, x, cache, hkv=Hkv, n_tok=comp_h, block_table=btab, n_pages=n_pages)
        elif uniform:
            tq.quantize_kv(spec, tab, x[:, :int(comp_h[0])], cache)
        else:  # one ragged call: each sequence appends its own length
            tq.quantize_kv_ragged(spec, tab, x, cache, hkv=Hkv, n_tok=comp_h)

    def attend(kcache, vcache):
        if args.paged:
            tq.attend_decode_paged(kspec, ktab, kcache, vspec, vtab, vcache, q, lens, out, ws, hkv=Hkv,
                                   block_table=btab, n_pages=n_pages, sink=S, sink_k=sink_k, sink_v=sink_v,
                                   v_skip=wl.v_skip, max_len=T)
            return
        tq.attend_decode(kspec, ktab, kcache, vspec, vtab, vcache, q, lens, out, ws, hkv=Hkv, sink=S,
                         sink_k=sink_k, sink_v=sink_v, v_skip=wl.v_skip, max_len=T)

    def step(i, ev=None):
        s, a = i % COPIES, (i + 1) % COPIES
        if ev is not None:
            ev[0].record(stream)
        quantize(kspec, ktab, xk[s], kc[s])
        if ev is not None:
            ev[1].record(stream)
        quantize(vspec, vtab, xv[s], vc[s])
        if ev is not None:
            ev[2].record(stream)
        attend(kc[a], vc[a])
        if ev is not None:
            ev[3].record(stream)

    for i in range(max(args.warmup, COPIES)):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    qk_step = np.array([e[0].elapsed_time(e[1]) for e in evs])
    qv_step = np.array([e[1].elapsed_time(e[2]) for e in evs])
    at_step = np.array([e[2].elapsed_time(e[3]) for e in evs])

    # Per-kernel launch durations: each phase launched back to back over the
    # rotating copies between two events (no event packets between launches),
    # as many launches as timed steps.
    def back_to_back(fn):
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ea.record(stream)
        for i in range(args.steps):
            fn(i)
        eb.record(stream)
        torch.cuda.synchronize()
        return ea.elapsed_time(eb) / args.steps

    qk_ms = back_to_back(lambda i: quantize(kspec, ktab, xk[i % COPIES], kc[i % COPIES]))
    qv_ms = back_to_back(lambda i: quantize(vspec, vtab, xv[i % COPIES], vc[i % COPIES]))
    # decode reads 31.5 MB per step: rotate over ten cache copies (315 MB, more
    # than the 256 MB Infinity Cache) so back-to-back steps still read HBM
    kc_b = kc + [tq.clone_cache(kc[i % COPIES]) for i in range(ATT_COPIES - COPIES)]
    vc_b = vc + [tq.clone_cache(vc[i % COPIES]) for i in range(ATT_COPIES - COPIES)]
    at_ms = back_to_back(lambda i: attend(kc_b[i % ATT_COPIES], vc_b[i % ATT_COPIES]))

    n_vec = int(Hkv * comp_h.sum())                        # compressed vectors per tensor
    kcb, vcb = tq.code_bytes(kspec), tq.code_bytes(vspec)
    nb = 2 if nf16 else 4                                            # bytes per stored norm
    k_tok = kcb + nb + (kspec.qjl_m // 8 + 4 if kspec.qjl_m else 0)  # codes, norm (+ signs, residual norm)
    v_tok = vcb + nb
    in_b = 512 if f32 else 256
    sink_bytes = int(Hkv * np.minimum(lens_h, S).sum()) * 2 * 128 * 2
    dec_bytes = n_vec * (k_tok + v_tok) + sink_bytes + 2 * B * Hq * 128 * 4
    qk_bytes = n_vec * (in_b + k_tok)
    qv_bytes = n_vec * (in_b + v_tok)
    dec_s = at_ms / 1e3
    quant_s = (qk_ms + qv_ms) / 1e3
    dec_gbs = dec_bytes / dec_s / 1e9
    quant_mvec = 2 * n_vec / quant_s / 1e6
    quant_gbs = (qk_bytes + qv_bytes) / quant_s / 1e9

    # dominant kernel of the step (largest device time): one of the two quantize launches
    ktag = f"{kb[0]},{kb[1]},{'f32' if f32 else 'bf16'},record{',qjl' if kspec.qjl_m else ''}"
    vtag = f"{wl.v.bits_lo},{wl.v.bits_hi},{'f32' if f32 else 'bf16'},tiled"
    kkern = "quantize_kernel" if kspec.qjl_m else "rotq_kernel"
    if qk_ms >= qv_ms:
        dom_name, dom_ms, dom_bytes, dom_kernel = "quantize_k", qk_ms, qk_bytes, f"{kkern}<{ktag}>"
    else:
        dom_name, dom_ms, dom_bytes, dom_kernel = "quantize_v", qv_ms, qv_bytes, f"rotq_kernel<{vtag}>"
    dom_gbs = dom_bytes / (dom_ms / 1e3) / 1e9
    default_cfg = not args.paged and args.kbits is None and not nf16 and args.rotation == "haar"
    traffic = read_traffic(wname, dom_name) if default_cfg else None
    roofline = {"bound": "hbm", "achieved": round(dom_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(dom_gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom_kernel,
                "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 2)}
    att_traffic = read_traffic(wname, "attend") if default_cfg else None
    roofline_attend = {"bound": "hbm", "achieved": round(dec_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "traffic": att_traffic,
                       "kernel": f"split_kernel<{kb[0]},{kb[1]},{wl.v.bits_lo},{wl.v.bits_hi}"
                                 f"{',qjl' if kspec.qjl_m else ''}{',paged' if args.paged else ''}> (+ combine_kernel when a stream has several splits;"
                                 f" one decode step)",
                       "algorithmic_bytes_per_launch": dec_bytes, "avg_launch_us": round(at_ms * 1e3, 2)}
    res = {
        "metric": METRIC, "value": round(dec_gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(total_ms / args.steps, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": wname, "batch": B, "q_heads": Hq, "kv_heads": Hkv, "d": 128,
                   "context": T if uniform else f"ragged {int(lens_h.min())}..{T}, sum {int(lens_h.sum())}",
                   "kv_dtype": wl.dtype, "k_bits": list(kb), "v_bits": [wl.v.bits_lo, wl.v.bits_hi],
                   "split": kspec.split, "qjl": bool(kspec.qjl_m), "sink": S, "v_skip": wl.v_skip,
                   "structure": wl.structure, "rotation": args.rotation,
                   "cache": f"paged ({tq.PAGE_TOKENS}-token pages)" if args.paged else "contiguous",
                   "norms": args.norms},
        "decode_pct_hbm_peak": round(100 * dec_gbs / HBM_PEAK_GBS, 2),
        "decode_us": round(at_ms * 1e3, 2),
        "quantize_Mvec_s": round(quant_mvec, 1), "quantize_GB_s": round(quant_gbs, 2),
        "quantize_pct_hbm_peak": round(100 * quant_gbs / HBM_PEAK_GBS, 2),
        "quantize_us": {"k": round(qk_ms * 1e3, 2), "v": round(qv_ms * 1e3, 2)},
        "in_step_us": {"quantize_k": round(qk_step.mean() * 1e3, 2), "quantize_v": round(qv_step.mean() * 1e3, 2),
                       "decode": round(at_step.mean() * 1e3, 2)},
        "roofline": roofline, "roofline_attend": roofline_attend,
    }
    if args.copy_calibration:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline and not args.paged:
        # a bounded sample: the first sequences up to about 600k compressed token-heads
        sample, tot = [], 0
        for b in range(B):
            if tot >= 600_000:
                break
            if comp_h[b] > 0:
                sample.append(b)
                tot += int(comp_h[b]) * Hkv
        res["cpu_baseline"] = cpu_baseline(inp, wl, kspec, vspec, kc[0], vc[0], comp_h, sample, k_tok + v_tok)
    if wl.v_skip > 0:
        # The value tiles are loaded two tiles ahead, before their weights are
        # known, so a skipped token saves its dequantization and MFMA work,
        # not its bytes: no bytes are subtracted from the decode figures.
        res["v_skip"] = {"threshold": wl.v_skip, "v_bytes_subtracted": 0,
                         "oracle_skip_rate": res.get("cpu_baseline", {}).get("v_skip_rate_oracle"),
                         "note": "skip rate of the exact rule (final weight < threshold) on the cpu_baseline "
                                 "decode sample; the kernel's one-pass rule skips a subset of those tokens"}
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
