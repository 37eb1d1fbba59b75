"""Summaries of rocprofv3 runs of ``bench.py`` for the ``profiles/`` folder.

Usage (after the rocprofv3 runs named in each summary's header):

    python -m sparse_weight_only_amd.profiling stats  <kernel_stats.csv> <out.txt> "<command>" [<kernel_trace.csv>]
    python -m sparse_weight_only_amd.profiling traffic <fetch counter_collection.csv>
                     <write counter_collection.csv> <out.json> "<fetch command>" "<write command>"
    python -m sparse_weight_only_amd.profiling counters <out.txt> <counter_collection.csv>... -- "<command>"...
    python -m sparse_weight_only_amd.profiling roofline <kernel_trace.csv> <bench.json> <out.txt>
                     "<trace command>" "<bench command>"
    python -m sparse_weight_only_amd.profiling list <kernel_trace.csv> <fetch csv> <write csv> <sq csv>
                     <out.txt> -- "<command>"...

``list`` summarises the task-list launches of the decoder sequence (in the
sequence order and grouped by shape): per launch position, the traced
duration, the algorithmic bytes (from the library's own descriptors of the
decoder GEMVs), the scaled HBM bytes and the SQ counters.

``traffic`` scales FETCH_SIZE and WRITE_SIZE (KiB per dispatch) by what the
same counters read for the 64 MiB reference copy that ``bench.py`` performs
at start-up (64 MiB read, 64 MiB written), and records them per workload
layer together with a hash of the kernel sources, so that ``bench.py``
reports HBM traffic only while the kernels are unchanged.
"""
import csv
import hashlib
import json
import os
import re
import statistics
import sys
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
REF_KIB = 64 * 1024          # the reference copy: 64 MiB each way


def _code_only(text: str) -> str:
    """C/C++ source without comments and blank space, so that the hash follows the code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the library sources (code only: comment edits keep recorded counters valid)."""
    h = hashlib.sha256()
    csrc = os.path.join(HERE, "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + b"\0" + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("sgemv_dev::", "").split("(")[0]


def stats_summary(stats_csv: str, out_txt: str, command: str, trace_csv: str = None) -> None:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 kernel statistics (kernel sources {kernel_source_hash()})",
             f"# command: {command}", "",
             f"{'kernel':62s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'pct':>6s}"]
    for r in rows:
        lines.append(f"{short_name(r['Name'])[:62]:62s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.3f} "
                     f"{float(r['MinNs']) / 1e3:9.3f} {float(r['MaxNs']) / 1e3:9.3f} {float(r['Percentage']):6.2f}")
    if trace_csv:
        # one kernel instantiation serves several layers: split its dispatches
        # by launch shape (grid lanes x workgroup lanes), which names the layer
        by = defaultdict(list)
        for r in csv.DictReader(open(trace_csv)):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]), int(r["Workgroup_Size_X"]))
            by[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        lines += ["", "per launch shape (dispatch durations from the kernel trace, us)",
                  f"{'kernel':40s} {'grid':>7s} {'wg':>5s} {'calls':>6s} {'avg':>7s} {'median':>7s} "
                  f"{'p10':>7s} {'p90':>7s}"]
        for (name, grid, wg), v in sorted(by.items(), key=lambda kv: -sum(kv[1])):
            if len(v) < 20:
                continue
            q = statistics.quantiles(v, n=10)
            lines.append(f"{name[:40]:40s} {grid:7d} {wg:5d} {len(v):6d} {statistics.mean(v):7.3f} "
                         f"{statistics.median(v):7.3f} {q[0]:7.3f} {q[-1]:7.3f}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def roofline_summary(trace_csv: str, bench_json: str, out_txt: str, command: str, bench_command: str) -> None:
    """Per MLP layer: the traced dispatch duration (average and median over
    the kernel trace), the HIP-event time per launch from a bench.py run
    without the profiler, and the fraction of 8 TB/s that each implies for
    the layer's algorithmic bytes."""
    with open(bench_json) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    by = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        key = (short_name(r["Kernel_Name"]), int(r["Grid_Size_X"]))
        by[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = [f"# roofline per MLP layer (kernel sources {kernel_source_hash()})",
             f"# kernel trace: {command}",
             f"# HIP events:   {bench_command}",
             "# frac = algorithmic bytes / time / 8 TB/s",
             "",
             f"{'layer':30s} {'bytes':>9s} {'trace_avg':>9s} {'trace_med':>9s} {'event_us':>9s} "
             f"{'frac_avg':>8s} {'frac_med':>8s} {'frac_evt':>8s}"]
    for layer, (kname, grid) in _bench_layer_kernels().items():
        pl = bench["per_layer"][layer]
        v = [d for (n, gsz), ds in by.items() if kname in n and gsz == grid for d in ds]
        if not v:
            continue
        avg, med, ev, nb = statistics.mean(v), statistics.median(v), pl["us_per_call"], pl["bytes"]
        fr = lambda us: nb / (us * 1e-6) / 8e12
        lines.append(f"{layer:30s} {nb:9d} {avg:9.3f} {med:9.3f} {ev:9.3f} {fr(avg):8.4f} {fr(med):8.4f} {fr(ev):8.4f}")
    rf = bench.get("roofline", {})
    lines += ["", f"bench.py roofline: kernel {rf.get('kernel')} frac {rf.get('frac')} "
                  f"({rf.get('us_per_launch')} us per launch, {rf.get('timing')})"]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_medians(path: str, counter: str):
    by = defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        by[(r["Kernel_Name"], int(r["Grid_Size"]), int(r["Workgroup_Size"]))].append(float(r["Counter_Value"]))
    return {k: statistics.median(v) for k, v in by.items()}


def _reference(med: dict) -> float:
    """Counter value of the 64 MiB reference copy (the largest copy dispatch)."""
    cands = [(v, k) for k, v in med.items() if "copyBuffer" in k[0] or "elementwise" in k[0] and "copy" in k[0].lower()]
    cands = [c for c in cands if c[0] > REF_KIB / 8]
    if not cands:
        raise RuntimeError("reference copy not found in the counter run")
    return max(cands)[0]


def traffic_summary(fetch_csv: str, write_csv: str, out_json: str, fetch_cmd: str, write_cmd: str,
                    layer_kernels: dict) -> dict:
    """layer_kernels: layer name -> (kernel name substring, grid size in lanes)."""
    fm = _counter_medians(fetch_csv, "FETCH_SIZE")
    wm = _counter_medians(write_csv, "WRITE_SIZE")
    f_scale = REF_KIB / _reference(fm)
    w_scale = REF_KIB / _reference(wm)
    out = {"kernel_source_hash": kernel_source_hash(), "fetch_scale": round(f_scale, 4),
           "write_scale": round(w_scale, 4), "fetch_command": fetch_cmd, "write_command": write_cmd,
           "hbm_bytes_per_launch": {}, "raw_kib_per_dispatch": {}}
    for layer, (kname, grid) in layer_kernels.items():
        fk = [v for k, v in fm.items() if kname in k[0] and k[1] == grid]
        wk = [v for k, v in wm.items() if kname in k[0] and k[1] == grid]
        if len(fk) != 1 or len(wk) != 1:
            continue
        out["raw_kib_per_dispatch"][layer] = {"FETCH_SIZE": fk[0], "WRITE_SIZE": wk[0]}
        out["hbm_bytes_per_launch"][layer] = int(round((fk[0] * f_scale + wk[0] * w_scale) * 1024))
    with open(out_json, "w") as f:
        json.dump(out, f, indent=1)
    return out


def _bench_layer_kernels() -> dict:
    """Kernel name and grid of each bench layer, from the library's own launch plan."""
    sys.path.insert(0, os.path.dirname(HERE))
    import numpy as np
    import synth
    import sparse_weight_only_amd as sg
    res = {}
    for L in synth.cfg3():
        W = L.W()
        gs = sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
        d = sg.describe(L.N, L.K, L.nk, gs)
        pl = sg.plan(d, 1)
        bucket = lambda n: 1 if n <= 1 else 2 if n <= 2 else 4 if n <= 4 else 8
        name = f"sgemv_b1_kernel<{L.nk}, {bucket(pl.chunks_per_wave)}, {bucket(pl.x_loads)}>"
        res[L.name] = (name, int(pl.grid * pl.block))
    return res


def counters_summary(csvs, out_txt: str, commands, min_calls: int = 20) -> None:
    """Median of every counter per launch shape (kernel, grid, workgroup) over
    one or more --pmc runs; shapes with fewer than min_calls dispatches are
    left out. Values are per dispatch, summed over the chip as rocprofv3
    reports them."""
    by = defaultdict(lambda: defaultdict(list))
    for path in csvs:
        for r in csv.DictReader(open(path)):
            key = (short_name(r["Kernel_Name"]), int(r["Grid_Size"]), int(r["Workgroup_Size"]))
            by[key][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for v in by.values() for c in v})
    lines = [f"# rocprofv3 counters per dispatch, median per launch shape (kernel sources {kernel_source_hash()})"]
    lines += [f"# command: {c}" for c in commands]
    lines += ["", f"{'kernel':34s} {'grid':>7s} {'wg':>5s} {'calls':>6s}  " + "  ".join(f"{n:>26s}" for n in names)]
    for (name, grid, wg), v in sorted(by.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        calls = max(len(x) for x in v.values())
        if calls < min_calls:
            continue
        vals = "  ".join(f"{statistics.median(v[n]):26.1f}" if n in v else f"{'-':>26s}" for n in names)
        lines.append(f"{name[:34]:34s} {grid:7d} {wg:5d} {calls:6d}  {vals}")
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


LIST_PER_LAUNCH = 48   # GEMVs per task-list launch of the decoder sequence (the kernel-argument limit)


def decoder_list_order(keys, by_shape: bool):
    """Order in which the task-list launches of the decoder sequence take its
    GEMVs: the sequence order, or grouped by (N:M, K, N) (stable), so that
    each launch holds GEMVs of one or two shapes. keys[i] = (K, N, nk) of
    GEMV i. The launches take LIST_PER_LAUNCH GEMVs at a time in this order."""
    idx = list(range(len(keys)))
    if by_shape:
        idx.sort(key=lambda i: (keys[i][2], keys[i][0], keys[i][1]))
    return idx


def _decoder_list_bytes(by_shape: bool):
    """(GEMVs, algorithmic bytes) of each task-list launch of the decoder
    sequence, each GEMV described by the library from its group selection."""
    sys.path.insert(0, os.path.dirname(HERE))
    import synth
    import sparse_weight_only_amd as sg
    descs = {}
    for l in (0, 4):
        for m, (name, K, N) in enumerate(synth.LLAMA7B_MATS):
            key = (K, N, synth.layer_nk(l))
            if key in descs:
                continue
            L = synth.Layer(f"decoder_l{l:02d}_{name}", K, N, key[2], True, 4, l, m, 4)
            W = L.W()
            gs = sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
            descs[key] = sg.describe(N, K, L.nk, gs)
    keys = [(L.K, L.N, L.nk) for L in synth.cfg4()]
    seq = [sg.algorithmic_bytes(descs[k], 1) for k in keys]
    seq = [seq[i] for i in decoder_list_order(keys, by_shape)]
    per = LIST_PER_LAUNCH
    return [(len(seq[i:i + per]), sum(seq[i:i + per])) for i in range(0, len(seq), per)]


LIST_KERNEL, TABLE_KERNEL = "sgemv_list_kernel", "sgemv_list_table_kernel"


def _list_rows(path: str, value_key: str, counter: str = None, kernel: str = LIST_KERNEL):
    """The dispatches of one task-list kernel in one run, in dispatch order."""
    rows = [r for r in csv.DictReader(open(path)) if kernel in r["Kernel_Name"]
            and (counter is None or r["Counter_Name"] == counter)]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return [float(r[value_key]) for r in rows]


def list_summary(trace_csv: str, fetch_csv: str, write_csv: str, sq_csv: str, out_txt: str, commands) -> None:
    """Per launch position of the decoder sequence's task lists, for each of
    the two orders bench.py times one after the other (the sequence order,
    then grouped by shape; the same number of passes each), and for the one
    table launch of all 224 GEMVs: traced duration, algorithmic bytes,
    counter-scaled HBM bytes and SQ counters."""
    orders = [("sequence order", _decoder_list_bytes(False)), ("grouped by shape", _decoder_list_bytes(True))]
    durations = lambda kernel: [(float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3
                                for r in sorted((r for r in csv.DictReader(open(trace_csv)) if kernel in r["Kernel_Name"]),
                                                key=lambda r: int(r["Dispatch_Id"]))]
    dur = durations(LIST_KERNEL)
    f_scale = REF_KIB / _reference(_counter_medians(fetch_csv, "FETCH_SIZE"))
    w_scale = REF_KIB / _reference(_counter_medians(write_csv, "WRITE_SIZE"))
    fetch = _list_rows(fetch_csv, "Counter_Value", "FETCH_SIZE")
    write = _list_rows(write_csv, "Counter_Value", "WRITE_SIZE")
    sq_names = sorted({r["Counter_Name"] for r in csv.DictReader(open(sq_csv))})
    sq = {n: _list_rows(sq_csv, "Counter_Value", n) for n in sq_names}
    nl_all = sum(len(l) for _, l in orders)
    med = statistics.median
    lines = [f"# sgemv_list_kernel on the 224-GEMV decoder sequence, {LIST_PER_LAUNCH} GEMVs a launch, and "
             f"sgemv_list_table_kernel, all 224 in one launch (kernel sources {kernel_source_hash()})"]
    lines += [f"# command: {c}" for c in commands]
    lines += [f"# HBM bytes = FETCH_SIZE x {f_scale:.4f} + WRITE_SIZE x {w_scale:.4f} (KiB, scaled by the 64 MiB "
              "reference copy of the same command); frac = algorithmic bytes / traced duration / 8 TB/s"]
    for name, v in [("trace", dur), ("fetch", fetch), ("write", write)] + list(sq.items()):
        if len(v) % nl_all:
            raise RuntimeError(f"{name}: {len(v)} list dispatches is not a whole number of passes of both orders")
    first = 0
    for title, launches in orders:
        nl = len(launches)
        part = lambda v: v[first * len(v) // nl_all: (first + nl) * len(v) // nl_all]
        pos = lambda v, i: part(v)[i::nl]
        lines += ["", f"{title}: {nl} launches a pass",
                  f"{'launch':>6s} {'gemvs':>5s} {'alg_bytes':>11s} {'calls':>5s} {'avg_us':>8s} {'med_us':>8s} "
                  f"{'frac_med':>8s} {'hbm_bytes':>11s} {'hbm/alg':>7s}"]
        tot_alg = tot_us = 0.0
        for i, (g, nb) in enumerate(launches):
            d = pos(dur, i)
            hbm = (med(pos(fetch, i)) * f_scale + med(pos(write, i)) * w_scale) * 1024
            tot_alg += nb
            tot_us += med(d)
            lines.append(f"{i:6d} {g:5d} {nb:11d} {len(d):5d} {statistics.mean(d):8.2f} {med(d):8.2f} "
                         f"{nb / (med(d) * 1e-6) / 8e12:8.4f} {int(hbm):11d} {hbm / nb:7.4f}")
        lines.append(f"{'all':>6s} {sum(g for g, _ in launches):5d} {int(tot_alg):11d} {'':5s} {'':8s} {tot_us:8.2f} "
                     f"{tot_alg / (tot_us * 1e-6) / 8e12:8.4f}")
        lines += [f"SQ counters per dispatch (median per launch position):",
                  f"{'launch':>6s} " + " ".join(f"{n:>16s}" for n in sq_names)]
        for i in range(nl):
            lines.append(f"{i:6d} " + " ".join(f"{med(pos(sq[n], i)):16.0f}" for n in sq_names))
        first += nl
    tdur = durations(TABLE_KERNEL)
    if tdur:
        nb = sum(b for _, b in orders[0][1])
        g = sum(n for n, _ in orders[0][1])
        tf = _list_rows(fetch_csv, "Counter_Value", "FETCH_SIZE", TABLE_KERNEL)
        tw = _list_rows(write_csv, "Counter_Value", "WRITE_SIZE", TABLE_KERNEL)
        hbm = (med(tf) * f_scale + med(tw) * w_scale) * 1024
        lines += ["", "one table launch of all the GEMVs (sgemv_run_list_table)",
                  f"{'launch':>6s} {'gemvs':>5s} {'alg_bytes':>11s} {'calls':>5s} {'avg_us':>8s} {'med_us':>8s} "
                  f"{'frac_med':>8s} {'hbm_bytes':>11s} {'hbm/alg':>7s}",
                  f"{0:6d} {g:5d} {nb:11d} {len(tdur):5d} {statistics.mean(tdur):8.2f} {med(tdur):8.2f} "
                  f"{nb / (med(tdur) * 1e-6) / 8e12:8.4f} {int(hbm):11d} {hbm / nb:7.4f}",
                  "SQ counters per dispatch (median):",
                  f"{'launch':>6s} " + " ".join(f"{n:>16s}" for n in sq_names),
                  f"{0:6d} " + " ".join(f"{med(_list_rows(sq_csv, 'Counter_Value', n, TABLE_KERNEL)):16.0f}"
                                        for n in sq_names)]
    with open(out_txt, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "stats":
        stats_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5] if len(sys.argv) > 5 else None)
    elif len(sys.argv) >= 7 and sys.argv[1] == "roofline":
        # roofline <kernel_trace.csv> <bench.json> <out.txt> "<trace command>" "<bench command>"
        roofline_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6])
    elif len(sys.argv) >= 4 and sys.argv[1] == "counters":
        # counters <out.txt> <csv>... -- <command>...
        sep = sys.argv.index("--")
        counters_summary(sys.argv[3:sep], sys.argv[2], sys.argv[sep + 1:])
    elif len(sys.argv) >= 7 and sys.argv[1] == "traffic":
        print(json.dumps(traffic_summary(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6],
                                         _bench_layer_kernels()), indent=1))
    elif len(sys.argv) >= 9 and sys.argv[1] == "list":
        # list <trace.csv> <fetch.csv> <write.csv> <sq.csv> <out.txt> -- <command>...
        sep = sys.argv.index("--")
        list_summary(*sys.argv[2:7], sys.argv[sep + 1:])
    else:
        print(__doc__)
        sys.exit(2)
