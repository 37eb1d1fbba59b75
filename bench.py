#!/usr/bin/env python3
"""SparseGemv benchmark on one MI355X.

A step is one pass of the hot path over one batch: the four batch-1 GEMVs of
the LLaMA-7B-shaped MLP workload (up 4096 -> 11008 and down 11008 -> 4096,
each at 1:4 and at 2:4, adaptive INT4 groups: the 10 % most sensitive rows
use group 32, the rest group 128). Packing (prune, group choice, quantise,
2bit-CSR, layout) is offline host work done once before timing; its output
(the device blob) and x are resident in HBM when the timed region starts.

Timing protocol
* cold weights: every layer has R device copies, cycled so that the bytes
  touched between two uses of one copy exceed 512 MiB (twice the 256 MB
  Infinity Cache);
* exactly --warmup untimed steps, then exactly --steps timed steps, each set
  captured once in a HIP graph (so host dispatch cost is not measured) and
  replayed once; step i runs copy i % R of every layer, the timed steps
  continuing the cycle; HIP events on the launch stream bracket the timed
  replay, with a device synchronisation on both sides;
* per-layer µs/call: a graph of back-to-back launches of one layer (cycling
  its copies), timed the same way; beside it, for information only, the same
  launches on a single copy (``hot_us_per_call``: the blob stays in the
  Infinity Cache, so that figure is not an HBM rate);
* the practical ceiling of one launch (``ceiling``): an empty kernel, and a
  plain read of each layer's algorithmic bytes less y with one 16-byte load
  per lane, without and with a store of y's bytes, from the same cold
  copies and timed the same way as the layer;
* the oracle (NumPy FP64 dequantise-then-dot, and the dot alone on the
  pre-decoded W') is timed on the host cores on passes over the same four
  layers; for information, the library's packer and the oracle's pack the
  four layers once each beside it.

Beside the step, the same line reports
* ``ablation``: the up and down MLP weights as a dense INT4 layer (every
  element kept, same quantiser: the plain weight-only GEMV that SparseGemv
  extends), in the FP16-valued 2bit-CSR form (N:M sparsity without INT4) at
  2:4 and 1:4, and as a plain FP16 GEMV through torch (hipBLASLt, launched
  eagerly: a library call stays out of graph capture), at B = 1, cold, with
  the sparse layers' speedups;
* ``small_configs``: µs and GB/s per call of the single 1024 -> 1024 layer
  and the 4096 -> 4096 attention projection (2:4, uniform g = 128, B = 1),
  timed like the per-layer figures;
* ``beam``: µs and GB/s per call of the beam-batch shapes (up and down of
  decoder layers 0 (2:4) and 4 (1:4)) at B = 4, 8, 16, timed like the
  per-layer figures;
* ``decoder``: the 224 GEMVs of a 32-layer 7B-shaped decoder (q, k, v, o
  4096 -> 4096, gate and up 4096 -> 11008, down 11008 -> 4096; 2:4 in the
  first and last 4 layers, 1:4 elsewhere), launched back to back on one
  stream, each with its own x and y; 4 replays (after one warm replay) of a
  graph of 5 back-to-back passes over the whole sequence, once with one
  launch per GEMV, once with the launches a decode
  step can group (q, k and v together; o; gate and up together; down: 4
  launches per layer, sgemv_run_group), and twice as task lists of 48 GEMVs
  per launch (sgemv_run_list: 5 launches), once in the sequence order and
  once grouped by (N:M, K, N), and as one launch of all 224 from a task
  table in device memory (sgemv_list_table + sgemv_run_list_table). Every GEMV has its own device copy of its weights (1.79 GB in
  all, so the sequence is cold by construction); the copies of one (shape,
  N:M) pair are filled from one packed matrix, since the kernel's work and
  bytes depend only on the shape, the N:M choice and the number of rows per
  group size, which the adaptive policy fixes at ceil(N/10) fine rows.

Prints one JSON line. ``--gpus N`` with N > 1 is refused: the benchmark
measures one GPU (a multi-GPU layer would shard by output rows, each GPU
running this same kernel on its share).
"""
import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "SparseGemv µs/call + effective HBM GB/s (% of MI355X peak), batch 1"
HBM_PEAK_GBS = 8000.0
COLD_BYTES = 512 << 20


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layer-calls", type=int, default=400, help="launches per per-layer timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch from Python instead of a HIP graph")
    ap.add_argument("--no-beam", action="store_true", help="skip the beam-batch figures")
    ap.add_argument("--no-decoder", action="store_true", help="skip the 224-GEMV decoder sequence")
    ap.add_argument("--no-ablation", action="store_true", help="skip the dense INT4 / FP16 ablation")
    ap.add_argument("--no-small", action="store_true", help="skip the 1024x1024 and 4096x4096 layers")
    ap.add_argument("--no-hot", action="store_true", help="skip the cache-resident per-layer timing")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the empty-kernel and plain-read probes")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash():
    from sparse_weight_only_amd.profiling import kernel_source_hash as h
    return h()


def read_traffic(kernel_hash, layer_name):
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    path = os.path.join(ROOT, "profiles", "counters_cfg3.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_hash:
        return None
    return c.get("hbm_bytes_per_launch", {}).get(layer_name)


def cpu_baseline(layers_host):
    """The oracle, as it stands, on the host cores: (i) decode the 2bit-CSR
    arrays to a dense FP64 W' and np.dot, per layer; (ii) np.dot alone on the
    pre-decoded W'. One pass over the four layers is one sample; the median
    of (i) over as many passes as fill about 10 s (3 to 15) and of 5 (ii)
    passes is reported."""
    import numpy as np
    from oracle import gemv as ogemv
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in pools] + [1])
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in pools})) or "unknown"
    except Exception:
        threads, blas = int(os.environ.get("OMP_NUM_THREADS", "1")), "unknown"
    total_bytes = sum(l[3] for l in layers_host)
    t_dec = []
    passes = 3
    while len(t_dec) < passes:
        t0 = time.perf_counter()
        for (name, canon, X, nbytes, _, _) in layers_host:
            Wd = ogemv.dequant_dense(canon)
            ogemv.gemv(Wd, X)
            del Wd
        t_dec.append(time.perf_counter() - t0)
        if len(t_dec) == 1:
            passes = min(15, max(3, math.ceil(10.0 / t_dec[0])))
    dense = [(ogemv.dequant_dense(canon), X) for (_, canon, X, _, _, _) in layers_host]
    t_dot = []
    for rep in range(6):
        t0 = time.perf_counter()
        for Wd, X in dense:
            ogemv.gemv(Wd, X)
        if rep:                                   # the first pass warms up
            t_dot.append(time.perf_counter() - t0)
    del dense
    # information: the library's packer against the oracle's on the same
    # weights and group sizes (prune, INT4 quantisation, 2bit-CSR arrays)
    import sparse_weight_only_amd as sg
    from oracle import pack as opack
    t_lib = t_orc = 0.0
    for (_, _, _, _, L, gs) in layers_host:
        W = L.W()
        t0 = time.perf_counter()
        sg.pack(W, L.nk, gs)
        t_lib += time.perf_counter() - t0
        t0 = time.perf_counter()
        opack.pack_canonical(W, L.nk, gs)
        t_orc += time.perf_counter() - t0
        del W
    td, tt = statistics.median(t_dec), statistics.median(t_dot)
    return {"value": round(total_bytes / td / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "one pass over the 4 MLP layers: decode 2bit-CSR to dense FP64 W', then np.dot; "
                      f"median of {len(t_dec)} passes ({sum(t_dec):.1f} s in all), {td:.2f} s per pass",
            "dot_only": {"value": round(total_bytes / tt / 1e9, 4), "unit": "GB/s",
                         "sample": f"np.dot on the pre-decoded FP64 W' of the 4 layers, median of 5 passes, "
                                   f"{tt * 1e3:.1f} ms per pass"},
            "pack": {"library_s": round(t_lib, 3), "oracle_s": round(t_orc, 3),
                     "sample": "the 4 MLP layers packed once each (prune, INT4 quantisation, 2bit-CSR arrays) "
                               "from their FP16 weights and group sizes"},
            "affinity_cores": affinity, "blas": blas}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(a multi-GPU layer would shard by output rows, each GPU running the same kernel "
              "on its share)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synth
    import sparse_weight_only_amd as sg

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sg.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    # reference copy of known size (64 MiB read + 64 MiB written): the scale for
    # HBM byte counters collected over this same command
    ref_a = torch.empty(64 << 20, dtype=torch.uint8, device=dev).fill_(1)
    ref_b = torch.empty_like(ref_a)
    ref_b.copy_(ref_a)
    torch.cuda.synchronize()
    del ref_a, ref_b

    layers = synth.cfg3()
    t_pack = time.perf_counter()
    L_dev, layers_host = [], []
    for L in layers:
        W = L.W()
        gs = sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
        canon = sg.pack(W, L.nk, gs)
        desc = sg.describe(L.N, L.K, L.nk, gs)
        blob = sg.layout(desc, canon)
        nbytes = sg.algorithmic_bytes(desc, 1)
        X = L.X(1)
        L_dev.append({"L": L, "desc": desc, "blob_host": blob, "bytes": nbytes,
                      "x": torch.from_numpy(X).to(dev),
                      "y": torch.empty((1, L.N), dtype=torch.float16, device=dev)})
        layers_host.append((L.name, canon, X, nbytes, L, gs))
    t_pack = time.perf_counter() - t_pack
    step_bytes = sum(l["bytes"] for l in L_dev)
    for l in L_dev:
        # enough copies that one layer alone cycles through > 512 MiB
        l["R"] = max(2, -(-COLD_BYTES // l["desc"].blob_bytes))
        host = torch.from_numpy(l["blob_host"])
        l["copies"] = [host.to(dev) for _ in range(l["R"])]
    torch.cuda.synchronize()
    log(f"packed 4 layers in {t_pack:.1f} s; cold copies per layer: {[l['R'] for l in L_dev]}")

    # ---- timing helpers: a body of launches captured once in a HIP graph
    # (eager warm-up on the capture stream first), replayed on the current
    # stream between HIP events, with a device synchronisation either side
    def capture(body, eager_first=True):
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(dev)
        s.wait_stream(stream)
        if eager_first:
            with torch.cuda.stream(s):
                body()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            body()
        torch.cuda.synchronize()
        return g

    def replay_ms(g, reps):
        cur = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(cur)
        for r in range(reps):
            g.replay()
        e1.record(cur)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def timed(fn_graph_body, n_body, reps, warm):
        """ms per launch of a body of n_body launches, replayed reps times after warm replays."""
        if args.eager:
            for w in range(warm):
                fn_graph_body()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for r in range(reps):
                fn_graph_body()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / (reps * n_body)
        g = capture(fn_graph_body)
        for w in range(warm):
            g.replay()
        return replay_ms(g, reps) / (reps * n_body)

    # ---- whole step, exactly --warmup untimed then --steps timed steps; step
    # i runs copy i % R of every layer, the timed steps continuing the cycle
    # where the warm-up left it (the bytes between two uses of a copy stay
    # above 512 MiB, so every step is cold)
    def steps_body(first, count):
        def body():
            cur = torch.cuda.current_stream(dev)
            for i in range(first, first + count):
                for l in L_dev:
                    sg.run(l["desc"], l["copies"][i % l["R"]].data_ptr(), l["x"].data_ptr(), l["y"].data_ptr(), 1,
                           cur.cuda_stream)
        return body

    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)
    if args.eager:
        steps_body(0, args.warmup)()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        steps_body(args.warmup, args.steps)()
        e1.record(stream)
        torch.cuda.synchronize()
        ms_total = e0.elapsed_time(e1)
    else:
        # each layer's kernel launched once before capture (code-object
        # loading), not a step: the step graphs themselves are not run eagerly
        for l in L_dev:
            sg.run(l["desc"], l["copies"][0].data_ptr(), l["x"].data_ptr(), l["y"].data_ptr(), 1, stream.cuda_stream)
        torch.cuda.synchronize()
        g_timed = capture(steps_body(args.warmup, args.steps), eager_first=False)
        if args.warmup:
            g_warm = capture(steps_body(0, args.warmup), eager_first=False)
            g_warm.replay()
        ms_total = replay_ms(g_timed, 1)
    ms_per_step = ms_total / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # ---- per layer: back-to-back launches of one layer, cycling its copies
    per_layer = {}
    for l in L_dev:
        n_copies = l["R"]
        calls_per_graph = n_copies * max(1, args.layer_calls // (n_copies * 4))

        def body_layer(l=l, n=calls_per_graph):
            cur = torch.cuda.current_stream(dev)
            for i in range(n):
                sg.run(l["desc"], l["copies"][i % n_copies].data_ptr(), l["x"].data_ptr(), l["y"].data_ptr(), 1,
                       cur.cuda_stream)

        ms_call = timed(body_layer, calls_per_graph, 4, 1)
        us = ms_call * 1e3

        # informational: the same launches on one copy, whose blob then stays
        # in the 256 MB Infinity Cache between calls (not an HBM figure)
        def body_hot(l=l, n=calls_per_graph):
            cur = torch.cuda.current_stream(dev)
            for i in range(n):
                sg.run(l["desc"], l["copies"][0].data_ptr(), l["x"].data_ptr(), l["y"].data_ptr(), 1,
                       cur.cuda_stream)

        us_hot = None if args.no_hot else timed(body_hot, calls_per_graph, 4, 1) * 1e3
        pl = sg.plan(l["desc"], 1)
        per_layer[l["L"].name] = {"us_per_call": round(us, 3), "bytes": l["bytes"],
                                  "GBps": round(l["bytes"] / (us * 1e-6) / 1e9, 1),
                                  "pct_hbm_peak": round(100 * l["bytes"] / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                                  "hot_us_per_call": None if us_hot is None else round(us_hot, 3),
                                  "grid": pl.grid, "waves": pl.waves, "chunks_per_wave": pl.chunks_per_wave}

    # ---- the practical ceiling of one launch, timed the same way: an empty
    # kernel, and a plain 16-byte-per-lane read of the layer's algorithmic
    # bytes less y (from the same cold copies), without and with a store of
    # y's bytes
    ceiling = None
    if not args.no_ceiling:
        dst = torch.empty(max(l["L"].N for l in L_dev) * 2 + 64, dtype=torch.uint8, device=dev)

        def body_empty(n=400):
            cur = torch.cuda.current_stream(dev)
            for i in range(n):
                sg.probe_empty(1, 64, cur.cuda_stream)

        ceiling = {"empty_us": round(timed(body_empty, 400, 4, 1) * 1e3, 3), "layers": {}}
        for l in L_dev:
            n_copies = l["R"]
            n = n_copies * max(1, args.layer_calls // (n_copies * 4))
            y_bytes = 2 * l["L"].N
            rd = (l["bytes"] - y_bytes) // 16 * 16
            res = {"read_bytes": rd, "store_bytes": y_bytes}
            for key, st in (("read_us", 0), ("read_store_us", y_bytes)):
                def body_probe(l=l, n=n, st=st):
                    cur = torch.cuda.current_stream(dev)
                    for i in range(n):
                        sg.probe_read(l["copies"][i % n_copies].data_ptr(), rd, dst.data_ptr(), st,
                                      stream=cur.cuda_stream)
                res[key] = round(timed(body_probe, n, 4, 1) * 1e3, 3)
            pl_us = per_layer[l["L"].name]["us_per_call"]
            res["kernel_us"] = pl_us
            res["kernel_over_read_store"] = round(pl_us / res["read_store_us"], 3)
            res["read_store_pct_hbm_peak"] = round(100 * l["bytes"] / (res["read_store_us"] * 1e-6) / 1e9
                                                   / HBM_PEAK_GBS, 2)
            ceiling["layers"][l["L"].name] = res
        del dst
        log("ceiling probes timed")

    # dominant kernel: the layer with the largest time per step
    dom = max(per_layer, key=lambda k: per_layer[k]["us_per_call"])
    d = per_layer[dom]
    khash = kernel_source_hash()
    roofline = {"bound": "hbm", "achieved": d["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(d["GBps"] / HBM_PEAK_GBS, 4), "traffic": read_traffic(khash, dom),
                "kernel": dom, "bytes_per_launch": d["bytes"], "us_per_launch": d["us_per_call"],
                "timing": "HIP events around a graph of back-to-back launches cycling cold copies, per launch"}
    if ceiling is not None:
        c = ceiling["layers"][dom]
        roofline["frac_of_read_store_ceiling"] = round(c["read_store_us"] / d["us_per_call"], 4)
    # bytes per dense weight and per kept element: algorithmic, and from the
    # HBM counters where they were taken on these kernel sources
    for l in L_dev:
        L, pl = l["L"], per_layer[l["L"].name]
        dense, kept = L.N * L.K, L.N * L.K * L.nk // 4
        hbm = read_traffic(khash, L.name)
        pl["alg_bytes_per_dense_weight"] = round(l["bytes"] / dense, 4)
        pl["alg_bytes_per_kept"] = round(l["bytes"] / kept, 4)
        pl["hbm_bytes_per_launch"] = hbm
        pl["hbm_bytes_per_kept"] = None if hbm is None else round(hbm / kept, 4)

    def per_call_us(desc, copies, x, y, B, n_calls):
        n_copies = len(copies)
        n = n_copies * max(1, n_calls // (n_copies * 4))

        def body():
            cur = torch.cuda.current_stream(dev)
            for i in range(n):
                sg.run(desc, copies[i % n_copies].data_ptr(), x.data_ptr(), y.data_ptr(), B, cur.cuda_stream)

        return timed(body, n, 4, 1) * 1e3

    # ---- beam batches: up/down of decoder layers 0 (2:4) and 4 (1:4), B = 4, 8, 16
    beam = None
    if not args.no_beam:
        beam = {}
        for L in synth.cfg5():
            W = L.W()
            gs = sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
            desc = sg.describe(L.N, L.K, L.nk, gs)
            host = torch.from_numpy(sg.layout(desc, sg.pack(W, L.nk, gs)))
            R = max(2, -(-COLD_BYTES // desc.blob_bytes))
            copies = [host.to(dev) for _ in range(R)]
            beam[L.name] = {}
            for B in synth.CFG5_BATCHES:
                x = torch.from_numpy(L.X(B)).to(dev)
                y = torch.empty((B, L.N), dtype=torch.float16, device=dev)
                us = per_call_us(desc, copies, x, y, B, args.layer_calls)
                nb = sg.algorithmic_bytes(desc, B)
                beam[L.name][str(B)] = {"us_per_call": round(us, 3), "bytes": nb,
                                        "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                                        "pct_hbm_peak": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
            del copies
            torch.cuda.empty_cache()
        log("beam batches timed")

    # ---- the two single-layer configurations at B = 1: 1024 -> 1024 and the
    # 4096 -> 4096 attention projection (x with 1 % outlier channels), both
    # 2:4 with uniform g = 128, timed cold like the MLP layers
    small = None
    if not args.no_small:
        small = {}
        for L in synth.cfg1() + synth.cfg2():
            W = L.W()
            gs = np.full(L.N, synth.G_COARSE, dtype=np.int32)
            desc = sg.describe(L.N, L.K, L.nk, gs)
            host = torch.from_numpy(sg.layout(desc, sg.pack(W, L.nk, gs)))
            R = max(2, -(-COLD_BYTES // desc.blob_bytes))
            copies = [host.to(dev) for _ in range(R)]
            x = torch.from_numpy(L.X(1)).to(dev)
            y = torch.empty((1, L.N), dtype=torch.float16, device=dev)
            us = per_call_us(desc, copies, x, y, 1, args.layer_calls)
            nb = sg.algorithmic_bytes(desc, 1)
            small[L.name] = {"us_per_call": round(us, 3), "bytes": nb, "GBps": round(nb / (us * 1e-6) / 1e9, 1),
                             "pct_hbm_peak": round(100 * nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2),
                             "cold_copies": R}
            del copies
            torch.cuda.empty_cache()
        log("single-layer configurations timed")

    # ---- ablation at B = 1: the same MLP weights as a dense INT4 layer (every
    # element kept, same quantiser and groups policy) and as a plain FP16
    # GEMV through torch (hipBLASLt), each timed cold like the sparse layers
    ablation = None
    if not args.no_ablation:
        import dataclasses
        ablation = {}
        for L in [L for L in layers if L.nk == 2]:
            Ld = dataclasses.replace(L, nk=4)
            W = Ld.W()
            gs = sg.select_groups(W, 4, Ld.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
            desc = sg.describe(Ld.N, Ld.K, 4, gs)
            host = torch.from_numpy(sg.layout(desc, sg.pack(W, 4, gs)))
            R = max(2, -(-COLD_BYTES // desc.blob_bytes))
            copies = [host.to(dev) for _ in range(R)]
            x = torch.from_numpy(Ld.X(1)).to(dev)
            y = torch.empty((1, Ld.N), dtype=torch.float16, device=dev)
            us_d = per_call_us(desc, copies, x, y, 1, args.layer_calls)
            nb_d = sg.algorithmic_bytes(desc, 1)
            del copies
            w16 = torch.from_numpy(W).to(dev)
            R16 = max(2, -(-COLD_BYTES // (w16.numel() * 2)))
            wcopies = [w16.clone() for _ in range(R16)]
            n16 = R16 * max(1, args.layer_calls // (R16 * 4))

            # launched eagerly (a library GEMV is kept out of graph capture);
            # each call takes longer on the GPU than its host dispatch
            for i in range(R16):
                torch.nn.functional.linear(x, wcopies[i])
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            cur = torch.cuda.current_stream(dev)
            e0.record(cur)
            for i in range(n16):
                torch.nn.functional.linear(x, wcopies[i % R16])
            e1.record(cur)
            torch.cuda.synchronize()
            us_h = e0.elapsed_time(e1) * 1e3 / n16
            nb_h = w16.numel() * 2 + 2 * Ld.K + 2 * Ld.N
            del wcopies, w16
            torch.cuda.empty_cache()
            base = L.name.replace("_2of4", "")
            s24 = per_layer[base + "_2of4"]["us_per_call"]
            s14 = per_layer[base + "_1of4"]["us_per_call"]
            # the FP16-valued form (N:M sparsity without INT4) at both N:M choices
            f16 = {}
            for nk in (2, 1):
                d16 = sg.describe_fp16(Ld.N, Ld.K, nk)
                h16 = torch.from_numpy(sg.layout_fp16(d16, sg.pack_fp16(W, nk)))
                R = max(2, -(-COLD_BYTES // d16.blob_bytes))
                copies = [h16.to(dev) for _ in range(R)]
                us_f = per_call_us(d16, copies, x, y, 1, args.layer_calls)
                nb_f = sg.algorithmic_bytes(d16, 1)
                f16["2of4" if nk == 2 else "1of4"] = {"us_per_call": round(us_f, 3), "bytes": nb_f,
                                                      "GBps": round(nb_f / (us_f * 1e-6) / 1e9, 1)}
                del copies
            ablation[base] = {
                "dense_int4": {"us_per_call": round(us_d, 3), "bytes": nb_d, "GBps": round(nb_d / (us_d * 1e-6) / 1e9, 1)},
                "fp16_torch_linear": {"us_per_call": round(us_h, 3), "bytes": nb_h,
                                      "GBps": round(nb_h / (us_h * 1e-6) / 1e9, 1)},
                "fp16_values_2bitcsr": f16,
                "speedup_2of4_vs_dense_int4": round(us_d / s24, 3),
                "speedup_1of4_vs_dense_int4": round(us_d / s14, 3),
                "speedup_2of4_vs_fp16": round(us_h / s24, 3),
                "speedup_1of4_vs_fp16": round(us_h / s14, 3)}
        log("ablation timed")

    # ---- 224-GEMV decoder sequence, one launch per GEMV
    decoder = None
    if not args.no_decoder:
        # 5 sequences back to back per graph (as the per-layer figures time
        # back-to-back launches), replayed 4 times after one warm replay
        seqs_dec, reps_dec = 5, 4
        packed = {}
        for l in (0, 4):                        # one packed matrix per (shape, N:M)
            for m, (name, K, N) in enumerate(synth.LLAMA7B_MATS):
                key = (K, N, synth.layer_nk(l))
                if key in packed:
                    continue
                L = synth.Layer(f"decoder_l{l:02d}_{name}", K, N, key[2], True, 4, l, m, 4)
                W = L.W()
                gs = sg.select_groups(W, L.nk, L.Xcal(synth.CALIB_T), synth.FRAC_FINE, synth.G_FINE, synth.G_COARSE)
                desc = sg.describe(N, K, L.nk, gs)
                packed[key] = (desc, torch.from_numpy(sg.layout(desc, sg.pack(W, L.nk, gs))))
        seq = []
        dec_bytes = 0
        for i, L in enumerate(synth.cfg4()):
            desc, host = packed[(L.K, L.N, L.nk)]
            seq.append((desc, host.to(dev), torch.from_numpy(L.X(1)).to(dev),
                        torch.empty((1, L.N), dtype=torch.float16, device=dev)))
            dec_bytes += sg.algorithmic_bytes(desc, 1)
        torch.cuda.synchronize()

        def body_decoder():
            cur = torch.cuda.current_stream(dev)
            for (desc, blob, x, y) in seq:
                sg.run(desc, blob.data_ptr(), x.data_ptr(), y.data_ptr(), 1, cur.cuda_stream)

        # the same GEMVs grouped as a decode step can issue them: q, k, v
        # (inputs ready together); o; gate, up; down -> 4 launches per layer
        names = [name for name, _, _ in synth.LLAMA7B_MATS]
        launch_groups = [["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"], ["down_proj"]]
        grouped = []
        for l0 in range(0, len(seq), len(names)):
            for grp in launch_groups:
                grouped.append([(seq[l0 + names.index(m)][0], seq[l0 + names.index(m)][1].data_ptr(),
                                 seq[l0 + names.index(m)][2].data_ptr(), seq[l0 + names.index(m)][3].data_ptr())
                                for m in grp])

        def body_grouped():
            cur = torch.cuda.current_stream(dev)
            for tasks in grouped:
                sg.run_group(tasks, 1, cur.cuda_stream)

        # task-list launches of 48 GEMVs (the kernel-argument limit), 5 for
        # the 224: in the sequence order, and grouped by (N:M, K, N) so that a
        # launch holds one or two shapes (the GEMVs are independent: each has
        # its own x and y)
        from sparse_weight_only_amd.profiling import LIST_PER_LAUNCH, decoder_list_order
        keys = [(L.K, L.N, L.nk) for L in synth.cfg4()]

        def make_lists(by_shape):
            order = [seq[i] for i in decoder_list_order(keys, by_shape)]
            return [[(d, blob.data_ptr(), x.data_ptr(), y.data_ptr()) for (d, blob, x, y) in order[i: i + LIST_PER_LAUNCH]]
                    for i in range(0, len(order), LIST_PER_LAUNCH)]

        lists, lists_shape = make_lists(False), make_lists(True)

        def body_lists(ls):
            def body():
                cur = torch.cuda.current_stream(dev)
                for tasks in ls:
                    sg.run_list(tasks, 1, cur.cuda_stream)
            return body

        # all 224 as one launch: the task table in device memory
        table_host, table_launch = sg.list_table([(d, blob.data_ptr(), x.data_ptr(), y.data_ptr())
                                                  for (d, blob, x, y) in seq], 1)
        table_dev = torch.from_numpy(table_host).to(dev)

        def body_table():
            sg.run_list_table(table_dev.data_ptr(), table_launch, torch.cuda.current_stream(dev).cuda_stream)

        def times(body):
            def many():
                for _ in range(seqs_dec):
                    body()
            return timed(many, seqs_dec, reps_dec, 1)

        ms_seq = times(body_decoder)
        ms_grp = times(body_grouped)
        ms_lst = times(body_lists(lists))
        ms_lsh = times(body_lists(lists_shape))
        ms_tab = times(body_table)
        rate = lambda ms: {"us_per_sequence": round(ms * 1e3, 2), "GBps": round(dec_bytes / (ms * 1e-3) / 1e9, 1),
                           "pct_hbm_peak": round(100 * dec_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2)}
        decoder = {"gemvs": len(seq), "bytes": dec_bytes, "sequences_per_graph": seqs_dec, "replays": reps_dec,
                   "one_launch_per_gemv": dict(launches=len(seq), **rate(ms_seq)),
                   "grouped_qkv_o_gateup_down": dict(launches=len(grouped), **rate(ms_grp)),
                   "task_list": dict(launches=len(lists), gemvs_per_launch=LIST_PER_LAUNCH, order="sequence",
                                     **rate(ms_lst)),
                   "task_list_by_shape": dict(launches=len(lists_shape), gemvs_per_launch=LIST_PER_LAUNCH,
                                              order="grouped by N:M, K, N", **rate(ms_lsh)),
                   "task_table": dict(launches=1, gemvs_per_launch=len(seq), workgroups=table_launch.workgroups,
                                      grid_rows=table_launch.rows, **rate(ms_tab))}
        del seq, packed, table_dev
        torch.cuda.empty_cache()
        log("decoder sequence timed")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int4*f16->f32", "data": "synthetic",
        "config": {"workload": "cfg3: LLaMA-7B MLP up 4096->11008 and down 11008->4096, each at 1:4 and 2:4, "
                               "adaptive INT4 groups (ceil(N/10) rows g32, rest g128), FP16 x, batch 1",
                   "batch": 1, "step_bytes": step_bytes, "cold_copies": [l["R"] for l in L_dev],
                   "launch": "eager" if args.eager else "hip_graph"},
        "us_per_step": round(ms_per_step * 1e3, 3),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "per_layer": per_layer,
        "roofline": roofline,
        "ceiling": ceiling,
        "kernel_source_hash": khash,
        "pack_seconds": round(t_pack, 2),
    }
    if beam is not None:
        out["beam"] = beam
    if small is not None:
        out["small_configs"] = small
    if decoder is not None:
        out["decoder"] = decoder
    if ablation is not None:
        out["ablation"] = ablation
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers_host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
