"""Benchmark of the UNO decode-cycle sampling path on one MI355X.

A step is one full cycle of the hot path over one batch of synthetic logits
already resident in HBM: for the linear workloads one uno_sample_linear call
(filter every draft and target row, proposals, acceptance, residual / bonus);
for the tree workloads one uno_build_tree plus one uno_verify_tree call.
Inputs rotate over a pool of distinct cycles (> 1.5 GB) so the 256 MB
Infinity Cache cannot serve repeated steps.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import math
import numpy as np
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "verified vocab rows/sec + achieved HBM GB/s (vocab 151936, linear 8/1/8 b64)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
DOMINANT = "topk_stream_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "topk_stream_kernel_linear_8_1_8_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="linear_8_1_8")
    ap.add_argument("--pool", type=int, default=3, help="distinct input cycles rotated through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--traffic-probe", type=int, default=0, metavar="N",
                    help="only run N launches of the timed filter kernel and N plain device copies "
                         "of the same byte count (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs)")
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for f in ("filter_kernels.hip", "uno_device.h", "uno_internal.h", "exp2_table.inc"):
        with open(os.path.join(ROOT, "lossless_draft_verify_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_entry():
    """HBM bytes per launch of the dominant kernel from committed rocprofv3
    counter runs, if they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def traffic_probe(args, w, lib, pool, dt, sp, stream, dev):
    """The dominant kernel alone (the same uno_filter launch the bench times) and a
    plain device-to-device copy of the same number of bytes, N times each; the
    copy calibrates the HBM byte counters."""
    import ctypes
    import torch
    import lossless_draft_verify_amd as uno
    a = pool[0]["all"]
    nrows = a.shape[0]
    ids = torch.empty((nrows, w.top_k), dtype=torch.int32, device=dev)
    probs = torch.empty((nrows, w.top_k), dtype=torch.float64, device=dev)
    cnt = torch.empty(nrows, dtype=torch.int32, device=dev)
    fws_n = uno.workspace_bytes(uno.OP_FILTER, nrows, 0, 0, 0, w.vocab, dt, w.temperature, w.top_k, w.top_p,
                               w.order)
    fws = torch.empty(fws_n + 256, dtype=torch.uint8, device=dev)
    fws_p = ctypes.c_void_p((fws.data_ptr() + 255) // 256 * 256) if fws_n else None
    src = pool[1 % len(pool)]["all"]
    dst = torch.empty_like(src)
    for i in range(args.traffic_probe):
        st = lib.uno_filter(ctypes.c_void_p(pool[i % len(pool)]["all"].data_ptr()), dt, nrows, w.vocab,
                            sp, w.top_k, ctypes.c_void_p(ids.data_ptr()),
                            ctypes.c_void_p(probs.data_ptr()), ctypes.c_void_p(cnt.data_ptr()), None, fws_p,
                            fws_n, ctypes.c_void_p(stream.cuda_stream))
        assert st == 0, st
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] traffic probe: {args.traffic_probe} x uno_filter ({nrows} rows) + {args.traffic_probe} x copy "
        f"of {src.numel() * src.element_size()} bytes")


def read_reference(lib, pool, nbytes, row_bytes, n, stream, dev):
    """Achievable streaming rate on this device: uno_stream_read over the same
    rows the filter reads, once with one workgroup per row (the top-k stream's
    decomposition) and once in 2048 equal ranges; HIP events on the launch
    stream over n launches each."""
    import ctypes
    import torch
    out = {"bytes": nbytes}
    res = torch.empty(nbytes // row_bytes + 4096, dtype=torch.int32, device=dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flat = (nbytes // 2048 + 15) // 16 * 16
    for key, wg in (("row_per_workgroup", row_bytes), ("flat", flat)):
        def go(i):
            st = lib.uno_stream_read(ctypes.c_void_p(pool[i % len(pool)]["all"].data_ptr()), nbytes, wg,
                                     ctypes.c_void_p(res.data_ptr()), ctypes.c_void_p(stream.cuda_stream))
            assert st == 0, st
        for i in range(10):
            go(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(n):
            go(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        us = ev0.elapsed_time(ev1) * 1e3 / n
        out[key + "_us"] = round(us, 2)
        out[key + "_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        log(f"[bench] read-only reference ({key}, {nbytes // wg} workgroups): {us:.1f} us -> "
            f"{out[key + '_gbs']:.0f} GB/s")
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def bench_tree_attention(args, uno, synth, dev):
    """uno_tree_attention at a tree workload's verify shape: K timed calls."""
    import torch
    a = synth.ATTENTION_WORKLOADS[args.workload]
    batch, n, Hq, Hkv, D = a["batch"], a["n"], a["Hq"], a["Hkv"], a["D"]
    q, k, v, op, lp, par = synth.attention_inputs(batch, n, Hq, Hkv, D, a["seed"], device=dev)
    scale = float(1.0 / math.sqrt(D))
    out = dict(o=torch.empty_like(q), lse=torch.empty_like(lp))
    stream = torch.cuda.current_stream()
    uno.tree_attention(q, k, v, op, lp, par, None, scale, out=out)      # argument checks once
    # then direct C-ABI calls with pre-built arguments
    import ctypes
    lib = uno.load_library()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    cargs = (P(q), P(k), P(v), P(op), P(lp), P(par), None, 1, batch, n, Hq, Hkv, D, ctypes.c_float(scale),
             P(out["o"]), P(out["lse"]), ctypes.c_void_p(stream.cuda_stream))
    call = lib.uno_tree_attention
    for _ in range(args.warmup):
        assert call(*cargs) == 0
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        call(*cargs)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    us = ev0.elapsed_time(ev1) * 1e3 / args.steps
    T = batch * n
    # one read of q, k, v, o_prefix, lse_prefix and the parents, one write of o and lse
    nbytes = 2 * T * (3 * Hq + 2 * Hkv) * D + 8 * T * Hq + 4 * T
    achieved = nbytes / (us * 1e-6) / 1e9
    log(f"[bench] {args.workload}: {us:.2f} us/call (events), {T} verify tokens, {nbytes / 1e6:.1f} MB, "
        f"{achieved:.0f} GB/s ({100 * achieved / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f})")
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        f = lambda t: t.float().cpu().numpy()
        qs, ks, vs, os_, ls, ps = (f(t) if t.dtype != torch.int32 else t.cpu().numpy() for t in (q, k, v, op, lp, par))
        t0 = time.perf_counter()
        reps = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 5.0):
            oracle.tree_attention(qs, ks, vs, os_, ls, ps, [n] * batch, scale)
            reps += 1
        el = time.perf_counter() - t0
        cpu = {"value": round(reps * T / el, 1), "unit": "verify tokens/s", "cores": oracle.num_threads(),
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"{reps} calls of {args.workload} ({T} tokens each), {el:.1f} s"}
    res = {
        "metric": "verify tokens/s (tree-suffix attention merged with the prefix state)",
        "value": round(T / (us * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(us / 1e3, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "batch": batch, "verify_tokens": n, "heads": Hq, "kv_heads": Hkv,
                   "head_dim": D},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "tree_attention_kernel",
                     "kernel_us": round(us, 3), "bytes_per_launch": nbytes},
        "cpu_baseline": cpu,
        "wall_s": round(wall, 4),
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sampling path runs on one GPU; requests shard across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import torch
    import lossless_draft_verify_amd as uno
    from lossless_draft_verify_amd import synth
    from lossless_draft_verify_amd import build as hip_build

    if not os.path.exists(hip_build.LIB):
        hip_build.build()
    uno.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.workload in synth.ATTENTION_WORKLOADS:
        bench_tree_attention(args, uno, synth, dev)
        return
    w = synth.WORKLOADS[args.workload]
    stream = torch.cuda.current_stream()

    # ---- input pool -------------------------------------------------------------
    pool = []
    t0 = time.time()
    for c in range(args.pool):
        if w.mode == "linear":
            # draft and target rows in one buffer, so uno_filter can replay the
            # exact filter launch of the step over the same rows
            draft, target = synth.linear_inputs(w, cycle=c, device=dev)
            allrows = torch.empty((w.batch * (2 * w.B + 1), w.vocab), dtype=draft.dtype, device=dev)
            nd = w.batch * w.B
            allrows[:nd] = draft.view(nd, w.vocab)
            allrows[nd:] = target.view(-1, w.vocab)
            del draft, target
            d = allrows[:nd].view(w.batch, w.B, w.vocab)
            t = allrows[nd:].view(w.batch, w.B + 1, w.vocab)
            pool.append(dict(all=allrows, draft=d, target=t))
        else:
            draft, R = synth.tree_inputs(w, cycle=c, device=dev)
            tree = uno.build_tree(draft, w.K, w.V, w.temperature, w.top_k, w.top_p, order=w.order)
            tgt = synth.tree_target_rows(R, tree["node_depth"], tree["num_nodes"], w.V)
            del R
            pool.append(dict(draft=draft, target=tgt))
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: pool of {args.pool} cycles ready in {time.time() - t0:.1f}s "
        f"({w.bytes_per_cycle / 1e6:.1f} MB per cycle)")

    # ---- step: direct C-ABI calls with pre-built arguments -------------------------
    import ctypes
    lib = uno.load_library()
    dt = 0 if w.dtype == "f32" else 1
    # one parameter set, or one per request (the mixed workload)
    sets = [w.request_params(b) for b in range(w.batch)] if w.mixed else [w.request_params(0)]
    sp = (uno.Sampling * len(sets))(*[uno.Sampling(*x) for x in sets])
    spr, nsp = sp, len(sets)
    cols = [np.array([x[j] for x in sets]) for j in range(4)] if w.mixed else \
        [w.temperature, w.top_k, w.top_p, w.order]
    sptr = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None

    def wsbuf(op, K, V):
        n = uno.workspace_bytes(op, w.batch, w.B, K, V, w.vocab, dt, *cols)
        if n == 0:
            return None, 0
        t = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        a = (t.data_ptr() + 255) // 256 * 256
        return (t, ctypes.c_void_p(a)), t.numel() - (a - t.data_ptr())

    if w.mode == "linear":
        tokens = torch.empty((w.batch, w.B + 1), dtype=torch.int32, device=dev)
        acc = torch.empty(w.batch, dtype=torch.int32, device=dev)
        prop = torch.empty((w.batch, w.B), dtype=torch.int32, device=dev)
        flags = torch.empty(w.batch, dtype=torch.int32, device=dev)
        ws, wsn = wsbuf(uno.OP_SAMPLE_LINEAR, 1, w.B)
        ptrs = [(P(p["draft"]), P(p["target"])) for p in pool]

        def step(i):
            d, t = ptrs[i % len(ptrs)]
            st = lib.uno_sample_linear_ex(d, t, dt, w.batch, w.B, w.vocab, spr, nsp, w.seed, i, None, P(tokens), P(acc),
                                       P(prop), P(flags), ws[1] if ws else None, wsn, sptr)
            if st != 0:
                raise uno.UnoError(st, "uno_sample_linear")
            return acc
    else:
        ntok = torch.empty((w.batch, w.V + 1), dtype=torch.int32, device=dev)
        npar = torch.empty_like(ntok)
        ndep = torch.empty_like(ntok)
        nnum = torch.empty(w.batch, dtype=torch.int32, device=dev)
        tokens = torch.empty((w.batch, w.B + 1), dtype=torch.int32, device=dev)
        path = torch.empty_like(tokens)
        acc = torch.empty(w.batch, dtype=torch.int32, device=dev)
        flags = torch.empty(w.batch, dtype=torch.int32, device=dev)
        wsb, wsbn = wsbuf(uno.OP_BUILD_TREE, w.K, w.V)
        wsv, wsvn = wsbuf(uno.OP_VERIFY_TREE, 1, w.V)
        ptrs = [(P(p["draft"]), P(p["target"])) for p in pool]

        def step(i):
            d, t = ptrs[i % len(ptrs)]
            st = lib.uno_build_tree_ex(d, dt, w.batch, w.B, w.K, w.V, w.vocab, spr, nsp, P(ntok), P(npar), P(ndep), None,
                                    P(nnum), wsb[1] if wsb else None, wsbn, sptr)
            if st != 0:
                raise uno.UnoError(st, "uno_build_tree")
            st = lib.uno_verify_tree_ex(t, dt, w.batch, w.B, w.V, w.vocab, spr, nsp, w.seed, i, None, P(ntok), P(npar),
                                     P(nnum), P(tokens), P(path), P(acc), P(flags), wsv[1] if wsv else None,
                                     wsvn, sptr)
            if st != 0:
                raise uno.UnoError(st, "uno_verify_tree")
            return acc

    if args.traffic_probe:
        traffic_probe(args, w, lib, pool, dt, sp, stream, dev)
        return

    # warm-up steps also give the tokens-per-forward figure (outside the timed region)
    acc_total = 0
    for i in range(args.warmup):
        acc_total += int(step(i).sum().item())
    tpf = acc_total / (2.0 * w.batch * max(args.warmup, 1))
    torch.cuda.synchronize()

    # ---- timed steps --------------------------------------------------------------
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = 1e3 * wall / args.steps
    rows_per_s = w.rows_per_cycle * args.steps / wall
    gbs = w.bytes_per_cycle * args.steps / wall / 1e9
    log(f"[bench] {args.steps} steps: {ms_per_step * 1e3:.1f} us/step (events {ev_ms / args.steps * 1e3:.1f} us), "
        f"{rows_per_s / 1e6:.2f} M rows/s, {gbs:.0f} GB/s algorithmic, TPF {tpf:.3f} (warm-up steps)")

    # ---- dominant kernel: the same filter launch, timed alone with HIP events ------
    roofline = None
    if w.mode == "linear" and w.top_k > 0 and w.order == uno.ORDER_TOPK_FIRST and not w.mixed:
        ids = torch.empty((pool[0]["all"].shape[0], w.top_k), dtype=torch.int32, device=dev)
        probs = torch.empty((pool[0]["all"].shape[0], w.top_k), dtype=torch.float64, device=dev)
        cnt = torch.empty(pool[0]["all"].shape[0], dtype=torch.int32, device=dev)
        nrows = pool[0]["all"].shape[0]
        n_f = max(50, min(args.steps, 500))
        fws_n = uno.workspace_bytes(uno.OP_FILTER, nrows, 0, 0, 0, w.vocab, dt, w.temperature, w.top_k, w.top_p,
                               w.order)
        fws = torch.empty(fws_n + 256, dtype=torch.uint8, device=dev)
        fws_p = ctypes.c_void_p((fws.data_ptr() + 255) // 256 * 256) if fws_n else None

        def filt(i):
            a = pool[i % len(pool)]["all"]
            st = lib.uno_filter(ctypes.c_void_p(a.data_ptr()), dt, nrows, w.vocab, sp, w.top_k,
                                ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(probs.data_ptr()),
                                ctypes.c_void_p(cnt.data_ptr()), None, fws_p, fws_n,
                                ctypes.c_void_p(stream.cuda_stream))
            assert st == 0, st
        for i in range(10):
            filt(i)
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(n_f):
            filt(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        k_us = ev0.elapsed_time(ev1) * 1e3 / n_f
        alg_bytes = nrows * w.vocab * w.elem_bytes
        achieved = alg_bytes / (k_us * 1e-6) / 1e9
        traffic = traffic_entry()
        ref = read_reference(lib, pool, alg_bytes, w.vocab * w.elem_bytes, n_f, stream, dev)
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "kernel": DOMINANT, "kernel_us": round(k_us, 2), "bytes_per_launch": alg_bytes,
                    "read_reference": ref,
                    "frac_of_read_reference": round(achieved / ref["flat_gbs"], 4)}
        log(f"[bench] {DOMINANT}: {k_us:.1f} us/launch over {n_f} launches -> {achieved:.0f} GB/s "
            f"({100 * achieved / HBM_PEAK_GBS:.1f}% of {HBM_PEAK_GBS:.0f}, "
            f"{100 * achieved / ref['flat_gbs']:.1f}% of the read-only reference)")

    # ---- CPU baseline: the oracle on a bounded sample of the same workload ----------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        p = pool[0]
        n_req = 0
        rows = 0
        t0 = time.perf_counter()
        if w.mode == "linear":
            dnp = synth.as_float32_numpy(p["draft"])
            tnp = synth.as_float32_numpy(p["target"])
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < args.cpu_seconds and n_req < w.batch * 8:
                lo = n_req % w.batch
                hi = min(lo + 16, w.batch)
                if w.mixed:
                    for b in range(lo, hi):
                        T, k, p_, o = w.request_params(b)
                        oracle.linear(dnp[b:b + 1], tnp[b:b + 1], T, k, p_, w.seed, 0,
                                      request_ids=np.array([b], dtype=np.uint32), order=o)
                else:
                    oracle.linear(dnp[lo:hi], tnp[lo:hi], w.temperature, w.top_k, w.top_p, w.seed, 0,
                                  request_ids=np.arange(lo, hi, dtype=np.uint32), order=w.order)
                n_req += hi - lo
                rows += (hi - lo) * (2 * w.B + 1)
        else:
            dnp = synth.as_float32_numpy(p["draft"])
            tnp = synth.as_float32_numpy(p["target"])
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < args.cpu_seconds and n_req < w.batch * 8:
                lo = n_req % w.batch
                hi = min(lo + 16, w.batch)
                tr = oracle.build_tree(dnp[lo:hi], w.K, w.V, w.temperature, w.top_k, w.top_p, order=w.order)
                oracle.verify_tree(tnp[lo:hi], w.B, tr["node_token"], tr["node_parent"], tr["num_nodes"],
                                   w.temperature, w.top_k, w.top_p, w.seed, 0,
                                   request_ids=np.arange(lo, hi, dtype=np.uint32), order=w.order)
                n_req += hi - lo
                rows += (hi - lo) * (w.B + w.V + 1)
        el = time.perf_counter() - t0
        cpu = {"value": round(rows / el, 1), "unit": "rows/s", "cores": oracle.num_threads(),
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"{n_req} request-cycles ({rows} rows) of {w.name}, {el:.1f} s"}
        log(f"[bench] oracle: {rows / el:.0f} rows/s on {oracle.num_threads()} threads ({n_req} requests)")

    res = {
        "metric": METRIC,
        "value": round(rows_per_s, 1),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "B": w.B, "K": w.K, "V": w.V or w.B,
                   "vocab": w.vocab, "logits": w.dtype, "temperature": w.temperature, "top_k": w.top_k,
                   "top_p": w.top_p, "rows_per_step": w.rows_per_cycle, "bytes_per_step": w.bytes_per_cycle,
                   "pool_cycles": args.pool,
                   **({"per_request": [list(x) for x in w.sets]} if w.mixed else {})},
        "hbm_gbs_algorithmic": round(gbs, 1),
        "tpf": round(tpf, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
