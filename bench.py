"""Benchmark of the CSA decode step on one MI355X.

One step = score every packed indexer row, select the exact top-512, attend
over the selected packed KV rows, for every session of the workload (all of
it inside libcsa.so).  Inputs are seeded synthetic data already resident in
HBM.  Before every timed step the 256 MB Infinity Cache (MALL) and the L2s
are flushed by reading a 1 GiB buffer outside the step's events, so each
step streams its history from HBM ("cold"); back-to-back ("warm") timing is
reported as a secondary figure.

Prints one JSON line (rank 0).  Usage:
    python bench.py [--gpus 1] [--steps 50] [--warmup 3] [--workload frontier-1m-rows]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "CSA decode-step latency (ms) + achieved HBM GB/s vs peak at 128K–1M rows"


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="frontier-1m-rows")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-rows", type=int, default=0,
                   help="rows of session 0 the oracle runs on (0: the whole session)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="repeat the oracle step until this much CPU time has been measured")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (scale for the HBM byte counters)")
    p.add_argument("--no-sweep", action="store_true",
                   help="skip the per-history-length figures of the other workloads")
    p.add_argument("--sweep-steps", type=int, default=20)
    p.add_argument("--no-fit", action="store_true", help="skip the fixed + marginal cost fit over history lengths")
    p.add_argument("--steps-only", action="store_true",
                   help="run decode steps only (no MXFP4-query leg, no filter diagnostics, no fit, no sweep, no CPU "
                        "baseline): for kernel traces and counters")
    p.add_argument("--query-format", default="fp32", choices=("fp32", "mxfp4"),
                   help="indexer query format of the headline steps")
    return p.parse_args()


# Kernel sources whose HBM counters profiles/ records; the recorded figures
# are used only while these files are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tile_kernel_frontier-1m-rows_hbm_counters.txt")
TRAFFIC_SOURCES = ["csa_topk_tile.hip", "csa_score.hpp", "csa_bound.hpp", "csa_select.hpp", "csa_stream.hpp",
                   "csa_device.hpp", "csa_attn.hpp", "csa_internal.hpp"]


def kernel_source_hash() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, "long_context_sparse_score_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the fused tile kernel from the recorded
    FETCH_SIZE / WRITE_SIZE counters, each scaled by what the same counter
    read for a copy of known size; None if not recorded for this workload or
    the kernel sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        if kv.get("workload") != workload or kv.get("source_sha256_16") != kernel_source_hash():
            return None
        return int(round(float(kv["scaled_fetch_bytes_per_launch"]) + float(kv["scaled_write_bytes_per_launch"])))
    except (KeyError, ValueError):
        return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(mib: int):
    import torch

    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads n bytes, writes n bytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}),
          flush=True)


def algorithmic_bytes(n_rows: int, n_idx_heads: int, n_heads: int) -> dict:
    """Bytes a decode step must move at least once (one session)."""
    k = min(512, n_rows)
    score = 68 * n_rows + 4 * 128 * n_idx_heads + 4 * n_idx_heads
    attn = 583 * k + 4 * 512 * n_heads + 4 * 512 * n_heads + 4 * n_heads + 4 * 512 + 4 * 512
    return {"score": score, "attention": attn, "step": score + attn}


def measure(wl, steps, warmup, flush, dev, csa, gen, np, torch, keep_host, query_format="fp32", sess_np=None,
            n_rows=None):
    """Cold / warm / per-stage timing of `steps` decode steps of workload wl
    (or of the first n_rows rows of the given host sessions); returns the
    host sessions and the timings (with keep_host, also the filter
    diagnostics of session 0)."""
    t0 = time.time()
    if sess_np is None:
        sess_np = [gen.session(wl.cid, s=i) for i in range(wl.n_sessions)]
    sess = []
    for s in sess_np:
        d = {k: torch.from_numpy(s[k]).to(dev) for k in ("q_idx", "w_idx", "q_attn")}
        for k in ("idx_rows", "kv_rows"):
            d[k] = torch.from_numpy(s[k][:n_rows] if n_rows is not None else s[k]).to(dev)
        sess.append(d)
    scale = sess_np[0]["softmax_scale"]
    print(f"[bench] workload {wl.name}: {len(sess)} x {sess[0]['idx_rows'].shape[0]} rows ({query_format} query), "
          f"ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    step = csa.DecodeStep(sess, scale, query_format=query_format)
    stream = torch.cuda.current_stream()

    def do_flush():
        flush.sum()

    for _ in range(warmup):
        do_flush()
        step()
    torch.cuda.synchronize()

    # cold steps: events bracket the decode step only
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for e0, e1 in ev:
        do_flush()
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    cold = [e0.elapsed_time(e1) for e0, e1 in ev]

    # warm steps: back to back
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(steps):
        step()
    w1.record(stream)
    torch.cuda.synchronize()
    warm = w0.elapsed_time(w1) / steps

    # per-stage times (same work; events recorded between the stage launches
    # on the launching stream)
    nst = len(csa.STAGES)
    st_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)] for _ in range(steps)]
    for evs in st_ev:
        do_flush()
        step.timed(evs)
    torch.cuda.synchronize()
    stage_ms = [statistics.mean(evs[2 * i].elapsed_time(evs[2 * i + 1]) for evs in st_ev) for i in range(nst)]
    r = {
        "mean_ms": statistics.mean(cold),
        "median_ms": statistics.median(cold),
        "p10_ms": float(np.percentile(cold, 10)),
        "p90_ms": float(np.percentile(cold, 90)),
        "warm_ms": warm,
        "wall_ms": wall * 1e3 / steps,
        "stage_ms": stage_ms,
        "score_ms": stage_ms[0],  # the score kernel's launch
    }
    if keep_host:
        r["filter"] = filter_diagnostics(sess[0], step.sessions[0], csa, np, torch, query_format)
    del step, sess
    torch.cuda.synchronize()
    return sess_np, r


def measure_dense(n_rows, steps, flush, dev, csa, gen, np, torch):
    """Cold time of csa_dense_attn over n_rows KV rows (64 heads): the HCA
    layers' dense attention.  Rows and query from the 1M-row workload's
    generator (prefix), cold as the decode step."""
    s = gen.session(3, n_rows=n_rows)
    kv = torch.from_numpy(s["kv_rows"]).to(dev)
    q = torch.from_numpy(s["q_attn"]).to(dev)
    ws = torch.empty(int(csa.lib.csa_dense_workspace_bytes(n_rows)), dtype=torch.uint8, device=dev)
    out = torch.empty((q.shape[0], 512), dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[0], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        flush.sum()
        csa.dense_attn(kv, q, s["softmax_scale"], ws=ws, out=out, lse=lse)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in ev:
        flush.sum()
        e0.record(stream)
        csa.dense_attn(kv, q, s["softmax_scale"], ws=ws, out=out, lse=lse)
        e1.record(stream)
    torch.cuda.synchronize()
    t = [e0.elapsed_time(e1) for e0, e1 in ev]
    alg = 583 * n_rows + 4 * 512 * 64 * 2 + 4 * 64
    med = statistics.median(t)
    return {"rows": n_rows, "heads": int(q.shape[0]), "cold_median_ms": round(med, 5),
            "algorithmic_bytes": alg, "hbm_gbs": round(alg / (med * 1e-3) / 1e9, 2)}


def measure_layer_parts(steps, flush, dev, csa, gen, np, torch):
    """Cold times of the rest of a decode layer around the CSA step: the
    append of one new row (its 583-byte KV row and 68-byte indexer row), the
    dense attention over a 256-row raw sliding-window ring, and the merge of
    the two attention results."""
    s = gen.session(2, n_rows=256)
    ring = torch.from_numpy(s["kv_rows"]).to(dev)
    q = torch.from_numpy(s["q_attn"]).to(dev)
    g = torch.Generator().manual_seed(7)
    kv_new = torch.randn((1, 512), generator=g).to(dev)
    idx_new = torch.randn((1, 128), generator=g).to(dev)
    kv_slot = torch.empty((1, 583), dtype=torch.uint8, device=dev)
    idx_slot = torch.empty((1, 68), dtype=torch.uint8, device=dev)
    ws = torch.empty(int(csa.lib.csa_dense_workspace_bytes(256)), dtype=torch.uint8, device=dev)
    o_r = torch.empty((64, 512), dtype=torch.float32, device=dev)
    l_r = torch.empty(64, dtype=torch.float32, device=dev)
    o_c, l_c = torch.randn((64, 512), device=dev), torch.randn(64, device=dev)
    stream = torch.cuda.current_stream()
    parts = {
        "append_one_row_us": lambda: csa.pack_rows(kv_new, idx_new, kv_rows=kv_slot, idx_rows=idx_slot),
        "ring_attention_256_rows_us": lambda: csa.dense_attn(ring, q, s["softmax_scale"], ws=ws, out=o_r, lse=l_r),
        "lse_merge_us": lambda: csa.lse_merge(o_c, l_c, o_r, l_r),
    }
    res = {}
    for name, fn in parts.items():
        for _ in range(3):
            fn()
        t = []
        for _ in range(steps):
            flush.sum()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            t.append(e0.elapsed_time(e1) * 1e3)
        res[name] = round(statistics.median(t), 2)
    return res


def measure_multi_token(n_tokens, steps, flush, dev, csa, gen, np, torch):
    """Cold time of csa_score_topk_multi: n_tokens queries over the 1M-row
    history, each with its exact top-512."""
    s = gen.session(3)
    rows = torch.from_numpy(s["idx_rows"]).to(dev)
    g = torch.Generator().manual_seed(11)
    q = torch.randn((n_tokens, 64, 128), generator=g).to(dev)
    w = torch.rand((n_tokens, 64), generator=g).to(dev)
    ws = csa.alloc_workspace(rows.shape[0], n_tokens, dev)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        flush.sum()
        csa.score_topk_multi(rows, q, w, ws=ws)
    t = []
    for _ in range(steps):
        flush.sum()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        csa.score_topk_multi(rows, q, w, ws=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        t.append(e0.elapsed_time(e1))
    med = statistics.median(t)
    return {"tokens": n_tokens, "rows": int(rows.shape[0]), "cold_median_ms": round(med, 5),
            "ms_per_token": round(med / n_tokens, 5),
            "indexer_gbs_once": round(68 * rows.shape[0] / (med * 1e-3) / 1e9, 1)}


def filter_diagnostics(d, outs, csa, np, torch, query_format):
    """How much the matrix-core filter leaves to the exact rescoring, on
    session 0 (outside the timed steps, library calls only): the brackets'
    relative half-widths, the band (rows whose upper bound reaches the exact
    512th score: the fewest rows any exact rescoring must visit) and the
    largest relative error of the step's selected scores against csa_score's
    exact scores of the same rows."""
    q = d["q_idx"]
    if query_format == "mxfp4":
        q = csa.dequant_idx(csa.quantize_query(q))
    up, lo = csa.score_bounds(d["idx_rows"], d["q_idx"], d["w_idx"], query_format=query_format)
    exact = csa.score(d["idx_rows"], q, d["w_idx"])
    torch.cuda.synchronize()
    up, lo, ex = up.cpu().numpy().astype(np.float64), lo.cpu().numpy().astype(np.float64), exact.cpu().numpy()
    k_eff = min(512, ex.shape[0])
    sel = outs["sel"].cpu().numpy()[:k_eff]
    sel_score = outs["sel_score"].cpu().numpy()[:k_eff].astype(np.float64)
    fin = np.isfinite(up) & np.isfinite(lo) & (ex != 0)
    half = (up - lo)[fin] / 2.0 / np.abs(ex[fin].astype(np.float64))
    T = float(np.sort(ex)[::-1][k_eff - 1]) if k_eff else float("inf")
    ref = ex[sel].astype(np.float64)
    err = np.abs(sel_score - ref) / np.maximum(np.abs(ref), 1e-30) if k_eff else np.zeros(1)
    return {
        "rows": int(ex.shape[0]),
        "median_rel_bracket_halfwidth": float(np.median(half)) if half.size else 0.0,
        "max_rel_bracket_halfwidth": float(np.max(half)) if half.size else 0.0,
        "band_rows": int(np.sum(up >= T)),
        "sel_score_max_rel_err": float(np.max(err)),
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {a.gpus} is not supported "
              "(the row-sharded multi-GPU plan is described, not built)", file=sys.stderr)
        sys.exit(2)

    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return

    if a.steps_only:
        a.no_fit = a.no_sweep = a.no_cpu_baseline = True

    import numpy as np
    import torch

    import gen
    import long_context_sparse_score_amd as csa

    workloads = {w.name: w for w in gen.WORKLOADS}
    wl = workloads[a.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB: evicts the MALL and the L2s

    sess_np, r = measure(wl, a.steps, a.warmup, flush, dev, csa, gen, np, torch, keep_host=not a.steps_only,
                         query_format=a.query_format)
    r_q4 = None
    if not a.steps_only:  # the MXFP4-quantized-query scorer on the same data
        _, r_q4 = measure(wl, a.sweep_steps, 2, flush, dev, csa, gen, np, torch, keep_host=True, query_format="mxfp4",
                          sess_np=sess_np)
    scale = sess_np[0]["softmax_scale"]
    ab = algorithmic_bytes(wl.n_rows, wl.n_idx_heads, wl.n_heads)
    ms = r["mean_ms"]
    step_bytes = ab["step"] * wl.n_sessions
    score_gbs = ab["score"] * wl.n_sessions / (r["score_ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(ms, 5),
        "unit": "ms",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) rows packed to MXFP4 / E4M3+FP16+UE8M0)",
        "config": {
            "workload": wl.name,
            "rows_per_session": wl.n_rows,
            "sessions": wl.n_sessions,
            "indexer_heads": wl.n_idx_heads,
            "attention_heads": wl.n_heads,
            "topk": 512,
            "indexer_query": a.query_format,
            "cache": "cold: MALL and L2 flushed before each step, outside its events",
        },
        "median_ms": round(r["median_ms"], 5),
        "p10_ms": round(r["p10_ms"], 5),
        "p90_ms": round(r["p90_ms"], 5),
        "warm_ms_per_step": round(r["warm_ms"], 5),
        "wall_ms_per_step_incl_flush": round(r["wall_ms"], 5),
        "step_algorithmic_bytes": step_bytes,
        "step_hbm_gbs": round(step_bytes / (ms * 1e-3) / 1e9, 2),
        "stage_ms": {name: round(t, 5) for name, t in zip(csa.STAGES, r["stage_ms"])},
        "roofline": {
            "kernel": "tile_kernel: query split + score + tile heads (all sessions, one launch)",
            "bound": "hbm",
            "achieved": round(score_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(score_gbs / HBM_PEAK_GBS, 5),
            "traffic": measured_traffic(wl.name),
            "launch_ms": round(r["score_ms"], 5),
            "algorithmic_bytes_per_launch": ab["score"] * wl.n_sessions,
        },
    }

    if "filter" in r:
        line["filter"] = r["filter"]
    if not a.steps_only:  # dense attention of a ratio-128 (HCA) layer at a 1M-token context
        line["dense_attention"] = measure_dense(8194, a.sweep_steps, flush, dev, csa, gen, np, torch)
        line["layer_parts"] = measure_layer_parts(a.sweep_steps, flush, dev, csa, gen, np, torch)
        line["multi_token_topk"] = [measure_multi_token(t, a.sweep_steps, flush, dev, csa, gen, np, torch) for t in (1, 4)]
    if r_q4 is not None:
        line["mxfp4_query"] = {
            "cold_median_ms": round(r_q4["median_ms"], 5),
            "warm_ms": round(r_q4["warm_ms"], 5),
            "stage_ms": {name: round(t, 5) for name, t in zip(csa.STAGES, r_q4["stage_ms"])},
            "score_kernel_hbm_frac": round(ab["score"] * wl.n_sessions / (r_q4["score_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
            "filter": r_q4["filter"],
        }
    if not a.no_fit and wl.n_sessions == 1:
        # fixed + marginal cost: cold step time over history prefixes of
        # 2^11 .. 2^20 rows of the same session, least squares ms = a + b MB
        pts = []
        for lg in range(11, 21):
            n = 1 << lg
            if n > wl.n_rows:
                break
            _, rf = measure(wl, a.sweep_steps, 2, flush, dev, csa, gen, np, torch, keep_host=False,
                            sess_np=sess_np[:1], n_rows=n)
            mb = algorithmic_bytes(n, wl.n_idx_heads, wl.n_heads)["step"] / 1e6
            pts.append((n, mb, rf["median_ms"]))
        x = np.array([p[1] for p in pts])
        y = np.array([p[2] for p in pts])
        b, a0 = np.polyfit(x, y, 1)
        line["cost_fit"] = {
            "model": "cold step ms = fixed_ms + ms_per_mb * algorithmic MB",
            "fixed_ms": round(float(a0), 5),
            "ms_per_mb": round(float(b), 7),
            "marginal_gbs": round(1.0 / float(b), 1) if b > 0 else None,  # MB per ms = GB/s
            "points": [{"rows": n, "mb": round(mb, 3), "ms": round(ms, 5)} for n, mb, ms in pts],
        }

    if not a.no_sweep:
        # every history length of the workload set: cold step latency, the
        # score kernel's HBM fraction and the whole step's algorithmic GB/s
        by = {}
        for w in gen.WORKLOADS:
            if w.name == wl.name:
                rw = r
            else:
                _, rw = measure(w, a.sweep_steps, 2, flush, dev, csa, gen, np, torch, keep_host=False)
            abw = algorithmic_bytes(w.n_rows, w.n_idx_heads, w.n_heads)
            sg = abw["score"] * w.n_sessions / (rw["score_ms"] * 1e-3) / 1e9
            by[w.name] = {
                "rows_per_session": w.n_rows,
                "sessions": w.n_sessions,
                "cold_median_ms": round(rw["median_ms"], 5),
                "warm_ms": round(rw["warm_ms"], 5),
                "step_hbm_gbs": round(abw["step"] * w.n_sessions / (rw["median_ms"] * 1e-3) / 1e9, 2),
                "stage_ms": {name: round(t, 5) for name, t in zip(csa.STAGES, rw["stage_ms"])},
                "score_kernel_ms": round(rw["score_ms"], 5),
                "score_kernel_hbm_frac": round(sg / HBM_PEAK_GBS, 5),
            }
            print(f"[bench] {w.name}: {by[w.name]}", file=sys.stderr, flush=True)
        line["by_workload"] = by

    if not a.no_cpu_baseline:
        import oracle

        s0 = sess_np[0]
        n = a.cpu_sample_rows or wl.n_rows
        o = oracle.get()
        reps, dt = 0, 0.0
        while dt < a.cpu_seconds and reps < 20:
            t = time.perf_counter()
            o.decode_step(s0["idx_rows"][:n], s0["kv_rows"][:n], s0["q_idx"], s0["w_idx"], s0["q_attn"], scale)
            dt += time.perf_counter() - t
            reps += 1
        per_session_ms = dt / reps * 1e3 * (wl.n_rows / n)
        line["cpu_baseline"] = {
            "value": round(per_session_ms * wl.n_sessions, 3),
            "unit": "ms",
            "cores": 1,
            "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(),
            "kind": "oracle",
            "sample": f"{reps} decode steps of session 0 over its first {n} rows "
                      f"({dt:.2f} s measured), mean scaled by rows x sessions to the whole workload",
        }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
