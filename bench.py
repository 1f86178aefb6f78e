"""Benchmark of one DSA decode step (indexer -> top-k -> sparse MLA) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--extra-workloads A,B]

A step is one pass of the whole hot path over one batch: dsa_indexer_logits,
dsa_topk and sparse_mla_decode (with its split-KV combine) on one stream. The
inputs are generated on the host, copied to HBM before timing, and stay
resident. Prints one JSON line:

* value: decode tokens/s = rows per step / step time (one token per request);
* sparse_attn_hbm_gbps: algorithmic sparse-attention bytes / attention time;
* roofline: the dominant kernel's algorithmic bytes (or FLOPs, when its FLOP
  per byte is above the MFMA ridge) per launch over its average launch time,
  against the MI355X peak;
* extra: the same step on further workloads (by default the batch-64 decode
  with every context at 32,768 keys, the literal "ctx 32k" of the metric, and
  the ragged batch with the fused indexer + top-k call);
* cpu_baseline: the float64 oracle timed on a bounded sample of the same
  workload on this host's cores.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s + sparse-attn HBM GB/s, 1 GPU, ctx 32k, top-k 2048"
HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def visible_lengths(seq_lens_k, cu_seqlens_q):
    """Keys each query row sees: a decode row its whole request; the j-th of a
    request's q_len rows seq_len - q_len + j + 1 (bottom-right causal)."""
    lens = np.asarray(seq_lens_k, dtype=np.int64)
    if cu_seqlens_q is None:
        return np.maximum(lens, 0), np.arange(len(lens))
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    q_lens = np.diff(cu)
    seq = np.repeat(np.arange(len(lens)), q_lens)
    j = np.arange(int(cu[-1])) - np.repeat(cu[:-1], q_lens)
    vis = lens[seq] - q_lens[seq] + j + 1
    return np.maximum(vis, 0), seq


def _bound(flops, nbytes, mfma_peak_tflops):
    """The roofline a stage sits under: MFMA when its FLOP per byte is above
    the ridge of its MFMA dtype, HBM otherwise."""
    ridge = mfma_peak_tflops * 1e12 / (HBM_PEAK_GBPS * 1e9)
    return "mfma" if flops and flops / max(nbytes, 1) > ridge else "hbm"


def algorithmic_work(wl):
    """Bytes and FLOPs each stage must move or compute at minimum (per step).

    * indexer: every index key a request's rows see is read once per request
      (its rows share the read), 132 B per key for fp8 x 128 + fp32 scale;
      each row reads its q and gates and writes 4 B per visible logit;
      2 H D FLOP per (row, visible key).
    * top-k: each row reads its visible logits (4 B each) and writes k indices.
    * indexer + top-k fused: the indexer's reads and the top-k's writes.
    * sparse MLA: each selected row is gathered once per query row that
      selects it (1,152 B for bf16 576-wide rows); decode rows of different
      requests share nothing, so this is HBM traffic. Rows of one request
      (prefill, multi-token decode) select overlapping sets out of at most
      seq_len cached rows, so HBM traffic is counted as the distinct rows
      (at most seq_len per request) and the per-row gather is reported
      separately as cache-served traffic. Plus q, out, indices and lse.
      FLOPs: Hm (2 (Dl + Dr) + 2 Dl) per selected (row, head-independent entry).
    """
    cfg = wl.cfg
    vis, seq = visible_lengths(wl.seq_lens_k, wl.cu_seqlens_q)
    T = len(vis)
    H, D, k = cfg.idx_heads, cfg.idx_dim, cfg.topk
    esize = 1 if cfg.idx_kind == "fp8" else 4
    key_bytes = D * esize + 4                       # 132 B for fp8 x 128 + fp32 scale
    per_req_keys = np.zeros(len(wl.seq_lens_k), dtype=np.int64)
    np.maximum.at(per_req_keys, seq, vis)
    idx_bytes = (int(per_req_keys.sum()) * key_bytes + int(vis.sum()) * 4
                 + T * (H * D * esize + 4 * H))
    idx_flops = int(vis.sum()) * 2 * H * D
    topk_bytes = int(vis.sum()) * 4 + T * 4 * k
    fused_bytes = idx_bytes - int(vis.sum()) * 4 + T * 4 * k
    sel = np.minimum(vis, k)
    Hm, Dl, Dr = cfg.mla_heads, cfg.d_latent, cfg.d_rope
    msize = {"bf16": 2, "fp8": 1}.get(cfg.mla_kind, 4)          # cached row and query element
    osize = 4 if cfg.mla_kind == "f32" else 2                    # output element (bf16 for fp8 too)
    row_bytes = (Dl + Dr) * msize
    per_row_io = Hm * (Dl + Dr) * msize + Hm * Dl * osize + 4 * k + 4 * Hm
    gathered = int(sel.sum()) * row_bytes
    if wl.cu_seqlens_q is None:
        distinct = int(sel.sum())
    else:
        per_req_sel = np.zeros(len(wl.seq_lens_k), dtype=np.int64)
        np.add.at(per_req_sel, seq, sel)
        distinct = int(np.minimum(per_req_sel, np.asarray(wl.seq_lens_k, dtype=np.int64)).sum())
    mla_bytes = distinct * row_bytes + T * per_row_io
    mla_flops = int(sel.sum()) * Hm * (2 * (Dl + Dr) + 2 * Dl)
    idx_peak = FP8_PEAK_TFLOPS if cfg.idx_kind == "fp8" else FP32_PEAK_TFLOPS
    mla_peak = {"bf16": BF16_PEAK_TFLOPS, "fp8": FP8_PEAK_TFLOPS}.get(cfg.mla_kind, FP32_PEAK_TFLOPS)
    return {
        "indexer": {"bytes": idx_bytes, "flops": idx_flops, "peak_tflops": idx_peak,
                    "bound": _bound(idx_flops, idx_bytes, idx_peak),
                    "per_unit": f"{key_bytes} B per key of a request (read once for its rows) + 4 B per "
                                f"(row, visible key) logit + {H * D * esize + 4 * H} B per row; "
                                f"{2 * H * D} FLOP per (row, visible key)",
                    "units": int(vis.sum())},
        "topk": {"bytes": topk_bytes, "flops": 0, "peak_tflops": None, "bound": "hbm",
                 "per_unit": f"4 B per visible score (+{4 * k} B per row)", "units": int(vis.sum())},
        # the fused call reads the keys, q and gates and writes the lists: no logits
        "indexer_topk": {"bytes": fused_bytes, "flops": idx_flops, "peak_tflops": idx_peak,
                         "bound": _bound(idx_flops, fused_bytes, idx_peak),
                         "per_unit": f"{key_bytes} B per key of a request (read once for its rows) + "
                                     f"{H * D * esize + 4 * H + 4 * k} B per row; {2 * H * D} FLOP per "
                                     f"(row, visible key)",
                         "units": int(vis.sum())},
        "sparse_mla": {"bytes": mla_bytes, "flops": mla_flops, "peak_tflops": mla_peak,
                       "bound": _bound(mla_flops, mla_bytes, mla_peak),
                       "gather_bytes": gathered + T * per_row_io,
                       "per_unit": f"{row_bytes} B per distinct selected cache row (+{per_row_io} B per "
                                   f"query row); {Hm * (2 * (Dl + Dr) + 2 * Dl)} FLOP per selected entry",
                       "units": int(sel.sum())},
    }


def time_input_side(wl, K, stream):
    """Average launch time of the indexer's input side for this batch, outside
    the step: dsa_quant_index_q on every query row (bf16 [T, H, 128] in) and
    dsa_store_index_k of one new key per query row, each key on its own page
    (a scratch cache, so the step's cache keeps its keys)."""
    import torch
    import sparse_mla_attention_dsa_amd as dsa
    cfg = wl.cfg
    if cfg.idx_kind != "fp8":
        return None
    T, H, D, P = wl.num_rows, cfg.idx_heads, cfg.idx_dim, cfg.page_size
    gen = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn((T, H, D), generator=gen, device="cuda").to(torch.bfloat16)
    w = torch.randn((T, H), generator=gen, device="cuda") / 8.0
    q8 = torch.empty((T, H, D), dtype=torch.uint8, device="cuda")
    w_eff = torch.empty((T, H), dtype=torch.float32, device="cuda")
    key = torch.randn((T, D), generator=gen, device="cuda").to(torch.bfloat16)
    cache = torch.zeros((T, (D + 4) * P), dtype=torch.uint8, device="cuda")
    slots = (torch.arange(T, device="cuda", dtype=torch.int64) * P
             + torch.randint(0, P, (T,), generator=gen, device="cuda"))
    out = {}
    for name, fn, nbytes in (
            ("quant_index_q", lambda: dsa.dsa_quant_index_q(q, w, q8, w_eff), T * H * (2 * D + 4 + D + 4)),
            ("store_index_k", lambda: dsa.dsa_store_index_k(key, slots, cache, P), T * (2 * D + 8 + D + 4))):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(20_000_000)                    # the host queues the launches meanwhile
        except Exception:
            pass
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / K
        out[name] = {"us": us, "algorithmic_bytes": nbytes, "hbm_gbps": nbytes / (us * 1e-6) / 1e9}
    return out


def cpu_baseline(wl, budget_s=12.0, max_rows=4096):
    """Oracle (float64 numpy) on whole rows of the workload until ~budget_s of CPU work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    cfg = wl.cfg
    vis = [r.visible for r in oracle.row_layout(wl.seq_lens_k, wl.cu_seqlens_q)]
    t0 = time.perf_counter()
    done = 0
    order = [t % wl.num_rows for t in range(max_rows)]
    for t in order:
        logits = oracle.indexer_logits(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                                       wl.cu_seqlens_q, cfg.page_size, cfg.idx_kind, rows=[t])[t]
        idx = oracle.topk_row(logits, vis[t], cfg.topk)
        full_idx = np.full((wl.num_rows, cfg.topk), -1, dtype=np.int64)
        full_idx[t] = idx
        oracle.sparse_mla(wl.q_mla, wl.latent, full_idx, wl.block_table, wl.seq_lens_k, wl.cu_seqlens_q,
                          cfg.page_size, cfg.d_latent, cfg.softmax_scale, cfg.mla_kind, rows=[t])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} decode rows (rows 0.. of the {wl.num_rows}-row batch, cycling), all three "
                      f"stages per row (float64 numpy), {el:.1f} s",
            "cpu_model": _cpu_model(), "blas": _blas_vendor(),
            "host_cores_available": len(os.sched_getaffinity(0))}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _blas_vendor():
    """numpy's BLAS library as threadpoolctl reports it (name, version, threads)."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
    except Exception:
        pass
    return None


def copy_calibration(mib):
    """A plain copy of a known size: 2 * mib MiB of algorithmic HBM traffic
    (mib read + mib written), to scale the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n}))


def measure(cfg, K, W, graph=True, with_input_side=True, fused=False):
    """Generate `cfg`, run W eager warm-up steps, time K steps, time the stages.

    The K timed steps are one HIP graph (captured once, replayed once), as a
    serving loop would run them: host launch overhead is not part of the step.
    The per-stage times come from a second pass of K eager steps with events
    recorded on the stream between the stages; a GPU spin queued in front lets
    the host enqueue the whole pass first, so the kernels run back to back
    (same order, same data, same cache state) and each event pair brackets one
    stage's kernels."""
    import torch

    from dsa_workloads import generate
    from dsa_workloads.device import make_step

    t_gen = time.perf_counter()
    wl = generate(cfg)
    print(f"[bench] generated {cfg.name} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    step = make_step(wl, device="cuda:0", fused=fused)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    for _ in range(W):
        step.run()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: warmup done ({W} steps)", file=sys.stderr, flush=True)

    if fused:
        stages = (("indexer_topk", step.index_select), ("sparse_mla", step.attend))
    else:
        stages = (("indexer", step.indexer), ("topk", step.select), ("sparse_mla", step.attend))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if not graph:
        run_all = lambda: [step.run() for _ in range(K)]
    else:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step.run()                                       # warm the capture stream
        stream.wait_stream(side)
        torch.cuda.synchronize()
        g_all = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_all):
            for _ in range(K):
                step.run()
        g_all.replay()                                       # untimed replay
        torch.cuda.synchronize()
        run_all = g_all.replay
    torch.cuda.synchronize()
    start.record(stream)
    run_all()
    end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / K

    try:
        torch.cuda._sleep(40_000_000)                        # ~20 ms of GPU spin
    except Exception:
        pass
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        for j, (_, fn) in enumerate(stages):
            fn()
            ev[i][j + 1].record(stream)
    torch.cuda.synchronize()
    stage_ms = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in ev]))
                for j, (name, _) in enumerate(stages)}
    # per-step spread of the eager pass (each step bracketed by its own events)
    eager_us = np.array([e[0].elapsed_time(e[-1]) * 1e3 for e in ev])
    eager = {"p10_us": float(np.percentile(eager_us, 10)), "median_us": float(np.median(eager_us)),
             "p90_us": float(np.percentile(eager_us, 90)), "steps": int(K)}
    print(f"[bench] {cfg.name}: timed {K} steps: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    input_side = time_input_side(wl, K, stream) if with_input_side else None

    work = algorithmic_work(wl)
    kernels = {}
    for name in stage_ms:
        w = work[name]
        t_s = stage_ms[name] * 1e-3
        gbps = w["bytes"] / t_s / 1e9
        kernels[name] = {
            "us": stage_ms[name] * 1e3,
            "bound": w["bound"],
            "algorithmic_bytes": w["bytes"],
            "algorithmic_flops": w["flops"],
            "hbm_gbps": gbps,
            "hbm_frac": gbps / HBM_PEAK_GBPS,
            "per_unit": w["per_unit"],
            "units": w["units"],
        }
        if "gather_bytes" in w and w["gather_bytes"] != w["bytes"]:
            kernels[name]["gather_bytes"] = w["gather_bytes"]
            kernels[name]["gather_gbps"] = w["gather_bytes"] / t_s / 1e9
        if w["flops"]:
            kernels[name]["tflops"] = w["flops"] / t_s / 1e12
            kernels[name]["mfma_peak_tflops"] = w["peak_tflops"]
            kernels[name]["mfma_frac"] = kernels[name]["tflops"] / w["peak_tflops"]
    dominant = max(stage_ms, key=stage_ms.get)
    dk = kernels[dominant]
    traffic = None
    prof = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(prof):
        try:
            from sparse_mla_attention_dsa_amd.build import source_digest
            rec = json.load(open(prof)).get(f"{cfg.name}:{dominant}")
            if rec and rec.get("source_digest") == source_digest():
                traffic = rec["bytes_per_launch"]
        except Exception:
            traffic = None
    if dk["bound"] == "mfma":
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": dk["tflops"], "peak": dk["mfma_peak_tflops"],
                    "unit": "TFLOP/s", "frac": dk["mfma_frac"], "traffic": traffic}
    else:
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": dk["hbm_gbps"], "peak": HBM_PEAK_GBPS,
                    "unit": "GB/s", "frac": dk["hbm_frac"], "traffic": traffic}
    return wl, {
        "tokens_per_s": wl.num_rows / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "stages": kernels,
        "input_side": input_side,
        "roofline": roofline,
        "eager_step": eager,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode_b64_ragged")
    ap.add_argument("--extra-workloads", default="decode_b64_32k,decode_b64_ragged:fused",
                    help="comma-separated workloads also timed and reported under `extra` ('' for none); "
                         "NAME:fused or NAME:two-call picks the selection path")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="launch the timed steps eagerly")
    ap.add_argument("--fused", action="store_true",
                    help="indexer and top-k as one call (dsa_indexer_topk, no logits in memory)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB mebibytes (counter calibration)")
    args = ap.parse_args()

    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the DSA step is not "
              "sharded across GPUs in this library", file=sys.stderr)
        sys.exit(2)

    import torch

    from dsa_workloads import CONFIGS

    cfg = CONFIGS[args.workload]
    wl, m = measure(cfg, args.steps, args.warmup, graph=not args.no_graph, fused=args.fused)
    result = {
        "metric": METRIC,
        "value": m["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.mla_kind != "fp8" else "fp8+bf16",
        "dtype_detail": ("indexer fp8 e4m3 MFMA with fp32 accumulate; attention bf16 MFMA with fp32 softmax"
                         if cfg.mla_kind != "fp8" else
                         "indexer fp8 e4m3 MFMA; attention scores fp8 e4m3 MFMA, P.V bf16 MFMA (cache codes "
                         "converted exactly), fp32 accumulate and softmax"),
        "data": "synthetic",
        "launch": "eager" if args.no_graph else "hip graph of the timed steps",
        "selection": ("dsa_indexer_topk (fused, no logits in memory)" if args.fused
                      else "dsa_indexer_logits + dsa_topk"),
        "config": {"workload": cfg.name, "description": cfg.note, "batch": cfg.batch,
                   "ctx_total": int(wl.seq_lens_k.sum()), "ctx_max": wl.max_seq_len_k, "topk": cfg.topk,
                   "page_size": cfg.page_size, "indexer": f"{cfg.idx_heads}x{cfg.idx_dim} {cfg.idx_kind}",
                   "mla": f"{cfg.mla_heads} heads x {cfg.d_latent}+{cfg.d_rope} {cfg.mla_kind}"},
        "sparse_attn_hbm_gbps": m["stages"]["sparse_mla"]["hbm_gbps"],
        "eager_step_us": m["eager_step"],
        "stages": m["stages"],
        "input_side": m["input_side"],
        "roofline": m["roofline"],
    }
    extra = {}
    for spec in [x for x in args.extra_workloads.split(",") if x]:
        # NAME, or NAME:fused / NAME:two-call to choose the selection path
        name, _, path = spec.partition(":")
        fused_x = args.fused if not path else path == "fused"
        if name == cfg.name and fused_x == args.fused:
            continue
        del wl
        torch.cuda.empty_cache()
        wl_x, mx = measure(CONFIGS[name], args.steps, args.warmup, graph=not args.no_graph,
                           with_input_side=False, fused=fused_x)
        extra[spec] = {"tokens_per_s": mx["tokens_per_s"], "ms_per_step": mx["ms_per_step"],
                       "selection": "dsa_indexer_topk" if fused_x else "dsa_indexer_logits + dsa_topk",
                       "description": CONFIGS[name].note, "ctx_total": int(wl_x.seq_lens_k.sum()),
                       "sparse_attn_hbm_gbps": mx["stages"]["sparse_mla"]["hbm_gbps"],
                       "stages": {k: {kk: v[kk] for kk in ("us", "bound", "hbm_frac", "mfma_frac") if kk in v}
                                  for k, v in mx["stages"].items()},
                       "roofline": mx["roofline"]}
        wl = wl_x
    if extra:
        result["extra"] = extra
    if not args.no_cpu_baseline:
        from dsa_workloads import generate
        print("[bench] timing the oracle on a sample", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(generate(cfg), budget_s=args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result))


if __name__ == "__main__":
    main()
