"""Benchmark: verified tree tokens/s of one speculative-decoding verification step.

A step is the whole hot path over one batch: tree_build -> tree_attention ->
tree_verify_greedy, on one GPU, inputs resident in HBM.  Default workload: long
ragged prefixes on a paged cache (batch 32, 64 query / 8 KV heads, head dim 128,
bf16, prefix lengths uniform in 8192..32768 tokens in 16-token blocks behind a
shuffled block table, 32-node random trees of depth <= 6, no vocabulary), the
largest single-GPU attention workload and the one the HBM-roofline goal is set
on.  Without a vocabulary the step is tree_build -> tree_attention.

Each timed step uses the next of R input copies (R chosen so the copies exceed
twice the 256 MB last-level cache), the way consecutive layers each bring their
own KV cache: a step never finds its inputs already cached.

tree_commit_kv (writing the accepted path's K/V into the cache),
tree_verify_stochastic (multi-step speculative sampling, the alternative to the
greedy walk) and the construction calls (tree_expand_topk, tree_merge_drafts)
are not part of the timed step; their own kernel times are reported
under kernel_us.  The commit writes the path verification accepted (or, on
workloads without a vocabulary, the root path to each tree's deepest node) into
cache room left after each prefix; stochastic verification runs on SSM logits
and uniforms generated for the same logits.  Kernels far shorter than a host
launch (all but tree_attention) are timed as K launches captured in one HIP
graph, so the figure is GPU time rather than the host's launch rate.

Prints ONE JSON line.  `value` = B*n / (wall time per step).  `roofline` covers
the dominant kernel (tree_attention) measured with HIP events on the launch
stream (the mean over K back-to-back launches; tree_attention_us_per_launch
adds the p10 / median / p90 of single launches, one event between each); `traffic` is read from the committed rocprofv3 counter summary when it
was taken on the current kernel source, else null.  `cpu_baseline` times the
CPU oracle on the same workload.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--config 4]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-attn HBM GB/s & MFMA util (% peak); verified tree tokens/sec at 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
MALL_BYTES = 256 << 20


def kernel_source_hash() -> str:
    """Hash of everything that decides what tree_attention launches: the attention
    kernels, the host plan and dispatch (capi.hip), and the compiler flags."""
    from token_tree_verification_02_amd import build as _build
    h = hashlib.sha256()
    for f in ("attn_bf16.hip", "attn_sk.hip", "attn_bf16_common.h", "attn_f32.hip", "tv_internal.h", "capi.hip"):
        with open(os.path.join(ROOT, "token_tree_verification_02_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(_build.FLAGS[1:]).replace(_build.ROOT, "").encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    path = os.path.join(ROOT, "profiles", f"tree_attention_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t


def cpu_baseline(w, budget_s: float):
    """The oracle (as it stands) on the whole batch, repeated until the budget is used."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    cfg = w["cfg"]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.tree_build(w["parent"], w["depth"], w["prefix_len"])
        oracle.tree_attention(w)
        if cfg.vocab:
            oracle.verify_greedy(w["logits"], w["tokens"], w["parent"], cfg.dtype)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": reps * cfg.B * cfg.n / el, "unit": "verified tree tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{reps} full pass(es) of the {cfg.name} batch (B={cfg.B}, n={cfg.n}), float64 NumPy, "
                      f"{el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--dtype", choices=["bf16", "f16"], default=None,
                    help="element type of q/K/V/out/logits (default: the workload's)")
    ap.add_argument("--kv", choices=["fp8"], default=None, help="store the prefix KV cache as fp8 (E4M3) codes")
    ap.add_argument("--copies", type=int, default=0, help="input copies to rotate (0 = auto)")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true", help="launch each step eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU form (each sequence and each KV head "
              "is independent; see the sharding notes in the design document)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}))
        return

    from token_tree_verification_02_amd import runner
    from token_tree_verification_02_amd import workloads as W

    over = {"dtype": args.dtype} if args.dtype else {}
    if args.kv:
        over["kv"] = args.kv
    cfg = W.config(args.config, **over)
    t_gen = time.perf_counter()
    w = W.make(cfg, room=cfg.n)
    # stochastic verification and top-k expansion take bf16 or fp32 logits
    ws = W.make_stochastic(cfg, w=w) if cfg.vocab and cfg.dtype != "f16" else None
    t_gen = time.perf_counter() - t_gen
    refb = W.reference_bytes(w)
    per_copy = refb["attn_bytes"] + refb["verify_bytes"]
    R = args.copies or max(1, math.ceil(2 * MALL_BYTES / per_copy))
    copies = [runner.upload(w) for _ in range(R)]
    steps = [runner.Step(d) for d in copies]
    if cfg.vocab:
        cargs = [st.commit_args(d["path"], d["path_len"]) for st, d in zip(steps, copies)]
    else:
        deep = np.argmax(w["depth"], axis=1)
        hp = np.full((cfg.B, cfg.n), -1, np.int32)
        hl = np.zeros(cfg.B, np.int32)
        for b in range(cfg.B):
            chain = [int(deep[b])]
            while chain[-1] != 0:
                chain.append(int(w["parent"][b][chain[-1]]))
            hp[b, :len(chain)] = chain[::-1]
            hl[b] = len(chain)
        dev_path = [(torch.from_numpy(hp).cuda(), torch.from_numpy(hl).cuda()) for _ in copies]
        cargs = [st.commit_args(p, l) for st, (p, l) in zip(steps, dev_path)]
    mss = None
    if ws is not None:
        from token_tree_verification_02_amd import _lib
        mss = [dict(ssm=runner._t(ws["ssm_logits"], "cuda", dtype=cfg.dtype), tok=runner._t(ws["tokens"], "cuda"),
                    ua=runner._t(ws["u_accept"], "cuda"), us=runner._t(ws["u_sample"], "cuda"),
                    path=torch.empty((cfg.B, cfg.n), dtype=torch.int32, device="cuda"),
                    plen=torch.empty(cfg.B, dtype=torch.int32, device="cuda"),
                    bonus=torch.empty(cfg.B, dtype=torch.int32, device="cuda"),
                    status=torch.empty(cfg.B, dtype=torch.int32, device="cuda"),
                    ws=torch.empty(_lib.stochastic_workspace_size(cfg.B, cfg.n, cfg.vocab), dtype=torch.uint8,
                                   device="cuda")) for _ in range(R)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    # per-kernel durations: HIP events on the launch stream around K back-to-back
    # launches of one call (rotating over the input copies), so the figure is the
    # kernel's own average duration, not the dispatch latency around one call
    K = args.steps
    for i in range(max(args.warmup, R)):
        steps[i % R]()
    torch.cuda.synchronize()

    def timed(fn):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(K):
            fn(k % R, sh)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / K

    def timed_graph(fn):
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fn(0, side.cuda_stream)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for k in range(K):
                fn(k % R, cs)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / K

    def timed_each(fn):
        """Per-launch durations: an event between consecutive launches (p10, median, p90 in us)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        ev[0].record(stream)
        for k in range(K):
            fn(k % R, sh)
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        d = np.array([ev[k].elapsed_time(ev[k + 1]) * 1e3 for k in range(K)])
        return {"p10": round(float(np.percentile(d, 10)), 2), "median": round(float(np.median(d)), 2),
                "p90": round(float(np.percentile(d, 90)), 2), "launches": K}

    t_build = timed_graph(lambda i, h: steps[i].build(h))
    t_attn = timed(lambda i, h: steps[i].attention(h))
    attn_dist = timed_each(lambda i, h: steps[i].attention(h))
    t_ver = timed_graph(lambda i, h: steps[i].verify(h)) if cfg.vocab else 0.0
    steps[0].verify(sh)
    torch.cuda.synchronize()
    committed = int(copies[0]["path_len"].sum().item()) if cfg.vocab else int(hl.sum())
    t_commit = None
    if cfg.kv != "fp8":  # committing into an fp8 cache is not supported
        t_commit = timed_graph(lambda i, h: steps[i].commit(cargs[i], h))
        torch.cuda.synchronize()
        if not (copies[0]["commit_status"] == 0).all().item():
            raise RuntimeError("tree_commit_kv rejected a sequence of the benchmark batch")
    mss_out = None
    if mss is not None:
        def mss_call(i, h):
            m, d = mss[i], copies[i]
            _lib.tree_verify_stochastic(d["logits"], m["ssm"], m["tok"], d["parent"], m["ua"], m["us"],
                                        path=m["path"], path_len=m["plen"], bonus=m["bonus"], status=m["status"],
                                        workspace=m["ws"], stream=torch.cuda.ExternalStream(h))
        t_mss = timed_graph(mss_call)
        m0 = mss[0]
        if not (m0["status"] == 0).all().item():
            raise RuntimeError("tree_verify_stochastic rejected a sequence of the benchmark batch")
        plen_h = m0["plen"].cpu().numpy()
        path_h = m0["path"].cpu().numpy()
        # rows the walk has to read: each visited node's LLM row and the SSM rows
        # of the children it tested (all of them at the last node)
        rows = 0
        for b in range(cfg.B):
            par = w["parent"][b]
            vis = list(path_h[b, :plen_h[b]])
            for j, u in enumerate(vis):
                ch = [v for v in range(cfg.n) if par[v] == u]
                rows += 1 + (ch.index(vis[j + 1]) + 1 if j + 1 < len(vis) else len(ch))
        es_l = 2 if W.is16(cfg.dtype) else 4
        # the call's automatic mode: all row statistics first while all rows fit in 1 GiB
        pre = 2.0 * cfg.B * cfg.n * cfg.vocab * es_l <= float(1 << 30)
        if pre:   # every LLM row and every non-root SSM row, then the walk's residual and draw passes
            rows_all = cfg.B * (2 * cfg.n - 1)
        mss_out = {"us": round(t_mss * 1e6, 2), "mean_path_len": round(float(plen_h.mean()), 3),
                   "mode": "all-row statistics, walk over vocabulary slices" if pre else "visited rows, walk over vocabulary slices",
                   "rows_read": rows_all if pre else rows,
                   "hbm_gbs": round((rows_all if pre else rows) * cfg.vocab * es_l / t_mss / 1e9, 1)}
    # tree construction: one expansion step (4 frontier nodes per sequence, k = 4,
    # on the SSM rows) and a merge of 8 drafts of 8 tokens per sequence
    cons_out = None
    if mss is not None:
        Fx, kx = min(4, cfg.n - 1), 4
        nmx = cfg.n + Fx * kx
        pad = lambda a: np.pad(a, ((0, 0), (0, nmx - cfg.n)), constant_values=-1).astype(np.int32)
        ex_par = torch.from_numpy(pad(w["parent"])).cuda()
        ex_dep = torch.from_numpy(pad(w["depth"])).cuda()
        ex_tok = torch.from_numpy(pad(w["tokens"])).cuda()
        # frontier nodes 1..Fx and their SSM rows (the root's SSM row is a constant placeholder)
        ex_rows = mss[0]["ssm"][:, 1:1 + Fx].contiguous()
        ex_front = torch.arange(1, 1 + Fx, dtype=torch.int32, device="cuda").repeat(cfg.B, 1).contiguous()
        ex_ncur = torch.full((cfg.B,), cfg.n, dtype=torch.int32, device="cuda")
        ex_nout = torch.empty(cfg.B, dtype=torch.int32, device="cuda")
        ex_st = torch.empty(cfg.B, dtype=torch.int32, device="cuda")
        t_exp = timed_graph(lambda i, h: _lib.tree_expand_topk(ex_rows, ex_front, ex_ncur, ex_par, ex_dep, ex_tok, kx,
                                                               n_out=ex_nout, status=ex_st,
                                                               stream=torch.cuda.ExternalStream(h)))
        drng = np.random.default_rng(1)
        Md, Ldd = 8, 8
        mg_dr = torch.from_numpy(drng.integers(0, 4, size=(cfg.B, Md, Ldd)).astype(np.int32)).cuda()
        mg_len = torch.full((cfg.B, Md), Ldd, dtype=torch.int32, device="cuda")
        mg_out = [torch.empty(sh_, dtype=torch.int32, device="cuda")
                  for sh_ in ((cfg.B, 256), (cfg.B, 256), (cfg.B, 256), (cfg.B,), (cfg.B, Md, Ldd), (cfg.B,))]
        t_mrg = timed_graph(lambda i, h: _lib.tree_merge_drafts(mg_dr, mg_len, 256, parent=mg_out[0], depth=mg_out[1],
                                                                tokens=mg_out[2], n_out=mg_out[3], node_of=mg_out[4],
                                                                status=mg_out[5], stream=torch.cuda.ExternalStream(h)))
        if not ((ex_st == 0).all().item() and (mg_out[5] == 0).all().item()):
            raise RuntimeError("tree construction rejected a sequence of the benchmark batch")
        es_l = 2 if W.is16(cfg.dtype) else 4
        cons_out = {"expand_us": round(t_exp * 1e6, 2), "expand_rows": cfg.B * Fx, "k": kx,
                    "expand_hbm_gbs": round(cfg.B * Fx * cfg.vocab * es_l / t_exp / 1e9, 1),
                    "merge_us": round(t_mrg * 1e6, 2), "merge_drafts": [Md, Ldd]}

    # throughput: K whole steps back to back.  Default: one HIP graph holding one step
    # per input copy (R steps), replayed K/R times; --eager launches each call.
    if args.eager:
        for i in range(args.warmup):
            steps[i % R]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            steps[k % R]()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        K = max(R, K // R * R)
        graph = runner.capture_steps(steps)
        for i in range(max(1, args.warmup // R)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K // R):
            graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    ms_step = wall / K * 1e3
    tokens = cfg.B * cfg.n
    value = tokens / (wall / K)

    es = 2 if W.is16(cfg.dtype) else 4
    attn_gbs = refb["attn_bytes"] / t_attn / 1e9
    peak_tf = BF16_PEAK_TFLOPS if W.is16(cfg.dtype) else FP32_PEAK_TFLOPS  # fp16 dense MFMA peak = bf16's
    mfma_pct = refb["attn_flops"] / t_attn / 1e12 / peak_tf * 100
    # the workload as measured: element type and cache format are part of its name, so a
    # counter summary is only used for the variant it was taken on
    wname = cfg.name + ("_f16" if cfg.dtype == "f16" else "") + ("_fp8kv" if cfg.kv == "fp8" else "")
    traffic = load_traffic(wname)
    # the binding resource is the one whose peak takes longer for the algorithmic work:
    # HBM bytes at 8 TB/s, or the products at the dense matrix peak (fp32: the vector ALUs)
    t_hbm = refb["attn_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_flop = refb["attn_flops"] / (peak_tf * 1e12)
    if t_hbm >= t_flop:
        roofline = {"bound": "hbm", "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(attn_gbs / HBM_PEAK_GBS, 4)}
    else:
        attn_tfs = refb["attn_flops"] / t_attn / 1e12
        roofline = {"bound": "mfma" if W.is16(cfg.dtype) else "alu", "achieved": round(attn_tfs, 1), "peak": peak_tf,
                    "unit": "TFLOP/s", "frac": round(attn_tfs / peak_tf, 4)}
    roofline.update({"traffic": None if traffic is None else traffic["bytes_per_launch"],
                     "kernel": "tree_attention", "avg_launch_us": round(t_attn * 1e6, 2),
                     "algorithmic_bytes": refb["attn_bytes"], "algorithmic_flops": refb["attn_flops"]})

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "verified tree tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded, N(0,1) Q/K/V)",
        "config": {"workload": wname, "B": cfg.B, "n": cfg.n,
                   "Hq": cfg.Hq, "Hkv": cfg.Hkv, "D": cfg.D, "kv_cache": cfg.kv or cfg.dtype,
                   "prefix_len": [cfg.L_lo, cfg.L_hi], "paged": cfg.paged, "vocab": cfg.vocab,
                   "input_copies": R, "launch": "eager" if args.eager else "hip_graph"},
        "roofline": roofline,
        "attn_hbm_gbs": round(attn_gbs, 1), "mfma_util_pct": round(mfma_pct, 2),
        "tree_attention_us_per_launch": attn_dist,
        "kernel_us": {"tree_build": round(t_build * 1e6, 2), "tree_attention": round(t_attn * 1e6, 2),
                      "tree_verify_greedy": round(t_ver * 1e6, 2),
                      "tree_commit_kv": round(t_commit * 1e6, 2) if t_commit else None,
                      "tree_verify_stochastic": mss_out["us"] if mss_out else None},
        "stochastic": mss_out,
        "construct": cons_out,
        "commit": ({"tokens": committed, "hbm_gbs": round(4 * committed * cfg.Hkv * cfg.D * es / t_commit / 1e9, 1)}
                   if t_commit else None),
        "verify_hbm_gbs": round(refb["verify_bytes"] / t_ver / 1e9, 1) if cfg.vocab and t_ver else None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
