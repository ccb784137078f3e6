#!/usr/bin/env python3
"""Benchmark of the per-step hot path on one MI355X.

A step is one pass of the whole hot path over every layer of the model shape,
each layer on its own buffers (so the 256 MB last-level cache cannot hold the
working set):
    tree verification attention (full cache)   x layers
    draft attention (partial cache)            x layers
    partial-KV selection (score/select/gather) x layers
    penalty / temperature / top-p / min-p over the step's logits rows
    tree acceptance and the KV commit of the accepted path (all layers, one launch)
    the next step's draft tree: 4-gram retrieval over the last W tokens, random
    choice of k = 20, head candidates and chains (one launch)
The headline value is the verification attention time per layer-step,
measured with HIP events around the layers' verification launches on the
stream the library launches on. Inputs are seeded synthetic tensors of the
model's shapes, resident in HBM before timing starts. The float64 oracle is
timed beside every kernel on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 8b] [--T 24] [--n-ctx 100000]
    python bench.py --sweep      # one JSON line per workload cell (model classes, T and context sweeps)
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 / f16 matrix peak
METRIC = "tree-verify attn us/layer-step @100K ctx (8B GQA); achieved HBM GB/s vs peak"

# The workload cells of the sweep: the 8B shape over every tree size and
# context length of its sweep, the two wide trees (88 nodes: [1,9,9,9] plus
# 20 n-gram chains; 128 nodes) at 100K rows, and the other model classes at
# 100K rows with their own trees.
SWEEP = [("8b", T, L) for T in (24, 4, 64) for L in (100_000, 65_536, 32_768, 8_192)] + \
        [("8b", 88, 100_000), ("8b", 128, 100_000)] + \
        [("1.5b", 24, 100_000), ("7b", 24, 100_000), ("14b", 64, 100_000)]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="8b")
    ap.add_argument("--T", type=int, default=None, help="tree nodes (default: the workload's)")
    ap.add_argument("--n-ctx", type=int, default=None)
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--verify-only", action="store_true", help="time only the verification launches")
    ap.add_argument("--fused-scores", action="store_true",
                    help="verification also writes the selection scores; the selection reads them (no K pass)")
    ap.add_argument("--eta", action="store_true",
                    help="eta-sampling (epsilon 3e-4, alpha sqrt(epsilon)) in place of top-p and min-p")
    ap.add_argument("--sweep", action="store_true",
                    help="one JSON line per workload cell (fewer steps each; oracle beside every kernel)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=None,
                    help="oracle time budget per kernel (default 6 s, 2 s in the sweep)")
    ap.add_argument("--no-copy-bw", action="store_true",
                    help="skip the streaming-copy bandwidth measured after the timed steps")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one 1 GiB device-to-device copy first (reference for HBM byte counters)")
    return ap.parse_args()


def verify_flops(Hq, d, n_ctx, T):
    """Algorithmic flops of one verification launch: S = Q K^T and P V, two
    multiply-adds per query row, cache row and channel each."""
    return 4 * Hq * T * (n_ctx + T) * d


def verify_bytes(Hq, Hkv, d, n_ctx, T):
    """Algorithmic bytes of one verification launch: K and V over n_ctx + T rows
    (bf16), the queries (bf16) and the fp32 output."""
    return 2 * Hkv * (n_ctx + T) * d * 2 + Hq * T * d * 2 + Hq * T * d * 4


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover - reporting only
        return len(os.sched_getaffinity(0))


def _timed_samples(fn, n_max, budget_s):
    """Run fn(i) for i = 0, 1, ... until budget_s has passed or n_max samples
    are done (at least one); returns the per-sample times in seconds."""
    times = []
    t_start = time.perf_counter()
    while not times or (time.perf_counter() - t_start < budget_s and len(times) < n_max):
        t0 = time.perf_counter()
        fn(len(times))
        times.append(time.perf_counter() - t0)
    return times


def cpu_baselines(cfg, T, n_ctx, budget_s, kernels=("verify", "draft", "select", "penalty")):
    """The float64 oracle on the host on a bounded sample of each kernel's
    workload (whole KV-head groups of one layer, or whole logit rows), scaled
    to the kernel's unit. Input generation is outside the timed region; the
    bf16 -> float64 conversion is inside."""
    import numpy as np
    from oracle import bf16_to_f64, draft_attention, partial_kv_select, penalty_sample, verify_attention
    from oracle.select import gather_partial
    from synth import attention_inputs, penalty_inputs, tree_parent

    out = {}
    G, Hkv, d = cfg["Hq"] // cfg["Hkv"], cfg["Hkv"], cfg["d"]
    threads = _threads()
    parent = tree_parent("chain" if T <= 4 else ("wide" if T > 64 else "tokenswift"), T)   # the GPU step's tree
    if "verify" in kernels:
        x = attention_inputs(cfg["seed"], G, 1, d, n_ctx, T)   # one KV head and its query group
        ts_ = _timed_samples(lambda i: verify_attention(bf16_to_f64(x["q"]), bf16_to_f64(x["k"]), bf16_to_f64(x["v"]),
                                                        n_ctx, parent), Hkv, budget_s)
        out["verify"] = {"value": round(float(np.mean(ts_)) * Hkv * 1e6, 1), "unit": "us/layer-step", "cores": threads,
                         "kind": "oracle",
                         "sample": f"{len(ts_)} KV-head group(s) of one layer (G={G} query heads x T={T}, {n_ctx} "
                                   f"context rows, float64 NumPy), mean time per group x {Hkv} groups"}
        del x
    n_part = cfg["n_sink"] + cfg["budget"] + cfg["n_recent"]
    if "draft" in kernels:
        Tq = 4
        x = attention_inputs(cfg["seed"] + 1, G, 1, d, n_part, Tq)
        ts_ = _timed_samples(lambda i: draft_attention(bf16_to_f64(x["q"]), bf16_to_f64(x["k"]), bf16_to_f64(x["v"]),
                                                       n_part), 64, budget_s)
        out["draft"] = {"value": round(float(np.mean(ts_)) * Hkv * 1e6, 1), "unit": "us/layer-step", "cores": threads,
                        "kind": "oracle",
                        "sample": f"{len(ts_)} run(s) of one KV-head group (G={G} x Tq={Tq} over {n_part} partial "
                                  f"rows), mean x {Hkv} groups"}
        del x
    if "select" in kernels:
        x = attention_inputs(cfg["seed"] + 2, G, 1, d, n_ctx, T)

        def select_and_gather(i):
            r = partial_kv_select(bf16_to_f64(x["q"]), bf16_to_f64(x["k"]), n_ctx, 1, cfg["n_sink"], cfg["budget"],
                                  cfg["n_recent"])
            gather_partial(x["k"], x["v"], r.rows)

        ts_ = _timed_samples(select_and_gather, Hkv, budget_s)
        out["select"] = {"value": round(float(np.mean(ts_)) * Hkv * 1e6, 1), "unit": "us/layer-step", "cores": threads,
                         "kind": "oracle",
                         "sample": f"{len(ts_)} KV head(s) of one layer (scores of G={G} x T={T} queries over {n_ctx} "
                                   f"rows, top-{cfg['budget']} selection and the row gather), mean x {Hkv} heads"}
        del x
    if "penalty" in kernels:
        rows = T + 4
        px = penalty_inputs(cfg["seed"], 1, cfg["V"], cfg["W"], sigma=cfg.get("sigma", 2.0))
        ts_ = _timed_samples(lambda i: penalty_sample(px["logits"], px["window"], 1.2, 1.0, 0.9, 0.05, px["u"]), rows,
                             budget_s)
        out["penalty"] = {"value": round(float(np.mean(ts_)) * rows * 1e6, 1), "unit": "us/step", "cores": threads,
                          "kind": "oracle",
                          "sample": f"{len(ts_)} logit row(s) of V={cfg['V']} (window {cfg['W']}), mean x {rows} rows "
                                    "per step"}
    return out


def run_cell(args, name, T, n_ctx, steps, warmup, copy_bw, cpu_budget, cpu_kernels):
    """Time `steps` steps of one workload cell and return the result object."""
    import torch
    import long_kv_attention_amd as ts
    from synth import CONFIGS, ngram_window, tree_parent

    cfg = dict(CONFIGS[name])
    Hq, Hkv, d, layers = cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["layers"]
    reselect = cfg.get("reselect", 1)
    Tq = 4                                   # drafting: the accepted token + 3 heads' tokens
    n_sink, budget, n_recent = cfg["n_sink"], cfg["budget"], cfg["n_recent"]
    n_part = n_sink + budget + n_recent
    V, W = cfg["V"], cfg["W"]
    rows_logits = T + Tq
    parent = tree_parent("chain" if T <= 4 else ("wide" if T > 64 else "tokenswift"), T)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    gen = torch.Generator(device=dev)
    gen.manual_seed(cfg["seed"] * 1000)

    def randn(shape, dtype=torch.bfloat16):
        return torch.randn(shape, generator=gen, device=dev, dtype=torch.float32).to(dtype)

    # caches of all layers in one tensor each (the commit moves rows of every layer in one launch)
    K = torch.empty((layers, Hkv, n_ctx + T, d), dtype=torch.bfloat16, device=dev)
    Vc = torch.empty_like(K)
    part_cap = n_part + max(Tq, T)
    KP = torch.empty((layers, Hkv, part_cap, d), dtype=torch.bfloat16, device=dev)
    VP = torch.empty_like(KP)
    L = []
    for l in range(layers):
        k = randn((Hkv, n_ctx + T, d))
        if "k_scale" in cfg:
            lo, hi = cfg["k_scale"]
            k = (k.float() * (lo + (hi - lo) * torch.rand((Hkv, 1, d), generator=gen, device=dev))).to(torch.bfloat16)
        K[l] = k
        Vc[l] = randn((Hkv, n_ctx + T, d))
        KP[l] = randn((Hkv, part_cap, d))
        VP[l] = randn((Hkv, part_cap, d))
        del k
        L.append(dict(
            q=randn((Hq, T, d)), k=K[l], v=Vc[l],
            qd=randn((Hq, Tq, d)),
            kp=KP[l], vp=VP[l],
            kp2=torch.empty((Hkv, n_part + Tq, d), dtype=torch.bfloat16, device=dev),
            vp2=torch.empty((Hkv, n_part + Tq, d), dtype=torch.bfloat16, device=dev),
            out=torch.empty((Hq, T, d), dtype=torch.float32, device=dev),
            outd=torch.empty((Hq, Tq, d), dtype=torch.float32, device=dev),
            sel=torch.empty((Hkv, budget), dtype=torch.int32, device=dev),
            sc=torch.empty((Hkv, n_ctx), dtype=torch.float32, device=dev) if args.fused_scores else None,
        ))
    logits = randn((rows_logits, V), torch.float32) * cfg.get("sigma", 2.0)
    window = torch.randint(0, V, (rows_logits, W), generator=gen, device=dev, dtype=torch.int32)
    u = torch.rand(rows_logits, generator=gen, device=dev)
    lib = ts.lib()
    ws_v = torch.empty(max(1, lib.ts_verify_attn_workspace_size(n_ctx, T, Hq, Hkv, d, args.n_split)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, lib.ts_draft_attn_workspace_size(n_part, Tq, Hq, Hkv, d, 0)), dtype=torch.uint8, device=dev)
    ws_s = torch.zeros(max(1, lib.ts_partial_kv_select_workspace_size(n_ctx, T, Hq, Hkv, d, budget)), dtype=torch.uint8, device=dev)
    ws_ss = torch.zeros(max(1, lib.ts_partial_kv_select_scored_workspace_size(n_ctx, Hkv, d, budget)), dtype=torch.uint8, device=dev)
    z_out = torch.empty_like(logits)
    torch.cuda.synchronize()

    if args.calibrate_copy:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counters give the
        # scale between the counters and bytes moved (see the profiles' notes).
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    # the committed tokens' window for the n-gram tree (repeated phrases, as generated text has)
    ng_window = torch.from_numpy(ngram_window(cfg["seed"], W, vocab=V, repeat=0.5, n_phrases=8)).to(dev)
    ng_head = torch.randint(0, V, (3, 3), generator=gen, device=dev, dtype=torch.int32)
    ng_out = [torch.empty(T, dtype=torch.int32, device=dev), torch.empty(T, dtype=torch.int32, device=dev),
              torch.empty(4, dtype=torch.int32, device=dev)]
    # Draft tokens of the tree: planted once so that the top head path (three
    # drafted tokens) matches the target's tokens, which the step recomputes
    # identically (same logits and u): 4 rows committed per step.
    ts.penalty_sample(logits, window, 1.2, 1.0, 0.9, 0.05, u=u, out=z_out)
    tok0 = ts.penalty_sample(logits, window, 1.2, 1.0, 0.9, 0.05, u=u, want_keep=False, want_probs=False)[3]
    target_host = tok0[:T].cpu().numpy()
    node_host = [-1] * T
    node_i = 0
    while True:
        kids = [c for c in range(T) if parent[c] == node_i]
        if not kids:
            break
        node_host[kids[0]] = int(target_host[node_i])
        node_i = kids[0]
    node_tok = torch.tensor(node_host, dtype=torch.int32, device=dev)
    accept_res = torch.empty(T + 2, dtype=torch.int32, device=dev)
    token_out = torch.empty(rows_logits, dtype=torch.int32, device=dev)

    def step(e=None):
        if e:
            e[0].record(stream)
        for Ld in L:
            if args.fused_scores:
                ts.verify_attn_scored(Ld["q"], Ld["k"], Ld["v"], n_ctx, parent, n_split=args.n_split, out=Ld["out"],
                                      scores=Ld["sc"], ws=ws_v)
            else:
                ts.verify_attn(Ld["q"], Ld["k"], Ld["v"], n_ctx, parent, n_split=args.n_split, out=Ld["out"], ws=ws_v)
        if e:
            e[1].record(stream)
        if not args.verify_only:
            for Ld in L:
                ts.draft_attn(Ld["qd"], Ld["kp"], Ld["vp"], n_part, out=Ld["outd"], ws=ws_d)
        if e:
            e[2].record(stream)
        if not args.verify_only:
            # timed every step; a cadence of `reselect` steps is applied to the
            # per-step figure below
            for Ld in L:
                if args.fused_scores:
                    ts.partial_kv_select_scored(Ld["sc"], Ld["k"], Ld["v"], n_ctx, n_sink, budget, n_recent,
                                                k_part=Ld["kp2"], v_part=Ld["vp2"], sel_idx=Ld["sel"], ws=ws_ss)
                else:
                    ts.partial_kv_select(Ld["q"], Ld["k"], Ld["v"], n_ctx, n_sink, budget, n_recent, k_part=Ld["kp2"],
                                         v_part=Ld["vp2"], sel_idx=Ld["sel"], ws=ws_s)
        if e:
            e[3].record(stream)
        if not args.verify_only:
            if args.eta:
                ts.penalty_sample_eta(logits, window, 1.2, 1.0, 3e-4, 3e-4 ** 0.5, u=u, out=z_out, token_out=token_out)
            else:
                ts.penalty_sample(logits, window, 1.2, 1.0, 0.9, 0.05, u=u, out=z_out, token_out=token_out)
        if e:
            e[4].record(stream)
        if not args.verify_only:
            ts.tree_accept(parent, node_tok, token_out[:T], result=accept_res)
            ts.kv_commit(accept_res, T, K, Vc, n_ctx, KP, VP, n_part)
        if e:
            e[5].record(stream)
        if not args.verify_only:
            ts.ngram_tree(ng_window, 20, 12345, ng_head, T, parent=ng_out[0], node_token=ng_out[1], info=ng_out[2])
        if e:
            e[6].record(stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        step(ev[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    def avg(i, j):
        return sum(ev[s][i].elapsed_time(ev[s][j]) for s in range(steps)) / steps * 1e3  # us

    verify_us = avg(0, 1) / layers
    per_step = sorted(ev[s][0].elapsed_time(ev[s][1]) * 1e3 / layers for s in range(steps))
    verify_med = per_step[len(per_step) // 2] if len(per_step) % 2 else 0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    draft_us = avg(1, 2) / layers
    select_us = avg(2, 3) / layers
    penalty_us = avg(3, 4)
    commit_us = avg(4, 5)
    ngram_us = avg(5, 6)
    step_ms = avg(0, 6) / 1e3
    # the partial cache is refreshed every `reselect` steps: its per-step share
    step_ms_cadence = step_ms - select_us * layers * (1 - 1 / reselect) / 1e3
    vb = verify_bytes(Hq, Hkv, d, n_ctx, T)
    achieved = vb / (verify_us * 1e-6) / 1e9

    del L, K, Vc, KP, VP
    torch.cuda.empty_cache()

    # streaming-copy bandwidth measured in the same process after the timed
    # region (a secondary denominator next to the vendor peak): device-to-device
    # copies of 1 GiB, read + write bytes over event time
    copy_gbps = None
    if copy_bw:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(5):
            dst.copy_(src)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del src, dst

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "verify_attn_traffic.json")
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            key = f"{name}_L{n_ctx}_T{T}"
            if tj.get("kernel_source_sha") == _attn_source_sha() and key in tj.get("bytes_per_launch", {}):
                traffic = tj["bytes_per_launch"][key]
        except Exception:
            traffic = None

    # The call's bound by its arithmetic intensity against the ridge (peak flops
    # over peak bandwidth, 312.5 flop/B): below it the HBM roofline, above it
    # the matrix cores' (wide trees, the 14B shape).
    vf = verify_flops(Hq, d, n_ctx, T)
    if vf / vb <= MFMA_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9):
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic}
    else:
        tflops = vf / (verify_us * 1e-6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                    "hbm_GBps": round(achieved, 1), "hbm_frac": round(achieved / HBM_PEAK_GBPS, 4)}
    res = {
        "metric": METRIC,
        "value": round(verify_us, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name}-class {'GQA' if Hq != Hkv else 'MHA'} tree verification, "
                               f"{Hq} q / {Hkv} kv heads, d={d}, {n_ctx} context rows, T={T} tree nodes, {layers} layers",
                   "global_batch": 1, "seq_len": n_ctx, "tree_nodes": T, "layers": layers,
                   "reselect_every": reselect,
                   "fused_scores": bool(args.fused_scores), "eta_sampling": bool(args.eta),
                   "parallelism": "single-gpu"},
        "roofline": roofline,
        "stream_copy": None if copy_gbps is None else
                       {"GBps": round(copy_gbps, 1), "bytes_per_copy": 2 * (1 << 30),
                        "verify_frac_of_copy": round(achieved / copy_gbps, 4)},
        "env": _gpu_env(torch),
        "kernels_us": {"verify_per_layer": round(verify_us, 3),
                       "verify_per_layer_median": round(verify_med, 3), "verify_per_layer_min": round(per_step[0], 3),
                       "verify_per_layer_max": round(per_step[-1], 3), "draft_per_layer": round(draft_us, 3),
                       "select_per_layer": round(select_us, 3),
                       "select_per_layer_per_step": round(select_us / reselect, 3),
                       "penalty_per_step": round(penalty_us, 3),
                       "accept_commit_per_step": round(commit_us, 3), "ngram_tree_per_step": round(ngram_us, 3),
                       "verify_bytes_per_launch": vb, "verify_flops_per_launch": vf},
        "ms_per_step_with_reselect_cadence": round(step_ms_cadence, 4),
        "wall_s": round(wall, 3),
    }
    if cpu_budget:
        base = cpu_baselines(cfg, T, n_ctx, cpu_budget, cpu_kernels)
        if "verify" in base:
            res["cpu_baseline"] = base.pop("verify")
        if base:
            res["cpu_baseline_other_kernels"] = base
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the multi-GPU sharding of this path "
              "is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    from synth import CONFIGS

    if not args.sweep:
        cfg = CONFIGS[args.config]
        T = args.T or cfg["T"]
        n_ctx = args.n_ctx or cfg["n_ctx"]
        budget = None if args.no_cpu_baseline else (args.cpu_seconds or 6.0)
        res = run_cell(args, args.config, T, n_ctx, args.steps, args.warmup, not args.no_copy_bw, budget,
                       ("verify", "draft", "select", "penalty"))
        print(json.dumps(res), flush=True)
        return

    # sweep: fewer steps per cell; the oracle beside the verification kernel in
    # every cell and beside the other kernels once per model class
    steps = min(args.steps, 8)
    warmup = min(args.warmup, 2)
    budget = None if args.no_cpu_baseline else (args.cpu_seconds or 2.0)
    seen = set()
    for name, T, n_ctx in SWEEP:
        kernels = ("verify",) if name in seen else ("verify", "draft", "select", "penalty")
        seen.add(name)
        res = run_cell(args, name, T, n_ctx, steps, warmup, False, budget, kernels)
        res["sweep_cell"] = f"{name}_L{n_ctx}_T{T}"
        print(json.dumps(res), flush=True)


def _gpu_env(torch):
    """Device name, ROCm / HIP / torch versions and the engine and memory
    clocks' top DPM levels (read from sysfs; None where not readable)."""
    import glob
    import re
    env = {"gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip, "torch": torch.__version__, "rocm": None,
           "sclk_max_mhz": None, "mclk_max_mhz": None}
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        pass
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        for name, key in (("pp_dpm_sclk", "sclk_max_mhz"), ("pp_dpm_mclk", "mclk_max_mhz")):
            try:
                with open(os.path.join(dev, name)) as f:
                    levels = [int(m) for m in re.findall(r"(\d+)\s*Mhz", f.read(), re.I)]
            except OSError:
                continue
            if levels:
                env[key] = max(levels)
        if env["sclk_max_mhz"] is not None:
            break
    return env


def _attn_source_sha():
    import hashlib
    p = os.path.join(ROOT, "long_kv_attention_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
