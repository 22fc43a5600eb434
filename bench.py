#!/usr/bin/env python
"""Benchmark: ms per 10-step action chunk and denoise steps/s of the Pi0-scale
action expert (bf16 weights, fp32 accumulate, batch 1, 816-token prefix KV,
chunk 50 x 32) on one MI355X.

One bench step = one whole action chunk: `steps` Euler steps of the suffix
(in_proj + time embedding, 18 decoder blocks over [prefix KV ; suffix],
out_proj, Euler update), replayed as one captured graph with the noise
already resident in HBM. Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
RIDGE_BF16 = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # FLOP per HBM byte where the two roofs meet


def kernel_bytes(cfg):
    """Algorithmic HBM bytes per launch of each kernel: weights (and KV) read once."""
    w, F, dh, nq, nkv, A = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.action_dim
    wb = 2 if cfg.weight_dtype == "bf16" else 4
    mb = {"bf16": 2, "fp8": 1, "f32": 4}[cfg.mlp_dtype]
    sc = 4 if cfg.mlp_dtype == "fp8" else 0
    kvb = 2 if cfg.kv_dtype == "bf16" else 4
    kb = {
        "qkv_rope": (nq + 2 * nkv) * dh * w * wb,
        "attn": 2 * (cfg.prefix_len + cfg.horizon) * nkv * dh * kvb,
        "o_proj_resid": w * nq * dh * wb,
        "gate_up_geglu": 2 * F * w * mb + 2 * F * sc,
        "down_resid": w * F * mb + w * sc,
        "in_proj": w * A * wb,
        "out_proj_euler": A * w * wb,
    }
    # the persistent step kernel: one launch is one whole Euler step of one robot (every layer's
    # weights, the robot's prefix K/V, in/out projections)
    prefix_kv = 2 * cfg.prefix_len * nkv * dh * kvb
    kb["fused_step"] = (cfg.n_layers * (kb["qkv_rope"] + kb["o_proj_resid"] + kb["gate_up_geglu"] + kb["down_resid"]
                                        + prefix_kv) + kb["in_proj"] + kb["out_proj_euler"])
    return kb


def kernel_flops(cfg, seqs):
    """Algorithmic FLOPs per launch of each kernel over `seqs` suffix sequences of H rows."""
    w, F, dh, nq, nkv, A, H = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.action_dim, cfg.horizon
    rows = seqs * H
    return {
        "qkv_rope": 2 * rows * (nq + 2 * nkv) * dh * w,
        "attn": seqs * 4 * nq * H * (cfg.prefix_len + H) * dh,
        "o_proj_resid": 2 * rows * w * nq * dh,
        "gate_up_geglu": 2 * rows * 2 * F * w,
        "down_resid": 2 * rows * w * F,
        "in_proj": 2 * rows * w * A,
        "out_proj_euler": 2 * rows * A * w,
        "fused_step": step_flops(cfg, seqs),
    }


def annotate(entry, alg_bytes, alg_flops, avg_us):
    """Both roofs of one kernel: HBM bytes and FLOPs per launch over its average duration; `bound` is the
    roof its arithmetic intensity puts it under (MFMA above the bf16 ridge), `frac` the fraction of it."""
    gbs = alg_bytes / (avg_us * 1e-6) / 1e9
    tfl = alg_flops / (avg_us * 1e-6) / 1e12
    entry.update({"alg_bytes": alg_bytes, "alg_flops": alg_flops, "GBs": round(gbs, 1), "TFLOPs": round(tfl, 2),
                  "hbm_frac": round(gbs / PEAK_HBM_GBS, 4), "mfma_frac": round(tfl / PEAK_BF16_TFLOPS, 4)})
    entry["bound"] = "mfma" if alg_flops > RIDGE_BF16 * alg_bytes else "hbm"
    entry["frac"] = entry["mfma_frac"] if entry["bound"] == "mfma" else entry["hbm_frac"]
    return entry


def roofline_of(kernels, dom, traffic=None):
    if not dom or "bound" not in kernels[dom]:
        return {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": None,
                "traffic": None}
    e = kernels[dom]
    mfma = e["bound"] == "mfma"
    return {"kernel": dom, "bound": e["bound"], "achieved": e["TFLOPs"] if mfma else e["GBs"],
            "peak": PEAK_BF16_TFLOPS if mfma else PEAK_HBM_GBS, "unit": "TFLOP/s" if mfma else "GB/s",
            "frac": e["frac"], "hbm_frac": e["hbm_frac"], "mfma_frac": e["mfma_frac"],
            "traffic": (traffic or {}).get(dom)}


def measured_traffic():
    """HBM bytes per launch of each kernel from the committed rocprofv3 counter summaries (profiles/*.md
    with a machine-readable table), keeping only those taken from the kernel sources as they are now."""
    import glob
    import hashlib
    sha = hashlib.sha256()
    for f in ("ae_kernels.hpp", "ae_fused.hpp", "ae_runtime.hip"):
        with open(os.path.join(ROOT, "flow_matching_action_euler_amd", "csrc", f), "rb") as fh:
            sha.update(fh.read())
    now = sha.hexdigest()[:16]
    out = {}
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        want, table = None, {}
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic_source_sha256_16:"):
                    want = line.split(":", 1)[1].strip()
                elif line.startswith("traffic_bytes_per_launch:"):
                    table = json.loads(line.split(":", 1)[1])
        if want == now:
            out.update(table)
    return out


def step_bytes(cfg, batch):
    kb = kernel_bytes(cfg)
    per_layer = kb["qkv_rope"] + kb["o_proj_resid"] + kb["gate_up_geglu"] + kb["down_resid"]
    kv = batch * (kb["attn"] - 2 * cfg.horizon * cfg.n_kv_heads * cfg.head_dim * (2 if cfg.kv_dtype == "bf16" else 4))
    return cfg.n_layers * (per_layer + kv) + kb["in_proj"] + kb["out_proj_euler"]


def step_flops(cfg, sequences):
    """FLOPs of one velocity pass over `sequences` suffix sequences of H rows: 2 per weight per row
    for every projection, plus Q.K^T and P.V of every query row over its P + H keys."""
    w, F, dh, nq, nkv, A, H = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.action_dim, cfg.horizon
    per_layer = (nq + 2 * nkv) * dh * w + w * nq * dh + 2 * F * w + w * F
    rows = sequences * H
    gemm = 2 * rows * (cfg.n_layers * per_layer + 2 * w * A)
    attn = cfg.n_layers * sequences * 4 * nq * H * (cfg.prefix_len + H) * dh
    return gemm + attn


def _cores():
    """Threads the oracle's BLAS uses on this host."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1]))
    except Exception:
        return int(os.cpu_count())


def _cpu_model():
    """The host CPU as /proc/cpuinfo names it, with family / model / stepping and the logical CPU count
    (some hosts give only a marketing name)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if ":" in line:
                    k, v = line.split(":", 1)
                    info.setdefault(k.strip(), v.strip())
    except OSError:
        return "unknown"
    name = info.get("model name", "unknown")
    return (f"{name} (vendor {info.get('vendor_id', '?')}, family {info.get('cpu family', '?')}, model "
            f"{info.get('model', '?')}, stepping {info.get('stepping', '?')}, {os.cpu_count()} logical CPUs visible, "
            f"{info.get('cpu MHz', '?')} MHz)")


def cpu_baseline(cfg, W, k, v, noise, budget_s=12.0, single_core_s=5.0):
    """The oracle as it stands, timed on this host: Euler steps of one robot until the budget is spent,
    with every BLAS thread, then again (a shorter budget) on one thread."""
    from oracle import ae_oracle as O
    cores = _cores()
    Wd = O.dequantize_weights(cfg, W)
    kk, vv = O.decode_kv(cfg, k, v)

    def run(budget, cap):
        x = noise[0].astype(np.float64)
        n = 0
        t0 = time.perf_counter()
        while True:
            x = x + (1.0 / cfg.steps) * O.velocity(cfg, Wd, kk, vv, x, (n % cfg.steps) / cfg.steps)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget or n >= cap:
                return n, el

    n, el = run(budget_s, 40)
    out = {"value": n / el, "unit": "denoise steps/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{n} Euler steps of one robot ({cfg.name}, P={cfg.prefix_len}, H={cfg.horizon}), fp64 numpy, "
                     f"{el:.1f} s", "cpu_model": _cpu_model()}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1, user_api="blas"):
            n1, el1 = run(single_core_s, 10)
        out["single_core"] = {"value": n1 / el1, "sample": f"{n1} Euler steps, one BLAS thread, {el1:.1f} s"}
    except ImportError:
        pass
    return out


def bench_verify(args, cfg, W, kvs, ex, stream):
    """Verify passes: every flow time of one draft in one batched pass (M = n_tau * H), timed
    like the chunks (warm-up, then events around each pass on the library's stream)."""
    import torch
    from workload import gen as G
    sp = stream.cuda_stream
    draft, noise, taus = G.make_verify_case(cfg, 0)
    n_tau = len(taus)
    d_draft = torch.from_numpy(draft).cuda()
    d_noise = torch.from_numpy(noise).cuda()
    d_taus = torch.from_numpy(taus).cuda()
    d_acc = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_sw = torch.zeros(1, dtype=torch.int32, device="cuda")
    d_dist = torch.zeros((n_tau, cfg.horizon), dtype=torch.float32, device="cuda")
    args_v = (0, d_draft.data_ptr(), d_noise.data_ptr(), d_taus.data_ptr(), n_tau, 0.05, d_acc.data_ptr(),
              d_sw.data_ptr(), d_dist.data_ptr(), sp)
    ex.verify(0, draft, noise, taus, 0.05)  # captures the graph; sets the inputs ae_kernel_times reuses
    for _ in range(args.warmup):
        ex.verify_async(*args_v)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        ex.verify_async(*args_v)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    pass_ms = np.array([a.elapsed_time(b) for a, b in evs])
    assert np.all(np.isfinite(d_dist.cpu().numpy()))
    kb = kernel_bytes(cfg)
    kernels = {}
    if not args.no_kernel_times:
        for name, launches, total in ex.kernel_times(3, n_tau, cfg.steps, args.kernel_iters):
            if launches == 0:
                continue
            avg_us = total * 1e3 / launches
            entry = {"launches_per_pass": launches // args.kernel_iters, "avg_us": round(avg_us, 3),
                     "ms_per_pass": round(total / args.kernel_iters, 4)}
            if name in kb:
                kvb = 2 if cfg.kv_dtype == "bf16" else 4
                suffix = 2 * cfg.horizon * cfg.n_kv_heads * cfg.head_dim * kvb  # every flow time shares the prefix
                per_launch = kb[name] + (n_tau - 1) * suffix if name == "attn" else kb[name]
                annotate(entry, per_launch, kernel_flops(cfg, n_tau)[name], avg_us)
            kernels[name] = entry
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_pass"]) if kernels else None
    sb = step_bytes(cfg, 1)
    ms = elapsed * 1e3 / args.steps
    result = {
        "metric": "verify passes/s (all flow times of one draft, Pi0-scale expert)",
        "value": round(args.steps / elapsed, 2),
        "unit": "verify passes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_is": "ms per bench step = one verify pass (every flow time of one draft)",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prefix KV, random-walk draft, N(0,1) noise)",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "width": cfg.width, "prefix_len": cfg.prefix_len,
                   "chunk": f"{cfg.horizon}x{cfg.action_dim}", "flow_times": n_tau, "rows": n_tau * cfg.horizon},
        "pass_ms_median": round(float(np.median(pass_ms)), 4),
        "pass_ms_p90": round(float(np.percentile(pass_ms, 90)), 4),
        "pass_alg_bytes": sb,
        "pass_hbm_frac": round(sb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "pass_flops": step_flops(cfg, n_tau),
        "pass_mfma_frac": round(step_flops(cfg, n_tau) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline_of(kernels, dom),
        "kernels": kernels,
    }
    result["rounds"] = bench_rounds(cfg, ex, args.steps)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_verify(cfg, W, kvs[0][0], kvs[0][1])
    ex.close()
    print(json.dumps(result))


def bench_rounds(cfg, ex, reps):
    """Dual-path rounds (ae_round, synchronous, host buffers): a fast round (the verification
    accepts: draft seed 0, no gripper switch, delta above every distance) and a full round (draft
    seed 1 switches the gripper: verification, then the 10-step denoise). Wall clock per call and
    the device-timeline figure of ae_last_gpu_ms, medians over `reps` rounds after one warm-up."""
    from workload import gen as G
    out = {}
    for name, seed in (("fast", 0), ("full", 1)):
        draft, noise, taus = G.make_verify_case(cfg, seed)
        nf = G.make_noise(cfg, 500 + seed, 1)[0]
        res = ex.round(0, draft, noise, taus, 1e9, nf, cfg.steps)  # captures the graphs
        assert res[3] == (name == "full")
        wall, gpu = [], []
        for _ in range(reps):
            t0 = time.perf_counter()
            ex.round(0, draft, noise, taus, 1e9, nf, cfg.steps)
            wall.append((time.perf_counter() - t0) * 1e3)
            gpu.append(ex.last_gpu_ms())
        out[name] = {"wall_ms": round(float(np.median(wall)), 4), "gpu_ms": round(float(np.median(gpu)), 4),
                     "accept": int(res[1]), "full_path": int(res[3])}
    return out


def bench_draft(args, cfg, W):
    """Draft-model passes: `value` from the device time of the graph replay of each ae_draft call (the
    feature K/V projection, the block over the action queries and the head; HIP events around the
    replay alone, the features resident when it starts), over `steps` calls after `warmup`; the
    synchronous call's rate (features uploaded, chunk copied back) is reported beside it."""
    from flow_matching_action_euler_amd import ActionExpert
    from workload import gen as G
    ex = ActionExpert(cfg, W)
    feats = G.make_features(cfg, 1)
    for _ in range(max(1, args.warmup)):
        ex.draft(feats)
    wall, gpu = [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        t1 = time.perf_counter()
        chunk = ex.draft(feats)
        wall.append((time.perf_counter() - t1) * 1e3)
        gpu.append(ex.last_gpu_ms())
    elapsed = time.perf_counter() - t0
    assert np.all(np.isfinite(chunk))
    w, F, dh, nq, nkv, A = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.action_dim
    block = ((nq + 2 * nkv) * dh * w + w * nq * dh + 3 * F * w) * 2 + A * w * 2
    gpu_ms = float(np.median(gpu))
    result = {
        "metric": "draft passes/s (FLASH draft model: one 2B-class Gemma block over image features and action queries)",
        "value": round(args.steps / (float(np.sum(gpu)) * 1e-3), 2),
        "unit": "draft passes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(gpu)), 4),
        "host_call": {"passes_per_s": round(args.steps / elapsed, 2), "ms_median": round(float(np.median(wall)), 4),
                      "note": "synchronous ae_draft: features uploaded, the chunk copied back"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) image features and queries)",
        "config": {"workload": cfg.name, "width": w, "heads": f"{nq}q/{nkv}kv", "head_dim": dh, "mlp_dim": F,
                   "image_tokens": cfg.prefix_len, "queries": cfg.horizon, "params": cfg.n_params},
        "gpu_ms_median": round(gpu_ms, 4),
        "roofline": {"kernel": "whole draft pass", "bound": "hbm", "achieved": round(block / (gpu_ms * 1e-3) / 1e9, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(block / (gpu_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_draft(cfg, W, feats)
    ex.close()
    print(json.dumps(result))


def cpu_baseline_draft(cfg, W, feats, budget_s=12.0):
    """The oracle's draft pass on the host (fp64 numpy), as many passes as fit in ~budget_s (at least one)."""
    from oracle import ae_oracle as O
    Wd = O.dequantize_weights(cfg, W)
    n, t0 = 0, time.perf_counter()
    while n == 0 or time.perf_counter() - t0 < budget_s:
        O.draft_chunk(cfg, Wd, feats)
        n += 1
    dt = time.perf_counter() - t0
    return {"value": round(n / dt, 3), "unit": "draft passes/s", "cores": _cores(), "kind": "oracle",
            "sample": f"{n} draft passes ({cfg.name}), fp64 numpy, {dt:.1f} s"}


def prefill_flops(cfg):
    """FLOPs of one prefill pass: 2 per weight per prefix token for every projection of every layer, plus
    Q.K^T and P.V of every token over all P prefix tokens."""
    w, F, dh, nq, nkv, P = cfg.width, cfg.mlp_dim, cfg.head_dim, cfg.n_q_heads, cfg.n_kv_heads, cfg.horizon
    per_layer = (nq + 2 * nkv) * dh * w + w * nq * dh + 3 * F * w
    return cfg.n_layers * (2 * P * per_layer + 4 * nq * P * P * dh)


def bench_prefill(args, cfg, W):
    """Prefill passes: `value` from the device time of the graph replay of each ae_prefill call (HIP
    events around the replay alone: the embeddings are resident when it starts), over `steps` calls
    after `warmup`; the synchronous call's rate (upload, copy back, unpack) is reported beside it."""
    from flow_matching_action_euler_amd import ActionExpert
    from workload import gen as G
    ex = ActionExpert(cfg, W)
    emb = G.make_prefix_embeddings(cfg, 1)
    for _ in range(max(1, args.warmup)):
        ex.prefill(emb)
    wall, gpu = [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        t1 = time.perf_counter()
        k, v = ex.prefill(emb)
        wall.append((time.perf_counter() - t1) * 1e3)
        gpu.append(ex.last_gpu_ms())
    elapsed = time.perf_counter() - t0
    assert k.shape[0] == cfg.n_layers
    gpu_ms = float(np.median(gpu))
    fl = prefill_flops(cfg)
    tflops = fl / (gpu_ms * 1e-3) / 1e12
    result = {
        "metric": "prefill passes/s (prefix KV cache of every layer from the prefix embeddings)",
        "value": round(args.steps / (float(np.sum(gpu)) * 1e-3), 2),
        "unit": "prefill passes/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(float(np.mean(gpu)), 4),
        "host_call": {"passes_per_s": round(args.steps / elapsed, 2), "ms_median": round(float(np.median(wall)), 4),
                      "note": "synchronous ae_prefill: embeddings uploaded, every layer's K/V copied back and unpacked"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if cfg.mlp_dtype == "bf16" else "bf16 (E4M3 MLP weights)",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prefix embeddings)",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "width": cfg.width,
                   "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv", "head_dim": cfg.head_dim, "mlp_dim": cfg.mlp_dim,
                   "prefix_tokens": cfg.horizon, "params": cfg.n_params},
        "gpu_ms_median": round(gpu_ms, 4),
        "roofline": {"kernel": "whole prefill pass", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_prefill(cfg, emb)
    ex.close()
    print(json.dumps(result))


def cpu_baseline_prefill(cfg, emb, layers=2):
    """The oracle's prefill on the host (fp64 numpy) over the first `layers` layers of the stack, scaled
    to whole passes (the layers have equal shapes and cost)."""
    from oracle import ae_oracle as O
    from workload import gen as G
    sub = cfg.with_(n_layers=layers)
    Wd = O.dequantize_weights(sub, G.make_weights(sub))
    t0 = time.perf_counter()
    O.prefill_kv(sub, Wd, emb)
    dt = time.perf_counter() - t0
    return {"value": round(layers / (dt * cfg.n_layers), 4), "unit": "prefill passes/s", "cores": _cores(),
            "kind": "oracle",
            "sample": f"{layers} of the {cfg.n_layers} layers over {cfg.horizon} prefix tokens ({cfg.name}), "
                      f"fp64 numpy, {dt:.1f} s, scaled by {cfg.n_layers}/{layers}"}


def cpu_baseline_verify(cfg, W, k, v, budget_s=12.0):
    """The oracle as it stands, timed on this host: verify passes (all flow times) of one draft."""
    from oracle import ae_oracle as O
    from workload import gen as G
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        cores = os.cpu_count()
    Wd = O.dequantize_weights(cfg, W)
    kk, vv = O.decode_kv(cfg, k, v)
    draft, noise, taus = G.make_verify_case(cfg, 0)
    n = 0
    t0 = time.perf_counter()
    while True:
        O.verify(cfg, Wd, kk, vv, draft, noise, taus, 0.05)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20:
            break
    return {"value": n / el, "unit": "verify passes/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n} verify passes of one draft ({cfg.name}, {len(taus)} flow times, P={cfg.prefix_len}, "
                      f"H={cfg.horizon}), fp64 numpy, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed action chunks")
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--config", default="pi0_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-iters", type=int, default=3, help="replays of each per-kernel timing graph")
    ap.add_argument("--no-kernel-times", action="store_true", help="skip the per-kernel timing pass")
    ap.add_argument("--copy-kernel-mib", type=int, default=0,
                    help="after the timed loop, run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no multi-GPU leg)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from flow_matching_action_euler_amd import ActionExpert
    from workload import configs as C
    from workload import gen as G

    cfg = C.config_by_name(args.config)
    B = cfg.batch
    t_setup = time.perf_counter()
    W = G.make_weights(cfg)
    if cfg.draft:
        torch.cuda.set_device(0)
        return bench_draft(args, cfg, W)
    if cfg.prefill:
        torch.cuda.set_device(0)
        return bench_prefill(args, cfg, W)
    kvs = [G.make_prefix_kv(cfg, cfg.kv_seed + r) for r in range(B)]
    noise = G.make_noise(cfg, batch=B)
    torch.cuda.set_device(0)
    ex = ActionExpert(cfg, W)
    for r in range(B):
        ex.load_prefix_kv(r, *kvs[r])
    d_noise = torch.from_numpy(noise).cuda()
    d_out = torch.empty_like(d_noise)
    stream = torch.cuda.Stream()  # the library enqueues on this stream; the events below bracket it
    sp = stream.cuda_stream
    torch.cuda.synchronize()
    print(f"setup {time.perf_counter() - t_setup:.1f} s", file=sys.stderr, flush=True)

    if cfg.max_taus > 0 and cfg.batch == 1 and cfg.name.endswith("verify"):
        return bench_verify(args, cfg, W, kvs, ex, stream)
    for _ in range(args.warmup):
        ex.denoise_async(B, d_noise.data_ptr(), cfg.steps, d_out.data_ptr(), sp)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        evs[i][0].record(stream)
        ex.denoise_async(B, d_noise.data_ptr(), cfg.steps, d_out.data_ptr(), sp)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    chunk_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms_per_chunk = elapsed * 1e3 / args.steps
    out = d_out.cpu().numpy()
    assert np.all(np.isfinite(out))
    if args.copy_kernel_mib > 0:  # known traffic: reads and writes copy_kernel_mib MiB once per copy
        src = torch.ones(args.copy_kernel_mib << 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Per-kernel timing on the library's stream. "in place": the chunk's launches in their
    # normal order, each with a HIP start/stop event pair bound to its dispatch, so a kernel is
    # timed in the cache state the whole chunk gives it (weights streamed from HBM); this is the
    # figure the roofline uses. "isolated": every launch of one kernel back to back in a graph of
    # its own (one kernel's weights for all layers may then stay in the 256 MB MALL).
    kb = kernel_bytes(cfg)
    kernels = {}
    if not args.no_kernel_times:
        iso = {n: (l, t) for n, l, t in ex.kernel_times(0, B, cfg.steps, args.kernel_iters)}
        for name, launches, total in ex.kernel_times(2, B, cfg.steps, args.kernel_iters):
            if launches == 0:
                continue
            avg_us = total * 1e3 / launches
            entry = {"launches_per_chunk": launches // args.kernel_iters, "avg_us": round(avg_us, 3),
                     "ms_per_chunk": round(total / args.kernel_iters, 4)}
            if name in iso and iso[name][0]:
                entry["isolated_avg_us"] = round(iso[name][1] * 1e3 / iso[name][0], 3)
            if name in kb:
                per_launch = kb[name] * (B if name == "attn" else 1)
                annotate(entry, per_launch, kernel_flops(cfg, 1 if name == "fused_step" else B)[name], avg_us)
            kernels[name] = entry
    traffic = measured_traffic() if cfg.name == "pi0_bf16" else {}
    for name, entry in kernels.items():
        if name in traffic:
            entry["traffic_bytes"] = traffic[name]
    dom = max(kernels, key=lambda n: kernels[n]["ms_per_chunk"]) if kernels else None
    sb = step_bytes(cfg, B)
    result = {
        "metric": "ms per 10-step action chunk & denoise steps/s (Pi0-scale expert, bs1)",
        "value": round(args.steps * cfg.steps / elapsed, 2),
        "unit": "denoise steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_chunk, 4),
        "ms_per_step_is": f"ms per bench step = one whole {cfg.steps}-Euler-step action chunk",
        "ms_per_euler_step": round(ms_per_chunk / cfg.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.mlp_dtype == "bf16" else ("fp8+bf16" if cfg.mlp_dtype == "fp8" else "f32"),
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prefix KV and noise)",
        "config": {"workload": cfg.name, "layers": cfg.n_layers, "width": cfg.width, "heads": f"{cfg.n_q_heads}q/{cfg.n_kv_heads}kv",
                   "head_dim": cfg.head_dim, "mlp_dim": cfg.mlp_dim, "prefix_len": cfg.prefix_len,
                   "chunk": f"{cfg.horizon}x{cfg.action_dim}", "euler_steps": cfg.steps, "robots": B},
        "robot_steps_per_s": round(B * args.steps * cfg.steps / elapsed, 2),
        "chunk_ms_median": round(float(np.median(chunk_ms)), 4),
        "chunk_ms_p90": round(float(np.percentile(chunk_ms, 90)), 4),
        "step_alg_bytes": sb,
        "whole_chunk_GBs": round(sb * cfg.steps / (ms_per_chunk * 1e-3) / 1e9, 1),
        "whole_chunk_hbm_frac": round(sb * cfg.steps / (ms_per_chunk * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "step_flops": step_flops(cfg, B),
        "whole_chunk_mfma_frac": round(step_flops(cfg, B) * cfg.steps / (ms_per_chunk * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline_of(kernels, dom, traffic),
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, W, kvs[0][0], kvs[0][1], noise)
    ex.close()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
