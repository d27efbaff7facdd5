"""Benchmark: SANTA systematic decode step on a Llama-3.1-8B-shaped layer at 32k.

One step = one santa_decode call over the whole decode batch of one attention
layer (B=1, 32 query heads, 8 KV heads, d=128, n_k=32768, fp16 K/V with 1%
planted heavy hitters, systematic sampling, S=128).  Inputs are resident in
HBM before timing starts; steps rotate over R distinct copies of the KV cache
(like consecutive layers) so that the 256 MiB Infinity Cache cannot serve K
from a previous step.

value = effective HBM bandwidth in TB/s = algorithmic bytes / step time, where
the algorithmic bytes are all of K (B * H_kv * n_k * d * 2) plus S value rows
per KV head (B * H_kv * S * d * 2).  The dense split-K kernel of the same
library is timed under the same protocol for the speedup figure, and the CPU
oracle on a bounded sample of the same workload gives `cpu_baseline`.

Prints one JSON line.  ``--gpus N`` with N > 1 exits: this build runs on one GPU.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
SPREAD_REPLAYS = 20  # further timed replays of the step graph, for percentiles of the step time
SETTLE_MS = 50.0     # untimed replays of the step graph before the timed one
CSRC = os.path.join(ROOT, "stochastic_sparse_decode_amd", "csrc")
KERNEL_SOURCES = ("santa_decode.hip", "score_stage.h", "device_common.h", "launch.h")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "santa_decode_llama8b_32k_traffic.txt")


def kernel_source_hash():
    """sha256 over the sources of the decode kernel (ties counter data to a kernel version)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    if it is missing or was taken on a different version of the kernel."""
    try:
        vals = {}
        with open(TRAFFIC_PROFILE) as fh:
            for line in fh:
                if ":" in line and not line.startswith(" "):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
        if vals.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama32k",
                    choices=["llama32k", "batched", "sweep131k", "sweep", "bernoulli", "llama32k-fp8k",
                             "batched-paged"])
    ap.add_argument("--n-k", type=int, default=131072, help="sweep workload: keys per sequence")
    ap.add_argument("--r", type=float, default=1.0, help="sweep workload: logit standard deviation")
    ap.add_argument("--mode", default="systematic", choices=["systematic", "stratified", "iid"])
    ap.add_argument("--S", type=int, default=128)
    ap.add_argument("--budget", type=int, default=0,
                    help="Bernoulli workload: 0 = ternary queries, m > 0 = the budget variant with m features")
    ap.add_argument("--rotate-bytes", type=float, default=2.0, help="GiB of distinct KV copies to rotate over")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python instead of a HIP graph")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for HBM counter calibration)")
    ap.add_argument("--steps-model", type=int, default=10)
    ap.add_argument("--model-step", action="store_true",
                    help="only time a synthetic 32-layer Llama-3.1-8B decode step (B=1, 32k context): attention "
                         "by SANTA or by the dense kernel, projections and MLP by torch matmuls on random weights")
    return ap.parse_args()


def make_workload(name, n_k=131072, r=1.0):
    from stochastic_sparse_decode_amd import workloads as W
    if name == "llama32k":
        return W.llama(B=1, n_k=32768, seed=1001), "Llama-3.1-8B decode layer, B=1, 32q/8kv, d=128, n_k=32768"
    if name == "llama32k-fp8k":
        return (W.llama(B=1, n_k=32768, seed=1001),
                "Llama-3.1-8B decode layer, B=1, 32q/8kv, d=128, n_k=32768, fp8 (OCP E4M3) key cache")
    if name == "batched-paged":
        return (W.llama(B=16, n_k_range=(8192, 32768), seed=1002),
                "Llama-3.1-8B decode layer, B=16, n_k~U[8192,32768], 32q/8kv, d=128, paged cache (256-key blocks, "
                "shuffled placement)")
    if name == "batched":
        return (W.llama(B=16, n_k_range=(8192, 32768), seed=1002),
                "Llama-3.1-8B decode layer, B=16, n_k~U[8192,32768], 32q/8kv, d=128")
    if name == "sweep131k":
        return W.sweep(B=4, n_k=131072, r=1.0, seed=1003), "context sweep B=4, n_k=131072, r=1, 32q/8kv, d=128"
    if name == "sweep":
        return (W.sweep(B=4, n_k=n_k, r=r, seed=1003),
                "context sweep B=4, n_k=%d, r=%g, 32q/8kv, d=128" % (n_k, r))
    return W.bernoulli(B=8, n_k=32768, seed=1004), "Bernoulli case B=8, n_k=32768, 32q/8kv, d=128"


def bernoulli_bytes(kept, wl, S):
    """Bytes a Bernoulli step must read: for each (sequence, KV head) the
    union of its G heads' kept features over all n_k keys (2 bytes each),
    plus S value rows per KV head."""
    G = wl.Hq // wl.Hkv
    union = kept.view(wl.B, wl.Hkv, G, wl.d).bool().any(dim=2).sum(dim=2).cpu().numpy()  # [B][H_kv]
    k_bytes = int((union.astype("int64") * wl.n_k.astype("int64")[:, None]).sum()) * 2
    return k_bytes + wl.B * wl.Hkv * S * wl.d * 2


def fp8k_bytes(wl, S):
    """Bytes of a step on an fp8 key cache: one byte per key element plus S
    fp16 value rows per KV head (the per-head key scales are negligible)."""
    return int(wl.n_k.astype("int64").sum()) * wl.Hkv * wl.d + wl.B * wl.Hkv * S * wl.d * 2


def algorithmic_bytes(wl, S, dense=False):
    k_bytes = int(wl.n_k.astype("int64").sum()) * wl.Hkv * wl.d * 2
    if dense:
        return 2 * k_bytes
    return k_bytes + wl.B * wl.Hkv * S * wl.d * 2


def value_rows(indices, Hkv, d):
    """V-row counts of one step from its sampled indices (B, H_q, S): the S rows
    per KV head the byte count assumes, the G*S rows if every query head read
    its own, and the distinct (sequence, KV head, key) rows actually sampled.
    Indices of -1 (an invalid length) are not rows."""
    import torch
    B, Hq, S = indices.shape
    per_kv = indices.reshape(B, Hkv, (Hq // Hkv) * S).to(torch.int64)
    srt = torch.sort(per_kv, dim=-1).values
    valid = srt >= 0
    first = torch.ones_like(valid)
    first[..., 1:] = srt[..., 1:] != srt[..., :-1]
    distinct = int((first & valid).sum().item())
    return {"S_per_kv_head": B * Hkv * S, "G_S_rows": B * Hq * S, "distinct_measured": distinct,
            "distinct_bytes": distinct * d * 2}


def timed(fn, sets, steps, warmup, graph=True, spread=None):
    """ms per step over exactly `steps` steps, rotating over the KV copies.

    With graph=True the `steps` launches are captured once into a HIP graph
    and the timed region is one replay, so host-side launch overhead (Python,
    ctypes) is not part of the measurement; the events are recorded on the
    stream the kernels run on.  With graph=False every step is launched from
    Python.  With a list in `spread` (graph=True), SPREAD_REPLAYS further
    replays are timed one by one after the timed one and their ms per step
    are left in it (for percentiles; the returned value is the timed replay's).
    """
    import torch
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(sets[i % len(sets)])
        # untimed replays for at least SETTLE_MS of GPU work: the first
        # milliseconds of work in a process run up to 5% slower per step
        t0 = time.perf_counter()
        for _ in range(200):
            g.replay()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= SETTLE_MS * 1e-3:
                break
        stream = torch.cuda.current_stream()
        start.record(stream)
        g.replay()
        stop.record(stream)
        if spread is not None:
            for _ in range(SPREAD_REPLAYS):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                g.replay()
                e1.record(stream)
                spread.append((e0, e1))
    else:
        stream = torch.cuda.current_stream()
        start.record(stream)
        for i in range(steps):
            fn(sets[i % len(sets)])
        stop.record(stream)
    torch.cuda.synchronize()
    if spread is not None:
        spread[:] = [e0.elapsed_time(e1) / steps for e0, e1 in spread]
    return start.elapsed_time(stop) / steps  # ms per step (= per launch: one launch per step)


def cpu_baseline(wl, S, mode, seconds, nbytes, bernoulli=False, fp8_cache=None, budget=0):
    """Time the fp64 oracle on whole decode steps of the same workload (bounded);
    nbytes = the step's algorithmic bytes (the Bernoulli steps use seed 1, as
    the timed GPU steps do, so their kept features and bytes are the same)."""
    from oracle import santa as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1

    def run(budget_s):
        t0 = time.perf_counter()
        n = 0
        while True:
            if bernoulli:
                O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, 1, wl.scale, budget=budget)
            elif fp8_cache is not None:
                O.santa_decode_fp8k(wl.q, fp8_cache[0], fp8_cache[1], wl.V, wl.n_k, S, mode, n, wl.scale)
            else:
                O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, n, wl.scale)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                return n, (time.perf_counter() - t0) / n

    n, per_step = run(seconds)
    res = {"value": nbytes / per_step / 1e12, "unit": "TB/s", "cores": threads, "kind": "oracle",
           "sample": "%d full decode step(s) of the same workload, %.2f s per step" % (n, per_step)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, per1 = run(seconds / 2)
        res["single_thread"] = {"value": nbytes / per1 / 1e12, "unit": "TB/s", "cores": 1,
                                "sample": "%d full decode step(s), %.2f s per step" % (n1, per1)}
    except ImportError:  # pragma: no cover
        pass
    return res


def model_step(args):
    """Synthetic decode step of a 32-layer Llama-3.1-8B-shaped model at B=1
    with a 32k context in every layer: per layer the fused QKV projection,
    attention over that layer's own KV cache (SANTA systematic S=128, or the
    dense kernel), the output projection and the gated MLP (torch matmuls,
    random fp16 weights; norms, rotary embedding and the cache append are left
    out: they move a few KiB).  Reports the token latency with each attention
    and the share attention takes of it."""
    import numpy as np
    import torch

    from stochastic_sparse_decode_amd import santa
    from stochastic_sparse_decode_amd import workloads as W

    dev = torch.device("cuda:0")
    L, hid, inter, Hq, Hkv, d, n_k = 32, 4096, 14336, 32, 8, 128, 32768
    wl = W.llama(B=1, n_k=n_k, seed=1001)
    g = torch.Generator(device=dev).manual_seed(7)

    def weight(rows, cols):
        return (torch.randn(rows, cols, generator=g, device=dev, dtype=torch.float16) / math.sqrt(rows)).contiguous()

    layers = []
    K0 = torch.from_numpy(wl.K).to(dev)
    V0 = torch.from_numpy(wl.V).to(dev)
    for _ in range(L):
        layers.append(dict(wqkv=weight(hid, (Hq + 2 * Hkv) * d), wo=weight(Hq * d, hid), wg=weight(hid, inter),
                           wu=weight(hid, inter), wd=weight(inter, hid), K=K0.clone(), V=V0.clone()))
    nk = torch.from_numpy(wl.n_k.astype(np.int32)).to(dev)
    q_probe = torch.from_numpy(wl.q).to(dev)  # the query when projections are left out
    ws = santa.new_workspace(santa.problem(q_probe, K0, wl.scale), dev)
    att = torch.empty((1, Hq, d), dtype=torch.float32, device=dev)
    x0 = torch.randn(1, hid, generator=g, device=dev, dtype=torch.float16)

    def attention(lay, q, dense):
        if dense:
            santa.santa_dense_decode(q, lay["K"], lay["V"], nk, wl.scale, out=att, workspace=ws)
        else:
            santa.santa_decode(q, lay["K"], lay["V"], nk, 128, 2, 1, wl.scale, out=att, workspace=ws)
        return att

    def step(dense=False, attn=True, other=True):
        x = x0
        q = q_probe
        for lay in layers:
            if other:
                qkv = x @ lay["wqkv"]
                q = qkv[:, :Hq * d].view(1, Hq, d)
            if attn:
                a = attention(lay, q, dense)
            if other:
                src = a.view(1, Hq * d).to(torch.float16) if attn else qkv[:, :Hq * d]
                x = x + src @ lay["wo"]
                h = torch.nn.functional.silu(x @ lay["wg"]) * (x @ lay["wu"])
                x = x + h @ lay["wd"]
        return x

    def timed_step(**kw):
        for _ in range(3):
            step(**kw)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(args.steps_model):
                step(**kw)
        gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        e0.record(st)
        gr.replay()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps_model * 1000.0  # us per token

    full_santa = timed_step(dense=False)
    full_dense = timed_step(dense=True)
    att_santa = timed_step(dense=False, other=False)
    att_dense = timed_step(dense=True, other=False)
    other = timed_step(attn=False)
    assert santa.santa_workspace_error(ws) == 0
    print(json.dumps({"model_step": {
        "model": "Llama-3.1-8B shape, 32 layers, random fp16 weights", "batch": 1, "context": n_k,
        "us_per_token_santa": full_santa, "us_per_token_dense": full_dense,
        "attention_us_santa": att_santa, "attention_us_dense": att_dense, "non_attention_us": other,
        "attention_share_santa": att_santa / full_santa, "attention_share_dense": att_dense / full_dense,
        "token_speedup_santa_vs_dense": full_dense / full_santa,
        "timing": "HIP graph of %d whole decode steps, one timed replay" % args.steps_model}}))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on a single GPU; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.model_step:
        model_step(args)
        return
    import numpy as np
    import torch

    from stochastic_sparse_decode_amd import santa
    from stochastic_sparse_decode_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": 1 << 30, "dispatches": 5}))
        return

    mode = santa.MODES[args.mode]
    wl, desc = make_workload(args.workload, args.n_k, args.r)
    q = torch.from_numpy(wl.q).to(dev)
    nk = torch.from_numpy(wl.n_k.astype(np.int32)).to(dev)
    K0 = torch.from_numpy(wl.K).to(dev)
    V0 = torch.from_numpy(wl.V).to(dev)
    set_bytes = 2 * K0.numel() * 2
    R = max(1, int(math.ceil(args.rotate_bytes * (1 << 30) / set_bytes)))
    sets = [(K0, V0)] + [(K0.clone(), V0.clone()) for _ in range(R - 1)]
    prob = santa.problem(q, K0, wl.scale)
    ws = santa.new_workspace(prob, dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    S = args.S

    rm_sets = sets  # row-major fp16 K
    fp8k = args.workload == "llama32k-fp8k"
    if fp8k:
        K8, ks = W.quantize_keys_fp8(wl.K, wl.n_k)
        K80 = torch.from_numpy(K8).to(dev)
        ks_d = torch.from_numpy(ks).to(dev)
        R8 = max(1, int(math.ceil(args.rotate_bytes * (1 << 30) / (K80.numel() + V0.numel() * 2))))
        sets = [(K80, V0)] + [(K80.clone(), V0.clone()) for _ in range(R8 - 1)]
        step = lambda kv: santa.santa_decode_fp8k(q, kv[0], ks_d, kv[1], nk, S, mode, 1, wl.scale,  # noqa: E731
                                                  out=out, workspace=ws)
    elif args.workload == "batched-paged":
        Kc, Vc, table, _ = W.paginate(wl.K, wl.V, wl.n_k, 256, seed=1)
        Kc0, Vc0 = torch.from_numpy(Kc).to(dev), torch.from_numpy(Vc).to(dev)
        tab = torch.from_numpy(table).to(dev)
        Rp = max(1, int(math.ceil(args.rotate_bytes * (1 << 30) / (2 * Kc0.numel() * 2))))
        sets = [(Kc0, Vc0)] + [(Kc0.clone(), Vc0.clone()) for _ in range(Rp - 1)]
        step = lambda kv: santa.santa_decode_paged(q, kv[0], kv[1], tab, nk, S, mode, 1, wl.scale,  # noqa: E731
                                                   out=out, workspace=ws)
    elif args.workload == "bernoulli":
        sets = [(santa.santa_pack_k_feature_major(k), v) for k, v in sets]
        step = lambda kv: santa.santa_bernoulli_qk(q, kv[0], kv[1], nk, S, mode, 1, wl.scale, out=out,  # noqa
                                                   workspace=ws, budget=args.budget)
    else:
        step = lambda kv: santa.santa_decode(q, kv[0], kv[1], nk, S, mode, 1, wl.scale, out=out,  # noqa: E731
                                             workspace=ws)
    spread = [] if not args.eager else None
    ms = timed(step, sets, args.steps, args.warmup, graph=not args.eager, spread=spread)
    assert santa.santa_workspace_error(ws) == 0
    # the graph's last step must equal an eager launch on the same KV copy
    last = out.clone()
    step(sets[(args.steps - 1) % len(sets)])
    torch.cuda.synchronize()
    # outputs agree up to the order of the fp32 adds of the splits' shares
    assert (last - out).abs().max().item() <= 1e-5, "graph replay differs from eager launch"
    eager_ms = timed(step, sets, min(args.steps, 50), 2, graph=False) if not args.eager else ms
    if args.workload == "bernoulli":
        # the kept features of the timed steps (every step uses seed 1)
        kept = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        santa.santa_bernoulli_qk(q, sets[0][0], sets[0][1], nk, S, mode, 1, wl.scale, out=out, kept=kept,
                                 workspace=ws, budget=args.budget)
        torch.cuda.synchronize()
        nbytes = bernoulli_bytes(kept, wl, S)
    elif fp8k:
        nbytes = fp8k_bytes(wl, S)
    else:
        nbytes = algorithmic_bytes(wl, S)
    gbs = nbytes / (ms * 1e-3) / 1e9
    vrows = None
    if args.workload in ("llama32k", "batched", "sweep131k", "sweep"):
        # the sampled rows of one step (untimed, same seed as the timed steps)
        idx = torch.empty((wl.B, q.shape[1], S), dtype=torch.int32, device=dev)
        santa.santa_decode(q, sets[0][0], sets[0][1], nk, S, mode, 1, wl.scale, out=out, indices=idx,
                           workspace=ws)
        torch.cuda.synchronize()
        vrows = value_rows(idx.cpu(), wl.Hkv, wl.d)

    exact_ms = None
    if (args.workload in ("bernoulli", "batched-paged") or fp8k) and not args.no_dense:
        # the same step with exact scores on the fp16 cache (all of K, row-major)
        estep = lambda kv: santa.santa_decode(q, kv[0], kv[1], nk, S, mode, 1, wl.scale, out=out,  # noqa: E731
                                              workspace=ws)
        exact_ms = timed(estep, rm_sets, args.steps, args.warmup, graph=not args.eager)
    dense_ms = None
    if not args.no_dense and args.workload != "bernoulli":
        dstep = lambda kv: santa.santa_dense_decode(q, kv[0], kv[1], nk, wl.scale, out=out, workspace=ws)  # noqa
        dense_ms = timed(dstep, rm_sets, args.steps, args.warmup, graph=not args.eager)

    res = {
        "metric": "decode-attention us/step + effective HBM TB/s (% peak), Llama-3.1-8B shape @32k",
        "value": gbs / 1000.0,
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": ms * 1000.0,
        "pct_hbm_peak": 100.0 * gbs / HBM_PEAK_GBS,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f8 (E4M3) keys, f16 q and values, f32 accumulate" if fp8k else "f16 in, f32 accumulate",
        "data": "synthetic (seeded; rotated over %d KV copies, %.2f GiB)" % (R, R * set_bytes / (1 << 30)),
        "config": {"workload": desc + (", budget %d features" % args.budget if args.budget else ""),
                   "mode": args.mode, "S": S, "global_batch": wl.B, "seq_len": int(wl.n_k.max()),
                   "parallelism": "none (1 GPU)"},
        "algorithmic_bytes_per_step": nbytes,
        "timing": "HIP graph of %d steps, one timed replay" % args.steps if not args.eager else "eager launches",
        "eager_us_per_step": eager_ms * 1000.0,
        "replay_us_per_step": ({"replays": len(spread), "mean": float(np.mean(spread)) * 1000.0,
                                "p10": float(np.percentile(spread, 10)) * 1000.0,
                                "p50": float(np.percentile(spread, 50)) * 1000.0,
                                "p90": float(np.percentile(spread, 90)) * 1000.0} if spread else None),
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic() if args.workload == "llama32k" and args.mode == "systematic"
                     and S == 128 else None},
    }
    if vrows is not None:
        res["value_rows"] = vrows
    if exact_ms is not None:
        key = {"llama32k-fp8k": "fp16_santa", "batched-paged": "contiguous_santa"}.get(args.workload, "exact_santa")
        res[key] = {"us_per_step": exact_ms * 1000.0,
                    "effective_GBs": algorithmic_bytes(wl, S) / (exact_ms * 1e-3) / 1e9}
        res["speedup_vs_" + key] = exact_ms / ms
    if dense_ms is not None:
        dbytes = algorithmic_bytes(wl, S, dense=True)
        res["dense"] = {"us_per_step": dense_ms * 1000.0, "effective_GBs": dbytes / (dense_ms * 1e-3) / 1e9,
                        "pct_hbm_peak": 100.0 * dbytes / (dense_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        res["speedup_vs_dense"] = dense_ms / ms
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, S, mode, args.cpu_seconds, nbytes, args.workload == "bernoulli",
                                           (K8, ks) if fp8k else None, args.budget)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
