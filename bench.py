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
                             "batched-paged", "ceiling", "layers32", "bernoulli-stats"])
    ap.add_argument("--n-k", type=int, default=131072, help="sweep workload: keys per sequence")
    ap.add_argument("--r", type=float, default=1.0, help="sweep workload: logit standard deviation")
    ap.add_argument("--mode", default="systematic", choices=["systematic", "stratified", "iid", "gumbel"])
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
    ap.add_argument("--deterministic", action="store_true",
                    help="sampling calls with the SANTA_DETERMINISTIC flag (exact sum, one rounding: bit-reproducible)")
    ap.add_argument("--seeds", type=int, default=2000, help="bernoulli-stats: sampling seeds per estimator")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="do not time the bare streaming read of the step's key bytes")
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


def cpu_baseline(wl, S, mode, seconds, nbytes, bernoulli=False, fp8_cache=None, budget=0, gpu_step=None):
    """Time the fp64 oracle on whole decode steps of the same workload (bounded);
    nbytes = the step's algorithmic bytes (the Bernoulli steps use seed 1, as
    the timed GPU steps do, so their kept features and bytes are the same).

    gpu_step = (indices, out) of the timed call's seed (1) on the GPU: the
    first oracle step uses that seed, and its result gives the index parity of
    the GPU's indices (exact, excused by the 1e-5 band at a CDF value, bad)
    and the largest output error: against the oracle's estimate on the GPU's
    index list (every head) and against the oracle's own output (heads whose
    indices all agree)."""
    from oracle import parity as OP
    from oracle import santa as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1

    parity = {}

    def one(seed, detail):
        if bernoulli:
            return O.bernoulli_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, 1, wl.scale, budget=budget,
                                      return_detail=detail)
        if fp8_cache is not None:
            return O.santa_decode_fp8k(wl.q, fp8_cache[0], fp8_cache[1], wl.V, wl.n_k, S, mode, seed, wl.scale,
                                       return_detail=detail)
        return O.santa_decode(wl.q, wl.K, wl.V, wl.n_k, S, mode, seed, wl.scale, return_detail=detail)

    def run(budget_s, first_parity):
        t0 = time.perf_counter()
        n = 0
        while True:
            res = one(1 if n == 0 else n, first_parity and n == 0 and gpu_step is not None)
            if first_parity and n == 0 and gpu_step is not None:
                parity.update(index_parity(res, gpu_step, wl, S, OP, O))
            n += 1
            if time.perf_counter() - t0 >= budget_s:
                return n, (time.perf_counter() - t0) / n

    n, per_step = run(seconds, True)
    res = {"value": nbytes / per_step / 1e12, "unit": "TB/s", "cores": threads, "kind": "oracle",
           "sample": "%d full decode step(s) of the same workload, %.2f s per step" % (n, per_step)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, per1 = run(seconds / 2, False)
        res["single_thread"] = {"value": nbytes / per1 / 1e12, "unit": "TB/s", "cores": 1,
                                "sample": "%d full decode step(s), %.2f s per step" % (n1, per1)}
    except ImportError:  # pragma: no cover
        pass
    return res, parity


def index_parity(oracle_res, gpu_step, wl, S, OP, O):
    """Index parity and output error of the GPU's step against the oracle's
    step on the same inputs and seed (see cpu_baseline)."""
    import numpy as np
    idx_g, out_g = gpu_step
    out_o, idx_o, det = oracle_res[0], oracle_res[1], oracle_res[-1]
    flips = set()
    rep = OP.compare_indices(idx_g, idx_o, det, 1e-5, flips)
    G = wl.Hq // wl.Hkv
    err_est, err_own = 0.0, 0.0
    for b in range(wl.B):
        n = int(wl.n_k[b])
        if not 1 <= n <= wl.max_n_k:
            continue
        for h in range(wl.Hq):
            est = O.gather_average(wl.V[b, h // G, :n].astype(np.float64), idx_g[b, h], S)
            err_est = max(err_est, float(np.abs(out_g[b, h] - est).max()))
            if (b, h) not in flips:
                err_own = max(err_own, float(np.abs(out_g[b, h] - out_o[b, h]).max()))
    return {"index_parity": dict(rep.as_dict(), band=1e-5),
            "out_max_abs_err": err_est, "out_max_abs_err_vs_oracle_output": err_own,
            "parity_heads_compared_with_oracle_output": wl.B * wl.Hq - rep.heads_with_flips}


def stream_ceiling(nbytes, sets_bytes, steps, warmup):
    """GB/s of the bare streaming read of `nbytes` bytes per launch (the best of
    1, 2 and 4 workgroups per CU), rotating over buffers that together hold
    sets_bytes, under the timed protocol of the decode step."""
    import torch

    from stochastic_sparse_decode_amd import santa
    nb = nbytes // 16 * 16
    R = max(1, int(math.ceil(sets_bytes / nb)))
    bufs = [torch.ones(nb // 2, dtype=torch.float16, device="cuda") for _ in range(R)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    best = None
    for wpc in (1, 2, 4):
        ms = timed(lambda b: santa.santa_stream_read(b, wpc, sink), bufs, steps, warmup)
        gbs = nb / (ms * 1e-3) / 1e9
        if best is None or gbs > best["GBs"]:
            best = {"GBs": gbs, "us_per_launch": ms * 1000.0, "workgroups_per_cu": wpc, "bytes": nb}
    return best


def layers32(args):
    """One token of attention through 32 Llama-3.1-8B-shaped layers (B=1,
    32/8 heads, d=128), each layer with its own 32k-key KV cache (4 GiB of KV
    in all, so no layer's keys are served from cache): 32 santa_decode calls
    (systematic, S=128), and the same with the dense kernel.  Only attention
    is timed: the projections and the MLP need model weights that are not
    here."""
    import numpy as np
    import torch

    from stochastic_sparse_decode_amd import santa
    from stochastic_sparse_decode_amd import workloads as W

    dev = torch.device("cuda:0")
    L = 32
    wl = W.llama(B=1, n_k=32768, seed=1001)
    q = torch.from_numpy(wl.q).to(dev)
    nk = torch.from_numpy(wl.n_k.astype(np.int32)).to(dev)
    K0 = torch.from_numpy(wl.K).to(dev)
    V0 = torch.from_numpy(wl.V).to(dev)
    layers = [(K0, V0)] + [(K0.clone(), V0.clone()) for _ in range(L - 1)]
    ws = santa.new_workspace(santa.problem(q, K0, wl.scale), dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)

    def token(dense):
        def fn(_):
            for i, (K, V) in enumerate(layers):
                if dense:
                    santa.santa_dense_decode(q, K, V, nk, wl.scale, out=out, workspace=ws)
                else:
                    santa.santa_decode(q, K, V, nk, 128, santa.SYSTEMATIC, 1 + i, wl.scale, out=out, workspace=ws,
                                       deterministic=args.deterministic)
        return fn

    steps = max(1, args.steps // L)
    ms_santa = timed(token(False), [None], steps, max(1, args.warmup // L))
    ms_dense = timed(token(True), [None], steps, max(1, args.warmup // L))
    assert santa.santa_workspace_error(ws) == 0
    nbytes = L * algorithmic_bytes(wl, 128)
    print(json.dumps({
        "metric": "attention us per token, 32 Llama-3.1-8B-shaped layers, 32k context each",
        "value": ms_santa * 1000.0, "unit": "us/token", "higher_is_better": False, "n_gpus": 1,
        "steps": steps, "warmup": max(1, args.warmup // L),
        "config": {"workload": "32 layers x (B=1, 32q/8kv, d=128, n_k=32768), systematic S=128, one KV cache per "
                               "layer", "parallelism": "none (1 GPU)"},
        "santa_us_per_token": ms_santa * 1000.0, "dense_us_per_token": ms_dense * 1000.0,
        "speedup_vs_dense": ms_dense / ms_santa,
        "santa_effective_TBs": nbytes / (ms_santa * 1e-3) / 1e12,
        "timing": "HIP graph of %d tokens (%d launches each), one timed replay" % (steps, L)}))


def bernoulli_stats(args):
    """Bias and variance of the Bernoulli qK^T step against exact-score SANTA
    and dense attention on the Bernoulli workload (B=8, n_k=32768, 32/8 heads,
    d=128, systematic S=128): `seeds` independent steps of each estimator (the
    seed drives both the ternary queries and the value sampling), their mean
    and per-coordinate variance over all B*H_q heads, against the dense output.
    bias = |mean - dense| (per-head Euclidean norm, averaged over heads),
    reported with its noise floor sqrt(sum of per-coordinate variances / seeds)
    (what |mean - E[out]| alone would typically give)."""
    import numpy as np
    import torch

    from stochastic_sparse_decode_amd import santa
    from stochastic_sparse_decode_amd import workloads as W

    dev = torch.device("cuda:0")
    wl = W.bernoulli(B=8, n_k=32768, seed=1004)
    q = torch.from_numpy(wl.q).to(dev)
    nk = torch.from_numpy(wl.n_k.astype(np.int32)).to(dev)
    K = torch.from_numpy(wl.K).to(dev)
    V = torch.from_numpy(wl.V).to(dev)
    K_fm = santa.santa_pack_k_feature_major(K)
    ws = santa.new_workspace(santa.problem(q, K, wl.scale), dev)
    out = torch.empty(q.shape, dtype=torch.float32, device=dev)
    dense = santa.santa_dense_decode(q, K, V, nk, wl.scale, workspace=ws).double()
    S, N = args.S, args.seeds
    kept = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    res = {"metric": "bias and variance of the Bernoulli qK^T estimate", "n_gpus": 1,
           "config": {"workload": "Bernoulli case B=8, n_k=32768, 32q/8kv, d=128, K,V,q ~ N(0,1)",
                      "mode": args.mode, "S": S, "seeds": N}, "estimators": {}}
    for name in ("bernoulli", "budget32", "exact_santa"):
        s1 = torch.zeros(q.shape, dtype=torch.float64, device=dev)
        s2 = torch.zeros_like(s1)
        kept_frac = 0.0
        for seed in range(N):
            if name == "exact_santa":
                santa.santa_decode(q, K, V, nk, S, santa.MODES[args.mode], seed, wl.scale, out=out, workspace=ws)
            else:
                santa.santa_bernoulli_qk(q, K_fm, V, nk, S, santa.MODES[args.mode], seed, wl.scale, out=out,
                                         kept=kept if seed < 64 else None, workspace=ws,
                                         budget=32 if name == "budget32" else 0)
                if seed < 64:
                    G = wl.Hq // wl.Hkv
                    kept_frac += kept.view(wl.B, wl.Hkv, G, wl.d).bool().any(dim=2).float().mean().item() / 64
            o = out.double()
            s1 += o
            s2 += o * o
        torch.cuda.synchronize()
        assert santa.santa_workspace_error(ws) == 0
        mean = s1 / N
        var = (s2 / N - mean * mean).clamp_min(0) * N / (N - 1)
        bias = (mean - dense).norm(dim=-1)            # per head
        floor = (var.sum(dim=-1) / N).sqrt()           # noise floor of |mean - E[out]| per head
        mse = ((s2 / N) - 2 * mean * dense + dense * dense).sum(dim=-1)  # E|out - dense|^2 per head
        e = {"bias_norm_mean": bias.mean().item(), "bias_norm_max": bias.max().item(),
             "bias_noise_floor_mean": floor.mean().item(),
             "bias_over_floor_mean": (bias / floor).mean().item(),
             "var_per_coord_mean": var.mean().item(), "mse_mean": mse.mean().item(),
             "dense_norm_mean": dense.norm(dim=-1).mean().item()}
        if name != "exact_santa":
            e["kept_feature_union_frac"] = kept_frac
        res["estimators"][name] = e
    print(json.dumps(res))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on a single GPU; --gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.workload == "layers32":
        layers32(args)
        return
    if args.workload == "bernoulli-stats":
        bernoulli_stats(args)
        return
    import numpy as np
    import torch

    from stochastic_sparse_decode_amd import santa
    from stochastic_sparse_decode_amd import workloads as W

    dev = torch.device("cuda:0")
    if args.workload == "ceiling":
        res = {"metric": "bare streaming read, GB/s per launch", "unit": "GB/s", "higher_is_better": True,
               "n_gpus": 1, "peak": HBM_PEAK_GBS, "sizes": {}}
        for mib in (32, 64, 256, 1024):
            res["sizes"]["%d MiB" % mib] = stream_ceiling(mib << 20, args.rotate_bytes * (1 << 30), args.steps,
                                                          args.warmup)
        print(json.dumps(res))
        return
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
                                                  out=out, workspace=ws, deterministic=args.deterministic)
    elif args.workload == "batched-paged":
        Kc, Vc, table, _ = W.paginate(wl.K, wl.V, wl.n_k, 256, seed=1)
        Kc0, Vc0 = torch.from_numpy(Kc).to(dev), torch.from_numpy(Vc).to(dev)
        tab = torch.from_numpy(table).to(dev)
        Rp = max(1, int(math.ceil(args.rotate_bytes * (1 << 30) / (2 * Kc0.numel() * 2))))
        sets = [(Kc0, Vc0)] + [(Kc0.clone(), Vc0.clone()) for _ in range(Rp - 1)]
        step = lambda kv: santa.santa_decode_paged(q, kv[0], kv[1], tab, nk, S, mode, 1, wl.scale,  # noqa: E731
                                                   out=out, workspace=ws, deterministic=args.deterministic)
    elif args.workload == "bernoulli":
        sets = [(santa.santa_pack_k_feature_major(k), v) for k, v in sets]
        step = lambda kv: santa.santa_bernoulli_qk(q, kv[0], kv[1], nk, S, mode, 1, wl.scale, out=out,  # noqa
                                                   workspace=ws, budget=args.budget, deterministic=args.deterministic)
    else:
        step = lambda kv: santa.santa_decode(q, kv[0], kv[1], nk, S, mode, 1, wl.scale, out=out,  # noqa: E731
                                             workspace=ws, deterministic=args.deterministic)
    spread = [] if not args.eager else None
    ms = timed(step, sets, args.steps, args.warmup, graph=not args.eager, spread=spread)
    assert santa.santa_workspace_error(ws) == 0
    # the graph's last step must equal an eager launch on the same KV copy
    last = out.clone()
    step(sets[(args.steps - 1) % len(sets)])
    torch.cuda.synchronize()
    if args.deterministic:  # exact sums: bit-identical
        if not torch.equal(last, out):
            d = last != out
            raise AssertionError("graph replay differs from eager launch: %d elements, max diff %g, heads %s, nan %d"
                                 % (int(d.sum()), float((last - out).abs().nan_to_num(0).max()),
                                    sorted(set(d.any(-1).nonzero()[:, 1].tolist()))[:16],
                                    int(torch.isnan(last).sum() + torch.isnan(out).sum())))
    else:  # outputs agree up to the order of the fp32 adds of the splits' shares
        assert (last - out).abs().max().item() <= 1e-5, "graph replay differs from eager launch"
    eager_ms = timed(step, sets, min(args.steps, 50), 2, graph=False) if not args.eager else ms
    if args.workload == "bernoulli":
        # the kept features of the timed steps (every step uses seed 1)
        kept = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        santa.santa_bernoulli_qk(q, sets[0][0], sets[0][1], nk, S, mode, 1, wl.scale, out=out, kept=kept,
                                 workspace=ws, budget=args.budget, deterministic=args.deterministic)
        torch.cuda.synchronize()
        nbytes = bernoulli_bytes(kept, wl, S)
    elif fp8k:
        nbytes = fp8k_bytes(wl, S)
    else:
        nbytes = algorithmic_bytes(wl, S)
    gbs = nbytes / (ms * 1e-3) / 1e9
    # the sampled indices of the timed call's seed (one untimed step with
    # indices): value-row counts here, index parity in the oracle leg
    idx = torch.empty((wl.B, q.shape[1], S), dtype=torch.int32, device=dev)
    out_idx = torch.empty_like(out)
    kv0 = sets[0]
    if fp8k:
        santa.santa_decode_fp8k(q, kv0[0], ks_d, kv0[1], nk, S, mode, 1, wl.scale, out=out_idx, indices=idx,
                                workspace=ws, deterministic=args.deterministic)
    elif args.workload == "batched-paged":
        santa.santa_decode_paged(q, kv0[0], kv0[1], tab, nk, S, mode, 1, wl.scale, out=out_idx, indices=idx,
                                 workspace=ws, deterministic=args.deterministic)
    elif args.workload == "bernoulli":
        santa.santa_bernoulli_qk(q, kv0[0], kv0[1], nk, S, mode, 1, wl.scale, out=out_idx, indices=idx,
                                 workspace=ws, budget=args.budget, deterministic=args.deterministic)
    else:
        santa.santa_decode(q, kv0[0], kv0[1], nk, S, mode, 1, wl.scale, out=out_idx, indices=idx, workspace=ws,
                           deterministic=args.deterministic)
    torch.cuda.synchronize()
    gpu_step = (idx.cpu().numpy(), last.cpu().numpy())  # indices, and the timed call's own output
    vrows = value_rows(idx.cpu(), wl.Hkv, wl.d) if args.workload != "bernoulli" else None
    ceiling = None
    if not args.no_ceiling:
        ceiling = stream_ceiling(nbytes, args.rotate_bytes * (1 << 30), args.steps, args.warmup)

    exact_ms = None
    if (args.workload in ("bernoulli", "batched-paged") or fp8k) and not args.no_dense:
        # the same step with exact scores on the fp16 cache (all of K, row-major)
        estep = lambda kv: santa.santa_decode(q, kv[0], kv[1], nk, S, mode, 1, wl.scale, out=out,  # noqa: E731
                                              workspace=ws, deterministic=args.deterministic)
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
    if ceiling is not None:
        # a bare streaming read of the same number of bytes per launch, same protocol
        res["roofline"]["ceiling"] = ceiling["GBs"]
        res["roofline"]["frac_of_ceiling"] = gbs / ceiling["GBs"]
        res["stream_read_ceiling"] = ceiling
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
        res["cpu_baseline"], parity = cpu_baseline(wl, S, mode, args.cpu_seconds, nbytes,
                                                   args.workload == "bernoulli", (K8, ks) if fp8k else None,
                                                   args.budget, gpu_step=gpu_step)
        res.update(parity)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
