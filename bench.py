"""Benchmark: RACE attention layer forward + backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]

One step = race_attn_fwd (bucket reduce, bank sums, readout) followed by
race_attn_bwd (Q-side gradients with the gradient-bank reduce, bank sums,
K/V-side gradients) over one batch of seeded synthetic inputs already
resident in HBM.  Default workload: non-causal, B=1, H=4, N=12,000,000,
d=128, P=4, L=2, beta=4, bf16 I/O with float32 accumulation.

Prints one JSON line.  ``roofline`` covers the kernel with the largest share
of the timed region: algorithmic bytes per launch (the token rows it must
read and write) over its mean launch time, measured with HIP events that the
library records on the launch stream during the timed steps.  ``traffic``
comes from committed rocprofv3 FETCH_SIZE / WRITE_SIZE counts of that kernel
(scaled by a plain copy kernel's counts), or null when the kernel sources
changed since they were taken.  ``cpu_baseline`` times the fp64 oracle on a
bounded sample on this host.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s

# bytes of token rows each kernel must move, per (token, head), in units of d * elem_size
ROW_PASSES = {
    "race_bucket_reduce": 2,   # read K, V
    "race_readout_norm": 2,    # read Q, write O
    "race_bwd_q": 3,           # read Q, dO, write dQ
    "race_bwd_kv": 4,          # read K, V, write dK, dV
    "race_causal_segsum": 2,   # read K, V
    "race_causal_fwd": 4,      # read Q, K, V, write O
    "race_causal_h": 4,        # read Q, K, V, dO (backward without O)
    "race_causal_h_from_o": 2, # read dO, O
    "race_causal_gradsum": 2,  # read Q, dO
    "race_causal_dv": 4,       # read K, Q, dO, write dV
    "race_causal_dq": 5,       # read Q, K, V, dO, write dQ
    "race_causal_dk": 5,       # read K, Q, dO, V, write dK
    "race_static_fwd": 2,      # read Q, write O (one fixed bank)
    "race_static_h": 2,        # read Q, dO
    "race_static_dv": 2,       # read K, write dV
    "race_static_dq": 3,       # read Q, dO, write dQ
    "race_static_dk": 3,       # read K, V, write dK
}


# algorithmic flops per (token, head) of the causal walks' contractions, with
# LR = L * 2^P buckets: the bank read out or contracted over columns (2 LR d),
# the bank update (2 LR (d + 1)), and for the transposed walks dX = dPre W
# (2 L P d); the chunked intra terms and the soft assignments are not counted.
# The static-bank walks (non-causal layer, wide tables) have no bank update.
def causal_flops(kernel: str, L: int, P: int, d: int):
    LR = L << P
    upd = 2 * LR * (d + 1)
    return {"race_causal_segsum": upd, "race_causal_gradsum": upd,
            "race_causal_fwd": 2 * LR * (d + 1) + upd, "race_causal_h": 2 * LR * (d + 1) + upd,
            "race_causal_dv": 2 * LR * d + upd,
            "race_causal_dq": 2 * LR * d + upd + 2 * L * P * d,
            "race_causal_dk": 2 * LR * d + upd + 2 * L * P * d,
            "race_static_fwd": 2 * LR * (d + 1), "race_static_h": 2 * LR * (d + 1),
            "race_static_dv": 2 * LR * d,
            "race_static_dq": 2 * LR * d + 2 * L * P * d,
            "race_static_dk": 2 * LR * d + 2 * L * P * d}.get(kernel)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "linear_attention_soft_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=None,
                    help="workload key (default 4; with --decode, 2)")
    ap.add_argument("--decode", action="store_true",
                    help="time the recurrent decode step instead: one new token per sequence per step from a "
                         "state prefilled with the workload's N tokens")
    ap.add_argument("--decode-batch", type=int, default=None, help="batch rows for --decode (default: workload's)")
    ap.add_argument("--decode-prompt", type=int, default=4096,
                    help="prompt tokens prefilled before --decode (the state size does not depend on it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dbeta", action="store_true",
                    help="also compute dL/dbeta in every backward (beta learned)")
    ap.add_argument("--dW", action="store_true",
                    help="also compute dL/dW in every backward (tables learned)")
    ap.add_argument("--per-head", action="store_true",
                    help="one set of tables per head (W is [H][L][P][d])")
    ap.add_argument("--P", type=int, default=None,
                    help="hyperplanes per table instead of the workload's (e.g. the scaling settings (2, 2), (3, 3), "
                         "(4, 4) of the single-layer runs at d = 128)")
    ap.add_argument("--L", type=int, default=None, help="tables instead of the workload's")
    ap.add_argument("--variant", choices=("causal", "noncausal"), default=None,
                    help="the other variant of the workload's layer (e.g. the non-causal layer at P = 6, L = 4)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=None,
                    help="oracle sample length (default: sized for about 20 s of CPU work)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the same step captured once in a HIP graph and replayed")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after timing, copy 1 GiB once (reference kernel for rocprofv3 byte counters)")
    return ap.parse_args()


def cpu_baseline(inp, w, n_tok=None, target_s=20.0):
    """fp64 oracle on head (0, 0)'s first n tokens taken as one sequence
    (forward, plus backward for training workloads).

    n is n_tok when given; otherwise probes of 256, 1024, 4096, ... tokens
    run until one takes an eighth of target_s, and n is scaled from it so that
    one pass takes about target_s seconds (the causal oracle keeps a bank per
    token and costs ~1000x more per token than the non-causal one).  Samples
    shorter than a second are repeated until a second has passed.  A token of
    the metric carries all H heads, so the rate is scaled by 1/H: the whole
    job would take H times the sample's time per token."""
    from oracle import race_oracle as orc
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    Wn = inp["W"].double().numpy()
    train = "bwd" in w.phases

    def run(n):
        f64 = lambda t: t[0, 0, :n].to("cpu").double().numpy()
        Q, K, V = (f64(inp[k]) for k in ("Q", "K", "V"))
        dO = f64(inp["dO"]) if train else None
        t0 = time.perf_counter()
        if w.causal:
            orc.causal_forward_head(Q, K, V, Wn, w.beta)
        else:
            orc.forward_head(Q, K, V, Wn, w.beta)
        if train:
            orc.backward_head(Q, K, V, Wn, w.beta, dO, w.causal)
        return time.perf_counter() - t0

    if n_tok is None:
        cap = min(w.N, 1 << 22)
        probe = min(cap, 256)
        t_probe = run(probe)
        while t_probe < target_s / 8 and probe < cap:
            probe = min(cap, 4 * probe)
            t_probe = run(probe)
        n = min(cap, max(probe, int(probe * target_s / max(t_probe, 1e-6)) // 256 * 256))
    else:
        n = min(n_tok, w.N)
    print(f"# oracle sample: {n} tokens of head (0,0)", file=sys.stderr, flush=True)
    reps, dt = 0, 0.0
    while reps == 0 or dt < 1.0:
        dt += run(n)
        reps += 1
    ph = "fwd+bwd" if train else "fwd"
    whole = n >= w.N and w.B * w.H == 1
    return {"value": n * reps / (dt * w.H), "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "extrapolated": not whole,
            "sample": f"head (0,0), first {n} of {w.N} tokens as one sequence, {ph} fp64 numpy, {reps} pass(es) "
                      f"in {dt:.2f} s; value extrapolated to the whole workload ({w.B} x {w.H} sequences of "
                      f"{w.N} tokens) as sample tokens / (H = {w.H} heads per token x sample time)"
                      if not whole else
                      f"the whole workload, {ph} fp64 numpy, {reps} pass(es) in {dt:.2f} s"}


def load_traffic(workload_name: str, kernel: str, launches_tokens: int):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_hash") != source_hash():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k:
        return None
    return float(k["bytes_per_launch"])


def bench_decode(args):
    """Decode steps: every (batch, head) sequence takes one new token per step
    (update-then-read on its fixed-size bank), inputs resident in HBM.  The
    timed steps replay a HIP graph of 16 captured steps; the per-call rate
    of the same steps launched one by one is reported beside it."""
    import torch
    import linear_attention_soft_amd as race
    import race_inputs as ri

    w = ri.WORKLOADS[2 if args.workload is None else args.workload]
    w = w.with_size(N=min(w.N, args.decode_prompt), B=args.decode_batch or w.B)
    dev = "cuda"
    steps, n_new = args.steps * 10, 1
    print(f"# decode on {w.name}: prompt of {w.N} tokens, {steps} steps of {n_new} token", file=sys.stderr,
          flush=True)
    prompt = ri.make_inputs(w, device=dev)
    W = prompt["W"].to(dev)
    st = race.race_attn_decode_prefill(prompt["K"], prompt["V"], W, w.beta, w.P, w.L)
    nw = w.with_size(N=(args.warmup + steps) * n_new)
    new = ri.make_inputs(nw, device=dev, seed_base=7000 + w.key)
    toks = [{k: new[k][:, :, i * n_new:(i + 1) * n_new].contiguous() for k in ("Q", "K", "V")}
            for i in range(args.warmup + steps)]
    O = torch.empty_like(toks[0]["Q"])
    race.profile_enable(False)
    for i in range(args.warmup):
        race.race_attn_decode(toks[i]["Q"], toks[i]["K"], toks[i]["V"], W, w.beta, w.P, w.L, st, O=O)
    torch.cuda.synchronize()
    race.profile_reset()
    race.profile_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.warmup, args.warmup + steps):
        race.race_attn_decode(toks[i]["Q"], toks[i]["K"], toks[i]["V"], W, w.beta, w.P, w.L, st, O=O)
    e1.record()
    torch.cuda.synchronize()
    race.profile_enable(False)
    eager_ms = e0.elapsed_time(e1) / steps
    kern = race.profile_report()
    cnt, tot = kern.get("race_decode", (1, eager_ms))
    avg_ms = tot / cnt
    # the same kind of steps captured in a HIP graph of G steps and replayed:
    # a serving loop pays one launch per G tokens instead of one per token
    G = 16
    reps = max(1, steps // G)
    Ob = torch.empty_like(O)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(G):
            t = toks[args.warmup + i % steps]
            race.race_attn_decode(t["Q"], t["K"], t["V"], W, w.beta, w.P, w.L, st, O=Ob)
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (reps * G)
    s = 2 if w.dtype == "bf16" else 4
    state_bytes = st.numel() * 4
    alg = 2 * state_bytes + 4 * w.B * w.H * n_new * w.d * s   # state read + write; q, k, v, o rows
    # one launch per step inside the graph: its average duration over the
    # timed region (the event-bracketed eager launches carry the events' own cost)
    achieved = alg / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "RACE decode tokens/s (one new token per sequence per step, fixed-size state)",
        "value": w.B * n_new / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": reps * G,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (seeded)",
        "config": {"workload": "decode_" + w.name, "B": w.B, "H": w.H, "prompt_tokens": w.N, "d": w.d, "P": w.P,
                   "L": w.L, "beta": w.beta, "new_tokens_per_step": n_new, "state_bytes": state_bytes,
                   "launch": f"HIP graph of {G} steps, replayed"},
        "eager_ms_per_step": eager_ms,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "race_decode",
                     "alg_bytes_per_launch": alg, "avg_launch_ms": ms_step, "eager_event_launch_ms": avg_ms},
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported (across GPUs the "
              f"layer would shard by heads, or by sequence segments with one all-reduce of the banks)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import linear_attention_soft_amd as race
    import race_inputs as ri

    if args.decode:
        return bench_decode(args)
    w = ri.WORKLOADS[4 if args.workload is None else args.workload]
    if args.P is not None or args.L is not None:
        from dataclasses import replace
        P = w.P if args.P is None else args.P
        L = w.L if args.L is None else args.L
        w = replace(w, P=P, L=L, name=f"{w.name}_p{P}l{L}")
    if args.variant is not None and (args.variant == "causal") != w.causal:
        from dataclasses import replace
        w = replace(w, causal=args.variant == "causal", name=f"{w.name}_as_{args.variant}")
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    race.lib()
    dev = "cuda"
    print(f"# workload {w.name}: generating inputs on the GPU", file=sys.stderr, flush=True)
    inp = ri.make_inputs(w, device=dev, with_grad_out=True)
    Q, K, V, dO = inp["Q"], inp["K"], inp["V"], inp["dO"]
    W = (ri.make_W_per_head(w) if args.per_head else inp["W"]).to(dev)
    O = torch.empty_like(Q)
    dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    shape = race._shape_of(Q, W, w.L, w.P)
    st = torch.empty(race.race_attn_state_bytes(shape, w.P, w.L, w.causal), dtype=torch.uint8, device=dev)
    wsf = torch.empty(race.race_attn_workspace_bytes(shape, w.P, w.L, w.causal, False), dtype=torch.uint8, device=dev)
    wsb = torch.empty(race.race_attn_workspace_bytes(shape, w.P, w.L, w.causal, 2 if args.dW else 1),
                      dtype=torch.uint8, device=dev)
    db = torch.zeros(1, dtype=torch.float32, device=dev)
    dW = torch.zeros_like(W) if args.dW else None
    torch.cuda.synchronize()
    # forward-only workloads (the pages' inference-shaped runs) time the forward alone
    train = "bwd" in w.phases

    def step():
        race.race_attn_fwd(Q, K, V, W, w.beta, w.P, w.L, w.causal, O=O, state=st, workspace=wsf)
        if train:
            race.race_attn_bwd(Q, K, V, W, w.beta, w.P, w.L, w.causal, dO, st, O=O, dQ=dQ, dK=dK, dV=dV,
                               dbeta=db if args.dbeta else None, dW=dW, workspace=wsb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps); timing {args.steps} steps", file=sys.stderr, flush=True)

    race.profile_reset()
    race.profile_enable(True)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    race.profile_enable(False)
    kern = race.profile_report()
    ms_step = e0.elapsed_time(e1) / args.steps
    tokens = w.B * w.N
    value = tokens * args.steps / (max(ms_step * args.steps, wall * 1e3) * 1e-3)

    elem = 2 if w.dtype == "bf16" else 4
    row_bytes = w.B * w.H * w.N * w.d * elem
    dom = max(kern.items(), key=lambda kv: kv[1][1])
    dname, (dl, dms) = dom
    avg_ms = dms / dl
    alg_bytes = ROW_PASSES.get(dname, 0) * row_bytes
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    traffic = load_traffic(w.name, dname, tokens)

    # the runtime's own 1 GiB device copy, timed in the same run: the stream
    # rate a read + write kernel reaches on this part (context for frac)
    src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(5):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * src.numel() * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    if args.calibrate_copy:
        dst.copy_(src)
        torch.cuda.synchronize()
    del src, dst

    graph_ms = None
    if args.graph:
        # the same step captured once and replayed: the launch cost per step
        # drops to one graph launch (the library enqueues kernels only)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        del g

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the fp64 oracle on a CPU sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(inp, w, args.cpu_sample_tokens)

    if w.key == 4 and args.P is None and args.L is None and args.variant in (None, "noncausal"):
        metric = "RACE layer fwd+bwd tokens/s at N=12M, H=4, d=128; % of HBM roofline"
    else:
        metric = f"RACE layer {'fwd+bwd' if train else 'fwd'} tokens/s, workload {w.name}; % of HBM roofline"
    dist = {"iid": "iid N(0,1) Q, K, V, dO", "iid_over_sqrt_d": "iid N(0,1)/sqrt(d) Q, K, V",
            "lognormal_norms": "rows with isotropic directions and log-uniform norms in [0.5, 2]; iid dO",
            "clustered_keys": "K around 256 unit centroids plus 0.3 N(0,1) noise; iid Q, V, dO"}[w.dist]
    out = {
        "metric": metric,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": f"synthetic (seeded; {dist}; Gaussian W)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "P": w.P, "L": w.L,
                   "beta": w.beta, "causal": w.causal, "phases": "fwd+bwd" if train else "fwd",
                   "dbeta": bool(args.dbeta), "dW": bool(args.dW),
                   "per_head_tables": bool(args.per_head), "global_batch": w.B,
                   "seq_len": w.N},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": dname, "alg_bytes_per_launch": alg_bytes, "avg_launch_ms": avg_ms,
                     "device_copy_GBps_same_run": copy_gbps},
        "step_hbm_frac": ((11 if train else 4) * row_bytes) / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "kernels_ms_per_launch": {k: v[1] / v[0] for k, v in kern.items()},
        "cpu_baseline": cpu,
    }
    if graph_ms is not None:
        out["graph_ms_per_step"] = graph_ms
        out["graph_tokens_per_s"] = tokens / (graph_ms * 1e-3)
    fl = causal_flops(dname, w.L, w.P, w.d)
    if fl:
        # the walks also sit far below the MFMA roofline: bf16 dense peak
        tf = fl * w.B * w.H * w.N / (avg_ms * 1e-3) / 1e12
        peak = 2500.0 if w.dtype == "bf16" else 157.3
        out["roofline_mfma"] = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                                "frac": tf / peak, "kernel": dname, "alg_flops_per_launch": fl * w.B * w.H * w.N}
    if args.dW and "race_dw_partial" in kern:
        # the table-gradient stream: both sides' rows plus their float32 dPre
        pe = max(w.P, 3)
        lrp = -(-(w.L << pe) // 32) * 32
        nhp = (lrp >> pe) * pe
        dpre_bytes = 2 * w.B * w.H * w.N * nhp * 4
        c, ms = kern["race_dw_partial"]
        out["dw_partial"] = {"avg_launch_ms": ms / c, "alg_bytes_per_launch": 2 * row_bytes + dpre_bytes,
                             "achieved_GBps": (2 * row_bytes + dpre_bytes) / (ms / c * 1e-3) / 1e9}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
