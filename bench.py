"""Benchmark of the MSA block-sparse attention path on one MI355X.

One step = the whole hot path over one batch of resident synthetic inputs:
msa_index_score -> msa_topk_select -> msa_sparse_attn_fwd.  W warm-up steps,
then K timed steps bracketed by torch.cuda.synchronize(); per-stage HIP events
(on the stream the kernels run on) give each stage's average duration.

Prints ONE JSON line.  `value` is tokens/s for prefill workloads and GB/s of
algorithmic traffic for the decode workload.  `roofline` is for the dominant
stage; `cpu_baseline` times the CPU oracle on a bounded sample of the same
workload (after the GPU timing).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--schedule S]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tokens/s + TFLOP/s (% MFMA peak); decode GB/s (% HBM)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def algorithmic_work(w, len_q, len_kv):
    """FLOPs of the index scan and of attention over the kept keys, and decode bytes.

    Index: 2*G*d_idx per (query, causal key).  Attention: 4*H*d per (query,
    kept causal key), with n_sel(p) = min(p+1, (k-1)*B + p%B + 1) kept keys
    (every non-current kept block is full).  Decode bytes: the k_idx scan,
    the kept K and V rows, q, q_idx, out, and the score/index round trips."""
    G, H, d, di, B, k = (w.num_kv_groups, w.num_q_heads, w.head_dim, w.idx_dim,
                         w.block_size, w.top_k)
    f_idx = f_attn = 0.0
    nbytes = 0.0
    for lq, lkv in zip(len_q, len_kv):
        base = lkv - lq
        sum_p = (base + lkv - 1) * lq / 2.0          # sum of p over base .. lkv-1
        f_idx += 2.0 * G * di * (sum_p + lq)
        n_sel = 0
        for p in range(base, lkv):
            n_sel += min(p + 1, (k - 1) * B + p % B + 1)
        f_attn += 4.0 * H * d * n_sel
        nb = -(-lkv // B)
        nbytes += (lkv * G * di * 2 + G * n_sel * d * 2 * 2 + lq * (G * di * 2 + 2 * H * d * 2)
                   + lq * G * nb * 4 * 2 + lq * G * k * 4 * 2)
    return f_idx, f_attn, nbytes


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill-32k")
    ap.add_argument("--schedule", default="auto", choices=["auto", "query_major", "kv_major"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import block_sparse_long_msa_amd as msa
    import workloads as W

    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.make_inputs(w, device=dev, seed=0)
    lq, lkv = inp["len_q"], inp["len_kv"]
    prob = msa.Problem(inp["cu_q"], inp["cu_kv"], lq, lkv, w.num_q_heads, w.num_kv_groups,
                       w.head_dim, w.idx_dim, w.block_size, w.top_k, w.dtype,
                       1.0 / math.sqrt(w.head_dim), args.schedule)
    scores = torch.empty((prob.G, prob.total_q, prob.nb_max), dtype=torch.float32, device=dev)
    block_idx = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((prob.total_q, prob.H, prob.d), dtype=prob.torch_dtype, device=dev)
    wbytes = msa.workspace_size(prob)
    workspace = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        msa.index_score(prob, inp["q_idx"], inp["k_idx"], scores, stream=sid)
        if ev is not None:
            ev[1].record(stream)
        msa.topk_select(prob, scores, block_idx, stream=sid)
        if ev is not None:
            ev[2].record(stream)
        msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], block_idx, out,
                            workspace=workspace, stream=sid)
        if ev is not None:
            ev[3].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(events[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    st_ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events]))
             for i, name in enumerate(("index_score", "topk_select", "sparse_attn_fwd"))}

    f_idx, f_attn, nbytes = algorithmic_work(w, lq, lkv)
    decode = prob.max_q_len == 1
    tokens = prob.total_q
    res = {"metric": METRIC}
    stages = {
        "index_score": {"ms": st_ms["index_score"], "tflops": f_idx / st_ms["index_score"] / 1e9},
        "topk_select": {"ms": st_ms["topk_select"]},
        "sparse_attn_fwd": {"ms": st_ms["sparse_attn_fwd"],
                            "tflops": f_attn / st_ms["sparse_attn_fwd"] / 1e9},
    }
    for s in ("index_score", "sparse_attn_fwd"):
        stages[s]["pct_mfma_peak"] = 100.0 * stages[s]["tflops"] / PEAK_BF16_TFLOPS
    if decode:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        dom = "index_score"
        dom_bytes = sum(x * w.num_kv_groups * w.idx_dim * 2 for x in lkv)
        achieved = dom_bytes / (st_ms[dom] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                "algorithmic_bytes_per_launch": dom_bytes}
        extra = {"gbps_step": value, "pct_hbm_peak": 100.0 * value / PEAK_HBM_GBS,
                 "bytes_per_step": nbytes}
    else:
        value = tokens / (ms_per_step * 1e-3)
        unit = "tokens/s"
        dom = max(("index_score", "sparse_attn_fwd"), key=lambda s: st_ms[s])
        flops = f_idx if dom == "index_score" else f_attn
        achieved = flops / (st_ms[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                "algorithmic_flops_per_launch": flops}
        extra = {"tflops_effective_attention": f_attn / (st_ms["sparse_attn_fwd"] * 1e-3) / 1e12,
                 "tflops_pipeline": (f_idx + f_attn) / (ms_per_step * 1e-3) / 1e12,
                 "flops_index": f_idx, "flops_attention": f_attn}
    res.update({"value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
                "config": {"workload": w.name, "num_seqs": len(lq), "len_q": max(lq),
                           "len_kv": max(lkv), "total_kv": sum(lkv), "H": w.num_q_heads,
                           "G": w.num_kv_groups, "d": w.head_dim, "d_idx": w.idx_dim,
                           "block": w.block_size, "top_k": w.top_k, "schedule": args.schedule},
                "roofline": roof, "stages": stages, "extra": extra,
                "wall_s_timed": wall})

    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, inp, decode, args.cpu_seconds, unit)
    print(json.dumps(res), flush=True)


def cpu_baseline(w, inp, decode, budget_s, unit):
    """The CPU oracle, as is, on a bounded seeded sample of the same workload."""
    import numpy as np
    import torch

    from oracle import msa_oracle as O

    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    scale = 1.0 / math.sqrt(w.head_dim)
    lq, lkv = inp["len_q"], inp["len_kv"]
    rng = np.random.default_rng(0)
    t_start = time.perf_counter()
    done_rows = 0
    done_bytes = 0.0
    if decode:
        # whole sequences (one query each) until the budget is spent
        cu = np.concatenate([[0], np.cumsum(lkv)])
        order = rng.permutation(len(lkv))
        for b in order:
            sl = slice(int(cu[b]), int(cu[b + 1]))
            k_idx = inp["k_idx"][sl].cpu()
            k = inp["k"][sl].cpu()
            v = inp["v"][sl].cpu()
            O.msa_forward(inp["q"][b:b + 1].cpu(), k, v, inp["q_idx"][b:b + 1].cpu(), k_idx, 1,
                          lkv[b], w.block_size, w.top_k, scale)
            done_rows += 1
            _, _, nb = _decode_bytes(w, lkv[b])
            done_bytes += nb
            if time.perf_counter() - t_start > budget_s:
                break
        el = time.perf_counter() - t_start
        return {"value": done_bytes / el / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
                "sample": f"{done_rows} of {len(lkv)} decode sequences (whole path, fp64 numpy)",
                "seconds": el}
    n_q = lq[0]
    host = {k: inp[k].cpu() for k in ("q", "k", "v", "q_idx", "k_idx")}
    while time.perf_counter() - t_start < budget_s:
        rows = np.sort(rng.choice(n_q, size=32, replace=False))
        O.msa_forward(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], n_q, lkv[0],
                      w.block_size, w.top_k, scale, rows=rows)
        done_rows += len(rows)
    el = time.perf_counter() - t_start
    return {"value": done_rows / el, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{done_rows} seeded random query rows of {n_q} (whole path, fp64 numpy)",
            "seconds": el}


def _decode_bytes(w, lkv):
    from types import SimpleNamespace
    return algorithmic_work(SimpleNamespace(**{f: getattr(w, f) for f in (
        "num_kv_groups", "num_q_heads", "head_dim", "idx_dim", "block_size", "top_k")}),
        [1], [lkv])


if __name__ == "__main__":
    main()
