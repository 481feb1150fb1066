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
import ctypes
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


def kvmajor_partial_work(w, len_q, len_kv, block_idx):
    """FLOPs of the current (diagonal) blocks, and the algorithmic bytes of the
    KV-major partial kernel: per (query, group, kept non-current block) it
    reads the group's H/G query rows and writes H/G partial rows (bf16 O and
    an fp32 log-sum-exp); each distinct kept (group, block) pair is staged
    once (K and V)."""
    import torch
    G, H, d, B = w.num_kv_groups, w.num_q_heads, w.head_dim, w.block_size
    hpg = H // G
    f_diag = 0.0
    for lq, lkv in zip(len_q, len_kv):
        base = lkv - lq
        f_diag += 4.0 * H * d * sum(p % B + 1 for p in range(base, lkv))
    # entries = kept blocks strictly below the query's current block
    cu = [0]
    for lq in len_q:
        cu.append(cu[-1] + lq)
    n_entries = 0
    n_buckets = 0
    for si, (lq, lkv) in enumerate(zip(len_q, len_kv)):
        if lq == 0:
            continue
        bi = block_idx[:, cu[si]:cu[si + 1], :]
        pos = torch.arange(lkv - lq, lkv, device=bi.device)
        J = (pos // B).view(1, -1, 1)
        valid = (bi >= 0) & (bi < J)
        n_entries += int(valid.sum().item())
        nb = -(-lkv // B)
        keyed = torch.where(valid, bi + nb * torch.arange(G, device=bi.device).view(-1, 1, 1),
                            torch.full_like(bi, -1))
        n_buckets += int(torch.unique(keyed[keyed >= 0]).numel())
    part_bytes = n_entries * hpg * (d * 2 + d * 2 + 8) + n_buckets * 2 * B * d * 2
    return f_diag, part_bytes


def copy_calibration(mib: int) -> None:
    """A plain copy of known size: reads and writes exactly mib MiB per launch."""
    import torch
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary for this kernel
    and workload, or None if there is none or the kernel source has changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm-traffic.json")
    src = {"kv_partial": "attn_kvmajor.hip", "index_score_mfma": "index_score.hip",
           "index_score_decode": "index_score.hip"}.get(kernel)
    if src is None or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, "block_sparse_long_msa_amd", "csrc", src), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill-32k")
    ap.add_argument("--schedule", default="auto", choices=["auto", "query_major", "kv_major"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--layers", type=int, default=1,
                    help="cross-layer index reuse: one index + Top-k pass, then the attention "
                         "of this many layers (own q, k, v each) on the same kept-block lists")
    ap.add_argument("--indexer-kl", action="store_true",
                    help="training step of the indexer: the attention also returns the Main "
                         "Branch block mass, then the indexer's KL loss, its score gradient and "
                         "the max-pooling backward to q_idx and k_idx follow")
    ap.add_argument("--attn-bwd", action="store_true",
                    help="training step of the Main Branch: the attention also returns its LSE, "
                         "then the attention backward for a seeded upstream gradient follows")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
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
    # further layers reuse the kept-block lists with their own q, k, v
    layers = [(inp["q"], inp["k"], inp["v"])]
    for li in range(1, args.layers):
        lin = W.make_inputs(w, device=dev, seed=1000 + li)
        layers.append((lin["q"], lin["k"], lin["v"]))
        del lin
    if args.indexer_kl or args.attn_bwd:
        lse_buf = torch.empty((prob.total_q, prob.H), dtype=torch.float32, device=dev)
    if args.attn_bwd:
        dout = W.random_out_grad(1, prob.total_q, prob.H, prob.d, w.dtype, device=dev)
        nab = ctypes.c_size_t(0)
        msa._check(msa.load_library().msa_sparse_attn_bwd_workspace_size(prob.ref(),
                                                                         ctypes.byref(nab)))
        ab_ws = torch.empty(max(nab.value, 1), dtype=torch.uint8, device=dev)
        ab_kernels = ["ab_dsum", "ab_buckets", "ab_zero_unkept", "ab_item", "ab_reduce", "ab_dq"]
    if args.indexer_kl:
        mass = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.float32, device=dev)
        kl = torch.empty((prob.G, prob.total_q), dtype=torch.float32, device=dev)
        kl_grad = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.float32, device=dev)
        nbw = ctypes.c_size_t(0)
        msa._check(msa.load_library().msa_indexer_bwd_workspace_size(prob.ref(), ctypes.byref(nbw)))
        bwd_ws = torch.empty(max(nbw.value, 1), dtype=torch.uint8, device=dev)
    wbytes = msa.workspace_size(prob)
    workspace = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sid = stream.cuda_stream

    decode = prob.max_q_len == 1
    if decode:
        attn_kernels = ["attn_qmajor", "combine_splits"] if prob.top_k > 4 else ["attn_qmajor"]
    elif prob.dtype == "bf16" and args.schedule != "query_major":
        attn_kernels = ["kv_clear", "kv_count", "kv_scan", "kv_scatter", "kv_items",
                        "kv_partial", "kv_diag", "kv_merge"]
    else:
        attn_kernels = ["attn_qmajor"]
    index_kernel = "index_score_decode" if decode else "index_score_mfma"

    def attention():
        if args.indexer_kl:
            msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], block_idx, out, lse_buf,
                                     mass, workspace=workspace, stream=sid)
        else:
            msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], block_idx, out,
                                workspace=workspace, stream=sid,
                                lse=lse_buf if args.attn_bwd else None)

    def step(ev=None, pev=None, bev=None):
        if ev is not None:
            ev[0].record(stream)
        msa.index_score(prob, inp["q_idx"], inp["k_idx"], scores, stream=sid)
        if ev is not None:
            ev[1].record(stream)
        msa.topk_select(prob, scores, block_idx, stream=sid)
        if ev is not None:
            ev[2].record(stream)
        if pev is not None:
            with pev:
                attention()
        else:
            attention()
        for lq_, lk_, lv_ in layers[1:]:
            msa.sparse_attn_fwd(prob, lq_, lk_, lv_, block_idx, out, workspace=workspace, stream=sid)
        if ev is not None:
            ev[3].record(stream)
        if args.indexer_kl:
            msa.indexer_kl(prob, scores, block_idx, mass, kl, kl_grad, stream=sid)
            if ev is not None:
                ev[4].record(stream)
            msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], block_idx, kl_grad,
                            workspace=bwd_ws, stream=sid)
        if ev is not None:
            ev[5].record(stream)
        if args.attn_bwd:
            def backward():
                msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], block_idx, out, lse_buf,
                                    dout, workspace=ab_ws, stream=sid)
            if bev is not None:
                with bev:
                    backward()
            else:
                backward()
        if ev is not None:
            ev[6].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(args.steps)]
    pevents = [msa.ProfileEvents(len(attn_kernels), dev) for _ in range(args.steps)]
    bevents = [msa.ProfileEvents(len(ab_kernels), dev) if args.attn_bwd else None
               for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(args.steps):
        step(events[i], pevents[i], bevents[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    st_ms = {name: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in events]))
             for i, name in enumerate(("index_score", "topk_select", "sparse_attn_fwd"))}
    # per-kernel averages: kernel i of the attention call ends at its profile event i
    kern_ms = {index_kernel: st_ms["index_score"], "topk": st_ms["topk_select"]}
    for i, name in enumerate(attn_kernels):
        vals = []
        for e, pe in zip(events, pevents):
            prev = e[2] if i == 0 else pe.events[i - 1]
            vals.append(prev.elapsed_time(pe.events[i]))
        kern_ms[name] = float(np.mean(vals))
    if args.indexer_kl:
        kern_ms["indexer_kl"] = float(np.mean([e[3].elapsed_time(e[4]) for e in events]))
        kern_ms["indexer_bwd"] = float(np.mean([e[4].elapsed_time(e[5]) for e in events]))
    if args.attn_bwd:
        for i, name in enumerate(ab_kernels):
            vals = []
            for e, be in zip(events, bevents):
                prev = e[5] if i == 0 else be.events[i - 1]
                vals.append(prev.elapsed_time(be.events[i]))
            kern_ms[name] = float(np.mean(vals))

    f_idx, f_attn, nbytes = algorithmic_work(w, lq, lkv)
    f_diag, part_bytes = kvmajor_partial_work(w, lq, lkv, block_idx)
    tokens = prob.total_q
    res = {"metric": METRIC}
    stages = {
        "index_score": {"ms": st_ms["index_score"], "tflops": f_idx / st_ms["index_score"] / 1e9},
        "topk_select": {"ms": st_ms["topk_select"]},
        "sparse_attn_fwd": {"ms": st_ms["sparse_attn_fwd"],
                            "tflops": f_attn * args.layers / st_ms["sparse_attn_fwd"] / 1e9},
    }
    # backward: S, dP, dV, dK and dQ products over the same kept keys, 5/2 of the forward's
    f_bwd = 2.5 * f_attn
    if args.attn_bwd:
        bwd_ms = float(np.mean([e[5].elapsed_time(e[6]) for e in events]))
        stages["sparse_attn_bwd"] = {"ms": bwd_ms, "tflops": f_bwd / bwd_ms / 1e9}
    for s in ("index_score", "sparse_attn_fwd", "sparse_attn_bwd"):
        if s in stages:
            stages[s]["pct_mfma_peak"] = 100.0 * stages[s]["tflops"] / PEAK_BF16_TFLOPS
    dom = max(kern_ms, key=lambda k: kern_ms[k])
    dom_s = kern_ms[dom] * 1e-3
    if dom == "index_score_mfma":
        achieved = f_idx / dom_s / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                "algorithmic_flops_per_launch": f_idx}
    elif dom == "ab_item":
        achieved = f_bwd / dom_s / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                "algorithmic_flops_per_launch": f_bwd}
    elif dom == "kv_partial":
        achieved = part_bytes / dom_s / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                "algorithmic_bytes_per_launch": part_bytes,
                "tflops": (f_attn - f_diag) / dom_s / 1e12}
    elif dom == "index_score_decode":
        dom_bytes = sum(x * w.num_kv_groups * w.idx_dim * 2 for x in lkv)
        achieved = dom_bytes / dom_s / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
                "algorithmic_bytes_per_launch": dom_bytes}
    else:
        achieved = f_attn / dom_s / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                "algorithmic_flops_per_launch": f_attn}
    if decode:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        extra = {"gbps_step": value, "pct_hbm_peak": 100.0 * value / PEAK_HBM_GBS,
                 "bytes_per_step": nbytes}
    else:
        value = tokens / (ms_per_step * 1e-3)
        unit = "tokens/s"
        extra = {"tflops_effective_attention": f_attn * args.layers / (st_ms["sparse_attn_fwd"] * 1e-3) / 1e12,
                 "tflops_pipeline": (f_idx + f_attn * args.layers) / (ms_per_step * 1e-3) / 1e12,
                 "flops_index": f_idx, "flops_attention": f_attn}
    extra["kernels_ms"] = kern_ms
    if args.layers > 1:
        extra["layers"] = args.layers
        extra["ms_per_layer"] = ms_per_step / args.layers
        extra["index_and_topk_share"] = (st_ms["index_score"] + st_ms["topk_select"]) / ms_per_step
        extra["layer_tokens_per_s"] = tokens * args.layers / (ms_per_step * 1e-3)
    roof["traffic"] = measured_traffic(dom, w.name)
    res.update({"value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
                "config": {"workload": w.name, "num_seqs": len(lq), "len_q": max(lq),
                           "len_kv": max(lkv), "total_kv": sum(lkv), "H": w.num_q_heads,
                           "G": w.num_kv_groups, "d": w.head_dim, "d_idx": w.idx_dim,
                           "block": w.block_size, "top_k": w.top_k, "schedule": args.schedule,
                           **({"layers_per_index": args.layers} if args.layers > 1 else {}),
                           **({"indexer_kl": True} if args.indexer_kl else {}),
                           **({"attn_bwd": True} if args.attn_bwd else {})},
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
