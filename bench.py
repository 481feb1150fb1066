"""Benchmark of the MSA block-sparse attention path on one MI355X.

One step = the whole hot path over one batch of resident synthetic inputs:
msa_index_score -> msa_topk_select -> msa_sparse_attn_fwd.  W warm-up steps,
then K timed steps bracketed by torch.cuda.synchronize(); per-stage HIP events
(on the stream the kernels run on) and per-kernel events inside the library
calls give each stage's and kernel's median duration.

Prints ONE JSON line for the main workload (default: the 128K-token prefill).
`value` is tokens/s for prefill workloads and GB/s of algorithmic traffic for
decode.  `roofline` grades the main workload's longest kernel against its own
bound: bf16 MFMA peak on its algorithmic FLOPs for the prefill kernels, HBM
peak on its algorithmic bytes for the decode index scan.  The decode and the
1M-context chunk workloads are measured in the same run (fewer steps) and
reported under extra.workloads.  `cpu_baseline` times the CPU oracle on a
bounded seeded sample of the main workload after the GPU timing, and the
rows it computes are checked against the GPU's outputs of the last step
(`parity`).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--also A,B]
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
MAIN_WORKLOAD = "prefill-128k"
ALSO_WORKLOADS = "decode-64x256k,chunked-prefill-1m"


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


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
    """FLOPs of the current (diagonal) blocks, and the design bytes of the
    KV-major partial kernel: per (query, group, kept non-current block) it
    reads the group's H/G query rows and writes H/G partial rows (bf16 O and
    an fp32 (m, l) pair); each distinct kept (group, block) pair is staged
    once (K and V)."""
    import torch
    G, H, d, B = w.num_kv_groups, w.num_q_heads, w.head_dim, w.block_size
    hpg = H // G
    f_diag = 0.0
    for lq, lkv in zip(len_q, len_kv):
        base = lkv - lq
        f_diag += 4.0 * H * d * sum(p % B + 1 for p in range(base, lkv))
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
    return f_diag, part_bytes, n_entries


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


def copy_bandwidth(mib: int = 1024, reps: int = 10) -> float:
    """GB/s (bytes read + written) of torch's device copy of mib MiB, median of reps."""
    import numpy as np
    import torch
    n = mib << 20
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    b.copy_(a)
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    return 2.0 * n / (float(np.median(ts)) * 1e-3) / 1e9


def measured_traffic(kernel: str, workload: str, launches: int = 1):
    """HBM bytes per launch from the committed counter summary for this kernel
    and workload, or None if there is none, it was taken with another number
    of launches per step (passes), or the kernel source has changed since the
    counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm-traffic.json")
    src = {"kv_partial": "attn_kvmajor.hip", "kv_merge": "attn_kvmajor.hip",
           "index_score_mfma": "index_score.hip",
           "index_score_decode": "index_score.hip"}.get(kernel)
    if src is None or not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(os.path.join(ROOT, "block_sparse_long_msa_amd", "csrc", src), "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("source_sha256") != sha or rec.get("launches_per_step", 1) != launches:
        return None
    return rec.get("hbm_bytes_per_launch")


def mfma_roof(kernel, flops, ms):
    achieved = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
            "algorithmic_flops_per_launch": flops, "avg_launch_ms": ms}


def hbm_roof(kernel, nbytes, ms):
    achieved = nbytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": kernel, "achieved": achieved, "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": None,
            "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms}


class _nullctx:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def decode_shape(prob) -> bool:
    return prob.max_q_len == 1


def run_workload(name, steps, warmup, args, keep_state=False):
    """Times `steps` steps of one workload.  Returns (result dict, state);
    state (inputs and the last step's outputs) only when keep_state."""
    import numpy as np
    import torch

    import block_sparse_long_msa_amd as msa
    import workloads as W

    w = W.WORKLOADS[name]
    dev = torch.device("cuda:0")
    log(f"[bench] {name}: generating inputs")
    inp = W.make_inputs(w, device=dev, seed=0)
    lq, lkv = inp["len_q"], inp["len_kv"]
    prob = msa.Problem(inp["cu_q"], inp["cu_kv"], lq, lkv, w.num_q_heads, w.num_kv_groups,
                       w.head_dim, w.idx_dim, w.block_size, w.top_k, w.dtype,
                       1.0 / math.sqrt(w.head_dim), args.schedule)
    scores = torch.empty((prob.G, prob.total_q, prob.nb_max), dtype=torch.float32, device=dev)
    block_idx = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.int32, device=dev)
    out = torch.empty((prob.total_q, prob.H, prob.d), dtype=prob.torch_dtype, device=dev)
    layers = [(inp["q"], inp["k"], inp["v"])]
    for li in range(1, args.layers):
        lin = W.make_inputs(w, device=dev, seed=1000 + li)
        layers.append((lin["q"], lin["k"], lin["v"]))
        del lin
    train = keep_state and (args.indexer_kl or args.attn_bwd)
    ab_passes, ab_kernels = 1, []
    if train:
        lse_buf = torch.empty((prob.total_q, prob.H), dtype=torch.float32, device=dev)
    if train and args.attn_bwd:
        dout = W.random_out_grad(1, prob.total_q, prob.H, prob.d, w.dtype, device=dev)
        nab = ctypes.c_size_t(0)
        msa._check(msa.load_library().msa_sparse_attn_bwd_workspace_size(prob.ref(),
                                                                         ctypes.byref(nab)))
        ab_bytes = nab.value
        if args.attn_workspace_gib > 0:  # bounded: the backward's rows run in passes too
            ab_bytes = max(msa.sparse_attn_bwd_workspace_size(prob, minimum=True),
                           min(ab_bytes, int(args.attn_workspace_gib * 2**30)))
        ab_passes = -(-prob.total_q // max(1, msa.sparse_attn_bwd_rows_per_pass(prob, ab_bytes)))
        ab_ws = torch.empty(max(ab_bytes, 1), dtype=torch.uint8, device=dev)
        ab_kernels = ["ab_dsum", "ab_buckets", "ab_zero_unkept", "ab_item", "ab_reduce", "ab_dq"]
    if train and args.indexer_kl:
        mass = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.float32, device=dev)
        kl = torch.empty((prob.G, prob.total_q), dtype=torch.float32, device=dev)
        kl_grad = torch.empty((prob.G, prob.total_q, prob.top_k), dtype=torch.float32, device=dev)
        nbw = ctypes.c_size_t(0)
        msa._check(msa.load_library().msa_indexer_bwd_workspace_size(prob.ref(), ctypes.byref(nbw)))
        bwd_ws = torch.empty(max(nbw.value, 1), dtype=torch.uint8, device=dev)
    wbytes = msa.workspace_size(prob)
    if args.attn_workspace_gib > 0:  # bounded workspace: the KV-major rows run in passes
        wbytes = max(msa.workspace_size_min(prob), min(wbytes, int(args.attn_workspace_gib * 2**30)))
    passes = -(-prob.total_q // max(1, msa.rows_per_pass(prob, wbytes))) if prob.total_q else 1
    workspace = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    fused = args.fused_topk and not decode_shape(prob)
    hier = args.hier_index and not fused
    if hier:
        hier_keep = args.hier_keep or max(1, -(-2 * (prob.top_k - 1) // args.hier_chunk))
        hier_ws = torch.empty(max(msa.index_topk_hier_workspace_size(prob, args.hier_chunk,
                                                                     hier_keep), 1),
                              dtype=torch.uint8, device=dev)
    if fused:
        itk_ws = torch.empty(max(msa.index_topk_workspace_size(prob), 1), dtype=torch.uint8,
                             device=dev)
        del scores
        scores = None
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
    use_kl = train and args.indexer_kl
    use_bwd = train and args.attn_bwd

    def attention():
        if use_kl:
            msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], block_idx, out, lse_buf,
                                     mass, workspace=workspace, stream=sid)
        else:
            msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], block_idx, out,
                                workspace=workspace, stream=sid,
                                lse=lse_buf if use_bwd else None)

    def step(ev=None, pev=None, bev=None, fev=None):
        if ev is not None:
            ev[0].record(stream)
        if fused:
            with fev if fev is not None else _nullctx():
                msa.index_topk(prob, inp["q_idx"], inp["k_idx"], block_idx, workspace=itk_ws,
                               stream=sid)
            if ev is not None:
                ev[1].record(stream)
        elif hier:
            with fev if fev is not None else _nullctx():
                msa.index_topk_hier(prob, inp["q_idx"], inp["k_idx"], args.hier_chunk, hier_keep,
                                    block_idx, workspace=hier_ws, stream=sid)
            if ev is not None:
                ev[1].record(stream)
        else:
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
        if use_kl:
            msa.indexer_kl(prob, scores, block_idx, mass, kl, kl_grad, stream=sid)
            if ev is not None:
                ev[4].record(stream)
            msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], block_idx, kl_grad,
                            workspace=bwd_ws, stream=sid)
        if ev is not None:
            ev[5].record(stream)
        if use_bwd:
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

    log(f"[bench] {name}: {warmup} warm-up steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(steps)]
    pevents = [msa.ProfileEvents(len(attn_kernels) * passes, dev) for _ in range(steps)]
    bevents = [msa.ProfileEvents(1 + (len(ab_kernels) - 1) * ab_passes, dev) if use_bwd else None
               for _ in range(steps)]
    hier_kernels = ["hi_mean", "hi_coarse", "hi_buckets", "hi_fine", "hi_final"]
    fevents = [msa.ProfileEvents(2, dev) if fused else
               (msa.ProfileEvents(len(hier_kernels), dev) if hier else None) for _ in range(steps)]
    log(f"[bench] {name}: {steps} timed steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        step(events[i], pevents[i], bevents[i], fevents[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / steps
    med = lambda xs: float(np.median(xs))          # noqa: E731
    st_ms = {nm: med([e[i].elapsed_time(e[i + 1]) for e in events])
             for i, nm in enumerate(("index_score", "topk_select", "sparse_attn_fwd"))}
    # per-kernel durations over the timed steps: kernel i of the attention call
    # ends at its profile event i
    if fused:
        kern_all = {"index_topk": [e[0].elapsed_time(fe.events[0]) for e, fe in zip(events, fevents)],
                    "index_topk_merge": [fe.events[0].elapsed_time(fe.events[1]) for fe in fevents]}
    elif hier:
        kern_all = {}
        for i, kn in enumerate(hier_kernels):
            kern_all[kn] = [(e[0] if i == 0 else fe.events[i - 1]).elapsed_time(fe.events[i])
                            for e, fe in zip(events, fevents)]
    else:
        kern_all = {index_kernel: [e[0].elapsed_time(e[1]) for e in events],
                    "topk": [e[1].elapsed_time(e[2]) for e in events]}
    na = len(attn_kernels)
    for i, kn in enumerate(attn_kernels):  # summed over the passes of a step
        kern_all[kn] = [sum((e[2] if j == 0 else pe.events[j - 1]).elapsed_time(pe.events[j])
                            for j in range(i, na * passes, na))
                        for e, pe in zip(events, pevents)]
    if use_kl:
        kern_all["indexer_kl"] = [e[3].elapsed_time(e[4]) for e in events]
        kern_all["indexer_bwd"] = [e[4].elapsed_time(e[5]) for e in events]
    if use_bwd:  # the D kernel, then per pass the other kernels (summed over the passes)
        nb_ = len(ab_kernels) - 1
        kern_all[ab_kernels[0]] = [e[5].elapsed_time(be.events[0]) for e, be in zip(events, bevents)]
        for i, kn in enumerate(ab_kernels[1:], start=1):
            kern_all[kn] = [sum(be.events[j - 1].elapsed_time(be.events[j])
                                for j in range(i, 1 + nb_ * ab_passes, nb_))
                            for e, be in zip(events, bevents)]
    kern_ms = {kn: float(np.mean(v)) for kn, v in kern_all.items()}        # average launch
    kern_med = {kn: med(v) for kn, v in kern_all.items()}

    f_idx, f_attn, nbytes = algorithmic_work(w, lq, lkv)
    tokens = prob.total_q
    stages = {
        "index_score": {"ms": st_ms["index_score"], "tflops": f_idx / st_ms["index_score"] / 1e9},
        "topk_select": {"ms": st_ms["topk_select"]},
        "sparse_attn_fwd": {"ms": st_ms["sparse_attn_fwd"],
                            "tflops": f_attn * args.layers / st_ms["sparse_attn_fwd"] / 1e9},
    }
    f_bwd = 2.5 * f_attn     # S, dP, dV, dK and dQ products over the same kept keys
    if use_bwd:
        bwd_ms = med([e[5].elapsed_time(e[6]) for e in events])
        stages["sparse_attn_bwd"] = {"ms": bwd_ms, "tflops": f_bwd / bwd_ms / 1e9}
    for s_ in ("index_score", "sparse_attn_fwd", "sparse_attn_bwd"):
        if s_ in stages:
            stages[s_]["pct_mfma_peak"] = 100.0 * stages[s_]["tflops"] / PEAK_BF16_TFLOPS
    extra = {"kernels_ms_mean": kern_ms, "kernels_ms_median": kern_med}
    part_flops = None
    if "kv_partial" in kern_ms:
        f_diag, part_bytes, n_entries = kvmajor_partial_work(w, lq, lkv, block_idx)
        part_flops = f_attn - f_diag
        extra["kv_partial"] = {"flops": part_flops, "entries": n_entries,
                               "design_bytes": part_bytes,
                               "design_gbps": part_bytes / (kern_ms["kv_partial"] * 1e-3) / 1e9}
    dom = max(kern_ms, key=lambda kk: kern_ms[kk])
    # the KV-major kernels launch once per pass: the roofline is per launch
    # (the step's work and time divided by the launches), like the counters
    nl = passes if dom in attn_kernels else (ab_passes if dom in ab_kernels[1:] else 1)
    if dom in ("index_score_mfma", "index_topk"):
        roof = mfma_roof(dom, f_idx, kern_ms[dom])
    elif dom == "ab_item":
        roof = mfma_roof(dom, f_bwd / nl, kern_ms[dom] / nl)
    elif dom == "kv_partial":
        roof = mfma_roof(dom, part_flops / nl, kern_ms[dom] / nl)
    elif dom == "index_score_decode":
        roof = hbm_roof(dom, sum(x * w.num_kv_groups * w.idx_dim * 2 for x in lkv), kern_ms[dom])
    else:
        roof = mfma_roof(dom, f_attn / nl, kern_ms[dom] / nl)
    roof["launches_per_step"] = nl
    roof["traffic"] = measured_traffic(dom, w.name, nl)
    if decode:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        extra.update({"gbps_step": value, "pct_hbm_peak": 100.0 * value / PEAK_HBM_GBS,
                      "bytes_per_step": nbytes})
    else:
        value = tokens / (ms_per_step * 1e-3)
        unit = "tokens/s"
        extra.update({"tflops_effective_attention": f_attn * args.layers / (st_ms["sparse_attn_fwd"] * 1e-3) / 1e12,
                      "tflops_pipeline": (f_idx + f_attn * args.layers) / (ms_per_step * 1e-3) / 1e12,
                      "flops_index": f_idx, "flops_attention": f_attn})
    if args.layers > 1:
        extra["layers"] = args.layers
        extra["ms_per_layer"] = ms_per_step / args.layers
        extra["index_and_topk_share"] = (st_ms["index_score"] + st_ms["topk_select"]) / ms_per_step
        extra["layer_tokens_per_s"] = tokens * args.layers / (ms_per_step * 1e-3)
    config = {"workload": w.name, "num_seqs": len(lq), "len_q": max(lq), "len_kv": max(lkv),
              "total_kv": sum(lkv), "H": w.num_q_heads, "G": w.num_kv_groups, "d": w.head_dim,
              "d_idx": w.idx_dim, "block": w.block_size, "top_k": w.top_k,
              "schedule": args.schedule,
              **({"layers_per_index": args.layers} if args.layers > 1 else {}),
              **({"indexer_kl": True} if use_kl else {}),
              **({"fused_topk": True} if fused else {}),
              **({"hier_index": {"chunk_blocks": args.hier_chunk, "keep_chunks": hier_keep}}
                 if hier else {}),
              **({"attn_bwd": True} if use_bwd else {}),
              **({"attn_workspace_bytes": wbytes, "attn_passes": passes}
                 if args.attn_workspace_gib > 0 or passes > 1 else {}),
              **({"attn_bwd_workspace_bytes": ab_bytes, "attn_bwd_passes": ab_passes}
                 if args.attn_workspace_gib > 0 and use_bwd else {})}
    res = {"value": value, "unit": unit, "ms_per_step": ms_per_step, "dtype": w.dtype,
           "config": config, "roofline": roof, "stages": stages, "extra": extra,
           "wall_s_timed": wall, "steps": steps, "warmup": warmup}
    log(f"[bench] {name}: {ms_per_step:.3f} ms/step, {value:.4g} {unit}")
    state = None
    if hier:
        # recall of the approximation's free picks against the exact selection
        exact = msa.topk_select(prob, msa.index_score(prob, inp["q_idx"], inp["k_idx"]))
        hit = tot = 0
        q0 = 0
        for lq_, lkv_ in zip(lq, lkv):
            pos = torch.arange(lkv_ - lq_, lkv_, device=dev)
            Jr = (pos // prob.B).view(1, -1, 1)
            e_, h_ = exact[:, q0:q0 + lq_], block_idx[:, q0:q0 + lq_]
            fe = (e_ >= 0) & (e_ < Jr)
            fh = (h_ >= 0) & (h_ < Jr)
            hit += int((fe.unsqueeze(3) & fh.unsqueeze(2) & (e_.unsqueeze(3) == h_.unsqueeze(2))).sum())
            tot += int(fe.sum())
            q0 += lq_
        extra["hier_recall"] = hit / max(tot, 1)
        del exact
    if keep_state and (fused or hier):
        # the fused call leaves no score tensor: the parity leg scores the rows itself
        scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    if keep_state:
        state = {"w": w, "inp": inp, "scores": scores, "block_idx": block_idx, "out": out,
                 "decode": decode, "unit": unit}
    else:
        del inp, scores, block_idx, out, workspace, layers
    return res, state


def cpu_baseline(st, budget_s, check=True):
    """The CPU oracle, as is, on a bounded seeded sample of the same workload,
    timed on the host cores; the rows it computes are then checked against
    the GPU's outputs of the last timed step under the acceptance rules of
    the parity tests (scores within the fp32 rounding bound, a delta-valid
    Top-k, attention within 2e-2 where the GPU kept the oracle's blocks)."""
    import numpy as np
    import torch

    from oracle import msa_oracle as O
    from tests import msa_check as C

    w, inp, decode, unit = st["w"], st["inp"], st["decode"], st["unit"]
    cores = len(os.sched_getaffinity(0))
    torch.set_num_threads(cores)
    scale = 1.0 / math.sqrt(w.head_dim)
    lq, lkv = inp["len_q"], inp["len_kv"]
    rng = np.random.default_rng(0)
    B, k = w.block_size, w.top_k
    parity = {"rows": 0, "score_ratio": 0.0, "unseparated": 0, "out_err": 0.0,
              "rows_attention_compared": 0}
    s_gpu, i_gpu, o_gpu = st["scores"], st["block_idx"], st["out"]

    def check_rows(ref, q_idx_rows, k_idx, grows):
        if not check:
            return
        gr = torch.from_numpy(grows).to(s_gpu.device)
        nbs = ref["scores"].shape[2]
        s_g = s_gpu[:, gr, :nbs].cpu().numpy()
        bound = C.score_bound(q_idx_rows, k_idx, ref["pos"], B, cheap=True)
        parity["score_ratio"] = max(parity["score_ratio"],
                                    C.check_scores(s_g, ref["scores"], bound, w.idx_dim))
        ig = i_gpu[:, gr, :].cpu().numpy()
        parity["unseparated"] += C.check_selection(ig, ref["block_idx"], ref["scores"],
                                                   ref["pos"], B, k)
        same = np.all(ig == ref["block_idx"], axis=2)           # [G, n]
        og = o_gpu[gr].float().cpu().numpy()
        hpg = w.num_q_heads // w.num_kv_groups
        for g in range(w.num_kv_groups):
            rr = np.nonzero(same[g])[0]
            if rr.size:
                hs = slice(g * hpg, (g + 1) * hpg)
                parity["out_err"] = max(parity["out_err"], C.check_attention(
                    og[rr, hs], None, ref["out"][rr, hs], ref["lse"][rr, hs], w.dtype))
                parity["rows_attention_compared"] += int(rr.size)
        parity["rows"] += len(grows)

    t_start = time.perf_counter()
    done_rows = 0
    done_bytes = 0.0
    if decode:
        cu = np.concatenate([[0], np.cumsum(lkv)])
        order = rng.permutation(len(lkv))
        oracle_s = 0.0
        for b in order:
            sl = slice(int(cu[b]), int(cu[b + 1]))
            k_idx = inp["k_idx"][sl].cpu()
            k_ = inp["k"][sl].cpu()
            v_ = inp["v"][sl].cpu()
            q_idx_b = inp["q_idx"][b:b + 1].cpu()
            t1 = time.perf_counter()
            ref = O.msa_forward(inp["q"][b:b + 1].cpu(), k_, v_, q_idx_b, k_idx, 1, lkv[b],
                                B, k, scale, workers=cores)
            oracle_s += time.perf_counter() - t1
            check_rows(ref, q_idx_b, k_idx, np.array([b]))
            done_rows += 1
            done_bytes += algorithmic_work(w, [1], [lkv[b]])[2]
            if time.perf_counter() - t_start > budget_s:
                break
        return ({"value": done_bytes / oracle_s / 1e9, "unit": "GB/s", "cores": cores,
                 "kind": "oracle",
                 "sample": f"{done_rows} of {len(lkv)} decode sequences, whole path (index, "
                           f"Top-k, attention), fp64 numpy", "seconds": oracle_s}, parity)
    n_q = lq[0]
    host = {key: inp[key].cpu() for key in ("q", "k", "v", "q_idx", "k_idx")}
    host["k"], host["v"] = O._f64(host["k"]), O._f64(host["v"])    # upcast once
    oracle_s = 0.0
    while time.perf_counter() - t_start < budget_s:
        rows = np.sort(rng.choice(n_q, size=32, replace=False))
        t1 = time.perf_counter()
        ref = O.msa_forward(host["q"], host["k"], host["v"], host["q_idx"], host["k_idx"], n_q,
                            lkv[0], B, k, scale, rows=rows, workers=cores)
        oracle_s += time.perf_counter() - t1
        check_rows(ref, host["q_idx"][torch.from_numpy(rows)], host["k_idx"], rows)
        done_rows += len(rows)
    return ({"value": done_rows / oracle_s, "unit": unit, "cores": cores, "kind": "oracle",
             "sample": f"{done_rows} seeded random query rows of {n_q} (32 at a time), whole "
                       f"path (index over all causal keys, Top-k, attention), fp64 numpy",
             "seconds": oracle_s}, parity)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=MAIN_WORKLOAD)
    ap.add_argument("--also", default=None,
                    help="comma-separated workloads measured after the main one and reported "
                         f"under extra.workloads (default with the main workload: {ALSO_WORKLOADS}; "
                         "'none' for none)")
    ap.add_argument("--schedule", default="auto", choices=["auto", "query_major", "kv_major"])
    ap.add_argument("--attn-workspace-gib", type=float, default=0.0,
                    help="bound the attention workspace (GiB): the KV-major schedule then runs "
                         "its query rows in passes (0: one pass)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
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
    ap.add_argument("--fused-topk", action="store_true",
                    help="index scoring and Top-k in one call (msa_index_topk, no score tensor) "
                         "instead of msa_index_score + msa_topk_select")
    ap.add_argument("--hier-index", action="store_true",
                    help="hierarchical coarse-to-fine selection (msa_index_topk_hier, an "
                         "approximation) in place of msa_index_score + msa_topk_select; the "
                         "recall of its free picks against the exact selection is reported")
    ap.add_argument("--hier-chunk", type=int, default=16, help="blocks per coarse chunk")
    ap.add_argument("--hier-keep", type=int, default=0,
                    help="coarse chunks kept per query (0: enough for twice the free picks)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times (counter calibration)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        msg = ("bench.py measures one GPU only (the path would shard by KV group with no "
               "exchange between GPUs); run it with --gpus 1")
        print(msg, file=sys.stderr, flush=True)
        sys.exit(2)

    if args.fused_topk and args.indexer_kl:
        print("--indexer-kl needs the score tensor, which --fused-topk does not produce",
              file=sys.stderr, flush=True)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    also = args.also
    if also is None:
        also = ALSO_WORKLOADS if (args.workload == MAIN_WORKLOAD and args.layers == 1
                                  and not args.indexer_kl and not args.attn_bwd) else "none"
    also = [a for a in also.split(",") if a and a != "none" and a != args.workload]

    main_res, st = run_workload(args.workload, args.steps, args.warmup, args, keep_state=True)
    res = {"metric": METRIC, "value": main_res["value"], "unit": main_res["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": main_res["dtype"], "data": "synthetic", "config": main_res["config"],
           "roofline": main_res["roofline"], "stages": main_res["stages"],
           "extra": main_res["extra"], "wall_s_timed": main_res["wall_s_timed"]}
    parity_failed = False
    if not args.no_cpu_baseline:
        log(f"[bench] CPU oracle baseline ({args.cpu_seconds:.0f} s budget) + parity of its rows")
        try:
            res["cpu_baseline"], res["parity"] = cpu_baseline(st, args.cpu_seconds,
                                                              check=args.layers == 1)
        except AssertionError as e:          # a parity rule failed: report it, exit non-zero
            res["parity"] = {"ok": False, "error": str(e)}
            parity_failed = True
        else:
            res["parity"]["ok"] = True
    del st
    torch.cuda.empty_cache()
    res["extra"]["hbm_copy_gbps"] = copy_bandwidth()
    if also:
        res["extra"]["workloads"] = {}
        for name in also:
            r, _ = run_workload(name, min(args.steps, 10), min(args.warmup, 2), args)
            torch.cuda.empty_cache()
            r.pop("extra", None)
            if r["unit"] == "GB/s":
                r["pct_of_copy_bandwidth"] = 100.0 * r["value"] / res["extra"]["hbm_copy_gbps"]
            res["extra"]["workloads"][name] = r
    print(json.dumps(res), flush=True)
    if parity_failed:
        sys.exit(1)


if __name__ == "__main__":
    main()
