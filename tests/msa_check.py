"""Helpers for the GPU parity tests: run the HIP library through its C ABI and
compare with the CPU oracle under the acceptance rules below.

Acceptance rules
  * scores: |S_gpu - S| <= 2 * gamma_{d_idx} * max_s sum_c |q_c k_{s,c}| per block
    (the fp32 dot-product rounding bound, gamma_n = n u / (1 - n u), u = 2^-24,
    doubled because the MFMA's internal summation order is not sequential),
    and -inf at exactly the oracle's -inf positions;
  * selection on the GPU's own fp32 scores: every row is a delta-valid Top-k
    (current block present, right count, ascending, -1 padded, and no dropped
    candidate beats a kept one by more than delta = 1e-3 * max(|s_(k-1)|, |s_k|)
    in the oracle's fp64 scores); rows whose (k-1)-th and k-th best candidates
    differ by more than delta must match the oracle exactly;
  * attention, given the ORACLE's kept blocks: max |O_gpu - O| <= 2e-2 (bf16)
    or 1e-4 (fp32); the same bound on LSE.
Expected values come only from the oracle; the GPU's outputs are never fed to it.
"""
from __future__ import annotations

import math
import time
from typing import Dict, Optional, Sequence

import numpy as np
import torch

import block_sparse_long_msa_amd as msa
from oracle import msa_oracle as O

U = 2.0 ** -24
TOL_OUT = {"bf16": 2e-2, "f32": 1e-4}


def gamma(n: int) -> float:
    return n * U / (1 - n * U)


def problem_for(inp: Dict, H: int, G: int, d: int, d_idx: int, B: int, k: int, dtype: str,
                schedule: str = "auto") -> msa.Problem:
    return msa.Problem(inp["cu_q"], inp["cu_kv"], inp["len_q"], inp["len_kv"], H, G, d, d_idx, B,
                       k, dtype, 1.0 / math.sqrt(d), schedule)


def score_bound(q_idx_rows, k_idx, pos, B: int, cheap: bool = False) -> np.ndarray:
    """Per-block max of sum_c |q_c k_c| over causal keys (the same pooling as S).

    cheap: the Cauchy-Schwarz bound |q|_2 * max over the block's keys of
    |k_s|_2 instead (never smaller, so the acceptance bound only loosens;
    it costs one norm per key instead of a second scoring pass)."""
    if not cheap:
        qa = np.abs(O._f64(q_idx_rows))
        ka = np.abs(O._f64(k_idx))
        return O.block_scores(qa, ka, pos, B)
    q = O._f64(q_idx_rows)
    n, G, _ = q.shape
    L = k_idx.shape[0]
    nb = O.num_blocks(L, B)
    qn = np.sqrt((q * q).sum(axis=2))                                   # [n, G]
    kn = np.zeros((nb * B, G))
    for g in range(G):
        kg = O._f64(k_idx[:, g, :])
        kn[:L, g] = np.sqrt((kg * kg).sum(axis=1))
    kmax = kn.reshape(nb, B, G).max(axis=1)                              # [nb, G]
    return qn.T[:, :, None] * kmax.T[:, None, :]                         # [G, n, nb]


def check_scores(gpu: np.ndarray, ref: np.ndarray, bound: np.ndarray, d_idx: int) -> float:
    """gpu/ref/bound: [G, n, NB].  Returns the worst |err| / allowed ratio."""
    ninf_g, ninf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(ninf_g, ninf_r), "-inf positions differ"
    fin = ~ninf_r
    assert np.all(np.isfinite(gpu[fin]))
    allowed = 2 * gamma(d_idx) * bound[fin] + 1e-30
    err = np.abs(gpu[fin].astype(np.float64) - ref[fin])
    worst = float((err / allowed).max()) if err.size else 0.0
    assert worst <= 1.0, f"score error {worst:.3g} x the rounding bound"
    return worst


def check_selection(gpu_idx: np.ndarray, ref_idx: np.ndarray, S: np.ndarray, pos: np.ndarray,
                    B: int, k: int) -> int:
    """gpu_idx/ref_idx: [G, n, k]; S: oracle fp64 scores [G, n, NB].  Returns #unseparated rows."""
    G, n, _ = gpu_idx.shape
    unsep = 0
    for g in range(G):
        for t in range(n):
            J = int(pos[t] // B)
            row = [int(x) for x in gpu_idx[g, t]]
            valid = [x for x in row if x >= 0]
            cnt = min(J + 1, k)
            assert len(valid) == cnt and row[cnt:] == [-1] * (k - cnt), (g, t, row)
            assert valid == sorted(valid) and len(set(valid)) == cnt, (g, t, row)
            assert valid[-1] == J, (g, t, row, J)
            if J <= k - 1:
                assert valid == list(range(J + 1))
                continue
            if k == 1:          # only the current block is kept
                continue
            cand = S[g, t, :J]
            order = np.sort(cand)[::-1]
            delta = 1e-3 * max(abs(order[k - 2]), abs(order[k - 1]))
            kept = np.array(valid[:-1])
            dropped = np.setdiff1d(np.arange(J), kept)
            assert cand[kept].min() >= cand[dropped].max() - delta, (g, t)
            if order[k - 2] - order[k - 1] > delta:
                assert row == [int(x) for x in ref_idx[g, t]], (g, t, row, list(ref_idx[g, t]))
            else:
                unsep += 1
    return unsep


def check_attention(out_gpu: np.ndarray, lse_gpu: Optional[np.ndarray], out_ref: np.ndarray,
                    lse_ref: np.ndarray, dtype: str) -> float:
    tol = TOL_OUT[dtype]
    err = float(np.abs(out_gpu.astype(np.float64) - out_ref).max()) if out_ref.size else 0.0
    assert err <= tol, f"max |O_gpu - O| = {err:.3g} > {tol}"
    if lse_gpu is not None and lse_ref.size:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin)
        lerr = float(np.abs(lse_gpu[fin].astype(np.float64) - lse_ref[fin]).max()) if fin.any() else 0.0
        assert lerr <= tol, f"max |lse_gpu - lse| = {lerr:.3g}"
    return err


def check_topk_every_row(scores, idx_gpu, inp: Dict, B: int, k: int, workers: int = 16) -> int:
    """The Top-k step on its own, on every row: the library's kept lists must
    equal the oracle's selection rule applied to the scores the library was
    given (its own fp32 index scores; the selection is exact on its input).
    The scores themselves are checked against the oracle's on sampled rows.
    Returns the number of (group, row) lists checked."""
    s_h = scores.cpu().numpy()
    i_h = idx_gpu.cpu().numpy()
    q0 = 0
    n = 0
    for lq, lkv in zip(inp["len_q"], inp["len_kv"]):
        if lq == 0:
            continue
        pos = O.query_positions(lq, lkv)
        ref = O.select_blocks_vectorised(s_h[:, q0:q0 + lq, :], pos, B, k, workers=workers)
        bad = np.argwhere(np.any(ref != i_h[:, q0:q0 + lq, :], axis=2))
        assert bad.size == 0, f"{len(bad)} rows differ from the rule, first (group, row) {bad[0]}"
        n += ref.shape[0] * ref.shape[1]
        q0 += lq
    return n


def run_and_check(inp: Dict, H: int, G: int, d: int, d_idx: int, B: int, k: int, dtype: str,
                  rows_per_seq: Optional[Sequence[Sequence[int]]] = None,
                  schedule: str = "auto", shuffle_slots: bool = False,
                  topk_every_row: bool = False, cheap_bound: bool = False,
                  progress: bool = False) -> Dict[str, float]:
    """Run the whole path on the GPU and check sampled rows (all rows if None).

    With shuffle_slots, the attention gets every row's kept-block list in a
    seeded random order (the -1 padding included): the result must not
    depend on the order of the list.  With topk_every_row, the selection of
    every row is also checked against the rule applied to the library's own
    scores (check_topk_every_row).  cheap_bound takes the Cauchy-Schwarz score
    bound (score_bound).  progress prints a line per oracle sequence."""
    prob = problem_for(inp, H, G, d, d_idx, B, k, dtype, schedule)
    dev = inp["q"].device
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    idx_gpu = msa.topk_select(prob, scores)
    cu_q = [0]
    for a in inp["len_q"]:
        cu_q.append(cu_q[-1] + a)
    cu_kv = [0]
    for b in inp["len_kv"]:
        cu_kv.append(cu_kv[-1] + b)
    # oracle per sequence on the sampled rows
    ref = []
    for si, (lq, lkv) in enumerate(zip(inp["len_q"], inp["len_kv"])):
        rows = np.arange(lq) if rows_per_seq is None else np.asarray(rows_per_seq[si], dtype=np.int64)
        if lq == 0 or rows.size == 0:
            ref.append(None)
            continue
        q0, kv0 = cu_q[si], cu_kv[si]
        sl_q, sl_kv = slice(q0, q0 + lq), slice(kv0, kv0 + lkv)
        q_idx_h = inp["q_idx"][sl_q].cpu()
        k_idx_h = inp["k_idx"][sl_kv].cpu()
        k_h = inp["k"][sl_kv].cpu()
        v_h = inp["v"][sl_kv].cpu()
        q_h = inp["q"][sl_q].cpu()
        t0 = time.perf_counter()
        if progress and len(rows) > 128:
            # many rows: upcast K and V once, run the oracle 128 rows at a
            # time and report each piece
            k_h, v_h = O._f64(k_h), O._f64(v_h)
            parts = []
            for c0 in range(0, len(rows), 128):
                parts.append(O.msa_forward(q_h, k_h, v_h, q_idx_h, k_idx_h, lq, lkv, B, k,
                                           1.0 / math.sqrt(d), rows=rows[c0:c0 + 128],
                                           workers=16))
                print(f"  oracle: sequence {si}, rows {c0 + len(parts[-1]['pos'])} of "
                      f"{len(rows)} after {time.perf_counter() - t0:.1f} s", flush=True)
            r = {key: np.concatenate([p[key] for p in parts], axis=1 if key in
                                     ("scores", "block_idx") else 0) for key in parts[0]}
        else:
            r = O.msa_forward(q_h, k_h, v_h, q_idx_h, k_idx_h, lq, lkv, B, k, 1.0 / math.sqrt(d),
                              rows=rows, workers=16)
            if progress:
                print(f"  oracle: sequence {si}, {len(rows)} rows after "
                      f"{time.perf_counter() - t0:.1f} s", flush=True)
        r["rows"] = rows
        r["global_rows"] = rows + q0
        r["bound"] = score_bound(q_idx_h[torch.from_numpy(rows)], k_idx_h, r["pos"], B,
                                 cheap=cheap_bound)
        ref.append(r)
    # attention on the oracle's selection for the sampled rows
    idx_in = idx_gpu.clone()
    for r in ref:
        if r is not None:
            gr = torch.from_numpy(r["global_rows"]).to(dev)
            idx_in[:, gr, :] = torch.from_numpy(r["block_idx"]).to(dev)
    if shuffle_slots:
        gen = torch.Generator(device="cpu").manual_seed(1234)
        perm = torch.rand(idx_in.shape, generator=gen).argsort(dim=-1).to(dev)
        idx_in = torch.gather(idx_in, -1, perm).contiguous()
    out, lse = msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], idx_in, return_lse=True)
    torch.cuda.synchronize()
    stats = {"score_ratio": 0.0, "unseparated": 0, "out_err": 0.0, "rows": 0}
    if topk_every_row:
        t0 = time.perf_counter()
        stats["topk_rows_checked"] = check_topk_every_row(scores, idx_gpu, inp, B, k)
        if progress:
            print(f"  Top-k of every row checked in {time.perf_counter() - t0:.1f} s", flush=True)
    for r in ref:
        if r is None:
            continue
        gr = torch.from_numpy(r["global_rows"]).to(dev)
        nbs = r["scores"].shape[2]
        s_g = scores[:, gr, :].cpu().numpy()
        assert np.all(np.isneginf(s_g[:, :, nbs:])), "padding columns must be -inf"
        stats["score_ratio"] = max(stats["score_ratio"],
                                   check_scores(s_g[:, :, :nbs], r["scores"], r["bound"], d_idx))
        stats["unseparated"] += check_selection(idx_gpu[:, gr, :].cpu().numpy(), r["block_idx"],
                                                r["scores"], r["pos"], B, k)
        stats["out_err"] = max(stats["out_err"], check_attention(
            out[gr].float().cpu().numpy(), lse[gr].cpu().numpy(), r["out"], r["lse"], dtype))
        stats["rows"] += len(r["rows"])
    return stats


def argmax_tie_band(q_idx_rows, k_idx, block_idx: np.ndarray, pos: np.ndarray, B: int,
                    d_idx: int):
    """Slots of the max-pooling backward whose arg-max key fp32 rounding may
    decide either way.

    The oracle takes each kept slot's arg-max from fp64 dot products (ties to
    the lower key).  The library sums each dot product in fp32, within
    gamma_{d_idx} * sum_c |q_c k_c| of the exact value.  A slot is ambiguous
    when some other causal key s of its block comes within the two rounding
    bounds of the winner a: dot_s + bound_s >= dot_a - bound_a.  Returns
    (ambiguous [G, n, k] bool, keys: list over groups of the set of keys that
    an ambiguous slot may pick, its winner included)."""
    q = O._f64(q_idx_rows)
    G, n, K = block_idx.shape
    L = k_idx.shape[0]
    gam = gamma(d_idx)
    amb = np.zeros((G, n, K), dtype=bool)
    keys = [set() for _ in range(G)]
    for g in range(G):
        kg = O._f64(k_idx[:, g, :])
        for t in range(n):
            for i in range(K):
                j = int(block_idx[g, t, i])
                if j < 0:
                    continue
                s0 = j * B
                s1 = min(s0 + B, int(pos[t]) + 1, L)
                if s1 - s0 < 2:
                    continue
                kr = kg[s0:s1]
                dots = kr @ q[t, g]
                bound = gam * (np.abs(kr) @ np.abs(q[t, g]))
                a = int(np.argmax(dots))
                near = dots + bound >= dots[a] - bound[a]
                if near.sum() > 1:
                    amb[g, t, i] = True
                    keys[g].update((s0 + np.flatnonzero(near)).tolist())
    return amb, keys
