"""GPU parity of msa_index_topk_hier (hierarchical coarse-to-fine selection,
an approximation of index scoring + Top-k) against the oracle's
hierarchical_select.

* Keeping every chunk reduces it to the exact selection: the kept lists must
  equal msa_topk_select on msa_index_score's scores bit for bit (the fine
  scores use the same MFMA arithmetic).
* With few kept chunks: the coarse scores are fp32 (chunk means summed in
  fp32, then an fp32 dot product); where the C-th and (C+1)-th coarse scores
  of a row lie within twice their rounding bound, either chunk may be kept.
  Rows outside that band must keep exactly the oracle's chunks, and their
  final lists must be a delta-valid Top-k of the oracle's fine scores over the
  oracle's fine candidates.  Rows inside the band are counted.
* Recall against the exact selection is reported (a metric, not a bar).
"""
import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_long_msa_amd as msa
import workloads as W
from oracle import msa_oracle as O
from tests import msa_check as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _coarse_band(q_idx_rows, k_idx, pos, B, S, keep, d_idx):
    """Rows (g, t) whose keep-th and (keep+1)-th coarse scores are within twice
    the fp32 rounding bound of the chunk means and the dot product."""
    q = O._f64(q_idx_rows)
    k = O._f64(k_idx)
    L, G, di = k.shape
    span = B * S
    nfull = L // span
    kbar = k[:nfull * span].reshape(nfull, span, G, di).mean(axis=1)
    kabs = np.abs(k[:nfull * span]).reshape(nfull, span, G, di).mean(axis=1)
    g_mean = C.gamma(span // 4 + 3)           # four ordered partial sums, then three adds
    g_dot = C.gamma(d_idx)
    n = q.shape[0]
    amb = np.zeros((G, n), dtype=bool)
    for g in range(G):
        for t in range(n):
            cJ = int(pos[t] // B) // S
            if cJ <= keep:
                continue
            sc = kbar[:cJ, g] @ q[t, g]
            bd = (g_dot * (np.abs(kbar[:cJ, g]) @ np.abs(q[t, g]))
                  + g_mean * (kabs[:cJ, g] @ np.abs(q[t, g])))
            order = np.sort(sc)[::-1]
            if order[keep - 1] - order[keep] <= 2 * bd.max():
                amb[g, t] = True
    return amb


def _check_against_oracle(got_idx, got_kept, q_idx_rows, k_idx, pos, B, k, S, keep, d_idx):
    """got_*: [G, n, *] numpy for the rows at `pos`.  Returns (rows checked, rows in the band)."""
    ref = O.hierarchical_select(q_idx_rows, k_idx, pos, B, k, S, keep)
    amb = _coarse_band(q_idx_rows, k_idx, pos, B, S, keep, d_idx)
    G, n, _ = got_idx.shape
    checked = 0
    for g in range(G):
        for t in range(n):
            row = [int(x) for x in got_idx[g, t]]
            J = int(pos[t] // B)
            valid = [x for x in row if x >= 0]
            assert len(valid) == min(J + 1, k) and valid == sorted(valid) and valid[-1] == J
            if amb[g, t]:
                continue
            assert got_kept[g, t].tolist() == ref["kept_chunks"][g, t].tolist(), (g, t)
            if J <= k - 1:
                assert valid == list(range(J + 1))
                checked += 1
                continue
            fine = ref["fine"][g, t]
            cand = np.flatnonzero(np.isfinite(fine[:J]))
            kept = np.array(valid[:-1])
            assert np.all(np.isin(kept, cand)), (g, t)
            order = np.sort(fine[cand])[::-1]
            if k > 1 and len(cand) > k - 1:
                delta = 1e-3 * max(abs(order[k - 2]), abs(order[k - 1]))
                dropped = np.setdiff1d(cand, kept)
                assert fine[kept].min() >= fine[dropped].max() - delta, (g, t)
                if order[k - 2] - order[k - 1] > delta:
                    assert row == [int(x) for x in ref["block_idx"][g, t]], (g, t)
            checked += 1
    return checked, int(amb.sum())


CASES = [
    # name, len_q, len_kv, G, d_idx, B, k, S, keep
    ("b128-s4-keep3", [1500], [6000], 2, 64, 128, 4, 4, 3),
    ("b64-s8-keep2-varlen", [700, 1, 300], [9000, 513, 300], 2, 32, 64, 6, 8, 2),
    ("b64-s2-keep6-k12", [800], [12000], 1, 128, 64, 12, 2, 6),
    ("decode", [1] * 5, [9000, 127, 70000, 3000, 40000], 2, 64, 128, 8, 8, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_hier_small(case):
    name, lq, lkv, G, di, B, k, S, keep = case
    inp = W.random_case(CASES.index(case) + 120, lq, lkv, 2 * G, G, 64, di, B, k, "bf16",
                        device=DEV)
    prob = C.problem_for(inp, 2 * G, G, 64, di, B, k, "bf16")
    # every chunk kept: the exact selection, bit for bit
    nch = -(-prob.nb_max // S)
    exact = msa.topk_select(prob, msa.index_score(prob, inp["q_idx"], inp["k_idx"]))
    full = msa.index_topk_hier(prob, inp["q_idx"], inp["k_idx"], S, max(nch, keep))
    torch.cuda.synchronize()
    assert torch.equal(full, exact), "keeping every chunk must give the exact selection"
    got, kept = msa.index_topk_hier(prob, inp["q_idx"], inp["k_idx"], S, keep, return_kept=True)
    again = msa.index_topk_hier(prob, inp["q_idx"], inp["k_idx"], S, keep)
    torch.cuda.synchronize()
    assert torch.equal(got, again)
    q0 = kv0 = 0
    checked = band = 0
    for a, b in zip(lq, lkv):
        pos = O.query_positions(a, b)
        c_, b_ = _check_against_oracle(got[:, q0:q0 + a].cpu().numpy(), kept[:, q0:q0 + a].cpu().numpy(),
                                       inp["q_idx"][q0:q0 + a].cpu(), inp["k_idx"][kv0:kv0 + b].cpu(),
                                       pos, B, k, S, keep, di)
        checked, band = checked + c_, band + b_
        q0, kv0 = q0 + a, kv0 + b
    rec = float(O.selection_recall(got.cpu().numpy(), exact.cpu().numpy(),
                                   np.concatenate([O.query_positions(a, b) for a, b in zip(lq, lkv)]),
                                   B, k))
    _log(f"{name}: {checked} (group, row) lists match the oracle, {band} in the coarse tie band; "
         f"recall vs exact {rec:.3f}")


def hier_defaults(w):
    """Chunks of 16 blocks; keep enough for twice the free picks."""
    S = 16
    return S, max(1, -(-2 * (w.top_k - 1) // S))


@pytest.mark.parametrize("name", ["prefill-128k", "chunked-prefill-1m"])
def test_hier_full_size(name):
    """The benchmark workloads with the default chunking: every row well
    formed, 160 rows against the oracle, and the recall of every row against
    the exact selection (reported; an approximation has no exactness bar)."""
    w = W.WORKLOADS[name]
    S, keep = hier_defaults(w)
    _log(f"{name}: generating (chunks of {S} blocks, keep {keep})")
    inp = W.make_inputs(w, device=DEV, seed=0, with_attention=False)
    inp["q"] = inp["q_idx"]
    lq, lkv = inp["len_q"][0], inp["len_kv"][0]
    B, k = w.block_size, w.top_k
    prob = C.problem_for(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim, B, k, w.dtype)
    got, kept = msa.index_topk_hier(prob, inp["q_idx"], inp["k_idx"], S, keep, return_kept=True)
    exact = msa.topk_select(prob, msa.index_score(prob, inp["q_idx"], inp["k_idx"]))
    torch.cuda.synchronize()
    pos = torch.arange(lkv - lq, lkv, device=DEV)
    J = (pos // B).view(1, -1, 1)
    valid = got >= 0
    assert torch.all(valid.sum(dim=2) == torch.clamp(J[:, :, 0] + 1, max=k))
    assert torch.all(torch.where(valid, got, torch.full_like(got, -1)).max(dim=2).values == J[:, :, 0])
    # recall of the free picks, every row with J > k-1
    free_e = (exact >= 0) & (exact < J)
    free_h = (got >= 0) & (got < J)
    hit = (free_e.unsqueeze(3) & free_h.unsqueeze(2) & (exact.unsqueeze(3) == got.unsqueeze(2))).sum()
    recall = float(hit) / float(free_e.sum())
    # planted queries: share of the planted blocks the exact selection keeps that survive
    hitp = totp = 0
    for g in range(w.num_kv_groups):
        rows = torch.tensor(inp["planted_q"][0][g], device=DEV)
        blocks = torch.tensor(inp["planted_blocks"][0][g], device=DEV)
        e_rows, h_rows = exact[g, rows], got[g, rows]
        pe = torch.isin(e_rows, blocks) & (e_rows < J[0, rows])
        inter = (pe.unsqueeze(2) & (e_rows.unsqueeze(2) == h_rows.unsqueeze(1))).any(dim=2)
        hitp += int(inter.sum())
        totp += int(pe.sum())
    _log(f"{name}: recall of the exact free picks {recall:.3f}; of the planted blocks on planted "
         f"queries {hitp / max(totp, 1):.3f}")
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(lq - 64, lq), rng.integers(0, lq, 96)]))
    tr = torch.from_numpy(rows).to(DEV)
    checked, band = _check_against_oracle(got[:, tr].cpu().numpy(), kept[:, tr].cpu().numpy(),
                                          inp["q_idx"][tr].cpu(), inp["k_idx"].cpu(),
                                          O.query_positions(lq, lkv)[rows], B, k, S, keep,
                                          w.idx_dim)
    _log(f"{name}: {checked} sampled (group, row) lists match the oracle, {band} in the coarse "
         f"tie band")
