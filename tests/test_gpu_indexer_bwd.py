"""GPU parity of msa_indexer_bwd (the Index Branch max-pooling backward)
against the oracle's index_backward.

The oracle takes each kept slot's arg-max key from fp64 dot products (ties to
the lower key); the library from fp32 sums.  Where another causal key of the
block comes within the two fp32 rounding bounds of the winner, either key is a
correct arg-max: those slots are flagged (msa_check.argmax_tie_band), the rows
and keys they touch are left out of the element-wise comparison and counted,
and every other row and key must be within 1e-4 + 1e-5 |ref| of the oracle's
fp64 sums.  On small-integer inputs every fp32 sum is exact, so nothing is
left out there, exact ties included.  At full size, where the key-side sums cannot be
sampled, the identity sum_s <dk_idx[s], k_idx[s]> = sum_r <dq_idx[r], q_idx[r]>
= sum over kept slots of grad * score (a max-pooled score is linear in the
query and in its arg-max key) is checked for every group.
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


def _close(gpu, ref, name):
    err = np.abs(gpu - ref) / (1e-4 + 1e-5 * np.abs(ref))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= 1.0, f"{name}: error {worst:.3g} x the tolerance"
    return worst


BWD_CASES = [
    # name, len_q, len_kv, G, d_idx, B, k, dtype
    ("varlen-bf16", [700, 1, 300, 0], [1500, 513, 300, 64], 2, 64, 128, 6, "bf16"),
    ("di32-B64-bf16", [640], [2000], 4, 32, 64, 20, "bf16"),
    ("di128-f32", [500, 260], [500, 900], 1, 128, 64, 9, "f32"),
]


def _compare_outside_band(dq, dk, q_idx, k_idx, lists, pos, B, grad, di, exact=False):
    """dq [n, G, di] and dk [L, G, di] of one sequence against the oracle,
    except the rows and keys an ambiguous slot touches.  Returns (worst
    error / tolerance, rows left out, keys left out)."""
    dq_r, dk_r = O.index_backward(q_idx, k_idx, lists, pos, B, grad)
    G = lists.shape[0]
    row_ok = np.ones((dq_r.shape[0], G), dtype=bool)
    key_ok = np.ones((dk_r.shape[0], G), dtype=bool)
    if not exact:
        amb, keys = C.argmax_tie_band(q_idx, k_idx, lists, pos, B, di)
        row_ok &= ~amb.any(axis=2).T
        for g in range(G):
            key_ok[sorted(keys[g]), g] = False
    worst = max(_close(dq[row_ok], dq_r[row_ok], "dq_idx"),
                _close(dk[key_ok], dk_r[key_ok], "dk_idx"))
    return worst, int((~row_ok).sum()), int((~key_ok).sum())


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_index_backward_small(case):
    """Seeded kept lists (distinct blocks up to J, any order, empty rows) and
    seeded slot gradients; every row and key outside the rounding tie band
    checked."""
    name, lq, lkv, G, di, B, k, dtype = case
    H, d = 2 * G, 64
    inp = W.random_case(41, lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    lists = W.random_block_lists(41, lq, lkv, G, B, k)
    grad = W.random_slot_grads(41, G, sum(lq), k)
    prob = C.problem_for(inp, H, G, d, di, B, k, dtype)
    _log(f"{name}: GPU")
    dq, dk = msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], lists.to(DEV), grad.to(DEV))
    dq2, dk2 = msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], lists.to(DEV), grad.to(DEV))
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2), "not deterministic"
    _log(f"{name}: oracle")
    q0 = kv0 = 0
    worst, rows_out, keys_out = 0.0, 0, 0
    for a, b in zip(lq, lkv):
        pos = O.query_positions(a, b) if a > 0 else np.zeros(0, np.int64)
        wst, ro, ko = _compare_outside_band(
            dq[q0:q0 + a].cpu().numpy(), dk[kv0:kv0 + b].cpu().numpy(),
            inp["q_idx"][q0:q0 + a].cpu(), inp["k_idx"][kv0:kv0 + b].cpu(),
            lists[:, q0:q0 + a, :].numpy(), pos, B, grad[:, q0:q0 + a, :].numpy(), di)
        worst, rows_out, keys_out = max(worst, wst), rows_out + ro, keys_out + ko
        q0, kv0 = q0 + a, kv0 + b
    _log(f"  worst error / tolerance {worst:.3g}; left out (tie band): "
         f"{rows_out} (row, group) pairs of {sum(lq) * G}, {keys_out} (key, group) pairs "
         f"of {sum(lkv) * G}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_index_backward_exact_ties_small_integers(dtype):
    """Index vectors of small integers: every dot product and every fp32
    partial sum is exact, so the library's arg-max must be the oracle's on
    every slot, exact ties (to the lower key) included, with no tie band."""
    lq, lkv, G, di, B, k = [400, 130], [900, 130], 2, 64, 64, 7
    H, d = 2 * G, 64
    inp = W.random_case(43, lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    inp["q_idx"] = W.small_int_tensor(43, (sum(lq), G, di), 2, dtype).to(DEV)
    inp["k_idx"] = W.small_int_tensor(44, (sum(lkv), G, di), 1, dtype).to(DEV)
    lists = W.random_block_lists(43, lq, lkv, G, B, k)
    grad = W.random_slot_grads(43, G, sum(lq), k)
    prob = C.problem_for(inp, H, G, d, di, B, k, dtype)
    dq, dk = msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], lists.to(DEV), grad.to(DEV))
    torch.cuda.synchronize()
    q0 = kv0 = 0
    ties, worst = 0, 0.0
    for a, b in zip(lq, lkv):
        pos = O.query_positions(a, b)
        qh, kh = inp["q_idx"][q0:q0 + a].cpu(), inp["k_idx"][kv0:kv0 + b].cpu()
        li = lists[:, q0:q0 + a, :].numpy()
        wst, ro, ko = _compare_outside_band(dq[q0:q0 + a].cpu().numpy(),
                                            dk[kv0:kv0 + b].cpu().numpy(), qh, kh, li, pos, B,
                                            grad[:, q0:q0 + a, :].numpy(), di, exact=True)
        assert ro == 0 and ko == 0
        worst = max(worst, wst)
        amb, _ = C.argmax_tie_band(qh, kh, li, pos, B, di)
        ties += int(amb.sum())      # slots with an exact tie (the band is 0 here)
        q0, kv0 = q0 + a, kv0 + b
    assert ties > 0, "the case should hold exact ties"
    _log(f"  {dtype}: worst error / tolerance {worst:.3g}; slots with a tied maximum: {ties}")


@pytest.mark.parametrize("name", ["prefill-32k", "prefill-128k", "chunked-prefill-1m"])
def test_index_backward_full_size(name):
    """The long-context workloads after the GPU's own index scores and Top-k:
    the identity above on every group, and dq_idx on sampled rows against
    the oracle (their kept lists are the oracle's own selection)."""
    w = W.WORKLOADS[name]
    _log(f"{name}: generating")
    inp = W.make_inputs(w, device=DEV, seed=0, with_attention=False)
    G, di, B, k = w.num_kv_groups, w.idx_dim, w.block_size, w.top_k
    prob = C.problem_for(inp, w.num_q_heads, G, w.head_dim, di, B, k, w.dtype)
    lq, lkv = inp["len_q"][0], inp["len_kv"][0]
    rng = np.random.default_rng(5)
    rows = np.array(sorted(set([0, 1, 127, 128, lq - 1] + rng.integers(0, lq, 16).tolist())))
    _log(f"{name}: oracle selection on {len(rows)} rows")
    pos = O.query_positions(lq, lkv)[rows]
    q_idx_h, k_idx_h = inp["q_idx"].cpu(), inp["k_idx"].cpu()
    S_ref = O.block_scores(q_idx_h[torch.from_numpy(rows)], k_idx_h, pos, B)
    idx_ref = O.select_blocks(S_ref, pos, B, k)
    grad = W.random_slot_grads(7, G, lq, k)
    _log(f"{name}: GPU")
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    idx = msa.topk_select(prob, scores)
    gr = torch.from_numpy(rows).to(DEV)
    idx[:, gr, :] = torch.from_numpy(idx_ref).to(DEV)
    dq, dk = msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], idx, grad.to(DEV))
    torch.cuda.synchronize()
    # identity per group, in fp64 on the GPU's outputs and its own scores
    qf, kf = inp["q_idx"].double(), inp["k_idx"].double()
    sc = torch.gather(scores, 2, idx.clamp(min=0).long()).double()
    lhs_all = (dq.double() * qf).sum(dim=(0, 2))
    rhs_all = (dk.double() * kf).sum(dim=(0, 2))
    gsum = (grad.to(DEV).double() * sc * (idx >= 0)).sum(dim=(1, 2))
    for g in range(G):
        scale = float((grad.to(DEV).double().abs() * sc.abs() * (idx >= 0))[g].sum())
        for what, v in (("<dq, q>", lhs_all[g]), ("<dk, k>", rhs_all[g])):
            rel = abs(float(v) - float(gsum[g])) / scale
            assert rel < 1e-5, f"{name}, group {g}: {what} off by {rel:.3g} of sum |grad * score|"
    # sampled rows against the oracle, outside the rounding tie band
    dq_r, _ = O.index_backward(q_idx_h[torch.from_numpy(rows)], k_idx_h, idx_ref, pos, B,
                               grad[:, torch.from_numpy(rows), :].numpy())
    amb, _ = C.argmax_tie_band(q_idx_h[torch.from_numpy(rows)], k_idx_h, idx_ref, pos, B, di)
    row_ok = ~amb.any(axis=2).T
    worst = _close(dq[gr].cpu().numpy()[row_ok], dq_r[row_ok], "dq_idx")
    _log(f"  sampled dq_idx worst error / tolerance {worst:.3g}; "
         f"{int((~row_ok).sum())} of {row_ok.size} (row, group) pairs in the tie band")
    # dk_idx on every key of two blocks (a late one, and the one of group G-1
    # the most rows keep): the oracle over every (row, slot) that names the
    # block, which are the only slots whose gradient reaches its keys
    idx_h, grad_h = idx.cpu().numpy(), grad.numpy()
    pos_all = O.query_positions(lq, lkv)
    nb = (lkv + B - 1) // B
    last = idx_h[G - 1]
    popular = int(np.argmax(np.bincount(last[last >= 0], minlength=nb)))
    for g, jb in ((0, nb - 2), (G - 1, popular)):
        hit = idx_h[g] == jb                       # [lq, k]
        keep = np.nonzero(hit.any(axis=1))[0]
        _log(f"{name}: oracle dk_idx of block {jb}, group {g} ({keep.size} rows keep it)")
        sub = np.full((G, keep.size, k), -1, dtype=np.int32)
        sub[g] = np.where(hit[keep], jb, -1)
        gsub = np.zeros((G, keep.size, k))
        gsub[g] = np.where(hit[keep], grad_h[g][keep], 0.0)
        tk = torch.from_numpy(keep)
        _, dk_r = O.index_backward(q_idx_h[tk], k_idx_h, sub, pos_all[keep], B, gsub)
        _, band = C.argmax_tie_band(q_idx_h[tk], k_idx_h, sub, pos_all[keep], B, di)
        ks = np.array([s for s in range(jb * B, min((jb + 1) * B, lkv)) if s not in band[g]])
        e = _close(dk[torch.from_numpy(ks).to(DEV), g].cpu().numpy(), dk_r[ks, g],
                   f"dk_idx block {jb} group {g}")
        _log(f"  dk_idx worst error / tolerance {e:.3g}; {B - ks.size} keys in the tie band")


def test_training_calls_with_more_queries_than_keys():
    """Rows at negative positions (a sequence with len_q > len_kv) have no
    causal key: their block mass, loss, score gradient and index-query
    gradient are 0 and they add nothing to dk_idx.  Every other output equals,
    bit for bit, that of the trimmed problem (the sequence keeps its last
    len_kv queries), whose rows the small-case tests check against the oracle."""
    H, G, d, di, B, k = 8, 2, 128, 64, 128, 4
    inp = W.random_case(78, [300, 400], [200, 500], H, G, d, di, B, k, "bf16", device=DEV)
    cut = 100
    trim = dict(inp)
    trim["len_q"] = [200, 400]
    trim["cu_q"] = torch.tensor([0, 200, 600], dtype=torch.int64, device=DEV)
    for key in ("q_idx", "q"):
        trim[key] = inp[key][cut:].contiguous()
    res = []
    for case in (inp, trim):
        prob = C.problem_for(case, H, G, d, di, B, k, "bf16")
        scores = msa.index_score(prob, case["q_idx"], case["k_idx"])
        idx = msa.topk_select(prob, scores)
        _, _, mass = msa.sparse_attn_fwd_mass(prob, case["q"], case["k"], case["v"], idx)
        kl, grad = msa.indexer_kl(prob, scores, idx, mass)
        dq, dk = msa.indexer_bwd(prob, case["q_idx"], case["k_idx"], idx, grad)
        res.append((mass, kl, grad, dq, dk))
    torch.cuda.synchronize()
    (m_f, kl_f, g_f, dq_f, dk_f), (m_t, kl_t, g_t, dq_t, dk_t) = res
    assert torch.all(m_f[:, :cut] == 0) and torch.all(kl_f[:, :cut] == 0)
    assert torch.all(g_f[:, :cut] == 0) and torch.all(dq_f[:cut] == 0)
    assert torch.equal(m_f[:, cut:], m_t) and torch.equal(kl_f[:, cut:], kl_t)
    assert torch.equal(g_f[:, cut:], g_t) and torch.equal(dq_f[cut:], dq_t)
    assert torch.equal(dk_f, dk_t)
