"""GPU parity of the indexer-KL training calls against the oracle.

msa_sparse_attn_fwd_mass returns the Main Branch mass of every kept block
(averaged over the group's heads) next to the forward pass, and
msa_indexer_kl turns it and the block scores into KL(p || softmax of the
kept scores) and its gradient in the scores.  The oracle's block_mass and
indexer_kl are the references (pinned in test_oracle_pins.py).

Tolerances: the mass comes from fp32 (max, sum) pairs of exact bf16
products, so it is good to ~1e-6; 1e-5 is allowed.  The loss and its
gradient also see the fp32 block scores (relative error ~1e-6 of scores of
magnitude up to ~20): 1e-4 + 1e-4 |kl| for the loss, 2e-5 for the gradient.
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
TOL_MASS = 1e-5
TOL_GRAD = 2e-5


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check(mass, kl, grad, m_ref, kl_ref, g_ref):
    em = float(np.abs(mass - m_ref).max()) if m_ref.size else 0.0
    ek = float((np.abs(kl - kl_ref) / (1e-4 + 1e-4 * np.abs(kl_ref))).max()) if kl_ref.size else 0.0
    eg = float(np.abs(grad - g_ref).max()) if g_ref.size else 0.0
    assert em <= TOL_MASS, f"mass error {em:.3g}"
    assert ek <= 1.0, f"kl error {ek:.3g} x the tolerance"
    assert eg <= TOL_GRAD, f"grad error {eg:.3g}"
    return em, ek, eg


# (H, G, d, d_idx, B, k): k = 6, 20 and 40 take the loss kernel's 16-, 32-
# and 64-lane row segments; the last case has 16 heads per group and B = 64.
KL_CASES = [(8, 2, 128, 64, 128, 6), (4, 4, 64, 32, 64, 20), (16, 1, 64, 64, 64, 40)]


@pytest.mark.parametrize("case", KL_CASES, ids=[f"k{c[5]}-B{c[4]}-hpg{c[0] // c[1]}" for c in KL_CASES])
def test_mass_and_kl_on_arbitrary_lists(case):
    """Seeded kept-block lists (any count of distinct blocks up to J, any slot
    order, empty rows and an empty sequence included), every row checked.
    The forward outputs of the mass call equal msa_sparse_attn_fwd's bit for
    bit."""
    H, G, d, di, B, k = case
    lq, lkv = [700, 1, 300, 0], [3000, 513, 300, 64]
    inp = W.random_case(91, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    lists = W.random_block_lists(91, lq, lkv, G, B, k)
    idx = lists.to(DEV)
    prob = C.problem_for(inp, H, G, d, di, B, k, "bf16")
    _log(f"arbitrary lists {case}: GPU")
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    out_m, lse_m, mass = msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], idx)
    out, lse = msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], idx, return_lse=True)
    kl, grad = msa.indexer_kl(prob, scores, idx, mass)
    torch.cuda.synchronize()
    assert torch.equal(out_m, out) and torch.equal(lse_m, lse)
    _log("arbitrary lists: oracle")
    scale = 1.0 / math.sqrt(d)
    q0 = kv0 = 0
    stats = []
    for a, b in zip(lq, lkv):
        if a > 0:
            pos = O.query_positions(a, b)
            L = lists[:, q0:q0 + a, :].numpy()
            S = O.block_scores(inp["q_idx"][q0:q0 + a].cpu(), inp["k_idx"][kv0:kv0 + b].cpu(), pos, B)
            m_ref = O.block_mass(inp["q"][q0:q0 + a].cpu(), inp["k"][kv0:kv0 + b].cpu(), L, pos, B, scale)
            kl_ref, g_ref = O.indexer_kl(S, L, m_ref)
            stats.append(_check(mass[:, q0:q0 + a].cpu().numpy(), kl[:, q0:q0 + a].cpu().numpy(),
                                grad[:, q0:q0 + a].cpu().numpy(), m_ref, kl_ref, g_ref))
        q0, kv0 = q0 + a, kv0 + b
    _log(f"  (mass err, kl err / tol, grad err) per sequence: {stats}")


def _sample(lq, planted, seed):
    rng = np.random.default_rng(seed)
    rows = set(range(0, 8)) | set(range(lq - 8, lq)) | {127, 128, 4095, 4096}
    rows.update(rng.integers(0, lq, 12).tolist())
    for g_rows in planted:
        if g_rows:
            rows.update(rng.choice(g_rows, size=min(2, len(g_rows)), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < lq))


@pytest.mark.parametrize("name", ["prefill-32k", "prefill-128k", "chunked-prefill-1m"])
def test_mass_and_kl_full_size(name):
    """The long-context workloads in the benchmark's launch configuration:
    properties on every row, the oracle on sampled rows (whose kept lists
    are the oracle's own selection, fed to the GPU)."""
    w = W.WORKLOADS[name]
    _log(f"{name}: generating")
    inp = W.make_inputs(w, device=DEV, seed=0)
    H, G, d, di, B, k = w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim, w.block_size, w.top_k
    prob = C.problem_for(inp, H, G, d, di, B, k, w.dtype)
    lq, lkv = inp["len_q"][0], inp["len_kv"][0]
    rows = _sample(lq, inp["planted_q"][0], 3)
    _log(f"{name}: oracle on {len(rows)} rows")
    scale = 1.0 / math.sqrt(d)
    q_h, k_h, v_h = inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu()
    r = O.msa_forward(q_h, k_h, v_h, inp["q_idx"].cpu(), inp["k_idx"].cpu(), lq, lkv, B, k, scale,
                      rows=rows)
    m_ref = O.block_mass(q_h[torch.from_numpy(rows)], k_h, r["block_idx"], r["pos"], B, scale)
    kl_ref, g_ref = O.indexer_kl(r["scores"], r["block_idx"], m_ref)
    _log(f"{name}: GPU")
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    idx = msa.topk_select(prob, scores)
    gr = torch.from_numpy(rows).to(DEV)
    idx[:, gr, :] = torch.from_numpy(r["block_idx"]).to(DEV)
    _, _, mass = msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], idx)
    kl, grad = msa.indexer_kl(prob, scores, idx, mass)
    torch.cuda.synchronize()
    # every row: a distribution over its kept slots, a loss >= 0, gradients summing to 0
    pad = idx < 0
    assert torch.all(mass >= 0) and torch.all(mass[pad] == 0) and torch.all(grad[pad] == 0)
    assert float((mass.sum(dim=2) - 1).abs().max()) <= 1e-4
    assert float(grad.sum(dim=2).abs().max()) <= 1e-5
    assert float(kl.min()) >= -1e-5
    st = _check(mass[:, gr].cpu().numpy(), kl[:, gr].cpu().numpy(), grad[:, gr].cpu().numpy(),
                m_ref, kl_ref, g_ref)
    _log(f"  mass err {st[0]:.3g}, kl err / tol {st[1]:.3g}, grad err {st[2]:.3g}; "
         f"kl mean {float(kl.mean()):.4f}")
