"""GPU parity of msa_index_topk (index scoring fused with the Top-k; no score
tensor).  The fused call must give, on every row, exactly the kept lists of
msa_topk_select on msa_index_score's scores (it scores every candidate block
with the same arithmetic and applies the same rule), and those lists must be
delta-valid against the oracle's fp64 selection (exact where the (k-1)-th and
k-th candidates are separated) on the rows the oracle computes."""
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


CASES = [
    # name, len_q, len_kv, G, d_idx, B, k
    ("ragged-1000", [1000], [1000], 2, 64, 128, 4),
    ("varlen-chunked", [300, 1, 700, 0], [300, 513, 1500, 64], 4, 32, 64, 3),
    ("dsi128-k8", [777], [777], 1, 128, 64, 8),
    ("k1", [520], [600], 2, 64, 128, 1),
    ("k-covers-all", [640], [640], 1, 64, 64, 16),
    ("long-rows-k20", [700], [40000], 2, 64, 64, 20),
    ("long-rows-k8-B128", [1500], [90000], 2, 64, 128, 8),
    ("long-rows-k64", [300], [33000], 1, 64, 64, 64),
    ("more-queries-than-keys", [300, 400], [200, 500], 2, 64, 128, 4),
    ("decode", [1] * 7, [1, 127, 128, 129, 5000, 64, 3000], 2, 64, 128, 4),
]


def _fused_vs_unfused(inp, G, di, B, k):
    prob = C.problem_for(inp, 2 * G, G, 64, di, B, k, "bf16")
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    ref = msa.topk_select(prob, scores)
    got = msa.index_topk(prob, inp["q_idx"], inp["k_idx"])
    again = msa.index_topk(prob, inp["q_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    bad = (got != ref).any(dim=2).nonzero()
    assert bad.numel() == 0, f"{bad.shape[0]} (group, row) lists differ from the two-call path, " \
                             f"first {bad[0].tolist()}"
    assert torch.equal(got, again)
    return prob, got


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fused_small_every_row(case):
    name, lq, lkv, G, di, B, k = case
    inp = W.random_case(CASES.index(case) + 80, lq, lkv, 2 * G, G, 64, di, B, k, "bf16",
                        device=DEV)
    prob, got = _fused_vs_unfused(inp, G, di, B, k)
    got_h = got.cpu().numpy()
    q0 = kv0 = 0
    unsep = 0
    for a, b in zip(lq, lkv):
        if a == 0:
            continue
        base = b - a
        rows = np.arange(max(0, -base), a)          # rows with a causal key
        if rows.size:
            pos = O.query_positions(a - rows[0], b)
            S = O.block_scores(inp["q_idx"][q0 + rows[0]:q0 + a].cpu(), inp["k_idx"][kv0:kv0 + b].cpu(),
                               pos, B)
            ref = O.select_blocks(S, pos, B, k)
            unsep += C.check_selection(got_h[:, q0 + rows[0]:q0 + a, :], ref, S, pos, B, k)
        if rows.size < a:
            assert np.all(got_h[:, q0:q0 + (a - rows.size), :] == -1)
        q0, kv0 = q0 + a, kv0 + b
    _log(f"{name}: fused == two-call on every row; delta-valid, {unsep} unseparated rows")


@pytest.mark.parametrize("name", ["prefill-32k", "prefill-128k", "chunked-prefill-1m"])
def test_fused_full_size(name):
    """Every row equal to the two-call path; >= 256 rows (the whole first and
    last 128-query blocks and random rows) delta-valid against the oracle."""
    w = W.WORKLOADS[name]
    _log(f"{name}: generating")
    inp = W.make_inputs(w, device=DEV, seed=0, with_attention=False)
    inp["q"] = inp["q_idx"]     # (unused by the index calls; problem_for reads only lengths)
    lq, lkv = inp["len_q"][0], inp["len_kv"][0]
    prob = C.problem_for(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                         w.block_size, w.top_k, w.dtype)
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    ref = msa.topk_select(prob, scores)
    del scores
    got = msa.index_topk(prob, inp["q_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    bad = (got != ref).any(dim=2).nonzero()
    assert bad.numel() == 0, f"{bad.shape[0]} lists differ, first {bad[0].tolist()}"
    _log(f"{name}: fused == two-call on all {got.shape[0] * got.shape[1]} (group, row) lists")
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(128), np.arange(lq - 128, lq),
                                     rng.integers(0, lq, 64)]))
    pos = O.query_positions(lq, lkv)[rows]
    S = O.block_scores(inp["q_idx"][torch.from_numpy(rows).to(DEV)].cpu(), inp["k_idx"].cpu(), pos,
                       w.block_size, workers=16)
    sel = O.select_blocks(S, pos, w.block_size, w.top_k)
    unsep = C.check_selection(got[:, torch.from_numpy(rows).to(DEV), :].cpu().numpy(), sel, S, pos,
                              w.block_size, w.top_k)
    _log(f"{name}: {len(rows)} rows delta-valid against the oracle ({unsep} unseparated)")
