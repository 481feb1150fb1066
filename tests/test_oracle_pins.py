"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test ties one oracle function to something independent: a hand-worked
example, an exhaustive search, a closed form, or a different library's
implementation of a special case (torch's scaled_dot_product_attention in
float64 on the CPU, scipy's softmax).  A plausible slip in the oracle (a
dropped causal mask, an off-by-one block edge, a wrong tie order, a
transposed operand, a per-block instead of joint softmax) fails at least one.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import msa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_small.json")
GOLDEN_CHUNK = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_chunk.json")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


# ----------------------------------------------------------------- golden ---

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def test_golden_scores_and_selection():
    gd = _golden()
    k_idx = np.array(gd["k_idx"], float)[:, None, :]
    q_idx = np.array(gd["q_idx"], float)[:, None, :]
    pos = O.query_positions(6, 6)
    S = O.block_scores(q_idx, k_idx, pos, gd["block_size"])
    exp = np.array([[np.nan if v is None else v for v in row] for row in gd["scores"]])
    got = S[0]
    assert np.array_equal(np.isinf(got), np.isnan(exp))
    assert np.array_equal(got[~np.isinf(got)], exp[~np.isnan(exp)])
    idx = O.select_blocks(S, pos, gd["block_size"], gd["top_k"])
    assert idx[0].tolist() == gd["block_idx"]


def test_golden_attention_zero_q():
    gd = _golden()
    a = gd["attention_zero_q"]
    pos = O.query_positions(6, 6)
    idx = np.array(gd["block_idx"], np.int32)[None]
    q = np.zeros((6, 1, 1))
    k = np.array(gd["k_idx"], float)[:, None, :1]   # any keys: Q = 0
    v = np.array(a["v"], float)[:, None, None]
    out, lse = O.sparse_attention(q, k, v, idx, pos, gd["block_size"], 1.0)
    assert np.allclose(out[:, 0, 0], a["out"], rtol=0, atol=1e-15)
    assert np.allclose(lse[:, 0], np.log(a["lse_terms"]), rtol=0, atol=1e-15)
    for t in range(6):
        assert O.kept_keys(idx[0, t], t, gd["block_size"]).tolist() == a["kept_keys"][t]


def test_golden_attention_pow2():
    gd = _golden()
    a = gd["attention_pow2"]
    pos = O.query_positions(6, 6)
    idx = np.array(gd["block_idx"], np.int32)[None]
    q = np.full((6, 1, 1), math.log(2.0))
    k = np.array(a["k"], float)[:, None, None]
    v = np.array(a["v"], float)[:, None, None]
    out, lse = O.sparse_attention(q, k, v, idx, pos, gd["block_size"], 1.0)
    rows = a["rows"]
    assert np.allclose(out[rows, 0, 0], a["out"], rtol=0, atol=1e-14)
    assert np.allclose(lse[rows, 0], np.log(a["lse_terms"]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("levels", [0, 1, 3])
def test_select_blocks_vectorised_equals_select_blocks(levels):
    """The whole-tensor form of the selection rule gives the row loop's
    result, on rows with many exact ties (integer scores), constant rows,
    rows with J <= k-1, and k = 1."""
    rng = np.random.default_rng(31 + levels)
    for nb, n, B, k in ((40, 300, 8, 7), (33, 129, 8, 1), (64, 120, 2, 64), (17, 60, 4, 2)):
        L = nb * B
        pos = O.query_positions(n, L)
        if levels:
            S = rng.integers(-levels, levels + 1, (2, n, nb)).astype(np.float32)
        else:
            S = rng.standard_normal((2, n, nb)).astype(np.float32)
        S[:, ::11, :] = 0.5
        ref = O.select_blocks(S, pos, B, k)
        got = O.select_blocks_vectorised(S, pos, B, k, row_chunk=37)
        assert np.array_equal(got, ref), (nb, n, B, k)


def test_golden_selection_ties():
    gd = _golden()["selection_ties"]
    S = np.array(gd["scores"], float)[None, None, :]
    pos = np.array([gd["position"]])
    for k, expected in gd["cases"]:
        assert O.select_blocks(S, pos, gd["block_size"], k)[0, 0].tolist() == expected


@pytest.mark.parametrize("part", ["chunk", "decode"])
def test_golden_fewer_queries_than_keys(part):
    """Queries are the LAST len_q tokens: a 2-query chunk and a decode row of
    a 6-token sequence, worked by hand with their positions written out
    (hand_worked_chunk.json).  The whole-path call derives the positions from
    (len_q, len_kv) itself, so an oracle that put the queries at the first
    len_q positions fails here."""
    with open(GOLDEN_CHUNK) as f:
        gd = json.load(f)
    c = gd[part]
    B, k = gd["block_size"], gd["top_k"]
    k_idx = np.array(gd["k_idx"], float)[:, None, :]
    q_idx = np.array(c["q_idx"], float)[:, None, :]
    n, L = c["len_q"], c["len_kv"]
    assert O.query_positions(n, L).tolist() == c["positions"]
    v = np.arange(L, dtype=float)[:, None, None]
    kk = np.zeros((L, 1, 1))
    q0 = np.zeros((n, 1, 1))
    r = O.msa_forward(q0, kk, v, q_idx, k_idx, n, L, B, k, 1.0)
    assert r["pos"].tolist() == c["positions"]
    assert np.array_equal(r["scores"][0], np.array(c["scores"], float))
    assert r["block_idx"][0].tolist() == c["block_idx"]
    assert np.allclose(r["out"][:, 0, 0], c["zero_q_out"], rtol=0, atol=1e-15)
    assert np.allclose(r["lse"][:, 0], np.log(c["zero_q_lse_terms"]), rtol=0, atol=1e-15)
    # the same rows through the step functions with the hand-written positions
    pos = np.array(c["positions"])
    S = O.block_scores(q_idx, k_idx, pos, B)
    assert np.array_equal(S[0], np.array(c["scores"], float))
    assert O.select_blocks(S, pos, B, k)[0].tolist() == c["block_idx"]


# ------------------------------------------------------------ block scores ---

def _scores_by_loops(q_idx, k_idx, pos, B):
    """Brute force with Python loops and math.fsum (no matrix products)."""
    n, G, _ = q_idx.shape
    L = k_idx.shape[0]
    nb = -(-L // B)
    S = np.full((G, n, nb), -np.inf)
    for g in range(G):
        for t in range(n):
            for s in range(L):
                if s > pos[t]:
                    continue
                dot = math.fsum(float(a) * float(b) for a, b in zip(q_idx[t, g], k_idx[s, g]))
                j = s // B
                S[g, t, j] = max(S[g, t, j], dot)
    return S


@pytest.mark.parametrize("L,lq,B,G,di", [(37, 37, 8, 2, 3), (50, 7, 16, 1, 5), (9, 9, 4, 3, 2),
                                          (64, 64, 64, 1, 4), (65, 1, 8, 2, 3)])
def test_scores_match_loop_bruteforce(L, lq, B, G, di):
    rng = np.random.default_rng(L * 100 + B)
    q = _rand(rng, lq, G, di)
    k = _rand(rng, L, G, di)
    pos = O.query_positions(lq, L)
    S = O.block_scores(q, k, pos, B)
    ref = _scores_by_loops(q, k, pos, B)
    assert np.array_equal(np.isinf(S), np.isinf(ref))
    fin = ~np.isinf(ref)
    assert np.allclose(S[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_scores_block_one_is_masked_dot_matrix():
    """B = 1: every block is one key, so S is the causally masked q_idx k_idx^T."""
    rng = np.random.default_rng(3)
    q = _rand(rng, 20, 2, 6)
    k = _rand(rng, 20, 2, 6)
    pos = O.query_positions(20, 20)
    S = O.block_scores(q, k, pos, 1)
    for g in range(2):
        full = torch.from_numpy(q[:, g]) @ torch.from_numpy(k[:, g]).T   # torch, not numpy
        full = full.masked_fill(torch.ones(20, 20, dtype=torch.bool).triu(1), -math.inf)
        fin = ~np.isinf(S[g])
        assert np.array_equal(fin, ~np.isinf(full.numpy()))
        assert np.allclose(S[g][fin], full.numpy()[fin], rtol=1e-13, atol=1e-13)


def test_scores_invariant_to_key_order_inside_block():
    rng = np.random.default_rng(4)
    L, B = 96, 16
    q = _rand(rng, 8, 2, 4)
    k = _rand(rng, L, 2, 4)
    pos = O.query_positions(8, L)          # positions 88..95: blocks 0..4 fully causal
    S = O.block_scores(q, k, pos, B)
    k2 = k.copy()
    for j in range(5):
        perm = rng.permutation(B)
        k2[j * B:(j + 1) * B] = k[j * B + perm]
    S2 = O.block_scores(q, k2, pos, B)
    assert np.allclose(S, S2, rtol=1e-13, atol=1e-13)


def test_scores_pick_max_not_other_pooling():
    """A single huge key in a block must set the block score (max-pooling)."""
    L, B = 32, 8
    q = np.ones((1, 1, 2))
    k = np.zeros((L, 1, 2))
    k[13, 0] = [5.0, 5.0]       # block 1
    k[2, 0] = [-50.0, 0.0]      # block 0: a large negative key must not matter
    S = O.block_scores(q, k, np.array([31]), B)
    assert S[0, 0].tolist() == [0.0, 10.0, 0.0, 0.0]


# --------------------------------------------------------------- selection ---

def _dominates(S_row, sel, cand):
    """Every kept candidate beats every dropped one under (score desc, index asc)."""
    for a in sel:
        for b in cand:
            if b in sel:
                continue
            if not (S_row[a] > S_row[b] or (S_row[a] == S_row[b] and a < b)):
                return False
    return True


@pytest.mark.parametrize("seed", range(6))
def test_selection_is_the_unique_dominating_subset(seed):
    """Exhaustive search over all subsets of size k-1 on tiny rows with many ties."""
    rng = np.random.default_rng(seed)
    B, L = 2, 16
    nb = L // B
    n = L
    S = rng.integers(-2, 3, size=(1, n, nb)).astype(float)   # small integers -> ties
    pos = O.query_positions(n, L)
    for k in (1, 2, 3, 5, 9):
        idx = O.select_blocks(S, pos, B, k)
        for t in range(n):
            J = pos[t] // B
            cand = list(range(J))
            row = idx[0, t]
            valid = [int(j) for j in row if j >= 0]
            assert valid == sorted(valid), "output must be ascending"
            assert valid[-1] == J, "current block must be kept"
            assert all(j == -1 for j in row[len(valid):])
            if len(cand) <= k - 1:
                assert valid == list(range(J + 1))
                continue
            winners = [set(c) for c in itertools.combinations(cand, k - 1)
                       if _dominates(S[0, t], set(c), cand)]
            assert len(winners) == 1
            assert set(valid[:-1]) == winners[0]


def test_selection_forced_block_even_if_worst():
    S = np.array([[[9.0, 8.0, 7.0, -100.0]]])
    idx = O.select_blocks(S, np.array([7]), 2, 2)    # current block 3 scores worst
    assert idx[0, 0].tolist() == [0, 3]


# --------------------------------------------------------------- attention ---

def _case(seed, L, lq, H, G, d, B):
    rng = np.random.default_rng(seed)
    return (_rand(rng, lq, H, d), _rand(rng, L, G, d), _rand(rng, L, G, d),
            O.query_positions(lq, L))


def _sdpa(q, k, v, mask, scale):
    """torch SDPA in float64 on CPU; mask [n, L] bool (True = attend)."""
    n, H, d = q.shape
    G = k.shape[1]
    hpg = H // G
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [H, n, d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hpg, 0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hpg, 0).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("L,lq,B", [(40, 40, 8), (64, 64, 16), (70, 13, 16), (33, 1, 8)])
def test_dense_when_k_covers_every_block(L, lq, B):
    """k >= number of blocks: MSA is plain causal attention (torch SDPA, fp64)."""
    H, G, d = 4, 2, 8
    q, k, v, pos = _case(L + lq, L, lq, H, G, d, B)
    q_idx = np.random.default_rng(1).standard_normal((lq, G, 3))
    k_idx = np.random.default_rng(2).standard_normal((L, G, 3))
    scale = 1 / math.sqrt(d)
    nb = -(-L // B)
    res = O.msa_forward(q, k, v, q_idx, k_idx, lq, L, B, nb, scale)
    mask = np.arange(L)[None, :] <= pos[:, None]
    ref = _sdpa(q, k, v, mask, scale)
    assert np.abs(res["out"] - ref).max() < 1e-12


@pytest.mark.parametrize("L,lq,B", [(48, 48, 8), (70, 20, 16)])
def test_k1_attends_only_current_block(L, lq, B):
    """k = 1: only keys in [B*floor(p/B), p] are attended (local causal window)."""
    H, G, d = 2, 1, 8
    q, k, v, pos = _case(7, L, lq, H, G, d, B)
    rng = np.random.default_rng(8)
    q_idx, k_idx = rng.standard_normal((lq, G, 4)), rng.standard_normal((L, G, 4))
    scale = 0.3
    res = O.msa_forward(q, k, v, q_idx, k_idx, lq, L, B, 1, scale)
    s = np.arange(L)[None, :]
    mask = (s <= pos[:, None]) & (s >= (pos[:, None] // B) * B)
    ref = _sdpa(q, k, v, mask, scale)
    assert np.abs(res["out"] - ref).max() < 1e-12


def _random_selection(rng, G, pos, B, k):
    """Arbitrary valid kept-block lists (not the oracle's Top-k), to test attention alone."""
    n = len(pos)
    idx = np.full((G, n, k), -1, np.int32)
    for g in range(G):
        for t in range(n):
            J = int(pos[t] // B)
            others = rng.permutation(J)[:k - 1] if J > 0 else np.array([], int)
            kept = sorted(int(x) for x in others) + [J]
            idx[g, t, :len(kept)] = kept
    return idx


def _mask_from_selection(idx_row, p, L, B):
    """Independent key mask: key s attended iff its block is listed and s <= p."""
    blocks = set(int(j) for j in idx_row if j >= 0)
    return np.array([(s <= p) and (s // B in blocks) for s in range(L)])


def test_attention_matches_sdpa_on_arbitrary_selection():
    L, lq, B, H, G, d, k = 90, 30, 8, 6, 3, 16, 4
    q, kk, v, pos = _case(11, L, lq, H, G, d, B)
    idx = _random_selection(np.random.default_rng(12), G, pos, B, k)
    scale = 0.2
    out, lse = O.sparse_attention(q, kk, v, idx, pos, B, scale)
    hpg = H // G
    for g in range(G):
        mask = np.stack([_mask_from_selection(idx[g, t], pos[t], L, B) for t in range(lq)])
        ref = _sdpa(q[:, g * hpg:(g + 1) * hpg], kk[:, g:g + 1], v[:, g:g + 1], mask, scale)
        assert np.abs(out[:, g * hpg:(g + 1) * hpg] - ref).max() < 1e-12


def test_attention_constant_v():
    L, lq, B, H, G, d, k = 50, 50, 8, 4, 2, 8, 3
    q, kk, v, pos = _case(13, L, lq, H, G, d, B)
    c = np.linspace(-2, 3, d)
    v[:] = c
    idx = _random_selection(np.random.default_rng(14), G, pos, B, k)
    out, _ = O.sparse_attention(q, kk, v, idx, pos, B, 0.7)
    assert np.abs(out - c).max() < 1e-12


def test_attention_zero_q_is_mean_over_kept_keys():
    L, lq, B, H, G, d, k = 60, 60, 8, 2, 2, 4, 3
    _, kk, v, pos = _case(15, L, lq, H, G, d, B)
    q = np.zeros((lq, H, d))
    idx = _random_selection(np.random.default_rng(16), G, pos, B, k)
    out, lse = O.sparse_attention(q, kk, v, idx, pos, B, 1.0)
    for g in range(G):
        for t in range(lq):
            m = _mask_from_selection(idx[g, t], pos[t], L, B)
            assert np.allclose(out[t, g], v[m, g].mean(axis=0), atol=1e-13)
            assert abs(lse[t, g] - math.log(m.sum())) < 1e-13


def test_attention_weights_via_one_hot_v():
    """V = identity rows exposes the weights: they sum to 1, vanish off the kept keys,
    and equal scipy's softmax of the kept logits (one joint softmax, not per block)."""
    L, lq, B, H, G, d, k = 24, 24, 4, 1, 1, 5, 3
    rng = np.random.default_rng(17)
    q = rng.standard_normal((lq, H, d))
    kk = rng.standard_normal((L, G, d))
    v = np.eye(L)[:, None, :]                  # value of key s is e_s
    pos = O.query_positions(lq, L)
    idx = _random_selection(rng, G, pos, B, k)
    scale = 0.9
    out, lse = O.sparse_attention(q, kk, v, idx, pos, B, scale)
    for t in range(lq):
        m = _mask_from_selection(idx[0, t], pos[t], L, B)
        w = out[t, 0]
        assert abs(w.sum() - 1) < 1e-13
        assert np.all(w[~m] == 0) and np.all(w[m] > 0)
        z = scale * (kk[m, 0] @ q[t, 0])
        assert np.allclose(w[m], scipy.special.softmax(z), atol=1e-14)
        assert abs(lse[t, 0] - scipy.special.logsumexp(z)) < 1e-12


def test_lse_bruteforce_fsum():
    L, lq, B, H, G, d, k = 30, 10, 4, 2, 1, 3, 3
    q, kk, v, pos = _case(19, L, lq, H, G, d, B)
    idx = _random_selection(np.random.default_rng(20), G, pos, B, k)
    _, lse = O.sparse_attention(q, kk, v, idx, pos, B, 1.3)
    for t in range(lq):
        keys = [s for s in range(L) if _mask_from_selection(idx[0, t], pos[t], L, B)[s]]
        for h in range(H):
            z = [1.3 * math.fsum(q[t, h, c] * kk[s, 0, c] for c in range(d)) for s in keys]
            ref = math.log(math.fsum(math.exp(x) for x in z))
            assert abs(lse[t, h] - ref) < 1e-12


def test_attention_invariant_to_block_list_order():
    L, lq, B, H, G, d, k = 64, 16, 8, 2, 1, 8, 4
    q, kk, v, pos = _case(21, L, lq, H, G, d, B)
    idx = _random_selection(np.random.default_rng(22), G, pos, B, k)
    out1, _ = O.sparse_attention(q, kk, v, idx, pos, B, 0.5)
    out2, _ = O.sparse_attention(q, kk, v, idx[:, :, ::-1].copy(), pos, B, 0.5)
    assert np.abs(out1 - out2).max() < 1e-13


def test_head_to_group_map_is_contiguous():
    """Heads g*hpg .. g*hpg+hpg-1 use group g: giving group 1 constant values shows it."""
    L, lq, B, H, G, d = 32, 32, 8, 4, 2, 4
    q, kk, v, pos = _case(23, L, lq, H, G, d, B)
    v[:, 1, :] = 7.0
    idx = _random_selection(np.random.default_rng(24), G, pos, B, 2)
    out, _ = O.sparse_attention(q, kk, v, idx, pos, B, 1.0)
    assert np.abs(out[:, 2:4] - 7.0).max() < 1e-12
    assert np.abs(out[:, 0:2] - 7.0).min() > 1e-6


# -------------------------------------------------------------- workloads ---

def test_planted_queries_keep_planted_blocks():
    """On a planted workload, a planted query keeps every causal planted block
    whenever there are at most k-1 of them (their scores sit far above the rest)."""
    import workloads as W
    w = W.Workload("pin-planted", 4, 2, 8, 64, 128, 16, "f32", True,
                   len_q=(4096,), len_kv=(4096,))
    inp = W.make_inputs(w, with_attention=False)
    pos = O.query_positions(4096, 4096)
    rows = np.array(inp["planted_q"][0][0][-40:] + inp["planted_q"][0][1][-40:])
    S = O.block_scores(inp["q_idx"][rows], inp["k_idx"], pos[rows], 128)
    idx = O.select_blocks(S, pos[rows], 128, 16)
    checked = 0
    for g in range(2):
        pb = set(inp["planted_blocks"][0][g])
        for i, t in enumerate(rows):
            if t not in inp["planted_q"][0][g]:
                continue
            J = pos[t] // 128
            causal_planted = {j for j in pb if j < J}
            if 0 < len(causal_planted) <= 15:
                assert causal_planted <= set(idx[g, i].tolist())
                checked += 1
    assert checked > 20


# ------------------------------------------- indexer KL target and loss ---
# Reading of the page's training objective (Summary, paragraph 2): p is the
# Main Branch's attention mass per kept block averaged over the group's
# heads; q is the softmax of the raw block scores over the kept blocks; the
# loss is KL(p || q) with p held fixed.

GOLDEN_KL = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_kl.json")


def test_golden_block_mass_and_kl():
    gd = _golden()
    a = gd["attention_pow2"]
    with open(GOLDEN_KL) as f:
        gk = json.load(f)
    rows = gk["rows"]
    pos = O.query_positions(6, 6)[rows]
    idx = np.array(gk["block_idx"], np.int32)[None]
    q = np.full((len(rows), 1, 1), math.log(2.0))
    k = np.array(a["k"], float)[:, None, None]
    mass = O.block_mass(q, k, idx, pos, gd["block_size"], 1.0)
    assert np.allclose(mass[0], gk["mass"], rtol=0, atol=1e-15)
    k_idx = np.array(gd["k_idx"], float)[:, None, :]
    q_idx = np.array(gd["q_idx"], float)[rows][:, None, :]
    S = O.block_scores(q_idx, k_idx, pos, gd["block_size"])
    kl, grad = O.indexer_kl(S, idx, mass)
    assert np.allclose(kl[0], gk["kl"], rtol=0, atol=1e-14)
    assert np.allclose(grad[0], gk["grad"], rtol=0, atol=1e-14)


def _kl_case(seed, H=4, G=2, L=300, lq=40, B=32, k=3, d=16):
    rng = np.random.default_rng(seed)
    q, kk = _rand(rng, lq, H, d), _rand(rng, L, G, d)
    q_idx, k_idx = _rand(rng, lq, G, 8), _rand(rng, L, G, 8)
    pos = O.query_positions(lq, L)
    S = O.block_scores(q_idx, k_idx, pos, B)
    idx = O.select_blocks(S, pos, B, k)
    return q, kk, pos, S, idx


@pytest.mark.parametrize("seed", [1, 2])
def test_block_mass_is_one_hot_value_attention(seed):
    """With V[s] = one-hot of s's block, the attention output of head h is
    its mass on each block; the group average, read at each kept slot's
    block, is the block mass (sparse_attention is pinned separately)."""
    q, kk, pos, S, idx = _kl_case(seed)
    B, G, H = 32, 2, 4
    L = kk.shape[0]
    nb = O.num_blocks(L, B)
    v = np.zeros((L, G, nb))
    v[np.arange(L), :, np.arange(L) // B] = 1.0
    out, _ = O.sparse_attention(q, kk, v, idx, pos, B, 0.25)
    mass = O.block_mass(q, kk, idx, pos, B, 0.25)
    hpg = H // G
    for g in range(G):
        avg = out[:, g * hpg:(g + 1) * hpg, :].mean(axis=1)          # [n, nb]
        for t in range(len(pos)):
            for i, j in enumerate(idx[g, t]):
                want = 0.0 if j < 0 else avg[t, j]
                assert abs(mass[g, t, i] - want) < 1e-13


def test_block_mass_dense_bruteforce():
    """k covering every block: the mass is the dense causal softmax of the
    full score matrix (torch fp64), summed over each block's keys and
    averaged over the group's heads."""
    rng = np.random.default_rng(5)
    L, lq, B, H, G, d = 96, 96, 16, 4, 2, 8
    q, kk = _rand(rng, lq, H, d), _rand(rng, L, G, d)
    pos = O.query_positions(lq, L)
    nb = O.num_blocks(L, B)
    idx = np.full((G, lq, nb), -1, np.int32)
    for t, p in enumerate(pos):
        idx[:, t, :p // B + 1] = np.arange(p // B + 1)
    mass = O.block_mass(q, kk, idx, pos, B, 0.5)
    qt, kt = torch.from_numpy(q), torch.from_numpy(kk)
    for g in range(G):
        z = 0.5 * torch.einsum("thd,sd->ths", qt[:, 2 * g:2 * g + 2], kt[:, g])
        z = z.masked_fill(torch.arange(L)[None, None, :] > torch.from_numpy(pos)[:, None, None],
                          float("-inf"))
        a = torch.softmax(z, dim=-1).mean(dim=1)                      # [lq, L]
        per_block = a.reshape(lq, nb, B).sum(dim=-1).numpy()
        for t in range(lq):
            for i, j in enumerate(idx[g, t]):
                want = 0.0 if j < 0 else per_block[t, j]
                assert abs(mass[g, t, i] - want) < 1e-13


def test_block_mass_sums_to_one_and_pads_zero():
    q, kk, pos, S, idx = _kl_case(3, lq=60, L=200)
    mass = O.block_mass(q, kk, idx, pos, 32, 0.25)
    assert np.allclose(mass.sum(axis=2), 1.0, rtol=0, atol=1e-13)
    assert np.all(mass[idx < 0] == 0.0)
    assert np.all(mass >= 0.0)


def test_kl_matches_scipy_rel_entr():
    q, kk, pos, S, idx = _kl_case(4)
    mass = O.block_mass(q, kk, idx, pos, 32, 0.25)
    kl, _ = O.indexer_kl(S, idx, mass)
    G, n, _ = idx.shape
    for g in range(G):
        for t in range(n):
            sel = idx[g, t] >= 0
            qd = scipy.special.softmax(S[g, t, idx[g, t, sel]])
            want = scipy.special.rel_entr(mass[g, t, sel], qd).sum()
            assert abs(kl[g, t] - want) < 1e-12
    assert np.all(kl >= -1e-15)


def test_kl_zero_when_scores_are_log_mass():
    q, kk, pos, S, idx = _kl_case(6)
    mass = O.block_mass(q, kk, idx, pos, 32, 0.25)
    S2 = np.full_like(S, -np.inf)
    G, n, K = idx.shape
    for g in range(G):
        for t in range(n):
            for i in range(K):
                if idx[g, t, i] >= 0:
                    S2[g, t, idx[g, t, i]] = math.log(mass[g, t, i]) + 3.0 * g - 0.01 * t
    kl, grad = O.indexer_kl(S2, idx, mass)
    assert np.abs(kl).max() < 1e-12
    assert np.abs(grad).max() < 1e-12


def test_kl_gradient_is_finite_difference_of_kl():
    """Central differences of the loss in each kept block's score."""
    q, kk, pos, S, idx = _kl_case(7, lq=12)
    mass = O.block_mass(q, kk, idx, pos, 32, 0.25)
    _, grad = O.indexer_kl(S, idx, mass)
    eps = 1e-6
    G, n, K = idx.shape
    for g in range(G):
        for t in range(n):
            for i in range(K):
                j = idx[g, t, i]
                if j < 0:
                    assert grad[g, t, i] == 0.0
                    continue
                Sp, Sm = S.copy(), S.copy()
                Sp[g, t, j] += eps
                Sm[g, t, j] -= eps
                fd = (O.indexer_kl(Sp, idx, mass)[0][g, t] - O.indexer_kl(Sm, idx, mass)[0][g, t]) / (2 * eps)
                assert abs(fd - grad[g, t, i]) < 1e-8


# --------------------------------------- Index Branch max-pooling backward ---

GOLDEN_IBWD = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_index_bwd.json")


def test_golden_index_backward():
    gd = _golden()
    with open(GOLDEN_IBWD) as f:
        gb = json.load(f)
    rows = gb["rows"]
    k_idx = np.array(gd["k_idx"], float)[:, None, :]
    q_idx = np.array(gd["q_idx"], float)[rows][:, None, :]
    pos = O.query_positions(6, 6)[rows]
    idx = np.array(gb["block_idx"], np.int32)[None]
    for r, row in enumerate(gb["argmax"]):
        for i, a in enumerate(row):
            s0 = idx[0, r, i] * gd["block_size"]
            s1 = min(s0 + gd["block_size"], pos[r] + 1)
            assert s0 + O.block_argmax(q_idx[r, 0], k_idx[s0:s1, 0]) == a
    dq, dk = O.index_backward(q_idx, k_idx, idx, pos, gd["block_size"],
                              np.array(gb["grad"], float)[None])
    assert np.array_equal(dq[:, 0], np.array(gb["dq"], float))
    assert np.array_equal(dk[:, 0], np.array(gb["dk"], float))


def _ibwd_case(seed, L=200, lq=30, G=2, di=8, B=16, k=4):
    rng = np.random.default_rng(seed)
    q_idx, k_idx = _rand(rng, lq, G, di), _rand(rng, L, G, di)
    pos = O.query_positions(lq, L)
    S = O.block_scores(q_idx, k_idx, pos, B)
    idx = O.select_blocks(S, pos, B, k)
    grad = _rand(rng, G, lq, k)
    grad[idx < 0] = 0.0
    return q_idx, k_idx, pos, idx, grad


def test_index_backward_matches_torch_autograd():
    """The same loss, sum of grad * S over the kept slots, written with torch
    (fp64 masked dot products, max over each block's keys) and
    differentiated by autograd."""
    B = 16
    q_idx, k_idx, pos, idx, grad = _ibwd_case(11)
    dq, dk = O.index_backward(q_idx, k_idx, idx, pos, B, grad)
    qt = torch.tensor(q_idx, requires_grad=True)
    kt = torch.tensor(k_idx, requires_grad=True)
    L, G = k_idx.shape[0], k_idx.shape[1]
    loss = torch.zeros((), dtype=torch.float64)
    for g in range(G):
        dots = qt[:, g, :] @ kt[:, g, :].T                                   # [n, L]
        dots = dots.masked_fill(torch.arange(L)[None, :] > torch.from_numpy(pos)[:, None],
                                float("-inf"))
        for t in range(len(pos)):
            for i in range(idx.shape[2]):
                j = idx[g, t, i]
                if j >= 0:
                    loss = loss + grad[g, t, i] * dots[t, j * B:(j + 1) * B].max()
    loss.backward()
    assert np.allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-12)


def test_index_backward_is_finite_difference_of_scores():
    """Central differences of sum(grad * S) through block_scores, for a few
    coordinates of q_idx and k_idx (the max is locally linear)."""
    B = 16
    q_idx, k_idx, pos, idx, grad = _ibwd_case(12, L=96, lq=20)
    dq, dk = O.index_backward(q_idx, k_idx, idx, pos, B, grad)

    def loss(qi, ki):
        S = O.block_scores(qi, ki, pos, B)
        tot = 0.0
        G, n, K = idx.shape
        for g in range(G):
            for t in range(n):
                for i in range(K):
                    if idx[g, t, i] >= 0:
                        tot += grad[g, t, i] * S[g, t, idx[g, t, i]]
        return tot

    eps = 1e-6
    rng = np.random.default_rng(3)
    for _ in range(12):
        t, g, c = rng.integers(20), rng.integers(2), rng.integers(8)
        qp, qm = q_idx.copy(), q_idx.copy()
        qp[t, g, c] += eps
        qm[t, g, c] -= eps
        assert abs((loss(qp, k_idx) - loss(qm, k_idx)) / (2 * eps) - dq[t, g, c]) < 1e-7
        s = rng.integers(96)
        kp, km = k_idx.copy(), k_idx.copy()
        kp[s, g, c] += eps
        km[s, g, c] -= eps
        assert abs((loss(q_idx, kp) - loss(q_idx, km)) / (2 * eps) - dk[s, g, c]) < 1e-7


def test_block_argmax_is_first_maximum_of_exact_dots():
    """The arg-max key is the first maximum of the exactly summed dot
    products (math.fsum of products that are exact in fp64: bf16-valued
    inputs), with exact ties planted by repeating rows."""
    rng = np.random.default_rng(4)
    for it in range(200):
        q = torch.tensor(rng.standard_normal(8)).to(torch.bfloat16).double().numpy()
        kr = torch.tensor(rng.standard_normal((16, 8))).to(torch.bfloat16).double().numpy()
        if it % 2:
            kr[rng.integers(16)] = kr[rng.integers(16)]      # an exact tie, in either order
        exact = [math.fsum(float(a) * float(b) for a, b in zip(q, row)) for row in kr]
        best = max(exact)
        assert O.block_argmax(q, kr) == exact.index(best)


def test_block_argmax_is_not_fp32_channel_order():
    """A block where fp32 summation in channel order picks the wrong key:
    key 0 = (2^24, 1, -2^24) dots q = (1, 1, 1) to exactly 1, but fp32 adds
    2^24 + 1 -> 2^24 and then returns 0; key 1 = (0.5, 0, 0) dots to 0.5.
    The arg-max of the definition is key 0."""
    q = np.array([1.0, 1.0, 1.0])
    kr = np.array([[2.0 ** 24, 1.0, -2.0 ** 24], [0.5, 0.0, 0.0]])
    assert O.block_argmax(q, kr) == 0


# ------------------------------------------------ Main Branch backward ---

def test_attention_backward_matches_torch_autograd():
    """Autograd of the same attention written with torch (fp64): one masked
    softmax per (row, head) over the kept causal keys, on kept lists from a
    real selection."""
    rng = np.random.default_rng(21)
    L, lq, H, G, d, B, k = 150, 40, 4, 2, 8, 16, 3
    q, kk, vv = _rand(rng, lq, H, d), _rand(rng, L, G, d), _rand(rng, L, G, d)
    q_idx, k_idx = _rand(rng, lq, G, 4), _rand(rng, L, G, 4)
    pos = O.query_positions(lq, L)
    idx = O.select_blocks(O.block_scores(q_idx, k_idx, pos, B), pos, B, k)
    dout = _rand(rng, lq, H, d)
    dq, dk, dv = O.sparse_attention_backward(q, kk, vv, idx, pos, B, 0.3, dout)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kk, requires_grad=True)
    vt = torch.tensor(vv, requires_grad=True)
    hpg = H // G
    loss = torch.zeros((), dtype=torch.float64)
    for t in range(lq):
        for g in range(G):
            mask = torch.zeros(L, dtype=torch.bool)
            for j in idx[g, t]:
                if j >= 0:
                    mask[j * B:min((j + 1) * B, pos[t] + 1)] = True
            for h in range(g * hpg, (g + 1) * hpg):
                z = 0.3 * (kt[:, g, :] @ qt[t, h])
                a = torch.softmax(z.masked_fill(~mask, float("-inf")), dim=0)
                loss = loss + (torch.tensor(dout[t, h]) * (a @ vt[:, g, :])).sum()
    loss.backward()
    assert np.allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-12)


def test_attention_backward_dense_is_sdpa_backward():
    """k covering every block: the gradients of torch's causal SDPA (fp64),
    with the GQA head map expanded."""
    rng = np.random.default_rng(22)
    L, H, G, d, B = 64, 4, 2, 8, 16
    q, kk, vv = _rand(rng, L, H, d), _rand(rng, L, G, d), _rand(rng, L, G, d)
    pos = O.query_positions(L, L)
    nb = O.num_blocks(L, B)
    idx = np.full((G, L, nb), -1, np.int32)
    for t, p in enumerate(pos):
        idx[:, t, :p // B + 1] = np.arange(p // B + 1)
    dout = _rand(rng, L, H, d)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = O.sparse_attention_backward(q, kk, vv, idx, pos, B, scale, dout)
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(kk, requires_grad=True)
    vt = torch.tensor(vv, requires_grad=True)
    hpg = H // G
    ke = kt.repeat_interleave(hpg, dim=1).transpose(0, 1)   # [H, L, d]
    ve = vt.repeat_interleave(hpg, dim=1).transpose(0, 1)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt.transpose(0, 1)[None], ke[None], ve[None], is_causal=True, scale=scale)[0]
    (out.transpose(0, 1) * torch.tensor(dout)).sum().backward()
    assert np.allclose(dq, qt.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dk, kt.grad.numpy(), rtol=0, atol=1e-12)
    assert np.allclose(dv, vt.grad.numpy(), rtol=0, atol=1e-12)


def test_attention_backward_finite_differences():
    """Central differences of sum(dout * out) in a few coordinates of q, k, v."""
    rng = np.random.default_rng(23)
    L, lq, H, G, d, B, k = 80, 10, 2, 1, 4, 16, 2
    q, kk, vv = _rand(rng, lq, H, d), _rand(rng, L, G, d), _rand(rng, L, G, d)
    pos = O.query_positions(lq, L)
    idx = O.select_blocks(O.block_scores(_rand(rng, lq, G, 4), _rand(rng, L, G, 4), pos, B),
                          pos, B, k)
    dout = _rand(rng, lq, H, d)
    dq, dk, dv = O.sparse_attention_backward(q, kk, vv, idx, pos, B, 0.5, dout)

    def loss(qq, k2, v2):
        out, _ = O.sparse_attention(qq, k2, v2, idx, pos, B, 0.5)
        return float((out * dout).sum())

    eps = 1e-6
    for (arr, grad, which) in ((q, dq, 0), (kk, dk, 1), (vv, dv, 2)):
        for flat in rng.choice(arr.size, 6, replace=False):
            ix = np.unravel_index(flat, arr.shape)
            ap, am = arr.copy(), arr.copy()
            ap[ix] += eps
            am[ix] -= eps
            args_p = [q, kk, vv]
            args_m = [q, kk, vv]
            args_p[which], args_m[which] = ap, am
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[ix]) < 1e-7


# ------------------------------------------------ hierarchical indexing ---

GOLDEN_HIER = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_hier.json")


def test_golden_hierarchical_selection():
    """A hand-worked coarse-to-fine example: mean-pooled chunk keys (a chunk
    whose max-pooled score would win loses on its mean), a coarse tie going
    to the lower chunk, and the fine pick among the kept chunk's blocks."""
    with open(GOLDEN_HIER) as f:
        gd = json.load(f)
    k_idx = np.array(gd["k_idx"], float)[:, None, :]
    q_idx = np.array(gd["q_idx"], float)[:, None, :]
    pos = np.array([gd["position"]])
    r = O.hierarchical_select(q_idx, k_idx, pos, gd["block_size"], gd["top_k"],
                              gd["chunk_blocks"], gd["keep_chunks"])
    assert np.array_equal(r["coarse"][0, 0], np.array(gd["coarse"], float))
    assert r["kept_chunks"][0, 0].tolist() == gd["kept_chunks"]
    assert r["block_idx"][0, 0].tolist() == gd["block_idx"]
    ex = O.select_blocks(O.block_scores(q_idx, k_idx, pos, gd["block_size"]), pos,
                         gd["block_size"], gd["top_k"])
    assert ex[0, 0].tolist() == gd["exact_block_idx"]
    assert O.selection_recall(r["block_idx"], ex, pos, gd["block_size"], gd["top_k"]) == 0.5


def _hier_by_loops(q_idx, k_idx, pos, B, k, S, C):
    """Brute force of the hierarchical reading with Python loops, math.fsum and
    sorted() (no numpy reductions or lexsort)."""
    n, G, di = q_idx.shape
    L = k_idx.shape[0]
    span = B * S
    out = np.full((G, n, k), -1, np.int32)
    for g in range(G):
        kbar = []
        for c in range(L // span):
            kbar.append([math.fsum(k_idx[c * span + s, g, x] for s in range(span)) / span
                         for x in range(di)])
        for t in range(n):
            p = int(pos[t])
            J = p // B
            if J <= k - 1:
                sel = list(range(J + 1))
            else:
                cJ = J // S
                cs = [(-math.fsum(q_idx[t, g, x] * kbar[c][x] for x in range(di)), c)
                      for c in range(cJ)]
                keep = [c for _, c in sorted(cs)[:C]]
                blocks = [c * S + s for c in keep for s in range(S)] + list(range(cJ * S, J))
                fs = []
                for j in blocks:
                    best = max(math.fsum(q_idx[t, g, x] * k_idx[s, g, x] for x in range(di))
                               for s in range(j * B, min(j * B + B, p + 1)))
                    fs.append((-best, j))
                sel = sorted(j for _, j in sorted(fs)[:k - 1]) + [J]
            out[g, t, :len(sel)] = sel
    return out


@pytest.mark.parametrize("L,lq,B,S,C,k", [(96, 40, 4, 2, 3, 4), (130, 130, 2, 2, 2, 5),
                                          (200, 17, 8, 2, 1, 3), (64, 64, 1, 4, 2, 6)])
def test_hierarchical_matches_loop_bruteforce(L, lq, B, S, C, k):
    """Small integers and chunk spans B*S that are powers of two keep every
    mean and dot product exact on both sides, so exact ties are decided by
    the same rule (lower chunk, lower block) rather than by rounding."""
    rng = np.random.default_rng(L + 7 * S + C)
    G, di = 2, 3
    q = rng.integers(-2, 3, (lq, G, di)).astype(float)   # small integers: many exact ties
    kk = rng.integers(-2, 3, (L, G, di)).astype(float)
    pos = O.query_positions(lq, L)
    r = O.hierarchical_select(q, kk, pos, B, k, S, C)
    assert np.array_equal(r["block_idx"], _hier_by_loops(q, kk, pos, B, k, S, C))


def test_chunk_keys_and_coarse_scores_by_loops():
    """The coarse key of a full chunk is the MEAN of its B*S index keys (a sum
    would rank the same, so the values are pinned, not only the selection);
    the trailing partial chunk has none; a row's coarse scores are its dot
    products with the coarse keys of the chunks below its current chunk and
    -inf elsewhere."""
    rng = np.random.default_rng(12)
    L, lq, G, di, B, S, C, k = 150, 60, 2, 3, 4, 4, 2, 4
    q, kk = _rand(rng, lq, G, di), _rand(rng, L, G, di)
    span = B * S
    kbar = O.chunk_keys(kk, B, S)
    assert kbar.shape == (L // span, G, di)  # 9 full chunks; keys 144..149 form none
    for c in range(L // span):
        for g in range(G):
            for x in range(di):
                want = math.fsum(float(kk[c * span + s, g, x]) for s in range(span)) / span
                assert abs(kbar[c, g, x] - want) <= 1e-15 * max(1.0, abs(want))
    pos = O.query_positions(lq, L)
    r = O.hierarchical_select(q, kk, pos, B, k, S, C)
    for g in range(G):
        for t in range(lq):
            cJ = (int(pos[t]) // B) // S
            for c in range(L // span):
                got = r["coarse"][g, t, c]
                if c < cJ:
                    want = math.fsum(float(q[t, g, x]) * kbar[c, g, x] for x in range(di))
                    assert abs(got - want) <= 1e-12 * max(1.0, abs(want))
                else:
                    assert got == -np.inf


def test_hierarchical_keeping_every_chunk_is_exact():
    """C at least the number of chunks: every candidate block is scored, so
    the hierarchical selection is select_blocks' exactly, and recall is 1."""
    rng = np.random.default_rng(9)
    L, lq, G, di, B, S, k = 700, 300, 2, 4, 8, 4, 7
    q, kk = _rand(rng, lq, G, di), _rand(rng, L, G, di)
    pos = O.query_positions(lq, L)
    ex = O.select_blocks(O.block_scores(q, kk, pos, B), pos, B, k)
    r = O.hierarchical_select(q, kk, pos, B, k, S, L // (B * S))
    assert np.array_equal(r["block_idx"], ex)
    assert O.selection_recall(r["block_idx"], ex, pos, B, k) == 1.0


def test_hierarchical_structure():
    """Every row keeps J last, only blocks below J besides it, blocks of kept
    chunks or of the current chunk, and k - 1 free picks once J > k - 1; the
    coarse candidates are exactly the chunks below the current chunk."""
    rng = np.random.default_rng(10)
    L, lq, G, di, B, S, C, k = 900, 400, 2, 4, 4, 5, 3, 6
    q, kk = _rand(rng, lq, G, di), _rand(rng, L, G, di)
    pos = O.query_positions(lq, L)
    r = O.hierarchical_select(q, kk, pos, B, k, S, C)
    for g in range(G):
        for t in range(lq):
            J = pos[t] // B
            cJ = J // S
            assert np.all(np.isfinite(r["coarse"][g, t, :cJ]))
            assert np.all(np.isneginf(r["coarse"][g, t, cJ:]))
            row = [int(x) for x in r["block_idx"][g, t] if x >= 0]
            assert row[-1] == J and row == sorted(row)
            assert len(row) == min(J + 1, k)
            kept = set(int(c) for c in r["kept_chunks"][g, t] if c >= 0)
            assert len(kept) == min(cJ, C)
            for j in row[:-1]:
                assert j < J and (j // S in kept or j // S == cJ)
