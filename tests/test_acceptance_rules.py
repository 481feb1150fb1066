"""The GPU acceptance rules of tests/msa_check.py, checked on the CPU.

The parity tests are only as strict as these rules, so each rule is shown to
accept what it should (errors inside the bound, alternatives inside the tie
band) and to reject what it should (errors past the bound, a dropped winner,
a missing current block, bad padding or order, mismatched -inf positions).
No GPU and no library call is involved.
"""
import math

import numpy as np
import pytest

import msa_check as C
from oracle import msa_oracle as O


def _scores(rng, G, n, nb):
    return rng.standard_normal((G, n, nb))


# ------------------------------------------------------------- scores ---

def test_score_bound_is_max_of_abs_products():
    rng = np.random.default_rng(0)
    L, n, G, di, B = 23, 5, 2, 3, 4
    q, k = rng.standard_normal((n, G, di)), rng.standard_normal((L, G, di))
    pos = O.query_positions(n, L)
    b = C.score_bound(q, k, pos, B)
    for g in range(G):
        for t in range(n):
            for j in range(O.num_blocks(L, B)):
                keys = [s for s in range(j * B, min(j * B + B, L)) if s <= pos[t]]
                if not keys:
                    assert b[g, t, j] == -np.inf
                    continue
                want = max(math.fsum(abs(q[t, g, c] * k[s, g, c]) for c in range(di)) for s in keys)
                assert abs(b[g, t, j] - want) <= 1e-12 * want
    cheap = C.score_bound(q, k, pos, B, cheap=True)
    fin = np.isfinite(b)
    assert np.all(cheap[fin] >= b[fin] * (1 - 1e-12))  # Cauchy-Schwarz never tighter


def test_check_scores_accepts_inside_and_rejects_outside_the_bound():
    rng = np.random.default_rng(1)
    G, n, nb, di = 2, 6, 5, 64
    ref = _scores(rng, G, n, nb)
    ref[0, 0, 3:] = -np.inf
    bound = np.abs(rng.standard_normal((G, n, nb))) + 1.0
    allowed = 2 * C.gamma(di) * bound
    sign = np.where(rng.random((G, n, nb)) < 0.5, -1.0, 1.0)
    gpu = np.where(np.isneginf(ref), ref, ref + 0.9 * allowed * sign)
    assert C.check_scores(gpu, ref, bound, di) <= 0.9 + 1e-9
    bad = gpu.copy()
    bad[1, 2, 1] = ref[1, 2, 1] + 1.1 * allowed[1, 2, 1]
    with pytest.raises(AssertionError):
        C.check_scores(bad, ref, bound, di)
    bad = gpu.copy()
    bad[0, 0, 3] = 0.0  # a finite score where the oracle has none
    with pytest.raises(AssertionError):
        C.check_scores(bad, ref, bound, di)
    bad = gpu.copy()
    bad[1, 0, 0] = np.nan
    with pytest.raises(AssertionError):
        C.check_scores(bad, ref, bound, di)


# ---------------------------------------------------------- selection ---

def _sel_case(seed=2, G=2, n=8, L=80, B=8, k=4):
    rng = np.random.default_rng(seed)
    pos = O.query_positions(n, L)
    S = _scores(rng, G, n, O.num_blocks(L, B))
    return S, pos, B, k


def test_check_selection_accepts_the_oracle_selection():
    S, pos, B, k = _sel_case()
    ref = O.select_blocks(S, pos, B, k)
    assert C.check_selection(ref.copy(), ref, S, pos, B, k) == 0


def test_check_selection_rejects_a_dropped_winner():
    S, pos, B, k = _sel_case()
    ref = O.select_blocks(S, pos, B, k)
    g, t = 1, 5
    J = int(pos[t] // B)
    kept = [int(x) for x in ref[g, t] if 0 <= x < J]
    worst_dropped = min((j for j in range(J) if j not in kept), key=lambda j: S[g, t, j])
    row = sorted(kept[1:] + [worst_dropped]) + [J]
    bad = ref.copy()
    bad[g, t] = row
    with pytest.raises(AssertionError):
        C.check_selection(bad, ref, S, pos, B, k)


@pytest.mark.parametrize("mistake", ["no current block", "unsorted", "bad padding",
                                     "duplicate", "short row"])
def test_check_selection_rejects_malformed_rows(mistake):
    S, pos, B, k = _sel_case()
    ref = O.select_blocks(S, pos, B, k)
    bad = ref.copy()
    g, t = 0, 6
    J = int(pos[t] // B)
    row = [int(x) for x in bad[g, t]]
    if mistake == "no current block":
        others = [j for j in range(J) if j not in row]
        row = sorted(row[:-1] + [others[0]])
    elif mistake == "unsorted":
        row = row[::-1]
    elif mistake == "bad padding":
        row = row[:-1] + [-1]
    elif mistake == "duplicate":
        row = [row[0]] + row[:-1]
        row = sorted(row)
    else:  # a row with J <= k - 1 that drops one of 0..J
        t = 0
        S2 = S.copy()
        pos2 = pos.copy()
        pos2[t] = 2 * B + 1            # J = 2 <= k - 1: must keep 0, 1, 2
        ref = O.select_blocks(S2, pos2, B, k)
        bad = ref.copy()
        bad[g, t] = [0, 2, -1, -1]
        with pytest.raises(AssertionError):
            C.check_selection(bad, ref, S2, pos2, B, k)
        return
    bad[g, t] = row
    with pytest.raises(AssertionError):
        C.check_selection(bad, ref, S, pos, B, k)


def test_check_selection_allows_either_pick_inside_the_tie_band():
    S, pos, B, k = _sel_case(seed=3)
    g, t = 0, 7
    J = int(pos[t] // B)
    cand = S[g, t, :J]
    order = np.argsort(-cand, kind="stable")
    a, b = int(order[k - 2]), int(order[k - 1])          # last kept, first dropped
    S[g, t, b] = S[g, t, a] * (1 - 1e-4 * np.sign(S[g, t, a]))  # within 1e-3 relative
    ref = O.select_blocks(S, pos, B, k)
    alt = ref.copy()
    row = [int(x) for x in ref[g, t]]
    free = [x for x in row if x != J]
    if a in free:
        free[free.index(a)] = b
    else:
        free[free.index(b)] = a
    alt[g, t] = sorted(free) + [J]
    assert not np.array_equal(alt, ref)
    assert C.check_selection(alt, ref, S, pos, B, k) >= 1


# ---------------------------------------------------------- attention ---

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_check_attention_bounds(dtype):
    rng = np.random.default_rng(4)
    tol = C.TOL_OUT[dtype]
    ref = rng.standard_normal((5, 4, 8))
    lse = rng.standard_normal((5, 4))
    lse[2, 1] = -np.inf                                   # a row without keys
    assert C.check_attention(ref + 0.9 * tol, lse + 0.9 * tol, ref, lse, dtype) <= tol
    bad = ref.copy()
    bad[1, 2, 3] += 1.1 * tol
    with pytest.raises(AssertionError):
        C.check_attention(bad, lse, ref, lse, dtype)
    bad_lse = lse.copy()
    bad_lse[0, 0] += 1.1 * tol
    with pytest.raises(AssertionError):
        C.check_attention(ref, bad_lse, ref, lse, dtype)
    bad_lse = lse.copy()
    bad_lse[2, 1] = 0.0                                    # finite where the oracle has none
    with pytest.raises(AssertionError):
        C.check_attention(ref, bad_lse, ref, lse, dtype)


# --------------------------------------------------------- arg-max band ---

def test_argmax_tie_band_flags_near_ties_only():
    """Block 0 holds an exact tie (flagged, both keys listed); block 1 a
    clear winner (not flagged); a one-key block is never flagged."""
    di, B, G = 4, 4, 1
    q = np.array([[[1.0, 0.5, -0.25, 2.0]]])               # one row, one group
    k = np.zeros((9, G, di))
    k[0, 0] = [1.0, 0.0, 0.0, 1.0]                          # dot 3.0
    k[2, 0] = [1.0, 2.0, 0.0, 0.5]                          # dot 3.0: exact tie with key 0
    k[1, 0] = k[3, 0] = [0.0, 0.0, 1.0, 0.0]                # dot -0.25
    k[4, 0] = [4.0, 0.0, 0.0, 0.0]                          # dot 4.0: clear winner of block 1
    k[5, 0] = k[6, 0] = k[7, 0] = [1.0, 0.0, 0.0, 0.0]      # dot 1.0
    k[8, 0] = [1.0, 1.0, 1.0, 1.0]                          # block 2: one key
    pos = np.array([8])
    bi = np.array([[[0, 1, 2]]], dtype=np.int32)
    amb, keys = C.argmax_tie_band(q, k, bi, pos, B, di)
    assert amb[0, 0].tolist() == [True, False, False]
    assert keys[0] == {0, 2}
