"""Plain fp64 CPU oracle for MSA block-sparse attention.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only
the tests, the smoke check and the CPU-baseline leg of the benchmark import
it.  The HIP library never calls it and shares no code with it.

What it computes follows the "MiniMax Sparse Attention" page (paper by Lai
et al., 2026), section Summary, second paragraph, and section Key points,
bullet "Benchmark configuration":

  * Index Branch: each key/value block is scored by max-pooling token-level
    dot products of an index query with the block's index keys;
  * each GQA group picks its own Top-k blocks, and the block that holds the
    query's own position is always kept (k counts that block: B_k = 128 and
    k = 16 give 2,048 attended tokens per query);
  * Main Branch: exact softmax attention restricted to the kept blocks, for
    every query head of the group.

Readings where the page is silent (each also listed in the design notes):
  * queries are the LAST len_q tokens of their sequence, so query i sits at
    position p = len_kv - len_q + i and sees keys 0..p (causal);
  * the score is the raw dot product (no scale), pooled over causal keys
    only; a block with no causal key scores -inf;
  * selection is per (query token, group); ties go to the lower block
    index; the output lists the kept blocks in ascending order, padded with
    -1 when fewer than k blocks are causal;
  * one softmax over the union of the kept keys (not one per block), scaled
    by `scale`; LSE is the natural log-sum-exp of the scaled logits;
  * query head h belongs to group h // (H / G);
  * the indexer's training target (Summary, paragraph 2: a KL objective that
    matches the group-averaged Main Branch distribution, with the Main Branch
    detached) is read as: p = the Main Branch's attention mass on each kept
    block, averaged over the group's heads; q = the softmax of the raw block
    scores over the same kept blocks; loss KL(p || q) per (group, row); the
    gradient flows into the scores only.

Everything runs in float64 on exact upcasts of the inputs.  Loops are over
rows; the inner steps are numpy matrix products and reductions.

Every function here is pinned to something other than itself by
tests/test_oracle_pins.py (hand-worked fixtures, brute force, closed forms,
library routines on special cases); none is parity-unpinned.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    """Exact upcast of an fp32/bf16/fp64 array (numpy or torch) to float64."""
    if hasattr(x, "detach"):  # torch tensor: upcast exactly before leaving torch
        import torch
        x = x.detach().to("cpu", torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _gather_f64(x, keys: np.ndarray, g: int) -> np.ndarray:
    """Rows `keys` of group g of a [L, G, d] array (numpy or CPU torch), as float64."""
    if hasattr(x, "detach"):
        import torch
        return _f64(x[torch.from_numpy(keys), g, :])
    return _f64(x[keys, g, :])


def query_positions(len_q: int, len_kv: int) -> np.ndarray:
    """Absolute positions of a sequence's queries: the last len_q tokens."""
    if len_q > len_kv:
        raise ValueError("a sequence cannot have more queries than keys")
    return np.arange(len_kv - len_q, len_kv, dtype=np.int64)


def num_blocks(len_kv: int, block_size: int) -> int:
    return -(-len_kv // block_size)


def block_scores(q_idx, k_idx, pos, block_size: int, num_block_cols: int | None = None,
                 row_chunk: int = 256, workers: int = 1) -> np.ndarray:
    """Index Branch block scores of one sequence (Summary, paragraph 2).

    q_idx: [n, G, d_idx] index queries of the rows to score;
    k_idx: [len_kv, G, d_idx] index keys of the whole sequence;
    pos:   [n] absolute positions of those rows.
    Returns S [G, n, NB] with S[g,t,j] = max over keys s of block j with
    s <= pos[t] of <q_idx[t,g], k_idx[s,g]>, and -inf where block j holds no
    such key.  NB defaults to ceil(len_kv / B); a larger num_block_cols pads
    with -inf columns.  Row chunks of each group run on `workers` threads
    (numpy releases the interpreter lock inside the array operations).
    """
    q = _f64(q_idx)
    pos = np.asarray(pos, dtype=np.int64)
    n, G, _ = q.shape
    L = k_idx.shape[0]
    nb = num_blocks(L, block_size)
    ncol = nb if num_block_cols is None else num_block_cols
    S = np.full((G, n, ncol), NEG_INF)
    key_pos = np.arange(nb * block_size)
    row_chunk = max(1, min(row_chunk, (1 << 24) // max(L, 1)))
    for g in range(G):
        kg = _f64(k_idx[:, g, :])

        def one_chunk(r0):
            r1 = min(n, r0 + row_chunk)
            dots = np.full((r1 - r0, nb * block_size), NEG_INF)
            dots[:, :L] = q[r0:r1, g, :] @ kg.T           # token-level dot products
            dots[key_pos[None, :] > pos[r0:r1, None]] = NEG_INF   # causal keys only
            S[g, r0:r1, :nb] = dots.reshape(r1 - r0, nb, block_size).max(axis=2)

        chunks = range(0, n, row_chunk)
        if workers <= 1:
            for r0 in chunks:
                one_chunk(r0)
        else:
            from concurrent.futures import ThreadPoolExecutor
            with ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(one_chunk, chunks))
    return S


def select_blocks(S, pos, block_size: int, top_k: int) -> np.ndarray:
    """Per-group Top-k with the current block always kept (Summary, paragraph 2).

    S: [G, n, NB] block scores; pos: [n].
    For row t the current block is J = pos[t] // B.  The candidates are the
    blocks 0..J-1.  If there are at most k-1 of them all are kept; otherwise
    the k-1 best are kept, ordered by score (higher first) and then by block
    index (lower first).  J is added.  Returns int32 [G, n, k], ascending,
    padded with -1.
    """
    S = np.asarray(S, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    G, n, _ = S.shape
    out = np.full((G, n, top_k), -1, dtype=np.int32)
    for g in range(G):
        for t in range(n):
            J = int(pos[t] // block_size)
            if J <= top_k - 1:
                kept = list(range(J + 1))
            else:
                cand = np.arange(J)
                # lexsort: last key is primary -> score descending, then index ascending
                order = np.lexsort((cand, -S[g, t, :J]))
                kept = sorted(int(j) for j in cand[order[:top_k - 1]]) + [J]
            out[g, t, :len(kept)] = kept
    return out


def select_blocks_vectorised(S, pos, block_size: int, top_k: int,
                             row_chunk: int = 1024, workers: int = 1) -> np.ndarray:
    """The rule of select_blocks for many rows at once (same result on every
    input; pinned against it), for checking whole score tensors.

    Per row with current block J and m = k-1 free picks: if J <= m, keep
    0..J.  Otherwise let tau be the m-th largest of the candidates 0..J-1;
    keep every candidate above tau and, of those equal to tau, the lowest
    indices until m are kept (this is "score descending, then index
    ascending"); add J.  S may be fp32: comparisons are exact in any
    precision.  Row chunks run on `workers` threads (numpy releases the
    interpreter lock inside these array operations).  Returns int32
    [G, n, k], ascending, padded with -1."""
    S = np.asarray(S)
    pos = np.asarray(pos, dtype=np.int64)
    G, n, nb = S.shape
    m = top_k - 1
    out = np.full((G, n, top_k), -1, dtype=np.int32)
    cols = np.arange(nb)

    def one_chunk(g, r0):
        r1 = min(n, r0 + row_chunk)
        J = pos[r0:r1] // block_size
        keep = cols[None, :] <= J[:, None]            # rows with J <= m keep 0..J
        big = J > m
        if m > 0 and big.any():
            x = S[g, r0:r1][big]
            cand = cols[None, :] < J[big][:, None]
            x = np.where(cand, x, -np.inf)
            tau = -np.partition(-x, m - 1, axis=1)[:, m - 1:m]   # m-th largest
            gt = x > tau
            eq = (x == tau) & cand
            need = m - gt.sum(axis=1, keepdims=True)
            kb = gt | (eq & (np.cumsum(eq, axis=1) <= need))
            kb |= cols[None, :] == J[big][:, None]
            keep[big] = kb
        elif big.any():                                  # k = 1: only the current block
            keep[big] = cols[None, :] == J[big][:, None]
        cnt = keep.sum(axis=1)
        first = np.argsort(~keep, axis=1, kind="stable")[:, :top_k].astype(np.int32)
        first[np.arange(top_k)[None, :] >= cnt[:, None]] = -1
        out[g, r0:r1] = first

    jobs = [(g, r0) for g in range(G) for r0 in range(0, n, row_chunk)]
    if workers <= 1:
        for g, r0 in jobs:
            one_chunk(g, r0)
    else:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(lambda a: one_chunk(*a), jobs))
    return out


def kept_keys(block_row, p: int, block_size: int) -> np.ndarray:
    """Key positions attended by a query at position p given its kept blocks."""
    keys = []
    for j in np.asarray(block_row):
        if j < 0:
            continue
        s0 = int(j) * block_size
        s1 = min(s0 + block_size, p + 1)
        keys.extend(range(s0, s1))
    return np.array(sorted(keys), dtype=np.int64)


def sparse_attention(q, k, v, block_idx, pos, block_size: int, scale: float):
    """Main Branch: exact softmax attention over the kept blocks (Summary, paragraph 2).

    q: [n, H, d]; k, v: [len_kv, G, d]; block_idx: [G, n, k]; pos: [n].
    For row t and head h of group g, the key set is every causal key
    (s <= pos[t]) of the kept blocks of (g, t).  One softmax over that set:
      z_s = scale * <q[t,h], k[s,g]>,  w = exp(z - max z),
      out[t,h] = sum_s w_s v[s,g] / sum_s w_s,  lse[t,h] = max z + log sum w.
    The heads of a group share the key set, so they are taken together (one
    column of z per head).  Returns (out [n, H, d], lse [n, H]) in float64.
    """
    qf = _f64(q)
    n, H, d = qf.shape
    G = block_idx.shape[0]
    hpg = H // G
    dv = v.shape[-1]                      # value width (the library requires dv == d)
    out = np.zeros((n, H, dv))
    lse = np.full((n, H), NEG_INF)
    pos = np.asarray(pos, dtype=np.int64)
    for g in range(G):
        k_all = _f64(k[:, g, :])              # the group's keys and values, upcast once
        v_all = _f64(v[:, g, :])
        for t in range(n):
            keys = kept_keys(block_idx[g, t], int(pos[t]), block_size)
            if keys.size == 0:
                continue
            kg = k_all[keys]
            vg = v_all[keys]
            hs = slice(g * hpg, (g + 1) * hpg)
            z = scale * (kg @ qf[t, hs].T)           # [keys, heads]
            m = z.max(axis=0)
            w = np.exp(z - m)
            l = w.sum(axis=0)
            out[t, hs] = (w.T @ vg) / l[:, None]
            lse[t, hs] = m + np.log(l)
    return out, lse


def msa_forward(q, k, v, q_idx, k_idx, len_q: int, len_kv: int, block_size: int,
                top_k: int, scale: float, rows=None, workers: int = 1):
    """Whole path for one sequence: scores -> kept blocks -> attention.

    `rows` optionally restricts the computation to a subset of the
    sequence's query rows (indices into 0..len_q-1); the inputs are always
    the whole sequence.  `workers` threads share the scoring.  Returns
    dict(scores, block_idx, out, lse, pos).
    """
    pos_all = query_positions(len_q, len_kv)
    rows = np.arange(len_q) if rows is None else np.asarray(rows, dtype=np.int64)
    pos = pos_all[rows]
    S = block_scores(q_idx[rows], k_idx, pos, block_size, workers=workers)
    idx = select_blocks(S, pos, block_size, top_k)
    out, lse = sparse_attention(q[rows], k, v, idx, pos, block_size, scale)
    return {"scores": S, "block_idx": idx, "out": out, "lse": lse, "pos": pos}


def block_mass(q, k, block_idx, pos, block_size: int, scale: float) -> np.ndarray:
    """Main Branch distribution over the kept blocks, averaged over the heads
    of each group: the target of the indexer's KL objective (Summary,
    paragraph 2).

    q: [n, H, d]; k: [len_kv, G, d]; block_idx: [G, n, k]; pos: [n].
    With a[t,h,s] the attention weight of key s for head h of row t (the
    softmax of sparse_attention over the union of the kept causal keys),
      p[g, t, i] = (1/hpg) * sum_{h in g} sum_{s in block block_idx[g,t,i], s <= pos[t]} a[t,h,s].
    Padding slots (-1) and rows with no causal key get 0.  Returns float64
    [G, n, k]; each row with a causal key sums to 1.
    """
    qf = _f64(q)
    n, H, _ = qf.shape
    G, _, K = block_idx.shape
    hpg = H // G
    pos = np.asarray(pos, dtype=np.int64)
    mass = np.zeros((G, n, K))
    for t in range(n):
        p = int(pos[t])
        for g in range(G):
            slot_keys = []
            for j in block_idx[g, t]:
                if j < 0:
                    slot_keys.append(np.zeros(0, dtype=np.int64))
                    continue
                s0 = int(j) * block_size
                slot_keys.append(np.arange(s0, min(s0 + block_size, p + 1), dtype=np.int64))
            keys = np.concatenate(slot_keys)
            if keys.size == 0:
                continue
            kg = _gather_f64(k, keys, g)
            for h in range(g * hpg, (g + 1) * hpg):
                z = scale * (kg @ qf[t, h])
                a = np.exp(z - z.max())
                a /= a.sum()
                at = 0
                for i, sk in enumerate(slot_keys):
                    mass[g, t, i] += a[at:at + sk.size].sum() / hpg
                    at += sk.size
    return mass


def indexer_kl(S, block_idx, mass):
    """KL objective of the Index Branch over the kept blocks (Summary,
    paragraph 2), with the Main Branch detached.

    S: [G, n, NB] block scores; block_idx: [G, n, k]; mass: [G, n, k] (the
    block_mass target p).  For row (g, t) with kept slots i:
      q_i  = exp(S[g,t,j_i]) / sum_i' exp(S[g,t,j_i'])    (softmax over the kept blocks)
      kl   = sum_i p_i (log p_i - log q_i)                 (terms with p_i = 0 are 0)
      grad_i = d kl / d S[g,t,j_i] = q_i * sum_i' p_i' - p_i   (p held fixed)
    Padding slots get grad 0; a row without kept blocks gets kl 0.  Returns
    (kl [G, n], grad [G, n, k]) in float64.
    """
    S = np.asarray(S, dtype=np.float64)
    mass = np.asarray(mass, dtype=np.float64)
    G, n, K = block_idx.shape
    kl = np.zeros((G, n))
    grad = np.zeros((G, n, K))
    for g in range(G):
        for t in range(n):
            slots = [i for i in range(K) if block_idx[g, t, i] >= 0]
            if not slots:
                continue
            s = np.array([S[g, t, block_idx[g, t, i]] for i in slots])
            p = mass[g, t, slots]
            logq = s - s.max() - np.log(np.exp(s - s.max()).sum())
            q = np.exp(logq)
            pos_p = p > 0
            kl[g, t] = float((p[pos_p] * (np.log(p[pos_p]) - logq[pos_p])).sum())
            grad[g, t, slots] = q * p.sum() - p
    return kl, grad


def block_argmax(q_row, k_rows) -> int:
    """Index of the largest dot product of q_row with each row of k_rows, ties
    to the lowest index: the key that attains a max-pooled block score
    (Summary, paragraph 2).  fp64 dot products of the upcast inputs, as every
    score of this module; no lower precision is imitated."""
    dots = _f64(k_rows) @ _f64(q_row)
    return int(np.argmax(dots))          # first maximum: the lowest index


def index_backward(q_idx, k_idx, block_idx, pos, block_size: int, grad,
                   return_argmax: bool = False):
    """Backward of the Index Branch's max-pooling (Summary, paragraph 2: the
    scores are max-pooled token-level dot products, so a score's gradient
    reaches the one causal key that attains the block's maximum).

    q_idx: [n, G, d_idx]; k_idx: [len_kv, G, d_idx]; block_idx, grad: [G, n, k];
    pos: [n].  For every kept slot (g, t, i) with block j = block_idx[g,t,i] >= 0
    and causal keys s <= pos[t] of block j, a = the arg-max key
    (block_argmax: fp64 dot products, ties to the lower key), and
      dq_idx[t, g] += grad[g,t,i] * k_idx[a, g]
      dk_idx[a, g] += grad[g,t,i] * q_idx[t, g]
    Slots whose block holds no causal key contribute nothing.  Returns
    (dq_idx [n, G, d_idx], dk_idx [len_kv, G, d_idx]) in float64, and with
    return_argmax also argmax [G, n, k] int64 (the key of each slot, -1 where
    the slot adds nothing).
    """
    G, n, K = block_idx.shape
    L, _, di = k_idx.shape
    pos = np.asarray(pos, dtype=np.int64)
    grad = np.asarray(grad, dtype=np.float64)
    dq = np.zeros((n, G, di))
    dk = np.zeros((L, G, di))
    amax = np.full((G, n, K), -1, dtype=np.int64)
    for g in range(G):
        kg = _f64(k_idx[:, g, :])
        for t in range(n):
            qt = _f64(q_idx[t, g, :])
            for i in range(K):
                j = int(block_idx[g, t, i])
                if j < 0:
                    continue
                s0 = j * block_size
                s1 = min(s0 + block_size, int(pos[t]) + 1, L)
                if s1 <= s0:
                    continue
                a = s0 + block_argmax(qt, kg[s0:s1])
                amax[g, t, i] = a
                dq[t, g] += grad[g, t, i] * kg[a]
                dk[a, g] += grad[g, t, i] * qt
    if return_argmax:
        return dq, dk, amax
    return dq, dk


def sparse_attention_backward(q, k, v, block_idx, pos, block_size: int, scale: float, dout):
    """Gradients of the Main Branch (Summary, paragraph 2: exact softmax
    attention over the kept blocks) with respect to q, k and v, for an
    upstream gradient dout of its output.

    Same key sets as sparse_attention.  For row t and head h of group g, with
    z_s = scale * <q[t,h], k[s,g]>, a = softmax(z), out = sum_s a_s v[s,g]:
      dv[s,g]  += a_s dout[t,h]
      dz_s      = a_s (<dout[t,h], v[s,g]> - <dout[t,h], out[t,h]>)
      dq[t,h]  += scale * sum_s dz_s k[s,g]
      dk[s,g]  += scale * dz_s q[t,h]
    Returns (dq [n, H, d], dk [len_kv, G, d], dv [len_kv, G, dv]) in float64.
    """
    qf = _f64(q)
    do = _f64(dout)
    n, H, d = qf.shape
    G = block_idx.shape[0]
    hpg = H // G
    L = k.shape[0]
    dq = np.zeros_like(qf)
    dk = np.zeros((L, G, d))
    dv = np.zeros((L, G, v.shape[-1]))
    pos = np.asarray(pos, dtype=np.int64)
    for t in range(n):
        for g in range(G):
            keys = kept_keys(block_idx[g, t], int(pos[t]), block_size)
            if keys.size == 0:
                continue
            kg = _gather_f64(k, keys, g)
            vg = _gather_f64(v, keys, g)
            # the keys are distinct and ascending (so are the kept blocks):
            # runs of consecutive positions, each added to dk and dv as a slice
            cut = np.concatenate(([0], np.flatnonzero(np.diff(keys) != 1) + 1, [keys.size]))
            for h in range(g * hpg, (g + 1) * hpg):
                z = scale * (kg @ qf[t, h])
                a = np.exp(z - z.max())
                a /= a.sum()
                out = a @ vg
                dp = vg @ do[t, h]
                dz = a * (dp - do[t, h] @ out)
                dq[t, h] += scale * (dz @ kg)
                gk = scale * np.outer(dz, qf[t, h])
                gv = np.outer(a, do[t, h])
                for r0, r1 in zip(cut[:-1], cut[1:]):
                    s0 = int(keys[r0])
                    dk[s0:s0 + r1 - r0, g, :] += gk[r0:r1]
                    dv[s0:s0 + r1 - r0, g, :] += gv[r0:r1]
    return dq, dk, dv


# ------------------------------------------------------------------------
# Hierarchical (coarse-to-fine) indexing: an approximation of the selection
# ("LongCat Sparse Attention" page, Abstract, strategy (3): a coarse-to-fine
# scoring scheme narrows each query's candidate set to cut the indexing
# computation).  The page gives no formula; the reading taken here:
#   * chunks of S consecutive blocks; a chunk's coarse key is the mean of
#     its B*S index keys (a chunk summary, computed once per cache);
#   * for a query at position p (current block J, current chunk cJ = J // S),
#     the coarse candidates are the chunks c < cJ, all of whose keys are
#     causal; each scores <q_idx, coarse key>;
#   * the C best of them (score descending, chunk ascending) are kept, or all
#     of them when there are at most C;
#   * the fine candidates are the blocks of the kept chunks plus the blocks
#     of the current chunk below J (the nearby blocks are always scored);
#     each gets the exact max-pooled block score;
#   * the k-1 best fine candidates (score descending, block ascending) and J
#     are kept, as in select_blocks; rows with J <= k-1 keep 0..J.
# With C at least the number of chunks every candidate block is scored and
# the result is select_blocks' exactly.
# ------------------------------------------------------------------------

def chunk_keys(k_idx, block_size: int, chunk_blocks: int) -> np.ndarray:
    """Coarse keys of one sequence: [n_full_chunks, G, d_idx] fp64, the mean
    of the index keys of every full chunk of chunk_blocks blocks."""
    k = _f64(k_idx)
    L, G, di = k.shape
    span = block_size * chunk_blocks
    nfull = L // span
    return k[:nfull * span].reshape(nfull, span, G, di).mean(axis=1)


def hierarchical_select(q_idx, k_idx, pos, block_size: int, top_k: int, chunk_blocks: int,
                        keep_chunks: int):
    """Kept blocks of the hierarchical reading above, for rows q_idx [n, G, d_idx]
    at positions pos of one sequence (k_idx [len_kv, G, d_idx]).

    Returns dict(coarse [G, n, n_full_chunks] (-inf where not a candidate),
    kept_chunks [G, n, keep_chunks] ascending, -1 padded, fine [G, n, NB]
    (-inf where not a fine candidate), block_idx [G, n, top_k] ascending,
    -1 padded)."""
    q = _f64(q_idx)
    pos = np.asarray(pos, dtype=np.int64)
    n, G, _ = q.shape
    B, S, C, k = block_size, chunk_blocks, keep_chunks, top_k
    kbar = chunk_keys(k_idx, B, S)
    nch = kbar.shape[0]
    nb = num_blocks(k_idx.shape[0], B)
    exact = block_scores(q_idx, k_idx, pos, B)          # fine scores are exact block scores
    coarse = np.full((G, n, nch), NEG_INF)
    kept = np.full((G, n, C), -1, dtype=np.int32)
    fine = np.full((G, n, nb), NEG_INF)
    out = np.full((G, n, k), -1, dtype=np.int32)
    for g in range(G):
        for t in range(n):
            J = int(pos[t] // B)
            cJ = J // S
            cand_chunks = np.arange(cJ)
            coarse[g, t, :cJ] = kbar[:cJ, g, :] @ q[t, g]
            if cJ <= C:
                keep = cand_chunks
            else:
                order = np.lexsort((cand_chunks, -coarse[g, t, :cJ]))
                keep = np.sort(cand_chunks[order[:C]])
            kept[g, t, :len(keep)] = keep
            blocks = [c * S + s for c in keep for s in range(S)] + list(range(cJ * S, J))
            blocks = np.array(sorted(blocks), dtype=np.int64)
            fine[g, t, blocks] = exact[g, t, blocks]
            if J <= k - 1:
                sel = list(range(J + 1))
            else:
                order = np.lexsort((blocks, -fine[g, t, blocks]))
                sel = sorted(int(j) for j in blocks[order[:k - 1]]) + [J]
            out[g, t, :len(sel)] = sel
    return {"coarse": coarse, "kept_chunks": kept, "fine": fine, "block_idx": out}


def selection_recall(sel, ref, pos, block_size: int, top_k: int) -> float:
    """Share of the reference's freely chosen blocks (all but the forced
    current block, on rows with more than k-1 candidates) that sel keeps."""
    pos = np.asarray(pos, dtype=np.int64)
    hit = tot = 0
    G, n, _ = ref.shape
    for g in range(G):
        for t in range(n):
            J = int(pos[t] // block_size)
            if J <= top_k - 1:
                continue
            r = set(int(x) for x in ref[g, t] if 0 <= x < J)
            s = set(int(x) for x in sel[g, t] if 0 <= x < J)
            hit += len(r & s)
            tot += len(r)
    return hit / tot if tot else 1.0
