"""GPU parity of msa_sparse_attn_bwd (the Main Branch backward) against the
oracle's sparse_attention_backward.

Tolerance: every gradient within 2e-2 x max |ref| of the oracle's fp64 value
(the bar of the bf16 forward output, taken relative to the gradient's
scale).  The kernels read bf16 inputs, round P and dS to bf16 before the
MFMA products that use them and each slot's share of dq to bf16, and sum in
fp32: a relative error of a few 2^-9 per term, well inside the bar, while a
wrong index, sign or mask gives errors of the order of the gradient itself.

At full size, where the key-side sums cannot be formed by the oracle for
every key, dq is checked on sampled rows, dk and dv on every key of two late
blocks (all rows that keep them), and on every key through two
identities of attention's gradient: sum_s dk[s, g] = 0 (each row's dS sums
to 0 over its keys) and sum_s <dv[s, g], v[s, g]> = sum over the group's
(row, head) of <dout, out>.
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
TOL = 2e-2


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _close(gpu, ref, name, tol=TOL):
    scale = max(float(np.abs(ref).max()) if ref.size else 0.0, 1e-30)
    err = float(np.abs(gpu - ref).max()) / scale if ref.size else 0.0
    assert err <= tol, f"{name}: max error {err:.3g} x max |ref| > {tol}"
    return err


def _cu(lengths):
    cu = [0]
    for x in lengths:
        cu.append(cu[-1] + x)
    return cu


def _forward_and_backward(inp, H, G, d, di, B, k, block_idx=None, seed=5, dtype="bf16"):
    prob = C.problem_for(inp, H, G, d, di, B, k, dtype)
    if block_idx is None:
        scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
        block_idx = msa.topk_select(prob, scores)
    out, lse = msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], block_idx, return_lse=True)
    dout = W.random_out_grad(seed, prob.total_q, H, d, dtype, device=DEV)
    dq, dk, dv = msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], block_idx, out, lse, dout)
    torch.cuda.synchronize()
    return prob, block_idx, out, lse, dout, dq, dk, dv


def _oracle_all(inp, block_idx, dout, B, d):
    """Oracle gradients of every row and key, sequence by sequence."""
    cu_q, cu_kv = _cu(inp["len_q"]), _cu(inp["len_kv"])
    bi = block_idx.cpu().numpy()
    dq = np.zeros(tuple(inp["q"].shape))
    dk = np.zeros(tuple(inp["k"].shape))
    dv = np.zeros(tuple(inp["v"].shape))
    for si, (lq, lkv) in enumerate(zip(inp["len_q"], inp["len_kv"])):
        if lq == 0:
            continue
        sq, skv = slice(cu_q[si], cu_q[si] + lq), slice(cu_kv[si], cu_kv[si] + lkv)
        pos = O.query_positions(lq, lkv)
        a, b_, c = O.sparse_attention_backward(
            inp["q"][sq].cpu(), inp["k"][skv].cpu(), inp["v"][skv].cpu(), bi[:, sq, :], pos, B,
            1.0 / math.sqrt(d), dout[sq].cpu())
        dq[sq], dk[skv], dv[skv] = a, b_, c
    return dq, dk, dv


BWD_CASES = [
    # name, len_q, len_kv, H, G, k  (head dim 128, block size 128)
    ("varlen-hpg4", [200, 1, 0, 130], [600, 513, 64, 130], 4, 1, 4),
    ("hpg1", [400], [1000], 2, 2, 6),
    ("hpg8", [256, 130], [384, 130], 8, 1, 3),
    ("hpg16-shared-buckets", [300], [400], 16, 1, 3),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_attn_backward_small(case):
    """The path's own selection; every row and key against the oracle.  The
    hpg16 case has buckets of more than one work item (partial sums)."""
    name, lq, lkv, H, G, k = case
    d, di, B = 128, 64, 128
    inp = W.random_case(61, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    _log(f"{name}: GPU")
    prob, bi, out, lse, dout, dq, dk, dv = _forward_and_backward(inp, H, G, d, di, B, k)
    _, _, _, _, _, dq2, dk2, dv2 = _forward_and_backward(inp, H, G, d, di, B, k, block_idx=bi)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), \
        "two runs differ: the sums must be deterministic"
    _log(f"{name}: oracle")
    rq, rk, rv = _oracle_all(inp, bi, dout, B, d)
    e = (_close(dq.cpu().numpy(), rq, "dq"), _close(dk.cpu().numpy(), rk, "dk"),
         _close(dv.cpu().numpy(), rv, "dv"))
    _log(f"{name}: errors dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")


def _bwd_with_workspace(prob, inp, bi, out, lse, dout, nbytes):
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    got = msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], bi, out, lse, dout, workspace=ws)
    torch.cuda.synchronize()
    return got


def _check_passes(prob, inp, bi, out, lse, dout, ref, nbytes, tag):
    """The backward over a workspace of nbytes (passes over the query rows):
    dq equal to the single pass bit for bit, dk and dv within fp32 rounding
    of it (the passes' sums are added in pass order), two runs identical."""
    dq, dk, dv = _bwd_with_workspace(prob, inp, bi, out, lse, dout, nbytes)
    dq2, dk2, dv2 = _bwd_with_workspace(prob, inp, bi, out, lse, dout, nbytes)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    assert torch.equal(dq, ref[0]), f"{tag}: dq differs from the single pass"
    for got, r, nm in ((dk, ref[1], "dk"), (dv, ref[2], "dv")):
        scale = float(r.abs().max())
        err = float((got - r).abs().max()) / max(scale, 1e-30)
        assert err <= 1e-5, f"{tag}: {nm} differs from the single pass by {err:.2e} x max"
    _log(f"  {tag}: workspace {nbytes} bytes: dq equal, dk / dv within rounding")
    return dq, dk, dv


@pytest.mark.parametrize("case", [BWD_CASES[0], BWD_CASES[1], BWD_CASES[3]],
                         ids=[BWD_CASES[0][0], BWD_CASES[1][0], BWD_CASES[3][0]])
def test_attn_backward_passes_small(case):
    """A workspace below the single-pass size runs the rows in passes (256
    rows at the least): results as above, and against the oracle."""
    name, lq, lkv, H, G, k = case
    d, di, B = 128, 64, 128
    inp = W.random_case(71, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    prob, bi, out, lse, dout, dq, dk, dv = _forward_and_backward(inp, H, G, d, di, B, k)
    full = msa.sparse_attn_bwd_workspace_size(prob)
    least = msa.sparse_attn_bwd_workspace_size(prob, minimum=True)
    assert 0 < least < full
    with pytest.raises(msa.MsaError) as e:
        _bwd_with_workspace(prob, inp, bi, out, lse, dout, least - 1)
    assert e.value.status == 5
    got = _check_passes(prob, inp, bi, out, lse, dout, (dq, dk, dv), least, name)
    rq, rk, rv = _oracle_all(inp, bi, dout, B, d)
    for g_, r_, nm in zip(got, (rq, rk, rv), ("dq", "dk", "dv")):
        _close(g_.cpu().numpy(), r_, nm)


def test_attn_backward_passes_prefill_32k():
    """prefill-32k with the least workspace (128 passes) and a quarter of the
    single-pass one."""
    w = W.WORKLOADS["prefill-32k"]
    inp = W.make_inputs(w, device=DEV, seed=0)
    H, G, d, di, B, k = w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim, w.block_size, w.top_k
    prob, bi, out, lse, dout, dq, dk, dv = _forward_and_backward(inp, H, G, d, di, B, k)
    full = msa.sparse_attn_bwd_workspace_size(prob)
    least = msa.sparse_attn_bwd_workspace_size(prob, minimum=True)
    for nbytes in (least, full // 4):
        _check_passes(prob, inp, bi, out, lse, dout, (dq, dk, dv), nbytes, "prefill-32k")


@pytest.mark.parametrize("seed", [3, 4])
def test_attn_backward_arbitrary_lists(seed):
    """Kept-block lists that no selection produced: distinct blocks up to J,
    the current block present or not, any slot order, empty rows (dq 0)."""
    lq, lkv, H, G, k = [300, 1, 130], [700, 513, 130], 4, 2, 5
    d, di, B = 128, 64, 128
    inp = W.random_case(seed, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    lists = W.random_block_lists(seed, lq, lkv, G, B, k).to(DEV)
    _log(f"arbitrary lists seed {seed}: GPU")
    _, _, _, _, dout, dq, dk, dv = _forward_and_backward(inp, H, G, d, di, B, k, block_idx=lists)
    rq, rk, rv = _oracle_all(inp, lists, dout, B, d)
    _close(dq.cpu().numpy(), rq, "dq")
    _close(dk.cpu().numpy(), rk, "dk")
    _close(dv.cpu().numpy(), rv, "dv")
    empty = (lists.cpu() < 0).all(dim=2)  # [G, total_q] rows of a group without a kept block
    hpg = H // G
    for g in range(G):
        rows = torch.nonzero(empty[g]).flatten()
        if rows.numel():
            assert torch.all(dq[rows][:, g * hpg:(g + 1) * hpg] == 0)


def test_attn_backward_more_queries_than_keys():
    """Rows at negative positions (len_q > len_kv) have no causal key: dq 0,
    and every other output equals, bit for bit, that of the trimmed problem."""
    H, G, d, di, B, k = 8, 2, 128, 64, 128, 4
    inp = W.random_case(79, [300, 400], [200, 500], H, G, d, di, B, k, "bf16", device=DEV)
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
        out, lse = msa.sparse_attn_fwd(prob, case["q"], case["k"], case["v"], idx, return_lse=True)
        dout = W.random_out_grad(9, 700, H, d, "bf16", device=DEV)
        if case is trim:
            dout = dout[cut:].contiguous()
        res.append(msa.sparse_attn_bwd(prob, case["q"], case["k"], case["v"], idx, out, lse, dout))
    torch.cuda.synchronize()
    (dq_f, dk_f, dv_f), (dq_t, dk_t, dv_t) = res
    assert torch.all(dq_f[:cut] == 0)
    assert torch.equal(dq_f[cut:], dq_t)
    assert torch.equal(dk_f, dk_t) and torch.equal(dv_f, dv_t)


@pytest.mark.parametrize("name", ["prefill-32k", "prefill-128k", "chunked-prefill-1m"])
def test_attn_backward_full_size(name):
    """The long-context workloads with the default (single-pass) workspace:
    sampled dq rows, every key of block NB-2 of group 0, of block NB-1 of
    group G-1 and of a block of group 1 kept by more rows than one work item
    holds (all rows that keep them), and the two identities over every
    key."""
    w = W.WORKLOADS[name]
    _log(f"{name}: generating")
    inp = W.make_inputs(w, device=DEV, seed=0)
    H, G, d, di, B, k = w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim, w.block_size, w.top_k
    _log(f"{name}: GPU")
    prob, bi, out, lse, dout, dq, dk, dv = _forward_and_backward(inp, H, G, d, di, B, k)
    lq, L = inp["len_q"][0], inp["len_kv"][0]
    pos_all = O.query_positions(lq, L)
    scale = 1.0 / math.sqrt(d)
    bi_h = bi.cpu().numpy()
    q_h, k_h, v_h, do_h = inp["q"].cpu(), inp["k"].cpu(), inp["v"].cpu(), dout.cpu()
    # sampled rows: dq of a row depends on that row alone
    rows = np.unique(np.array([0, 1, 127, 128, lq // 7, lq // 2, lq - 1], dtype=np.int64))
    _log(f"{name}: oracle dq rows")
    tr = torch.from_numpy(rows)
    rq, _, _ = O.sparse_attention_backward(q_h[tr], k_h, v_h, bi_h[:, rows, :], pos_all[rows], B,
                                           scale, do_h[tr])
    e_q = _close(dq[torch.from_numpy(rows).to(DEV)].cpu().numpy(), rq, "dq rows")
    # two late blocks, and a block whose list the matrix-core backward splits
    # into two work items (4096 (query, head) rows each) summed in item
    # order: all rows that keep them, on their group alone (its heads, keys
    # and values; the other groups do not reach these keys)
    nb = (L + B - 1) // B
    hpg = H // G
    per_item = 4096 // hpg
    counts = np.bincount(bi_h[1][bi_h[1] >= 0], minlength=nb)
    two = np.nonzero(counts > per_item)[0]
    blocks = [(0, nb - 2), (G - 1, nb - 1)]
    if two.size:
        blocks.append((1, int(two[np.argmin(counts[two])])))
    e_k = e_v = 0.0
    for g, jb in blocks:
        keep = np.nonzero((bi_h[g] == jb).any(axis=1))[0]
        _log(f"{name}: oracle block {jb} of group {g} ({keep.size} rows keep it)")
        assert keep.size > 0
        tk, hs = torch.from_numpy(keep), slice(g * hpg, (g + 1) * hpg)
        _, rk, rv = O.sparse_attention_backward(q_h[tk][:, hs], k_h[:, g:g + 1], v_h[:, g:g + 1],
                                                bi_h[g:g + 1, keep], pos_all[keep], B, scale,
                                                do_h[tk][:, hs])
        ks = slice(jb * B, min((jb + 1) * B, L))
        e_k = max(e_k, _close(dk[ks, g].cpu().numpy(), rk[ks, 0], f"dk block {jb} group {g}"))
        e_v = max(e_v, _close(dv[ks, g].cpu().numpy(), rv[ks, 0], f"dv block {jb} group {g}"))
        del rk, rv
    # identities over every key
    dk64, dv64 = dk.double(), dv.double()
    ksum = dk64.sum(dim=0)                     # [G, d]
    kabs = dk64.abs().sum(dim=0)
    del dk64
    assert float((ksum.abs() / kabs.clamp_min(1e-30)).max()) <= TOL, "sum over keys of dk is not 0"
    lhs = (dv64 * inp["v"].double()).sum(dim=(0, 2))      # [G]
    del dv64
    dd = (dout.double() * out.double()).sum(dim=2)        # [total_q, H]
    rhs = dd.view(-1, G, H // G).sum(dim=(0, 2))
    n_terms = dd.numel() / G
    bound = TOL * dd.abs().view(-1, G, H // G).sum(dim=(0, 2)) / math.sqrt(n_terms)
    assert torch.all((lhs - rhs).abs() <= bound), f"sum <dv, v> {lhs} vs sum <dout, out> {rhs}"
    _log(f"{name}: dq rows {e_q:.2e}, late blocks dk {e_k:.2e} dv {e_v:.2e}")


def test_attn_backward_no_query_rows():
    """No query row at all: the call only clears dk and dv (no workspace)."""
    H, G, d, di, B, k = 8, 2, 128, 64, 128, 4
    inp = W.random_case(80, [0], [300], H, G, d, di, B, k, "bf16", device=DEV)
    prob = C.problem_for(inp, H, G, d, di, B, k, "bf16")
    empty_idx = torch.empty((G, 0, k), dtype=torch.int32, device=DEV)
    empty_rows = torch.empty((0, H, d), dtype=torch.bfloat16, device=DEV)
    empty_lse = torch.empty((0, H), dtype=torch.float32, device=DEV)
    dq, dk, dv = msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], empty_idx, empty_rows,
                                     empty_lse, empty_rows)
    torch.cuda.synchronize()
    assert dq.numel() == 0
    assert torch.all(dk == 0) and torch.all(dv == 0)


FMA_CASES = [
    # name, len_q, len_kv, H, G, d, B, k, dtype, tolerance (x max |ref|)
    ("f32-d64-B64", [300, 1, 130], [500, 129, 130], 4, 2, 64, 64, 4, "f32", 1e-4),
    ("f32-d128-B128", [200, 70], [400, 70], 2, 1, 128, 128, 3, "f32", 1e-4),
    ("bf16-d64-B64", [250, 100], [600, 100], 8, 2, 64, 64, 5, "bf16", TOL),
    ("bf16-hpg3", [200], [450], 6, 2, 128, 128, 3, "bf16", TOL),
]


@pytest.mark.parametrize("case", FMA_CASES, ids=[c[0] for c in FMA_CASES])
def test_attn_backward_fma_path(case):
    """Problems outside the MFMA kernel's shapes (fp32, head dim 64, block size
    64, 3 heads per group) take the plain fp32 FMA kernels: every row and key
    against the oracle; fp32 inputs to 1e-4 of max |ref|.  Deterministic."""
    name, lq, lkv, H, G, d, B, k, dtype, tol = case
    di = 64
    inp = W.random_case(62, lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    _log(f"{name}: GPU")
    prob, bi, out, lse, dout, dq, dk, dv = _forward_and_backward(inp, H, G, d, di, B, k,
                                                                 dtype=dtype)
    _, _, _, _, _, dq2, dk2, dv2 = _forward_and_backward(inp, H, G, d, di, B, k, block_idx=bi,
                                                         dtype=dtype)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)
    _log(f"{name}: oracle")
    rq, rk, rv = _oracle_all(inp, bi, dout, B, d)
    e = (_close(dq.cpu().numpy(), rq, "dq", tol), _close(dk.cpu().numpy(), rk, "dk", tol),
         _close(dv.cpu().numpy(), rv, "dv", tol))
    _log(f"{name}: errors dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")


@pytest.mark.parametrize("shape", ["query-major-forward", "decode-rows"])
def test_attn_backward_other_forward_shapes(shape):
    """The backward from the query-major forward's out and LSE, and on
    decode-shaped rows (one query per sequence: many single-entry buckets),
    every row and key against the oracle."""
    d, di, B = 128, 64, 128
    if shape == "query-major-forward":
        lq, lkv, H, G, k, sched = [300, 130], [700, 130], 8, 2, 4, "query_major"
    else:
        lq, lkv, H, G, k, sched = [1] * 9, [130, 1000, 257, 64, 1, 700, 384, 129, 2048], 8, 2, 6, "auto"
    inp = W.random_case(63, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    prob = C.problem_for(inp, H, G, d, di, B, k, "bf16", sched)
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    bi = msa.topk_select(prob, scores)
    out, lse = msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], bi, return_lse=True)
    dout = W.random_out_grad(6, prob.total_q, H, d, "bf16", device=DEV)
    _log(f"{shape}: GPU")
    dq, dk, dv = msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], bi, out, lse, dout)
    torch.cuda.synchronize()
    rq, rk, rv = _oracle_all(inp, bi, dout, B, d)
    e = (_close(dq.cpu().numpy(), rq, "dq"), _close(dk.cpu().numpy(), rk, "dk"),
         _close(dv.cpu().numpy(), rv, "dv"))
    _log(f"{shape}: errors dq {e[0]:.2e} dk {e[1]:.2e} dv {e[2]:.2e}")
