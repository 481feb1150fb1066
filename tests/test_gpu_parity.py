"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Small cases are checked on every row; the long-context workloads on sampled
rows (first rows, block edges, planted rows, random rows, last rows), with the
launch configuration the benchmark times.
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


SMALL = [
    # name, len_q, len_kv, H, G, d, d_idx, B, k
    ("ragged-1000", [1000], [1000], 8, 2, 128, 64, 128, 4),
    ("varlen-chunked", [300, 1, 700, 0], [300, 513, 1500, 64], 4, 4, 64, 32, 64, 3),
    ("hpg16-dsi128", [777], [777], 16, 1, 128, 128, 64, 8),
    ("k1", [520], [600], 4, 2, 64, 64, 128, 1),
    ("k-covers-all", [640], [640], 4, 1, 128, 64, 64, 16),
    ("two-tiles-of-queries", [600], [2000], 8, 8, 128, 64, 128, 5),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_all_rows(case, dtype):
    name, lq, lkv, H, G, d, di, B, k = case
    _log(f"case {name} {dtype}")
    inp = W.random_case(SMALL.index(case), lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    st = C.run_and_check(inp, H, G, d, di, B, k, dtype)
    _log(f"  {st}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_kv_major_schedule(dtype):
    """Both prefill schedules give the oracle's result."""
    name, lq, lkv, H, G, d, di, B, k = SMALL[0]
    inp = W.random_case(5, lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    for sched in ("query_major", "kv_major"):
        if sched == "kv_major" and dtype == "f32":
            continue
        _log(f"schedule {sched} {dtype}")
        C.run_and_check(inp, H, G, d, di, B, k, dtype, schedule=sched)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", [SMALL[0], SMALL[1]], ids=[SMALL[0][0], SMALL[1][0]])
def test_unsorted_block_lists(case, dtype):
    """The kept-block lists are sets: any order of a row's entries gives the oracle's result."""
    name, lq, lkv, H, G, d, di, B, k = case
    inp = W.random_case(40 + SMALL.index(case), lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    for sched in ("query_major", "kv_major"):
        if sched == "kv_major" and dtype == "f32":
            continue
        _log(f"unsorted lists {name} {sched} {dtype}")
        C.run_and_check(inp, H, G, d, di, B, k, dtype, schedule=sched, shuffle_slots=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_decode_batch(dtype):
    """max_q_len == 1: streaming index kernel and split-KV attention."""
    lkv = [1, 127, 128, 129, 5000, 64, 3000]
    inp = W.random_case(11, [1] * len(lkv), lkv, 8, 2, 128, 64, 128, 4, dtype, device=DEV)
    C.run_and_check(inp, 8, 2, 128, 64, 128, 4, dtype)
    inp = W.random_case(12, [1] * 3, [4096, 70, 9000], 16, 8, 64, 64, 64, 9, dtype, device=DEV)
    C.run_and_check(inp, 16, 8, 64, 64, 64, 9, dtype)


def test_tiny_fp32_workload_every_row():
    w = W.WORKLOADS["tiny-fp32"]
    inp = W.make_inputs(w, device=DEV, seed=0)
    st = C.run_and_check(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                         w.block_size, w.top_k, w.dtype)
    _log(f"tiny-fp32 {st}")
    assert st["rows"] == 1024


def test_topk_exact_on_synthetic_scores():
    """Selection alone, on generated score rows with many exact ties: bit-exact.

    Row lengths reach every kernel variant: one wave per row with 1, 8 and 32
    chunks of 64 keys in registers, and four waves per row (up to 4096 and
    8192 blocks); every 17th row is constant, which forces the exact search
    over the whole row."""
    for nb, lq, levels, B, k in ((16, 1024, 3, 64, 13), (300, 300 * 64, 2, 64, 13),
                                 (1100, 70000, 0, 64, 13), (3000, 4000, 2, 64, 13),
                                 (3000, 3000, 1, 64, 64), (8192, 2048, 5, 128, 64)):
        lkv = nb * B
        lq = min(lq, lkv)
        G = 2
        prob = msa.Problem.from_lengths([lq], [lkv], 4, G, 64, 64, B, k, "bf16", DEV)
        scores = W.random_scores(nb, G, lq, nb, levels=levels)
        idx = msa.topk_select(prob, scores.to(DEV)).cpu().numpy()
        pos = O.query_positions(lq, lkv)
        rows = np.unique(np.concatenate([np.arange(0, lq, max(1, lq // 300)), [lq - 1]]))
        ref = O.select_blocks(scores[:, rows, :].numpy(), pos[rows], B, k)
        assert np.array_equal(idx[:, rows, :], ref), f"nb={nb}"
        _log(f"topk nb={nb} rows={len(rows)} ok")


def test_closed_forms_constant_v_and_zero_q():
    """Constant V gives that constant; Q = 0 gives the mean of V over the kept keys.

    Partial results are held in bf16 before the merge, so the constant comes
    back within one bf16 step of it (2^-6 for |c| in [2, 4)); the bound is the
    bf16 output tolerance, 2e-2."""
    lq, lkv, H, G, d, di, B, k = [900], [1300], 8, 2, 128, 64, 128, 4
    inp = W.random_case(21, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    prob = C.problem_for(inp, H, G, d, di, B, k, "bf16")
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    idx = msa.topk_select(prob, scores)
    c = torch.linspace(-3, 3, d, device=DEV).to(torch.bfloat16)
    v_const = c.expand(lkv[0], G, d).contiguous()
    for sched in ("query_major", "kv_major"):
        p2 = prob.with_schedule(sched)
        out, _ = msa.sparse_attn_fwd(p2, inp["q"], inp["k"], v_const, idx)
        assert (out.float() - c.float()).abs().max().item() <= 2e-2
        q0 = torch.zeros_like(inp["q"])
        out0, lse0 = msa.sparse_attn_fwd(p2, q0, inp["k"], inp["v"], idx, return_lse=True)
        idx_h = idx.cpu().numpy()
        pos = O.query_positions(lq[0], lkv[0])
        v_h = inp["v"].float().cpu().numpy()
        out0_h = out0.float().cpu().numpy()
        lse0_h = lse0.cpu().numpy()
        for t in range(0, lq[0], 37):
            for g in range(G):
                keys = [s for s in range(lkv[0]) if s <= pos[t] and (s // B) in set(idx_h[g, t])]
                mean = v_h[keys, g].mean(axis=0)
                for h in range(g * (H // G), (g + 1) * (H // G)):
                    assert np.abs(out0_h[t, h] - mean).max() <= 1e-2
                    assert abs(lse0_h[t, h] - math.log(len(keys))) <= 1e-4


def test_deterministic():
    lq, lkv, H, G, d, di, B, k = [1000], [1000], 8, 2, 128, 64, 128, 6
    inp = W.random_case(31, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    for sched in ("query_major", "kv_major"):
        prob = C.problem_for(inp, H, G, d, di, B, k, "bf16", sched)
        a = msa.msa_forward(prob, inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], True)
        b = msa.msa_forward(prob, inp["q"], inp["k"], inp["v"], inp["q_idx"], inp["k_idx"], True)
        for x, y in zip(a, b):
            assert torch.equal(x, y)


def test_empty_batch():
    prob = msa.Problem.from_lengths([0], [0], 4, 2, 64, 64, 64, 4, "bf16", DEV)
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((0, 4, 64), dtype=torch.bfloat16, device=DEV)
    s = msa.index_score(prob, e, e)
    idx = msa.topk_select(prob, s)
    out, _ = msa.sparse_attn_fwd(prob, q, e, e, idx)
    assert out.shape == (0, 4, 64)


# ---------------------------------------------------------- full workloads --

def _full_size_rows(lq, planted, seed, B=128):
    """Rows the oracle checks on a long workload (>= 512): the whole first and
    last 128-query blocks, the whole block holding the most planted queries of
    group 0 (besides those two), 8 planted rows of every group, both sides of
    16 block edges and 128 random rows."""
    rng = np.random.default_rng(seed)
    rows = set(range(0, min(B, lq)))
    rows.update(range(max(0, lq - B), lq))
    if planted and planted[0]:
        counts = np.bincount(np.asarray(planted[0]) // B, minlength=-(-lq // B))
        counts[0] = counts[-1] = -1
        b = int(np.argmax(counts))
        rows.update(range(b * B, min(lq, (b + 1) * B)))
        for g_rows in planted:
            rows.update(rng.choice(g_rows, size=min(8, len(g_rows)), replace=False).tolist())
    for e in rng.integers(1, max(2, lq // B), 16).tolist():
        rows.update([e * B - 1, e * B])
    rows.update(rng.integers(0, lq, 128).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < lq))


@pytest.mark.parametrize("name", ["prefill-32k", "prefill-128k", "chunked-prefill-1m"])
def test_long_prefill(name):
    """The benchmark's workloads at full size: >= 512 rows against the oracle
    (scores within the rounding bound, delta-valid selection, attention on the
    oracle's selection), and the Top-k of every row against the selection rule
    on the library's own scores."""
    w = W.WORKLOADS[name]
    _log(f"workload {name}: generating")
    inp = W.make_inputs(w, device=DEV, seed=0)
    rows = [_full_size_rows(inp["len_q"][0], inp["planted_q"][0] if inp["planted_q"] else [], 1)]
    assert len(rows[0]) >= 512
    _log(f"workload {name}: running + oracle on {len(rows[0])} rows, Top-k on every row")
    st = C.run_and_check(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                         w.block_size, w.top_k, w.dtype, rows_per_seq=rows,
                         topk_every_row=True, cheap_bound=True, progress=True)
    _log(f"  {st}")


def test_large_varlen_batch():
    """A packed batch of four planted sequences of the prefill-32k shape with
    mixed lengths (a full prefill, a single-query row at 70K keys, a 9K-query
    chunk at the end of 40K keys, and the longest prefill last): the KV-major
    schedule's segments and entries span sequences.  Sampled rows of every
    sequence against the oracle, and the Top-k of every row against the
    selection rule on the library's own scores."""
    w = W.Workload("varlen-batch", 32, 8, 128, 64, 128, 16, "bf16", True,
                   len_q=(20000, 1, 9000, 30000), len_kv=(20000, 70000, 40000, 30000),
                   num_seqs=4)
    _log("varlen batch: generating")
    inp = W.make_inputs(w, device=DEV, seed=11)
    rng = np.random.default_rng(11)
    rows = []
    for lq in w.len_q:
        r = set(range(min(64, lq))) | set(range(max(0, lq - 64), lq))
        r |= set(rng.integers(0, lq, 64).tolist())
        rows.append(np.array(sorted(r)))
    _log(f"varlen batch: oracle on {sum(len(r) for r in rows)} rows, Top-k on every row")
    st = C.run_and_check(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                         w.block_size, w.top_k, w.dtype, rows_per_seq=rows,
                         topk_every_row=True, cheap_bound=True, progress=True)
    assert st["rows"] == sum(len(r) for r in rows)
    _log(f"  {st}")


def test_decode_workload_every_sequence():
    w = W.WORKLOADS["decode-64x256k"]
    _log("decode workload: generating")
    inp = W.make_inputs(w, device=DEV, seed=0)
    rows = [[0]] * w.num_seqs
    st = C.run_and_check(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                         w.block_size, w.top_k, w.dtype, rows_per_seq=rows, cheap_bound=True,
                         progress=True)
    assert st["rows"] == w.num_seqs
    _log(f"  {st}")


def test_more_queries_than_keys():
    """A sequence with len_q > len_kv (the ABI treats its rows at negative
    positions as having no causal key): those rows get scores -inf, no kept
    block, output 0 and LSE -inf; every other row equals, bit for bit, the same
    row of the trimmed problem (the sequence keeps its last len_kv queries),
    which is checked against the oracle."""
    H, G, d, di, B, k = 8, 2, 128, 64, 128, 4
    inp = W.random_case(77, [300, 400], [200, 500], H, G, d, di, B, k, "bf16", device=DEV)
    cut = 100  # rows 0..99 of sequence 0 sit at positions -100..-1
    trim = dict(inp)
    trim["len_q"] = [200, 400]
    trim["cu_q"] = torch.tensor([0, 200, 600], dtype=torch.int64, device=DEV)
    for key in ("q_idx", "q"):
        trim[key] = inp[key][cut:].contiguous()
    _log("trimmed problem against the oracle")
    C.run_and_check(trim, H, G, d, di, B, k, "bf16")
    for sched in ("query_major", "kv_major"):
        _log(f"more queries than keys, {sched}")
        res = []
        for case in (inp, trim):
            prob = C.problem_for(case, H, G, d, di, B, k, "bf16", sched)
            scores = msa.index_score(prob, case["q_idx"], case["k_idx"])
            idx = msa.topk_select(prob, scores)
            out, lse = msa.sparse_attn_fwd(prob, case["q"], case["k"], case["v"], idx,
                                           return_lse=True)
            res.append((scores, idx, out, lse))
        (s_f, i_f, o_f, l_f), (s_t, i_t, o_t, l_t) = res
        assert torch.all(s_f[:, :cut, :] == -math.inf)
        assert torch.all(i_f[:, :cut, :] == -1)
        assert torch.all(o_f[:cut] == 0)
        assert torch.all(l_f[:cut] == -math.inf)
        nb_t = s_t.shape[2]
        assert torch.equal(s_f[:, cut:, :nb_t], s_t)
        assert torch.equal(i_f[:, cut:, :], i_t)
        assert torch.equal(o_f[cut:], o_t)
        assert torch.equal(l_f[cut:], l_t)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_arbitrary_kept_lists(dtype):
    """The attention call on kept-block lists that no selection produced: any
    number of distinct blocks up to J, the current block present or not, in
    any slot order, empty rows included (output 0, LSE -inf), against the
    oracle's attention on the same lists.  Prefill on both schedules, and
    decode."""
    H, G, d, di, B, k = 8, 2, 128, 64, 128, 6
    cases = [("prefill", [700, 1, 300], [900, 513, 300], ("query_major", "kv_major")),
             ("decode", [1] * 5, [1, 127, 129, 3000, 900], ("auto",))]
    for name, lq, lkv, scheds in cases:
        inp = W.random_case(61, lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
        lists = W.random_block_lists(61, lq, lkv, G, B, k)
        idx = lists.to(DEV)
        q_h, k_h, v_h = (inp[t].float().cpu() for t in ("q", "k", "v"))
        refs = []
        q0 = kv0 = 0
        for a, b in zip(lq, lkv):
            pos = O.query_positions(a, b)
            o, l = O.sparse_attention(q_h[q0:q0 + a], k_h[kv0:kv0 + b], v_h[kv0:kv0 + b],
                                      lists[:, q0:q0 + a, :].numpy(), pos, B, 1.0 / math.sqrt(d))
            refs.append((o, l))
            q0, kv0 = q0 + a, kv0 + b
        ref_o = np.concatenate([r[0] for r in refs])
        ref_l = np.concatenate([r[1] for r in refs])
        for sched in scheds:
            if sched == "kv_major" and dtype == "f32":
                continue
            _log(f"arbitrary lists {name} {sched} {dtype}")
            prob = C.problem_for(inp, H, G, d, di, B, k, dtype, sched)
            out, lse = msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], idx, return_lse=True)
            err = C.check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, dtype)
            _log(f"  max |O - O_ref| = {err:.3g}")


def test_cross_layer_reuse():
    """Cross-layer index reuse (LongCat Sparse Attention page, Abstract,
    strategy (2)): one Index Branch pass selects the kept blocks, and the
    attention of two layers, each with its own q, k and v, runs on that one
    kept list.  The library's selection must be delta-valid against the
    oracle's; each layer's attention on the oracle's kept lists must match the
    oracle's attention of that layer on the same lists, on both prefill
    schedules."""
    lq, lkv, H, G, d, di, B, k = [900, 333], [1300, 333], 8, 2, 128, 64, 128, 4
    layer1 = W.random_case(71, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    layer2 = W.random_case(72, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    prob = C.problem_for(layer1, H, G, d, di, B, k, "bf16")
    scores = msa.index_score(prob, layer1["q_idx"], layer1["k_idx"])
    idx_gpu = msa.topk_select(prob, scores)
    lists, refs = [], {1: [], 2: []}
    q0 = kv0 = 0
    for a, b in zip(lq, lkv):
        sq, skv = slice(q0, q0 + a), slice(kv0, kv0 + b)
        r = O.msa_forward(layer1["q"][sq].cpu(), layer1["k"][skv].cpu(), layer1["v"][skv].cpu(),
                          layer1["q_idx"][sq].cpu(), layer1["k_idx"][skv].cpu(), a, b, B, k,
                          1.0 / math.sqrt(d))
        C.check_selection(idx_gpu[:, sq, :].cpu().numpy(), r["block_idx"], r["scores"],
                          r["pos"], B, k)
        lists.append(r["block_idx"])
        refs[1].append((r["out"], r["lse"]))
        refs[2].append(O.sparse_attention(layer2["q"][sq].cpu(), layer2["k"][skv].cpu(),
                                          layer2["v"][skv].cpu(), r["block_idx"], r["pos"], B,
                                          1.0 / math.sqrt(d)))
        q0, kv0 = q0 + a, kv0 + b
    kept = torch.from_numpy(np.concatenate(lists, axis=1)).to(DEV).contiguous()
    for sched in ("kv_major", "query_major"):
        p2 = prob.with_schedule(sched)
        for layer, inp in ((1, layer1), (2, layer2)):
            out, lse = msa.sparse_attn_fwd(p2, inp["q"], inp["k"], inp["v"], kept,
                                           return_lse=True)
            ref_o = np.concatenate([x[0] for x in refs[layer]])
            ref_l = np.concatenate([x[1] for x in refs[layer]])
            err = C.check_attention(out.float().cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l,
                                    "bf16")
            _log(f"cross-layer reuse, {sched}, layer {layer}: max |O - O_ref| = {err:.3g}")


def _passes_equal_single_pass(inp, H, G, d, di, B, k, sizes):
    """The KV-major forward with a workspace below its default size runs the
    query rows in (more) passes; every output equals that of the default
    workspace bit for bit (out, LSE and the block mass).  The default is one
    pass except on long prefills (prefill-128k: passes of 16,384 rows)."""
    prob = msa.Problem(inp["cu_q"], inp["cu_kv"], inp["len_q"], inp["len_kv"], H, G, d, di, B, k,
                       "bf16")
    bi = msa.topk_select(prob, msa.index_score(prob, inp["q_idx"], inp["k_idx"]))
    ref = msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], bi)
    full, least = msa.workspace_size(prob), msa.workspace_size_min(prob)
    assert 0 < least < full
    with pytest.raises(msa.MsaError) as e:
        ws = torch.empty(least - 1, dtype=torch.uint8, device=DEV)
        msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], bi, workspace=ws)
    assert e.value.status == 5
    for nbytes in sizes(least, full):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        got = msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], bi, workspace=ws)
        o2, l2 = msa.sparse_attn_fwd(prob, inp["q"], inp["k"], inp["v"], bi, return_lse=True,
                                     workspace=ws)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))
        assert torch.equal(o2.view(torch.int16), ref[0].view(torch.int16))
        assert torch.equal(l2.view(torch.int32), ref[1].view(torch.int32))
        _log(f"  workspace {nbytes} of {full} bytes: equal to the default workspace's outputs")
        del ws


@pytest.mark.parametrize("case", [SMALL[0], SMALL[1], SMALL[5]],
                         ids=[SMALL[0][0], SMALL[1][0], SMALL[5][0]])
def test_kv_major_passes_small(case):
    name, lq, lkv, H, G, d, di, B, k = case
    _log(f"passes {name}")
    inp = W.random_case(60 + SMALL.index(case), lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    _passes_equal_single_pass(inp, H, G, d, di, B, k,
                              lambda least, full: [least, (least + full) // 2, full - 1])


@pytest.mark.parametrize("name", ["chunked-prefill-1m", "prefill-128k"])
def test_kv_major_passes_full_size(name):
    """The long workloads with a bounded workspace: the 1M chunk in passes of
    the fewest rows (256) and of a quarter of its rows (its default is one
    pass); prefill-128k within 8 GiB (9 passes against the default 8)."""
    w = W.WORKLOADS[name]
    _log(f"passes {name}: generating")
    inp = W.make_inputs(w, device=DEV, seed=0)
    if name == "prefill-128k":
        sizes = lambda least, full: [8 << 30]  # noqa: E731
    else:
        sizes = lambda least, full: [least, full // 4 + 1]  # noqa: E731
    _passes_equal_single_pass(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                              w.block_size, w.top_k, sizes)
