"""The debug library (libmsa_debug.so, built with -DMSA_DEBUG) on the GPU.

Its kernels count, on the device, the gather index checks they run and
those that fail (bucket entries, work-item descriptors, candidate and chunk
lists, kept-block lists).  Every entry point runs here through the debug
library on ragged, varlen, decode and full-size prefill problems: checks
must have run, none may fail, and every output must equal the release
library's bit for bit (the checks read, they never change what is
computed).
"""
import sys

import pytest
import torch

import block_sparse_long_msa_amd as msa
import workloads as W

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not __import__("os").path.exists(msa.DEBUG_LIB_PATH),
                                 reason="libmsa_debug.so not built")]
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_all(inp, H, G, d, di, B, k, dtype, hier=None):
    """Every entry point on one problem; returns the outputs in a fixed order."""
    lq, lkv = inp["len_q"], inp["len_kv"]
    outs = []
    prob = msa.Problem(inp["cu_q"], inp["cu_kv"], lq, lkv, H, G, d, di, B, k, dtype)
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    bi = msa.topk_select(prob, scores)
    outs += [scores, bi]
    scheds = ("query_major", "kv_major") if dtype == "bf16" and max(lq) > 1 else ("auto",)
    for sc in scheds:
        o, lse = msa.sparse_attn_fwd(prob.with_schedule(sc), inp["q"], inp["k"], inp["v"], bi,
                                     return_lse=True)
        outs += [o, lse]
    if dtype == "bf16":
        outs.append(msa.index_topk(prob, inp["q_idx"], inp["k_idx"]))
        if hier is not None:
            outs += list(msa.index_topk_hier(prob, inp["q_idx"], inp["k_idx"], hier[0], hier[1],
                                             return_kept=True))
    if dtype == "bf16" and max(lq) > 1:
        o, lse, mass = msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], bi)
        kl, grad = msa.indexer_kl(prob, scores, bi, mass)
        outs += [o, lse, mass, kl, grad]
        outs += list(msa.indexer_bwd(prob, inp["q_idx"], inp["k_idx"], bi, grad))
        dout = W.random_out_grad(3, prob.total_q, H, d, dtype, device=DEV)
        outs += list(msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], bi, o, lse, dout))
    torch.cuda.synchronize()
    return outs


def _compare(rel, dbg):
    assert len(rel) == len(dbg)
    for i, (a, b) in enumerate(zip(rel, dbg)):
        assert a.shape == b.shape and a.dtype == b.dtype, i
        if a.is_floating_point():
            # NaN-aware bitwise equality (rows without keys hold -inf LSEs)
            assert torch.equal(a.view(torch.int32 if a.element_size() == 4 else torch.int16),
                               b.view(torch.int32 if b.element_size() == 4 else torch.int16)), i
        else:
            assert torch.equal(a, b), i


CASES = [
    # name, len_q, len_kv, H, G, d, d_idx, B, k, dtype, (chunk_blocks, keep_chunks)
    ("ragged-1000", [1000], [1000], 8, 2, 128, 64, 128, 4, "bf16", (2, 2)),
    ("varlen-chunked", [300, 1, 700, 0], [300, 513, 1500, 64], 4, 4, 64, 32, 64, 3, "bf16",
     (4, 2)),
    ("hpg16-dsi128", [777], [777], 16, 1, 128, 128, 64, 8, "bf16", (2, 4)),
    ("k1", [520], [600], 4, 2, 64, 64, 128, 1, "bf16", None),
    ("long-rows", [1500], [24000], 16, 2, 128, 64, 128, 8, "bf16", (8, 3)),
    ("decode", [1] * 7, [1, 127, 128, 129, 5000, 64, 3000], 8, 2, 128, 64, 128, 4, "bf16",
     (8, 2)),
    ("f32-varlen", [300, 1, 700], [300, 513, 1500], 4, 2, 64, 32, 64, 3, "f32", None),
]


@pytest.fixture
def debug_then_release():
    """Runs the test body's calls through the debug library, then restores the
    library that was in use."""
    prev = msa.current_library_path() or msa.LIB_PATH
    yield
    msa.select_library(prev)


def _both(inp, *args, **kw):
    msa.select_library(msa.LIB_PATH)
    rel = _run_all(inp, *args, **kw)
    msa.select_library(msa.DEBUG_LIB_PATH)
    msa.debug_bounds_violations(reset=True)  # clear whatever an earlier call left
    dbg = _run_all(inp, *args, **kw)
    bad, ran = msa.debug_bounds_violations(reset=True)
    _log(f"  {ran} lane checks, {bad} failed")
    assert ran > 0  # the checks ran
    return rel, dbg, bad


def test_release_library_has_no_counters(debug_then_release):
    msa.select_library(msa.LIB_PATH)
    with pytest.raises(msa.MsaError) as e:
        msa.debug_bounds_violations()
    assert e.value.status == 7


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_debug_build_counts_no_violation(case, debug_then_release):
    name, lq, lkv, H, G, d, di, B, k, dtype, hier = case
    _log(f"debug bounds {name}")
    inp = W.random_case(CASES.index(case), lq, lkv, H, G, d, di, B, k, dtype, device=DEV)
    rel, dbg, n = _both(inp, H, G, d, di, B, k, dtype, hier=hier)
    assert n == 0, f"{n} failed bounds checks"
    _compare(rel, dbg)


def test_debug_build_prefill_32k(debug_then_release):
    """The prefill-32k workload at full size (planted index keys), every entry point."""
    w = W.WORKLOADS["prefill-32k"]
    _log("debug bounds prefill-32k")
    inp = W.make_inputs(w, device=DEV, seed=0)
    rel, dbg, n = _both(inp, w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim,
                        w.block_size, w.top_k, w.dtype, hier=(16, 2))
    assert n == 0, f"{n} failed bounds checks"
    _compare(rel, dbg)


@pytest.mark.parametrize("case", [CASES[0], CASES[1], CASES[4]],
                         ids=[CASES[0][0], CASES[1][0], CASES[4][0]])
def test_debug_build_kv_major_passes(case, debug_then_release):
    """The KV-major forward and the backward in passes of 256 rows (the
    least workspaces)."""
    name, lq, lkv, H, G, d, di, B, k, dtype, _ = case
    _log(f"debug bounds, passes: {name}")
    inp = W.random_case(CASES.index(case), lq, lkv, H, G, d, di, B, k, dtype, device=DEV)

    def run():
        prob = msa.Problem(inp["cu_q"], inp["cu_kv"], lq, lkv, H, G, d, di, B, k, dtype)
        bi = msa.topk_select(prob, msa.index_score(prob, inp["q_idx"], inp["k_idx"]))
        ws = torch.empty(msa.workspace_size_min(prob), dtype=torch.uint8, device=DEV)
        outs = list(msa.sparse_attn_fwd_mass(prob, inp["q"], inp["k"], inp["v"], bi, workspace=ws))
        dout = W.random_out_grad(4, prob.total_q, H, d, dtype, device=DEV)
        bws = torch.empty(msa.sparse_attn_bwd_workspace_size(prob, minimum=True),
                          dtype=torch.uint8, device=DEV)
        outs += list(msa.sparse_attn_bwd(prob, inp["q"], inp["k"], inp["v"], bi, outs[0], outs[1],
                                         dout, workspace=bws))
        torch.cuda.synchronize()
        return outs

    msa.select_library(msa.LIB_PATH)
    rel = run()
    msa.select_library(msa.DEBUG_LIB_PATH)
    msa.debug_bounds_violations(reset=True)
    dbg = run()
    bad, ran = msa.debug_bounds_violations(reset=True)
    _log(f"  {ran} lane checks, {bad} failed")
    assert ran > 0 and bad == 0
    _compare(rel, dbg)
