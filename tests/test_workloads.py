"""The seeded input generator follows its stated recipe (CPU only).

workloads.py draws every tensor N(0, 1) from its own seeded generator and,
for planted workloads, adds 2 u_g to the index keys of 5% of the key blocks
and u_g to the index queries of 20% of the queries of every group.  These
tests rebuild the unplanted draws and check that exactly that structure was
added, and that the named workloads have the shapes of the long-context
configurations they stand for.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W


def _tiny_planted(**kw):
    base = W.Workload("planted-test", 4, 2, 16, 8, 8, 4, "f32", True,
                      len_q=(120, 0, 37), len_kv=(400, 64, 37), num_seqs=3)
    return dataclasses.replace(base, **kw)


def test_plant_adds_exactly_the_stated_offsets():
    w = _tiny_planted()
    inp = W.make_inputs(w, seed=3)
    G, di, B = w.num_kv_groups, w.idx_dim, w.block_size
    tq, tkv = sum(w.len_q), sum(w.len_kv)
    base_q = W._randn((tq, G, di), W._seed(3, w.name, 4), torch.device("cpu"))
    base_k = W._randn((tkv, G, di), W._seed(3, w.name, 5), torch.device("cpu"))
    dq = (inp["q_idx"] - base_q).numpy()
    dk = (inp["k_idx"] - base_k).numpy()
    cu_q, cu_kv = inp["cu_q"].tolist(), inp["cu_kv"].tolist()
    for si, (a, b) in enumerate(zip(w.len_q, w.len_kv)):
        nb = -(-b // B)
        for g in range(G):
            blocks = inp["planted_blocks"][si][g]
            queries = inp["planted_q"][si][g]
            assert len(blocks) == int(round(0.05 * nb)) and blocks == sorted(set(blocks))
            assert len(queries) == int(round(0.2 * a)) and queries == sorted(set(queries))
            assert all(0 <= j < nb for j in blocks) and all(0 <= t < a for t in queries)
            u = None
            for t in range(a):
                row = dq[cu_q[si] + t, g]
                if t in queries:
                    u = row if u is None else u
                    np.testing.assert_allclose(row, u, rtol=0, atol=1e-6)
                else:
                    assert np.all(row == 0)
            for s in range(b):
                row = dk[cu_kv[si] + s, g]
                if s // B in blocks:
                    if u is None:  # no planted query in this sequence: take u from the keys
                        u = row / 2
                    np.testing.assert_allclose(row, 2 * u, rtol=0, atol=1e-6)
                else:
                    assert np.all(row == 0)
    # attention tensors are plain draws, never planted
    base_v = W._randn((tkv, G, w.head_dim), W._seed(3, w.name, 3), torch.device("cpu"))
    assert torch.equal(inp["v"], base_v)


def test_draws_are_seeded_and_distinct():
    w = _tiny_planted()
    a, b, c = W.make_inputs(w, seed=0), W.make_inputs(w, seed=0), W.make_inputs(w, seed=1)
    for name in ("q", "k", "v", "q_idx", "k_idx"):
        assert torch.equal(a[name], b[name])
        assert not torch.equal(a[name], c[name])
    assert not torch.equal(a["k"], a["v"])  # every tensor has its own generator


def test_bf16_is_a_round_to_nearest_even_cast_of_the_fp32_draw():
    w = _tiny_planted(dtype="bf16", planted=False)
    inp = W.make_inputs(w, seed=5)
    base = W._randn((sum(w.len_q), w.num_q_heads, w.head_dim), W._seed(5, w.name, 1),
                    torch.device("cpu"))
    assert inp["q"].dtype == torch.bfloat16
    x = base.numpy().view(np.uint32).astype(np.uint64)
    rne = ((x + 0x7FFF + ((x >> 16) & 1)) >> 16).astype(np.uint16)  # round half to even
    assert np.array_equal(inp["q"].view(torch.int16).numpy().view(np.uint16), rne)


def test_decode_lengths_are_drawn_in_range():
    w = W.WORKLOADS["decode-64x256k"]
    lq, lkv = W.seq_lengths(w, seed=0)
    assert lq == [1] * 64 and len(lkv) == 64
    assert all(65536 <= x <= 262144 for x in lkv)
    assert len(set(lkv)) > 60
    assert W.seq_lengths(w, seed=0) == (lq, lkv)


@pytest.mark.parametrize("name,H,G,d,di,B,k,lq,lkv", [
    ("tiny-fp32", 4, 1, 64, 32, 64, 4, 1024, 1024),
    ("prefill-32k", 32, 8, 128, 64, 128, 16, 32768, 32768),
    ("prefill-128k", 64, 8, 128, 64, 128, 32, 131072, 131072),
    ("chunked-prefill-1m", 64, 8, 128, 64, 128, 64, 8192, 1048576),
])
def test_named_workload_shapes(name, H, G, d, di, B, k, lq, lkv):
    w = W.WORKLOADS[name]
    assert (w.num_q_heads, w.num_kv_groups, w.head_dim, w.idx_dim, w.block_size, w.top_k) == \
        (H, G, d, di, B, k)
    assert W.seq_lengths(w) == ([lq], [lkv])
    assert w.dtype == ("f32" if name == "tiny-fp32" else "bf16")
    assert w.planted == (name != "tiny-fp32")
