"""Seeded synthetic workloads for the MSA block-sparse attention path.

This module builds INPUTS only: the attention tensors Q, K, V, the index
tensors q_idx / k_idx and the packed-sequence offsets.  It holds none of the
method's arithmetic, so both sides of every parity check (the HIP library and
the CPU oracle) can take their inputs from here without sharing code.

Shapes follow the long-context setting of the "MiniMax Sparse Attention"
page (section Key points, "Benchmark configuration": key/value blocks of 128
tokens, head dimension 128, GQA with several query heads per key/value
head).  The pages measure on a trained model and on evaluation suites that
are not available here; these seeded tensors stand in for them.

Value recipe (all workloads):
  * every tensor is drawn i.i.d. N(0, 1) in fp32 from its own seeded torch
    generator, then cast to bf16 with round-to-nearest-even (the tiny fp32
    workload stays fp32);
  * planted workloads add structure to the index tensors before the cast:
    for each KV group g a direction u_g ~ N(0, I) is drawn; 5% of the key
    blocks (distinct, uniform) get 2*u_g added to k_idx of every key in the
    block, and 20% of the queries (distinct, uniform) get u_g added to their
    q_idx.  Planted queries therefore score planted blocks far above the
    rest, which gives the selection a realistic skew in block popularity.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    num_q_heads: int        # H
    num_kv_groups: int      # G (GQA key/value heads)
    head_dim: int           # d
    idx_dim: int            # d_idx of the index branch
    block_size: int         # B
    top_k: int              # k, counting the always-kept current block
    dtype: str              # "f32" or "bf16"
    planted: bool
    len_q: Tuple[int, ...] = ()      # per sequence; empty -> one query per sequence
    len_kv: Tuple[int, ...] = ()     # per sequence; empty -> drawn (decode)
    num_seqs: int = 1
    kv_len_range: Tuple[int, int] = (0, 0)   # inclusive range for drawn KV lengths

    @property
    def hpg(self) -> int:
        return self.num_q_heads // self.num_kv_groups


WORKLOADS: Dict[str, Workload] = {
    # Small enough for the oracle to check every output in seconds.
    "tiny-fp32": Workload("tiny-fp32", 4, 1, 64, 32, 64, 4, "f32", False,
                          len_q=(1024,), len_kv=(1024,)),
    # Full causal prefill, 32K tokens.
    "prefill-32k": Workload("prefill-32k", 32, 8, 128, 64, 128, 16, "bf16", True,
                            len_q=(32768,), len_kv=(32768,)),
    # Full causal prefill, 128K tokens.
    "prefill-128k": Workload("prefill-128k", 64, 8, 128, 64, 128, 32, "bf16", True,
                             len_q=(131072,), len_kv=(131072,)),
    # Batched decode: 64 sequences, one new token each, KV lengths 64K..256K.
    "decode-64x256k": Workload("decode-64x256k", 64, 8, 128, 64, 128, 32, "bf16", False,
                               num_seqs=64, kv_len_range=(65536, 262144)),
    # Last 8192-token chunk of a 1M-token prefill.
    "chunked-prefill-1m": Workload("chunked-prefill-1m", 64, 8, 128, 64, 128, 64, "bf16", True,
                                   len_q=(8192,), len_kv=(1048576,)),
}


def _seed(seed: int, name: str, tensor_id: int) -> int:
    """Deterministic 63-bit seed per (run seed, workload, tensor)."""
    tag = sum((i + 1) * ord(c) for i, c in enumerate(name))
    ss = np.random.SeedSequence([seed, tag, tensor_id])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def seq_lengths(w: Workload, seed: int = 0) -> Tuple[List[int], List[int]]:
    """Per-sequence query and key/value lengths (queries are the last len_q tokens)."""
    if w.len_kv:
        lq = list(w.len_q) if w.len_q else [1] * len(w.len_kv)
        return lq, list(w.len_kv)
    g = torch.Generator(device="cpu").manual_seed(_seed(seed, w.name, 7))
    lo, hi = w.kv_len_range
    lkv = torch.randint(lo, hi + 1, (w.num_seqs,), generator=g).tolist()
    return [1] * w.num_seqs, lkv


def _randn(shape, seed: int, device, chunk_rows: int = 1 << 20) -> torch.Tensor:
    """fp32 N(0,1) draw; large tensors are drawn in row chunks of one generator."""
    g = torch.Generator(device=device).manual_seed(seed)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g,
                                 device=device, dtype=torch.float32)
    return out


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x if dtype == "f32" else x.to(torch.bfloat16)


def make_inputs(w: Workload, device="cpu", seed: int = 0,
                with_attention: bool = True) -> Dict[str, object]:
    """Build one workload's inputs on `device`.

    Returns a dict with
      q [Tq, H, d], k [Tkv, G, d], v [Tkv, G, d]        (omitted if not with_attention)
      q_idx [Tq, G, d_idx], k_idx [Tkv, G, d_idx]
      cu_q, cu_kv: int64 [num_seqs + 1] packed row offsets (on `device`)
      len_q, len_kv: python lists
      planted_q, planted_blocks: per sequence, per group, sorted index lists
                                 (empty when the workload is not planted)
    Rows of all sequences are packed back to back; the queries of a sequence
    are its last len_q tokens.
    """
    device = torch.device(device)
    lq, lkv = seq_lengths(w, seed)
    tq, tkv = sum(lq), sum(lkv)
    G, H = w.num_kv_groups, w.num_q_heads
    out: Dict[str, object] = {"len_q": lq, "len_kv": lkv}
    cu_q = [0]
    cu_kv = [0]
    for a, b in zip(lq, lkv):
        cu_q.append(cu_q[-1] + a)
        cu_kv.append(cu_kv[-1] + b)
    out["cu_q"] = torch.tensor(cu_q, dtype=torch.int64, device=device)
    out["cu_kv"] = torch.tensor(cu_kv, dtype=torch.int64, device=device)

    q_idx = _randn((tq, G, w.idx_dim), _seed(seed, w.name, 4), device)
    k_idx = _randn((tkv, G, w.idx_dim), _seed(seed, w.name, 5), device)
    planted_q: List[List[List[int]]] = []
    planted_b: List[List[List[int]]] = []
    if w.planted:
        gp = torch.Generator(device="cpu").manual_seed(_seed(seed, w.name, 6))
        for si, (a, b) in enumerate(zip(lq, lkv)):
            nb = -(-b // w.block_size)
            n_blk = int(round(0.05 * nb))
            n_q = int(round(0.2 * a))
            pq, pb = [], []
            for g in range(G):
                u = torch.randn((w.idx_dim,), generator=gp, dtype=torch.float32)
                blocks = torch.randperm(nb, generator=gp)[:n_blk].sort().values
                queries = torch.randperm(a, generator=gp)[:n_q].sort().values
                u_dev = u.to(device)
                for j in blocks.tolist():
                    s0 = cu_kv[si] + j * w.block_size
                    s1 = min(cu_kv[si] + b, s0 + w.block_size)
                    k_idx[s0:s1, g, :] += 2.0 * u_dev
                rows = (queries + cu_q[si]).to(device)
                q_idx[rows, g, :] += u_dev
                pq.append(queries.tolist())
                pb.append(blocks.tolist())
            planted_q.append(pq)
            planted_b.append(pb)
    out["planted_q"] = planted_q
    out["planted_blocks"] = planted_b
    out["q_idx"] = _cast(q_idx, w.dtype)
    del q_idx
    out["k_idx"] = _cast(k_idx, w.dtype)
    del k_idx
    if with_attention:
        for name, tid, rows, heads, dim in (("q", 1, tq, H, w.head_dim),
                                            ("k", 2, tkv, G, w.head_dim),
                                            ("v", 3, tkv, G, w.head_dim)):
            out[name] = _cast(_randn((rows, heads, dim), _seed(seed, w.name, tid), device), w.dtype)
    return out


def random_case(seed: int, len_q: Sequence[int], len_kv: Sequence[int], H: int, G: int,
                d: int, d_idx: int, block_size: int, top_k: int, dtype: str = "f32",
                device="cpu") -> Dict[str, object]:
    """Small ad-hoc case (for edge-case tests): i.i.d. N(0,1), no plant."""
    w = Workload(f"case-{seed}", H, G, d, d_idx, block_size, top_k, dtype, False,
                 len_q=tuple(len_q), len_kv=tuple(len_kv))
    return make_inputs(w, device=device, seed=seed)


def random_scores(seed: int, G: int, total_q: int, nb: int, levels: int = 0,
                  device="cpu") -> torch.Tensor:
    """Synthetic fp32 block-score rows [G, total_q, nb] for checking selection alone.

    levels > 0 draws integers in [-levels, levels] (many exact ties);
    levels == 0 draws N(0, 1).  A few rows are made constant (all tied)."""
    g = torch.Generator(device="cpu").manual_seed(_seed(seed, "scores", nb))
    if levels > 0:
        s = torch.randint(-levels, levels + 1, (G, total_q, nb), generator=g).to(torch.float32)
    else:
        s = torch.randn((G, total_q, nb), generator=g, dtype=torch.float32)
    s[:, ::17, :] = 1.0
    return s.to(device)


def random_block_lists(seed: int, len_q: Sequence[int], len_kv: Sequence[int], G: int,
                       block_size: int, top_k: int) -> torch.Tensor:
    """Seeded kept-block lists [G, total_q, top_k] int32 that satisfy the
    attention call's contract without coming from a selection: per (group,
    row), a random number (0..top_k) of distinct blocks from 0..J (the
    current block J is included or not at random), in random slot order, the
    other slots -1.  Rows at negative positions get empty lists."""
    rng = np.random.default_rng(_seed(seed, "block-lists", top_k))
    rows = []
    for lq, lkv in zip(len_q, len_kv):
        for i in range(lq):
            p = lkv - lq + i
            rows.append(-1 if p < 0 else p // block_size)
    out = np.full((G, len(rows), top_k), -1, dtype=np.int32)
    for g in range(G):
        for r, J in enumerate(rows):
            if J < 0:
                continue
            n = int(rng.integers(0, min(top_k, J + 1) + 1))
            picks = rng.choice(J + 1, size=n, replace=False)
            slots = rng.choice(top_k, size=n, replace=False)
            out[g, r, slots] = picks
    return torch.from_numpy(out)


def random_slot_grads(seed: int, G: int, total_q: int, top_k: int) -> torch.Tensor:
    """Seeded fp32 N(0, 1) gradients for every kept slot [G, total_q, top_k]:
    the input of the Index Branch backward when it is checked on its own."""
    g = torch.Generator(device="cpu").manual_seed(_seed(seed, "slot-grads", top_k))
    return torch.randn((G, total_q, top_k), generator=g, dtype=torch.float32)


def small_int_tensor(seed: int, shape, bound: int, dtype: str = "bf16") -> torch.Tensor:
    """Seeded integers drawn uniformly from [-bound, bound] (CPU), in the
    given dtype: every product and every partial sum of a short dot product
    of such vectors is exact in fp32, and exact ties are frequent."""
    g = torch.Generator(device="cpu").manual_seed(_seed(seed, "small-int", bound))
    x = torch.randint(-bound, bound + 1, tuple(shape), generator=g).to(torch.float32)
    return _cast(x, dtype).contiguous()


def random_out_grad(seed: int, total_q: int, H: int, d: int, dtype: str = "bf16",
                    device="cpu") -> torch.Tensor:
    """Seeded N(0, 1) upstream gradient of the attention output [total_q, H, d],
    drawn in fp32 and cast to the problem's dtype (round to nearest even):
    the input of the Main Branch backward when it is checked on its own."""
    g = _seed(seed, "out-grad", H * 1000 + d)
    return _cast(_randn((total_q, H, d), g, device), dtype).contiguous()
