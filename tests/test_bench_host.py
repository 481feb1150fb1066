"""Host-side logic of bench.py (CPU only): the algorithmic work the roofline
divides by, checked against brute-force counts on small problems, and the
one-GPU guard."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _w(H=8, G=2, d=64, di=32, B=16, k=3):
    return SimpleNamespace(num_kv_groups=G, num_q_heads=H, head_dim=d, idx_dim=di,
                           block_size=B, top_k=k)


def test_algorithmic_work_matches_brute_force_counts():
    """Index FLOPs count every causal key of every query; attention FLOPs
    count the keys of min(k - 1, J) full earlier blocks plus the current
    block's causal keys (the selection keeps k - 1 earlier blocks when J
    allows it)."""
    w = _w()
    len_q, len_kv = [5, 40, 1, 0], [70, 40, 33, 16]
    f_idx, f_attn, _ = bench.algorithmic_work(w, len_q, len_kv)
    causal = kept = 0
    for lq, lkv in zip(len_q, len_kv):
        for p in range(lkv - lq, lkv):
            causal += p + 1
            J = p // w.block_size
            kept += min(w.top_k - 1, J) * w.block_size + (p - J * w.block_size + 1)
    assert f_idx == 2.0 * w.num_kv_groups * w.idx_dim * causal
    assert f_attn == 4.0 * w.num_q_heads * w.head_dim * kept


def test_partial_work_counts_entries_below_the_current_block():
    """The KV-major partial kernel's entries are the kept slots strictly
    below the row's current block; the diagonal FLOPs cover each row's
    causal keys of its current block."""
    w = _w(k=4)
    len_q, len_kv = [20, 7], [50, 30]
    rng = np.random.default_rng(0)
    tq = sum(len_q)
    bi = rng.integers(-1, 5, size=(w.num_kv_groups, tq, w.top_k)).astype(np.int32)
    f_diag, _, n_entries = bench.kvmajor_partial_work(w, len_q, len_kv, torch.from_numpy(bi))
    want_entries = 0
    want_diag = 0
    row = 0
    for lq, lkv in zip(len_q, len_kv):
        for p in range(lkv - lq, lkv):
            J = p // w.block_size
            want_diag += p % w.block_size + 1
            for g in range(w.num_kv_groups):
                want_entries += sum(1 for j in bi[g, row] if 0 <= j < J)
            row += 1
    assert n_entries == want_entries
    assert f_diag == 4.0 * w.num_q_heads * w.head_dim * want_diag


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
