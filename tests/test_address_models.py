"""CPU address models of the selection kernels (no GPU needed).

For every parity case and every full-size workload, these models walk the
global addresses that the fused index/Top-k kernels and the hierarchical
selection kernels form, exactly as the kernels derive them from the problem,
and check that each lands inside its buffer: the candidate workspace (whose
size the library itself reports through the C ABI), the index keys of the
sequence, and the workspace regions of the hierarchical pass.  They are the
host-side half of the bounds checking; the debug library checks the
data-dependent indices on the device (tests/test_gpu_debug_bounds.py).
"""
import ctypes
import os

import pytest

import block_sparse_long_msa_amd as msa

pytestmark = pytest.mark.skipif(not os.path.exists(msa.LIB_PATH),
                                reason="libmsa.so not built (run __graft_entry__.build())")

FAKE = 0x10000  # a 16-byte aligned non-null address; size queries never dereference it


def _prob(lq, lkv, G, DI, B, k):
    return msa.CProblem(num_seqs=len(lq), num_q_heads=G, num_kv_groups=G, head_dim=128,
                        idx_dim=DI, block_size=B, top_k=k, dtype=0, schedule=0,
                        max_q_len=max(lq), max_kv_len=max(lkv), total_q=sum(lq),
                        total_kv=sum(lkv), softmax_scale=0.088, cu_q=FAKE, cu_kv=FAKE)


def _ceil(a, b):
    return -(-a // b)


# ------------------------------------------------------- fused index + Top-k

def _list_len(k):
    """Candidates kept per (row, segment): the power of two >= k - 1, at least 4
    (no lists at all for k = 1)."""
    if k <= 1:
        return 0
    c = 4
    while c < k - 1:
        c *= 2
    return c


def fused_model(lq, lkv, G, B, k):
    """Largest candidate-key index written by the scoring kernel and read by
    the merge kernel, and the largest index-key row read, per the kernels'
    tiling: 512-query tiles, segments of 8 * max(4, L) blocks, L keys per
    (group, row, segment)."""
    tq = sum(lq)
    nb_max = _ceil(max(lkv), B)
    lst = _list_len(k)
    seg = 8 * max(4, lst)
    nseg = max(1, _ceil(nb_max, seg))
    QT = 512
    worst_write = worst_read = worst_key = -1
    kv0 = q0 = 0
    for a, L in zip(lq, lkv):
        base = L - a
        if k > 1 and nb_max > 1:
            for s_id in range(nseg):
                for t0 in range(0, a, QT):
                    nq = min(QT, a - t0)
                    p_last = base + t0 + nq - 1
                    if p_last < 0:
                        continue
                    js, je = s_id * seg, min(s_id * seg + seg, p_last // B)
                    if je <= js:
                        continue
                    assert je * B <= L, "index-key row past the sequence"
                    worst_key = max(worst_key, kv0 + je * B - 1)
                    for qn in range(nq):
                        pos = base + t0 + qn
                        if pos >= 0 and pos // B > js:
                            idx = (((G - 1) * tq + q0 + t0 + qn) * nseg + s_id) * lst + lst - 1
                            worst_write = max(worst_write, idx)
        for i in range(a):
            pos = base + i
            if pos < 0 or k == 1 or pos // B <= k - 1:
                continue
            ns = _ceil(pos // B, seg)
            assert ns <= nseg and ns * lst <= 64 * 16
            worst_read = max(worst_read, ((G - 1) * tq + q0 + i) * nseg * lst + ns * lst - 1)
        kv0 += L
        q0 += a
    return worst_write, worst_read, worst_key, nseg * lst


FUSED_CASES = [
    ("ragged-1000", [1000], [1000], 2, 64, 128, 4),
    ("varlen-chunked", [300, 1, 700, 0], [300, 513, 1500, 64], 4, 64, 64, 3),
    ("k8-b64", [777], [777], 1, 128, 64, 8),
    ("k1", [520], [600], 2, 64, 128, 1),
    ("k-covers-all", [640], [640], 1, 64, 64, 16),
    ("long-rows-k20", [700], [40000], 2, 64, 64, 20),
    ("long-rows-k8-b128", [1500], [90000], 2, 64, 128, 8),
    ("long-rows-k64", [300], [33000], 1, 64, 64, 64),
    ("more-keys-than-queries", [300, 400], [300, 500], 2, 64, 128, 4),
    ("decode", [1] * 7, [1, 127, 128, 129, 5000, 64, 3000], 2, 64, 128, 4),
    ("prefill-32k", [32768], [32768], 8, 64, 128, 16),
]
FULL_FUSED = [
    ("prefill-128k", [131072], [131072], 8, 64, 128, 32),
    ("chunked-prefill-1m", [8192], [1048576], 8, 64, 128, 64),
]


@pytest.mark.parametrize("name,lq,lkv,G,DI,B,k", FUSED_CASES + FULL_FUSED,
                         ids=[c[0] for c in FUSED_CASES + FULL_FUSED])
def test_fused_selection_addresses(name, lq, lkv, G, DI, B, k):
    lib = msa.load_library()
    n = ctypes.c_size_t(0)
    p = _prob(lq, lkv, G, DI, B, k)
    assert lib.msa_index_topk_workspace_size(ctypes.byref(p), ctypes.byref(n)) == 0
    keys = n.value // 8
    worst_write, worst_read, worst_key, per_row = fused_model(lq, lkv, G, B, k)
    assert keys == G * sum(lq) * per_row  # the library sizes the workspace as the model does
    assert worst_write < keys and worst_read < keys
    assert worst_key < sum(lkv)
    if k == 1:  # the merge reads nothing: only J is kept, and there is no workspace
        assert keys == 0 and worst_read == -1


# ---------------------------------------------------- hierarchical selection

def _hal256(x):
    return (x + 255) // 256 * 256


def hier_model(lq, lkv, G, DI, B, k, S, C):
    """Walks the coarse-key, coarse, fine and final kernels' addresses; returns
    the byte sizes of the key, slot and fine-score regions they address."""
    tq, tkv = sum(lq), sum(lkv)
    nb_max = _ceil(max(lkv), B)
    nch = max(1, _ceil(nb_max, S))
    K1, span = C + 1, B * S
    assert _ceil(nch, 64) <= 16 and _ceil(K1 * S, 64) <= 16
    kbar_n, sel_n = len(lq) * nch * G * DI, G * tq * K1
    fine_n = sel_n * S
    buckets = {}
    q0 = kv0 = 0
    for b, (a, L) in enumerate(zip(lq, lkv)):
        base = L - a
        for c in range(nch):  # coarse keys of full chunks only
            if (c + 1) * span <= L:
                assert kv0 + (c + 1) * span <= tkv
                assert (b * nch + c + 1) * G * DI <= kbar_n
        for i in range(a):
            p = base + i
            if p < 0 or p // B <= k - 1:
                continue
            J = p // B
            cJ = J // S
            assert cJ < nch
            for c in range(cJ):  # coarse candidates: full chunks below the current one
                assert ((b * nch + c) * G + G) * DI <= kbar_n and (c + 1) * span <= L
            slots = list(range(min(cJ, C))) + ([cJ] if cJ * S < J else [])
            for c in slots:
                assert c * span <= p
                buckets.setdefault((b, c), []).append((q0 + i, J))
        q0 += a
        kv0 += L
    for (b, c), ents in buckets.items():  # fine work items of 256 entries
        for s0 in range(0, len(ents), 256):
            item = ents[s0:s0 + 256]
            nblk = min(S, max(J for _, J in item) - c * S)
            assert nblk >= 1
            assert (c * S + nblk) * B <= lkv[b], "fine scoring past the sequence's keys"
            for row, _ in item:
                assert ((G - 1) * tq + row + 1) * K1 * S <= fine_n
    return [4 * kbar_n, 4 * sel_n, 4 * fine_n]


HIER_CASES = [
    ("b128-s4-keep3", [1500], [6000], 2, 64, 128, 4, 4, 3),
    ("b64-s8-keep2-varlen", [700, 1, 300], [9000, 513, 300], 2, 32, 64, 6, 8, 2),
    ("b64-s2-keep6-k12", [800], [12000], 1, 128, 64, 12, 2, 6),
    ("decode", [1] * 5, [9000, 127, 70000, 3000, 40000], 2, 64, 128, 8, 8, 2),
    ("prefill-32k", [32768], [32768], 8, 64, 128, 16, 16, 2),
]
FULL_HIER = [
    ("prefill-128k", [131072], [131072], 8, 64, 128, 32, 16, 4),
    ("chunked-prefill-1m", [8192], [1048576], 8, 64, 128, 64, 16, 8),
]


@pytest.mark.parametrize("name,lq,lkv,G,DI,B,k,S,C", HIER_CASES + FULL_HIER,
                         ids=[c[0] for c in HIER_CASES + FULL_HIER])
@pytest.mark.parametrize("all_chunks", [False, True])
def test_hierarchical_selection_addresses(name, lq, lkv, G, DI, B, k, S, C, all_chunks):
    if all_chunks:  # keeping every chunk: the coarse pass selects nothing away
        if name in ("prefill-128k", "chunked-prefill-1m"):
            pytest.skip("keeping every chunk at full size exceeds the fine-score limit")
        C = max(C, _ceil(_ceil(max(lkv), B), S))
    lib = msa.load_library()
    n = ctypes.c_size_t(0)
    p = _prob(lq, lkv, G, DI, B, k)
    assert lib.msa_index_topk_hier_workspace_size(ctypes.byref(p), S, C, ctypes.byref(n)) == 0
    regions = hier_model(lq, lkv, G, DI, B, k, S, C)
    assert sum(_hal256(r) for r in regions) <= n.value
