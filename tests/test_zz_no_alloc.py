"""GPU check of msa_sparse_attn_fwd_noalloc (the attention call on the
library's fixed device scratch, for callers that cannot allocate): through
the C ABI, its outputs must equal those of msa_sparse_attn_fwd (same kernels,
its own workspace) bit for bit, on two calls in a row with the second one
smaller, for the decode (split-KV) path and the KV-major prefill path."""
import sys

import pytest
import torch

import block_sparse_long_msa_amd as msa
import workloads as W
from tests import msa_check as C

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(seed, lq, lkv, H, G, d, di, B, k):
    inp = W.random_case(seed, lq, lkv, H, G, d, di, B, k, "bf16", device=DEV)
    prob = C.problem_for(inp, H, G, d, di, B, k, "bf16")
    scores = msa.index_score(prob, inp["q_idx"], inp["k_idx"])
    idx = msa.topk_select(prob, scores)
    return inp, prob, idx


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_noalloc_matches_workspace_call(kind):
    if kind == "decode":
        big = (91, [1] * 40, [1 + 223 * i for i in range(40)], 16, 4, 128, 64, 128, 32)
        small = (92, [1] * 9, [7000, 1, 129, 300, 4096, 65, 2, 900, 128], 16, 4, 128, 64, 128, 32)
    else:
        big = (93, [1000, 37], [1000, 300], 8, 2, 128, 64, 128, 6)
        small = (94, [300], [700], 8, 2, 128, 64, 128, 6)
    cases = [_case(*c) for c in (big, small)]
    for (inp, prob, idx), name in zip(cases, ("first", "second (smaller)")):
        need = msa.workspace_size(prob)
        assert 0 < need <= 64 << 20, need
        _log(f"{kind}, {name} call: workspace {need} bytes")
    # two no-allocation calls in a row, the second smaller, then the reference calls
    got = [msa.sparse_attn_fwd_noalloc(p, i["q"], i["k"], i["v"], x, return_lse=True)
           for i, p, x in cases]
    ref = [msa.sparse_attn_fwd(p, i["q"], i["k"], i["v"], x, return_lse=True)
           for i, p, x in cases]
    torch.cuda.synchronize()
    for (o, l), (ro, rl) in zip(got, ref):
        assert torch.equal(o, ro)
        assert torch.equal(l, rl)
    # and once more in the other order: the scratch keeps the last call's contents
    got2 = [msa.sparse_attn_fwd_noalloc(p, i["q"], i["k"], i["v"], x, return_lse=True)
            for i, p, x in reversed(cases)]
    torch.cuda.synchronize()
    for (o, l), (ro, rl) in zip(got2, reversed(ref)):
        assert torch.equal(o, ro)
        assert torch.equal(l, rl)
    _log(f"{kind}: no-allocation outputs equal the workspace call's bit for bit")


def test_noalloc_rejects_a_problem_beyond_its_scratch():
    """A problem needing more than the 64 MiB scratch is rejected before any
    launch, with the output untouched."""
    lq = 20000
    inp, prob, idx = _case(95, [lq], [lq], 8, 2, 128, 64, 128, 16)
    assert msa.workspace_size(prob) > 64 << 20
    out = torch.full((lq, 8, 128), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(msa.MsaError) as e:
        msa.sparse_attn_fwd_noalloc(prob, inp["q"], inp["k"], inp["v"], idx, out=out)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
