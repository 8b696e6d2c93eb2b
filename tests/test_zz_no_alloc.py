"""The allocation-free decode entry point (dsa_forward_decode_noalloc) against dsa_forward_decode, through
the C ABI, on the GPU: two calls in a row on the shared device scratch, the second with a smaller input,
each compared with the workspace entry point on the same inputs (the same kernels run, so the selection,
output and log-sum-exp must agree bit for bit).  The second call leaves the selection in the scratch
(no idx_out), so that part of the scratch is exercised too."""
import math

import pytest
import torch

from sparse_attention_13_amd import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def dsa():
    from sparse_attention_13_amd import dsa as d
    d.lib()
    return d


def _both(dsa, B, S, seed, own_idx):
    x = synth.decode(B, S, seed=seed, device=DEV)
    k, sm = 2048, 1.0 / math.sqrt(576)
    args = (x["q8"], x["q_scale"], x["k8"], x["k_scale"], x["w"], x["q"], x["kv"])
    o_ref = torch.empty((B, 128, 512), dtype=torch.bfloat16, device=DEV)
    l_ref = torch.empty((B, 128), dtype=torch.float32, device=DEV)
    i_ref = torch.empty((B, k), dtype=torch.int32, device=DEV)
    dsa.forward(*args, k, 512, sm, decode=True, out=o_ref, lse=l_ref, idx_out=i_ref)
    o = torch.full_like(o_ref, float("nan"))
    lse = torch.full_like(l_ref, float("nan"))
    idx = torch.full_like(i_ref, -7) if own_idx else None
    dsa.forward_decode_noalloc(*args, k, 512, sm, out=o, lse=lse, idx_out=idx)
    torch.cuda.synchronize()
    return (i_ref, o_ref, l_ref), (idx, o, lse)


def test_noalloc_decode_matches_workspace_entry_point(dsa):
    assert dsa.lib().dsa_forward_decode_noalloc_max_bytes() == 128 << 20
    # the headline decode shape, then a smaller one on the same (shared) scratch
    for B, S, seed, own_idx in [(64, 131072, 3, True), (5, 40000, 4, False)]:
        print(f"[noalloc] B={B} S={S} seed={seed} idx_out={'caller' if own_idx else 'scratch'}", flush=True)
        ref, got = _both(dsa, B, S, seed, own_idx)
        pairs = [(r, g) for r, g in zip(ref, got) if g is not None]
        print("[noalloc]   identical: " + ", ".join(str(torch.equal(r, g)) for r, g in pairs), flush=True)
        assert len(pairs) == (3 if own_idx else 2)
        for r, g in pairs:
            assert torch.equal(r, g)
