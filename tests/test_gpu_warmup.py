"""Indexer warm-up loss (target from the main attention, KL, gradients through the indexer) vs the CPU oracle,
through the C ABI, on the GPU.

The indexer inputs are exact-integer e4m3 codes with power-of-two scales and weights: every index score is
then exact on both sides (whatever the summation order) and so is every ReLU decision of the backward pass,
and the comparison measures the target, the loss and the gradient arithmetic alone.  The main attention's
log-sum-exp comes from the attention kernel run over the full causal selection, as the dense forward pass of
the warm-up stage would produce it.
"""
import math

import numpy as np
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


def f32(orc, t):
    return orc.bf16_to_f32(synth.bf16_bits(t))


def exact_indexer_inputs(B, L, n_q, seed):
    """e4m3 codes of small integers (q: 4x{-4..4} at scale 1/4, k: {-4..4}/2 at scale 2) and weights that are
    integers times 2^-10: exact products and sums on both sides, scores of moderate size."""
    g = torch.Generator().manual_seed(seed)
    qi = torch.randint(-4, 5, (B, n_q, 64, 128), generator=g).float()
    ki = torch.randint(-4, 5, (B, L, 128), generator=g).float()
    wi = torch.randint(-3, 4, (B, n_q, 64), generator=g).float() / 1024.0
    return dict(q8=(qi * 4).to(torch.float8_e4m3fn).view(torch.uint8), qs=torch.full((B, n_q, 64), 0.25),
                k8=(ki / 2).to(torch.float8_e4m3fn).view(torch.uint8), ks=torch.full((B, L), 2.0), w=wi)


def dense_idx(L, n_q):
    pos = torch.arange(L - n_q, L)[:, None]
    s = torch.arange(L)[None, :]
    return torch.where(s <= pos, s, torch.full_like(s, -1)).to(torch.int32)


@pytest.mark.parametrize("B,L,n_q", [(2, 256, 256), (1, 333, 100)])
def test_warmup_loss_vs_oracle(orc, dsa, B, L, n_q):
    xi = exact_indexer_inputs(B, L, n_q, seed=L)
    xs = [synth.prefill(L, seed=10 + b, device=DEV, n_q=n_q) for b in range(B)]
    q = torch.stack([x["q"] for x in xs]).contiguous()
    kv = torch.stack([x["kv"] for x in xs]).contiguous()
    sm = 1.0 / math.sqrt(576)
    idx = dense_idx(L, n_q)[None].expand(B, n_q, L).contiguous().to(DEV)
    _, lse = dsa.sparse_mla_attn(q, kv, idx, 512, sm)
    scores = torch.full((B, n_q, L + 5), float("nan"), device=DEV)
    dsa.indexer_scores(xi["q8"].to(DEV), xi["qs"].to(DEV), xi["k8"].to(DEV), xi["ks"].to(DEV), xi["w"].to(DEV), scores)
    loss, target = dsa.warmup_loss(q, kv, lse, scores, sm)
    torch.cuda.synchronize()
    pos = np.arange(L - n_q, L, dtype=np.int64)
    gs, gt, gl = scores.cpu().numpy(), target.cpu().numpy(), loss.cpu().numpy()
    for b in range(B):
        p_o = orc.warmup_target(f32(orc, q[b]), f32(orc, kv[b]), pos, sm, ld=L + 5)
        i_o = orc.indexer(orc.dequant_e4m3(xi["q8"][b].numpy(), xi["qs"][b].numpy()), xi["w"][b].numpy(),
                          orc.dequant_e4m3(xi["k8"][b].numpy(), xi["ks"][b].numpy()), pos, ld=L + 5)
        l_o, g_o = orc.warmup_loss(p_o, i_o, pos)
        for r, ps in enumerate(pos):
            n = ps + 1
            # target: the head mean of exponentials of fp32 logits against the attention kernel's lse
            assert np.all(np.abs(gt[b, r, :n] - p_o[r, :n]) <= 2e-3 * p_o[r, :n] + 1e-7), (b, r)
            assert np.all(np.isnan(gs[b, r, n:]))  # past the query: untouched
            sm_i = g_o[r, :n] + p_o[r, :n]
            assert np.all(np.abs(gs[b, r, :n] - g_o[r, :n]) <= 2e-3 * (sm_i + p_o[r, :n]) + 1e-7), (b, r)
        np.testing.assert_allclose(gl[b], l_o, rtol=2e-3, atol=1e-5)
