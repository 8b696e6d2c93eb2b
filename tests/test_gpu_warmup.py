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


@pytest.mark.parametrize("B,L,n_q", [(2, 256, 256), (1, 333, 100), (1, 150, 77)])  # odd n_q: a lone last query
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


def backward_bounds(orc, xi, b, g, pos):
    """Sums of the magnitudes of every term of dq, dw and dk (float64), from the dequantised inputs: the
    scale of the rounding of each term (bf16 operands of the second products, fp32 accumulation)."""
    qh = orc.dequant_e4m3(xi["q8"][b].numpy(), xi["qs"][b].numpy()).astype(np.float64)
    kh = orc.dequant_e4m3(xi["k8"][b].numpy(), xi["ks"][b].numpy()).astype(np.float64)
    w = xi["w"][b].numpy().astype(np.float64)
    S = kh.shape[0]
    d = np.einsum("rhd,sd->rhs", qh, kh)
    vis = np.arange(S)[None, :] <= pos[:, None]
    ga = np.where(vis, np.abs(g[:, :S].astype(np.float64)), 0.0)
    on = (d > 0) * ga[:, None, :]                                   # [R, H, S]: |g| [d > 0]
    bq = np.einsum("rhs,sd->rhd", on, np.abs(kh)) * np.abs(w)[:, :, None]
    bw = np.einsum("rhs,rhs->rh", on, np.maximum(d, 0))
    bk = np.einsum("rhs,rhd->sd", on * np.abs(w)[:, :, None], np.abs(qh))
    return bq, bw, bk


def run_backward(dsa, xi, g):
    return [t.cpu().numpy() for t in dsa.warmup_indexer_backward(
        xi["q8"].to(DEV), xi["qs"].to(DEV), xi["k8"].to(DEV), xi["ks"].to(DEV), xi["w"].to(DEV), g.to(DEV))]


# several key blocks and query parts with ragged ends, fewer queries than keys, fewer than 8 queries
@pytest.mark.parametrize("B,L,n_q,exact", [(2, 256, 256, True), (1, 333, 100, True), (1, 70, 3, True),
                                           (1, 600, 600, True), (2, 300, 170, False), (1, 129, 129, False)])
def test_warmup_backward_vs_oracle(orc, dsa, B, L, n_q, exact):
    """dq, dw and dk against the oracle.  With exact=True, g holds multiples of 2^-10 below 2^-5: every
    bf16 operand and every product is then exact and only the fp32 summation order differs (the bound is
    2^-20 of the sum of the terms' magnitudes).  Otherwise g is a general float: the second products round
    g k_scale and g w q_scale to bf16 (relative error at most 2^-9 per term), so the bound is 2^-8 of that
    sum.  dw is an fp32 sum of exact products in both cases.  Entries of g past each query's position are
    NaN and must not be read."""
    xi = exact_indexer_inputs(B, L, n_q, seed=3 * L + n_q)
    gen = torch.Generator().manual_seed(L + 7)
    ld = L + 3
    if exact:
        g = torch.randint(-31, 32, (B, n_q, ld), generator=gen).float() / 1024.0
    else:
        g = torch.randn((B, n_q, ld), generator=gen) * 1e-3
    pos = np.arange(L - n_q, L, dtype=np.int64)
    for r, p in enumerate(pos):
        g[:, r, p + 1:] = float("nan")
    dq, dw, dk = run_backward(dsa, xi, g)
    rel = 2.0 ** -20 if exact else 2.0 ** -8
    for b in range(B):
        gb = g[b].numpy()
        q_o, w_o, k_o = orc.warmup_backward(orc.dequant_e4m3(xi["q8"][b].numpy(), xi["qs"][b].numpy()),
                                            xi["w"][b].numpy(),
                                            orc.dequant_e4m3(xi["k8"][b].numpy(), xi["ks"][b].numpy()),
                                            np.nan_to_num(gb, nan=0.0), pos)
        bq, bw, bk = backward_bounds(orc, xi, b, np.nan_to_num(gb, nan=0.0), pos)
        assert np.all(np.abs(dq[b] - q_o) <= rel * bq + 1e-30), (b, np.max(np.abs(dq[b] - q_o) - rel * bq))
        assert np.all(np.abs(dw[b] - w_o) <= 2.0 ** -20 * bw + 1e-30), (b, np.max(np.abs(dw[b] - w_o)))
        assert np.all(np.abs(dk[b] - k_o) <= rel * bk + 1e-30), (b, np.max(np.abs(dk[b] - k_o) - rel * bk))
        assert np.abs(q_o).max() > 0 and np.abs(k_o).max() > 0


def test_warmup_backward_full_8k(orc, dsa):
    """8192 queries over 8192 keys, the benchmark's launch configuration: dq and dw on sampled query rows,
    dk on sampled keys (each as a one-key problem over every query that sees it).  Exact inputs as above."""
    L = 8192
    xi = exact_indexer_inputs(1, L, L, seed=81)
    g = torch.randint(-31, 32, (1, L, L), generator=torch.Generator().manual_seed(82)).float() / 1024.0
    dq, dw, dk = run_backward(dsa, xi, g)
    qh = orc.dequant_e4m3(xi["q8"][0].numpy(), xi["qs"][0].numpy())
    kh = orc.dequant_e4m3(xi["k8"][0].numpy(), xi["ks"][0].numpy())
    w, gb = xi["w"][0].numpy(), g[0].numpy()
    rows = np.array([0, 1, 31, 32, 127, 2048, 4097, 8000, 8190, 8191])
    q_o, w_o, _ = orc.warmup_backward(qh[rows], w[rows], kh, gb[rows], rows.astype(np.int64))
    d = np.matmul(qh[rows].astype(np.float64), kh.T.astype(np.float64))        # [rows, 64, 8192]
    on = (d > 0) * np.where(np.arange(L)[None, :] <= rows[:, None], np.abs(gb[rows]), 0.0)[:, None, :]
    bq = np.matmul(on, np.abs(kh).astype(np.float64)) * np.abs(w[rows])[:, :, None]
    bw = np.sum(on * np.maximum(d, 0), axis=2)
    assert np.all(np.abs(dq[0][rows] - q_o) <= 2.0 ** -20 * bq + 1e-30)
    assert np.all(np.abs(dw[0][rows] - w_o) <= 2.0 ** -20 * bw + 1e-30)
    for s in (0, 1, 127, 128, 3000, 8191):
        t = np.arange(s, L)
        _, _, k_o = orc.warmup_backward(qh[t], w[t], kh[s:s + 1], gb[t][:, s:s + 1].copy(),
                                        np.zeros(len(t), np.int64))
        dts = np.matmul(qh[t], kh[s])                                            # [T, 64]
        wt = (dts > 0) * np.abs(gb[t, s])[:, None] * np.abs(w[t])
        bk = np.einsum("th,thd->d", wt.astype(np.float64), np.abs(qh[t]).astype(np.float64))
        assert np.all(np.abs(dk[0][s] - k_o[0]) <= 2.0 ** -20 * bk + 1e-30), s


def test_warmup_backward_key_block_major_order(orc, dsa):
    """Four sequences of 6144 queries over 6144 keys: the query codes (4 x 6144 x 8 KiB, 201 MB) pass the
    size at which the dk kernel runs its workgroups key block by key block instead of part by part, with
    the sequence as the third grid dimension.  dq and dw on sampled rows, dk on sampled keys of every
    sequence (each as a one-key problem over the queries that see it).  Exact inputs as above."""
    B, L = 4, 6144
    xi = exact_indexer_inputs(B, L, L, seed=91)
    g = torch.randint(-31, 32, (B, L, L), generator=torch.Generator().manual_seed(92)).float() / 1024.0
    dq, dw, dk = run_backward(dsa, xi, g)
    rows = np.array([0, 31, 1024, 4097, 6143])
    for b in range(B):
        qh = orc.dequant_e4m3(xi["q8"][b].numpy(), xi["qs"][b].numpy())
        kh = orc.dequant_e4m3(xi["k8"][b].numpy(), xi["ks"][b].numpy())
        w, gb = xi["w"][b].numpy(), g[b].numpy()
        q_o, w_o, _ = orc.warmup_backward(qh[rows], w[rows], kh, gb[rows], rows.astype(np.int64))
        d = np.matmul(qh[rows].astype(np.float64), kh.T.astype(np.float64))
        on = (d > 0) * np.where(np.arange(L)[None, :] <= rows[:, None], np.abs(gb[rows]), 0.0)[:, None, :]
        bq = np.matmul(on, np.abs(kh).astype(np.float64)) * np.abs(w[rows])[:, :, None]
        bw = np.sum(on * np.maximum(d, 0), axis=2)
        assert np.all(np.abs(dq[b][rows] - q_o) <= 2.0 ** -20 * bq + 1e-30), b
        assert np.all(np.abs(dw[b][rows] - w_o) <= 2.0 ** -20 * bw + 1e-30), b
        for s in (0, 255, 256, 3071, 6143):
            t = np.arange(s, L)
            _, _, k_o = orc.warmup_backward(qh[t], w[t], kh[s:s + 1], gb[t][:, s:s + 1].copy(),
                                            np.zeros(len(t), np.int64))
            dts = np.matmul(qh[t], kh[s])
            wt = (dts > 0) * np.abs(gb[t, s])[:, None] * np.abs(w[t])
            bk = np.einsum("th,thd->d", wt.astype(np.float64), np.abs(qh[t]).astype(np.float64))
            assert np.all(np.abs(dk[b][s] - k_o[0]) <= 2.0 ** -20 * bk + 1e-30), (b, s)
            assert np.abs(k_o).max() > 0
