"""Sparse training backward (dq, dkv and the head-mean target through the sparse MQA attention) and the
stage-2 indexer loss vs the CPU oracle, through the C ABI, on the GPU.  Tolerances: tests/parity.py
(sparse backward rule).  The forward's out and lse come from the attention kernel, as in training."""
import numpy as np
import pytest
import torch

import parity
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


def run(dsa, L, n_q, B, idx, seed):
    xs = [synth.prefill(L, seed=seed + b, device=DEV, n_q=n_q) for b in range(B)]
    q = torch.stack([x["q"] for x in xs]).contiguous()
    kv = torch.stack([x["kv"] for x in xs]).contiguous()
    sm = xs[0]["sm_scale"]
    gi = torch.from_numpy(idx).to(DEV)
    out, lse = dsa.sparse_mla_attn(q, kv, gi, 512, sm)
    dout = synth.sparse_grad((B, n_q, 128, 512), seed=seed, device=DEV)
    dq, dkv, pbar = dsa.sparse_mla_backward(q, kv, gi, out, lse, dout, sm)
    torch.cuda.synchronize()
    return q, kv, dout, sm, dq.cpu().numpy(), dkv.cpu().numpy(), pbar.cpu().numpy()


def check(orc, q, kv, idx, dout, sm, dq, dkv, pbar, what):
    qf, kf, df = f32(orc, q), f32(orc, kv), f32(orc, dout)
    q_o, kv_o, pb_o = orc.sparse_attn_backward(qf, kf, idx, 512, sm, df)
    mq, mkv = parity.sparse_bwd_magnitudes(qf, kf, idx, df, sm, 512)
    e_q = np.abs(dq - q_o) - parity.BWD_REL * mq
    e_k = np.abs(dkv - kv_o) - parity.BWD_REL * mkv
    assert e_q.max() <= 0, (what, "dq", float(e_q.max()), float(np.abs(dq - q_o).max()))
    assert e_k.max() <= 0, (what, "dkv", float(e_k.max()), float(np.abs(dkv - kv_o).max()))
    np.testing.assert_allclose(pbar, pb_o, rtol=1e-5, atol=1e-7)
    assert np.abs(q_o).max() > 0 and np.abs(kv_o).max() > 0


# several steps with a ragged last one (k not a multiple of 32), rows with fewer candidates than k,
# more than one workgroup chunk (512 query rows), two sequences
@pytest.mark.parametrize("B,L,n_q,k", [(1, 300, 300, 64), (2, 200, 77, 50), (1, 1000, 100, 2048),
                                       (1, 700, 700, 32)])
def test_sparse_backward_vs_oracle(orc, dsa, B, L, n_q, k):
    idx = synth.selection(L, n_q, k, seed=L + k, B=B)
    q, kv, dout, sm, dq, dkv, pbar = run(dsa, L, n_q, B, idx, seed=L)
    for b in range(B):
        check(orc, q[b], kv[b], idx[b], dout[b], sm, dq[b], dkv[b], pbar[b], (B, L, n_q, k, b))


def test_sparse_backward_ignored_entries(orc, dsa):
    """Entries -1 or past the keys carry no gradient (as the forward attention skips them); a row with none
    gets dq = 0 and pbar = 0; an entry past the query's position counts as the forward counts it; entries
    in any order."""
    L, n_q, k = 400, 150, 40
    rng = np.random.default_rng(9)
    pos = np.arange(L - n_q, L)
    idx = np.stack([rng.choice(L + 30, size=k, replace=False) for _ in range(n_q)]).astype(np.int32)
    idx[:, ::5] = -1
    idx[7, :] = -1
    idx[8, :] = L + 3
    idx[9, :] = -1
    idx[9, 0] = pos[9] + 1
    clean = np.where(idx < L, idx, -1).astype(np.int32)
    q, kv, dout, sm, dq, dkv, pbar = run(dsa, L, n_q, 1, idx[None], seed=5)
    check(orc, q[0], kv[0], clean, dout[0], sm, dq[0], dkv[0], pbar[0], "ignored")
    for r in (7, 8):
        assert np.all(dq[0, r] == 0.0) and np.all(pbar[0, r] == 0.0)
    # one entry: P = 1 and the entry's pbar is 1 (dq = 0 up to D formed from the bf16 output: checked above)
    assert abs(pbar[0, 9, 0] - 1.0) <= 1e-6 and np.all(pbar[0, 9, 1:] == 0.0)


def test_sparse_backward_full_8k(orc, dsa):
    """8192 queries, k = 2048, the benchmark's launch configuration: dq and pbar on sampled rows; dkv on
    late keys, each complete from the few rows that can select it; and at every size the column sums of
    dkv: the key part sums to zero (the softmax Jacobian), the value part to the sum of dout over rows
    that select anything."""
    L, k = 8192, 2048
    idx = synth.selection(L, L, k, seed=1)
    q, kv, dout, sm, dq, dkv, pbar = run(dsa, L, L, 1, idx, seed=3)
    kf = f32(orc, kv[0])

    def rows_f32(t, rows):
        return f32(orc, t[0][torch.from_numpy(rows).to(DEV)])

    rows = np.array([0, 1, 31, 2047, 2048, 4097, 8190, 8191])
    qf, df = rows_f32(q, rows), rows_f32(dout, rows)
    q_o, _, pb_o = orc.sparse_attn_backward(qf, kf, idx[0][rows], 512, sm, df)
    mq, _ = parity.sparse_bwd_magnitudes(qf, kf, idx[0][rows], df, sm, 512)
    assert np.all(np.abs(dq[0][rows] - q_o) <= parity.BWD_REL * mq)
    np.testing.assert_allclose(pbar[0][rows], pb_o, rtol=1e-5, atol=1e-7)
    late = np.arange(L - 24, L)                       # rows that can select keys >= L - 24
    qf, df = rows_f32(q, late), rows_f32(dout, late)
    _, kv_o, _ = orc.sparse_attn_backward(qf, kf, idx[0][late], 512, sm, df)
    _, mkv = parity.sparse_bwd_magnitudes(qf, kf, idx[0][late], df, sm, 512)
    keys = np.array([L - 1, L - 2, L - 7, L - 20])
    assert np.all(np.abs(dkv[0][keys] - kv_o[keys]) <= parity.BWD_REL * mkv[keys])
    col = dkv[0].astype(np.float64).sum(axis=0)
    ref_v = dout[0].double().sum(dim=(0, 1)).cpu().numpy()
    scale = np.abs(dkv[0]).astype(np.float64).sum(axis=0)
    assert np.all(np.abs(col[:512] - ref_v) <= 2.0 ** -7 * scale[:512] + 1e-3)
    assert np.all(np.abs(col[512:]) <= 2.0 ** -7 * scale[512:] + 1e-3)


@pytest.mark.parametrize("B,L,n_q,k", [(1, 300, 300, 64), (2, 500, 120, 100)])
def test_sparse_kl_loss_vs_oracle(orc, dsa, B, L, n_q, k):
    """Stage-2 indexer loss from the kernel's own pbar: loss and gradient against the oracle fed the oracle's
    pbar of the same attention."""
    idx = synth.selection(L, n_q, k, seed=k, B=B)
    q, kv, dout, sm, dq, dkv, pbar = run(dsa, L, n_q, B, idx, seed=11)
    gen = torch.Generator().manual_seed(L)
    scores = torch.randn((B, n_q, L + 3), generator=gen)
    pos = np.arange(L - n_q, L, dtype=np.int64)
    sg = scores.to(DEV)
    loss = dsa.sparse_kl_loss(sg, torch.from_numpy(pbar).to(DEV), torch.from_numpy(idx).to(DEV), n_kv=L)
    torch.cuda.synchronize()
    g, l = sg.cpu().numpy(), loss.cpu().numpy()
    for b in range(B):
        _, _, pb_o = orc.sparse_attn_backward(f32(orc, q[b]), f32(orc, kv[b]), idx[b], 512, sm, f32(orc, dout[b]))
        l_o, g_o = orc.sparse_kl_loss(pb_o, idx[b], scores[b].numpy(), pos)
        np.testing.assert_allclose(l[b], l_o, rtol=1e-4, atol=1e-6)
        for r, p in enumerate(pos):
            np.testing.assert_allclose(g[b, r, :p + 1], g_o[r, :p + 1], rtol=1e-4, atol=1e-6)
            assert np.array_equal(g[b, r, p + 1:], scores[b, r, p + 1:].numpy())   # past the query: untouched
