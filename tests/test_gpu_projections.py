"""MQA-mode projections (query absorption of W_UK, output up-projection W_UV) vs the CPU oracle, through the
C ABI, on the GPU.  Tolerances: tests/parity.py (projection rule)."""
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


def check(g, o):
    d = np.abs(g.astype(np.float64) - o)
    ratio = float((d / (parity.PROJ_ABS + parity.PROJ_REL * np.abs(o))).max())
    assert ratio <= 1.0, (ratio, float(d.max()))


@pytest.mark.parametrize("rows,H", [(300, 3), (128, 1), (1, 2), (1000, 5)])
def test_projections_vs_oracle(orc, dsa, rows, H):
    g = torch.Generator(device=DEV).manual_seed(rows + H)
    q = torch.randn((rows, H, 192), generator=g, device=DEV).to(torch.bfloat16)
    o_lat = torch.randn((rows, H, 512), generator=g, device=DEV).to(torch.bfloat16)
    w = synth.mla_weights(H, seed=rows, device=DEV)
    q_mqa = dsa.mla_absorb_q(q, w["w_ukt"])
    o = dsa.mla_out_proj(o_lat, w["w_uv"])
    torch.cuda.synchronize()
    qf, wk = f32(orc, q), f32(orc, w["w_ukt"])
    ref = orc.absorb_q(qf, wk)
    gq = f32(orc, q_mqa)
    check(gq[..., :512], ref[..., :512])
    assert np.array_equal(synth.bf16_bits(q_mqa)[..., 512:], synth.bf16_bits(q)[..., 128:])  # rope copied
    check(f32(orc, o), orc.out_proj(f32(orc, o_lat), f32(orc, w["w_uv"])))


def test_projections_exact_integers(orc, dsa):
    """Entries in {-1, 0, 1}: every sum is an integer of magnitude <= 512 (<= 128 for the absorption), so
    fp32 accumulation is exact in any order and bf16 holds the absorbed query exactly."""
    g = torch.Generator(device=DEV).manual_seed(7)
    rows, H = 257, 2
    ri = lambda shape: torch.randint(-1, 2, shape, generator=g, device=DEV).to(torch.bfloat16)
    q, wk = ri((rows, H, 192)), ri((H, 512, 128))
    q_mqa = dsa.mla_absorb_q(q, wk)
    torch.cuda.synchronize()
    ref = orc.absorb_q(f32(orc, q), f32(orc, wk))
    assert np.array_equal(f32(orc, q_mqa).astype(np.float64), ref)
    o_lat, wv = ri((rows, H, 512)), ri((H, 128, 512))
    o = dsa.mla_out_proj(o_lat, wv)
    torch.cuda.synchronize()
    ref = orc.out_proj(f32(orc, o_lat), f32(orc, wv))
    # sums up to 512 in magnitude: bf16 keeps 8 significant bits, so compare after rounding the reference
    ref_bf16 = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    assert np.array_equal(f32(orc, o), ref_bf16)


def test_projections_full_32k(orc, dsa):
    """32768 tokens x 128 heads, the size of the prefill workload; rows sampled across row tiles."""
    rows, H = 32768, 128
    g = torch.Generator(device=DEV).manual_seed(3)
    q = torch.randn((rows, H, 192), generator=g, device=DEV).to(torch.bfloat16)
    o_lat = torch.randn((rows, H, 512), generator=g, device=DEV).to(torch.bfloat16)
    w = synth.mla_weights(H, seed=0, device=DEV)
    q_mqa = dsa.mla_absorb_q(q, w["w_ukt"])
    o = dsa.mla_out_proj(o_lat, w["w_uv"])
    torch.cuda.synchronize()
    sel = torch.tensor([0, 1, 127, 128, 5000, 16383, 32640, 32767], device=DEV)
    ref = orc.absorb_q(f32(orc, q[sel]), f32(orc, w["w_ukt"]))
    check(f32(orc, q_mqa[sel])[..., :512], ref[..., :512])
    check(f32(orc, o[sel]), orc.out_proj(f32(orc, o_lat[sel]), f32(orc, w["w_uv"])))
    assert torch.isfinite(q_mqa.float()).all() and torch.isfinite(o.float()).all()
