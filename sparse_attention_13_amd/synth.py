"""Seeded synthetic inputs for the DSA path.

This module only draws random inputs and stores them in the formats the path consumes (fp8 e4m3
codes with per-row fp32 scales, bf16, fp32).  It holds none of the method's arithmetic, imports
neither the HIP binding nor the oracle, and is the single source of inputs for both.

Workload recipes (fixed sizes; all draws come from one ``torch.Generator`` per call, in the order
written below, so a seed and a device reproduce the same bytes):

* ``tiny``: one sequence of L=256, fp32 throughout.  Indexer H_I=4, d_I=32, q/k ~ N(0,1),
  w ~ N(0,1)/sqrt(H_I); top-k 32; MQA-MLA with 8 heads, d_qk=80 (64 + 16 rope), d_v=64,
  entries ~ N(0,1), softmax scale 1/sqrt(80).
* ``prefill``: one sequence; indexer H_I=64, d_I=128 stored as e4m3 codes with fp32 scales
  (amax/448 per (token, head) row of q and per token of k), w ~ N(0,1)/8; 128 MLA heads,
  d_qk=576, d_v=512, bf16 ~ N(0,1); softmax scale 1/sqrt(576); k=2048.  "Needle" keys make the
  selection non-trivial: with a unit direction u (scaled to norm sqrt(d_I)), a needle key is
  sqrt(.8) u + sqrt(.2) n, and every query head is sign(w) (sqrt(.8) u + sqrt(.2) n), so heads
  with positive weight see cosine ~0.8 with every needle and the others see ~-0.8, which the
  ReLU removes.  Non-needle keys are plain N(0,1).
* ``decode``: B sequences with one query each at the last position of S cached tokens, per-sequence
  seeds (seed + b), no needles, same dtypes and distributions as ``prefill``.
* ``selection``: a top-k-shaped selection drawn directly (numpy Generator): for query t at position
  pos = L - n_q + t, n = min(k, pos + 1) distinct keys in [0, pos], ascending, -1 padded; all keys when
  n = pos + 1, else the n/4 most recent keys plus (n - n/4) drawn uniformly from the rest.
* ``sparse_grad``: dout ~ N(0,1) in bf16, the upstream gradient of the attention output.
"""
from __future__ import annotations

import math

import torch

E4M3_MAX = 448.0


def quantize_e4m3_rows(x: torch.Tensor):
    """Store x (float32, [..., C]) as e4m3fn codes with one fp32 scale per row: scale = amax/448.

    Returns (codes uint8 [..., C], scales float32 [...]).  Rows of zeros get scale 1."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    codes = (x / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), scale.contiguous()


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _randn(shape, g, device, dtype=torch.float32, chunk_rows: int | None = None):
    """N(0,1) draws, generated in fp32 (row chunks keep the temporary small) and cast to dtype."""
    if chunk_rows is None or shape[0] <= chunk_rows:
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)
    out = torch.empty(shape, device=device, dtype=dtype)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device,
                                 dtype=torch.float32).to(dtype)
    return out


def tiny(seed: int = 0, device="cpu", L: int = 256, H_I: int = 4, d_I: int = 32, H: int = 8,
         d_qk: int = 80, d_v: int = 64, k: int = 32) -> dict:
    """The tiny fp32 causal case.  Draw order: q_i, k_i, w, q, kv."""
    g = _gen(seed, device)
    q_i = _randn((L, H_I, d_I), g, device)
    k_i = _randn((L, d_I), g, device)
    w = _randn((L, H_I), g, device) / math.sqrt(H_I)
    q = _randn((L, H, d_qk), g, device)
    kv = _randn((L, d_qk), g, device)
    return dict(kind="tiny", dtype="f32", L=L, n_q=L, n_kv=L, H_I=H_I, d_I=d_I, H=H, d_qk=d_qk,
                d_v=d_v, k=k, sm_scale=1.0 / math.sqrt(d_qk), q_i=q_i, k_i=k_i, w=w, q=q, kv=kv)


def needle_positions(L: int, n: int, layout: str, g: torch.Generator, device) -> torch.Tensor:
    """Sorted distinct token positions of the planted keys: 'random' (uniform without replacement)
    or 'even' (position floor((i + 1/2) * L / n))."""
    if n == 0:
        return torch.zeros(0, dtype=torch.int64)
    if layout == "even":
        return torch.tensor([int((i + 0.5) * L / n) for i in range(n)], dtype=torch.int64)
    perm = torch.randperm(L, generator=g, device=device)[:n]
    return torch.sort(perm.cpu())[0]


def prefill(L: int, seed: int = 0, device="cpu", n_needles: int = 0, needle_layout: str = "random",
            n_q: int | None = None, H_I: int = 64, d_I: int = 128, H: int = 128, d_qk: int = 576,
            d_v: int = 512, k: int = 2048, with_mla: bool = True) -> dict:
    """One sequence of L tokens whose last n_q (default L) tokens are the queries.

    Draw order: u, needle positions, w, query noise, key noise, needle-key noise, q (MLA), kv (MLA).
    Returns fp8 codes/scales for the indexer, fp32 w, bf16 q/kv."""
    n_q = L if n_q is None else n_q
    g = _gen(seed, device)
    u = _randn((d_I,), g, device)
    u = u / u.norm() * math.sqrt(d_I)
    npos = needle_positions(L, n_needles, needle_layout, g, device)
    w = _randn((n_q, H_I), g, device) / 8.0
    qn = _randn((n_q, H_I, d_I), g, device, chunk_rows=4096)
    kn = _randn((L, d_I), g, device)
    if n_needles:
        a, b = math.sqrt(0.8), math.sqrt(0.2)
        sign = torch.where(w >= 0, 1.0, -1.0).unsqueeze(-1)
        q_i = sign * (a * u + b * qn)
        nn = _randn((n_needles, d_I), g, device)
        kn[npos.to(device)] = a * u + b * nn
    else:
        q_i = qn
    del qn
    q8, q_scale = quantize_e4m3_rows(q_i)
    del q_i
    k8, k_scale = quantize_e4m3_rows(kn)
    out = dict(kind="prefill", dtype="fp8/bf16", L=L, n_q=n_q, n_kv=L, H_I=H_I, d_I=d_I, H=H, d_qk=d_qk,
               d_v=d_v, k=k, sm_scale=1.0 / math.sqrt(d_qk), q8=q8, q_scale=q_scale, k8=k8,
               k_scale=k_scale, w=w, needles=npos)
    if with_mla:
        out["q"] = _randn((n_q, H, d_qk), g, device, torch.bfloat16, chunk_rows=1024)
        out["kv"] = _randn((L, d_qk), g, device, torch.bfloat16, chunk_rows=8192)
    return out


def mha_heads(L: int, seed: int = 0, device="cpu", n_q: int | None = None, H: int = 128, d_qk: int = 192,
              d_v: int = 128) -> dict:
    """MHA-form attention inputs of one sequence (masked MHA mode): per-head queries of the last n_q
    tokens and per-head key and value rows of all L tokens, bf16 ~ N(0, 1), token-major.
    Draw order: q, k, v (a generator of its own, seed + 1000003, so the indexer inputs of the same
    seed stay as prefill() draws them)."""
    n_q = L if n_q is None else n_q
    g = _gen(seed + 1000003, device)
    return dict(kind="mha", L=L, n_q=n_q, H=H, d_qk=d_qk, d_v=d_v, sm_scale=1.0 / math.sqrt(d_qk),
                q=_randn((n_q, H, d_qk), g, device, torch.bfloat16, chunk_rows=1024),
                k=_randn((L, H, d_qk), g, device, torch.bfloat16, chunk_rows=1024),
                v=_randn((L, H, d_v), g, device, torch.bfloat16, chunk_rows=1024))


def mla_weights(H: int = 128, seed: int = 0, device="cpu", d_nope: int = 128, d_c: int = 512, d_v: int = 128) -> dict:
    """Random up-projection weights of MLA (no trained weights are used): W_UK,h [d_nope, d_c] and
    W_UV,h [d_v, d_c], entries N(0, 1) / sqrt(fan-in), bf16, stored with the contraction dimension last:
    w_ukt [H, d_c, d_nope] (the transpose of W_UK,h) and w_uv [H, d_v, d_c].
    Draw order: W_UK, W_UV (a generator of its own, seed + 2000003)."""
    g = _gen(seed + 2000003, device)
    w_uk = _randn((H, d_nope, d_c), g, device) / math.sqrt(d_nope)
    w_uv = _randn((H, d_v, d_c), g, device) / math.sqrt(d_c)
    return dict(w_ukt=w_uk.transpose(1, 2).contiguous().to(torch.bfloat16), w_uv=w_uv.to(torch.bfloat16))


def decode(B: int, S: int, seed: int = 0, device="cpu", H_I: int = 64, d_I: int = 128, H: int = 128,
           d_qk: int = 576, d_v: int = 512, k: int = 2048) -> dict:
    """B sequences, one new query each at position S-1 over S cached tokens (per-sequence seed
    seed + b; per sequence the draw order is w, q_i, k_i, q, kv)."""
    q8 = torch.empty((B, H_I, d_I), dtype=torch.uint8, device=device)
    q_scale = torch.empty((B, H_I), dtype=torch.float32, device=device)
    w = torch.empty((B, H_I), dtype=torch.float32, device=device)
    k8 = torch.empty((B, S, d_I), dtype=torch.uint8, device=device)
    k_scale = torch.empty((B, S), dtype=torch.float32, device=device)
    q = torch.empty((B, H, d_qk), dtype=torch.bfloat16, device=device)
    kv = torch.empty((B, S, d_qk), dtype=torch.bfloat16, device=device)
    for b in range(B):
        g = _gen(seed + b, device)
        w[b] = _randn((H_I,), g, device) / 8.0
        qb, sb = quantize_e4m3_rows(_randn((H_I, d_I), g, device))
        q8[b], q_scale[b] = qb, sb
        kb, ksb = quantize_e4m3_rows(_randn((S, d_I), g, device, chunk_rows=65536))
        k8[b], k_scale[b] = kb, ksb
        q[b] = _randn((H, d_qk), g, device, torch.bfloat16)
        kv[b] = _randn((S, d_qk), g, device, torch.bfloat16, chunk_rows=16384)
    return dict(kind="decode", dtype="fp8/bf16", B=B, S=S, n_q=1, n_kv=S, H_I=H_I, d_I=d_I, H=H,
                d_qk=d_qk, d_v=d_v, k=k, sm_scale=1.0 / math.sqrt(d_qk), q8=q8, q_scale=q_scale,
                k8=k8, k_scale=k_scale, w=w, q=q, kv=kv)


def bf16_bits(x: torch.Tensor):
    """The raw uint16 bit patterns of a bf16 tensor, on the host, as numpy."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view("uint16")


def u8(x: torch.Tensor):
    """A uint8 tensor on the host, as numpy."""
    return x.detach().contiguous().cpu().numpy()


def selection(L: int, n_q: int, k: int, seed: int = 0, B: int = 1):
    """A selection with the shape and structure of the top-k output (see the module notes), as numpy
    int32 [B, n_q, k]: it stands in for an indexer-driven selection where the oracle cannot afford to
    recompute the index scores."""
    import numpy as np
    gen = np.random.default_rng(int(seed) + 3000017)
    out = np.full((B, n_q, k), -1, np.int32)
    for b in range(B):
        for t in range(n_q):
            pos = L - n_q + t
            n = min(k, pos + 1)
            if n == pos + 1:
                out[b, t, :n] = np.arange(n, dtype=np.int32)
                continue
            w = n // 4
            far = gen.choice(pos + 1 - w, size=n - w, replace=False)
            out[b, t, :n] = np.sort(np.concatenate([far, np.arange(pos + 1 - w, pos + 1)])).astype(np.int32)
    return out


def sparse_grad(shape, seed: int = 0, device="cpu"):
    """dout ~ N(0,1) as bf16 with the given shape."""
    return _randn(tuple(shape), _gen(int(seed) + 4000037, device), device, torch.bfloat16)
