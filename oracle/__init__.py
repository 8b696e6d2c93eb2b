"""Plain CPU oracle for the DSA path (lightning indexer -> top-k -> sparse MLA attention).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the CPU-baseline leg of
the benchmark, never by the product library.  It shares no code with the HIP path; the arithmetic
lives in ``dsa_oracle.c`` (plain C, built with gcc) and this module only marshals numpy arrays.

Sources (web pages on DeepSeek-V3.2):
  * velog summary "DeepSeek-V3.2: Pushing the Frontier of Open Large Language Models",
    section 1.1 (lightning indexer equation for I_{t,s}, ReLU, FP8, previous tokens),
    section 1.2 (top-k retrieval and u_t = Attn(h_t, {c_s})), section 1.3 (MQA mode: each
    latent KV entry shared by all query heads), Continued Pre-Training stage 2 (k = 2048).
  * notes.yuuk.io page of the same title, section "DeepSeek Sparse Attention (DSA)".

``forward`` composes the three steps in the pages' order.  Every function is pinned by
``tests/test_oracle_pins.py`` against closed forms, library routines, invariants and brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile dsa_oracle.c with gcc into oracle/liboracle.so (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_to_f32.restype = ctypes.c_float
        lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f32.restype = ctypes.c_float
        lib.oracle_decode_e4m3.argtypes = [P, I64, P]
        lib.oracle_decode_bf16.argtypes = [P, I64, P]
        lib.oracle_dequant_e4m3.argtypes = [P, P, I64, I64, P]
        lib.oracle_indexer.argtypes = [P, P, P, I64, P, I, I, P, I64, P, P]
        lib.oracle_topk.argtypes = [P, I64, I64, P, I, P, P]
        lib.oracle_sparse_attn.argtypes = [P, P, P, I64, I, I, I, I, ctypes.c_double, P, P]
        lib.oracle_sparse_attn_mha.argtypes = [P, P, P, P, I64, I, I, I, I, ctypes.c_double, P, P]
        lib.oracle_warmup_target.argtypes = [P, P, I64, P, I, I, ctypes.c_double, P, I64]
        lib.oracle_warmup_loss.argtypes = [P, P, I64, P, I64, I64, P, P, I64]
        lib.oracle_warmup_backward.argtypes = [P, P, P, P, I64, P, I, I, I64, I64, P, P, P]
        lib.oracle_sparse_attn_backward.argtypes = [P, P, P, I64, I, I, I, I, ctypes.c_double, P, I64, P, P, P]
        lib.oracle_threads.restype = I
        _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def threads() -> int:
    """Number of host threads the oracle's parallel loops use."""
    return int(_load().oracle_threads())


def e4m3_to_f32(codes: np.ndarray) -> np.ndarray:
    """Decode OCP e4m3fn byte codes to float32 (exact)."""
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float32)
    _load().oracle_decode_e4m3(_p(codes), codes.size, _p(out))
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 (exact)."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float32)
    _load().oracle_decode_bf16(_p(bits), bits.size, _p(out))
    return out


def dequant_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp32(e4m3(code) * scale) with one scale per leading-row: codes [..., C], scales [...]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    cols = codes.shape[-1]
    rows = codes.size // cols
    assert scales.size == rows, (scales.shape, codes.shape)
    out = np.empty(codes.shape, np.float32)
    _load().oracle_dequant_e4m3(_p(codes), _p(scales), rows, cols, _p(out))
    return out


def indexer(q: np.ndarray, w: np.ndarray, k: np.ndarray, pos: np.ndarray, ld: int | None = None,
            with_mag: bool = False):
    """Index scores I[r, s] = sum_j w[r, j] * ReLU(q[r, j, :] . k[s, :]) for s <= pos[r].

    q [R, H, d] float32, w [R, H] float32, k [S, d] float32, pos [R] int64.
    Returns scores [R, ld] float32 with -inf where s > pos[r]; with_mag=True returns
    (scores, mag, absmag): mag = sum_j |w| ReLU(q.k), absmag = sum_j |w| sum_i |q_i k_i|."""
    q = _c(q, np.float32)
    w = _c(w, np.float32)
    k = _c(k, np.float32)
    pos = _c(pos, np.int64)
    R, H, d = q.shape
    assert w.shape == (R, H) and k.shape[1] == d and pos.shape == (R,)
    assert R == 0 or pos.max() < k.shape[0]
    if ld is None:
        ld = int(pos.max()) + 1 if R else 1
    scores = np.full((R, ld), -np.inf, np.float32)
    mag = np.zeros((R, ld), np.float32) if with_mag else None
    absmag = np.zeros((R, ld), np.float32) if with_mag else None
    _load().oracle_indexer(_p(q), _p(w), _p(k), R, _p(pos), H, d, _p(scores), ld,
                           _p(mag) if with_mag else None, _p(absmag) if with_mag else None)
    return (scores, mag, absmag) if with_mag else scores


def topk(scores: np.ndarray, pos: np.ndarray, k: int):
    """Per row: the k largest of scores[r, 0..pos[r]] (ties -> lower index), ascending, -1 padded.

    Returns (idx [R, k] int32, kth [R] float32 = k-th largest score or -inf if <= k candidates)."""
    scores = _c(scores, np.float32)
    pos = _c(pos, np.int64)
    R = scores.shape[0]
    assert pos.shape == (R,) and (R == 0 or pos.max() < scores.shape[1])
    idx = np.empty((R, k), np.int32)
    kth = np.empty((R,), np.float32)
    _load().oracle_topk(_p(scores), scores.shape[1], R, _p(pos), int(k), _p(idx), _p(kth))
    return idx, kth


def sparse_attn(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, d_v: int, sm_scale: float):
    """MQA-mode attention over the selected latent rows (all in double).

    q [R, H, d_qk] float32, kv [S, d_qk] float32 (shared by all heads), idx [R, k] int32 (-1 skipped).
    Returns (out [R, H, d_v] float64, lse [R, H] float64)."""
    q = _c(q, np.float32)
    kv = _c(kv, np.float32)
    idx = _c(idx, np.int32)
    R, H, d_qk = q.shape
    k = idx.shape[1]
    assert idx.shape[0] == R and kv.shape[1] == d_qk and 0 < d_v <= d_qk
    assert idx.size == 0 or idx.max() < kv.shape[0]
    out = np.empty((R, H, d_v), np.float64)
    lse = np.empty((R, H), np.float64)
    _load().oracle_sparse_attn(_p(q), _p(kv), _p(idx), R, H, d_qk, d_v, k, float(sm_scale),
                               _p(out), _p(lse))
    return out, lse


def sparse_attn_mha(q: np.ndarray, k: np.ndarray, v: np.ndarray, idx: np.ndarray, sm_scale: float):
    """Masked MHA mode: attention over the selected entries with per-head key and value rows (all in
    double).  Masking every unselected key out of a dense softmax leaves exactly this sum.

    q [R, H, d_qk], k [S, H, d_qk], v [S, H, d_v] float32, idx [R, k_sel] int32 (-1 skipped).
    Returns (out [R, H, d_v] float64, lse [R, H] float64)."""
    q = _c(q, np.float32)
    k = _c(k, np.float32)
    v = _c(v, np.float32)
    idx = _c(idx, np.int32)
    R, H, d_qk = q.shape
    S, d_v = k.shape[0], v.shape[2]
    k_sel = idx.shape[1]
    assert idx.shape[0] == R and k.shape[1:] == (H, d_qk) and v.shape[:2] == (S, H)
    assert idx.size == 0 or idx.max() < S
    out = np.empty((R, H, d_v), np.float64)
    lse = np.empty((R, H), np.float64)
    _load().oracle_sparse_attn_mha(_p(q), _p(k), _p(v), _p(idx), R, H, d_qk, d_v, k_sel, float(sm_scale),
                                   _p(out), _p(lse))
    return out, lse


def forward(q_i: np.ndarray, w: np.ndarray, k_i: np.ndarray, q: np.ndarray, kv: np.ndarray,
            pos: np.ndarray, k: int, d_v: int, sm_scale: float):
    """The whole path for the query rows given by ``pos``: indexer -> top-k -> sparse attention.

    q_i [R, H_I, d_I], w [R, H_I], k_i [S, d_I] fp32 (dequantised); q [R, H, d_qk], kv [S, d_qk] fp32.
    Returns dict(scores, kth, idx, out, lse)."""
    scores = indexer(q_i, w, k_i, pos)
    idx, kth = topk(scores, pos, k)
    out, lse = sparse_attn(q, kv, idx, d_v, sm_scale)
    return dict(scores=scores, kth=kth, idx=idx, out=out, lse=lse)


def absorb_q(q_mha: np.ndarray, w_ukt: np.ndarray) -> np.ndarray:
    """MQA-mode query of MLA (velog summary, section 1.3: every latent entry serves all heads): the
    no-rope part of each head's query is carried into latent space by that head's key up-projection,
    q'_h = [W_UK,h^T q_nope,h ; q_rope,h], so that q'_h . [c ; k_rope] equals the MHA-form logit.

    q_mha [R, H, d_nope + d_rope], w_ukt [H, d_c, d_nope] (row c of head h holds W_UK,h[:, c]).
    Returns [R, H, d_c + d_rope] float64 (a float64 matmul as the step)."""
    d_c, d_nope = w_ukt.shape[1:]
    qn = np.asarray(q_mha[..., :d_nope], np.float64)
    lat = np.einsum("rhd,hcd->rhc", qn, np.asarray(w_ukt, np.float64))
    return np.concatenate([lat, np.asarray(q_mha[..., d_nope:], np.float64)], -1)


def out_proj(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Per-head value up-projection applied after MQA-mode attention: o_h = W_UV,h o'_h, where o'_h is the
    attention output in latent space (the first d_c latent columns are the values).

    o_lat [R, H, d_c], w_uv [H, d_v, d_c].  Returns [R, H, d_v] float64 (a float64 matmul as the step)."""
    return np.einsum("rhc,hvc->rhv", np.asarray(o_lat, np.float64), np.asarray(w_uv, np.float64))


def warmup_target(q: np.ndarray, kv: np.ndarray, pos: np.ndarray, sm_scale: float, ld: int | None = None):
    """Dense warm-up target (velog summary, Continued Pre-Training, Stage 1): the main MQA-mode attention
    summed over heads and L1-normalised, p[r][s] for s <= pos[r] (float64, zero elsewhere).
    q [R, H, d_qk], kv [S, d_qk] float32."""
    q = _c(q, np.float32)
    kv = _c(kv, np.float32)
    pos = _c(pos, np.int64)
    R, H, d_qk = q.shape
    ld = kv.shape[0] if ld is None else ld
    assert kv.shape[1] == d_qk and (R == 0 or pos.max() < kv.shape[0])
    p = np.zeros((R, ld), np.float64)
    _load().oracle_warmup_target(_p(q), _p(kv), R, _p(pos), H, d_qk, float(sm_scale), _p(p), ld)
    return p


def warmup_loss(p: np.ndarray, scores: np.ndarray, pos: np.ndarray):
    """KL(p[r] || softmax(I[r])) over s <= pos[r] and its gradient with respect to I, g = softmax(I) - p.
    p [R, ld] float64, scores [R, ld_s] float32.  Returns (loss [R] float64, g [R, ld] float64)."""
    p = _c(p, np.float64)
    scores = _c(scores, np.float32)
    pos = _c(pos, np.int64)
    R = p.shape[0]
    loss = np.empty(R, np.float64)
    g = np.zeros_like(p)
    _load().oracle_warmup_loss(_p(p), _p(scores), R, _p(pos), p.shape[1], scores.shape[1], _p(loss), _p(g),
                               g.shape[1])
    return loss, g


def warmup_backward(q: np.ndarray, w: np.ndarray, k: np.ndarray, g: np.ndarray, pos: np.ndarray):
    """Gradients of the warm-up loss through the indexer, given g = dL/dI [R, ld] (float64):
    returns (dq [R, H, d], dw [R, H], dk [S, d]) float64 with respect to the dequantised q, the weights w and
    the dequantised k."""
    q = _c(q, np.float32)
    w = _c(w, np.float32)
    k = _c(k, np.float32)
    g = _c(g, np.float64)
    pos = _c(pos, np.int64)
    R, H, d = q.shape
    S = k.shape[0]
    dq = np.empty((R, H, d), np.float64)
    dw = np.empty((R, H), np.float64)
    dk = np.empty((S, d), np.float64)
    _load().oracle_warmup_backward(_p(q), _p(w), _p(k), _p(g), R, _p(pos), H, d, S, g.shape[1], _p(dq), _p(dw),
                                   _p(dk))
    return dq, dw, dk



def sparse_attn_backward(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, d_v: int, sm_scale: float,
                         dout: np.ndarray):
    """Gradients of the MQA-mode sparse attention (sparse training stage), all in double.

    q [R, H, d_qk], kv [S, d_qk], dout [R, H, d_v] float32, idx [R, k] int32 (-1 skipped).
    Returns (dq [R, H, d_qk], dkv [S, d_qk], pbar [R, k]) float64: dL/dq, dL/dkv (the key and value
    gradients summed on the shared latent row) for dL/dout = dout, and the head mean of the attention
    probabilities of each selected entry (the indexer's target in that stage)."""
    q = _c(q, np.float32)
    kv = _c(kv, np.float32)
    idx = _c(idx, np.int32)
    dout = _c(dout, np.float32)
    R, H, d_qk = q.shape
    S = kv.shape[0]
    k = idx.shape[1]
    assert idx.shape[0] == R and kv.shape[1] == d_qk and dout.shape == (R, H, d_v) and 0 < d_v <= d_qk
    assert idx.size == 0 or idx.max() < S
    dq = np.empty((R, H, d_qk), np.float64)
    dkv = np.empty((S, d_qk), np.float64)
    pbar = np.empty((R, k), np.float64)
    _load().oracle_sparse_attn_backward(_p(q), _p(kv), _p(idx), R, H, d_qk, d_v, k, float(sm_scale), _p(dout), S,
                                        _p(dq), _p(dkv), _p(pbar))
    return dq, dkv, pbar


def sparse_kl_loss(pbar: np.ndarray, idx: np.ndarray, scores: np.ndarray, pos: np.ndarray):
    """The indexer loss of the sparse training stage: L_t = KL(p_t || softmax(I_t)) over s <= pos_t, with p_t
    the head mean of the sparse attention (pbar on the selected entries, 0 elsewhere).

    pbar [R, k] float64, idx [R, k] int32 (-1 skipped), scores [R, ld] float32.
    Returns (loss [R], g [R, ld]) float64 with g = softmax(I) - p over s <= pos (0 past it)."""
    pbar = _c(pbar, np.float64)
    idx = _c(idx, np.int32)
    R, ld = scores.shape
    p = np.zeros((R, ld), np.float64)
    for r in range(R):
        ok = idx[r] >= 0
        np.add.at(p[r], idx[r][ok], pbar[r][ok])
    return warmup_loss(p, scores, pos)
