"""Python binding of libdsa.so (include/dsa.h): argument marshalling only.

Every computation runs in the library's HIP kernels on the GPU; torch tensors are used only as
device memory and the current HIP stream.  If the library is missing this module raises on load:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2

# Every entry point of include/dsa.h, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "dsa_version": ([], _I),
    "dsa_status_string": ([_I], ctypes.c_char_p),
    "dsa_last_error": ([], ctypes.c_char_p),
    "dsa_indexer_scores": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I64, _P], _I),
    "dsa_topk": ([_P, _I64, _I, _I, _I, _I, _P, _P, _SZ, _P], _I),
    "dsa_topk_workspace_size": ([_I, _I, _I, _I], _SZ),
    "dsa_sparse_mla_attn": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _SZ, _P], _I),
    "dsa_sparse_mla_attn_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "dsa_forward_prefill": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P,
                             _P, _P, _SZ, _P], _I),
    "dsa_forward_decode": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P, _P,
                            _P, _SZ, _P], _I),
    "dsa_forward_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "dsa_masked_mha_attn": ([_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _SZ, _P], _I),
    "dsa_masked_mha_workspace_size": ([_I, _I, _I], _SZ),
    "dsa_warmup_loss": ([_P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _I64, _P, _I64, _P, _P], _I),
    "dsa_warmup_indexer_backward": ([_P, _P, _P, _P, _P, _P, _I64, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P], _I),
    "dsa_sparse_mla_backward_workspace_size": ([_I, _I, _I, _I, _I, _I, _I, _I], _SZ),
    "dsa_sparse_mla_backward": ([_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _P, _SZ,
                                 _P], _I),
    "dsa_sparse_kl_loss": ([_P, _I64, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "dsa_mla_absorb_q": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _P], _I),
    "dsa_mla_out_proj": ([_P, _P, _P, _I, _I, _I, _I, _I, _P], _I),
    "dsa_indexer_scores_decode": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I64, _P], _I),
    "dsa_topk_decode": ([_P, _I64, _I, _I, _I, _P, _P, _SZ, _P], _I),
    "dsa_topk_decode_workspace_size": ([_I, _I, _I], _SZ),
    "dsa_sparse_mla_attn_decode": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _P, _SZ, _P], _I),
    "dsa_sparse_mla_attn_decode_workspace_size": ([_I, _I, _I, _I, _I, _I, _I], _SZ),
    "dsa_forward_prefill_masked_mha": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                                        _I, _P, _P, _P, _P, _SZ, _P], _I),
    "dsa_forward_prefill_masked_mha_workspace_size": ([_I, _I, _I, _I], _SZ),
    "dsa_forward_decode_noalloc": ([_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _P,
                                    _P, _P], _I),
    "dsa_forward_decode_noalloc_max_bytes": ([], _SZ),
}

_lib = None


class DSAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status


def _status_name(st: int) -> str:
    return ["DSA_OK", "DSA_ERR_INVALID_ARG", "DSA_ERR_UNSUPPORTED", "DSA_ERR_WORKSPACE", "DSA_ERR_HIP"][st] \
        if 0 <= st <= 4 else f"status {st}"


def lib():
    """The loaded library (raises if libdsa.so has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with sparse_attention_13_amd/build.py "
                               "(or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(st: int):
    if st != DSA_OK:
        raise DSAError(st, lib().dsa_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("all tensors must be on the GPU")
            if not t.is_contiguous():
                raise ValueError("all tensors must be contiguous")


def version() -> int:
    return lib().dsa_version()


def indexer_scores(q, q_scale, k, k_scale, w, scores, n_q=None, stream=None):
    """scores[b, t, s] for s <= n_kv - n_q + t.  q [B, n_q, H_I, d_I] (uint8 e4m3 codes or f32),
    k [B, n_kv, d_I], w [B, n_q, H_I], scores [B, n_q, ld] f32 (written in place)."""
    _dev(q, q_scale, k, k_scale, w, scores)
    B, nq, H_I, d_I = q.shape
    n_kv = k.shape[1]
    _check(lib().dsa_indexer_scores(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), B, nq, n_kv, H_I, d_I,
                                    _dtype_code(q), _ptr(scores), scores.shape[-1], _stream(stream)))
    return scores


def topk_workspace_size(B: int, n_q: int, n_kv: int, k: int) -> int:
    return int(lib().dsa_topk_workspace_size(B, n_q, n_kv, k))


def topk(scores, n_kv: int, k: int, idx=None, workspace=None, stream=None):
    """Per row the k best s <= pos_t (ascending, -1 padded).  scores [B, n_q, ld] f32 -> idx [B, n_q, k] int32.
    workspace: uint8 device tensor of at least topk_workspace_size(...) bytes (allocated when missing)."""
    _dev(scores, idx, workspace)
    B, nq, ld = scores.shape
    if idx is None:
        idx = torch.empty((B, nq, k), dtype=torch.int32, device=scores.device)
    ws = topk_workspace_size(B, nq, n_kv, k)
    if ws and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=scores.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dsa_topk(_ptr(scores), ld, B, nq, n_kv, k, _ptr(idx), _ptr(workspace), wsz, _stream(stream)))
    return idx


def sparse_mla_attn(q, kv, idx, d_v: int, sm_scale: float, out=None, lse=None, workspace=None, stream=None):
    """MQA-mode attention over the selected latent rows.  q [B, n_q, H, d_qk], kv [B, n_kv, d_qk],
    idx [B, n_q, k] int32 -> out [B, n_q, H, d_v] (q's dtype), lse [B, n_q, H] f32."""
    _dev(q, kv, idx, out, lse, workspace)
    B, nq, H, d_qk = q.shape
    n_kv = kv.shape[1]
    k = idx.shape[-1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, nq, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, nq, H), dtype=torch.float32, device=q.device)
    ws = lib().dsa_sparse_mla_attn_workspace_size(B, nq, n_kv, H, d_qk, d_v, k, dt)
    if ws and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dsa_sparse_mla_attn(_ptr(q), _ptr(kv), _ptr(idx), B, nq, n_kv, H, d_qk, d_v, k, float(sm_scale), dt,
                                     _ptr(out), _ptr(lse), _ptr(workspace), wsz, _stream(stream)))
    return out, lse


def masked_mha_workspace_size(B: int, n_q: int, n_kv: int) -> int:
    return int(lib().dsa_masked_mha_workspace_size(B, n_q, n_kv))


def masked_mha_attn(q, k, v, idx, sm_scale: float, out=None, lse=None, workspace=None, stream=None):
    """Masked MHA mode: dense attention with per-head rows under the top-k mask.  q [B, n_q, H, d_qk],
    k [B, n_kv, H, d_qk], v [B, n_kv, H, d_v] (bf16), idx [B, n_q, k_sel] int32 -> out [B, n_q, H, d_v]
    bf16, lse [B, n_q, H] f32.  workspace: uint8 device tensor (allocated when missing)."""
    _dev(q, k, v, idx, out, lse, workspace)
    B, nq, H, d_qk = q.shape
    n_kv, d_v = k.shape[1], v.shape[-1]
    k_sel = idx.shape[-1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, nq, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, nq, H), dtype=torch.float32, device=q.device)
    ws = masked_mha_workspace_size(B, nq, n_kv)
    if workspace is None or workspace.numel() * workspace.element_size() < ws:
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size()
    _check(lib().dsa_masked_mha_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(idx), B, nq, n_kv, H, d_qk, d_v, k_sel,
                                     float(sm_scale), dt, _ptr(out), _ptr(lse), _ptr(workspace), wsz, _stream(stream)))
    return out, lse


def warmup_loss(q, kv, lse, scores, sm_scale: float, target=None, loss=None, stream=None):
    """Indexer warm-up loss: q [B, n_q, 128, 576], kv [B, n_kv, 576] bf16, lse [B, n_q, 128] f32 (the main
    attention's), scores [B, n_q, ld] f32 (index scores in, gradient softmax(I) - target out).
    Returns (loss [B, n_q], target [B, n_q, ld])."""
    _dev(q, kv, lse, scores, target, loss)
    B, nq, H, d_qk = q.shape
    n_kv = kv.shape[1]
    if target is None:
        target = torch.zeros_like(scores)
    if loss is None:
        loss = torch.empty((B, nq), dtype=torch.float32, device=q.device)
    _check(lib().dsa_warmup_loss(_ptr(q), _ptr(kv), _ptr(lse), B, nq, n_kv, H, d_qk, float(sm_scale), _dtype_code(q),
                                 _ptr(scores), scores.shape[-1], _ptr(target), target.shape[-1], _ptr(loss),
                                 _stream(stream)))
    return loss, target


def warmup_indexer_backward(q_i, q_i_scale, k_i, k_i_scale, w, grad, dq=None, dw=None, dk=None, stream=None):
    """Gradients of the warm-up loss through the fp8 indexer, given grad = dL/dI [B, n_q, ld] (f32).
    Returns (dq_i [B, n_q, 64, 128], dw [B, n_q, 64], dk_i [B, n_kv, 128]) f32."""
    _dev(q_i, q_i_scale, k_i, k_i_scale, w, grad, dq, dw, dk)
    B, nq, H_I, d_I = q_i.shape
    n_kv = k_i.shape[1]
    if dq is None:
        dq = torch.empty((B, nq, H_I, d_I), dtype=torch.float32, device=q_i.device)
    if dw is None:
        dw = torch.empty((B, nq, H_I), dtype=torch.float32, device=q_i.device)
    if dk is None:
        dk = torch.empty((B, n_kv, d_I), dtype=torch.float32, device=q_i.device)
    _check(lib().dsa_warmup_indexer_backward(_ptr(q_i), _ptr(q_i_scale), _ptr(k_i), _ptr(k_i_scale), _ptr(w),
                                             _ptr(grad), grad.shape[-1], B, nq, n_kv, H_I, d_I, _dtype_code(q_i),
                                             _ptr(dq), _ptr(dw), _ptr(dk), _stream(stream)))
    return dq, dw, dk


def sparse_mla_backward_workspace_size(B, n_q, n_kv, k):
    return int(lib().dsa_sparse_mla_backward_workspace_size(B, n_q, n_kv, 128, 576, 512, k, DSA_BF16))


def sparse_mla_backward(q, kv, idx, out, lse, dout, sm_scale: float, dq=None, dkv=None, pbar=None, workspace=None,
                        with_pbar: bool = True, stream=None):
    """Gradients of sparse_mla_attn: q [B, n_q, 128, 576], kv [B, n_kv, 576], out/dout [B, n_q, 128, 512] bf16,
    lse [B, n_q, 128] f32, idx [B, n_q, k] int32.  Returns (dq [B, n_q, 128, 576], dkv [B, n_kv, 576],
    pbar [B, n_q, k] or None) f32."""
    _dev(q, kv, idx, out, lse, dout, dq, dkv, pbar, workspace)
    B, nq, H, d_qk = q.shape
    n_kv, k = kv.shape[1], idx.shape[-1]
    if dq is None:
        dq = torch.empty((B, nq, H, d_qk), dtype=torch.float32, device=q.device)
    if dkv is None:
        dkv = torch.empty((B, n_kv, d_qk), dtype=torch.float32, device=q.device)
    if pbar is None and with_pbar:
        pbar = torch.empty((B, nq, k), dtype=torch.float32, device=q.device)
    ws = lib().dsa_sparse_mla_backward_workspace_size(B, nq, n_kv, H, d_qk, out.shape[-1], k, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device)
    _check(lib().dsa_sparse_mla_backward(_ptr(q), _ptr(kv), _ptr(idx), _ptr(out), _ptr(lse), _ptr(dout), B, nq, n_kv,
                                         H, d_qk, out.shape[-1], k, float(sm_scale), _dtype_code(q), _ptr(dq),
                                         _ptr(dkv), _ptr(pbar) if pbar is not None else None, _ptr(workspace),
                                         workspace.numel(), _stream(stream)))
    return dq, dkv, pbar


def sparse_kl_loss(scores, pbar, idx, n_kv=None, loss=None, stream=None):
    """Stage-2 indexer loss: scores [B, n_q, ld] f32 (index scores in, gradient softmax(I) - p out), pbar and
    idx [B, n_q, k].  Returns loss [B, n_q] f32."""
    _dev(scores, pbar, idx, loss)
    B, nq, ld = scores.shape
    n_kv = ld if n_kv is None else n_kv
    if loss is None:
        loss = torch.empty((B, nq), dtype=torch.float32, device=scores.device)
    _check(lib().dsa_sparse_kl_loss(_ptr(scores), ld, _ptr(pbar), _ptr(idx), B, nq, n_kv, idx.shape[-1], _ptr(loss),
                                    _stream(stream)))
    return loss


def mla_absorb_q(q_mha, w_ukt, q_mqa=None, stream=None):
    """MQA-mode query: q_mha [..., H, 192] bf16 (no-rope 128 + rope 64), w_ukt [H, 512, 128] bf16 ->
    q_mqa [..., H, 576] bf16 (W_UK absorbed into the no-rope part, rope copied)."""
    _dev(q_mha, w_ukt, q_mqa)
    H = q_mha.shape[-2]
    rows = q_mha.numel() // (H * 192)
    if q_mqa is None:
        q_mqa = torch.empty(tuple(q_mha.shape[:-1]) + (576,), dtype=q_mha.dtype, device=q_mha.device)
    _check(lib().dsa_mla_absorb_q(_ptr(q_mha), _ptr(w_ukt), _ptr(q_mqa), rows, H, 128, 64, 512, _dtype_code(q_mha),
                                  _stream(stream)))
    return q_mqa


def mla_out_proj(o_lat, w_uv, o=None, stream=None):
    """Per-head value up-projection: o_lat [..., H, 512] bf16, w_uv [H, 128, 512] bf16 -> o [..., H, 128]."""
    _dev(o_lat, w_uv, o)
    H = o_lat.shape[-2]
    rows = o_lat.numel() // (H * 512)
    if o is None:
        o = torch.empty(tuple(o_lat.shape[:-1]) + (128,), dtype=o_lat.dtype, device=o_lat.device)
    _check(lib().dsa_mla_out_proj(_ptr(o_lat), _ptr(w_uv), _ptr(o), rows, H, 512, 128, _dtype_code(o_lat),
                                  _stream(stream)))
    return o


def forward_workspace_size(B, n_q, n_kv, H, d_qk, d_v, k, attn_dtype) -> int:
    return int(lib().dsa_forward_workspace_size(B, n_q, n_kv, H, d_qk, d_v, k, attn_dtype))


def forward(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, k: int, d_v: int, sm_scale: float, decode: bool = False,
            out=None, lse=None, idx_out=None, workspace=None, stream=None):
    """Indexer -> top-k -> sparse attention on one stream.

    Prefill: q_i [B, n_q, H_I, d_I], w [B, n_q, H_I], q [B, n_q, H, d_qk].  Decode (decode=True):
    q_i [B, H_I, d_I], w [B, H_I], q [B, H, d_qk] (one query per sequence at position n_kv - 1).
    k_i [B, n_kv, d_I], kv [B, n_kv, d_qk].  Returns (out, lse, idx_out)."""
    _dev(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, out, lse, idx_out, workspace)
    if decode:
        B, H_I, d_I = q_i.shape
        n_q = 1
        H, d_qk = q.shape[1], q.shape[2]
    else:
        B, n_q, H_I, d_I = q_i.shape
        H, d_qk = q.shape[2], q.shape[3]
    n_kv = k_i.shape[1]
    adt = _dtype_code(q)
    idt = _dtype_code(q_i)
    if out is None:
        out = torch.empty((B, n_q, H, d_v) if not decode else (B, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, n_q, H) if not decode else (B, H), dtype=torch.float32, device=q.device)
    ws = forward_workspace_size(B, n_q, n_kv, H, d_qk, d_v, k, adt)
    if workspace is None or workspace.numel() * workspace.element_size() < ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size()
    L = lib()
    if decode:
        st = L.dsa_forward_decode(_ptr(q_i), _ptr(q_i_scale), _ptr(k_i), _ptr(k_i_scale), _ptr(w), _ptr(q), _ptr(kv),
                                  B, n_kv, H_I, d_I, H, d_qk, d_v, k, float(sm_scale), idt, adt, _ptr(out),
                                  _ptr(lse), _ptr(idx_out), _ptr(workspace), wsz, _stream(stream))
    else:
        st = L.dsa_forward_prefill(_ptr(q_i), _ptr(q_i_scale), _ptr(k_i), _ptr(k_i_scale), _ptr(w), _ptr(q),
                                   _ptr(kv), B, n_q, n_kv, H_I, d_I, H, d_qk, d_v, k, float(sm_scale), idt, adt,
                                   _ptr(out), _ptr(lse), _ptr(idx_out), _ptr(workspace), wsz, _stream(stream))
    _check(st)
    return out, lse, idx_out


# ---------------------------------------------------------------------------------------------- decode stages

def indexer_scores_decode(q, q_scale, k, k_scale, w, scores, stream=None):
    """Decode form of indexer_scores: q [B, H_I, d_I], w [B, H_I], k [B, n_kv, d_I], scores [B, ld] f32."""
    _dev(q, q_scale, k, k_scale, w, scores)
    B, H_I, d_I = q.shape
    n_kv = k.shape[1]
    _check(lib().dsa_indexer_scores_decode(_ptr(q), _ptr(q_scale), _ptr(k), _ptr(k_scale), _ptr(w), B, n_kv, H_I, d_I,
                                           _dtype_code(q), _ptr(scores), scores.shape[-1], _stream(stream)))
    return scores


def topk_decode(scores, n_kv: int, k: int, idx=None, workspace=None, stream=None):
    """Decode form of topk: scores [B, ld] f32 -> idx [B, k] int32."""
    _dev(scores, idx, workspace)
    B, ld = scores.shape
    if idx is None:
        idx = torch.empty((B, k), dtype=torch.int32, device=scores.device)
    ws = int(lib().dsa_topk_decode_workspace_size(B, n_kv, k))
    if ws and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=scores.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dsa_topk_decode(_ptr(scores), ld, B, n_kv, k, _ptr(idx), _ptr(workspace), wsz, _stream(stream)))
    return idx


def sparse_mla_attn_decode(q, kv, idx, d_v: int, sm_scale: float, out=None, lse=None, workspace=None, stream=None):
    """Decode form of sparse_mla_attn: q [B, H, d_qk], kv [B, n_kv, d_qk], idx [B, k] -> out [B, H, d_v], lse [B, H]."""
    _dev(q, kv, idx, out, lse, workspace)
    B, H, d_qk = q.shape
    n_kv = kv.shape[1]
    k = idx.shape[-1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    ws = int(lib().dsa_sparse_mla_attn_decode_workspace_size(B, n_kv, H, d_qk, d_v, k, dt))
    if ws and (workspace is None or workspace.numel() * workspace.element_size() < ws):
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dsa_sparse_mla_attn_decode(_ptr(q), _ptr(kv), _ptr(idx), B, n_kv, H, d_qk, d_v, k, float(sm_scale),
                                            dt, _ptr(out), _ptr(lse), _ptr(workspace), wsz, _stream(stream)))
    return out, lse


# ---------------------------------------------------------------------------------------------- masked MHA mode forward

def forward_masked_mha_workspace_size(B, n_q, n_kv, k_sel) -> int:
    return int(lib().dsa_forward_prefill_masked_mha_workspace_size(B, n_q, n_kv, k_sel))


def forward_masked_mha(q_i, q_i_scale, k_i, k_i_scale, w, q, k, v, k_sel: int, sm_scale: float, out=None, lse=None,
                       idx_out=None, workspace=None, stream=None):
    """Indexer -> top-k -> masked MHA mode on one stream.  q_i [B, n_q, H_I, d_I], w [B, n_q, H_I],
    k_i [B, n_kv, d_I]; q [B, n_q, H, 192], k [B, n_kv, H, 192], v [B, n_kv, H, 128] bf16.
    Returns (out [B, n_q, H, 128], lse [B, n_q, H], idx_out)."""
    _dev(q_i, q_i_scale, k_i, k_i_scale, w, q, k, v, out, lse, idx_out, workspace)
    B, n_q, H_I, d_I = q_i.shape
    H, d_qk = q.shape[2], q.shape[3]
    d_v = v.shape[3]
    n_kv = k_i.shape[1]
    if out is None:
        out = torch.empty((B, n_q, H, d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, n_q, H), dtype=torch.float32, device=q.device)
    ws = forward_masked_mha_workspace_size(B, n_q, n_kv, k_sel)
    if workspace is None or workspace.numel() * workspace.element_size() < ws:
        workspace = torch.empty(ws, dtype=torch.uint8, device=q.device)
    wsz = workspace.numel() * workspace.element_size()
    _check(lib().dsa_forward_prefill_masked_mha(_ptr(q_i), _ptr(q_i_scale), _ptr(k_i), _ptr(k_i_scale), _ptr(w),
                                                _ptr(q), _ptr(k), _ptr(v), B, n_q, n_kv, H_I, d_I, H, d_qk, d_v, k_sel,
                                                float(sm_scale), _dtype_code(q_i), _dtype_code(q), _ptr(out),
                                                _ptr(lse), _ptr(idx_out), _ptr(workspace), wsz, _stream(stream)))
    return out, lse, idx_out


# ---------------------------------------------------------------------------------------------- allocation-free decode

def forward_decode_noalloc(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, k: int, d_v: int, sm_scale: float, out,
                           lse=None, idx_out=None, stream=None):
    """dsa_forward_decode without a workspace (the library's fixed device scratch): q_i [B, H_I, d_I],
    w [B, H_I], q [B, H, d_qk], k_i [B, n_kv, d_I], kv [B, n_kv, d_qk]; out [B, H, d_v] and the optional
    lse [B, H], idx_out [B, k] are the caller's.  Nothing is allocated."""
    _dev(q_i, q_i_scale, k_i, k_i_scale, w, q, kv, out, lse, idx_out)
    B, H_I, d_I = q_i.shape
    H, d_qk = q.shape[1], q.shape[2]
    n_kv = k_i.shape[1]
    _check(lib().dsa_forward_decode_noalloc(_ptr(q_i), _ptr(q_i_scale), _ptr(k_i), _ptr(k_i_scale), _ptr(w), _ptr(q),
                                            _ptr(kv), B, n_kv, H_I, d_I, H, d_qk, d_v, k, float(sm_scale),
                                            _dtype_code(q_i), _dtype_code(q), _ptr(out), _ptr(lse), _ptr(idx_out),
                                            _stream(stream)))
    return out, lse, idx_out
