"""Exact tiled attention (prefill forward -- dense, padded or packed variable-length -- and
backward, split-KV decode over contiguous or paged caches, LSE merge) on gfx950.

Thin torch-facing wrappers over the C ABI in include/fa.h.  Each function has
the name of the C entry point it marshals arguments for; all computation runs
in the HIP kernels of libfa.so (loaded on first use, never replaced by a CPU
path).
"""
import math

import torch

from . import _lib
from ._lib import FAError, FA_DECODE_SPLIT_ALIGN, FA_MAX_SPLITS, FA_NOALLOC_SCRATCH_BYTES  # noqa: F401

__all__ = ["fa_fwd", "fa_fwd_fp8", "fa_fwd_varlen", "fa_decode_splitkv", "fa_lse_merge", "fa_decode", "fa_decode_workspace_bytes",
           "fa_decode_noalloc",
           "fa_decode_paged", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string", "fa_last_error", "FAError",
           "default_scale", "attention"]

_DTYPES = {torch.bfloat16: _lib.FA_BF16, torch.float32: _lib.FA_F32}


def default_scale(d):
    return 1.0 / math.sqrt(d)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_tensor(t, name, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}")


def _lens(kv_seqlens, B, device):
    if kv_seqlens is None:
        return None
    _check_tensor(kv_seqlens, "kv_seqlens", torch.int32, 1, device)
    if kv_seqlens.numel() != B:
        raise ValueError("kv_seqlens must have B entries")
    return kv_seqlens


def fa_fwd(q, k, v, causal=False, kv_seqlens=None, scale=None, out=None, lse=None):
    """Exact attention forward.  q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] (bf16 or f32).

    Returns (o [B,Hq,Nq,d] in q's dtype, lse [B,Hq,Nq] float32).
    """
    _check_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    _check_tensor(k, "k", q.dtype, 4, q.device)
    _check_tensor(v, "v", q.dtype, 4, q.device)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    lens = _lens(kv_seqlens, B, q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", q.dtype, 4, q.device)
    _check_tensor(lse, "lse", torch.float32, 3, q.device)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("out/lse have the wrong shape")
    s = default_scale(d) if scale is None else float(scale)
    lib = _lib.load()
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, s,
                              int(bool(causal)), _ptr(lens), _DTYPES[q.dtype], _stream(q)))
    return out, lse


_FP8 = {torch.float8_e4m3fn: _lib.FA_FP8_E4M3, torch.float8_e5m2: _lib.FA_FP8_E5M2}


def fa_fwd_fp8(q, k, v, q_descale, k_descale, v_descale, causal=False, kv_seqlens=None, scale=None, out=None,
               lse=None):
    """Exact attention on FP8 inputs (d = 128).

    q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] are torch float8_e4m3fn or float8_e5m2
    tensors (one format for all three); the real inputs are descale * value.
    Returns (o [B,Hq,Nq,d] bfloat16, lse [B,Hq,Nq] float32).
    """
    _check_tensor(q, "q", ndim=4)
    if q.dtype not in _FP8:
        raise ValueError("q must be float8_e4m3fn or float8_e5m2")
    _check_tensor(k, "k", q.dtype, 4, q.device)
    _check_tensor(v, "v", q.dtype, 4, q.device)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    lens = _lens(kv_seqlens, B, q.device)
    if out is None:
        out = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", torch.bfloat16, 4, q.device)
    _check_tensor(lse, "lse", torch.float32, 3, q.device)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("out/lse have the wrong shape")
    s = default_scale(d) if scale is None else float(scale)
    lib = _lib.load()
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, s,
                                  int(bool(causal)), _ptr(lens), float(q_descale), float(k_descale), float(v_descale),
                                  _FP8[q.dtype], _stream(q)))
    return out, lse


def fa_fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, causal=False, scale=None, out=None,
                  lse=None):
    """Exact attention over packed variable-length sequences.

    q [Hq, total_q, d], k/v [Hkv, total_k, d] (bf16 or f32); cu_seqlens_q and
    cu_seqlens_k are int32 GPU tensors of B + 1 cumulative offsets;
    max_seqlen_q (a host int) is at least the longest query sequence.
    Returns (o [Hq, total_q, d] in q's dtype, lse [Hq, total_q] float32).
    """
    _check_tensor(q, "q", ndim=3)
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    _check_tensor(k, "k", q.dtype, 3, q.device)
    _check_tensor(v, "v", q.dtype, 3, q.device)
    Hq, total_q, d = q.shape
    Hkv, total_k = k.shape[0], k.shape[1]
    if tuple(k.shape) != (Hkv, total_k, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [Hkv, total_k, d] matching q")
    _check_tensor(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, q.device)
    _check_tensor(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, q.device)
    if cu_seqlens_q.numel() < 1 or cu_seqlens_k.numel() != cu_seqlens_q.numel():
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    B = cu_seqlens_q.numel() - 1
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    _check_tensor(out, "out", q.dtype, 3, q.device)
    _check_tensor(lse, "lse", torch.float32, 2, q.device)
    if tuple(out.shape) != tuple(q.shape) or tuple(lse.shape) != (Hq, total_q):
        raise ValueError("out/lse have the wrong shape")
    s = default_scale(d) if scale is None else float(scale)
    lib = _lib.load()
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens_q),
                                     _ptr(cu_seqlens_k), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q), d, s,
                                     int(bool(causal)), _DTYPES[q.dtype], _stream(q)))
    return out, lse


def fa_decode_workspace_bytes(B, Hq, d, num_splits):
    return int(_lib.load().fa_decode_workspace_bytes(B, Hq, d, num_splits))


def _decode_shapes(q, k_cache, v_cache):
    _check_tensor(q, "q", ndim=4)
    if q.dtype not in _DTYPES:
        raise ValueError("q must be bfloat16 or float32")
    _check_tensor(k_cache, "k_cache", q.dtype, 4, q.device)
    _check_tensor(v_cache, "v_cache", q.dtype, 4, q.device)
    B, Hq, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes q of shape [B, Hq, 1, d]")
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, Nk, d) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("caches must be [B, Hkv, Nk, d] matching q")
    return B, Hq, Hkv, Nk, d


def _check_decode_out(out, lse, q):
    """The merge writes B*Hq rows of d outputs and one LSE each: the C ABI
    cannot see buffer sizes, so they are checked here, before any launch."""
    B, Hq, _, d = q.shape
    _check_tensor(out, "out", q.dtype, 4, q.device)
    _check_tensor(lse, "lse", torch.float32, 3, q.device)
    if tuple(out.shape) != (B, Hq, 1, d) or tuple(lse.shape) != (B, Hq, 1):
        raise ValueError(f"out must be [{B}, {Hq}, 1, {d}] and lse [{B}, {Hq}, 1]")


def fa_decode_splitkv(q, k_cache, v_cache, num_splits=16, kv_seqlens=None, scale=None,
                      o_part=None, lse_part=None):
    """Split-KV decode partials: (o_part [B,Hq,S,d] f32, lse_part [B,Hq,S] f32)."""
    B, Hq, Hkv, Nk, d = _decode_shapes(q, k_cache, v_cache)
    lens = _lens(kv_seqlens, B, q.device)
    if o_part is None:
        o_part = torch.empty((B, Hq, num_splits, d), dtype=torch.float32, device=q.device)
    if lse_part is None:
        lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    _check_tensor(o_part, "o_part", torch.float32, 4, q.device)
    _check_tensor(lse_part, "lse_part", torch.float32, 3, q.device)
    if tuple(o_part.shape) != (B, Hq, num_splits, d) or tuple(lse_part.shape) != (B, Hq, num_splits):
        raise ValueError("o_part/lse_part have the wrong shape")
    s = default_scale(d) if scale is None else float(scale)
    lib = _lib.load()
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o_part), _ptr(lse_part),
                                         B, Hq, Hkv, Nk, d, s, _ptr(lens), num_splits, _DTYPES[q.dtype],
                                         _stream(q)))
    return o_part, lse_part


def fa_lse_merge(o_part, lse_part, dtype=torch.bfloat16, out=None, lse=None):
    """Merge partials [..., S, d] / [..., S] into (o [..., 1, d] dtype, lse [..., 1] f32)."""
    _check_tensor(o_part, "o_part", torch.float32)
    _check_tensor(lse_part, "lse_part", torch.float32, o_part.dim() - 1, o_part.device)
    S, d = o_part.shape[-2], o_part.shape[-1]
    lead = tuple(o_part.shape[:-2])
    if tuple(lse_part.shape) != lead + (S,):
        raise ValueError("lse_part must be o_part.shape[:-1]")
    rows = 1
    for x in lead:
        rows *= x
    if out is None:
        out = torch.empty(lead + (1, d), dtype=dtype, device=o_part.device)
    if lse is None:
        lse = torch.empty(lead + (1,), dtype=torch.float32, device=o_part.device)
    _check_tensor(out, "out", dtype, device=o_part.device)
    _check_tensor(lse, "lse", torch.float32, device=o_part.device)
    if out.numel() != rows * d or lse.numel() != rows:
        raise ValueError("out/lse have the wrong size")
    lib = _lib.load()
    with torch.cuda.device(o_part.device):  # kernels launch on the current device
        _lib.check(lib.fa_lse_merge(_ptr(o_part), _ptr(lse_part), _ptr(out), _ptr(lse), rows, d, S,
                                    _DTYPES[dtype], _stream(o_part)))
    return out, lse


def fa_decode(q, k_cache, v_cache, kv_seqlens=None, num_splits=16, scale=None, workspace=None,
              out=None, lse=None):
    """Single-token decode: split-KV partials then exact merge, one call.

    Returns (o [B,Hq,1,d] in q's dtype, lse [B,Hq,1] float32).
    """
    B, Hq, Hkv, Nk, d = _decode_shapes(q, k_cache, v_cache)
    lens = _lens(kv_seqlens, B, q.device)
    lib = _lib.load()
    need = int(lib.fa_decode_workspace_bytes(B, Hq, d, num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_tensor(workspace, "workspace", torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
    _check_decode_out(out, lse, q)
    s = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_decode(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, Hq, Hkv, Nk, d,
                                 s, _ptr(lens), num_splits, _ptr(workspace), workspace.numel(),
                                 _DTYPES[q.dtype], _stream(q)))
    return out, lse


def fa_decode_noalloc(q, k_cache, v_cache, out, lse, kv_seqlens=None, num_splits=16, scale=None):
    """fa_decode without a workspace, for callers that cannot allocate: the split
    partials live in the library's static per-GPU scratch (FA_NOALLOC_SCRATCH_BYTES).
    out [B,Hq,1,d] (q's dtype) and lse [B,Hq,1] float32 are caller-provided;
    nothing is allocated.  Calls that overlap on one GPU race on the scratch."""
    B, Hq, Hkv, Nk, d = _decode_shapes(q, k_cache, v_cache)
    lens = _lens(kv_seqlens, B, q.device)
    _check_decode_out(out, lse, q)
    s = default_scale(d) if scale is None else float(scale)
    lib = _lib.load()
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_decode_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), B, Hq, Hkv,
                                         Nk, d, s, _ptr(lens), num_splits, _DTYPES[q.dtype], _stream(q)))
    return out, lse


def fa_decode_paged(q, k_pages, v_pages, block_table, kv_seqlens, num_splits=16, scale=None, workspace=None,
                    out=None, lse=None):
    """Single-token decode over a paged KV cache (bf16).

    q [B,Hq,1,d]; k_pages, v_pages [num_pages, Hkv, page_size, d]; block_table [B, max_pages] int32;
    kv_seqlens [B] int32.  Returns (o [B,Hq,1,d], lse [B,Hq,1] float32).
    """
    _check_tensor(q, "q", torch.bfloat16, 4)
    _check_tensor(k_pages, "k_pages", torch.bfloat16, 4, q.device)
    _check_tensor(v_pages, "v_pages", torch.bfloat16, 4, q.device)
    _check_tensor(block_table, "block_table", torch.int32, 2, q.device)
    B, Hq, nq, d = q.shape
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    if nq != 1 or tuple(v_pages.shape) != tuple(k_pages.shape) or k_pages.shape[3] != d:
        raise ValueError("q must be [B,Hq,1,d] and k_pages/v_pages [num_pages,Hkv,page_size,d]")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have B rows")
    lens = _lens(kv_seqlens, B, q.device)
    if lens is None:
        raise ValueError("kv_seqlens is required for a paged cache")
    lib = _lib.load()
    need = int(lib.fa_decode_workspace_bytes(B, Hq, d, num_splits))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_tensor(workspace, "workspace", torch.uint8, device=q.device)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
    _check_decode_out(out, lse, q)
    s = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_decode_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), _ptr(out), _ptr(lse),
                                       B, Hq, Hkv, num_pages, page_size, block_table.shape[1], d, s, _ptr(lens),
                                       num_splits, _ptr(workspace), workspace.numel(), _lib.FA_BF16, _stream(q)))
    return out, lse


def fa_bwd_workspace_bytes(B, Hq, Nq, d):
    return int(_lib.load().fa_bwd_workspace_bytes(B, Hq, Nq, d))


def fa_bwd(q, k, v, o, lse, dout, causal=False, kv_seqlens=None, scale=None, workspace=None,
           dq=None, dk=None, dv=None):
    """Gradients of fa_fwd: given its inputs, its outputs (o, lse) and dout = dL/dO, returns
    (dq, dk, dv) shaped like q, k, v (bf16 only)."""
    _check_tensor(q, "q", torch.bfloat16, 4)
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check_tensor(t, name, torch.bfloat16, 4, q.device)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Nk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k and v must be [B, Hkv, Nk, d] matching q")
    if tuple(o.shape) != tuple(q.shape) or tuple(dout.shape) != tuple(q.shape):
        raise ValueError("o and dout must be shaped like q")
    _check_tensor(lse, "lse", torch.float32, 3, q.device)
    if tuple(lse.shape) != (B, Hq, Nq):
        raise ValueError("lse must be [B, Hq, Nq]")
    lens = _lens(kv_seqlens, B, q.device)
    lib = _lib.load()
    need = int(lib.fa_bwd_workspace_bytes(B, Hq, Nq, d))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check_tensor(workspace, "workspace", torch.uint8, device=q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for t, ref, name in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        _check_tensor(t, name, torch.bfloat16, 4, q.device)
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} has the wrong shape")
    s = default_scale(d) if scale is None else float(scale)
    with torch.cuda.device(q.device):  # kernels launch on the current device
        _lib.check(lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                              _ptr(dv), B, Hq, Hkv, Nq, Nk, d, s, int(bool(causal)), _ptr(lens), _ptr(workspace),
                              workspace.numel(), _lib.FA_BF16, _stream(q)))
    return dq, dk, dv


class _Attention(torch.autograd.Function):
    """fa_fwd in the forward pass, fa_bwd in the backward pass (bf16)."""

    @staticmethod
    def forward(ctx, q, k, v, causal, kv_seqlens, scale):
        o, lse = fa_fwd(q, k, v, causal=causal, kv_seqlens=kv_seqlens, scale=scale)
        ctx.save_for_backward(q, k, v, o, lse, kv_seqlens)
        ctx.causal, ctx.scale = causal, scale
        ctx.mark_non_differentiable(lse)
        return o, lse

    @staticmethod
    def backward(ctx, do, _dlse):
        q, k, v, o, lse, kv_seqlens = ctx.saved_tensors
        dq, dk, dv = fa_bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, kv_seqlens=kv_seqlens,
                            scale=ctx.scale)
        return dq, dk, dv, None, None, None


def attention(q, k, v, causal=False, kv_seqlens=None, scale=None):
    """Exact attention with autograd: returns O (bf16 [B, Hq, Nq, d]) and keeps what
    fa_bwd needs for the backward pass.  q [B, Hq, Nq, d], k/v [B, Hkv, Nk, d] in
    bf16; kv_seqlens and scale as in fa_fwd.  The LSE is not returned: gradients
    flow through O only."""
    if q.dtype != torch.bfloat16:
        raise ValueError("attention() with gradients takes bf16 inputs (the backward pass is bf16 only)")
    o, _ = _Attention.apply(q, k, v, bool(causal), kv_seqlens, scale)
    return o


def fa_status_string(status):
    return _lib.load().fa_status_string(status).decode()


def fa_last_error():
    return _lib.load().fa_last_error().decode()
